// Read-only gather of selected weight columns: the practical bandwidth ceiling
// of the index-list product's access pattern (Spark Transformer article,
// section 3.1: only the weight vectors of active inputs are read), with no
// gate, no arithmetic on the weights beyond a checksum, and no reduction.
//
// Grid: (row tile, index range) pairs of 1024-thread workgroups, two resident
// per compute unit (32 wavefronts: measured ~25 % more bandwidth than one
// workgroup per unit on this pattern). Each wavefront streams one column's
// 1 KB row-tile run per load (64 lanes x 16 bytes), eight runs in flight per
// lane. Index values are clamped into [0, n) so every load stays inside W.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace {

using sl::dev::u32x4;

constexpr int CT = 1024;  // threads per workgroup
constexpr int CU8 = 8;    // runs in flight per lane

__global__ __launch_bounds__(CT) void gather_ceiling_kernel(const u32x4* __restrict__ W, int vecs_per_col, int n,
                                                            const int32_t* __restrict__ idx, int count, int tiles,
                                                            int per, float* __restrict__ sink) {
  const int b = blockIdx.x, t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int tile = b % tiles, split = b / tiles;
  const int e0 = split * per, e1 = min(count, e0 + per);
  const int v = tile * 64 + lane;  // this lane's 16-byte vector within a column
  const bool vok = v < vecs_per_col;
  uint32_t acc = 0u;
  for (int e = e0 + w; e < e1; e += 16 * CU8) {
    u32x4 r[CU8];
#pragma unroll
    for (int u = 0; u < CU8; ++u) {
      const int k = e + u * 16;
      int col = k < e1 ? idx[k] : 0;
      col = col < 0 ? 0 : (col >= n ? n - 1 : col);
      r[u] = (k < e1 && vok) ? __builtin_nontemporal_load(W + (size_t)col * vecs_per_col + v) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < CU8; ++u) acc += r[u][0] ^ r[u][1] ^ r[u][2] ^ r[u][3];
  }
  // never true for real data; keeps the loads from being dropped
  if (acc == 0x9e3779b9u) sink[0] = (float)acc;
}

}  // namespace

namespace sl {

hipError_t launch_gather_ceiling(const sl_linear* h, const int32_t* idx, int count, float* sink, hipStream_t s) {
  const int esz = h->wdt == SL_BF16 ? 2 : 4;
  const int vecs_per_col = (int)(h->m * esz / 16);  // m is a multiple of the 16-byte run
  const int tiles = (vecs_per_col + 63) / 64;
  const int slots = 2 * std::max(1, h->cus);
  int splits = std::max(1, slots / tiles);
  splits = std::min(splits, std::max(1, count));
  const int per = std::max(1, (count + splits - 1) / splits);
  splits = std::max(1, (count + per - 1) / per);
  gather_ceiling_kernel<<<tiles * splits, CT, 0, s>>>((const u32x4*)h->Wt, vecs_per_col, (int)h->n, idx, count,
                                                     tiles, per, sink);
  return hipGetLastError();
}

}  // namespace sl
