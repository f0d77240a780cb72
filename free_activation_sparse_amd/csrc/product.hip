// Single-token product kernel: y = sum over kept j of x_j * W[:, j].
//
// This is the index-list product of the Spark Transformer article (section
// 3.1): only the weight vectors of active inputs are read. W is column-major,
// so each kept input contributes one contiguous run of m weights; the grid is
// (row tiles) x (input chunks) and every workgroup
//   1. re-evaluates the gate predicate for its chunk of inputs from x, c and
//      the gate's (kthr, jlast) pair, and compacts the kept inputs into LDS in
//      ascending order with wavefront ballots (no global index list),
//   2. streams the kept columns' row-tile runs with 16-byte non-temporal loads,
//      lanes of a group covering consecutive rows, several columns in flight,
//      fp32 accumulation,
//   3. reduces its column slots in LDS and either writes y (one chunk) or a
//      partial sum; the last workgroup of a row tile to arrive (counted with a
//      device-scope atomic after a release fence) adds the partials in split
//      order, so the result does not depend on scheduling.
#include "device_common.h"
#include "internal.h"

namespace {

using namespace sl::dev;

constexpr int PT = 256;  // threads per product workgroup (4 wavefronts)

template <typename WT, typename YT, int LPC, int U, bool DENSE>
__global__ __launch_bounds__(PT) void product_kernel(const WT* __restrict__ Wt, const WT* __restrict__ x,
                                                     const float* __restrict__ c,
                                                     const sl::GateOut* __restrict__ gout, int m, int n,
                                                     int tiles, int splits, int chunk,
                                                     float* __restrict__ partials, uint32_t* __restrict__ ctr,
                                                     YT* __restrict__ y) {
  constexpr int VEC = 16 / (int)sizeof(WT);  // elements per 16-byte run
  constexpr int R = LPC * VEC;               // rows per tile
  constexpr int CPW = 64 / LPC;              // column slots per wavefront
  constexpr int CS = 4 * CPW;                // column slots per workgroup
  __shared__ int2 list[sl::kMaxChunk];
  __shared__ uint32_t wcnt[4];
  __shared__ float red[CS * R];
  __shared__ uint32_t s_last;

  const int tile = blockIdx.x % tiles;
  const int split = blockIdx.x / tiles;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int j0 = split * chunk;
  const int j1 = min(j0 + chunk, n);

  // 1. kept inputs of this chunk, ascending, as (j, x_j) pairs in LDS
  uint32_t kthr = 0u;
  int jlast = 0;
  if (!DENSE) {
    kthr = gout->kthr;
    jlast = gout->jlast;
  }
  int cnt = 0;
  for (int jb = j0; jb < j1; jb += PT) {
    const int j = jb + t;
    bool keep = false;
    float xv = 0.f;
    if (j < j1) {
      xv = load_elem(x + j);
      keep = DENSE ? true : gate_keep(score_key(xv, c[j]), j, kthr, jlast);
    }
    const uint64_t bal = __ballot(keep);
    if (lane == 0) wcnt[w] = (uint32_t)__popcll(bal);
    __syncthreads();
    uint32_t off = (uint32_t)cnt;
    for (int k = 0; k < w; ++k) off += wcnt[k];
    if (keep) list[off + lanes_below(bal)] = make_int2(j, __float_as_int(xv));
    cnt += (int)(wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3]);
    __syncthreads();
  }

  // 2. stream the kept columns' runs for this row tile
  const int slot = w * CPW + lane / LPC;
  const int sub = lane % LPC;
  const int row = tile * R + sub * VEC;
  float acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
  if (row < m) {
    const WT* base = Wt + row;
    for (int k0 = slot; k0 < cnt; k0 += CS * U) {
      u32x4 wv[U];
      float xs[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = k0 + u * CS;
        if (k < cnt) {
          const int2 e = list[k];
          wv[u] = __builtin_nontemporal_load((const u32x4*)(base + (size_t)e.x * (size_t)m));
          xs[u] = __int_as_float(e.y);
        } else {
          wv[u] = u32x4{0u, 0u, 0u, 0u};
          xs[u] = 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) fma_run(acc, wv[u], xs[u]);
    }
  }

  // 3. reduce column slots, fixed order
#pragma unroll
  for (int v = 0; v < VEC; ++v) red[slot * R + sub * VEC + v] = acc[v];
  __syncthreads();
  float part[(R + PT - 1) / PT];
#pragma unroll
  for (int q = 0; q < (R + PT - 1) / PT; ++q) {
    const int r = t + q * PT;
    float s = 0.f;
    if (r < R) {
#pragma unroll
      for (int k = 0; k < CS; ++k) s += red[k * R + r];
    }
    part[q] = s;
  }

  if (splits == 1) {
#pragma unroll
    for (int q = 0; q < (R + PT - 1) / PT; ++q) {
      const int r = t + q * PT;
      const int gr = tile * R + r;
      if (r < R && gr < m) store_out(y + gr, part[q]);
    }
    return;
  }

#pragma unroll
  for (int q = 0; q < (R + PT - 1) / PT; ++q) {
    const int r = t + q * PT;
    const int gr = tile * R + r;
    if (r < R && gr < m) partials[(size_t)split * m + gr] = part[q];
  }
  __threadfence();
  __syncthreads();
  if (t == 0) s_last = (atomicAdd(&ctr[tile], 1u) == (uint32_t)(splits - 1)) ? 1u : 0u;
  __syncthreads();
  if (s_last == 0u) return;
  __threadfence();
#pragma unroll
  for (int q = 0; q < (R + PT - 1) / PT; ++q) {
    const int r = t + q * PT;
    const int gr = tile * R + r;
    if (r < R && gr < m) {
      float s = 0.f;
      for (int k = 0; k < splits; ++k) s += partials[(size_t)k * m + gr];
      store_out(y + gr, s);
    }
  }
  if (t == 0) atomicExch(&ctr[tile], 0u);
}

template <typename WT, typename YT, int LPC, bool DENSE>
hipError_t go(const sl_linear* h, const sl::Plan& p, const void* x, void* y, hipStream_t s) {
  const int grid = p.tiles * p.splits;
  product_kernel<WT, YT, LPC, 4, DENSE><<<grid, PT, 0, s>>>(
      (const WT*)h->Wt, (const WT*)x, h->c, h->gout, (int)h->m, (int)h->n, p.tiles, p.splits, p.chunk,
      h->partials, h->ctr, (YT*)y);
  return hipGetLastError();
}

template <typename WT, typename YT, bool DENSE>
hipError_t go_lpc(const sl_linear* h, const sl::Plan& p, const void* x, void* y, hipStream_t s) {
  switch (p.lpc) {
    case 16: return go<WT, YT, 16, DENSE>(h, p, x, y, s);
    case 32: return go<WT, YT, 32, DENSE>(h, p, x, y, s);
    default: return go<WT, YT, 64, DENSE>(h, p, x, y, s);
  }
}

template <typename WT, bool DENSE>
hipError_t go_y(const sl_linear* h, const sl::Plan& p, const void* x, void* y, sl_dtype ydt, hipStream_t s) {
  if (ydt == SL_BF16) return go_lpc<WT, uint16_t, DENSE>(h, p, x, y, s);
  return go_lpc<WT, float, DENSE>(h, p, x, y, s);
}

}  // namespace

namespace sl {

hipError_t launch_product(const sl_linear* h, const Plan& p, const void* x, bool dense, void* y,
                          sl_dtype ydt, hipStream_t s) {
  if (h->wdt == SL_BF16) {
    return dense ? go_y<uint16_t, true>(h, p, x, y, ydt, s) : go_y<uint16_t, false>(h, p, x, y, ydt, s);
  }
  return dense ? go_y<float, true>(h, p, x, y, ydt, s) : go_y<float, false>(h, p, x, y, ydt, s);
}

}  // namespace sl
