// Single-token product kernel: y = sum over kept j of x_j * W[:, j], on a
// grid of (row tiles) x (input chunks) of 256-thread workgroups that read the
// gate's (kthr, jlast) pair from the gate kernel's output. The phases (chunk
// predicate and compaction, column streaming, split reduction) are in
// product_body.h.
#include "product_body.h"

namespace {

using namespace sl::proddev;

constexpr int PT = 256;  // threads per product workgroup (4 wavefronts)

template <typename WT, typename YT, int LPC, int U, bool DENSE, bool ATOMIC>
__global__ __launch_bounds__(PT) void product_kernel(const WT* __restrict__ Wt, const WT* __restrict__ x,
                                                     const float* __restrict__ c,
                                                     const sl::GateOut* __restrict__ gout, int m, int n,
                                                     int tiles, int splits, int chunk,
                                                     float* __restrict__ partials, uint32_t* __restrict__ ctr,
                                                     YT* __restrict__ y) {
  __shared__ int2 list[sl::kMaxChunk];
  __shared__ uint32_t wcnt[sl::kMaxChunk / 64 + 1];
  __shared__ float red[red_floats<WT, PT>()];
  __shared__ uint32_t s_last;

  const int tile = blockIdx.x % tiles;
  const int split = blockIdx.x / tiles;
  const int j0 = split * chunk;
  const int j1 = min(j0 + chunk, n);

  uint32_t kthr = 0u;
  int jlast = 0;
  if (!DENSE) {
    kthr = gout->kthr;
    jlast = gout->jlast;
  }
  Chunk<PT> ch;
  load_chunk<WT, PT, DENSE>(x, c, j0, j1, ch);
  const int cnt = compact_chunk<PT, DENSE>(ch, j0, j1, kthr, jlast, list, wcnt);
  stream_reduce<WT, YT, LPC, U, PT, ATOMIC>(Wt, m, tile, split, splits, list, cnt, red, partials, ctr, &s_last, y);
}

// y[0..count) = 0 (fp32); precedes an atomic product when no gate kernel ran.
__global__ __launch_bounds__(256) void zero_kernel(float* __restrict__ y, int count) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < count) y[i] = 0.f;
}

template <typename WT, typename YT, int LPC, bool DENSE, bool ATOMIC>
hipError_t go(const sl_linear* h, const sl::Plan& p, const void* x, const sl::GateOut* g, void* y, hipStream_t s) {
  const int grid = p.tiles * p.splits;
  product_kernel<WT, YT, LPC, 8, DENSE, ATOMIC><<<grid, PT, 0, s>>>(
      (const WT*)h->Wt, (const WT*)x, h->c, g, (int)h->m, (int)h->n, p.tiles, p.splits, p.chunk, h->partials,
      h->ctr, (YT*)y);
  return hipGetLastError();
}

template <typename WT, typename YT, bool DENSE, bool ATOMIC>
hipError_t go_lpc(const sl_linear* h, const sl::Plan& p, const void* x, const sl::GateOut* g, void* y,
                  hipStream_t s) {
  switch (p.lpc) {
    case 16: return go<WT, YT, 16, DENSE, ATOMIC>(h, p, x, g, y, s);
    case 32: return go<WT, YT, 32, DENSE, ATOMIC>(h, p, x, g, y, s);
    default: return go<WT, YT, 64, DENSE, ATOMIC>(h, p, x, g, y, s);
  }
}

template <typename WT, bool DENSE>
hipError_t go_y(const sl_linear* h, const sl::Plan& p, const void* x, const sl::GateOut* g, void* y, sl_dtype ydt,
                hipStream_t s) {
  if (ydt == SL_BF16) return go_lpc<WT, uint16_t, DENSE, false>(h, p, x, g, y, s);
  if (p.atomic) return go_lpc<WT, float, DENSE, true>(h, p, x, g, y, s);
  return go_lpc<WT, float, DENSE, false>(h, p, x, g, y, s);
}

}  // namespace

namespace sl {

hipError_t launch_zero(float* y, int64_t count, hipStream_t s) {
  zero_kernel<<<(unsigned)((count + 255) / 256), 256, 0, s>>>(y, (int)count);
  return hipGetLastError();
}

hipError_t launch_product(const sl_linear* h, const Plan& p, const void* x, const GateOut* g, bool dense,
                          void* y, sl_dtype ydt, hipStream_t s) {
  if (h->wdt == SL_BF16) {
    return dense ? go_y<uint16_t, true>(h, p, x, g, y, ydt, s) : go_y<uint16_t, false>(h, p, x, g, y, ydt, s);
  }
  return dense ? go_y<float, true>(h, p, x, g, y, ydt, s) : go_y<float, false>(h, p, x, g, y, ydt, s);
}

}  // namespace sl
