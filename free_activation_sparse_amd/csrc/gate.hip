// Gate kernel: one 1024-thread workgroup per token computes the scores
// score_j = |x_j * c_j| (WINA article, section 一), decides the token's kept
// set and publishes it as a threshold pair (kthr, jlast); the product kernels
// re-evaluate the same predicate on their own input chunks. The selection
// itself lives in gate_body.h.
#include "gate_body.h"

namespace {

using namespace sl::gatedev;

template <typename XT, int G, int MODE>
__global__ __launch_bounds__(GT) void gate_kernel(const XT* __restrict__ x, const float* __restrict__ c, int n,
                                                  int K, double z, float tau, sl::GateOut* __restrict__ gout,
                                                  uint8_t* __restrict__ mask_out, int32_t* __restrict__ count_out,
                                                  double* __restrict__ thresh_out, float* __restrict__ zero_y,
                                                  int m, int vec) {
  __shared__ __align__(16) uint32_t h1[MODE == MODE_TOPK ? 4096 : 1];
  __shared__ __align__(16) uint32_t h2[MODE == MODE_TOPK ? 4096 : 1];
  __shared__ uint32_t h3[MODE == MODE_TOPK ? 128 : 1];
  __shared__ uint64_t cand[MODE == MODE_TOPK ? 64 : 1];
  __shared__ uint32_t wsum[GW];
  __shared__ uint32_t res[4];
  __shared__ Moments mrows[MODE == MODE_STAT ? 4 * GW : 1];
  __shared__ uint32_t kminmax[MODE == MODE_STAT ? GW : 1][2];
  uint32_t kthr;
  int jlast;
  if (vec)
    gate_body<XT, G, MODE, true>(x, c, n, K, z, tau, gout, mask_out, count_out, thresh_out, zero_y, m, h1, h2, h3,
                                 wsum, res, cand, mrows, kminmax, blockIdx.x, kthr, jlast);
  else
    gate_body<XT, G, MODE, false>(x, c, n, K, z, tau, gout, mask_out, count_out, thresh_out, zero_y, m, h1, h2,
                                  h3, wsum, res, cand, mrows, kminmax, blockIdx.x, kthr, jlast);
}

template <typename XT, int G>
hipError_t launch_g(const sl_linear* h, const void* x, int B, uint8_t* mask, int32_t* cnt, double* th, float* zy,
                    hipStream_t s) {
  const XT* xp = (const XT*)x;
  const int n = (int)h->n;
  const int vec = (n % 4 == 0 && ((uintptr_t)x % (4 * sizeof(XT))) == 0) ? 1 : 0;
  switch (h->gate) {
    case SL_GATE_TOPK:
      gate_kernel<XT, G, MODE_TOPK><<<B, GT, 0, s>>>(xp, h->c, n, (int)h->K, h->z, h->tau, h->gout, mask, cnt, th,
                                                     zy, (int)h->m, vec);
      break;
    case SL_GATE_STAT:
      gate_kernel<XT, G, MODE_STAT><<<B, GT, 0, s>>>(xp, h->c, n, (int)h->K, h->z, h->tau, h->gout, mask, cnt, th,
                                                     zy, (int)h->m, vec);
      break;
    default:
      gate_kernel<XT, G, MODE_FIXED><<<B, GT, 0, s>>>(xp, h->c, n, (int)h->K, h->z, h->tau, h->gout, mask, cnt,
                                                      th, zy, (int)h->m, vec);
      break;
  }
  return hipGetLastError();
}

template <typename XT>
hipError_t launch_t(const sl_linear* h, const void* x, int B, uint8_t* mask, int32_t* cnt, double* th, float* zy,
                    hipStream_t s) {
  const int groups = (int)((h->n + 4 * GT - 1) / (4 * GT));  // 1..8 for n <= 32768
  switch (groups) {
    case 1: return launch_g<XT, 1>(h, x, B, mask, cnt, th, zy, s);
    case 2: return launch_g<XT, 2>(h, x, B, mask, cnt, th, zy, s);
    case 3: return launch_g<XT, 3>(h, x, B, mask, cnt, th, zy, s);
    case 4: return launch_g<XT, 4>(h, x, B, mask, cnt, th, zy, s);
    case 5: return launch_g<XT, 5>(h, x, B, mask, cnt, th, zy, s);
    case 6: return launch_g<XT, 6>(h, x, B, mask, cnt, th, zy, s);
    default: return launch_g<XT, 8>(h, x, B, mask, cnt, th, zy, s);
  }
}

// The gates of up to kMaxGroupLinears linears that share their input, for B
// tokens, in one launch: workgroup l * B + b runs linear l's gate on token b
// (each with its own norms, K or keep fraction, state and y to clear).
struct GateGroup {
  const float* c[sl::kMaxGroupLinears];
  int K[sl::kMaxGroupLinears];
  double z[sl::kMaxGroupLinears];
  float tau[sl::kMaxGroupLinears];
  sl::GateOut* gout[sl::kMaxGroupLinears];
  float* zero_y[sl::kMaxGroupLinears];
  int m[sl::kMaxGroupLinears];
};

template <typename XT, int G, int MODE>
__global__ __launch_bounds__(GT) void gate_group_kernel(GateGroup gg, const XT* __restrict__ x, int n, int B,
                                                        int vec) {
  __shared__ __align__(16) uint32_t h1[MODE == MODE_TOPK ? 4096 : 1];
  __shared__ __align__(16) uint32_t h2[MODE == MODE_TOPK ? 4096 : 1];
  __shared__ uint32_t h3[MODE == MODE_TOPK ? 128 : 1];
  __shared__ uint64_t cand[MODE == MODE_TOPK ? 64 : 1];
  __shared__ uint32_t wsum[GW];
  __shared__ uint32_t res[4];
  __shared__ Moments mrows[MODE == MODE_STAT ? 4 * GW : 1];
  __shared__ uint32_t kminmax[MODE == MODE_STAT ? GW : 1][2];
  const int l = (int)blockIdx.x / B, b = (int)blockIdx.x % B;
  uint32_t kthr;
  int jlast;
  if (vec)
    gate_body<XT, G, MODE, true>(x, gg.c[l], n, gg.K[l], gg.z[l], gg.tau[l], gg.gout[l], nullptr, nullptr, nullptr,
                                 gg.zero_y[l], gg.m[l], h1, h2, h3, wsum, res, cand, mrows, kminmax, b, kthr, jlast);
  else
    gate_body<XT, G, MODE, false>(x, gg.c[l], n, gg.K[l], gg.z[l], gg.tau[l], gg.gout[l], nullptr, nullptr,
                                  nullptr, gg.zero_y[l], gg.m[l], h1, h2, h3, wsum, res, cand, mrows, kminmax, b,
                                  kthr, jlast);
}

template <int G>
hipError_t launch_group_g(const sl_linear* const* hs, int count, const void* x, int B, float* const* zero_y,
                          hipStream_t s) {
  GateGroup gg{};
  for (int l = 0; l < count; ++l) {
    gg.c[l] = hs[l]->c;
    gg.K[l] = (int)hs[l]->K;
    gg.z[l] = hs[l]->z;
    gg.tau[l] = hs[l]->tau;
    gg.gout[l] = hs[l]->gout;
    gg.zero_y[l] = zero_y[l];
    gg.m[l] = (int)hs[l]->m;
  }
  const int n = (int)hs[0]->n;
  const int vec = (n % 4 == 0 && ((uintptr_t)x % 8) == 0) ? 1 : 0;
  const uint16_t* xp = (const uint16_t*)x;
  if (hs[0]->gate == SL_GATE_STAT)
    gate_group_kernel<uint16_t, G, MODE_STAT><<<count * B, GT, 0, s>>>(gg, xp, n, B, vec);
  else
    gate_group_kernel<uint16_t, G, MODE_TOPK><<<count * B, GT, 0, s>>>(gg, xp, n, B, vec);
  return hipGetLastError();
}

}  // namespace

namespace sl {

hipError_t launch_gate_group(const sl_linear* const* hs, int count, const void* x, int B, float* const* zero_y,
                             hipStream_t s) {
  switch ((int)((hs[0]->n + 4 * GT - 1) / (4 * GT))) {  // 1..8 for n <= 32768
    case 1: return launch_group_g<1>(hs, count, x, B, zero_y, s);
    case 2: return launch_group_g<2>(hs, count, x, B, zero_y, s);
    case 3: return launch_group_g<3>(hs, count, x, B, zero_y, s);
    case 4: return launch_group_g<4>(hs, count, x, B, zero_y, s);
    case 5: return launch_group_g<5>(hs, count, x, B, zero_y, s);
    case 6: return launch_group_g<6>(hs, count, x, B, zero_y, s);
    default: return launch_group_g<8>(hs, count, x, B, zero_y, s);
  }
}

hipError_t launch_gate(const sl_linear* h, const void* x, int B, uint8_t* mask_out, int32_t* count_out,
                       double* thresh_out, float* zero_y, hipStream_t s) {
  if (h->wdt == SL_BF16) return launch_t<uint16_t>(h, x, B, mask_out, count_out, thresh_out, zero_y, s);
  return launch_t<float>(h, x, B, mask_out, count_out, thresh_out, zero_y, s);
}

}  // namespace sl
