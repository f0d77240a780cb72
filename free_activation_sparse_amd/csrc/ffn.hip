// Sparse FFN chain for one token (Spark Transformer article, section 2.1: the
// FFN computes its gating scores, selects, and computes only the selected
// part; section 3.1: the product over the active indices):
//
//   g = W_gate x, u = W_up x        each with its own weight-informed gate, in
//                                   one grouped launch (they share x)
//   h = bf16(SiLU(g) * u)           this file: the elementwise epilogue
//   y = W_down h                    with the WINA gate on h (its own K)
//
// The epilogue is one pass over m values (10 bytes each); SiLU(v) =
// v / (1 + exp(-v)) in fp32, then one round to nearest even into bf16, the
// dtype of the down projection's input.
#include "device_common.h"
#include "internal.h"

namespace {

using namespace sl::dev;

__global__ __launch_bounds__(256) void silu_mul_kernel(const float* __restrict__ g, const float* __restrict__ u,
                                                       uint16_t* __restrict__ h, int m) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < m) {
    const float v = g[i];
    const float s = v / (1.0f + expf(-v));
    h[i] = f32_to_bf16(s * u[i]);
  }
}

}  // namespace

namespace sl {

hipError_t launch_silu_mul(const float* g, const float* u, uint16_t* h, int64_t m, hipStream_t s) {
  silu_mul_kernel<<<(unsigned)((m + 255) / 256), 256, 0, s>>>(g, u, h, (int)m);
  return hipGetLastError();
}

}  // namespace sl
