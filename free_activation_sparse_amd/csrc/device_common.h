// Device helpers shared by the gfx950 kernels (gate, product, union product).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sl {
namespace dev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Widening loads of one input element (bf16 stored as raw 16-bit patterns).
__device__ __forceinline__ float load_elem(const uint16_t* p) {
  return __uint_as_float((uint32_t)(*p) << 16);
}
__device__ __forceinline__ float load_elem(const float* p) { return *p; }

// score_j = |x_j * c_j| as an fp32 bit pattern. The sign bit is always clear,
// so unsigned comparison of keys is numeric comparison of scores.
__device__ __forceinline__ uint32_t score_key(float xv, float cv) {
  return __float_as_uint(fabsf(xv) * fabsf(cv));
}

__device__ __forceinline__ bool gate_keep(uint32_t key, int j, uint32_t kthr, int jlast) {
  return key > kthr || (key == kthr && j <= jlast);
}

// Number of lanes below this one whose bit is set in a wave-wide ballot.
__device__ __forceinline__ uint32_t lanes_below(uint64_t bal) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_out(uint16_t* p, float v) { *p = f32_to_bf16(v); }

// acc[0..VEC) += xs * w, where w holds one 16-byte run of weights.
__device__ __forceinline__ void fma_run(float (&acc)[8], u32x4 w, float xs) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t b = w[q];
    acc[2 * q] = fmaf(xs, __uint_as_float(b << 16), acc[2 * q]);
    acc[2 * q + 1] = fmaf(xs, __uint_as_float(b & 0xffff0000u), acc[2 * q + 1]);
  }
}
__device__ __forceinline__ void fma_run(float (&acc)[4], u32x4 w, float xs) {
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = fmaf(xs, __uint_as_float(w[q]), acc[q]);
}

}  // namespace dev
}  // namespace sl
