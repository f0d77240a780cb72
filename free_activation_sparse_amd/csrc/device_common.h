// Device helpers shared by the gfx950 kernels (gate, product, union product).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Per-workgroup timestamps of the fused forward, compiled in only for the
// timeline build of the library (fused.hip compiled with SL_TIMELINE): word
// 32 * b + slot of the buffer that sparse_linear_set_timeline installs gets
// workgroup b's value for that slot. In every other build the macros expand
// to nothing and their arguments are not evaluated.
// A function that records declares SL_TL_DECL once at its top: the buffer
// address is then read once, before the weight stream starts, and kept in a
// register (read at every point, it was reloaded after each barrier, and each
// reload waited behind the stream).
#ifdef SL_TIMELINE
static __device__ unsigned long long* sl_timeline_buf = nullptr;
#define SL_TL_DECL unsigned long long* const sl_tl_ = sl_timeline_buf
#define SL_TL_AT(slot, cond, value)                                                    \
  do {                                                                                  \
    if (sl_tl_ != nullptr && (cond)) sl_tl_[(size_t)blockIdx.x * 32 + (slot)] = (value); \
  } while (0)
#define SL_TL_WAIT() __builtin_amdgcn_s_waitcnt(0)
#else
#define SL_TL_DECL ((void)0)
#define SL_TL_AT(slot, cond, value) ((void)0)
#define SL_TL_WAIT() ((void)0)
#endif
// thread 0's clock (100 MHz) at this point
#define SL_TL(slot) SL_TL_AT(slot, threadIdx.x == 0, __builtin_amdgcn_s_memrealtime())

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

// Index of this thread's wavefront in its workgroup, as a wavefront-uniform
// (scalar) value: branches on it are then plain scalar branches. Left as
// threadIdx.x / 64 the compiler treats them as lane-divergent and may place
// register copies in exec-masked code that the other wavefronts skip.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Number of lanes below this one whose bit is set in a wave-wide ballot.
__device__ __forceinline__ uint32_t lanes_below(uint64_t bal) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
}

// Cross-lane moves over DPP (data-parallel primitives): row_shr:k shifts
// within rows of 16 lanes, row_bcast:15 / row_bcast:31 pass lane 15 of each
// row (lane 31) on to the next row(s). Lanes whose source lies outside the
// row keep `old`.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_move(uint32_t v, uint32_t old = 0u) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, 0xf, 0xf, false);
}

// Inclusive prefix sum over the 64 lanes of a wavefront (all lanes active).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const uint32_t lane = threadIdx.x & 63u, rl = lane & 15u;
  uint32_t t;
  t = dpp_move<0x111>(v); if (rl >= 1u) v += t;   // row_shr:1
  t = dpp_move<0x112>(v); if (rl >= 2u) v += t;   // row_shr:2
  t = dpp_move<0x114>(v); if (rl >= 4u) v += t;   // row_shr:4
  t = dpp_move<0x118>(v); if (rl >= 8u) v += t;   // row_shr:8
  t = dpp_move<0x142>(v); if ((lane & 31u) >= 16u) v += t;  // row_bcast:15
  t = dpp_move<0x143>(v); if (lane >= 32u) v += t;          // row_bcast:31
  return v;
}

// Wavefront-uniform sum and maximum (all lanes active).
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(v), 63);
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  const uint32_t lane = threadIdx.x & 63u, rl = lane & 15u;
  uint32_t t;
  t = dpp_move<0x111>(v); if (rl >= 1u) v = max(v, t);
  t = dpp_move<0x112>(v); if (rl >= 2u) v = max(v, t);
  t = dpp_move<0x114>(v); if (rl >= 4u) v = max(v, t);
  t = dpp_move<0x118>(v); if (rl >= 8u) v = max(v, t);
  t = dpp_move<0x142>(v); if ((lane & 31u) >= 16u) v = max(v, t);
  t = dpp_move<0x143>(v); if (lane >= 32u) v = max(v, t);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Sum over each aligned group of 16 lanes, valid in the group's last lane.
__device__ __forceinline__ uint32_t row16_sum_in_last(uint32_t v) {
  const uint32_t rl = threadIdx.x & 15u;
  uint32_t t;
  t = dpp_move<0x111>(v); if (rl >= 1u) v += t;
  t = dpp_move<0x112>(v); if (rl >= 2u) v += t;
  t = dpp_move<0x114>(v); if (rl >= 4u) v += t;
  t = dpp_move<0x118>(v); if (rl >= 8u) v += t;
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
