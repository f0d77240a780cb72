// Init-time kernels: weight repack to the column-major layout and the fp64
// column-norm vector.
//
// Layout: the index-list product of the Spark Transformer article (section
// 3.1) reads one whole weight vector per active input; storing W column-major
// ([n][m], column j contiguous) makes each such vector one contiguous run of m
// elements, which the product kernels stream with 16-byte loads.
#include "internal.h"

namespace {

// 64x64 tiled transpose through LDS: W row-major [m][n] -> Wt [n][m].
template <typename T>
__global__ __launch_bounds__(256) void repack_kernel(const T* __restrict__ W, T* __restrict__ Wt,
                                                     int64_t m, int64_t n) {
  __shared__ T tile[64][65];
  const int64_t j0 = (int64_t)blockIdx.x * 64;  // input (column) block
  const int64_t i0 = (int64_t)blockIdx.y * 64;  // output (row) block
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
  for (int r = ty; r < 64; r += 4) {
    const int64_t i = i0 + r, j = j0 + tx;
    if (i < m && j < n) tile[r][tx] = W[i * n + j];
  }
  __syncthreads();
#pragma unroll
  for (int r = ty; r < 64; r += 4) {
    const int64_t j = j0 + r, i = i0 + tx;
    if (i < m && j < n) Wt[j * m + i] = tile[tx][r];
  }
}

__device__ inline double sq_f64(float v) { return (double)v * (double)v; }

// One wavefront per column: c_j = fp32(sqrt(sum_i W[i][j]^2)), fp64 sum.
// Squares of bf16/fp32 values are exact in fp64.
template <typename T>
__global__ __launch_bounds__(256) void norms_kernel(const T* __restrict__ Wt, float* __restrict__ c,
                                                    int64_t m, int64_t n) {
  const int lane = threadIdx.x & 63;
  const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= n) return;
  const T* col = Wt + j * m;
  double acc = 0.0;
  for (int64_t i = lane; i < m; i += 64) {
    float v;
    if constexpr (sizeof(T) == 2) {
      v = __uint_as_float((uint32_t)col[i] << 16);
    } else {
      v = col[i];
    }
    acc += sq_f64(v);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) acc += __shfl_xor(acc, d, 64);
  if (lane == 0) c[j] = __double2float_rn(sqrt(acc));
}

}  // namespace

namespace sl {

hipError_t launch_repack(const void* W, sl_dtype dt, int64_t m, int64_t n, void* Wt, hipStream_t s) {
  dim3 grid((unsigned)((n + 63) / 64), (unsigned)((m + 63) / 64));
  if (dt == SL_BF16) {
    repack_kernel<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)W, (uint16_t*)Wt, m, n);
  } else {
    repack_kernel<float><<<grid, 256, 0, s>>>((const float*)W, (float*)Wt, m, n);
  }
  return hipGetLastError();
}

hipError_t launch_norms(const void* Wt, sl_dtype dt, int64_t m, int64_t n, float* c, hipStream_t s) {
  dim3 grid((unsigned)((n + 3) / 4));
  if (dt == SL_BF16) {
    norms_kernel<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)Wt, c, m, n);
  } else {
    norms_kernel<float><<<grid, 256, 0, s>>>((const float*)Wt, c, m, n);
  }
  return hipGetLastError();
}

}  // namespace sl
