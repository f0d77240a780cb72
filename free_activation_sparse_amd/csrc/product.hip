// Single-token product kernel: y = sum over kept j of x_j * W[:, j].
//
// This is the index-list product of the Spark Transformer article (section
// 3.1): only the weight vectors of active inputs are read. W is column-major,
// so each kept input contributes one contiguous run of m weights; the grid is
// (row tiles) x (input chunks) and every workgroup
//   1. re-evaluates the gate predicate for its chunk of inputs from x, c and
//      the gate's (kthr, jlast) pair, and compacts the kept inputs into LDS in
//      ascending order with wavefront ballots (no global index list),
//   2. streams the kept columns' row-tile runs with 16-byte non-temporal loads:
//      each lane group owns every CS-th kept column and issues up to U of its
//      loads before consuming any, so a workgroup's whole share is in flight
//      after one pass; fp32 accumulation,
//   3. reduces its column slots in LDS and adds its partial into y:
//        ATOMIC    fp32 atomic adds into y (zeroed by the previous kernel in
//                  the stream); one memory round trip, summation order varies;
//        otherwise device-coherent partial stores, then the last workgroup of
//                  the tile to arrive (device-scope arrival counter) adds the
//                  partials in a fixed order: reproducible to the bit, and the
//                  path for bf16 outputs.
#include "device_common.h"
#include "internal.h"

namespace {

using namespace sl::dev;

constexpr int PT = 256;  // threads per product workgroup (4 wavefronts)

template <typename WT, typename YT, int LPC, int U, bool DENSE, bool ATOMIC>
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
  constexpr int ROUNDS = sl::kMaxChunk / PT; // predicate rounds at the largest chunk
  __shared__ int2 list[sl::kMaxChunk];
  __shared__ uint32_t wcnt[ROUNDS][4];
  __shared__ float red[CS * R];
  __shared__ uint32_t s_last;

  const int tile = blockIdx.x % tiles;
  const int split = blockIdx.x / tiles;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int j0 = split * chunk;
  const int j1 = min(j0 + chunk, n);

  // 1. kept inputs of this chunk, ascending, as (j, x_j) pairs in LDS; all
  //    x and c loads of the chunk are issued before the first ballot
  uint32_t kthr = 0u;
  int jlast = 0;
  if (!DENSE) {
    kthr = gout->kthr;
    jlast = gout->jlast;
  }
  const int nr = (j1 - j0 + PT - 1) / PT;
  float xv[ROUNDS];
  uint32_t kv[ROUNDS];
#pragma unroll
  for (int q = 0; q < ROUNDS; ++q) {
    // unconditional loads (index clamped into the chunk) so all are in flight
    const int j = j0 + q * PT + t;
    const int jc = j < j1 ? j : j1 - 1;
    xv[q] = load_elem(x + jc);
    kv[q] = DENSE ? 0u : score_key(xv[q], c[jc]);
  }
  uint64_t bal[ROUNDS];
#pragma unroll
  for (int q = 0; q < ROUNDS; ++q) {
    const int j = j0 + q * PT + t;
    const bool keep = q < nr && j < j1 && (DENSE || gate_keep(kv[q], j, kthr, jlast));
    bal[q] = __ballot(keep);
    if (lane == 0) wcnt[q][w] = (uint32_t)__popcll(bal[q]);
  }
  __syncthreads();
  int cnt = 0;
#pragma unroll
  for (int q = 0; q < ROUNDS; ++q) {
    if (q < nr) {
      uint32_t off = (uint32_t)cnt;
      for (int k = 0; k < w; ++k) off += wcnt[q][k];
      if ((bal[q] >> lane) & 1ull)
        list[off + lanes_below(bal[q])] = make_int2(j0 + q * PT + t, __float_as_int(xv[q]));
      cnt += (int)(wcnt[q][0] + wcnt[q][1] + wcnt[q][2] + wcnt[q][3]);
    }
  }
  __syncthreads();

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
      int2 e[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = k0 + u * CS;
        e[u] = list[k < cnt ? k : k0];
      }
      u32x4 wv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (k0 + u * CS < cnt)
          wv[u] = __builtin_nontemporal_load((const u32x4*)(base + (size_t)e[u].x * (size_t)m));
        else
          wv[u] = u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) fma_run(acc, wv[u], k0 + u * CS < cnt ? __int_as_float(e[u].y) : 0.f);
    }
  }

  // 3. reduce column slots in a fixed order
#pragma unroll
  for (int v = 0; v < VEC; ++v) red[slot * R + sub * VEC + v] = acc[v];
  __syncthreads();
  constexpr int RQ = (R + PT - 1) / PT;
  float part[RQ];
#pragma unroll
  for (int q = 0; q < RQ; ++q) {
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
    for (int q = 0; q < RQ; ++q) {
      const int r = t + q * PT;
      const int gr = tile * R + r;
      if (r < R && gr < m) store_out(y + gr, part[q]);
    }
    return;
  }

  if constexpr (ATOMIC) {
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      const int r = t + q * PT;
      const int gr = tile * R + r;
      if (r < R && gr < m) atomicAdd((float*)(y + gr), part[q]);
    }
    return;
  } else {
    // Ordered reduction without cache-wide fences: partial sums are written with
    // device-coherent stores, each workgroup waits for its stores to complete
    // before it bumps the tile's arrival counter, and the last arrival reads the
    // partials with device-coherent loads.
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      const int r = t + q * PT;
      const int gr = tile * R + r;
      if (r < R && gr < m)
        __hip_atomic_store(partials + (size_t)split * m + gr, part[q], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t == 0)
      s_last = (__hip_atomic_fetch_add(&ctr[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                (uint32_t)(splits - 1))
                   ? 1u
                   : 0u;
    __syncthreads();
    if (s_last == 0u) return;
    // Thread t sums, for row (t mod RW), the splits g, g+G, g+2G, ... with
    // g = t / RW (G groups), eight loads in flight at a time; the G group sums
    // are then added in group order.
    constexpr int RW = R < PT ? R : PT;
    constexpr int G = PT / RW;
    float* gsum = red;  // reuse: [G][R]
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      const int r = (t % RW) + q * RW;
      const int g = t / RW;
      const int gr = tile * R + r;
      float sacc = 0.f;
      if (r < R && gr < m) {
        const float* pp = partials + gr;
        int k = g;
        for (; k + 7 * G < splits; k += 8 * G) {
          float v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            v[u] = __hip_atomic_load(pp + (size_t)(k + u * G) * m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
          for (int u = 0; u < 8; ++u) sacc += v[u];
        }
        for (; k < splits; k += G)
          sacc += __hip_atomic_load(pp + (size_t)k * m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (G > 1) {
        gsum[g * R + r] = sacc;
        __syncthreads();
        if (g == 0 && r < R && gr < m) {
          float tot = 0.f;
#pragma unroll
          for (int hh = 0; hh < G; ++hh) tot += gsum[hh * R + r];
          store_out(y + gr, tot);
        }
      } else if (r < R && gr < m) {
        store_out(y + gr, sacc);
      }
    }
    if (t == 0) __hip_atomic_store(&ctr[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
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
