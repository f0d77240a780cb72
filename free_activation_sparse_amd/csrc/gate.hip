// Gate kernel: one 1024-thread workgroup per token computes the scores
// score_j = |x_j * c_j| (WINA article, section 一), decides the token's kept
// set and publishes it as a threshold pair (kthr, jlast); the product kernels
// re-evaluate the same predicate on their own input chunks.
//
//  * Top-K (WINA article, section 一): radix select of the K-th largest score
//    on its fp32 bit pattern, digits of 12, 12 and 7 bits with LDS histograms,
//    then the rank of the last kept tie in index order by wavefront ballots.
//  * Statistical threshold (Spark Transformer article, section 2.2): mean and
//    population variance of the scores in double-double arithmetic, each
//    rounded once to fp64; sigma by IEEE sqrt; t = fl(mu + fl(sigma * z)).
//  * Fixed threshold: kthr from the per-layer tau (WINA article, section 三,
//    calibrated per-layer thresholds).
//
// Element i of the token is held by thread (i mod 1024) in register slot
// (i / 1024), so every global load is one coalesced row of the token.
#include "device_common.h"
#include "internal.h"

#pragma clang fp contract(off)

namespace {

using namespace sl::dev;

constexpr int GT = 1024;      // threads per gate workgroup
constexpr int GW = GT / 64;   // wavefronts per gate workgroup
constexpr int MODE_TOPK = 0, MODE_STAT = 1, MODE_FIXED = 2;

// ---------------------------------------------------------------- scans
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  uint32_t off = 0;
  for (int k = 0; k < w; ++k) off += wsum[k];
  return inc + off;
}

// Find bin b of an NB-bin histogram such that (count of bins above b) < r <=
// (count of bins above b) + hist[b]. Writes res[0] = b, res[1] = count above.
template <int NB>
__device__ void find_bin(const uint32_t* hist, uint32_t r, uint32_t* wsum, uint32_t* res) {
  constexpr int BPT = (NB + GT - 1) / GT;
  const int t = threadIdx.x;
  uint32_t cnt[BPT];
  uint32_t L = 0;
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    const int b = NB - 1 - (t * BPT + q);
    cnt[q] = (b >= 0) ? hist[b] : 0u;
    L += cnt[q];
  }
  const uint32_t incl = block_incl_scan(L, wsum);
  const uint32_t excl = incl - L;
  if (excl < r && r <= incl) {
    uint32_t cum = excl;
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      if (cum + cnt[q] >= r) {
        res[0] = (uint32_t)(NB - 1 - (t * BPT + q));
        res[1] = cum;
        break;
      }
      cum += cnt[q];
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------- double-double
struct dd {
  double hi, lo;
};

__device__ __forceinline__ dd two_sum(double a, double b) {
  const double s = a + b;
  const double bb = s - a;
  const double e = (a - (s - bb)) + (b - bb);
  return {s, e};
}
__device__ __forceinline__ dd fast_two_sum(double a, double b) {
  const double s = a + b;
  return {s, b - (s - a)};
}
__device__ __forceinline__ dd dd_add(dd a, dd b) {
  const dd s = two_sum(a.hi, b.hi);
  const dd t = two_sum(a.lo, b.lo);
  dd u = fast_two_sum(s.hi, s.lo + t.hi);
  return fast_two_sum(u.hi, u.lo + t.lo);
}
__device__ __forceinline__ dd dd_div(dd a, double b) {
  const double q1 = a.hi / b;
  double r = fma(-q1, b, a.hi);  // exact remainder
  r = r + a.lo;
  const double q2 = r / b;
  return fast_two_sum(q1, q2);
}
__device__ __forceinline__ dd dd_sqr(dd a) {
  const double p = a.hi * a.hi;
  double e = fma(a.hi, a.hi, -p);  // exact error of the product
  e = e + 2.0 * a.hi * a.lo;
  return fast_two_sum(p, e);
}
__device__ __forceinline__ dd shfl_xor_dd(dd v, int d) {
  return {__shfl_xor(v.hi, d, 64), __shfl_xor(v.lo, d, 64)};
}

// Threshold t (>= 0 keeps score > t; < 0 keeps everything) as a key pair.
__device__ __forceinline__ void thresh_to_key(double t, int n, uint32_t& kthr, int& jlast) {
  if (t < 0.0) {
    kthr = 0u;
    jlast = n - 1;
  } else {
    // largest fp32 <= t: for fp32 s, s > t  <=>  s > round_down_f32(t)
    kthr = __float_as_uint(__double2float_rz(t)) & 0x7fffffffu;
    jlast = -1;
  }
}

template <typename XT, int E, int MODE>
__global__ __launch_bounds__(GT) void gate_kernel(const XT* __restrict__ x, const float* __restrict__ c,
                                                  int n, int K, double z, float tau,
                                                  sl::GateOut* __restrict__ gout,
                                                  uint8_t* __restrict__ mask_out,
                                                  int32_t* __restrict__ count_out,
                                                  double* __restrict__ thresh_out) {
  __shared__ uint32_t h1[MODE == MODE_TOPK ? 4096 : 1];
  __shared__ uint32_t h2[MODE == MODE_TOPK ? 4096 : 1];
  __shared__ uint32_t h3[MODE == MODE_TOPK ? 128 : 1];
  __shared__ uint32_t table[MODE == MODE_TOPK ? E * GW : 1];
  __shared__ uint32_t wsum[GW];
  __shared__ uint32_t res[4];
  __shared__ dd dsum[GW][2];
  __shared__ uint32_t kminmax[GW][2];
  __shared__ uint32_t s_kthr;
  __shared__ int s_jlast;

  const int b = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const XT* xb = x + (size_t)b * n;

  if constexpr (MODE == MODE_TOPK) {
    for (int i = t; i < 4096; i += GT) {
      h1[i] = 0u;
      h2[i] = 0u;
    }
    if (t < 128) h3[t] = 0u;
  }

  uint32_t key[E];
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const int i = r * GT + t;
    key[r] = (i < n) ? score_key(load_elem(xb + i), c[i]) : 0u;
  }

  uint32_t kthr = 0xffffffffu;
  int jlast = -1;
  int count = 0;
  double thresh = 0.0;

  if constexpr (MODE == MODE_TOPK) {
    count = K;
    if (K == 0) {
      thresh = __longlong_as_double(0x7ff0000000000000ll);  // +inf: nothing kept
    } else {
      __syncthreads();  // histograms cleared
      // pass 1: bits 30..19
#pragma unroll
      for (int r = 0; r < E; ++r)
        if (r * GT + t < n) atomicAdd(&h1[key[r] >> 19], 1u);
      __syncthreads();
      find_bin<4096>(h1, (uint32_t)K, wsum, res);
      const uint32_t b1 = res[0];
      uint32_t rr = (uint32_t)K - res[1];
      // pass 2: bits 18..7 among keys whose bits 30..19 equal b1
#pragma unroll
      for (int r = 0; r < E; ++r)
        if (r * GT + t < n && (key[r] >> 19) == b1) atomicAdd(&h2[(key[r] >> 7) & 0xfffu], 1u);
      __syncthreads();
      find_bin<4096>(h2, rr, wsum, res);
      const uint32_t p2 = (b1 << 12) | res[0];
      rr -= res[1];
      // pass 3: bits 6..0
#pragma unroll
      for (int r = 0; r < E; ++r)
        if (r * GT + t < n && (key[r] >> 7) == p2) atomicAdd(&h3[key[r] & 0x7fu], 1u);
      __syncthreads();
      find_bin<128>(h3, rr, wsum, res);
      const uint32_t vstar = (p2 << 7) | res[0];
      const uint32_t need = rr - res[1];  // ties at vstar to keep, lowest index first (>= 1)

      // rank of each tie in index order: per-(slot, wavefront) counts, scanned
#pragma unroll
      for (int r = 0; r < E; ++r) {
        const bool p = (r * GT + t < n) && key[r] == vstar;
        const uint64_t bal = __ballot(p);
        if (lane == 0) table[r * GW + w] = (uint32_t)__popcll(bal);
      }
      __syncthreads();
      if (w == 0) {
        constexpr int NT = E * GW;
        constexpr int PER = (NT + 63) / 64;
        uint32_t v[PER];
        uint32_t s = 0;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
          const int idx = lane * PER + q;
          v[q] = idx < NT ? table[idx] : 0u;
          s += v[q];
        }
        uint32_t run = wave_incl_scan(s) - s;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
          const int idx = lane * PER + q;
          if (idx < NT) table[idx] = run;
          run += v[q];
        }
      }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < E; ++r) {
        const int i = r * GT + t;
        const bool p = (i < n) && key[r] == vstar;
        const uint64_t bal = __ballot(p);
        if (p && table[r * GW + w] + lanes_below(bal) == need - 1u) res[2] = (uint32_t)i;
      }
      __syncthreads();
      kthr = vstar;
      jlast = (int)res[2];
      thresh = (double)__uint_as_float(vstar);
    }
  } else {
    if constexpr (MODE == MODE_STAT) {
      // per-thread cascaded sums of s and s^2 (s^2 of an fp32 value is exact in fp64)
      double a1 = 0.0, e1 = 0.0, a2 = 0.0, e2 = 0.0;
      uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
      for (int r = 0; r < E; ++r) {
        if (r * GT + t < n) {
          const double s = (double)__uint_as_float(key[r]);
          dd p = two_sum(a1, s);
          a1 = p.hi;
          e1 = e1 + p.lo;
          p = two_sum(a2, s * s);
          a2 = p.hi;
          e2 = e2 + p.lo;
          kmin = min(kmin, key[r]);
          kmax = max(kmax, key[r]);
        }
      }
      dd S1 = fast_two_sum(a1, e1), S2 = fast_two_sum(a2, e2);
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) {
        S1 = dd_add(S1, shfl_xor_dd(S1, d));
        S2 = dd_add(S2, shfl_xor_dd(S2, d));
        kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, d, 64));
        kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, d, 64));
      }
      if (lane == 0) {
        dsum[w][0] = S1;
        dsum[w][1] = S2;
        kminmax[w][0] = kmin;
        kminmax[w][1] = kmax;
      }
      __syncthreads();
      if (t == 0) {
        dd T1 = dsum[0][0], T2 = dsum[0][1];
        uint32_t lo = kminmax[0][0], hi = kminmax[0][1];
        for (int k = 1; k < GW; ++k) {
          T1 = dd_add(T1, dsum[k][0]);
          T2 = dd_add(T2, dsum[k][1]);
          lo = min(lo, kminmax[k][0]);
          hi = max(hi, kminmax[k][1]);
        }
        const double nd = (double)n;
        const dd mu = dd_div(T1, nd);
        double var;
        double mean = mu.hi;
        if (lo == hi) {  // all scores equal: exact mean, zero variance
          mean = (double)__uint_as_float(lo);
          var = 0.0;
        } else {
          const dd ex2 = dd_div(T2, nd);
          const dd msq = dd_sqr(mu);
          const dd v = dd_add(ex2, dd{-msq.hi, -msq.lo});
          var = v.hi > 0.0 ? v.hi : 0.0;
        }
        const double sigma = sqrt(var);
        const double tt = __dadd_rn(mean, __dmul_rn(sigma, z));
        uint32_t kt;
        int jl;
        thresh_to_key(tt, n, kt, jl);
        s_kthr = kt;
        s_jlast = jl;
        dsum[0][0].hi = tt;
      }
      __syncthreads();
      kthr = s_kthr;
      jlast = s_jlast;
      thresh = dsum[0][0].hi;
    } else {  // MODE_FIXED
      thresh = (double)tau;
      thresh_to_key(thresh, n, kthr, jlast);
    }
    if (count_out != nullptr) {
      uint32_t local = 0;
#pragma unroll
      for (int r = 0; r < E; ++r) {
        const int i = r * GT + t;
        local += (i < n && gate_keep(key[r], i, kthr, jlast)) ? 1u : 0u;
      }
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) local += (uint32_t)__shfl_xor((int)local, d, 64);
      if (lane == 0) wsum[w] = local;
      __syncthreads();
      uint32_t tot = 0;
      for (int k = 0; k < GW; ++k) tot += wsum[k];
      count = (int)tot;
    }
  }

  if (mask_out != nullptr) {
    uint8_t* mb = mask_out + (size_t)b * n;
#pragma unroll
    for (int r = 0; r < E; ++r) {
      const int i = r * GT + t;
      if (i < n) mb[i] = gate_keep(key[r], i, kthr, jlast) ? 1 : 0;
    }
  }
  if (t == 0) {
    sl::GateOut g;
    g.kthr = kthr;
    g.jlast = jlast;
    g.count = count;
    g.pad = 0;
    g.thresh = thresh;
    gout[b] = g;
    if (count_out != nullptr) count_out[b] = count;
    if (thresh_out != nullptr) thresh_out[b] = thresh;
  }
}

template <typename XT, int E>
hipError_t launch_e(const sl_linear* h, const void* x, int B, uint8_t* mask, int32_t* cnt, double* th,
                    hipStream_t s) {
  const XT* xp = (const XT*)x;
  const int n = (int)h->n;
  switch (h->gate) {
    case SL_GATE_TOPK:
      gate_kernel<XT, E, MODE_TOPK><<<B, GT, 0, s>>>(xp, h->c, n, (int)h->K, h->z, h->tau, h->gout, mask, cnt, th);
      break;
    case SL_GATE_STAT:
      gate_kernel<XT, E, MODE_STAT><<<B, GT, 0, s>>>(xp, h->c, n, (int)h->K, h->z, h->tau, h->gout, mask, cnt, th);
      break;
    default:
      gate_kernel<XT, E, MODE_FIXED><<<B, GT, 0, s>>>(xp, h->c, n, (int)h->K, h->z, h->tau, h->gout, mask, cnt, th);
      break;
  }
  return hipGetLastError();
}

template <typename XT>
hipError_t launch_t(const sl_linear* h, const void* x, int B, uint8_t* mask, int32_t* cnt, double* th,
                    hipStream_t s) {
  const int e = (int)((h->n + GT - 1) / GT);
  if (e <= 1) return launch_e<XT, 1>(h, x, B, mask, cnt, th, s);
  if (e <= 2) return launch_e<XT, 2>(h, x, B, mask, cnt, th, s);
  if (e <= 4) return launch_e<XT, 4>(h, x, B, mask, cnt, th, s);
  if (e <= 8) return launch_e<XT, 8>(h, x, B, mask, cnt, th, s);
  if (e <= 12) return launch_e<XT, 12>(h, x, B, mask, cnt, th, s);
  if (e <= 16) return launch_e<XT, 16>(h, x, B, mask, cnt, th, s);
  if (e <= 20) return launch_e<XT, 20>(h, x, B, mask, cnt, th, s);
  if (e <= 24) return launch_e<XT, 24>(h, x, B, mask, cnt, th, s);
  return launch_e<XT, 32>(h, x, B, mask, cnt, th, s);
}

}  // namespace

namespace sl {

hipError_t launch_gate(const sl_linear* h, const void* x, int B, uint8_t* mask_out, int32_t* count_out,
                       double* thresh_out, hipStream_t s) {
  if (h->wdt == SL_BF16) return launch_t<uint16_t>(h, x, B, mask_out, count_out, thresh_out, s);
  return launch_t<float>(h, x, B, mask_out, count_out, thresh_out, s);
}

}  // namespace sl
