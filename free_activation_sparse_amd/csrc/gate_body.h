// Gate body shared by the gate kernel and the fused gate + product kernel:
// one 1024-thread workgroup computes a token's scores and kept set.
//
//  * Top-K (WINA article, section 一): selection on the scores' fp32 bit
//    patterns (non-negative, so unsigned order is numeric order).
//    Window path (a previous call on this slot left its K-th key): one pass
//    counts the keys above a window around that key and histograms the
//    window's keys into 1024 LDS bins; one wavefront finds the bin holding
//    rank K, whose keys (at most 64) are ranked exactly. Otherwise, or when
//    rank K falls outside the window or in a bin of more than 64 keys:
//    Fast path: a 4096-bin LDS histogram of key>>14 over the eight binades
//    below the largest key (512 bins per binade: few atomic collisions),
//    searched by one wavefront; the pivot bin's keys (at most 64) are
//    compacted with ballots and ranked exactly under the order (score
//    descending, index ascending) by one wavefront.
//    General path (pivot below the window, or more than 64 keys in the pivot
//    bin, i.e. heavy ties): radix select on 12/12/7-bit key digits, then the
//    kept ties' last index by a radix select on the index (8/7 bits).
//  * Statistical threshold (Spark Transformer article, section 2.2): mean and
//    population variance of the scores, each rounded once to fp64; sigma by
//    IEEE sqrt; t = fl(mu + fl(sigma * z)), from the workgroup's own scores.
//    A first threshold from plain fp64 sums comes with a rigorous bound on
//    its distance from the exact t; when no score lies within that bound
//    (almost always) it decides the kept set, and the exact moments (sums
//    in double-double) are only computed for the threshold output or when a
//    score is that close.
//  * Fixed threshold: kthr from the per-layer tau (WINA article, section 三,
//    calibrated per-layer thresholds).
//
// Layout: elements come in groups of 4 consecutive inputs; thread t holds
// groups t, t + 1024, ... (G groups), loaded with vector loads (8 bytes of
// bf16 or 16 bytes of fp32 x, 16 bytes of c) when n is a multiple of 4 and x
// is aligned to its vector, else with scalar loads.
// Every load is unconditional (index clamped, value masked), so all of a
// thread's loads are in flight together.
#pragma once

#include "device_common.h"
#include "internal.h"

#pragma clang fp contract(off)

namespace sl {
namespace gatedev {

using namespace sl::dev;

constexpr int GT = 1024;      // threads per gate workgroup
constexpr int GW = GT / 64;   // wavefronts per gate workgroup
constexpr int MODE_TOPK = 0, MODE_STAT = 1, MODE_FIXED = 2;

// Top-K window select around the previous K-th key (see gate_select): the
// window's edges over the previous K-th score, and its histogram bins.
constexpr float kWinLow = 0.87f, kWinHigh = 1.15f;
constexpr int kWinBins = 1024;

// ---------------------------------------------------------------- scans
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  uint32_t off = 0;
#pragma unroll
  for (int k = 0; k < GW; ++k) off += (k < w) ? wsum[k] : 0u;
  return inc + off;
}

__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_sum(v);
  if (lane == 0) wsum[w] = v;
  __syncthreads();
  uint32_t tot = 0;
#pragma unroll
  for (int k = 0; k < GW; ++k) tot += wsum[k];
  return tot;
}

// Find bin b of an NB-bin histogram such that (count of bins above b) < r <=
// (count of bins above b) + hist[b]. Writes res[0] = b, res[1] = count above;
// leaves res untouched when the histogram holds fewer than r entries.
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

// find_bin for one wavefront (the caller's wavefront 0; all 64 lanes active):
// lane l sums the NB/64 bins NB - (l+1)*NB/64 .. NB - l*NB/64 - 1 (the top
// bins go to lane 0), a wavefront scan finds the lane whose range holds rank
// r, and a second scan over that lane's bins finds the bin. Writes res[0] =
// bin, res[1] = count above it, res[2] = its count; leaves res untouched when
// the histogram holds fewer than r entries. hist must be 16-byte aligned.
// Two dependent LDS round trips instead of a block-wide scan.
template <int NB, int MAXB>
__device__ __forceinline__ void find_bin_wave(const uint32_t* hist, uint32_t r, uint32_t* res) {
  constexpr int PER = NB / 64;  // bins per lane
  static_assert(PER % 4 == 0 && PER <= 64, "bins per lane");
  constexpr int V = PER / 4;
  const int lane = threadIdx.x & 63;
  const uint4* hp = (const uint4*)(hist + (NB - PER * (lane + 1)));
  // reads rotated so that 16 consecutive lanes hit 16 distinct bank groups;
  // issued in batches of up to 8 kept in flight together (bounded registers)
  constexpr int BATCH = V < MAXB ? V : MAXB;
  uint32_t L = 0;
#pragma unroll
  for (int q0 = 0; q0 < V; q0 += BATCH) {
    uint4 v[BATCH];
#pragma unroll
    for (int q = 0; q < BATCH; ++q) v[q] = hp[(q0 + q + lane) & (V - 1)];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < BATCH; ++q) L += v[q].x + v[q].y + v[q].z + v[q].w;
  }
  const uint32_t incl = wave_incl_scan(L);
  const uint32_t excl = incl - L;
  const uint64_t hit = __ballot(excl < r && r <= incl);
  if (hit == 0ull) return;
  const int lf = (int)__builtin_ctzll(hit);
  const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)excl, lf);
  const int b = NB - PER * lf - 1 - lane;  // lane q: the q-th bin of that range, from the top
  const uint32_t cb = lane < PER ? hist[b] : 0u;
  const uint32_t incl2 = wave_incl_scan(cb) + above;
  const uint32_t excl2 = incl2 - cb;
  const uint64_t hit2 = __ballot(lane < PER && excl2 < r && r <= incl2);
  if (lane == (int)__builtin_ctzll(hit2)) {
    res[0] = (uint32_t)b;
    res[1] = excl2;
    res[2] = cb;
  }
}

// Raw (untyped) buffer resources: word 3 of the descriptor on gfx9 parts, and
// the cache-policy operand of a buffer access that sets sc1 alone.
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kPolicySc1 = 16;

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
// 1/b as a double-double (the fma remainder is exact): ~2^-106 relative.
__device__ __forceinline__ dd dd_recip(double b) {
  const double h = 1.0 / b;
  return {h, fma(-h, b, 1.0) / b};
}
// a * r for a double-double reciprocal r: ~2^-104 relative, no division.
__device__ __forceinline__ dd dd_mul(dd a, dd r) {
  const double p = a.hi * r.hi;
  double e = fma(a.hi, r.hi, -p);  // exact error of the product
  e = e + (a.hi * r.lo + a.lo * r.hi);
  return fast_two_sum(p, e);
}
__device__ __forceinline__ dd dd_sqr(dd a) {
  const double p = a.hi * a.hi;
  double e = fma(a.hi, a.hi, -p);  // exact error of the product
  e = e + 2.0 * a.hi * a.lo;
  return fast_two_sum(p, e);
}

// ---------------------------------------------------------------- moments
// Sums of the scores and of their squares, to ~2^-100 relative, far below
// the single rounding to fp64 that the mean and the variance take. Every
// thread adds its E scores onto a power-of-two offset sigma >= E * (the
// workgroup's largest score), the same for all threads: each running sum
// stays in [sigma, 2 sigma), at or above each addend, so Fast2Sum yields
// each rounding error exactly (kept in a plain fp64 error sum), and the
// running sum itself is sigma plus an integer multiple of ulp(sigma), that
// integer being the mantissa field of its bit pattern. Those integers
// (< 2^52 per thread, < 2^62 over a workgroup) then add exactly in uint64,
// and only the tiny error sums round. Squares of fp32 values are exact in
// fp64; keys of 0 add nothing.
struct Moments {
  uint64_t i1, i2;  // sums of the running-sum mantissas (units of ulp(sigma))
  double e1, e2;    // sums of the rounding errors
};

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint64_t lo = dpp_move<CTRL>((uint32_t)v), hi = dpp_move<CTRL>((uint32_t)(v >> 32));
  return (hi << 32) | lo;
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  return __longlong_as_double((long long)dpp_u64<CTRL>((uint64_t)__double_as_longlong(v)));
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return (hi << 32) | lo;
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
  return __longlong_as_double((long long)readlane_u64((uint64_t)__double_as_longlong(v), l));
}
template <int CTRL>
__device__ __forceinline__ void moments_step(Moments& a) {
  a.i1 += dpp_u64<CTRL>(a.i1);
  a.i2 += dpp_u64<CTRL>(a.i2);
  a.e1 += dpp_f64<CTRL>(a.e1);
  a.e2 += dpp_f64<CTRL>(a.e2);
}
// Totals over each row of 16 lanes, in every lane of the row: a butterfly of
// lane swaps (quad_perm [1,0,3,2], [2,3,0,1], then the half-row and the row
// mirrored), each step adding a lane's partner's partial. Needs all lanes
// active.
__device__ __forceinline__ void row_sum_moments(Moments& a) {
  moments_step<0xb1>(a);   // quad_perm [1,0,3,2]
  moments_step<0x4e>(a);   // quad_perm [2,3,0,1]
  moments_step<0x141>(a);  // row_half_mirror
  moments_step<0x140>(a);  // row_mirror
}

// Totals of two doubles over each row of 16 lanes, in every lane of the row
// (the butterfly of row_sum_moments). Needs all lanes active.
__device__ __forceinline__ void row_sum2(double& a, double& b) {
  a += dpp_f64<0xb1>(a);
  b += dpp_f64<0xb1>(b);
  a += dpp_f64<0x4e>(a);
  b += dpp_f64<0x4e>(b);
  a += dpp_f64<0x141>(a);
  b += dpp_f64<0x141>(b);
  a += dpp_f64<0x140>(a);
  b += dpp_f64<0x140>(b);
}

// log2 of the offsets for the largest key kmax: sigma1 >= E * (largest
// score), sigma2 >= E * (its square).
template <int E>
__device__ __forceinline__ void moments_log2_sigma(uint32_t kmax, int& l1, int& l2) {
  constexpr int LE = E <= 1 ? 0 : 32 - __builtin_clz((unsigned)(E - 1));  // ceil(log2 E)
  const int eb = max((int)(kmax >> 23), 1);  // largest score < 2^(eb - 126), its square < 2^(2 eb - 252)
  l1 = eb - 126 + LE;
  l2 = 2 * eb - 252 + LE;
}

// A thread's share over its E keys (key e is input index(e); groups of four
// that lie wholly past n in every lane of the wavefront are skipped: their
// keys are 0). l1, l2: log2 of the workgroup's offsets.
template <int E>
__device__ __forceinline__ Moments thread_moments(const uint32_t (&key)[E], int l1, int l2, int n) {
  const int t = threadIdx.x, w = t >> 6;
  const double sig1 = __longlong_as_double((long long)(l1 + 1023) << 52);
  const double sig2 = __longlong_as_double((long long)(l2 + 1023) << 52);
  double a1 = sig1, e1 = 0.0, a2 = sig2, e2 = 0.0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if ((e & 3) == 0 && ((e >> 2) * GT + 64 * w) * 4 >= n) break;  // wavefront-uniform
    const double s = (double)__uint_as_float(key[e]);
    const double t1 = a1 + s;
    e1 += s - (t1 - a1);
    a1 = t1;
    const double q = s * s;
    const double t2 = a2 + q;
    e2 += q - (t2 - a2);
    a2 = t2;
  }
  constexpr uint64_t kMant = (1ull << 52) - 1ull;
  return {(uint64_t)__double_as_longlong(a1) & kMant, (uint64_t)__double_as_longlong(a2) & kMant, e1, e2};
}

// i * 2^l + e as a double-double (i < 2^62 splits exactly into two doubles;
// scaling by a power of two is exact).
__device__ __forceinline__ dd moments_total(uint64_t i, double e, int l) {
  const double sc = __longlong_as_double((long long)(l + 1023) << 52);
  const double hi = (double)(uint32_t)(i >> 32) * 4294967296.0 * sc;
  const double lo = (double)(uint32_t)i * sc;
  return dd_add(two_sum(hi, lo), dd{e, 0.0});
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

// ---------------------------------------------------------------- clearing
// Zeroes y[0 .. m) from threads tt = 0 .. nt - 1 with device-coherent stores
// (product workgroups on other XCDs add onto the zeros): the body in 16-byte
// buffer stores with the same cache policy as a relaxed agent-scope atomic
// store (sc1), a quarter of the store instructions of a per-float clear; the
// unaligned head and the tail (< 4 floats each) take atomic stores.
__device__ __forceinline__ void clear_coherent(float* yb, int m, int tt, int nt) {
  const int head = min(m, (int)((16u - ((uint32_t)(uintptr_t)yb & 15u)) & 15u) >> 2);
  const int body = (m - head) >> 2;  // 16-byte groups
  const int tail = m - head - 4 * body;
  if (tt < head) __hip_atomic_store(yb + tt, 0.f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tt < tail) __hip_atomic_store(yb + head + 4 * body + tt, 0.f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(yb + head, 0, 16 * body, kRawBufferWord3);
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  for (int i = tt; i < body; i += nt) __builtin_amdgcn_raw_buffer_store_b128(z4, r, 16 * i, 0, kPolicySc1);
}

// ---------------------------------------------------------------- loads
// Keys of group g (4 inputs starting at 4 * (g * GT + t)); out-of-range
// inputs get key 0 and must be masked by the caller with their index.
template <typename XT, bool VEC>
__device__ __forceinline__ void load_group(const XT* __restrict__ xb, const float* __restrict__ c, int n, int g,
                                           uint32_t (&k)[4]) {
  const int base = (g * GT + (int)threadIdx.x) * 4;
  float xv[4], cv[4];
  if constexpr (VEC) {
    const int bc = base < n ? base : 0;  // n % 4 == 0: groups are all-in or all-out
    if constexpr (sizeof(XT) == 2) {
      const uint2 v = *(const uint2*)(xb + bc);
      xv[0] = __uint_as_float(v.x << 16);
      xv[1] = __uint_as_float(v.x & 0xffff0000u);
      xv[2] = __uint_as_float(v.y << 16);
      xv[3] = __uint_as_float(v.y & 0xffff0000u);
    } else {
      const float4 a = *(const float4*)(xb + bc);
      xv[0] = a.x; xv[1] = a.y; xv[2] = a.z; xv[3] = a.w;
    }
    const float4 a = *(const float4*)(c + bc);
    cv[0] = a.x; cv[1] = a.y; cv[2] = a.z; cv[3] = a.w;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = base + e;
      const int ic = i < n ? i : n - 1;
      xv[e] = load_elem(xb + ic);
      cv[e] = c[ic];
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) k[e] = (base + e < n) ? score_key(xv[e], cv[e]) : 0u;
}

// Top-K: the previous call's K-th key for this slot (the prior of the window
// select in gate_select; any value is safe, it only picks the path), and that
// select's histogram (h2) and counters cleared before its keys are used. Ends
// with a barrier when it clears them.
template <int MODE>
__device__ __forceinline__ uint32_t gate_prologue(int K, const sl::GateOut* gout, int b, uint32_t* h2,
                                                  uint32_t* res) {
  uint32_t prevk = 0u;
  if constexpr (MODE == MODE_TOPK) {
    if (K > 0) {
      const int t = threadIdx.x;
      prevk = gout[b].kthr;
      for (int i = t; i < kWinBins; i += GT) h2[i] = 0u;
      if (t == 0) {
        res[0] = 0xffffffffu;
        res[3] = 0u;
      }
      __syncthreads();
    }
  }
  return prevk;
}

// The scores' keys of token b: thread t holds groups t, t + GT, ... of 4
// consecutive inputs (key[4 g + e] is input 4 (g GT + t) + e); 0 past n.
template <typename XT, int G, bool VEC>
__device__ __forceinline__ void gate_keys(const XT* __restrict__ x, const float* __restrict__ c, int n, int b,
                                          uint32_t (&key)[4 * G]) {
  const XT* xb = x + (size_t)b * n;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    uint32_t k4[4];
    load_group<XT, VEC>(xb, c, n, g, k4);
#pragma unroll
    for (int e = 0; e < 4; ++e) key[g * 4 + e] = k4[e];
  }
}

// The selection on keys from gate_keys, with prevk from gate_prologue (which
// must have run, in every thread, before it); outputs as gate_body.
template <int G, int MODE>
__device__ __forceinline__ void gate_select(const uint32_t (&key)[4 * G], uint32_t prevk, int n, int K, double z,
                                            float tau, sl::GateOut* __restrict__ gout,
                                            uint8_t* __restrict__ mask_out, int32_t* __restrict__ count_out,
                                            double* __restrict__ thresh_out, float* __restrict__ zero_y, int m,
                                            uint32_t* h1, uint32_t* h2, uint32_t* h3, uint32_t* wsum,
                                            uint32_t* res, uint64_t* cand, Moments* mrows,
                                            uint32_t (*kminmax)[2], int b, uint32_t& kthr_out, int& jlast_out) {
  SL_TL_DECL;
  constexpr int E = 4 * G;
  const int t = threadIdx.x, lane = t & 63, w = wave_id();
  auto index = [&](int e) { return ((e >> 2) * GT + t) * 4 + (e & 3); };

  // The product that follows adds its split partials into y atomically, so
  // y is cleared here with device-coherent stores (product workgroups of the
  // same launch on other XCDs add onto the zeros). They are issued by
  // wavefronts w_lo.. while wavefront 0 works alone (bin search, final
  // scalar steps): issued right behind the input loads, even as a fixed
  // number of stores per thread, they delayed the keys by ~0.4 us and the
  // top-K selection by ~0.9 us.
  auto clear_y = [&](int w_lo) {
    if (zero_y != nullptr && w >= w_lo) clear_coherent(zero_y + (size_t)b * m, m, t - 64 * w_lo, GT - 64 * w_lo);
  };

  uint32_t kthr = 0xffffffffu;
  int jlast = -1;
  int count = 0;
  double thresh = 0.0;

  if constexpr (MODE == MODE_TOPK) {
    count = K;
    if (K == 0) {
      clear_y(0);
      thresh = __longlong_as_double(0x7ff0000000000000ll);  // +inf: nothing kept
    } else {
      // The r-th (1-based) largest of the c1 <= 64 keys for which in_bin
      // holds, under (score descending, index ascending), into res[1] (key)
      // and res[2] (index): the keys are compacted as (key, ~index)
      // composites (larger composite = earlier in the order; composites are
      // distinct) with one LDS atomic per wavefront reserving its slots
      // (res[3] must be 0), then wavefront 0 ranks them, lane a comparing
      // candidate a with every other through readlane.
      auto rank_bin = [&](auto in_bin, uint32_t c1, uint32_t r) {
        uint64_t bal[E];
        uint32_t wtot = 0u;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          bal[e] = __ballot(in_bin(key[e]));
          wtot += (uint32_t)__popcll(bal[e]);
        }
        if (wtot != 0u) {
          uint32_t off = 0u;
          if (lane == 0) off = atomicAdd(&res[3], wtot);
          off = (uint32_t)__builtin_amdgcn_readfirstlane((int)off);
#pragma unroll
          for (int e = 0; e < E; ++e) {
            if (bal[e] != 0ull) {  // uniform: most slots hold no candidate
              if ((bal[e] >> lane) & 1ull)
                cand[off + lanes_below(bal[e])] = ((uint64_t)key[e] << 32) | (uint64_t)(~(uint32_t)index(e));
              off += (uint32_t)__popcll(bal[e]);
            }
          }
        }
        __syncthreads();
        SL_TL(10);
        if (w == 0) {
          const uint64_t ca = (uint32_t)lane < c1 ? cand[lane] : 0ull;
          const uint32_t chi = (uint32_t)(ca >> 32), clo = (uint32_t)ca;
          uint32_t above = 0u;
          for (int k = 0; k < (int)c1; ++k) {
            const uint64_t o = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)chi, k) << 32) |
                               (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)clo, k);
            above += (o > ca) ? 1u : 0u;
          }
          if ((uint32_t)lane < c1 && above == r - 1u) {
            res[1] = chi;
            res[2] = ~clo;
          }
        }
        __syncthreads();
        SL_TL(11);
      };

      // Window select around the prior: consecutive tokens' K-th scores
      // differ by a few percent, so the K-th key almost always lies in
      // [lo, hi) = [kWinLow, kWinHigh) times the previous one. One pass
      // counts the keys at or above hi (ballots) and histograms the keys in
      // the window into kWinBins bins (LDS atomics: only the window's keys,
      // a fraction of n); one wavefront finds the bin holding rank K, and
      // its keys are ranked exactly. No maximum, no full-range histogram.
      // Falls through to the full select when the K-th key lies outside the
      // window or its bin holds more than 64 keys (heavy ties). (Keeping
      // each bin's largest and smallest composite as well, to skip the
      // ranking when rank K is a bin's first or last entry, cost more in
      // 64-bit LDS atomics than the ranking it saved.)
      bool found = false;
      if (prevk != 0u && prevk < 0x7f800000u) {  // uniform
        const float pf = __uint_as_float(prevk);
        uint32_t hi = __float_as_uint(pf * kWinHigh), lo = __float_as_uint(pf * kWinLow);
        if (hi <= prevk) hi = prevk + 1u;
        if (lo > prevk) lo = prevk;
        if (lo == 0u) lo = 1u;  // padding keys (0) never enter the window
        const uint32_t span = hi - lo;
        const int sh = max(0, 22 - (int)__builtin_clz((span - 1u) | 1u));  // (span - 1) >> sh < kWinBins
        static_assert(kWinBins == 1024, "window shift assumes 1024 bins");
        uint32_t ws = 0u;
        SL_TL(3);  // wavefront 0's keys are in (their first use follows)
#pragma unroll
        for (int e = 0; e < E; ++e) {
          ws += (uint32_t)__popcll(__ballot(key[e] >= hi));
          const uint32_t d = key[e] - lo;  // wraps above span below the window
          if (d < span) atomicAdd(&h2[d >> sh], 1u);
        }
        if (lane == 0) wsum[w] = ws;
        __syncthreads();
        SL_TL(18);
        uint32_t above_hi = 0u;
#pragma unroll
        for (int k = 0; k < GW; ++k) above_hi += wsum[k];
        // (res[0] stays "not found" unless the window holds rank K)
        if (above_hi < (uint32_t)K) {  // uniform
          if (w == 0)
            find_bin_wave<kWinBins, 8>(h2, (uint32_t)K - above_hi, res);
          else
            clear_y(1);
        }
        // every wavefront has read wsum and res[0..2] is final before either
        // path below writes them
        __syncthreads();
        SL_TL(19);
        const uint32_t b1 = res[0], c1 = res[2];
        if (b1 != 0xffffffffu && c1 <= 64u) {  // uniform
          const uint32_t r1 = (uint32_t)K - above_hi - res[1];  // rank inside the bin, 1-based
          rank_bin([&](uint32_t k) { return k - lo < span && ((k - lo) >> sh) == b1; }, c1, r1);
          kthr = res[1];
          jlast = (int)res[2];
          found = true;
        }
      }

      if (!found) {
      for (int i = t; i < 4096; i += GT) h1[i] = 0u;
      uint32_t lmax = 0u;
#pragma unroll
      for (int e = 0; e < E; ++e) lmax = max(lmax, key[e]);  // padding keys are 0
      lmax = wave_max(lmax);
      SL_TL(3);  // wavefront 0's keys are in
      if (lane == 0) wsum[w] = lmax;
      if (t == 0) {
        res[0] = 0xffffffffu;  // "not found" unless find_bin writes it
        res[3] = 0u;           // candidate counter
      }
      __syncthreads();  // h1 cleared, maxima and res published
      SL_TL(7);
      uint32_t kmax = wsum[0];
#pragma unroll
      for (int k = 1; k < GW; ++k) kmax = max(kmax, wsum[k]);
      // window of 4096 bins of key>>14 ending at the largest key's bin; it
      // starts at bin 1 or above, so the padding keys (0) and any real key
      // in bin 0 fall outside it (the general path then takes over)
      const uint32_t top = kmax >> 14;
      const uint32_t base = top >= 4096u ? top - 4095u : 1u;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint32_t d = (key[e] >> 14) - base;  // wraps above 4095 when outside the window
        if (d < 4096u) atomicAdd(&h1[d], 1u);
      }
      __syncthreads();
      SL_TL(8);
      // fewer reads in flight when the keys take many registers
      if (w == 0)
        find_bin_wave<4096, (E <= 16 ? 8 : 2)>(h1, (uint32_t)K, res);
      else
        clear_y(1);
      __syncthreads();
      SL_TL(9);
      const bool in_window = res[0] != 0xffffffffu;
      const uint32_t c1 = in_window ? res[2] : 0u;
      if (in_window && c1 <= 64u) {
        const uint32_t b1 = res[0] + base;         // pivot bin of key>>14 (>= 1: never a padding key's)
        const uint32_t r1 = (uint32_t)K - res[1];  // rank wanted inside the pivot bin, 1-based
        rank_bin([&](uint32_t k) { return (k >> 14) == b1; }, c1, r1);
        kthr = res[1];
        jlast = (int)res[2];
      } else {
        // ---- general path: radix select on key digits 30..19, 18..7, 6..0
        for (int i = t; i < 4096; i += GT) {
          h1[i] = 0u;
          h2[i] = 0u;
        }
        if (t < 128) h3[t] = 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (index(e) < n) atomicAdd(&h1[key[e] >> 19], 1u);
        __syncthreads();
        find_bin<4096>(h1, (uint32_t)K, wsum, res);
        const uint32_t b1 = res[0];
        uint32_t rr = (uint32_t)K - res[1];
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (index(e) < n && (key[e] >> 19) == b1) atomicAdd(&h2[(key[e] >> 7) & 0xfffu], 1u);
        __syncthreads();
        find_bin<4096>(h2, rr, wsum, res);
        const uint32_t p2 = (b1 << 12) | res[0];
        rr -= res[1];
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (index(e) < n && (key[e] >> 7) == p2) atomicAdd(&h3[key[e] & 0x7fu], 1u);
        __syncthreads();
        find_bin<128>(h3, rr, wsum, res);
        const uint32_t vstar = (p2 << 7) | res[0];
        const uint32_t need = rr - res[1];  // ties at vstar to keep, lowest index first (>= 1)
        // the need-th smallest index among keys equal to vstar: bins are
        // stored reversed so that find_bin's descending search runs upwards
        if (t < 256) h2[t] = 0u;
        if (t < 128) h3[t] = 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int i = index(e);
          if (i < n && key[e] == vstar) atomicAdd(&h2[255 - (i >> 7)], 1u);
        }
        __syncthreads();
        find_bin<256>(h2, need, wsum, res);
        const uint32_t hiidx = 255u - res[0];
        const uint32_t need2 = need - res[1];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int i = index(e);
          if (i < n && key[e] == vstar && (uint32_t)(i >> 7) == hiidx) atomicAdd(&h3[127 - (i & 127)], 1u);
        }
        __syncthreads();
        find_bin<128>(h3, need2, wsum, res);
        kthr = vstar;
        jlast = (int)((hiidx << 7) | (127u - res[0]));
      }
      }  // !found
      thresh = (double)__uint_as_float(kthr);
    }
  } else {
    if constexpr (MODE == MODE_STAT) {
      const dd inv_n = dd_recip((double)n);  // early: its divisions stay off the final chain
      // One pass over the keys: the workgroup's extremes and plain fp64 sums
      // of s and s^2 (groups of four wholly past n are skipped: their keys
      // are 0).
      uint32_t kmax = 0u, kmin = 0xffffffffu;
      double f1 = 0.0, f2 = 0.0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if ((e & 3) == 0 && ((e >> 2) * GT + 64 * w) * 4 >= n) break;  // wavefront-uniform
        kmax = max(kmax, key[e]);  // padding keys are 0
        if (index(e) < n) kmin = min(kmin, key[e]);
        const double sv = (double)__uint_as_float(key[e]);
        f1 += sv;
        f2 += sv * sv;
      }
      kmax = wave_max(kmax);
      kmin = ~wave_max(~kmin);
      SL_TL(14);  // wavefront 0's keys are in
      row_sum2(f1, f2);
      if (lane == 0) {
        kminmax[w][0] = kmin;
        kminmax[w][1] = kmax;
      }
      if ((lane & 15) == 0) {
        mrows[4 * w + (lane >> 4)].e1 = f1;
        mrows[4 * w + (lane >> 4)].e2 = f2;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < GW; ++k) {
        kmin = min(kmin, kminmax[k][0]);
        kmax = max(kmax, kminmax[k][1]);
      }
      SL_TL(15);  // the workgroup's extremes and the plain sums' row totals known
      // A first threshold from the plain sums, with a rigorous bound on its
      // distance from the exact one: every sum adds non-negative terms, so
      // each total is within (n - 1) u <= 2^-38 (relative) of the exact sum
      // whatever the order; mu within 2^-36, E[s^2] - mu^2 within 2^-34 E[s^2],
      // sigma within 2^-34 E[s^2] / sigma, and t within
      // del = 2^-32 (mu + |z| sigma + |z| E[s^2] / sigma), a margin of 4 or
      // more over each term (the roundings of the exact t itself included).
      // If no score lies within del of this t, every score compares with
      // it as with the exact t, and the kept set is final; otherwise, for
      // near-constant scores, or when t is not safely positive, the exact
      // moments decide (below).
      clear_y(1);
      if (w == 0) {
        static_assert(4 * GW == 64, "one row total per lane of wavefront 0");
        double g1 = mrows[lane].e1, g2 = mrows[lane].e2;
        row_sum2(g1, g2);
        const double F1 = (readlane_f64(g1, 0) + readlane_f64(g1, 16)) + (readlane_f64(g1, 32) + readlane_f64(g1, 48));
        const double F2 = (readlane_f64(g2, 0) + readlane_f64(g2, 16)) + (readlane_f64(g2, 32) + readlane_f64(g2, 48));
        if (lane == 0) {
          const double mu = F1 * inv_n.hi, e2 = F2 * inv_n.hi;
          const double v = e2 - mu * mu;
          uint32_t ok = (kmin != kmax && v > 0x1p-20 * e2) ? 1u : 0u;
          const double sg = ok ? sqrt(v) : 1.0;
          const double t0 = mu + sg * z;
          const double az = fabs(z);
          const double del = 0x1p-32 * (mu + az * sg + az * (e2 / sg));
          const double lo = t0 - del, hi = t0 + del;
          if (!(lo > 0.0)) ok = 0u;
          res[0] = __float_as_uint(__double2float_rd(lo));
          res[1] = __float_as_uint(__double2float_ru(hi));
          res[2] = __float_as_uint(__double2float_rz(t0)) & 0x7fffffffu;
          res[3] = ok;
          cand[0] = (uint64_t)__double_as_longlong(t0);
        }
      }
      __syncthreads();
      const uint32_t klo = res[0], kspan = res[1] - res[0], kfast = res[2];
      const double tfast = __longlong_as_double((long long)cand[0]);
      bool fast = false;
      if (res[3] != 0u) {  // uniform
        bool amb = false;
#pragma unroll
        for (int e = 0; e < E; ++e) amb |= key[e] - klo <= kspan;  // (padding keys 0 lie below klo > 0)
        // per-wavefront flags in kminmax (read for the last time before the
        // barrier above; wsum is the count's, written without a barrier)
        const uint64_t ab = __ballot(amb);
        if (lane == 0) kminmax[w][0] = ab != 0ull ? 1u : 0u;
        __syncthreads();
        uint32_t anyamb = 0u;
#pragma unroll
        for (int k = 0; k < GW; ++k) anyamb |= kminmax[k][0];
        fast = anyamb == 0u;
      }
      SL_TL(16);  // the first threshold checked
      if (fast) {
        kthr = kfast;  // keys > kfast  <=>  score > t (no score within del of either)
        jlast = -1;
        thresh = tfast;
      }
      if (!fast || thresh_out != nullptr) {  // uniform
        // Exact moments: sums of s and s^2 to ~2^-100 relative, far below the
        // single rounding to fp64 that the mean and the variance take. Every
        // thread adds its E scores onto a power-of-two offset sigma >= E *
        // (the workgroup's largest score), the same for all threads (see
        // thread_moments); the running sums' mantissa fields add exactly in
        // uint64, and only the tiny error sums round.
        int l1, l2;
        moments_log2_sigma<E>(kmax, l1, l2);
        Moments mt = thread_moments<E>(key, l1, l2, n);
        row_sum_moments(mt);
        if ((lane & 15) == 0) mrows[4 * w + (lane >> 4)] = mt;
        __syncthreads();
        SL_TL(17);  // every row total in LDS
        if (w == 0) {
          // the 4 * GW row totals, one per lane: row sums again, then the four
          // rows of this wavefront in a fixed order
          mt = mrows[lane];
          row_sum_moments(mt);
          const uint64_t I1 = readlane_u64(mt.i1, 0) + readlane_u64(mt.i1, 16) + readlane_u64(mt.i1, 32) +
                              readlane_u64(mt.i1, 48);
          const uint64_t I2 = readlane_u64(mt.i2, 0) + readlane_u64(mt.i2, 16) + readlane_u64(mt.i2, 32) +
                              readlane_u64(mt.i2, 48);
          const double E1 = (readlane_f64(mt.e1, 0) + readlane_f64(mt.e1, 16)) +
                            (readlane_f64(mt.e1, 32) + readlane_f64(mt.e1, 48));
          const double E2 = (readlane_f64(mt.e2, 0) + readlane_f64(mt.e2, 16)) +
                            (readlane_f64(mt.e2, 32) + readlane_f64(mt.e2, 48));
          SL_TL(12);  // totals summed
          if (lane == 0) {
            // sums = I * ulp(sigma) + E, ulp(sigma) = 2^(log2 sigma - 52)
            const dd T1 = moments_total(I1, E1, l1 - 52), T2 = moments_total(I2, E2, l2 - 52);
            const dd mu = dd_mul(T1, inv_n);
            double var;
            double mean = mu.hi;
            if (kmin == kmax) {  // all scores equal: exact mean, zero variance
              mean = (double)__uint_as_float(kmin);
              var = 0.0;
            } else {
              const dd ex2 = dd_mul(T2, inv_n);
              const dd msq = dd_sqr(mu);
              const dd v = dd_add(ex2, dd{-msq.hi, -msq.lo});
              var = v.hi > 0.0 ? v.hi : 0.0;
            }
            const double sigma = sqrt(var);
            const double tt = __dadd_rn(mean, __dmul_rn(sigma, z));
            uint32_t kt;
            int jl;
            thresh_to_key(tt, n, kt, jl);
            const uint64_t tb = (uint64_t)__double_as_longlong(tt);
            res[0] = kt;
            res[1] = (uint32_t)jl;
            res[2] = (uint32_t)tb;
            res[3] = (uint32_t)(tb >> 32);
          }
          SL_TL(13);  // mu, sigma, t and the key pair computed
        }
        __syncthreads();
        SL_TL(5);  // exact threshold known
        if (!fast) {
          kthr = res[0];
          jlast = (int)res[1];
        }
        thresh = __longlong_as_double((long long)(((uint64_t)res[3] << 32) | res[2]));
      }
    } else {  // MODE_FIXED
      clear_y(0);
      thresh = (double)tau;
      thresh_to_key(thresh, n, kthr, jlast);
    }
    if (count_out != nullptr) {
      uint32_t local = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int i = index(e);
        local += (i < n && gate_keep(key[e], i, kthr, jlast)) ? 1u : 0u;
      }
      count = (int)block_sum(local, wsum);
    }
  }

  if (mask_out != nullptr) {
    uint8_t* mb = mask_out + (size_t)b * n;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = index(e);
      if (i < n) mb[i] = gate_keep(key[e], i, kthr, jlast) ? 1 : 0;
    }
  }
  if (t == 0) {
    sl::GateOut go;
    go.kthr = kthr;
    go.jlast = jlast;
    go.count = count;
    go.pad = 0;
    go.thresh = thresh;
    gout[b] = go;
    if (count_out != nullptr) count_out[b] = count;
    if (thresh_out != nullptr) thresh_out[b] = thresh;
  }
  SL_TL(6);
  kthr_out = kthr;
  jlast_out = jlast;
}

// One token's gate: keys, then the selection (prologue first, so that the
// select's histogram is cleared while the loads are in flight).
template <typename XT, int G, int MODE, bool VEC>
__device__ __forceinline__ void gate_body(const XT* __restrict__ x, const float* __restrict__ c, int n, int K,
                                          double z, float tau, sl::GateOut* __restrict__ gout,
                                          uint8_t* __restrict__ mask_out, int32_t* __restrict__ count_out,
                                          double* __restrict__ thresh_out, float* __restrict__ zero_y, int m,
                                          uint32_t* h1, uint32_t* h2, uint32_t* h3, uint32_t* wsum,
                                          uint32_t* res, uint64_t* cand, Moments* mrows,
                                          uint32_t (*kminmax)[2], int b, uint32_t& kthr_out,
                                          int& jlast_out) {
  const uint32_t prevk = gate_prologue<MODE>(K, gout, b, h2, res);
  uint32_t key[4 * G];
  gate_keys<XT, G, VEC>(x, c, n, b, key);
  gate_select<G, MODE>(key, prevk, n, K, z, tau, gout, mask_out, count_out, thresh_out, zero_y, m, h1, h2, h3,
                       wsum, res, cand, mrows, kminmax, b, kthr_out, jlast_out);
}

}  // namespace gatedev
}  // namespace sl
