// Gate body shared by the gate kernel and the fused gate + product kernel:
// one 1024-thread workgroup computes a token's scores and kept set.
//
//  * Top-K (WINA article, section 一): selection on the scores' fp32 bit
//    patterns (non-negative, so unsigned order is numeric order).
//    Fast path: a 4096-bin LDS histogram of key>>14 over the eight binades
//    below the largest key (512 bins per binade: few atomic collisions),
//    searched by one wavefront; the pivot bin's keys (at most 64) are
//    compacted with ballots and ranked exactly under the order (score
//    descending, index ascending) by one wavefront.
//    General path (pivot below the window, or more than 64 keys in the pivot
//    bin, i.e. heavy ties): radix select on 12/12/7-bit key digits, then the
//    kept ties' last index by a radix select on the index (8/7 bits).
//  * Statistical threshold (Spark Transformer article, section 2.2): mean and
//    population variance of the scores from double-double sums, each rounded
//    once to fp64; sigma by IEEE sqrt; t = fl(mu + fl(sigma * z)). The sums
//    come from this workgroup's own scores, or (fused forward) from partial
//    sums of 64-input slices that the product workgroups publish.
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
// Sums of non-negative terms as unnormalised double-double pairs: the high
// parts add error-free (two_sum), the low parts collect the rounding errors
// in plain fp64. With no cancellation the relative error stays near 2^-100,
// far below the single rounding to fp64 that the mean and the variance take.
struct sd {
  double hi, lo;
};
__device__ __forceinline__ sd sd_add(sd a, sd b) {
  const dd s = two_sum(a.hi, b.hi);
  return {s.hi, (a.lo + b.lo) + s.lo};
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint64_t lo = dpp_move<CTRL>((uint32_t)u), hi = dpp_move<CTRL>((uint32_t)(u >> 32));
  return __longlong_as_double((long long)((hi << 32) | lo));
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __longlong_as_double((long long)((hi << 32) | lo));
}
template <int CTRL>
__device__ __forceinline__ void sd_scan_step(sd& a, sd& b, bool take) {
  const sd ta{dpp_f64<CTRL>(a.hi), dpp_f64<CTRL>(a.lo)};
  const sd tb{dpp_f64<CTRL>(b.hi), dpp_f64<CTRL>(b.lo)};
  if (take) {
    a = sd_add(a, ta);
    b = sd_add(b, tb);
  }
}
// Wavefront totals of two pair sums in every lane (the inclusive scan's lane
// 63). Needs all 64 lanes active.
__device__ __forceinline__ void wave_sum_sd(sd& a, sd& b) {
  const uint32_t lane = threadIdx.x & 63u, rl = lane & 15u;
  sd_scan_step<0x111>(a, b, rl >= 1u);  // row_shr:1
  sd_scan_step<0x112>(a, b, rl >= 2u);  // row_shr:2
  sd_scan_step<0x114>(a, b, rl >= 4u);  // row_shr:4
  sd_scan_step<0x118>(a, b, rl >= 8u);  // row_shr:8
  sd_scan_step<0x142>(a, b, (lane & 31u) >= 16u);  // row_bcast:15
  sd_scan_step<0x143>(a, b, lane >= 32u);          // row_bcast:31
  a = {readlane_f64(a.hi, 63), readlane_f64(a.lo, 63)};
  b = {readlane_f64(b.hi, 63), readlane_f64(b.lo, 63)};
}

// Totals of two pair sums over lanes 0..15 (the first row's inclusive scan,
// read back from lane 15 to every lane). Needs all 64 lanes active.
__device__ __forceinline__ void row0_sum_sd(sd& a, sd& b) {
  const uint32_t rl = threadIdx.x & 15u;
  sd_scan_step<0x111>(a, b, rl >= 1u);  // row_shr:1
  sd_scan_step<0x112>(a, b, rl >= 2u);  // row_shr:2
  sd_scan_step<0x114>(a, b, rl >= 4u);  // row_shr:4
  sd_scan_step<0x118>(a, b, rl >= 8u);  // row_shr:8
  a = {readlane_f64(a.hi, 15), readlane_f64(a.lo, 15)};
  b = {readlane_f64(b.hi, 15), readlane_f64(b.lo, 15)};
}

// Sums of a thread's E scores (keys) and of their squares. A power-of-two
// offset sigma >= E * (largest score) goes in first: every running sum then
// lies in [sigma, 2 sigma), at or above each addend, so Fast2Sum yields each
// rounding error exactly, and taking sigma out at the end is exact
// (Sterbenz). Squares of fp32 values are exact in fp64. Keys of 0 add
// nothing.
template <int E>
__device__ __forceinline__ void thread_moments(const uint32_t (&key)[E], uint32_t kmax, sd& S1, sd& S2) {
  constexpr int LE = E <= 1 ? 0 : 32 - __builtin_clz((unsigned)(E - 1));  // ceil(log2 E)
  const int eb = max((int)(kmax >> 23), 1);  // largest score < 2^(eb - 126), its square < 2^(2 eb - 252)
  const double sig1 = __longlong_as_double((long long)(eb - 126 + LE + 1023) << 52);
  const double sig2 = __longlong_as_double((long long)(2 * eb - 252 + LE + 1023) << 52);
  double a1 = sig1, e1 = 0.0, a2 = sig2, e2 = 0.0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const double s = (double)__uint_as_float(key[e]);
    const double t1 = a1 + s;
    e1 += s - (t1 - a1);
    a1 = t1;
    const double q = s * s;
    const double t2 = a2 + q;
    e2 += q - (t2 - a2);
    a2 = t2;
  }
  S1 = {a1 - sig1, e1};
  S2 = {a2 - sig2, e2};
}

// Moment parts published by other workgroups of the same launch (fused
// forward). parts == nullptr: the gate workgroup sums its own scores, as it
// also does when the parts are not all in after wait_ticks.
struct PartsIn {
  const sl::MomentPart* parts = nullptr;
  int count = 0;            // parts expected (slices of 64 inputs)
  uint32_t tag = 0;         // tag of this launch's parts
  uint32_t wait_ticks = 0;  // s_memrealtime ticks (100 MHz) before the gate sums its own scores
};

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

template <typename XT, int G, int MODE, bool VEC>
__device__ __forceinline__ void gate_body(const XT* __restrict__ x, const float* __restrict__ c, int n, int K,
                                          double z, float tau, sl::GateOut* __restrict__ gout,
                                          uint8_t* __restrict__ mask_out, int32_t* __restrict__ count_out,
                                          double* __restrict__ thresh_out, float* __restrict__ zero_y, int m,
                                          uint32_t* h1, uint32_t* h2, uint32_t* h3, uint32_t* wsum,
                                          uint32_t* res, uint64_t* cand, sd (*dsum)[2],
                                          uint32_t (*kminmax)[2], int b, PartsIn pin, uint32_t& kthr_out,
                                          int& jlast_out) {
  constexpr int E = 4 * G;
  const int t = threadIdx.x, lane = t & 63, w = wave_id();
  const XT* xb = x + (size_t)b * n;
  auto index = [&](int e) { return ((e >> 2) * GT + t) * 4 + (e & 3); };

  uint32_t key[E];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    uint32_t k4[4];
    load_group<XT, VEC>(xb, c, n, g, k4);
#pragma unroll
    for (int e = 0; e < 4; ++e) key[g * 4 + e] = k4[e];
  }

  // The product that follows adds its split partials into y atomically, so
  // y is cleared here with device-coherent stores (product workgroups of the
  // same launch on other XCDs add onto the zeros). They are issued by
  // wavefronts w_lo.. while wavefront 0 works alone (bin search, final
  // scalar steps): issued beside the input loads they delayed those.
  auto clear_y = [&](int w_lo) {
    if (zero_y != nullptr && w >= w_lo) {
      float* yb = zero_y + (size_t)b * m;
      for (int i = t - 64 * w_lo; i < m; i += GT - 64 * w_lo)
        __hip_atomic_store(yb + i, 0.f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
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
      for (int i = t; i < 4096; i += GT) h1[i] = 0u;
      uint32_t lmax = 0u;
#pragma unroll
      for (int e = 0; e < E; ++e) lmax = max(lmax, key[e]);  // padding keys are 0
      lmax = wave_max(lmax);
      if (lane == 0) wsum[w] = lmax;
      if (t == 0) {
        res[0] = 0xffffffffu;  // "not found" unless find_bin writes it
        res[3] = 0u;           // candidate counter
      }
      __syncthreads();  // h1 cleared, maxima and res published
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
      // fewer reads in flight when the keys take many registers
      if (w == 0)
        find_bin_wave<4096, (E <= 16 ? 8 : 2)>(h1, (uint32_t)K, res);
      else
        clear_y(1);
      __syncthreads();
      const bool in_window = res[0] != 0xffffffffu;
      const uint32_t c1 = in_window ? res[2] : 0u;
      if (in_window && c1 <= 64u) {
        const uint32_t b1 = res[0] + base;         // pivot bin of key>>14 (>= 1: never a padding key's)
        const uint32_t r1 = (uint32_t)K - res[1];  // rank wanted inside the pivot bin, 1-based
        // candidates as (key, ~index): larger composite = earlier in the order
        // (score descending, index ascending); composites are distinct. One
        // LDS atomic per wavefront reserves its slots.
        uint64_t bal[E];
        uint32_t wtot = 0u;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          bal[e] = __ballot((key[e] >> 14) == b1);
          wtot += (uint32_t)__popcll(bal[e]);
        }
        if (wtot != 0u) {
          uint32_t off = 0u;
          if (lane == 0) off = atomicAdd(&res[3], wtot);
          off = (uint32_t)__builtin_amdgcn_readfirstlane((int)off);
#pragma unroll
          for (int e = 0; e < E; ++e) {
            if ((bal[e] >> lane) & 1ull)
              cand[off + lanes_below(bal[e])] = ((uint64_t)key[e] << 32) | (uint64_t)(~(uint32_t)index(e));
            off += (uint32_t)__popcll(bal[e]);
          }
        }
        __syncthreads();
        // rank of each candidate among the c1, by wavefront 0 (lane a holds
        // candidate a and compares it with every other through readlane)
        if (w == 0) {
          const uint64_t ca = (uint32_t)lane < c1 ? cand[lane] : 0ull;
          const uint32_t chi = (uint32_t)(ca >> 32), clo = (uint32_t)ca;
          uint32_t above = 0u;
          for (int k = 0; k < (int)c1; ++k) {
            const uint64_t o = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)chi, k) << 32) |
                               (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)clo, k);
            above += (o > ca) ? 1u : 0u;
          }
          if ((uint32_t)lane < c1 && above == r1 - 1u) {
            res[1] = chi;
            res[2] = ~clo;
          }
        }
        __syncthreads();
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
      thresh = (double)__uint_as_float(kthr);
    }
  } else {
    if constexpr (MODE == MODE_STAT) {
      sd S1{0.0, 0.0}, S2{0.0, 0.0};
      uint32_t kmin = 0xffffffffu, kmax = 0u;
      const dd inv_n = dd_recip((double)n);  // early: its divisions stay off the final chain
      bool local = pin.parts == nullptr;
      if (!local) {
        // parts of every 64-input slice, part q in lane q mod 64 of
        // wavefront q / 64: each such wavefront polls until all of its parts
        // carry this launch's tag, sums them over its lanes, and the
        // wavefront totals meet in LDS
        const int nw = (pin.count + 63) >> 6;  // <= GW: n <= 32768
        const int q = 64 * w + lane;
        const bool have = q < pin.count;
        bool all = false;
        if (w < nw) {
          // one round trip per poll: every word of the lane's part, each
          // carrying the writer's tag
          const uint64_t* pq = pin.parts[have ? q : 0].w;
          const uint64_t t_end = __builtin_amdgcn_s_memrealtime() + pin.wait_ticks;
          uint32_t v[sl::kMomentWords];
          for (;;) {
            bool in = true;
#pragma unroll
            for (int k = 0; k < sl::kMomentWords; ++k) {
              const uint64_t u = have ? __hip_atomic_load(pq + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                      : ((uint64_t)pin.tag << 32) | (k == 8 ? 0xffffffffull : 0ull);
              v[k] = (uint32_t)u;
              in &= (uint32_t)(u >> 32) == pin.tag;
            }
            all = __ballot(!in) == 0ull;
            if (all || __builtin_amdgcn_s_memrealtime() > t_end) break;
            __builtin_amdgcn_s_sleep(1);
          }
          auto dbl = [&](int k) {
            return __longlong_as_double((long long)(((uint64_t)v[k + 1] << 32) | v[k]));
          };
          S1 = sd{dbl(0), dbl(2)};
          S2 = sd{dbl(4), dbl(6)};
          wave_sum_sd(S1, S2);
          kmin = ~wave_max(~v[8]);
          kmax = wave_max(v[9]);
          if (lane == 0) {
            wsum[w] = all ? 1u : 0u;
            dsum[w][0] = S1;
            dsum[w][1] = S2;
            kminmax[w][0] = kmin;
            kminmax[w][1] = kmax;
          }
        }
        __syncthreads();
        all = true;
        for (int k = 0; k < nw; ++k) all &= wsum[k] != 0u;
        if (all && w == 0) {
          S1 = lane < nw ? dsum[lane][0] : sd{0.0, 0.0};
          S2 = lane < nw ? dsum[lane][1] : sd{0.0, 0.0};
          kmin = lane < nw ? kminmax[lane][0] : 0xffffffffu;
          kmax = lane < nw ? kminmax[lane][1] : 0u;
        }
        local = !all;
      }
      if (local) {
        // this workgroup's scores: per-thread sums, per-wavefront totals,
        // then the 16 wavefront totals in wavefront 0
        uint32_t kall = 0u;
        kmin = 0xffffffffu;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          kall = max(kall, key[e]);  // padding keys are 0
          if (index(e) < n) kmin = min(kmin, key[e]);
        }
        kmax = kall;
        thread_moments<E>(key, kall, S1, S2);
        wave_sum_sd(S1, S2);
        kmax = wave_max(kmax);
        kmin = ~wave_max(~kmin);
        if (lane == 0) {
          dsum[w][0] = S1;
          dsum[w][1] = S2;
          kminmax[w][0] = kmin;
          kminmax[w][1] = kmax;
        }
        __syncthreads();
        if (w == 0) {
          S1 = lane < GW ? dsum[lane][0] : sd{0.0, 0.0};
          S2 = lane < GW ? dsum[lane][1] : sd{0.0, 0.0};
          kmin = lane < GW ? kminmax[lane][0] : 0xffffffffu;
          kmax = lane < GW ? kminmax[lane][1] : 0u;
        }
      }
      clear_y(1);
      if (w == 0) {
        // the wavefront totals sit in lanes 0..15 (nothing above)
        row0_sum_sd(S1, S2);
        kmax = wave_max(kmax);
        kmin = ~wave_max(~kmin);
        if (lane == 0) {
          const dd T1 = fast_two_sum(S1.hi, S1.lo), T2 = fast_two_sum(S2.hi, S2.lo);
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
          res[0] = kt;
          res[1] = (uint32_t)jl;
          dsum[0][0].hi = tt;
        }
      }
      __syncthreads();
      kthr = res[0];
      jlast = (int)res[1];
      thresh = dsum[0][0].hi;
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
  kthr_out = kthr;
  jlast_out = jlast;
}

}  // namespace gatedev
}  // namespace sl
