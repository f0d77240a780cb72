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
//    population variance of the scores in double-double arithmetic, each
//    rounded once to fp64; sigma by IEEE sqrt; t = fl(mu + fl(sigma * z)).
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
                                          uint32_t* res, uint64_t* cand, dd (*dsum)[2],
                                          uint32_t (*kminmax)[2], int b, uint32_t& kthr_out, int& jlast_out) {
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

  // the product that follows adds its split partials into y atomically;
  // device-coherent stores, so that product workgroups of the same launch on
  // other XCDs add onto the zeros
  if (zero_y != nullptr) {
    float* yb = zero_y + (size_t)b * m;
    for (int i = t; i < m; i += GT) __hip_atomic_store(yb + i, 0.f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
      if (w == 0) find_bin_wave<4096, (E <= 16 ? 8 : 2)>(h1, (uint32_t)K, res);
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
      // per-thread cascaded sums of s and s^2 (s^2 of an fp32 value is exact in fp64)
      double a1 = 0.0, e1 = 0.0, a2 = 0.0, e2 = 0.0;
      uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (index(e) < n) {
          const double s = (double)__uint_as_float(key[e]);
          dd p = two_sum(a1, s);
          a1 = p.hi;
          e1 = e1 + p.lo;
          p = two_sum(a2, s * s);
          a2 = p.hi;
          e2 = e2 + p.lo;
          kmin = min(kmin, key[e]);
          kmax = max(kmax, key[e]);
        }
      }
      dd S1 = fast_two_sum(a1, e1), S2 = fast_two_sum(a2, e2);
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) {
        S1 = dd_add(S1, shfl_xor_dd(S1, d));
        S2 = dd_add(S2, shfl_xor_dd(S2, d));
      }
      kmax = wave_max(kmax);
      kmin = ~wave_max(~kmin);
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
        res[0] = kt;
        res[1] = (uint32_t)jl;
        dsum[0][0].hi = tt;
      }
      __syncthreads();
      kthr = res[0];
      jlast = (int)res[1];
      thresh = dsum[0][0].hi;
    } else {  // MODE_FIXED
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
