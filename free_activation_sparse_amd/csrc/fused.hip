// Fused single-token forward: the gate and the index-list product in one
// launch of 1024-thread workgroups.
//
//   workgroup 0      the gate (gate_body.h) for the token: scores, top-K or
//                    statistical threshold, the optional mask / count /
//                    threshold outputs; with the atomic split reduction it
//                    also clears y (device-coherent stores issued right after
//                    its input loads). It then publishes the kept-set pair
//                    (kthr, jlast) in one 64-bit device-coherent flag word,
//                    waits until every product workgroup has acknowledged it
//                    and clears the flag and the acknowledgement counters for
//                    the next launch.
//   workgroups 1..P  one (row tile, input chunk) each of the product
//                    (product_body.h): they load x and c of their chunk and
//                    score it while the gate runs, wait for the flag (bounded
//                    spin), then compact, stream the kept columns and reduce.
//
// One launch instead of two saves a kernel boundary per token and overlaps the
// product's chunk loads with the gate. Progress: workgroups are dispatched in
// index order on each XCD, so workgroup 0 holds a CU before any product
// workgroup exists; every spin is bounded, and a timeout is recorded in the
// handle's host-visible error word (reported by the handle's next call or by
// sparse_linear_sync_status) instead of hanging.
#include "gate_body.h"
#include "product_body.h"

#include <algorithm>

namespace {

using namespace sl::dev;

constexpr int FT = sl::gatedev::GT;  // threads per workgroup (16 wavefronts)
constexpr uint32_t kSpinLimit = 1u << 20;  // polls (>= 50 ns each) before giving up
constexpr float kSpecMargin = 1.15f;       // sure-set bound over the previous threshold score
constexpr float kBandLow = 0.97f;          // lower edge of the held band, over the previous threshold score
constexpr double kBandMaxKeep = 0.25;      // the held band only where at most this fraction of inputs is kept
constexpr int kBandMax = 512;              // band entries held (at most one stream step of any tile height)

struct GateSmem {
  alignas(16) uint32_t h1[4096];
  uint32_t h2[4096];
  uint32_t h3[128];
  uint64_t cand[64];
  uint32_t wsum[FT / 64];
  uint32_t res[4];
  sl::gatedev::Moments mrows[FT / 16];
  uint32_t kminmax[FT / 64][2];
};

template <typename WT>
struct ProdSmem {
  int2 list[sl::kMaxChunk];
  int2 blist[kBandMax];     // held band entries (j, x bits)
  uint32_t bkey[kBandMax];  // and their score keys
  uint32_t wcnt[2 * (FT / 64) + 2];
  float red[sl::proddev::red_floats<WT, FT>()];
  uint32_t s_last;
  uint64_t s_gate;
};

// (kthr, jlast) in one word that is never 0 (jlast >= -1) and never below
// 2^32, so 1 can mark a wait that timed out.
constexpr uint64_t kGateTimeout = 1ull;

// (kthr, jlast) in one word that is never 0 (jlast >= -1).
__device__ __forceinline__ uint64_t pack_gate(uint32_t kthr, int jlast) {
  return ((uint64_t)(uint32_t)(jlast + 2) << 32) | (uint64_t)kthr;
}

// One linear's share of a launch: its weights, gate and hand-off state,
// launch shape and output (a grouped launch carries several).
template <typename WT, typename YT>
struct FusedArgs {
  const WT* Wt;
  const float* c;
  int m, K;
  double z;
  float tau;
  sl::GateOut* gout;
  uint8_t* mask_out;
  int32_t* count_out;
  double* thresh_out;
  int tiles, splits, chunk;
  float* partials;
  uint32_t* ctr;
  sl::FusedSync* sync;
  uint32_t* err;  // host-visible record of a timed-out wait (system scope)
  YT* y;
};

template <typename WT>
union FusedSmem {
  GateSmem g;
  ProdSmem<WT> p;
};

// The gate workgroup of one linear: selection, the pair in the flag word,
// then the wait for every product workgroup's acknowledgement and the re-arm.
template <typename WT, typename YT, int G, int MODE, int LPC, bool ATOMIC>
__device__ __forceinline__ void fused_gate(const FusedArgs<WT, YT>& a, const WT* __restrict__ x, int n,
                                           FusedSmem<WT>& sm) {
  const float* __restrict__ c = a.c;
  const int m = a.m, K = a.K, tiles = a.tiles, splits = a.splits;
  const double z = a.z;
  const float tau = a.tau;
  sl::GateOut* __restrict__ gout = a.gout;
  sl::FusedSync* __restrict__ sync = a.sync;
  YT* __restrict__ y = a.y;
  const int t = threadIdx.x;
  const int nprod = tiles * splits;
  SL_TL_DECL;
  SL_TL(0);
  {
    uint32_t kthr;
    int jlast;
    float* zy = (ATOMIC && splits > 1) ? (float*)y : nullptr;
    sl::gatedev::gate_body<WT, G, MODE, true>(x, c, n, K, z, tau, gout, a.mask_out, a.count_out, a.thresh_out, zy, m,
                                              sm.g.h1, sm.g.h2, sm.g.h3, sm.g.wsum, sm.g.res, sm.g.cand,
                                              sm.g.mrows, sm.g.kminmax, 0, kthr, jlast);
    __builtin_amdgcn_s_waitcnt(0);  // this thread's clearing stores are complete
    __syncthreads();
    SL_TL(1);
    if (t == 0) __hip_atomic_store(&sync->flag, pack_gate(kthr, jlast), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (t < 64) {
      // wavefront 0 sums the acknowledgement slots until every product
      // workgroup has read the flag, then re-arms the hand-off
      const int slot = t < sl::kAckSlots ? t : 0;
      uint32_t it = 0, total = 0;
      for (;;) {
        const uint32_t ak = t < sl::kAckSlots
                                ? __hip_atomic_load(&sync->ack[16 * slot], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                : 0u;
        total = wave_sum(ak);
        if (total >= (uint32_t)nprod || ++it >= kSpinLimit) break;
        __builtin_amdgcn_s_sleep(8);
      }
      SL_TL(2);
      if (t == 0 && total < (uint32_t)nprod) __hip_atomic_store(a.err, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      if (t < sl::kAckSlots) __hip_atomic_store(&sync->ack[16 * slot], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (t == 0) __hip_atomic_store(&sync->flag, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// The speculative lists of one chunk (one input per thread): the sure set
// (keys >= g0) into list, ascending, and the band (gb <= key < g0) into blist
// with its keys in bkey, ascending, the first bmax of it only; held tells
// whether this thread's input is one of those. Returns (sure count, held band
// count). One pass: two ballots per wavefront, one scan, three barriers.
__device__ __forceinline__ int2 compact_sure_band(uint32_t key, float xv, int jt, int j1, uint32_t g0, uint32_t gb,
                                                  int bmax, int2* list, int2* blist, uint32_t* bkey, uint32_t* wcnt,
                                                  bool& held) {
  constexpr int NW = FT / 64;
  const int lane = threadIdx.x & 63, w = wave_id();
  const bool v = jt < j1;
  const bool sure = v && key >= g0;
  const bool band = v && key >= gb && key < g0;
  const uint64_t bs = __ballot(sure), bb = __ballot(band);
  if (lane == 0) {
    wcnt[w] = (uint32_t)__popcll(bs);
    wcnt[NW + w] = (uint32_t)__popcll(bb);
  }
  __syncthreads();
  if (w == 0) {
    // lanes 0..NW-1: sure counts; NW..2NW-1: band counts; exclusive offsets
    // within each list, totals in wcnt[2 NW] and wcnt[2 NW + 1]
    const uint32_t c0 = lane < 2 * NW ? wcnt[lane] : 0u;
    const uint32_t incl = wave_incl_scan(c0);
    const uint32_t sure_tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, NW - 1);
    const uint32_t all_tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 2 * NW - 1);
    if (lane < 2 * NW) wcnt[lane] = incl - c0 - (lane >= NW ? sure_tot : 0u);
    if (lane == 0) {
      wcnt[2 * NW] = sure_tot;
      wcnt[2 * NW + 1] = all_tot - sure_tot;
    }
  }
  __syncthreads();
  if (sure) list[wcnt[w] + lanes_below(bs)] = make_int2(jt, __float_as_int(xv));
  const int pos = (int)(wcnt[NW + w] + lanes_below(bb));
  held = band && pos < bmax;
  if (held) {
    blist[pos] = make_int2(jt, __float_as_int(xv));
    bkey[pos] = key;
  }
  const int2 cnt = make_int2((int)wcnt[2 * NW], min((int)wcnt[2 * NW + 1], bmax));
  __syncthreads();
  return cnt;
}

// Keys and indices of the held band entries that step_issue (step 0 of
// blist) gives this lane's column slot: entries slot + u CS.
template <int LPC, int U>
__device__ __forceinline__ void band_slot_keys(const int2* blist, const uint32_t* bkey, int cntb, uint32_t (&bk)[U],
                                               int (&bj)[U]) {
  constexpr int CPW = 64 / LPC;
  constexpr int CS = (FT / 64) * CPW;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int slot = w * CPW + lane / LPC;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int k = slot + u * CS;
    bk[u] = k < cntb ? bkey[k] : 0u;  // (empty slots carry x = 0 anyway)
    bj[u] = k < cntb ? blist[k].x : 0;
  }
}

// Product workgroup pw (0-based) of one linear. SPEC (speculation) only with
// the atomic reduction, whose summation order varies anyway: with the ordered
// reduction the result must not depend on the previous call.
template <typename WT, typename YT, int G, int MODE, int LPC, bool ATOMIC, bool SPEC, bool BAND>
__device__ __forceinline__ void fused_product(const FusedArgs<WT, YT>& a, const WT* __restrict__ x, int n, int pw,
                                              FusedSmem<WT>& sm) {
  const WT* __restrict__ Wt = a.Wt;
  const float* __restrict__ c = a.c;
  const int m = a.m, tiles = a.tiles, splits = a.splits, chunk = a.chunk;
  const float tau = a.tau;
  sl::GateOut* __restrict__ gout = a.gout;
  sl::FusedSync* __restrict__ sync = a.sync;
  float* __restrict__ partials = a.partials;
  uint32_t* __restrict__ ctr = a.ctr;
  YT* __restrict__ y = a.y;
  const int t = threadIdx.x;
  SL_TL_DECL;
  SL_TL(0);
  const int tile = pw % tiles;
  const int split = pw / tiles;
  const int j0 = split * chunk;
  const int j1 = min(j0 + chunk, n);
  // the handle's previous threshold key (any value read here is safe: it only
  // steers the speculation below, which is checked against the exact pair)
  const uint32_t prevk = SPEC ? __hip_atomic_load(&gout->kthr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
  static_assert(sl::proddev::Chunk<FT>::ROUNDS == 1, "one input per thread");
  sl::proddev::Chunk<FT> ch;
  sl::proddev::load_chunk<WT, FT, false>(x, c, j0, j1, ch);
  const int lane = t & 63, w = wave_id();
  const int jt = j0 + t;
  sl::proddev::Acc<WT> acc;
#pragma unroll
  for (int v = 0; v < sl::proddev::Acc<WT>::VEC; ++v) acc.v[v] = 0.f;

  // Speculation: while the gate runs, stream the inputs whose score is at
  // least kSpecMargin times the previous threshold (the sure set: consecutive
  // tokens' thresholds differ by a few percent, so these are almost always
  // kept). Where few inputs are kept (the sure stream ends long before the
  // gate does), also load, but do not yet add, the band of inputs between
  // kBandLow and kSpecMargin times it: its weights are held in registers
  // until the pair arrives, and then each band input is added with its x or
  // with 0 as the gate decided. (Where many are kept, the band's extra bytes
  // would lengthen the stream that bounds the launch.) The kept inputs that
  // neither covered are streamed after the pair; if the threshold rose above
  // the sure bound, the sums are dropped and every kept input is streamed.
  uint32_t g0 = 0xffffffffu;  // no speculation
  uint32_t gb = 0xffffffffu;  // band lower edge (empty band: gb >= g0)
  if (MODE == sl::gatedev::MODE_FIXED) {
    // a fixed threshold is known now: the "speculative" set is the kept set
    // itself (the gate's pair only confirms it and orders the adds after the
    // clearing of y)
    if (SPEC) {
      uint32_t kt;
      int jl;
      sl::gatedev::thresh_to_key((double)tau, n, kt, jl);
      g0 = jl >= 0 ? 0u : kt + 1u;  // keep all (jlast = n - 1) or keys > kt
      gb = g0;
    }
  } else if (SPEC && prevk != 0u && prevk < 0x7f800000u) {
    g0 = __float_as_uint(__uint_as_float(prevk) * kSpecMargin);
    if (g0 <= prevk) g0 = prevk + 1u;
    if (BAND) {
      gb = __float_as_uint(__uint_as_float(prevk) * kBandLow);
      if (gb > prevk) gb = prevk;
    }
  }
  if (t == 0) sm.p.s_gate = 0ull;  // ordered before its uses by the barriers below
  constexpr int STEP = sl::proddev::step_columns<LPC, 8, FT>();
  uint64_t pv = 0ull;
  const int jw = j0 + 64 * w;
  if constexpr (BAND) {
    static_assert(STEP <= kBandMax, "the held band is one stream step");
    bool held = false;
    int cnt0 = 0, cntb = 0;
    if (g0 != 0xffffffffu) {
      const int2 cn = compact_sure_band(ch.kv[0], ch.xv[0], jt, j1, g0, gb, STEP, sm.p.list, sm.p.blist, sm.p.bkey,
                                        sm.p.wcnt, held);
      cnt0 = cn.x;
      cntb = cn.y;
    }
    const int nsteps = (cnt0 + STEP - 1) / STEP;  // workgroup-uniform
    SL_TL(1);
    SL_TL_AT(21, t == 0, (unsigned long long)(cnt0 + cntb));

    for (int it = 0; it + 1 < nsteps; ++it)
      sl::proddev::stream_step<WT, LPC, 8, FT>(Wt, m, tile, sm.p.list, cnt0, it, acc);
    if (nsteps > 0 || cntb > 0) {
      // Each wavefront polls the flag just before its last sure step's and the
      // band's loads (loads complete in order, so the answer is in before
      // those weights are), and adds the last sure step before it waits.
      if (lane == 0) pv = __hip_atomic_load(&sync->flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      sl::proddev::Batch<WT, 8> last, band;
      if (nsteps > 0) sl::proddev::step_issue<WT, LPC, 8, FT>(Wt, m, tile, sm.p.list, cnt0, nsteps - 1, last);
      sl::proddev::step_issue<WT, LPC, 8, FT>(Wt, m, tile, sm.p.blist, cntb, 0, band);
      uint32_t bk[8];
      int bj[8];
      band_slot_keys<LPC, 8>(sm.p.blist, sm.p.bkey, cntb, bk, bj);
      pv = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(pv >> 32), 0) << 32) |
           (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)pv, 0);
      SL_TL(2);
      SL_TL_AT(20, t == 0, pv);
      if (nsteps > 0) sl::proddev::step_consume<WT, 8>(last, acc);
      if (pv != 0ull) {
        if (lane == 0) __hip_atomic_store(&sm.p.s_gate, pv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      } else {
        // the early poll came back empty: wavefront 0 polls memory (one poller
        // per workgroup: a poll storm on one line would stall the weight
        // stream), the others watch its copy in LDS; kGateTimeout marks a wait
        // that gave up
        if (lane == 0) {
          if (w == 0) {
            for (uint32_t it = 0; pv == 0ull && it < kSpinLimit; ++it) {
              __builtin_amdgcn_s_sleep(2);
              pv = __hip_atomic_load(&sync->flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            if (pv == 0ull) pv = kGateTimeout;
            __hip_atomic_store(&sm.p.s_gate, pv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          } else {
            for (uint32_t it = 0; pv == 0ull && it < 4u * kSpinLimit; ++it) {
              __builtin_amdgcn_s_sleep(1);
              pv = __hip_atomic_load(&sm.p.s_gate, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
          }
        }
        pv = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(pv >> 32), 0) << 32) |
             (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)pv, 0);
        if (pv == kGateTimeout) pv = 0ull;
        SL_TL(3);
      }
      if (pv != 0ull) {  // (0: the wait timed out, recorded in the error word)
        const uint32_t kthr = (uint32_t)pv;
        const int jlast = (int)(uint32_t)(pv >> 32) - 2;
        // the sure set is kept iff its bound lies above the threshold key
        const bool valid = g0 > kthr;
        if (valid) {
          // the held band: each input with its x if the gate kept it, else 0
  #pragma unroll
          for (int u = 0; u < 8; ++u)
            if (!gate_keep(bk[u], bj[u], kthr, jlast)) band.xs[u] = 0.f;
          sl::proddev::step_consume<WT, 8>(band, acc);
        } else {
  #pragma unroll
          for (int q = 0; q < sl::proddev::Acc<WT>::VEC; ++q) acc.v[q] = 0.f;
        }
        // the rest: each wavefront streams the kept inputs among its own 64
        // (one per lane) that neither the sure set nor the held band covered
        const bool rest = jt < j1 && gate_keep(ch.kv[0], jt, kthr, jlast) && (!valid || (ch.kv[0] < g0 && !held));
        sl::proddev::stream_wave_bits<WT, LPC, 8>(Wt, m, tile, jw, __ballot(rest), ch.xv[0], acc);
      }
    } else {
      // nothing to stream ahead of the gate: one thread waits for the pair
      if (t == 0) {
        for (uint32_t it = 0; it < kSpinLimit; ++it) {
          pv = __hip_atomic_load(&sync->flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (pv != 0ull) break;
          __builtin_amdgcn_s_sleep(1);
        }
        sm.p.s_gate = pv;
      }
      __syncthreads();
      pv = sm.p.s_gate;
      if (pv != 0ull) {
        const uint32_t kthr = (uint32_t)pv;
        const int jlast = (int)(uint32_t)(pv >> 32) - 2;
        const bool keep = jt < j1 && gate_keep(ch.kv[0], jt, kthr, jlast);
        sl::proddev::stream_wave_bits<WT, LPC, 8>(Wt, m, tile, jw, __ballot(keep), ch.xv[0], acc);
      }
    }
  } else {
    int cnt0 = 0;
    if (g0 != 0xffffffffu) cnt0 = sl::proddev::compact_chunk<FT, false>(ch, j0, j1, g0 - 1u, -1, sm.p.list, sm.p.wcnt);
    const int nsteps = (cnt0 + STEP - 1) / STEP;  // workgroup-uniform
    SL_TL(1);
    SL_TL_AT(21, t == 0, (unsigned long long)cnt0);

    // The speculative list, over all wavefronts' column slots. Each wavefront
    // issues its poll of the flag just before its last step's loads: loads
    // complete in order, so the answer is in before that step's weights are.
    // When the pair is there and the speculation holds, the first batch of the
    // rest (the kept inputs among the wavefront's own 64 that the speculation
    // did not cover) is issued before the last step's weights are consumed.
    bool rest_done = false;  // wavefront-uniform
    for (int it = 0; it + 1 < nsteps; ++it) sl::proddev::stream_step<WT, LPC, 8, FT>(Wt, m, tile, sm.p.list, cnt0, it, acc);
    if (nsteps > 0) {
      if (lane == 0) pv = __hip_atomic_load(&sync->flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      sl::proddev::Batch<WT, 8> last, rest;
      sl::proddev::step_issue<WT, LPC, 8, FT>(Wt, m, tile, sm.p.list, cnt0, nsteps - 1, last);
      pv = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(pv >> 32), 0) << 32) |
           (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)pv, 0);
      SL_TL(2);
      SL_TL_AT(20, t == 0, pv);
      uint64_t bal = 0ull;
      bool any = false;
      if (pv != 0ull && g0 > (uint32_t)pv) {  // pair known and the speculation holds
        const uint32_t kthr = (uint32_t)pv;
        const int jlast = (int)(uint32_t)(pv >> 32) - 2;
        bal = __ballot(jt < j1 && gate_keep(ch.kv[0], jt, kthr, jlast) && ch.kv[0] < g0);
        any = bal != 0ull;
        if (any) sl::proddev::bits_issue<WT, LPC, 8>(Wt, m, tile, jw, bal, ch.xv[0], rest);
        rest_done = true;
      }
      if (lane == 0 && pv != 0ull) __hip_atomic_store(&sm.p.s_gate, pv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      sl::proddev::step_consume<WT, 8>(last, acc);
      if (any) sl::proddev::step_consume<WT, 8>(rest, acc);
      if (rest_done) sl::proddev::stream_wave_bits<WT, LPC, 8>(Wt, m, tile, jw, bal, ch.xv[0], acc);  // leftovers
    }
    if (!rest_done) {
      if (nsteps == 0) {
        // nothing to stream ahead of the gate: one thread waits for the pair
        if (t == 0) {
          for (uint32_t it = 0; it < kSpinLimit; ++it) {
            pv = __hip_atomic_load(&sync->flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (pv != 0ull) break;
            __builtin_amdgcn_s_sleep(1);
          }
          sm.p.s_gate = pv;
        }
        __syncthreads();
        pv = sm.p.s_gate;
      } else if (pv == 0ull) {
        // the early poll came back empty: wavefront 0 polls memory (one poller
        // per workgroup: a poll storm on one line would stall the weight
        // stream), the others watch its copy in LDS; kGateTimeout marks a wait
        // that gave up
        if (lane == 0) {
          if (w == 0) {
            for (uint32_t it = 0; pv == 0ull && it < kSpinLimit; ++it) {
              __builtin_amdgcn_s_sleep(2);
              pv = __hip_atomic_load(&sync->flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            if (pv == 0ull) pv = kGateTimeout;
            __hip_atomic_store(&sm.p.s_gate, pv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          } else {
            for (uint32_t it = 0; pv == 0ull && it < 4u * kSpinLimit; ++it) {
              __builtin_amdgcn_s_sleep(1);
              pv = __hip_atomic_load(&sm.p.s_gate, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
          }
        }
        pv = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(pv >> 32), 0) << 32) |
             (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)pv, 0);
        if (pv == kGateTimeout) pv = 0ull;
        SL_TL(3);
      }
      if (pv != 0ull) {  // (0: the wait timed out, recorded in the error word)
        const uint32_t kthr = (uint32_t)pv;
        const int jlast = (int)(uint32_t)(pv >> 32) - 2;
        // every speculated input is kept iff the bound lies above the
        // threshold key; otherwise the speculative sums are dropped and all
        // kept inputs are streamed
        const bool valid = g0 == 0xffffffffu || g0 > kthr;
        if (!valid) {
  #pragma unroll
          for (int q = 0; q < sl::proddev::Acc<WT>::VEC; ++q) acc.v[q] = 0.f;
        }
        // the rest: each wavefront streams the kept inputs among its own 64
        // (one per lane) that the speculation did not cover, into its own slots
        const bool rest = jt < j1 && gate_keep(ch.kv[0], jt, kthr, jlast) && (!valid || ch.kv[0] < g0);
        sl::proddev::stream_wave_bits<WT, LPC, 8>(Wt, m, tile, jw, __ballot(rest), ch.xv[0], acc);
      }
    }
  }
  SL_TL_AT(4 + w, lane == 0, __builtin_amdgcn_s_memrealtime());
  if (t == 0) {
    if (pv == 0ull) __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_fetch_add(&sync->ack[16 * (pw % sl::kAckSlots)], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  sl::proddev::reduce_out<WT, YT, LPC, FT, ATOMIC>(acc, m, tile, split, splits, sm.p.red, partials, ctr,
                                                   &sm.p.s_last, y);
  SL_TL_WAIT();
  SL_TL(22);
}

// One linear: workgroup 0 is the gate, 1.. the product.
template <typename WT, typename YT, int G, int MODE, int LPC, bool ATOMIC, bool BAND, bool SPEC = ATOMIC>
__global__ __launch_bounds__(FT) void fused_kernel(FusedArgs<WT, YT> a, const WT* __restrict__ x, int n) {
  __shared__ FusedSmem<WT> sm;
  if (blockIdx.x == 0) {
    fused_gate<WT, YT, G, MODE, LPC, ATOMIC>(a, x, n, sm);
    return;
  }
  fused_product<WT, YT, G, MODE, LPC, ATOMIC, SPEC, BAND && SPEC>(a, x, n, blockIdx.x - 1, sm);
}

// Grouped linears that share their input x (B = 1, fp32 y, atomic split
// reduction): workgroups 0..count-1 are their gates, then each linear's
// product workgroups in order (begin[l] .. begin[l + 1] - 1). Every gate
// workgroup precedes every product workgroup in the dispatch order, as in
// the single-linear launch.
constexpr int kMaxGroup = sl::kMaxGroupLinears;
template <typename WT>
struct FusedGroup {
  FusedArgs<WT, float> lin[kMaxGroup];
  int begin[kMaxGroup + 1];
  int count;
};

template <typename WT, int G, int MODE, int LPC, bool BAND>
__global__ __launch_bounds__(FT) void fused_group_kernel(FusedGroup<WT> gr, const WT* __restrict__ x, int n) {
  __shared__ FusedSmem<WT> sm;
  const int b = blockIdx.x;
  if (b < gr.count) {
    fused_gate<WT, float, G, MODE, LPC, true>(gr.lin[b], x, n, sm);
    return;
  }
  const int pw = b - gr.count;
  int l = 0;
  while (l + 1 < gr.count && pw >= gr.begin[l + 1]) ++l;  // uniform
  fused_product<WT, float, G, MODE, LPC, true, true, BAND>(gr.lin[l], x, n, pw - gr.begin[l], sm);
}

// The held band pays where the gate, not the stream, bounds the launch: few
// kept inputs (the kept fraction the handle is configured for).
bool hold_band(const sl_linear* h) {
  if (h->gate == SL_GATE_TOPK) return h->n > 0 && (double)h->K <= kBandMaxKeep * (double)h->n;
  if (h->gate == SL_GATE_STAT) return h->s_keep <= kBandMaxKeep;
  return false;  // fixed threshold: its kept set is known at launch
}

struct FusedPlan {
  int tiles, splits, chunk;
};

// Row tiles of LPC * 8 rows; the input chunks are sized so that the product
// workgroups fill the device's remaining workgroup slots once (chunks of
// 32..kMaxChunk inputs), unless a split count is forced on the handle.
FusedPlan plan_fused(const sl_linear* h, int lpc, int per_cu) {
  FusedPlan p;
  const int64_t n = h->n;
  const int rows = lpc * 8;
  p.tiles = (int)((h->m + rows - 1) / rows);
  const int64_t slots = (int64_t)std::max(1, h->cus) * per_cu;
  int64_t splits = h->plan_splits > 0 ? h->plan_splits : std::max<int64_t>(1, (slots - 1) / p.tiles);
  splits = std::min<int64_t>(splits, std::min<int64_t>(sl::kMaxSplits, (n + 31) / 32));
  splits = std::max<int64_t>(splits, (n + sl::kMaxChunk - 1) / sl::kMaxChunk);
  p.chunk = (int)((n + splits - 1) / splits);
  p.splits = (int)((n + p.chunk - 1) / p.chunk);
  return p;
}

template <typename YT, int G, int MODE, int LPC, bool ATOMIC, bool BAND>
hipError_t go(const sl_linear* h, const void* x, sl::GateOut* g, uint8_t* mask, int32_t* cnt, double* th, void* y,
              hipStream_t s) {
  static const int per_cu = [] {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fused_kernel<uint16_t, YT, G, MODE, LPC, ATOMIC, BAND>, FT,
                                                     0) != hipSuccess)
      nb = 1;
    return std::max(1, nb);
  }();
  const FusedPlan p = plan_fused(h, LPC, per_cu);
  const FusedArgs<uint16_t, YT> a{(const uint16_t*)h->Wt, h->c, (int)h->m, (int)h->K, h->z, h->tau, g, mask, cnt,
                                 th, p.tiles, p.splits, p.chunk, h->partials, h->ctr, h->fsync, h->herr_dev, (YT*)y};
  fused_kernel<uint16_t, YT, G, MODE, LPC, ATOMIC, BAND><<<1 + p.tiles * p.splits, FT, 0, s>>>(
      a, (const uint16_t*)x, (int)h->n);
  return hipGetLastError();
}

// The held band exists only with the speculation (atomic reduction) and a
// gate whose threshold moves from token to token.
template <typename YT, int G, int MODE, int LPC, bool ATOMIC>
hipError_t go_band(const sl_linear* h, const void* x, sl::GateOut* g, uint8_t* mask, int32_t* cnt, double* th,
                   void* y, hipStream_t s) {
  if constexpr (ATOMIC && MODE != sl::gatedev::MODE_FIXED) {
    if (hold_band(h)) return go<YT, G, MODE, LPC, ATOMIC, true>(h, x, g, mask, cnt, th, y, s);
  }
  return go<YT, G, MODE, LPC, ATOMIC, false>(h, x, g, mask, cnt, th, y, s);
}

template <typename YT, int G, int MODE, bool ATOMIC>
hipError_t go_lpc(const sl_linear* h, const void* x, sl::GateOut* g, uint8_t* mask, int32_t* cnt,
                  double* th, void* y, hipStream_t s) {
  // 512-row tiles (1 KB column runs) from 2048 rows up: on the 4096-row
  // layers they beat 256-row tiles by ~3 % (fewer, longer runs per column)
  int lpc = h->plan_rows > 0 ? h->plan_rows / 8 : (h->m >= 2048 ? 64 : 16);
  // taller row tiles when the chunk limit alone would ask for more product
  // workgroups than the device holds at once (a late tail of workgroups)
  const int64_t min_splits = (h->n + sl::kMaxChunk - 1) / sl::kMaxChunk;
  while (h->plan_rows <= 0 && lpc < 64 && (h->m + 8 * lpc - 1) / (8 * lpc) * min_splits >= std::max(1, h->cus))
    lpc *= 2;
  switch (lpc) {
    case 16: return go_band<YT, G, MODE, 16, ATOMIC>(h, x, g, mask, cnt, th, y, s);
    case 32: return go_band<YT, G, MODE, 32, ATOMIC>(h, x, g, mask, cnt, th, y, s);
    default: return go_band<YT, G, MODE, 64, ATOMIC>(h, x, g, mask, cnt, th, y, s);
  }
}

template <typename YT, int G, bool ATOMIC>
hipError_t go_mode(const sl_linear* h, const void* x, sl::GateOut* g, uint8_t* mask, int32_t* cnt,
                   double* th, void* y, hipStream_t s) {
  if (h->gate == SL_GATE_STAT)
    return go_lpc<YT, G, sl::gatedev::MODE_STAT, ATOMIC>(h, x, g, mask, cnt, th, y, s);
  if (h->gate == SL_GATE_FIXED)
    return go_lpc<YT, G, sl::gatedev::MODE_FIXED, ATOMIC>(h, x, g, mask, cnt, th, y, s);
  return go_lpc<YT, G, sl::gatedev::MODE_TOPK, ATOMIC>(h, x, g, mask, cnt, th, y, s);
}

template <typename YT, bool ATOMIC>
hipError_t go_g(const sl_linear* h, const void* x, sl::GateOut* g, uint8_t* mask, int32_t* cnt,
                double* th, void* y, hipStream_t s) {
  const int64_t groups = (h->n + 4 * FT - 1) / (4 * FT);  // 1..8 for n <= 32768
  if (groups <= 2) return go_mode<YT, 2, ATOMIC>(h, x, g, mask, cnt, th, y, s);
  if (groups <= 3) return go_mode<YT, 3, ATOMIC>(h, x, g, mask, cnt, th, y, s);
  if (groups <= 4) return go_mode<YT, 4, ATOMIC>(h, x, g, mask, cnt, th, y, s);
  if (groups <= 5) return go_mode<YT, 5, ATOMIC>(h, x, g, mask, cnt, th, y, s);
  if (groups <= 6) return go_mode<YT, 6, ATOMIC>(h, x, g, mask, cnt, th, y, s);
  return go_mode<YT, 8, ATOMIC>(h, x, g, mask, cnt, th, y, s);
}

// Grouped launch: every linear gets tiles x (at least) the chunk limit's
// splits, and the remaining workgroup slots are shared in proportion to the
// linears' expected kept bytes (m times the kept count).
template <int G, int MODE, int LPC, bool BAND>
hipError_t go_group(const sl_linear* const* hs, int count, const void* x, float* const* ys, hipStream_t s) {
  static const int per_cu = [] {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fused_group_kernel<uint16_t, G, MODE, LPC, BAND>, FT, 0) !=
        hipSuccess)
      nb = 1;
    return std::max(1, nb);
  }();
  const int64_t n = hs[0]->n;
  const int rows = LPC * 8;
  const int64_t slots = (int64_t)std::max(1, hs[0]->cus) * per_cu - count;
  const int64_t min_splits = (n + sl::kMaxChunk - 1) / sl::kMaxChunk;
  const int64_t max_splits = std::min<int64_t>(sl::kMaxSplits, (n + 31) / 32);
  double wsum = 0.0;
  double wl[kMaxGroup];
  int64_t tiles[kMaxGroup];
  for (int l = 0; l < count; ++l) {
    const sl_linear* h = hs[l];
    const double kept = h->gate == SL_GATE_TOPK ? (double)h->K
                        : h->gate == SL_GATE_STAT ? h->s_keep * (double)n
                                                  : 0.5 * (double)n;
    wl[l] = (double)h->m * std::max(1.0, kept);
    wsum += wl[l];
    tiles[l] = (h->m + rows - 1) / rows;
  }
  FusedGroup<uint16_t> gr{};
  gr.count = count;
  int64_t total = 0;
  for (int l = 0; l < count; ++l) {
    const sl_linear* h = hs[l];
    int64_t splits = (int64_t)((double)slots * wl[l] / wsum) / tiles[l];
    splits = std::min(std::max(splits, (int64_t)1), max_splits);
    splits = std::max(splits, min_splits);
    const int chunk = (int)((n + splits - 1) / splits);
    splits = (n + chunk - 1) / chunk;
    gr.begin[l] = (int)total;
    gr.lin[l] = FusedArgs<uint16_t, float>{(const uint16_t*)h->Wt, h->c, (int)h->m, (int)h->K, h->z, h->tau,
                                           h->gout, nullptr, nullptr, nullptr, (int)tiles[l], (int)splits, chunk,
                                           h->partials, h->ctr, h->fsync, h->herr_dev, ys[l]};
    total += tiles[l] * splits;
  }
  gr.begin[count] = (int)total;
  fused_group_kernel<uint16_t, G, MODE, LPC, BAND><<<(unsigned)(count + total), FT, 0, s>>>(gr, (const uint16_t*)x,
                                                                                            (int)n);
  return hipGetLastError();
}

// The held band when every linear of the group asks for it.
template <int G, int MODE, int LPC>
hipError_t go_group_band(const sl_linear* const* hs, int count, const void* x, float* const* ys, hipStream_t s) {
  if constexpr (MODE != sl::gatedev::MODE_FIXED) {
    bool all = true;
    for (int l = 0; l < count; ++l) all = all && hold_band(hs[l]);
    if (all) return go_group<G, MODE, LPC, true>(hs, count, x, ys, s);
  }
  return go_group<G, MODE, LPC, false>(hs, count, x, ys, s);
}

template <int G, int MODE>
hipError_t go_group_lpc(const sl_linear* const* hs, int count, const void* x, float* const* ys, hipStream_t s) {
  int64_t mmin = hs[0]->m;
  for (int l = 1; l < count; ++l) mmin = std::min(mmin, hs[l]->m);
  // 512-row tiles unless a linear is shorter than two of them
  if (mmin >= 1024) return go_group_band<G, MODE, 64>(hs, count, x, ys, s);
  return go_group_band<G, MODE, 16>(hs, count, x, ys, s);
}

template <int G>
hipError_t go_group_mode(const sl_linear* const* hs, int count, const void* x, float* const* ys, hipStream_t s) {
  if (hs[0]->gate == SL_GATE_STAT) return go_group_lpc<G, sl::gatedev::MODE_STAT>(hs, count, x, ys, s);
  if (hs[0]->gate == SL_GATE_FIXED) return go_group_lpc<G, sl::gatedev::MODE_FIXED>(hs, count, x, ys, s);
  return go_group_lpc<G, sl::gatedev::MODE_TOPK>(hs, count, x, ys, s);
}

}  // namespace

namespace sl {

hipError_t launch_fused_group(const sl_linear* const* hs, int count, const void* x, float* const* ys,
                              hipStream_t s) {
  const int64_t groups = (hs[0]->n + 4 * FT - 1) / (4 * FT);  // 1..8 for n <= 32768
  if (groups <= 2) return go_group_mode<2>(hs, count, x, ys, s);
  if (groups <= 3) return go_group_mode<3>(hs, count, x, ys, s);
  if (groups <= 4) return go_group_mode<4>(hs, count, x, ys, s);
  if (groups <= 5) return go_group_mode<5>(hs, count, x, ys, s);
  if (groups <= 6) return go_group_mode<6>(hs, count, x, ys, s);
  return go_group_mode<8>(hs, count, x, ys, s);
}

hipError_t timeline_set(void* buf) {
#ifdef SL_TIMELINE
  return hipMemcpyToSymbol(HIP_SYMBOL(sl_timeline_buf), &buf, sizeof(buf));
#else
  (void)buf;
  return hipErrorNotSupported;
#endif
}

bool fused_supported(const sl_linear* h, const void* x) {
  return h->wdt == SL_BF16 && h->n % 4 == 0 &&
         ((uintptr_t)x % 8) == 0;
}

hipError_t launch_fused(const sl_linear* h, const void* x, GateOut* g, uint8_t* mask_out, int32_t* count_out,
                        double* thresh_out, void* y, sl_dtype ydt, bool atomic, hipStream_t s) {
  if (ydt == SL_BF16) return go_g<uint16_t, false>(h, x, g, mask_out, count_out, thresh_out, y, s);
  if (atomic) return go_g<float, true>(h, x, g, mask_out, count_out, thresh_out, y, s);
  return go_g<float, false>(h, x, g, mask_out, count_out, thresh_out, y, s);
}

}  // namespace sl
