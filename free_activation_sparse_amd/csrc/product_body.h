// Phases of the single-token index-list product, shared by the product kernel
// (256-thread workgroups) and the fused gate + product kernel (1024-thread
// workgroups). PT is the workgroup size.
//
// This is the index-list product of the Spark Transformer article (section
// 3.1): only the weight vectors of active inputs are read. W is column-major,
// so each kept input contributes one contiguous run of m weights. A workgroup
// owns one row tile and one chunk of inputs:
//   1. load_chunk: x and c of the chunk (all loads in flight together) and
//      the scores' keys;
//   2. compact_chunk: the gate predicate on each input and a ballot
//      compaction of the kept ones into LDS, ascending (no global index list);
//   3. stream_reduce: the kept columns' row-tile runs with 16-byte
//      non-temporal loads (each lane group owns every CS-th kept column and
//      issues up to U loads before consuming any), fp32 accumulation, a fixed
//      order reduction of the column slots in LDS, and the split reduction:
//        ATOMIC    fp32 atomic adds into y (which must start at zero); one
//                  memory round trip, summation order varies;
//        otherwise device-coherent partial stores, then the last workgroup of
//                  the tile to arrive (device-scope arrival counter) adds the
//                  partials in a fixed order: reproducible to the bit, and the
//                  path for bf16 outputs.
#pragma once

#include "device_common.h"
#include "internal.h"

namespace sl {
namespace proddev {

using namespace sl::dev;

// Thread t's share of a chunk: inputs j0 + q * PT + t.
template <int PT>
struct Chunk {
  static constexpr int ROUNDS = sl::kMaxChunk / PT;
  float xv[ROUNDS];
  uint32_t kv[ROUNDS];
};

// Loads are unconditional (index clamped into the chunk) so that all of them
// are in flight together; keys of a dense product are not needed.
template <typename WT, int PT, bool DENSE>
__device__ __forceinline__ void load_chunk(const WT* __restrict__ x, const float* __restrict__ c, int j0, int j1,
                                           Chunk<PT>& ch) {
  const int t = threadIdx.x;
#pragma unroll
  for (int q = 0; q < Chunk<PT>::ROUNDS; ++q) {
    const int j = j0 + q * PT + t;
    const int jc = j < j1 ? j : j1 - 1;
    ch.xv[q] = load_elem(x + jc);
    ch.kv[q] = DENSE ? 0u : score_key(ch.xv[q], c[jc]);
  }
}

// Kept inputs of [j0, j1) whose key is below `below`, as (j, x_j bits) pairs
// in list[0 .. count), in ascending order. wcnt holds ROUNDS * PT / 64 + 1
// words. Ends with a barrier.
template <int PT, bool DENSE>
__device__ __forceinline__ int compact_chunk(const Chunk<PT>& ch, int j0, int j1, uint32_t kthr, int jlast,
                                             int2* list, uint32_t* wcnt, uint32_t below = 0xffffffffu) {
  constexpr int ROUNDS = Chunk<PT>::ROUNDS;
  constexpr int NW = PT / 64;
  const int t = threadIdx.x, lane = t & 63, w = wave_id();
  const int nr = (j1 - j0 + PT - 1) / PT;
  uint64_t bal[ROUNDS];
#pragma unroll
  for (int q = 0; q < ROUNDS; ++q) {
    const int j = j0 + q * PT + t;
    const bool keep = q < nr && j < j1 && (DENSE || (gate_keep(ch.kv[q], j, kthr, jlast) && ch.kv[q] < below));
    bal[q] = __ballot(keep);
    if (lane == 0) wcnt[q * NW + w] = (uint32_t)__popcll(bal[q]);
  }
  __syncthreads();
  // wavefront 0 turns the ROUNDS * NW wavefront counts (round-major) into
  // exclusive offsets in place; the total goes to wcnt[ROUNDS * NW]
  static_assert(ROUNDS * NW <= 64, "one wavefront scans the counts");
  if (w == 0) {
    const uint32_t v = lane < ROUNDS * NW ? wcnt[lane] : 0u;
    const uint32_t incl = wave_incl_scan(v);
    if (lane < ROUNDS * NW) wcnt[lane] = incl - v;
    if (lane == 63) wcnt[ROUNDS * NW] = incl;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < ROUNDS; ++q) {
    if ((bal[q] >> lane) & 1ull)
      list[wcnt[q * NW + w] + lanes_below(bal[q])] = make_int2(j0 + q * PT + t, __float_as_int(ch.xv[q]));
  }
  const int cnt = (int)wcnt[ROUNDS * NW];
  __syncthreads();
  return cnt;
}

// LDS floats stream_reduce needs in red: one VEC-wide accumulator per thread.
template <typename WT, int PT>
constexpr int red_floats() {
  return PT * (16 / (int)sizeof(WT));
}

// Accumulator of one thread: rows tile * R + sub * VEC .. + VEC of its
// column slot.
template <typename WT>
struct Acc {
  static constexpr int VEC = 16 / (int)sizeof(WT);
  float v[VEC];
};

// Columns one stream step covers: each of the CS column slots of the
// workgroup takes up to U list entries.
template <int LPC, int U, int PT>
constexpr int step_columns() {
  return (PT / 64) * (64 / LPC) * U;
}

// Weights and inputs of one in-flight batch: U 16-byte runs per lane and
// the x each multiplies (0 where the slot has no column).
template <typename WT, int U>
struct Batch {
  u32x4 wv[U];
  float xs[U];
};

// Issues one stream step: list entries it * CS * U .. + CS * U (those below
// cnt), slot s taking entries s, s + CS, ... of the step (CS = NWS * CPW
// column slots of the NWS streaming wavefronts).
template <typename WT, int LPC, int U, int PT, int NWS = PT / 64>
__device__ __forceinline__ void step_issue(const WT* __restrict__ Wt, int m, int tile, const int2* list, int cnt,
                                           int it, Batch<WT, U>& b) {
  constexpr int VEC = Acc<WT>::VEC;          // elements per 16-byte run
  constexpr int R = LPC * VEC;               // rows per tile
  constexpr int CPW = 64 / LPC;              // column slots per wavefront
  constexpr int CS = NWS * CPW;              // column slots of the NWS streaming wavefronts
  const int t = threadIdx.x, lane = t & 63, w = wave_id();
  const int slot = w * CPW + lane / LPC;
  const int row = tile * R + (lane % LPC) * VEC;
  const int k0 = slot + it * CS * U;
  const bool rok = row < m;
  const WT* base = Wt + (rok ? row : 0);
  int2 e[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int k = k0 + u * CS;
    e[u] = list[k < cnt ? k : 0];
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const bool ok = rok && k0 + u * CS < cnt;
    b.wv[u] = ok ? __builtin_nontemporal_load((const u32x4*)(base + (size_t)e[u].x * (size_t)m))
                 : u32x4{0u, 0u, 0u, 0u};
    b.xs[u] = ok ? __int_as_float(e[u].y) : 0.f;
  }
}

template <typename WT, int U>
__device__ __forceinline__ void step_consume(const Batch<WT, U>& b, Acc<WT>& a) {
#pragma unroll
  for (int u = 0; u < U; ++u) fma_run(a.v, b.wv[u], b.xs[u]);
}

// One stream step: list entries it * step_columns() .. + step_columns()
// (those below cnt) into acc. Each slot issues its U loads before consuming
// any.
template <typename WT, int LPC, int U, int PT, int NWS = PT / 64>
__device__ __forceinline__ void stream_step(const WT* __restrict__ Wt, int m, int tile, const int2* list, int cnt,
                                            int it, Acc<WT>& a) {
  Batch<WT, U> b;
  step_issue<WT, LPC, U, PT, NWS>(Wt, m, tile, list, cnt, it, b);
  step_consume<WT, U>(b, a);
}

// Streams the row-tile runs of list[0 .. cnt) into acc (added to what it
// holds), over the column slots of wavefronts 0 .. NWS-1 (the calling
// wavefront must be one of them).
template <typename WT, int LPC, int U, int PT, int NWS = PT / 64>
__device__ __forceinline__ void stream_accum(const WT* __restrict__ Wt, int m, int tile, const int2* list, int cnt,
                                             Acc<WT>& a) {
  constexpr int STEP = NWS * (64 / LPC) * U;
  for (int it = 0; it * STEP < cnt; ++it) stream_step<WT, LPC, U, PT, NWS>(Wt, m, tile, list, cnt, it, a);
}

// Issues one batch of the columns jbase + b for the set bits b of the
// wavefront-uniform mask bal (the inputs of this wavefront's 64 lanes),
// removing them from bal; the x of input jbase + b is lane b's xv. The CPW
// column slots of the wavefront take the set bits in turn, U per slot.
template <typename WT, int LPC, int U>
__device__ __forceinline__ void bits_issue(const WT* __restrict__ Wt, int m, int tile, int jbase, uint64_t& bal,
                                           float xv, Batch<WT, U>& bt) {
  constexpr int VEC = Acc<WT>::VEC;
  constexpr int R = LPC * VEC;
  constexpr int CPW = 64 / LPC;
  constexpr int B = CPW * U;  // set bits per batch
  const int lane = threadIdx.x & 63, sw = lane / LPC;
  const int row = tile * R + (lane % LPC) * VEC;
  const bool rok = row < m;
  const WT* base = Wt + (rok ? row : 0);
  int bi[B];
  float xs[B];
#pragma unroll
  for (int i = 0; i < B; ++i) {  // scalar: the next set bit and its x
    const int b = bal != 0ull ? (int)__builtin_ctzll(bal) : -1;
    bal = bal != 0ull ? bal & (bal - 1ull) : 0ull;
    bi[i] = b;
    xs[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(xv), b < 0 ? 0 : b));
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    int b = -1;
    float xx = 0.f;
#pragma unroll
    for (int q = 0; q < CPW; ++q)
      if (sw == q) {
        b = bi[u * CPW + q];
        xx = xs[u * CPW + q];
      }
    const bool ok = b >= 0 && rok;
    bt.wv[u] = ok ? __builtin_nontemporal_load((const u32x4*)(base + (size_t)(jbase + b) * (size_t)m))
                  : u32x4{0u, 0u, 0u, 0u};
    bt.xs[u] = ok ? xx : 0.f;
  }
}

// Streams into acc the columns of every set bit of bal (see bits_issue).
template <typename WT, int LPC, int U>
__device__ __forceinline__ void stream_wave_bits(const WT* __restrict__ Wt, int m, int tile, int jbase, uint64_t bal,
                                                 float xv, Acc<WT>& a) {
  while (bal != 0ull) {
    Batch<WT, U> bt;
    bits_issue<WT, LPC, U>(Wt, m, tile, jbase, bal, xv, bt);
    step_consume<WT, U>(bt, a);
  }
}

// Adds the workgroup's column slots in a fixed order and the split partial
// into y (see the header comment for the two reductions).
template <typename WT, typename YT, int LPC, int PT, bool ATOMIC>
__device__ __forceinline__ void reduce_out(const Acc<WT>& a, int m, int tile, int split, int splits, float* red,
                                           float* __restrict__ partials, uint32_t* __restrict__ ctr,
                                           uint32_t* s_last, YT* __restrict__ y) {
  constexpr int VEC = Acc<WT>::VEC;
  constexpr int R = LPC * VEC;
  constexpr int CPW = 64 / LPC;
  constexpr int CS = (PT / 64) * CPW;
  static_assert(CS * R == red_floats<WT, PT>(), "slot buffer size");
  const int t = threadIdx.x, lane = t & 63, w = wave_id();
  const int slot = w * CPW + lane / LPC;
  const int sub = lane % LPC;
  const float* acc = a.v;

  // column slots in a fixed order
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
      *s_last = (__hip_atomic_fetch_add(&ctr[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 (uint32_t)(splits - 1))
                    ? 1u
                    : 0u;
    __syncthreads();
    if (*s_last == 0u) return;
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

template <typename WT, typename YT, int LPC, int U, int PT, bool ATOMIC>
__device__ __forceinline__ void stream_reduce(const WT* __restrict__ Wt, int m, int tile, int split, int splits,
                                              const int2* list, int cnt, float* red, float* __restrict__ partials,
                                              uint32_t* __restrict__ ctr, uint32_t* s_last, YT* __restrict__ y) {
  Acc<WT> a;
#pragma unroll
  for (int v = 0; v < Acc<WT>::VEC; ++v) a.v[v] = 0.f;
  stream_accum<WT, LPC, U, PT>(Wt, m, tile, list, cnt, a);
  reduce_out<WT, YT, LPC, PT, ATOMIC>(a, m, tile, split, splits, red, partials, ctr, s_last, y);
}

}  // namespace proddev
}  // namespace sl
