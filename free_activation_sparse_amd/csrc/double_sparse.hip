// Double Sparsity decode attention on gfx950 (Double Sparsity article, section
// 在线前向计算: gather the query at the calibrated channels, score every cached
// token against its contiguous label row, keep the k best tokens, attend over
// their full key and value rows; section 离线校准: the label cache).
//
// ds_decode_kernel: one 1024-thread workgroup per (sequence, head).
//   1. Label stream: thread t scores tokens t, t + 1024, ... (E per thread,
//      scores kept in registers as order-preserving 32-bit keys). Each token's
//      r label values are one contiguous 16/32/64-byte run; a wavefront's
//      loads cover 64 consecutive tokens. All row loads of the kernel are
//      non-temporal (every label, key and value row is read once per step).
//   2. Select: the k-th largest key and the last kept tie's index, with the
//      same machinery as the linear layer's top-K gate: a 4096-bin LDS
//      histogram window below the largest key, exact ranking of the pivot
//      bin's candidates by one wavefront, and a radix-select fallback on key
//      digits (12/12/8 bits) then on the reversed index (8/7 bits).
//   3. Compaction: ballots + a prefix over (slot, wavefront) counts, which
//      every wavefront scans itself, write the kept token indices to LDS in
//      ascending order.
//   4. Attention: 16 lanes per token row (16 or 8 bytes of the key and value
//      rows per lane), 64 rows per workgroup step, four steps of key and value
//      loads in flight; each 16-lane row keeps its own online softmax (running
//      max, sum, fp32 accumulators, exp2 with the scale folded into log2 e);
//      the rows merge by cross-lane shuffles within each wavefront, then the
//      16 wavefront partials through LDS.
// A sequence with n <= k tokens skips steps 1-3 and attends to all n.
//
// ds_label_kernel: one thread per (sequence, head, token): the r channels of
// the key row gathered into one contiguous label row.
#include <math.h>

#include <algorithm>

#include "device_common.h"
#include "gate_body.h"
#include "internal.h"

#pragma clang fp contract(off)

namespace {

using namespace sl::dev;
using sl::gatedev::GT;
using sl::gatedev::GW;
using sl::gatedev::find_bin;
using sl::gatedev::find_bin_wave;

constexpr int kMaxSeq = DS_MAX_SEQ;
constexpr int kRows = 64;  // token rows per workgroup step: 16 wavefronts x 4 rows of 16 lanes
constexpr int kSteps = 4;  // workgroup steps whose loads are issued together

// Signed fp32 score -> unsigned key with the same order (+0 and -0 both map
// to 0x80000000). Every finite or infinite score maps above 0, the key of the
// slots past the sequence's end.
__device__ __forceinline__ uint32_t signed_key(float s) {
  const uint32_t u = __float_as_uint(s == 0.f ? 0.f : s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Sum over each row of 16 lanes, returned to every lane of the row (rotations
// within the row; each step adds the same two values in every lane, so all
// lanes hold identical bits).
__device__ __forceinline__ float row16_allsum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false));  // row_ror:8
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false));  // row_ror:4
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xf, 0xf, false));  // row_ror:2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xf, 0xf, false));  // row_ror:1
  return v;
}

// VE consecutive bf16 of a row, widened to fp32 (VE = 8: one 16-byte load,
// VE = 4: one 8-byte load). Non-temporal: key and value rows are read once
// per step, and so are the label rows (measured ~11 % faster than cached loads).
template <int VE>
struct RowPart;
template <>
struct RowPart<8> {
  u32x4 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = __builtin_nontemporal_load((const u32x4*)p); }
  __device__ __forceinline__ float get(int e) const {
    const uint32_t w = v[e >> 1];
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};
template <>
struct RowPart<4> {
  uint2 v;
  __device__ __forceinline__ void load(const uint16_t* p) {
    const uint64_t u = __builtin_nontemporal_load((const uint64_t*)p);
    v = make_uint2((uint32_t)u, (uint32_t)(u >> 32));
  }
  __device__ __forceinline__ float get(int e) const {
    const uint32_t w = (e >> 1) ? v.y : v.x;
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};

// Up to 16384 tokens (E = 8 or 16) two workgroups share a compute unit (at
// most 64 registers per lane); up to 32768 (E = 32) one does.
template <int D, int R, int E>
__global__ __launch_bounds__(GT, E <= 16 ? 8 : 4) void ds_decode_kernel(sl::DsDecodeParams a) {
  constexpr int VE = D / 16;  // key/value elements per lane
  constexpr int RV = R / 8;   // 16-byte loads per label row
  constexpr int EB = RV >= 4 ? 1 : (RV == 2 ? (E <= 8 ? 2 : 1) : (E <= 8 ? 8 : 2));  // tokens per label batch
  // dynamic LDS: selection histograms (32 KB), then the kept list, then the
  // per-wavefront attention partials (16 x D floats); each use ends before
  // the next
  extern __shared__ __align__(16) uint32_t dyn[];
  __shared__ uint32_t h3[256], hi1[256], hi2[128];
  __shared__ uint32_t wsum[GW];
  __shared__ uint32_t res[4];
  __shared__ uint64_t cand[64];
  __shared__ uint32_t cnt[E * GW];
  __shared__ float wm[GW], wl[GW];

  uint32_t* h1 = dyn;
  uint32_t* h2 = dyn + 4096;
  int32_t* sel = (int32_t*)dyn;
  float* wacc = (float*)dyn;

  const int t = threadIdx.x, lane = t & 63, w = wave_id();
  const int bh = blockIdx.x;
  const int b = bh / a.heads, h = bh - b * a.heads;
  const int n = min(max(a.seq_len[b], 0), a.max_seq);
  const bool dense = a.k >= n;
  const int count = dense ? n : a.k;

  if (!dense) {
    // ---- 1. approximate scores over the label rows
    float ql[R];
    const int32_t* chp = a.channels + (size_t)h * R;
    const uint16_t* qb = a.q + (size_t)bh * D;
#pragma unroll
    for (int j = 0; j < R; ++j)  // uniform: held in scalar registers
      ql[j] = __uint_as_float((uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)qb[chp[j] & (D - 1)] << 16)));
    const u32x4* lb = (const u32x4*)(a.label + (size_t)bh * a.max_seq * R);
    uint32_t key[E];
    uint32_t dep = 0u;
#pragma unroll
    for (int e0 = 0; e0 < E; e0 += EB) {
      u32x4 v[EB][RV];
      // The first token of this batch goes through an empty asm that also
      // takes the previous batch's last key: the batch's loads cannot be
      // hoisted above that batch's scores, so at most EB * r / 2 registers
      // of label data are live (hoisted, every batch's loads spilled).
      int tok0 = e0 * GT + t;
      asm volatile("" : "+v"(tok0) : "v"(dep));
#pragma unroll
      for (int eb = 0; eb < EB; ++eb) {
        // unconditional loads (index clamped to the last token, result
        // discarded below): no branches, all of a batch in flight together
        const int tok = min(tok0 + eb * GT, n - 1);
#pragma unroll
        for (int q = 0; q < RV; ++q) v[eb][q] = __builtin_nontemporal_load(lb + (size_t)tok * RV + q);
      }
#pragma unroll
      for (int eb = 0; eb < EB; ++eb) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < R; ++j) {
          const uint32_t wd = v[eb][j >> 3][(j & 7) >> 1];
          const float lv = __uint_as_float((j & 1) ? (wd & 0xffff0000u) : (wd << 16));
          const float pr = ql[j] * lv;  // exact for bf16 operands
          s = s + pr;
        }
        key[e0 + eb] = ((e0 + eb) * GT + t < n) ? signed_key(s) : 0u;
      }
      dep = key[e0 + EB - 1];
    }

    // ---- 2. the k-th largest key (kthr) and the last kept tie's index (jlast)
    const uint32_t K = (uint32_t)a.k;  // 1 <= K < n
    uint32_t kthr, jlast_u;
    for (int i = t; i < 4096; i += GT) h1[i] = 0u;
    uint32_t lmax = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) lmax = max(lmax, key[e]);
    lmax = wave_max(lmax);
    if (lane == 0) wsum[w] = lmax;
    if (t == 0) {
      res[0] = 0xffffffffu;
      res[3] = 0u;
    }
    __syncthreads();
    uint32_t kmax = wsum[0];
#pragma unroll
    for (int q = 1; q < GW; ++q) kmax = max(kmax, wsum[q]);
    // window of 4096 bins of key>>14 ending at the largest key's bin (bin >= 1,
    // so the empty slots' key 0 never falls inside)
    const uint32_t top = kmax >> 14;
    const uint32_t base = top >= 4096u ? top - 4095u : 1u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t d = (key[e] >> 14) - base;
      if (d < 4096u) atomicAdd(&h1[d], 1u);
    }
    __syncthreads();
    if (w == 0) find_bin_wave<4096, 2>(h1, K, res);  // few reads in flight: registers are scarce here
    __syncthreads();
    const bool in_window = res[0] != 0xffffffffu;
    const uint32_t c1 = in_window ? res[2] : 0u;
    if (in_window && c1 <= 64u) {
      const uint32_t b1 = res[0] + base;
      const uint32_t r1 = K - res[1];  // rank wanted inside the pivot bin, 1-based
      // candidates as (key, ~index): larger composite = earlier in the order
      // (score descending, index ascending)
      // (ballots taken twice, to count and then to place: holding E of them
      // would cost 2E scalar registers)
      uint32_t wtot = 0u;
#pragma unroll
      for (int e = 0; e < E; ++e) wtot += (uint32_t)__popcll(__ballot((key[e] >> 14) == b1));
      if (wtot != 0u) {
        uint32_t off = 0u;
        if (lane == 0) off = atomicAdd(&res[3], wtot);
        off = (uint32_t)__builtin_amdgcn_readfirstlane((int)off);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const uint64_t bal = __ballot((key[e] >> 14) == b1);
          if ((bal >> lane) & 1ull)
            cand[off + lanes_below(bal)] = ((uint64_t)key[e] << 32) | (uint64_t)(~(uint32_t)(e * GT + t));
          off += (uint32_t)__popcll(bal);
        }
      }
      __syncthreads();
      if (w == 0) {
        const uint64_t ca = (uint32_t)lane < c1 ? cand[lane] : 0ull;
        const uint32_t chi = (uint32_t)(ca >> 32), clo = (uint32_t)ca;
        uint32_t above = 0u;
        for (int q = 0; q < (int)c1; ++q) {
          const uint64_t o = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)chi, q) << 32) |
                             (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)clo, q);
          above += (o > ca) ? 1u : 0u;
        }
        if ((uint32_t)lane < c1 && above == r1 - 1u) {
          res[1] = chi;
          res[2] = ~clo;
        }
      }
      __syncthreads();
      kthr = res[1];
      jlast_u = res[2];
    } else {
      // radix select on key digits 31..20, 19..8, 7..0
      for (int i = t; i < 4096; i += GT) {
        h1[i] = 0u;
        h2[i] = 0u;
      }
      if (t < 256) {
        h3[t] = 0u;
        hi1[t] = 0u;
      }
      if (t < 128) hi2[t] = 0u;
      __syncthreads();
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (e * GT + t < n) atomicAdd(&h1[key[e] >> 20], 1u);
      __syncthreads();
      find_bin<4096>(h1, K, wsum, res);
      const uint32_t d1 = res[0];
      uint32_t rr = K - res[1];
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (e * GT + t < n && (key[e] >> 20) == d1) atomicAdd(&h2[(key[e] >> 8) & 0xfffu], 1u);
      __syncthreads();
      find_bin<4096>(h2, rr, wsum, res);
      const uint32_t p2 = (d1 << 12) | res[0];
      rr -= res[1];
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (e * GT + t < n && (key[e] >> 8) == p2) atomicAdd(&h3[key[e] & 0xffu], 1u);
      __syncthreads();
      find_bin<256>(h3, rr, wsum, res);
      const uint32_t vstar = (p2 << 8) | res[0];
      rr -= res[1];  // ties of vstar to keep, >= 1
      // the rr-th smallest index among the ties: radix select on the
      // reversed index (kMaxSeq - 1 - index; 15 bits as 8 + 7)
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (e * GT + t < n && key[e] == vstar) atomicAdd(&hi1[(uint32_t)(kMaxSeq - 1 - (e * GT + t)) >> 7], 1u);
      __syncthreads();
      find_bin<256>(hi1, rr, wsum, res);
      const uint32_t q1 = res[0];
      rr -= res[1];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint32_t ri = (uint32_t)(kMaxSeq - 1 - (e * GT + t));
        if (e * GT + t < n && key[e] == vstar && (ri >> 7) == q1) atomicAdd(&hi2[ri & 127u], 1u);
      }
      __syncthreads();
      find_bin<128>(hi2, rr, wsum, res);
      kthr = vstar;
      jlast_u = (uint32_t)(kMaxSeq - 1) - ((q1 << 7) | res[0]);
    }
    const int jlast = (int)jlast_u;

    // ---- 3. kept tokens, ascending, into sel (the histograms are dead)
    auto kept = [&](int e) { return key[e] > kthr || (key[e] == kthr && e * GT + t <= jlast); };
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t c = (uint32_t)__popcll(__ballot(kept(e)));
      if (lane == 0) cnt[e * GW + w] = c;
    }
    __syncthreads();
    // every wavefront scans the E * 16 counts (slot-major, so in token order)
    // itself and reads off its own offsets: one block barrier, not three
    constexpr int CPL = (E * GW + 63) / 64;  // counts per lane
    uint32_t pre[CPL];
    uint32_t lsum = 0u;
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      const int idx = lane * CPL + q;
      pre[q] = lsum;
      lsum += idx < E * GW ? cnt[idx] : 0u;
    }
    const uint32_t lexcl = wave_incl_scan(lsum) - lsum;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int idx = e * GW + w;  // wavefront-uniform
      uint32_t mine = 0u;
#pragma unroll
      for (int q = 0; q < CPL; ++q) mine = (idx % CPL == q) ? pre[q] : mine;
      const uint32_t off = (uint32_t)__builtin_amdgcn_readlane((int)(lexcl + mine), idx / CPL);
      const uint64_t bal = __ballot(kept(e));
      if ((bal >> lane) & 1ull) sel[off + lanes_below(bal)] = e * GT + t;
    }
    __syncthreads();
  }

  if (a.tokens_out != nullptr) {
    int32_t* to = a.tokens_out + (size_t)bh * a.k;
    for (int i = t; i < a.k; i += GT) to[i] = i < count ? (dense ? i : sel[i]) : -1;
  }

  // ---- 4. attention over the kept rows
  const int g = lane >> 4, p = lane & 15;
  const int row = w * 4 + g;
  float qv[VE];
  {
    RowPart<VE> qp;
    qp.load(a.q + (size_t)bh * D + p * VE);
#pragma unroll
    for (int e = 0; e < VE; ++e) qv[e] = qp.get(e);
  }
  const uint16_t* kbase = a.key + (size_t)bh * a.max_seq * D + p * VE;
  const uint16_t* vbase = a.value + (size_t)bh * a.max_seq * D + p * VE;
  float m = -INFINITY, l = 0.f;
  float acc[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) acc[e] = 0.f;
  for (int i0 = 0; i0 < count; i0 += kRows * kSteps) {
    RowPart<VE> kr[kSteps], vr[kSteps];
    bool valid[kSteps];
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      const int i = i0 + u * kRows + row;
      valid[u] = i < count;
      const int tok = valid[u] ? (dense ? i : sel[i]) : 0;
      kr[u].load(kbase + (size_t)tok * D);
      vr[u].load(vbase + (size_t)tok * D);
    }
    float x[kSteps];
    float mx = m;
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < VE; ++e) dot = fmaf(qv[e], kr[u].get(e), dot);
      const float rdot = row16_allsum(dot);  // all lanes active
      x[u] = valid[u] ? rdot * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, x[u]);
    }
    if (mx != -INFINITY) {
      const float alpha = exp2f(m - mx);
      l *= alpha;
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[e] *= alpha;
#pragma unroll
      for (int u = 0; u < kSteps; ++u) {
        const float pu = exp2f(x[u] - mx);
        l += pu;
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[e] = fmaf(pu, vr[u].get(e), acc[e]);
      }
      m = mx;
    }
  }
  // merge the four rows of each wavefront (lanes l, l + 16, l + 32, l + 48
  // hold the same columns), then the 16 wavefronts through LDS
  const float mw = fmaxf(fmaxf(m, __shfl_xor(m, 16)), fmaxf(__shfl_xor(m, 32), __shfl_xor(m, 48)));
  const float sc = m == -INFINITY ? 0.f : exp2f(m - mw);  // an empty row weighs nothing
  float lw = l * sc;
  lw += __shfl_xor(lw, 16);
  lw += __shfl_xor(lw, 32);
#pragma unroll
  for (int e = 0; e < VE; ++e) {
    float v = acc[e] * sc;
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    acc[e] = v;
  }
  __syncthreads();  // the kept list is dead: the wavefront partials reuse its LDS
  if (lane < 16) {
#pragma unroll
    for (int e = 0; e < VE; ++e) wacc[w * D + lane * VE + e] = acc[e];
  }
  if (lane == 0) {
    wm[w] = mw;
    wl[w] = lw;
  }
  __syncthreads();
  if (t < D) {
    float M = -INFINITY;
#pragma unroll
    for (int q = 0; q < GW; ++q) M = fmaxf(M, wm[q]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int q = 0; q < GW; ++q) {
        const float wq = exp2f(wm[q] - M);  // 0 for a wavefront without rows
        L = fmaf(wq, wl[q], L);
        O = fmaf(wq, wacc[q * D + t], O);
      }
    }
    a.out[(size_t)bh * D + t] = M == -INFINITY ? 0.f : O / L;
  }
}

template <int D, int R>
__global__ __launch_bounds__(256) void ds_label_kernel(const uint16_t* __restrict__ key, uint16_t* __restrict__ label,
                                                       const int32_t* __restrict__ channels,
                                                       const int32_t* __restrict__ start, int heads, int max_seq,
                                                       int span) {
  const int bh = blockIdx.x;
  const int b = bh / heads, h = bh - b * heads;
  const int i = blockIdx.y * 256 + threadIdx.x;
  if (i >= span) return;
  const int64_t tok = (int64_t)(start != nullptr ? start[b] : 0) + i;
  if (tok < 0 || tok >= max_seq) return;
  const uint16_t* row = key + ((size_t)bh * max_seq + (size_t)tok) * D;
  const int32_t* chp = channels + (size_t)h * R;
  uint32_t wv[R / 2];
#pragma unroll
  for (int j = 0; j < R / 2; ++j)
    wv[j] = (uint32_t)row[chp[2 * j] & (D - 1)] | ((uint32_t)row[chp[2 * j + 1] & (D - 1)] << 16);
  u32x4* dst = (u32x4*)(label + ((size_t)bh * max_seq + (size_t)tok) * R);
#pragma unroll
  for (int q = 0; q < R / 8; ++q) dst[q] = u32x4{wv[4 * q], wv[4 * q + 1], wv[4 * q + 2], wv[4 * q + 3]};
}

template <int D, int R, int E>
hipError_t go_decode(const sl::DsDecodeParams& p, int batch, hipStream_t s) {
  const int kl = p.k < p.max_seq ? p.k : 0;  // kept-list entries (0: every sequence dense)
  size_t dyn = 4096 * 2 * sizeof(uint32_t);
  dyn = std::max(dyn, (size_t)kl * sizeof(int32_t));
  dyn = std::max(dyn, (size_t)GW * D * sizeof(float));
  ds_decode_kernel<D, R, E><<<(unsigned)(batch * p.heads), GT, dyn, s>>>(p);
  return hipGetLastError();
}

template <int D, int R>
hipError_t go_decode_e(const sl::DsDecodeParams& p, int batch, hipStream_t s) {
  if (p.max_seq <= 8 * GT) return go_decode<D, R, 8>(p, batch, s);
  if (p.max_seq <= 16 * GT) return go_decode<D, R, 16>(p, batch, s);
  return go_decode<D, R, 32>(p, batch, s);
}

template <int D>
hipError_t go_decode_r(const sl::DsDecodeParams& p, int batch, int r, hipStream_t s) {
  switch (r) {
    case 8: return go_decode_e<D, 8>(p, batch, s);
    case 16: return go_decode_e<D, 16>(p, batch, s);
    default: return go_decode_e<D, 32>(p, batch, s);
  }
}

template <int D>
hipError_t go_label_r(const uint16_t* key, uint16_t* label, const int32_t* channels, const int32_t* start,
                      int batch, int heads, int max_seq, int r, int span, hipStream_t s) {
  const dim3 grid((unsigned)(batch * heads), (unsigned)((span + 255) / 256));
  switch (r) {
    case 8: ds_label_kernel<D, 8><<<grid, 256, 0, s>>>(key, label, channels, start, heads, max_seq, span); break;
    case 16: ds_label_kernel<D, 16><<<grid, 256, 0, s>>>(key, label, channels, start, heads, max_seq, span); break;
    default: ds_label_kernel<D, 32><<<grid, 256, 0, s>>>(key, label, channels, start, heads, max_seq, span); break;
  }
  return hipGetLastError();
}

}  // namespace

namespace sl {

hipError_t launch_ds_decode(const DsDecodeParams& p, int batch, int head_dim, int r, hipStream_t s) {
  if (head_dim == 64) return go_decode_r<64>(p, batch, r, s);
  return go_decode_r<128>(p, batch, r, s);
}

hipError_t launch_ds_label(const uint16_t* key, uint16_t* label, const int32_t* channels, const int32_t* start,
                           int batch, int heads, int max_seq, int head_dim, int r, int span, hipStream_t s) {
  if (head_dim == 64) return go_label_r<64>(key, label, channels, start, batch, heads, max_seq, r, span, s);
  return go_label_r<128>(key, label, channels, start, batch, heads, max_seq, r, span, s);
}

}  // namespace sl
