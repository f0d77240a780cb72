// Batched product on the matrix cores: for B tokens with their own kept sets,
//   Y[b][:] = sum over j kept by token b of x_b[j] * W[:, j].
//
// Each token keeps its own inputs (WINA article, section 一: per-token gate);
// the columns of a batch are read once for all of them by running the product
// over the union U of the B kept sets, with the token-wise input matrix
// X_U[j][b] = x_b[j] if token b kept j, else 0. The zeros make every token's
// result exactly its own sparse sum, while W[:, U] X_U is a dense contraction
// that suits bf16 MFMA (v_mfma_f32_16x16x32_bf16: 16 output rows x 16 tokens
// x 32 union columns per instruction, fp32 accumulation).
//
// Grid: (row tiles of R = 128 or 256 rows) x (input chunks). Every workgroup
//   1. re-evaluates the B predicates for its chunk (x, c and the B gate
//      pairs), ORs them, compacts the union columns with wavefront ballots and
//      writes the zero-filled X_U tile to LDS (k-contiguous per token);
//   2. walks the union in steps of 32 columns: the step's W tile (32 columns
//      of R contiguous rows, 16-byte loads) goes to LDS in column order with a
//      padded pitch, and the MFMA A operand (one row, eight union columns per
//      lane) is read back with two transposing LDS reads (ds_read_b64_tr_b16)
//      free of bank conflicts; the loads of the next D steps are in flight
//      while the current one is multiplied;
//   3. stages its [R][B] partial through LDS so that every wavefront adds 64
//      consecutive rows of one token into Y: fp32 atomics, or the ordered
//      last-arrival reduction (bit-reproducible; bf16 outputs).
//
// Union column order inside a step. The contraction may take the 32 columns
// of a step in any order as long as A and B agree. Lane l (group G = l / 16)
// holds, as its eight k elements, the columns 4G + q (q = 0..3) and then
// 16 + 4G + q: each half is one transposing read of four consecutive columns
// per 16-lane group, and for the B operand one 8-byte read of X_U, which is
// stored k-contiguous per token.
#include "device_common.h"
#include "internal.h"

#include <algorithm>

namespace {

using namespace sl::dev;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int UT = 256;             // threads per workgroup (4 wavefronts)
constexpr int UK = 32;              // union columns per step (one MFMA k-depth)
// bytes per token row of X_U: 16 mod 256, so the 16 tokens of an 8-byte
// operand read fall on disjoint banks
constexpr int XPITCH = 2 * sl::kUnionMaxChunk + 16;

// Transposing LDS read: within each 16-lane group, lane i supplies the address
// of four consecutive bf16; lane l receives element (l mod 4) of the rows that
// lanes 4q + (l mod 16) / 4 addressed, q = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
}

__device__ __forceinline__ i16x4 lds_read_b64(const uint8_t* p) { return *(const i16x4*)p; }

// NB: 16-row MFMA blocks per wavefront (tile of R = 64 * NB rows); D: column
// steps whose loads are in flight ahead of the one being multiplied; SPEC:
// the first D steps are loaded before the union is known (a compile-time
// choice: behind a run-time branch the wait for the x loads became a wait
// for every load in flight, the speculative weights included).
template <typename YT, bool ATOMIC, int NB, int D, bool SPEC>
__global__ __launch_bounds__(UT) void union_kernel(const uint16_t* __restrict__ Wt, const uint16_t* __restrict__ x,
                                                   const float* __restrict__ c,
                                                   const sl::GateOut* __restrict__ gout, int m, int n, int B,
                                                   int tiles, int splits, int chunk, bool dense,
                                                   float* __restrict__ partials, uint32_t* __restrict__ ctr,
                                                   YT* __restrict__ y) {
  constexpr int UR = 64 * NB;          // rows per tile
  // bytes per staged column: 2R + 32 (32 mod 256), so the eight 32-byte
  // column pieces that 32 lanes of a transposing read address fall on
  // disjoint LDS banks; a multiple of 16 keeps the tile stores 16-byte wide
  constexpr int WPITCH = 2 * UR + 32;
  // fp32 [token][row] staging of the partial in phase 3 (reuses ws)
  constexpr int OPITCH = 4 * UR + 16;
  static_assert(16 * OPITCH <= 2 * UK * WPITCH, "partial staging must fit the W buffers");
  __shared__ __align__(16) uint8_t ws[2][UK * WPITCH];     // staged W tiles, column-major
  __shared__ __align__(16) uint8_t xu[16 * XPITCH];        // X_U, [token][k] bf16
  __shared__ uint16_t ulist[sl::kUnionMaxChunk + UK];      // union columns, offsets from j0
  __shared__ uint32_t wcnt[sl::kUnionMaxChunk / UT][4];
  __shared__ uint32_t s_last;

  const int tile = blockIdx.x % tiles;
  const int split = blockIdx.x / tiles;
  const int t = threadIdx.x, lane = t & 63, w = wave_id();
  const int j0 = split * chunk;
  const int j1 = min(j0 + chunk, n);
  const int row0 = tile * UR;
  constexpr int ROUNDS = sl::kUnionMaxChunk / UT;

  // 1. union of the B kept sets over this chunk, and the X_U tile
  const int nr = (j1 - j0 + UT - 1) / UT;
  uint32_t tmask[ROUNDS];
  uint64_t bal[ROUNDS];
  uint16_t xr[ROUNDS][16];
  float cr[ROUNDS];
  // the B gate pairs: lane b of every wavefront loads token b's pair, first
  // of all loads (one vector load; as 16 scalar loads the compiler issued
  // them in three dependent batches), and the pairs are read out per token
  // below; tokens >= B keep nothing, the dense product keeps everything
  const uint64_t* gp = (const uint64_t*)gout;  // GateOut: kthr, jlast first
  const uint64_t gpair = gp[(size_t)((lane & 15) < B ? (lane & 15) : 0) * (sizeof(sl::GateOut) / 8)];
  // all loads unconditional (token and input indices clamped) so they are in
  // flight together, and issued before any weight load (vector loads complete
  // in order); values of tokens >= B are masked out below
#pragma unroll
  for (int q = 0; q < ROUNDS; ++q) {
    const int j = j0 + q * UT + t;
    const int jc = j < j1 ? j : j1 - 1;
#pragma unroll
    for (int b = 0; b < 16; ++b) xr[q][b] = x[(size_t)(b < B ? b : B - 1) * n + jc];
    cr[q] = c[jc];
  }
  // Operand staging for step 2 (set up first: with spec the first D steps
  // are loaded before the union is known). Thread t moves NB 16-byte vectors
  // per step: vector v = t + UT * i covers rows 8 * (v mod R/8) .. +8 of step
  // column v / (R/8).
  constexpr int VPC = UR / 8;  // 16-byte vectors per column run
  int lcol[NB], lrow[NB];
  const uint16_t* gsrc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int v = t + UT * i;
    lcol[i] = v / VPC;
    lrow[i] = (v % VPC) * 8;
    // clamped into range; rows >= m are loaded from row m - 8 and never written
    gsrc[i] = Wt + (size_t)j0 * m + min(row0 + lrow[i], m - 8);
  }
  f32x4 acc[NB];
#pragma unroll
  for (int h = 0; h < NB; ++h) acc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int rb = w * 16 * NB;  // this wavefront's rows inside the tile
  const int ti = lane & 15;    // token (B operand column) / row within block
  const int kg = lane >> 4;    // k group (G)
  // transposing-read address of this lane: column 4G + ti/4 (+16 for the
  // second half), rows rb + 4 (ti mod 4) .. +4 (+16 per block h)
  const int aoff = (4 * kg + (ti >> 2)) * WPITCH + 2 * (rb + 4 * (ti & 3));
  u32x4 pr[D][NB];             // ring of prefetched steps: step q lives in slot q % D
  auto gload = [&](int slot, int q) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int col = ulist[q * UK + lcol[i]];
      pr[slot][i] = __builtin_nontemporal_load((const u32x4*)(gsrc[i] + (size_t)col * m));
    }
  };
  auto lstore = [&](int slot, int buf) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      *(u32x4*)(ws[buf] + lcol[i] * WPITCH + 2 * lrow[i]) = pr[slot][i];
    }
  };
  // Speculation (near-dense unions, chosen by the host from the expected
  // union density): the first D steps of a dense prefix, i.e. chunk columns
  // 0 .. 32 D - 1 (clamped into the chunk), go out now; they are kept once
  // the union turns out to start with exactly those columns.
  if constexpr (SPEC) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int col = min(d * UK + lcol[i], j1 - j0 - 1);
        pr[d][i] = __builtin_nontemporal_load((const u32x4*)(gsrc[i] + (size_t)col * m));
      }
    }
  }
  // (read out only after every load above has been issued)
  __builtin_amdgcn_sched_barrier(0);
  uint32_t gk[16];
  int gj[16];
#pragma unroll
  for (int b = 0; b < 16; ++b) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)gpair, b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(gpair >> 32), b);
    const bool tok = b < B;
    gk[b] = !tok ? 0xffffffffu : dense ? 0u : lo;
    gj[b] = !tok ? -1 : dense ? n : (int)hi;
  }
#pragma unroll
  for (int q = 0; q < ROUNDS; ++q) {
    const int j = j0 + q * UT + t;
    const int jc = j < j1 ? j : j1 - 1;
    const float cv = cr[q];
    uint32_t mk = 0u;
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const float xv = __uint_as_float((uint32_t)xr[q][b] << 16);
      mk |= gate_keep(score_key(xv, cv), jc, gk[b], gj[b]) ? (1u << b) : 0u;
    }
    tmask[q] = (q < nr && j < j1) ? mk : 0u;
    bal[q] = __ballot(tmask[q] != 0u);
    if (lane == 0) wcnt[q][w] = (uint32_t)__popcll(bal[q]);
  }
  __syncthreads();
  int cnt = 0;
#pragma unroll
  for (int q = 0; q < ROUNDS; ++q) {
    if (q < nr) {
      uint32_t off = (uint32_t)cnt;
      for (int k = 0; k < w; ++k) off += wcnt[q][k];
      if (tmask[q] != 0u) {
        const int pos = (int)(off + lanes_below(bal[q]));
        ulist[pos] = (uint16_t)(q * UT + t);
#pragma unroll
        for (int b = 0; b < 16; ++b)
          *(uint16_t*)(xu + b * XPITCH + 2 * pos) = ((tmask[q] >> b) & 1u) ? xr[q][b] : (uint16_t)0;
      }
      cnt += (int)(wcnt[q][0] + wcnt[q][1] + wcnt[q][2] + wcnt[q][3]);
    }
  }
  // pad the union to a multiple of UK: column j0 (any valid one) with zero inputs
  const int cntp = (cnt + UK - 1) / UK * UK;
  for (int k = cnt + t; k < cntp; k += UT) {
    ulist[k] = 0;
    for (int b = 0; b < 16; ++b) *(uint16_t*)(xu + b * XPITCH + 2 * k) = 0;
  }
  __syncthreads();

  // 2. stream the union columns' row tiles through LDS into the MFMAs
  const int nsteps = cntp / UK;
  // the speculative loads hold iff the union's first min(cnt, 32 D) columns
  // are chunk columns 0, 1, ... (the union list is ascending and distinct, so
  // its last entry there decides); steps past cnt are padding (zero inputs)
  const int L = min(cnt, D * UK);
  const bool held = SPEC && (L == 0 || ulist[L - 1] == L - 1);
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (d < nsteps && !held) gload(d, d);
  if (nsteps > 0) lstore(0, 0);
  __syncthreads();
  if (D < nsteps) gload(0, D);
  for (int s0 = 0; s0 < nsteps; s0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int s = s0 + u;  // s % D == u
      if (s < nsteps) {
        // B operand: X_U[the lane's eight step columns][token ti]
        const uint8_t* xb = xu + ti * XPITCH + 2 * (s * UK + 4 * kg);
        const bf16x8 bop = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(lds_read_b64(xb), lds_read_b64(xb + 32), 0, 1, 2, 3, 4, 5, 6, 7));
        const uint8_t* wb = ws[s & 1] + aoff;
#pragma unroll
        for (int h = 0; h < NB; ++h) {
          // A operand: W[row rb + 16h + ti][the same eight columns]
          const i16x4 lo = lds_read_tr(wb + 32 * h);
          const i16x4 hi = lds_read_tr(wb + 16 * WPITCH + 32 * h);
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bop, acc[h], 0, 0, 0);
        }
        if (s + 1 < nsteps) lstore((u + 1) % D, (s + 1) & 1);
        __syncthreads();
        if (s + 1 + D < nsteps) gload((u + 1) % D, s + 1 + D);
      }
    }
  }

  // 3. partial [rows][tokens] of this chunk into Y. Lane holds rows
  //    rb + 16h + 4*kg + q for token ti; after the last step's barrier the W
  //    buffers are free and take the partial as fp32 [token][row].
  uint8_t* ob = &ws[0][0];
#pragma unroll
  for (int h = 0; h < NB; ++h) *(f32x4*)(ob + ti * OPITCH + 4 * (rb + 16 * h + 4 * kg)) = acc[h];
  __syncthreads();
  const bool ordered = !(splits == 1 || ATOMIC);
  for (int e = t; e < UR * B; e += UT) {
    const int tk = e / UR, r = e % UR, row = row0 + r;
    if (row < m) {
      const float v = *(const float*)(ob + tk * OPITCH + 4 * r);
      if (splits == 1)
        store_out(y + (size_t)tk * m + row, v);
      else if (ATOMIC)
        atomicAdd((float*)(y + (size_t)tk * m + row), v);
      else
        __hip_atomic_store(partials + ((size_t)split * B + tk) * m + row, v, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (!ordered) return;
  // ordered reduction: the device-coherent partial stores [split][token][row]
  // above are complete; the last arrival of the tile adds them in split order
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (t == 0)
    s_last = (__hip_atomic_fetch_add(&ctr[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              (uint32_t)(splits - 1))
                 ? 1u
                 : 0u;
  __syncthreads();
  if (s_last == 0u) return;
  for (int e = t; e < UR * B; e += UT) {
    const int tk = e / UR, row = row0 + e % UR;
    if (row < m) {
      float s = 0.f;
      const float* pp = partials + (size_t)tk * m + row;
      int k = 0;
      for (; k + 7 < splits; k += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = __hip_atomic_load(pp + (size_t)(k + u) * B * m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
      }
      for (; k < splits; ++k)
        s += __hip_atomic_load(pp + (size_t)k * B * m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      store_out(y + (size_t)tk * m + row, s);
    }
  }
  if (t == 0) __hip_atomic_store(&ctr[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename YT, bool ATOMIC, int NB, int D>
hipError_t go_nd(const sl_linear* h, const sl::UnionPlan& p, const void* x, int B, bool dense, void* y,
                 hipStream_t s) {
  if (p.spec)
    union_kernel<YT, ATOMIC, NB, D, true><<<p.tiles * p.splits, UT, 0, s>>>(
        (const uint16_t*)h->Wt, (const uint16_t*)x, h->c, h->gout, (int)h->m, (int)h->n, B, p.tiles, p.splits,
        p.chunk, dense, h->upartials, h->uctr, (YT*)y);
  else
    union_kernel<YT, ATOMIC, NB, D, false><<<p.tiles * p.splits, UT, 0, s>>>(
        (const uint16_t*)h->Wt, (const uint16_t*)x, h->c, h->gout, (int)h->m, (int)h->n, B, p.tiles, p.splits,
        p.chunk, dense, h->upartials, h->uctr, (YT*)y);
  return hipGetLastError();
}

template <typename YT, bool ATOMIC, int NB, int D>
int per_cu_nd() {
  static const int nb = [] {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, union_kernel<YT, ATOMIC, NB, D, true>, UT, 0) != hipSuccess)
      v = 1;
    return std::max(1, v);
  }();
  return nb;
}

template <typename YT, bool ATOMIC>
int per_cu(int rows) {
  return rows == 256 ? per_cu_nd<YT, ATOMIC, 4, 2>() : per_cu_nd<YT, ATOMIC, 2, 4>();
}

template <typename YT, bool ATOMIC>
hipError_t go(const sl_linear* h, const sl::UnionPlan& p, const void* x, int B, bool dense, void* y,
              hipStream_t s) {
  if (p.rows == 256) return go_nd<YT, ATOMIC, 4, 2>(h, p, x, B, dense, y, s);
  return go_nd<YT, ATOMIC, 2, 4>(h, p, x, B, dense, y, s);
}

}  // namespace

namespace sl {

int union_workgroups_per_cu(int rows, sl_dtype ydt, bool atomic) {
  if (ydt == SL_BF16) return per_cu<uint16_t, false>(rows);
  if (atomic) return per_cu<float, true>(rows);
  return per_cu<float, false>(rows);
}

hipError_t launch_union_product(const sl_linear* h, const UnionPlan& p, const void* x, int B, bool dense, void* y,
                                sl_dtype ydt, hipStream_t s) {
  if (ydt == SL_BF16) return go<uint16_t, false>(h, p, x, B, dense, y, s);
  if (p.atomic) return go<float, true>(h, p, x, B, dense, y, s);
  return go<float, false>(h, p, x, B, dense, y, s);
}

}  // namespace sl
