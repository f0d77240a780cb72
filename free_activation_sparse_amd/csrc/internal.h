// Internal declarations shared by the host runtime and the gfx950 kernels of
// the weight-informed activation-sparse linear layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "double_sparse.h"
#include "sparse_linear.h"

namespace sl {

// Per-token result of the gate. The kept set is
//   { j : key_j > kthr  or  (key_j == kthr and j <= jlast) }
// where key_j is the fp32 bit pattern of score_j = |x_j * c_j| (non-negative,
// so unsigned order equals numeric order). Every gate mode reduces to this
// form: top-K puts the K-th largest key in kthr and the index of the last kept
// tie in jlast; a threshold t >= 0 becomes kthr = bits(round_down_f32(t)),
// jlast = -1.
struct GateOut {
  uint32_t kthr;
  int32_t jlast;
  int32_t count;
  int32_t pad;
  double thresh;
};
static_assert(sizeof(GateOut) == 24, "GateOut layout");

// Scratch limits of the single-token product kernel.
constexpr int kMaxSplits = 1024;   // K-splits per row tile
constexpr int kMaxChunk = 1024;    // inputs examined per workgroup
constexpr int kUnionMaxChunk = 512;  // inputs per workgroup of the union product
constexpr int kUnionMinChunk = 256;  // sizes the union partial buffer

struct Plan {
  int lpc;     // lanes per column run (16, 32 or 64)
  int rows;    // rows per tile (lpc * elements per 16-byte load)
  int tiles;   // ceil(m / rows)
  int splits;  // input chunks
  int chunk;   // inputs per chunk
  int unroll;  // columns in flight per lane group
  bool atomic; // fp32 atomic split reduction into y (else ordered, reproducible)
};

// Matrix-core (union) product plan.
struct UnionPlan {
  int rows;    // rows per tile: 128 or 256
  int tiles;   // row tiles
  int splits;  // input chunks
  int chunk;   // inputs per chunk (kUnionMinChunk..kUnionMaxChunk unless n is smaller)
  bool atomic; // fp32 atomic split reduction (else ordered, reproducible)
  bool spec;   // load the first steps before the union is known, assuming a dense prefix
};

// Hand-off from the gate workgroup to the product workgroups of one fused
// launch (device memory, zero between launches). Acknowledgements are spread
// over kAckSlots counters on separate 64-byte lines, so that the product
// workgroups' atomic increments do not queue on one address.
constexpr int kAckSlots = 64;
struct FusedSync {
  uint64_t flag;  // 0, or the kept-set pair: kthr | (jlast + 2) << 32
  uint32_t pad[14];
  uint32_t ack[kAckSlots * 16];  // slot i at ack[16 * i]: product workgroups pw = i mod kAckSlots
};
static_assert(sizeof(FusedSync) == 64 + 64 * kAckSlots, "FusedSync layout");

}  // namespace sl

struct sl_linear {
  int device = 0;
  int64_t m = 0, n = 0;
  sl_dtype wdt = SL_BF16;
  sl_gate gate = SL_GATE_TOPK;
  int64_t K = 0;
  double s_keep = 0.0;
  double z = 0.0;     // Phi^-1(fl(1 - s_keep)), STAT
  float tau = 0.0f;   // FIXED
  int max_batch = 1;

  void* Wt = nullptr;           // column-major [n][m], wdt
  float* c = nullptr;           // [n]
  sl::GateOut* gout = nullptr;  // [max_batch]
  float* partials = nullptr;    // [kMaxSplits * m] (single-token product)
  uint32_t* ctr = nullptr;      // [tiles] arrival counters, self-resetting
  int64_t ctr_len = 0;
  float* upartials = nullptr;   // [usplits][max_batch][m] (union product)
  int64_t upart_len = 0;
  uint32_t* uctr = nullptr;     // [utiles]
  sl::FusedSync* fsync = nullptr;  // fused gate + product hand-off
  // Timed-out hand-off record of the fused forward: pinned, mapped host memory
  // that the kernels write (system scope) and the host reads without a
  // synchronization; 1 = a product workgroup's wait for the gate, 2 = the gate
  // workgroup's wait for the product workgroups.
  uint32_t* herr = nullptr;        // host address
  uint32_t* herr_dev = nullptr;    // the same word as the device sees it
  int cus = 0;                     // compute units of the device

  int plan_rows = 0, plan_splits = 0;  // overrides (0 = automatic)
  int uplan_rows = 0, uplan_wgs = 0;   // union-product overrides (0 = automatic)
  bool deterministic = false;          // ordered split reduction for fp32 y too
  bool fused = true;                   // single-token forwards in one launch

};

namespace sl {

// Launchers (each returns the launch's hipError_t).
hipError_t launch_repack(const void* W, sl_dtype dt, int64_t m, int64_t n, void* Wt, hipStream_t s);
hipError_t launch_norms(const void* Wt, sl_dtype dt, int64_t m, int64_t n, float* c, hipStream_t s);
hipError_t launch_gate(const sl_linear* h, const void* x, int B, uint8_t* mask_out,
                       int32_t* count_out, double* thresh_out, float* zero_y, hipStream_t s);
hipError_t launch_zero(float* y, int64_t count, hipStream_t s);
hipError_t launch_product(const sl_linear* h, const Plan& p, const void* x, const GateOut* g, bool dense,
                          void* y, sl_dtype ydt, hipStream_t s);
// Static workspace of the allocation-free FFN chain: intermediate widths up to
// kFfnScratchMaxM (g, u fp32 and h bf16, each piece 256-byte aligned; the
// widest FFN of the Llama-2/3, Phi-4 and Qwen2.5 shapes is 18944).
constexpr int64_t kFfnScratchMaxM = 20480;
constexpr size_t kFfnScratchBytes = 2 * (4 * kFfnScratchMaxM) + 2 * kFfnScratchMaxM;  // 200 KiB
static_assert(kFfnScratchMaxM % 128 == 0, "every workspace piece stays 256-byte aligned");
// Device address of the static FFN workspace on `device`, which must be the
// current device; looked up once per device (hipGetSymbolAddress) and cached.
hipError_t ffn_scratch(int device, void** ptr);
// h = bf16(SiLU(g) * u) over m values (sparse FFN chain epilogue).
hipError_t launch_silu_mul(const float* g, const float* u, uint16_t* h, int64_t m, hipStream_t s);
// Grouped fused forward (one token) of count <= 8 linears that share x: all
// fused_supported, the same n and gate mode, fp32 y, atomic reduction.
constexpr int kMaxGroupLinears = 8;
// The gates of `count` bf16 linears that share x ([B][n]), top-K or
// statistical (the same mode), in one launch; zero_y[l] (or NULL) is cleared
// for linear l's atomic union product.
hipError_t launch_gate_group(const sl_linear* const* hs, int count, const void* x, int B, float* const* zero_y,
                             hipStream_t s);
hipError_t launch_fused_group(const sl_linear* const* hs, int count, const void* x, float* const* ys,
                              hipStream_t s);
// Fused gate + product for one token (bf16 weights, any gate, n % 4 == 0 and
// x 8-byte aligned: fused_supported).
bool fused_supported(const sl_linear* h, const void* x);
// Installs (or, with nullptr, removes) the per-workgroup timestamp buffer of
// the fused forward; hipErrorNotSupported unless fused.hip was compiled with
// SL_TIMELINE (the timeline build of the library).
hipError_t timeline_set(void* buf);
hipError_t launch_fused(const sl_linear* h, const void* x, GateOut* g, uint8_t* mask_out, int32_t* count_out,
                        double* thresh_out, void* y, sl_dtype ydt, bool atomic, hipStream_t s);
// Double Sparsity decode attention (layouts and semantics in double_sparse.h).
struct DsDecodeParams {
  const uint16_t* q;
  const uint16_t* key;
  const uint16_t* value;
  const uint16_t* label;
  const int32_t* channels;
  const int32_t* seq_len;
  int heads, max_seq, k;
  float scale_log2;  // softmax scale * log2(e)
  float* out;
  int32_t* tokens_out;
};
hipError_t launch_ds_decode(const DsDecodeParams& p, int batch, int head_dim, int r, hipStream_t s);
hipError_t launch_ds_label(const uint16_t* key, uint16_t* label, const int32_t* channels, const int32_t* start,
                           int batch, int heads, int max_seq, int head_dim, int r, int span, hipStream_t s);
// Read-only gather of the columns idx[0 .. count) (bandwidth ceiling probe).
hipError_t launch_gather_ceiling(const sl_linear* h, const int32_t* idx, int count, float* sink, hipStream_t s);
// Union-product workgroups resident per compute unit (occupancy query).
int union_workgroups_per_cu(int rows, sl_dtype ydt, bool atomic);
hipError_t launch_union_product(const sl_linear* h, const UnionPlan& p, const void* x, int B,
                                bool dense, void* y, sl_dtype ydt, hipStream_t s);

}  // namespace sl
