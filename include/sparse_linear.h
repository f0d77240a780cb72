/*
 * sparse_linear.h -- C ABI of the weight-informed activation-sparse linear
 * layer for LLM decode on AMD Instinct MI355X (gfx950).
 *
 * What one forward computes, per token b (pages cited by title and section):
 *
 *   score_j = |x_j * c_j|,  c_j = L2 norm of column j of W
 *       (WINA article, arXiv:2505.19427, section 一: the gate ranks inputs by
 *        hidden-state magnitude times the column norm of the weight they meet)
 *   keep    = the K largest scores, ties to the lower index   (SL_GATE_TOPK,
 *             WINA article, section 一: top-K binary gate)
 *           | score > t, t = mu + sigma * Phi^-1(1 - s)        (SL_GATE_STAT,
 *             Spark Transformer article, section 2.2: statistical top-k with
 *             mean and population variance of the score vector)
 *   y       = sum over kept j of x_j * W[:, j]
 *       (Spark Transformer article, section 3.1: the index-list product that
 *        touches only the weight vectors of active inputs)
 *
 * Shapes: W is m x n (m outputs, n inputs), x is [B][n], y is [B][m].
 *
 * Memory: every pointer argument named "device" is device memory of the
 * current HIP device; handles are bound to the device current at init.
 * Streams are hipStream_t values passed as void* (NULL = the default stream).
 *
 * Errors: every argument check happens before anything is enqueued; on error
 * nothing is launched and the out-parameters are untouched. HIP runtime
 * failures map to SL_ERR_HIP. No C++ exception crosses this interface.
 * sparse_linear_last_error() returns a message for the calling thread's most
 * recent failure. NaN or Inf inside x or c is not detected: the mask is then
 * unspecified and y propagates the NaN.
 */
#ifndef SPARSE_LINEAR_H
#define SPARSE_LINEAR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sl_linear* sl_handle; /* opaque, library-owned */

typedef enum {
  SL_OK = 0,
  SL_ERR_ARG = 1,         /* invalid argument (null pointer, range)        */
  SL_ERR_UNSUPPORTED = 2, /* valid but not supported (alignment, size)     */
  SL_ERR_OOM = 3,         /* device allocation failed                      */
  SL_ERR_HIP = 4          /* HIP runtime error (no device, launch failure) */
} sl_status;

typedef enum { SL_F32 = 0, SL_BF16 = 1 } sl_dtype;

typedef enum {
  SL_W_ROWMAJOR_OUT_IN = 0, /* W[i][j] at i*n + j: the torch nn.Linear layout */
  SL_W_COLMAJOR = 1         /* W[i][j] at j*m + i: column j contiguous        */
} sl_layout;

typedef enum {
  SL_GATE_TOPK = 0,  /* exact top-K of the scores                          */
  SL_GATE_STAT = 1,  /* Gaussian-fit threshold, keep fraction s_keep        */
  SL_GATE_FIXED = 2  /* calibrated per-layer threshold: keep score > tau    */
} sl_gate;

/* Limits of the library. */
#define SL_MAX_N 32768     /* inputs per token (the gate keeps them in LDS) */
#define SL_MAX_BATCH 16    /* tokens per forward                              */

/*
 * sparse_linear_init -- build a handle for one linear layer.
 *
 *   W        device, m*n elements of w_dtype in w_layout. Copied (and, for
 *            SL_W_ROWMAJOR_OUT_IN, transposed) into handle-owned column-major
 *            storage [n][m], so that the m weights that input j multiplies are
 *            one contiguous run (the weight vector W[j] of the index-list
 *            product, Spark Transformer article, section 3.1).
 *   c        device fp32[n], the column norms, copied; or NULL, in which case
 *            the library computes c_j = fp32(sqrt(sum_i W[i][j]^2)) with an
 *            fp64 sum (WINA article, section 一). Values must be finite.
 *   gate     SL_GATE_TOPK: K in [0, n] inputs kept per token.
 *            SL_GATE_STAT: s_keep in (0, 1); z = Phi^-1(fl(1 - s_keep)) is
 *            evaluated once here with Wichura's algorithm AS241.
 *            SL_GATE_FIXED: s_keep carries tau >= 0 (rounded to fp32); the
 *            gate keeps score > tau (a per-layer threshold of the kind the
 *            WINA article, section 三, calibrates from hidden-state
 *            distributions).
 *   max_batch  1..SL_MAX_BATCH, the largest B forward will accept; sizes the
 *            per-handle scratch.
 *   stream   the stream the copies run on; init synchronizes it before
 *            returning, so caller buffers may be freed afterwards.
 *
 * Requirements: m >= 1, 1 <= n <= SL_MAX_N; m % 8 == 0 for bf16 and m % 4 == 0
 * for fp32 (16-byte column runs), else SL_ERR_UNSUPPORTED.
 * Returns SL_ERR_HIP when no HIP device is usable.
 */
sl_status sparse_linear_init(sl_handle* out, const void* W, sl_dtype w_dtype, sl_layout w_layout,
                             int64_t m, int64_t n, const float* c, sl_gate gate, int64_t K,
                             double s_keep, int32_t max_batch, void* stream);

/*
 * sparse_linear_forward -- y = W[:, keep] x[keep] for B tokens.
 *
 *   x          device [B][n], same dtype as W.
 *   y          device [B][m] of y_dtype (fp32, or bf16 rounded to nearest even
 *              from the fp32 accumulator).
 *   mask_out   device uint8 [B][n] or NULL: 1 where input j was kept.
 *   count_out  device int32 [B] or NULL: number of kept inputs.
 *   thresh_out device double [B] or NULL: t (STAT), tau (FIXED) or the K-th
 *              largest score (TOPK; +inf when K == 0).
 *
 * Each token's kept set depends only on that token. For B > 1 the library
 * forms the union of the B masks and runs one matrix-core pass over the union
 * columns, feeding zero for inputs a token did not keep. A single bf16 token
 * (n % 4 == 0, x 8-byte aligned) runs as one fused launch: one workgroup
 * selects while the others load their input chunks, then stream the kept
 * columns (see sparse_linear_set_fused).
 * Asynchronous on `stream`; the caller keeps x, y and the optional outputs
 * alive until the stream has completed. A handle's scratch is shared by its
 * calls, so one handle must not run on two streams at once.
 *
 * Failed hand-off: the fused launch's workgroups wait for each other with
 * bounded spins. A wait that gives up (about a second; in-order workgroup
 * dispatch rules it out on a working device) leaves that forward's y
 * incomplete and is recorded in a host-visible word of the handle, without
 * any synchronization. The handle's next forward (any of the forward entry
 * points) then returns SL_ERR_HIP before enqueuing anything, and
 * sparse_linear_sync_status reports it at once. Callers that must know that a
 * particular forward completed call sparse_linear_sync_status after it.
 */
sl_status sparse_linear_forward(sl_handle h, const void* x, int32_t B, void* y, sl_dtype y_dtype,
                                uint8_t* mask_out, int32_t* count_out, double* thresh_out,
                                void* stream);

/*
 * sparse_linear_forward_group -- one token through `count` linears that share
 * their input x (e.g. the q, k and v projections of a decoder block, or its
 * gate and up projections), each with its own weights, norms and gate (WINA
 * article, section 一: per-layer K; the heterogeneous per-component sparsity
 * of the WAS framework), in one launch: the linears' gate workgroups run side
 * by side and the product workgroups are shared out in proportion to each
 * linear's expected kept bytes.
 *
 *   handles    host array of `count` handles, 1 <= count <= 8, all on the
 *              current device with the same n and weight dtype.
 *   x          device [n] (one token), the weights' dtype.
 *   ys         host array of `count` device pointers, ys[l] of [m_l] y_dtype.
 *
 * y_l equals sparse_linear_forward(handles[l], x, 1, ys[l], ...) up to the
 * split reduction's summation order. The single launch is taken when every
 * handle is bf16 with the fused forward enabled and the atomic reduction, the
 * gates share their mode, y_dtype is fp32, n % 4 == 0 and x is 8-byte
 * aligned; otherwise the linears run one after another. No mask, count or
 * threshold outputs. Errors: NULL arrays or pointers, count outside 1..8,
 * differing n or dtypes, the same handle twice, a handle on another device
 * (SL_ERR_ARG); a recorded failed hand-off of any of the handles
 * (SL_ERR_HIP, see sparse_linear_forward); nothing is launched then.
 * Asynchronous on `stream`; the handles' scratch is in use until it
 * completes.
 */
sl_status sparse_linear_forward_group(const sl_handle* handles, int32_t count, const void* x, void* const* ys,
                                      sl_dtype y_dtype, void* stream);

/*
 * sparse_linear_forward_group_batch -- sparse_linear_forward_group for a
 * batch of B tokens (WINA article, section 一: each token keeps its own
 * inputs, per linear).
 *
 *   x          device [B][n], the weights' dtype.
 *   ys         host array of `count` device pointers, ys[l] of [B][m_l] y_dtype.
 *   B          1 <= B <= every handle's max_batch.
 *
 * B == 1 is sparse_linear_forward_group. For B > 1 with bf16 weights and a
 * top-K or statistical gate shared by all linears, one launch runs every
 * linear's gate for every token (count * B workgroups), then each linear's
 * matrix-core pass over the union of its B kept sets follows, as in
 * sparse_linear_forward; otherwise the linears run one after another.
 * y_l equals sparse_linear_forward(handles[l], x, B, ys[l], ...) up to the
 * split reduction's summation order. No mask, count or threshold outputs.
 * Errors: those of sparse_linear_forward_group, and B outside
 * [1, max_batch] of any handle (SL_ERR_ARG); nothing is launched then.
 */
sl_status sparse_linear_forward_group_batch(const sl_handle* handles, int32_t count, const void* x, int32_t B,
                                            void* const* ys, sl_dtype y_dtype, void* stream);

/*
 * Sparse FFN chain for one token (Spark Transformer article, section 2.1: the
 * FFN scores, selects and computes only the selected part; WINA article,
 * section 一: each projection keeps its inputs by |x_j c_j|):
 *
 *   g = gate(x), u = up(x)     one grouped launch (sparse_linear_forward_group)
 *   h = bf16(SiLU(g) * u)      SiLU(v) = v / (1 + exp(-v)) in fp32, then one
 *                              round to nearest even
 *   y = down(h)                the down projection's own gate on h
 *
 *   gate, up   handles with the same shape [m][n] (bf16 weights).
 *   down       handle of shape [m2][m] (bf16 weights): its input is h.
 *   x          device [n] bf16.
 *   y          device [m2] of y_dtype.
 *   workspace  device memory the caller owns, 256-byte aligned, of at least
 *              sparse_linear_ffn_workspace_bytes(up) bytes: g and u (fp32 [m])
 *              and h (bf16 [m]) are left there after the call.
 *
 * Errors: NULL arguments, gate, up and down not three different handles,
 * shapes that do not chain, a short or misaligned workspace (SL_ERR_ARG);
 * weights other than bf16 (SL_ERR_UNSUPPORTED).
 * Asynchronous on `stream`; the workspace is in use until it completes.
 */
int64_t sparse_linear_ffn_workspace_bytes(sl_handle up);
sl_status sparse_linear_forward_ffn(sl_handle gate, sl_handle up, sl_handle down, const void* x, void* y,
                                    sl_dtype y_dtype, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * sparse_linear_forward_ffn_noalloc -- the sparse FFN chain of
 * sparse_linear_forward_ffn for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). It calls no hipMalloc, hipFree or allocating library routine:
 * g, u and h live in a static device array of the library (200 KiB, one copy
 * per GPU, held until the process ends), whose address is looked up once per
 * device at handle init.
 *
 *   gate, up, down, x, y, y_dtype, stream   as for sparse_linear_forward_ffn.
 *
 * Limit: the intermediate width (up's m) at most 20480, else
 * SL_ERR_UNSUPPORTED. Every call on a GPU shares that GPU's array, which keeps
 * the last call's g, u and h (each call overwrites what it reads; nothing has
 * to start at zero between calls): calls that overlap on one GPU, on one
 * stream or several, race and must not be made. Other errors as for
 * sparse_linear_forward_ffn.
 */
sl_status sparse_linear_forward_ffn_noalloc(sl_handle gate, sl_handle up, sl_handle down, const void* x, void* y,
                                            sl_dtype y_dtype, void* stream);

/*
 * sparse_linear_forward_dense -- y = W x for B tokens with every input kept,
 * run by the same product kernel as the sparse path over the identity index
 * list (the dense baseline the sparse forward is compared against).
 * Same argument rules as sparse_linear_forward.
 */
sl_status sparse_linear_forward_dense(sl_handle h, const void* x, int32_t B, void* y,
                                      sl_dtype y_dtype, void* stream);

/* Copy the handle's fp32 norm vector c into device fp32[n] (stream-ordered). */
sl_status sparse_linear_get_norms(sl_handle h, float* c_out, void* stream);

/* Release a handle. The handle's last stream must be idle. NULL is a no-op. */
sl_status sparse_linear_destroy(sl_handle h);

/* Static description of a status code. */
const char* sparse_linear_strerror(sl_status s);

/* Message for the calling thread's most recent failure ("" if none). */
const char* sparse_linear_last_error(void);

/*
 * Phi^-1(p) for 0 < p < 1 by Wichura's AS241 (Applied Statistics 37, 1988),
 * evaluated in fp64 on the host exactly as the STAT gate's init does. Returns
 * NaN outside (0, 1). Host-only; needs no device.
 */
double sparse_linear_normal_quantile(double p);

/*
 * sparse_linear_forward_stages -- run part of a forward, for measurement.
 * stages is a bit mask: SL_STAGE_GATE (scores and selection, writes the
 * optional outputs) and SL_STAGE_PRODUCT (the gathered product, using the
 * selection the handle's most recent gate stage left for those B tokens).
 * stages == SL_STAGE_GATE | SL_STAGE_PRODUCT is exactly sparse_linear_forward.
 * Running the product stage alone repeats the previous selection's product;
 * it lets a caller time each kernel on its own. Other arguments as for
 * sparse_linear_forward; stages outside 1..3 give SL_ERR_ARG.
 */
#define SL_STAGE_GATE 1
#define SL_STAGE_PRODUCT 2
sl_status sparse_linear_forward_stages(sl_handle h, const void* x, int32_t B, void* y, sl_dtype y_dtype,
                                       uint8_t* mask_out, int32_t* count_out, double* thresh_out,
                                       int32_t stages, void* stream);

/*
 * sparse_linear_gather_ceiling -- measurement only: read the handle's weight
 * columns idx[0 .. count) (device int32, each clamped into [0, n)) once, with
 * no gate, no product and no output beyond a checksum that is never stored in
 * practice (sink: device fp32[1], written only if the checksum hits a fixed
 * value). Its duration is the practical bandwidth ceiling of gathering the
 * same weight bytes that a forward with that kept set reads (Spark
 * Transformer article, section 3.1: only the active inputs' weight vectors
 * are read). count in [0, n], else SL_ERR_ARG; count == 0 launches nothing.
 * Asynchronous on `stream`.
 */
sl_status sparse_linear_gather_ceiling(sl_handle h, const int32_t* idx, int32_t count, float* sink, void* stream);

/*
 * sparse_linear_set_timeline -- measurement only: installs buf (device
 * uint64[32 * workgroups], caller-owned, zeroed by the caller) as the
 * per-workgroup timestamp buffer of the fused single-token forward, or
 * removes it (buf == NULL). While installed, every fused launch writes, for
 * workgroup b, the 100 MHz clock (s_memrealtime) at named points into word
 * 32 * b + slot: gate workgroup (b = 0): 0 start, 3 keys in, 7/8/9/10/11 the
 * top-K phases (first barrier, histogram, pivot bin, candidates, ranked);
 * for the statistical gate 14 keys in, 15 largest and smallest score known,
 * 16 row totals of the moment sums, 17 all row totals in LDS, 12 totals
 * summed, 13 mu, sigma and t computed (one lane) and 5 threshold known; then 6 selection done, 1 pair
 * published, 2 acknowledgements in; product workgroups: 0 start,
 * 1 speculative list compacted (21: its length, held band included),
 * 2 early poll back (20: the value it read), 3 pair seen by the second poll,
 * 4 + w end of wavefront w's stream, 22 end. Only the timeline build of the
 * library (libsparse_linear_timeline.so) records anything; the regular
 * library returns SL_ERR_UNSUPPORTED. Timestamps add a few stores per
 * workgroup, so absolute times run ~10 % above an uninstrumented launch.
 */
sl_status sparse_linear_set_timeline(void* buf);

/*
 * Split reduction mode. The product kernel splits the kept inputs into chunks
 * whose partial sums are added per output row. By default (on == 0) fp32
 * outputs take fp32 atomic adds, which is fastest but lets the summation order
 * vary between runs in the last bits. With on != 0 the partials are added in a
 * fixed order (bit-reproducible runs). bf16 outputs always use the fixed order.
 */
sl_status sparse_linear_set_deterministic(sl_handle h, int32_t on);

/*
 * Fused single-token forward (on != 0, the default) or the two-launch form
 * (gate kernel, then product kernel) for comparison. Both give the same
 * selection and outputs within the split reduction's summation order.
 */
sl_status sparse_linear_set_fused(sl_handle h, int32_t on);

/*
 * Synchronize `stream` and report whether any fused forward of this handle
 * since the last report had a hand-off wait time out (its gate workgroup not
 * running within about a second, which in-order workgroup dispatch rules out
 * on an otherwise working device). Returns SL_OK, or SL_ERR_HIP with
 * sparse_linear_last_error describing the wait; the record is then cleared.
 * Such a forward's y is incomplete. Without this call the record is reported
 * by the handle's next forward (see sparse_linear_forward).
 */
sl_status sparse_linear_sync_status(sl_handle h, void* stream);

/*
 * Launch-shape override for tuning sweeps: rows_per_tile in {128, 256, 512}
 * (0 = automatic) and splits >= 0 (0 = automatic) for the single-token product
 * kernel and the fused forward. Takes effect on the next forward.
 */
sl_status sparse_linear_set_plan(sl_handle h, int32_t rows_per_tile, int32_t splits);

/*
 * Launch-shape override of the batched (B > 1, bf16) union product:
 * rows_per_tile in {128, 256} (0 = automatic) and the target number of
 * workgroups (0 = automatic; input chunks stay within 256..512).
 */
sl_status sparse_linear_set_union_plan(sl_handle h, int32_t rows_per_tile, int32_t workgroups);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_LINEAR_H */
