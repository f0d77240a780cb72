/*
 * double_sparse.h -- C ABI of Double Sparsity decode attention on AMD
 * Instinct MI355X (gfx950): token sparsity chosen through channel sparsity.
 *
 * What one decode step computes, per sequence b and head h (Double Sparsity
 * article, youleyou.com repost of 53ai.com; sections cited by heading):
 *
 *   label[t][j] = key[t][ch[j]]          the label cache: the key's values at
 *       the r calibrated outlier channels ch[0..r), kept contiguous per token
 *       (section 离线校准: filled from the key cache at prefill, appended per
 *        decode step, so that scoring reads contiguous memory)
 *   s_t = sum_{j=0..r-1} q[ch[j]] * label[t][j]     for t < n = seq_len[b]
 *       (section 在线前向计算, steps one and two: the query gathered at the same
 *        channels scores every cached token against its label row)
 *   T   = the k tokens with the largest s_t, ties to the lower index; all n
 *         tokens when n <= k (section 在线前向计算, step three)
 *   out = sum_{t in T} softmax_t(scale * q.key[t]) * value[t]
 *       (step three: ordinary attention of the full query over the full key
 *        and value rows of the kept tokens only)
 *
 * Precision: q, the caches and the label cache are bf16. s_t is an fp32 sum
 * in channel-list order starting from +0 (every bf16 x bf16 product is exact
 * in fp32), so the kept set is a deterministic function of the inputs. The
 * attention runs in fp32 (products, online softmax with exp2, sums); out is
 * fp32.
 *
 * Layouts (row-major, element strides implied):
 *   q        [batch][heads][head_dim]
 *   key      [batch][heads][max_seq][head_dim]   (one key/value head per
 *   value    [batch][heads][max_seq][head_dim]    query head)
 *   label    [batch][heads][max_seq][r]
 *   channels [heads][r] int32, each in [0, head_dim); an index outside that
 *            range is taken modulo head_dim (never read out of bounds)
 *   seq_len  [batch] int32; values are clamped to [0, max_seq]; a sequence of
 *            length 0 gets out = 0 and no kept tokens
 *
 * Memory: all array arguments are device memory of the current HIP device,
 * owned by the caller; the library allocates nothing and keeps no state.
 * Streams are hipStream_t values passed as void* (NULL = default stream).
 * Errors: arguments are checked before anything is enqueued (SL_ERR_ARG,
 * SL_ERR_UNSUPPORTED); on error nothing is launched. Launch failures map to
 * SL_ERR_HIP. sparse_linear_last_error() holds the message. NaN or Inf in q or
 * in the label cache is not detected (the kept set is then unspecified).
 */
#ifndef DOUBLE_SPARSE_H
#define DOUBLE_SPARSE_H

#include <stdint.h>

#include "sparse_linear.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Limits of the library. */
#define DS_MAX_SEQ 32768  /* cached tokens per sequence (scores live in registers) */
#define DS_MAX_K 8192     /* kept tokens when k < max_seq (the kept list lives in LDS) */

/*
 * ds_label_cache_update -- copy the label channels of cached keys into the
 * label cache (Double Sparsity article, section 离线校准: prefill fills the
 * label cache from the key cache; every decode step appends the new token).
 *
 *   key, label, channels   as above (bf16 key and label; int32 channels)
 *   start    device int32[batch] first token to update per sequence, or NULL
 *            for 0; tokens start[b] .. start[b] + span - 1 are updated, those
 *            outside [0, max_seq) skipped
 *   span     tokens per sequence (prefill: the prompt length; decode: 1)
 *   head_dim 64 or 128; r 8, 16 or 32; label 16-byte aligned
 *
 * The copy is exact (bf16 values moved, not converted).
 */
sl_status ds_label_cache_update(const void* key, void* label, const int32_t* channels, const int32_t* start,
                                int32_t batch, int32_t heads, int32_t max_seq, int32_t head_dim, int32_t r,
                                int32_t span, void* stream);

/*
 * ds_decode_attention -- one decode step of Double Sparsity attention for a
 * batch of sequences (Double Sparsity article, section 在线前向计算, steps
 * one to three).
 *
 *   q, key, value, label, channels, seq_len   as above
 *   k          heavy tokens kept per (sequence, head): 1 <= k, and k <= DS_MAX_K
 *              unless k >= max_seq; a sequence with n <= k tokens attends to all
 *              of them and its label rows are not read (label may be NULL when
 *              k >= max_seq)
 *   scale      softmax scale (1/sqrt(head_dim) for the usual attention)
 *   out        device fp32 [batch][heads][head_dim]
 *   tokens_out device int32 [batch][heads][k] or NULL: the kept token indices
 *              in ascending order, then -1 for the k - |T| unused slots
 *              (requires k <= DS_MAX_SEQ)
 *   head_dim 64 or 128; r 8, 16 or 32; 1 <= max_seq <= DS_MAX_SEQ;
 *   batch * heads <= 2^31 - 1. Alignment: q, key and value to 16 bytes
 *   (head_dim 128) or 8 bytes (64), label to 16 bytes (SL_ERR_UNSUPPORTED
 *   otherwise).
 *
 * One launch; no host synchronisation; deterministic (the same inputs give
 * the same bits).
 */
sl_status ds_decode_attention(const void* q, const void* key, const void* value, const void* label,
                              const int32_t* channels, const int32_t* seq_len, int32_t batch, int32_t heads,
                              int32_t max_seq, int32_t head_dim, int32_t r, int32_t k, float scale, float* out,
                              int32_t* tokens_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DOUBLE_SPARSE_H */
