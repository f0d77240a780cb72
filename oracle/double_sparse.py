"""Plain reference of Double Sparsity decode attention (numpy, fp64 attention).

TEST INFRASTRUCTURE ONLY: the product path never imports, calls or links
anything here; only tests, the smoke check and the benchmark's CPU leg do. It
shares no code with the HIP library.

Definitions followed (Double Sparsity article, youleyou.com repost of
53ai.com; sections cited by their headings):

* ``label_cache`` -- section 离线校准 (offline calibration): the label cache
  holds, for every cached token, the key's values at the calibrated important
  ("outlier") channels, stored contiguously; prefill copies them from the key
  cache, each decode step appends the new token's. Stored in the key cache's
  dtype (the 4-bit label storage the section mentions is a compression whose
  quantiser the pages do not give; not modelled).
* ``approx_scores`` -- section 在线前向计算 (online forward), steps one and
  two: gather the query at the same channels, then score every cached token
  by the dot product of that sparse query with the token's label row.
  Precision reading: the pages fix none, and these scores decide which tokens
  are kept, so they are computed as fp32 sums in channel-list order starting
  from +0 (for bf16 operands every product is exact in fp32, so this is the
  sequential fp32 fused multiply-add the kernel performs, bit for bit).
* ``heavy_tokens`` -- same section, step three: keep the k tokens with the
  largest approximate scores (signed: largest value, not magnitude); ties go
  to the lower token index, a total order that makes the set unique. A
  sequence of n <= k tokens keeps all of them.
* ``sparse_attention`` -- same section, step three: ordinary attention of the
  full query over the full key and value rows of the kept tokens,
  softmax(scale * q.K^T) V, in fp64. An empty token set gives zeros.
* ``decode`` -- the three steps for every (sequence, head) pair of a batch.

Parity pins (tests/test_oracle_double_sparse.py): a hand-derived example with
closed-form outputs (selection order, sign, ties, scale), dense attention
against torch's scaled_dot_product_attention (k >= n), full-channel scores
against exact q.k selections, brute-force pairwise dominance of the kept set,
and invariance of the output to the content of unkept cache rows.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .sparse_linear import as_f64


def _as_f32(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a.astype(np.float32)


def label_cache(key: np.ndarray, channels: np.ndarray) -> np.ndarray:
    """label[..., h, t, j] = key[..., h, t, channels[h, j]] (values copied as
    stored). key: [..., H, S, d]; channels: [H, r] indices into d."""
    key = np.asarray(key)
    channels = np.asarray(channels)
    H = key.shape[-3]
    out = np.empty(key.shape[:-1] + (channels.shape[1],), key.dtype)
    for h in range(H):
        out[..., h, :, :] = key[..., h, :, :][..., channels[h]]
    return out


def approx_scores(q: np.ndarray, label: np.ndarray, channels: np.ndarray, n: int) -> np.ndarray:
    """One (sequence, head): q [d], label [S][r], channels [r]; float32 scores
    of tokens 0..n-1, summed over j = 0..r-1 in that order from +0."""
    qf = _as_f32(q)
    lf = _as_f32(label)[:n]
    acc = np.zeros(n, np.float32)
    for j, ch in enumerate(np.asarray(channels).tolist()):
        acc = acc + np.float32(qf[ch]) * lf[:, j]
    return acc


def heavy_tokens(scores: np.ndarray, k: int) -> np.ndarray:
    """Ascending indices of the k largest scores (ties: lower index first)."""
    s = np.asarray(scores)
    n = s.shape[0]
    if k >= n:
        return np.arange(n, dtype=np.int64)
    order = np.lexsort((np.arange(n), -s.astype(np.float64)))
    return np.sort(order[:k])


def sparse_attention(q: np.ndarray, key: np.ndarray, value: np.ndarray, idx: np.ndarray,
                     scale: float) -> np.ndarray:
    """softmax(scale * K[idx] q) over the kept tokens, times V[idx]; fp64."""
    qd = as_f64(q)
    idx = np.asarray(idx, dtype=np.int64)
    if idx.size == 0:
        return np.zeros(qd.shape[0])
    Ks = as_f64(key[idx])
    Vs = as_f64(value[idx])
    logits = (Ks @ qd) * scale
    w = np.exp(logits - logits.max())
    return (w @ Vs) / w.sum()


def decode(q: np.ndarray, key: np.ndarray, value: np.ndarray, channels: np.ndarray,
           seq_len: np.ndarray, k: int, scale: Optional[float] = None,
           label: Optional[np.ndarray] = None):
    """All (b, h) pairs. q [B][H][d], key/value [B][H][S][d], channels [H][r],
    seq_len [B]. Returns (out [B][H][d] fp64, kept: list of lists of index
    arrays). The label cache is built from the key cache unless given."""
    B, H, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if label is None:
        label = label_cache(key, channels)
    out = np.zeros((B, H, d))
    kept = []
    for b in range(B):
        n = int(seq_len[b])
        row = []
        for h in range(H):
            s = approx_scores(q[b, h], label[b, h], channels[h], n)
            idx = heavy_tokens(s, k)
            out[b, h] = sparse_attention(q[b, h], key[b, h], value[b, h], idx, scale)
            row.append(idx)
        kept.append(row)
    return out, kept
