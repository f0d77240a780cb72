"""Plain fp64 reference of the weight-informed activation-sparse linear.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports, calls or links anything here.

Definitions followed (pages cited by title and section):

* ``column_norms`` -- WINA article, section 一 (weight-aware activation) and
  section 二 (theory): c_j is the L2 norm of column j of W, the column that
  input x_j multiplies. Computed as the fp64 sum of squares (exact squares of
  bf16/fp32 values), fp64 sqrt, one rounding to fp32.
* ``scores`` -- WINA article, section 一: score_j = |x_j * c_j|. The product of
  two fp32 values is exact in fp64, so one rounding to fp32 reproduces an IEEE
  fp32 multiply bit for bit.
* ``topk_gate`` -- WINA article, section 一: m_j = 1 iff score_j is among the K
  largest; ties are ordered by larger score, then lower index (a total order,
  so the kept set is unique).
* ``stat_threshold`` / ``stat_gate`` -- Spark Transformer article, section 2.2
  (statistical top-k): mu = mean, sigma^2 = mean of squared deviations
  (population variance), t = mu + sigma * Phi^-1(1 - s), keep score > t
  (strict). mu and sigma^2 are computed exactly as rationals and rounded to
  fp64 once; sigma is the IEEE sqrt; t = fl(mu + fl(sigma * z)) without fused
  multiply-add; z is Wichura's AS241 (the routine behind Python's
  ``statistics.NormalDist.inv_cdf``) at fl(1 - s).
* ``sparse_product`` -- Spark Transformer article, section 3.1 (SVMM, the
  index-list product): y = sum over active j of x_j * W[:, j], in fp64.

* ``gate(mode="fixed")`` -- WINA article, section 三 (per-layer thresholds
  calibrated from hidden-state distributions): keep score > tau with tau
  rounded to fp32 first; the reported threshold is that fp32 value.

Parity pins (tests/test_oracle_*.py): brute-force pairwise dominance for the
top-K set, hypothesis tie-heavy cases, closed forms for scores, norms and the
statistical threshold, AS241 against mpmath, integer brute-force products,
the orthogonal-column error identity and the WINA <= TEAL error inequality;
for the fixed threshold, a score equal to fp32(tau) dropped, tau rounded
before the comparison, tau = 0 keeping exactly the nonzero scores, a tau above
every score keeping nothing, and the count of a sorted copy above fp32(tau).
Planted mistakes in each function fail these pins
(tests/test_oracle_mutations.py).
No page prints a worked numeric example, so no function is pinned to printed
values; every function has at least one independent pin above.
"""
from __future__ import annotations

import math
import statistics
from fractions import Fraction
from typing import Dict, Optional, Sequence

import numpy as np

_NORMAL = statistics.NormalDist()


# --------------------------------------------------------------------------
# dtype handling: fp32 arrays, or bf16 stored as uint16 bit patterns
# --------------------------------------------------------------------------
def as_f64(a: np.ndarray) -> np.ndarray:
    """Exact fp64 value of an fp32 array or of bf16 bit patterns (uint16)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if a.dtype == np.float32:
        return a.astype(np.float64)
    if a.dtype == np.float64:
        return a
    raise TypeError(f"unsupported dtype {a.dtype}")


# --------------------------------------------------------------------------
# Norm vector and scores
# --------------------------------------------------------------------------
def column_norms(W: np.ndarray, block_rows: int = 2048) -> np.ndarray:
    """c_j = ||W[:, j]||_2 for W in the [m][n] layout, returned as fp32.

    Squares of bf16/fp32 values are exact in fp64; the column sums are fp64;
    the sqrt is rounded to fp64 and then to fp32 (for sqrt this double rounding
    equals a single rounding of the fp64-sum's square root)."""
    m, n = W.shape
    acc = np.zeros(n, dtype=np.float64)
    for r0 in range(0, m, block_rows):
        blk = as_f64(W[r0:r0 + block_rows])
        acc += np.einsum("ij,ij->j", blk, blk)
    return np.sqrt(acc).astype(np.float32)


def scores(x: np.ndarray, c: np.ndarray) -> np.ndarray:
    """score_j = |x_j * c_j| as fp32 (exact fp64 product, one RNE rounding)."""
    c = np.asarray(c, dtype=np.float32)
    prod = np.abs(as_f64(x)) * np.abs(c.astype(np.float64))
    return prod.astype(np.float32)


# --------------------------------------------------------------------------
# Gates
# --------------------------------------------------------------------------
def topk_gate(s: np.ndarray, K: int):
    """Exact top-K under (score descending, index ascending).

    Returns (mask bool[n], thresh) with thresh the K-th largest score as a
    float (``inf`` when K == 0)."""
    s = np.asarray(s, dtype=np.float32)
    n = s.shape[0]
    if not 0 <= K <= n:
        raise ValueError("K out of range")
    order = np.lexsort((np.arange(n), -s.astype(np.float64)))
    mask = np.zeros(n, dtype=bool)
    mask[order[:K]] = True
    thresh = float(s[order[K - 1]]) if K > 0 else math.inf
    return mask, thresh


def normal_quantile(p: float) -> float:
    """Phi^-1(p) by Wichura's AS241 (the stdlib routine), fp64."""
    return _NORMAL.inv_cdf(p)


def stat_moments(s: np.ndarray):
    """(mu, sigma^2) of the fp32 scores, each the exact rational rounded once
    to fp64. Every fp32 value is an integer multiple of 2^-149, so the sums
    are taken over integers."""
    s = np.asarray(s, dtype=np.float32)
    n = s.shape[0]
    if n == 0:
        raise ValueError("empty score vector")
    scale = 2 ** 149
    q = [int(Fraction(float(v)) * scale) for v in s]
    S1 = sum(q)
    S2 = sum(v * v for v in q)
    mu = Fraction(S1, n * scale)
    var = Fraction(n * S2 - S1 * S1, n * n * scale * scale)
    return float(mu), float(var)


def stat_threshold(s: np.ndarray, s_keep: float) -> float:
    """t = fl(mu + fl(sigma * z)), z = Phi^-1(fl(1 - s_keep))."""
    mu, var = stat_moments(s)
    sigma = math.sqrt(var)
    z = normal_quantile(1.0 - s_keep)
    return mu + sigma * z


def stat_gate(s: np.ndarray, s_keep: float):
    """Statistical top-k: keep score > t (strict). Returns (mask, t)."""
    t = stat_threshold(s, s_keep)
    s64 = np.asarray(s, dtype=np.float32).astype(np.float64)
    return s64 > t, t


def active_indices(mask: np.ndarray) -> np.ndarray:
    """Ascending list of kept input indices."""
    return np.flatnonzero(mask).astype(np.int64)


# --------------------------------------------------------------------------
# Product
# --------------------------------------------------------------------------
def sparse_product(W: np.ndarray, x: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """y = sum_{j in idx} x_j * W[:, j] (fp64), W in the [m][n] layout."""
    idx = np.asarray(idx, dtype=np.int64)
    m = W.shape[0]
    if idx.size == 0:
        return np.zeros(m, dtype=np.float64)
    return as_f64(W[:, idx]) @ as_f64(x)[idx]


def sparse_product_rows(W: np.ndarray, x: np.ndarray, idx: np.ndarray,
                        rows: Sequence[int]) -> np.ndarray:
    """The same sum for a subset of output rows only."""
    idx = np.asarray(idx, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    if idx.size == 0:
        return np.zeros(rows.size, dtype=np.float64)
    sub = as_f64(W[rows][:, idx])
    return sub @ as_f64(x)[idx]


# --------------------------------------------------------------------------
# One token, end to end
# --------------------------------------------------------------------------
def gate(x: np.ndarray, c: np.ndarray, mode: str, K: Optional[int] = None,
         s_keep: Optional[float] = None, tau: Optional[float] = None) -> Dict[str, object]:
    """Score + select for one token. ``mode`` is 'topk', 'stat' or 'fixed'
    (keep score > tau, a calibrated per-layer threshold)."""
    s = scores(x, c)
    if mode == "topk":
        mask, thresh = topk_gate(s, K)
    elif mode == "stat":
        mask, thresh = stat_gate(s, s_keep)
    elif mode == "fixed":
        mask = s.astype(np.float64) > float(np.float32(tau))
        thresh = float(np.float32(tau))
    else:
        raise ValueError(mode)
    idx = active_indices(mask)
    return {"scores": s, "mask": mask, "idx": idx, "count": int(idx.size), "thresh": thresh}


def forward(W: np.ndarray, c: np.ndarray, x: np.ndarray, mode: str, K: Optional[int] = None,
            s_keep: Optional[float] = None, tau: Optional[float] = None,
            rows: Optional[Sequence[int]] = None) -> Dict[str, object]:
    """Gate + product for one token; ``rows`` limits the product to sampled
    output rows (for full-size layers)."""
    out = gate(x, c, mode, K=K, s_keep=s_keep, tau=tau)
    if rows is None:
        out["y"] = sparse_product(W, x, out["idx"])
    else:
        out["y"] = sparse_product_rows(W, x, out["idx"], rows)
    return out
