"""Pins for the oracle's norm vector, scores and top-K gate.

None of these checks re-types the oracle's formula: each compares it with an
IEEE closed form, a different library routine (numpy fp32 arithmetic), a
brute-force enumeration or a property of the unique top-K set under the order
(score descending, index ascending) that the WINA gate (WINA article,
section 一) and the tie rule define.
"""
import itertools
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from workloads import f32_to_bf16_bits


def _dominates(s, i, j):
    """i precedes j in the total order (score desc, index asc)."""
    return (s[i] > s[j]) or (s[i] == s[j] and i < j)


def _check_topk_set(s, K, mask):
    n = len(s)
    kept = [i for i in range(n) if mask[i]]
    dropped = [i for i in range(n) if not mask[i]]
    assert len(kept) == K
    for i in kept:
        for j in dropped:
            assert _dominates(s, i, j), (i, j, s[i], s[j])


# ---------------------------------------------------------------- scores
def test_scores_match_ieee_fp32_multiply():
    g = np.random.default_rng(1)
    # magnitudes spanning normals, subnormal products and large values
    x = (g.standard_normal(200000) * np.exp2(g.integers(-80, 60, 200000))).astype(np.float32)
    c = (np.abs(g.standard_normal(200000)) * np.exp2(g.integers(-80, 30, 200000))).astype(np.float32)
    want = np.abs(x) * c  # numpy float32 multiply: IEEE binary32, RNE, gradual underflow
    got = oracle.scores(x, c)
    assert got.dtype == np.float32
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


def test_scores_closed_forms():
    # 3 * fl32(1/3) = 1 + 2^-25 exactly -> below half an ulp of 1.0 -> 1.0
    third = np.float32(1.0 / 3.0)
    assert oracle.scores(np.array([3.0], np.float32), np.array([third]))[0] == 1.0
    # sign is dropped, -0 becomes +0
    s = oracle.scores(np.array([-2.0, -0.0, 0.5], np.float32), np.array([1.5, 7.0, -4.0], np.float32))
    assert s.tolist() == [3.0, 0.0, 2.0]
    assert s.view(np.uint32)[1] == 0
    # the smallest subnormal times 0.5 rounds to even (zero); times 1.5 rounds up to 2 * min
    tiny = np.float32(np.finfo(np.float32).smallest_subnormal)
    s = oracle.scores(np.array([tiny, tiny], np.float32), np.array([0.5, 1.5], np.float32))
    assert s[0] == 0.0 and s[1] == 2 * tiny


def test_scores_bf16_input_is_exact_widening():
    x32 = np.array([1.0, -3.140625, 2.0 ** -126, 65280.0], np.float32)  # all bf16-exact
    bits = f32_to_bf16_bits(x32)
    c = np.ones(4, np.float32)
    np.testing.assert_array_equal(oracle.scores(bits, c), np.abs(x32))


def test_teal_special_case_unit_norms():
    # with c = 1 the WINA score is |x|, i.e. the gate reduces to TEAL's
    # magnitude criterion (WINA article, section 二)
    g = np.random.default_rng(2)
    x = g.standard_normal(1000).astype(np.float32)
    np.testing.assert_array_equal(oracle.scores(x, np.ones(1000, np.float32)), np.abs(x))


# ---------------------------------------------------------------- norms
def test_column_norms_pythagorean_exact():
    W = np.array([[3.0, 1.0, 0.0], [4.0, 2.0, 0.0], [0.0, 2.0, 0.0]], np.float32)
    assert oracle.column_norms(W).tolist() == [5.0, 3.0, 0.0]


def test_column_norms_orthogonal_scaled_columns():
    g = np.random.default_rng(3)
    m, n = 96, 40
    Q, _ = np.linalg.qr(g.standard_normal((m, n)))
    d = np.exp(g.uniform(np.log(0.1), np.log(10.0), n))
    W = (Q * d).astype(np.float32)
    c = oracle.column_norms(W)
    # fp32 storage of W perturbs each column norm by ~1e-7 relative
    np.testing.assert_allclose(c, d, rtol=2e-6)


def test_column_norms_vs_linalg_norm():
    g = np.random.default_rng(4)
    W = f32_to_bf16_bits(g.standard_normal((300, 77), dtype=np.float32) * 0.02)
    Wf = oracle.as_f64(W)
    ref = np.linalg.norm(Wf, axis=0)  # LAPACK-style scaled norm, different algorithm
    got = oracle.column_norms(W).astype(np.float64)
    ulp = np.spacing(np.float32(ref).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got - ref) <= ulp)


# ---------------------------------------------------------------- top-K
def test_topk_exhaustive_tiny():
    """For n <= 7, enumerate every K-subset: exactly one satisfies dominance
    and it is the oracle's."""
    g = np.random.default_rng(5)
    for trial in range(60):
        n = int(g.integers(1, 8))
        s = g.integers(0, 3, n).astype(np.float32)  # heavy ties
        for K in range(n + 1):
            mask, _ = oracle.topk_gate(s, K)
            winners = []
            for sub in itertools.combinations(range(n), K):
                ss = set(sub)
                if all(_dominates(s, i, j) for i in ss for j in range(n) if j not in ss):
                    winners.append(ss)
            assert len(winners) == 1
            assert set(np.flatnonzero(mask).tolist()) == winners[0]


@settings(max_examples=300, deadline=None)
@given(st.lists(st.integers(0, 6), min_size=0, max_size=64), st.data())
def test_topk_dominance_property(vals, data):
    s = np.array(vals, dtype=np.float32) * np.float32(0.25)
    n = len(vals)
    K = data.draw(st.integers(0, n))
    mask, thresh = oracle.topk_gate(s, K)
    _check_topk_set(s, K, mask)
    if K > 0:
        assert thresh == float(min(s[mask]))
        # the threshold key: fewer than K scores lie strictly above it
        assert int(np.sum(s > thresh)) < K <= int(np.sum(s >= thresh))
    else:
        assert thresh == math.inf


def test_topk_special_cases():
    s = np.zeros(10, np.float32)
    mask, thresh = oracle.topk_gate(s, 4)
    assert np.flatnonzero(mask).tolist() == [0, 1, 2, 3] and thresh == 0.0
    s = np.arange(10, dtype=np.float32)
    assert not oracle.topk_gate(s, 0)[0].any()
    assert oracle.topk_gate(s, 10)[0].all()
    assert np.flatnonzero(oracle.topk_gate(s, 3)[0]).tolist() == [7, 8, 9]
    with pytest.raises(ValueError):
        oracle.topk_gate(s, 11)


def test_active_indices_ascending():
    mask = np.array([0, 1, 1, 0, 1, 0, 0, 1], bool)
    assert oracle.active_indices(mask).tolist() == [1, 2, 4, 7]


def test_gate_end_to_end_small():
    # hand-worked: x = [1, -4, 2, 0.5], c = [2, 1, 0.5, 8] -> scores [2, 4, 1, 4]
    # top-2 under (score desc, index asc) keeps indices 1 and 3; K-th score 4
    out = oracle.gate(np.array([1, -4, 2, 0.5], np.float32), np.array([2, 1, 0.5, 8], np.float32),
                      "topk", K=2)
    assert out["scores"].tolist() == [2.0, 4.0, 1.0, 4.0]
    assert out["idx"].tolist() == [1, 3] and out["count"] == 2 and out["thresh"] == 4.0
    out = oracle.gate(np.array([1, -4, 2, 0.5], np.float32), np.array([2, 1, 0.5, 8], np.float32),
                      "topk", K=3)
    assert out["idx"].tolist() == [0, 1, 3] and out["thresh"] == 2.0


# ---------------------------------------------------------------- fixed threshold
# A calibrated per-layer threshold (WINA article, section 三): keep score > tau,
# tau taken as an fp32 value. Each case below has an answer that follows from
# the definition alone, and a plausible mistake (>= for >, comparing against
# the unrounded tau, reporting a different threshold) fails at least one.
def _fixed(x, c, tau):
    return oracle.gate(np.asarray(x, np.float32), np.asarray(c, np.float32), "fixed", tau=tau)


def test_fixed_gate_strict_comparison():
    # scores [2, 4, 1, 4]: a score exactly equal to tau is dropped
    out = _fixed([1, -4, 2, 0.5], [2, 1, 0.5, 8], 2.0)
    assert out["idx"].tolist() == [1, 3] and out["count"] == 2 and out["thresh"] == 2.0
    out = _fixed([1, -4, 2, 0.5], [2, 1, 0.5, 8], 4.0)
    assert out["count"] == 0 and out["thresh"] == 4.0


def test_fixed_gate_rounds_tau_to_fp32_first():
    one = np.float32(1.0)
    below = float(np.nextafter(one, np.float32(0)))  # largest fp32 below 1
    # tau just below 1.0 (as fp64) rounds to fp32 1.0, so a score of exactly
    # 1.0 is dropped; compared unrounded, it would be kept
    tau = 1.0 - 2.0 ** -30
    assert float(np.float32(tau)) == 1.0
    out = _fixed([1.0, below, 1.5], [1, 1, 1], tau)
    assert out["idx"].tolist() == [2] and out["thresh"] == 1.0
    # tau just above the fp32 value below 1 rounds down onto it: 1.0 is kept,
    # the score equal to that fp32 value is not
    tau = below + 2.0 ** -40
    assert float(np.float32(tau)) == below
    out = _fixed([1.0, below, 0.5], [1, 1, 1], tau)
    assert out["idx"].tolist() == [0] and out["thresh"] == below


def test_fixed_gate_zero_and_huge_tau():
    g = np.random.default_rng(6)
    x = g.standard_normal(500).astype(np.float32)
    x[g.choice(500, 60, replace=False)] = 0.0
    c = np.abs(g.standard_normal(500)).astype(np.float32)
    c[:7] = 0.0
    # tau = 0 keeps exactly the inputs with a nonzero score (x_j != 0 and c_j != 0)
    out = _fixed(x, c, 0.0)
    want = np.flatnonzero((x != 0) & (c != 0))
    assert out["idx"].tolist() == want.tolist() and out["thresh"] == 0.0
    # a tau above every score keeps nothing; the largest fp32 keeps nothing too
    top = float(np.max(np.abs(x.astype(np.float64)) * c))
    assert _fixed(x, c, 2 * top)["count"] == 0
    assert _fixed(x, c, float(np.finfo(np.float32).max))["count"] == 0


def test_fixed_gate_matches_sorted_count():
    # the kept count equals the number of scores strictly above fp32(tau),
    # counted from a sorted copy (searchsorted, a different routine)
    g = np.random.default_rng(7)
    for trial in range(20):
        n = int(g.integers(1, 3000))
        x = g.standard_normal(n).astype(np.float32)
        c = np.abs(g.standard_normal(n)).astype(np.float32)
        s = np.sort(np.abs(x) * c)  # numpy fp32 multiply: the IEEE scores
        tau = float(s[int(g.integers(0, n))]) * float(g.choice([1.0, 1.0 + 2.0 ** -30, 0.999]))
        out = _fixed(x, c, tau)
        above = n - int(np.searchsorted(s, np.float32(tau), side="right"))
        assert out["count"] == above
