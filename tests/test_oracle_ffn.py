"""Pins for the FFN-chain oracle (oracle/ffn.py): SiLU, one-step bf16
rounding, the epilogue h = bf16(SiLU(g) u) and the chain's wiring.

Each check compares the oracle with something other than its own formula: a
limit or identity of the function, a different library routine (scipy's
logistic function), hand-built rounding midpoints whose correct result is
known, the nearest-value property of rounding, or a diagonal-weight chain in
which every stage reduces to scalar arithmetic on one input.
"""
import numpy as np
import pytest

import oracle
from oracle import ffn
from workloads import f32_to_bf16_bits


def _bf16_value(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- SiLU
def test_silu_zero_and_limits():
    assert ffn.silu(np.array([0.0]))[0] == 0.0
    # e^-v is below half an ulp of 1 for v >= 37.5: 1 + e^-v == 1, SiLU(v) == v
    big = np.array([40.0, 100.0, 1e6])
    np.testing.assert_array_equal(ffn.silu(big), big)
    # very negative: e^-v overflows, SiLU(v) is -0 (no NaN, no warning)
    neg = ffn.silu(np.array([-800.0, -1e6]))
    assert np.all(neg == 0.0) and not np.any(np.isnan(neg))
    # SiLU(v) -> v * e^v for v -> -inf (relative difference ~e^v)
    v = -30.0
    assert abs(ffn.silu(np.array([v]))[0] - v * np.exp(v)) <= 1e-12 * abs(v * np.exp(v))


def test_silu_odd_part_identity():
    # v s(v) - (-v) s(-v) = v (s(v) + s(-v)) = v, s the logistic function
    v = np.random.default_rng(0).standard_normal(5000) * 6
    d = ffn.silu(v) - ffn.silu(-v)
    np.testing.assert_allclose(d, v, rtol=4e-16 * 8, atol=1e-15)


def test_silu_matches_scipy_expit():
    special = pytest.importorskip("scipy.special")
    v = np.random.default_rng(1).standard_normal(20000) * 8
    # two roundings on each side (divide vs multiply): within 4 ulp
    np.testing.assert_allclose(ffn.silu(v), v * special.expit(v), rtol=4 * 2.0 ** -52, atol=0)


# ---------------------------------------------------------------- bf16 rounding
def test_bf16_round_ties_to_even():
    u = 2.0 ** -7   # bf16 ulp at 1.0
    cases = [
        (1.0 + u / 2, 1.0),              # halfway, even below
        (1.0 + 3 * u / 2, 1.0 + 2 * u),  # halfway, even above
        (1.0 + u / 2 + 2.0 ** -40, 1.0 + u),  # just past halfway rounds up
        (1.0 + u / 2 - 2.0 ** -40, 1.0),      # just before rounds down
        (-(1.0 + u / 2), -1.0),
        (-(1.0 + 3 * u / 2), -(1.0 + 2 * u)),
        (3.0 * 2.0 ** 100 + 2.0 ** 93, 3.0 * 2.0 ** 100),  # halfway at a large exponent
    ]
    for v, want in cases:
        got = _bf16_value(ffn.bf16_round(np.array([v])))[0]
        assert got == want, (v, got, want)


def test_bf16_round_subnormals_and_overflow():
    q = 2.0 ** -133  # smallest bf16 subnormal
    got = _bf16_value(ffn.bf16_round(np.array([q / 2, 3 * q / 2, 5 * q / 2, q * 0.51, 2.0 ** -126 * 1.5])))
    np.testing.assert_array_equal(got, [0.0, 2 * q, 2 * q, q, 2.0 ** -126 * 1.5])
    big = (2 - 2.0 ** -7) * 2.0 ** 127  # largest finite bf16
    mid = 2.0 ** 128 - 2.0 ** 119       # halfway between it and 2^128
    got = _bf16_value(ffn.bf16_round(np.array([big, mid - 2.0 ** 90, mid, -mid])))
    assert got[0] == big and got[1] == big and got[2] == np.inf and got[3] == -np.inf
    bits = ffn.bf16_round(np.array([0.0, -0.0, np.nan, np.inf]))
    assert bits[0] == 0 and bits[1] == 0x8000 and np.isnan(_bf16_value(bits[2:3])[0]) and bits[3] == 0x7F80


def test_bf16_round_is_nearest_on_random_values():
    g = np.random.default_rng(2)
    v = g.standard_normal(4000) * np.exp2(g.integers(-60, 60, 4000))
    r = _bf16_value(ffn.bf16_round(v))
    # neighbours of r on the bf16 grid: no bf16 value lies closer to v
    bits = ffn.bf16_round(v).astype(np.int64)
    up = _bf16_value((bits + 1).astype(np.uint16))
    dn = _bf16_value((bits - 1).astype(np.uint16))
    assert np.all(np.abs(r - v) <= np.abs(up - v))
    assert np.all(np.abs(r - v) <= np.abs(dn - v))
    # on the fp32 grid the same rounding is the library's RNE conversion of an
    # exactly representable fp32 value
    v32 = (g.standard_normal(4000) * 3).astype(np.float32)
    np.testing.assert_array_equal(ffn.bf16_round(v32.astype(np.float64)), f32_to_bf16_bits(v32))


def test_silu_mul_rounds_once():
    # SiLU(64) = 64 exactly; 64 * u hits the bf16 midpoint 1 + 2^-8 exactly:
    # one rounding gives 1 (even); rounding SiLU(g) * u first to fp32 would
    # too, so also check a case where fp32 double rounding would differ
    g = np.array([64.0, 64.0, 0.0, -900.0])
    u = np.array([(1.0 + 2.0 ** -8) / 64, (1.0 + 2.0 ** -8 + 2.0 ** -30) / 64, 5.0, 2.0])
    h = _bf16_value(ffn.silu_mul(g, u))
    # 1 + 2^-8 + 2^-30 rounds up to 1 + 2^-7 in one step; via fp32 it would
    # first become 1 + 2^-8 (the midpoint) and then round to even, 1.0
    np.testing.assert_array_equal(h, [1.0, 1.0 + 2.0 ** -7, 0.0, 0.0])


# ---------------------------------------------------------------- chain wiring
def test_ffn_chain_diagonal_weights():
    # diagonal gate, up and down weights: g_j = a_j x_j, u_j = b_j x_j,
    # h_j = bf16(SiLU(g_j) u_j), y_j = d_j h_j; dense gates keep everything,
    # so every stage is scalar arithmetic on input j
    n = 16
    g = np.random.default_rng(3)
    x32 = g.standard_normal(n).astype(np.float32)
    a, b, d = (np.float32(2.0) ** g.integers(-2, 3, n).astype(np.float32) for _ in range(3))
    Wg, Wu, Wd = (np.diag(v).astype(np.float32) for v in (a, b, d))
    x = x32
    cg, cu = oracle.column_norms(Wg), oracle.column_norms(Wu)
    dense = dict(mode="topk", K=n)
    h_ref = ffn.silu_mul(a.astype(np.float64) * x, b.astype(np.float64) * x)
    cd = oracle.column_norms(Wd)
    out = ffn.ffn_chain(Wg, cg, dense, Wu, cu, dense, Wd, cd, dense, x.astype(np.float32))
    np.testing.assert_array_equal(out["g"], a.astype(np.float64) * x)
    np.testing.assert_array_equal(out["u"], b.astype(np.float64) * x)
    np.testing.assert_array_equal(out["h"], h_ref)
    np.testing.assert_array_equal(out["y"], d.astype(np.float64) * _bf16_value(h_ref))
    # the down gate sees h: keep the 5 largest |h_j| |d_j|
    out5 = ffn.ffn_chain(Wg, cg, dense, Wu, cu, dense, Wd, cd, dict(mode="topk", K=5), x)
    sc = np.abs(_bf16_value(h_ref)) * np.abs(d.astype(np.float64))
    keep = np.lexsort((np.arange(n), -sc))[:5]
    want = np.zeros(n)
    want[keep] = d[keep].astype(np.float64) * _bf16_value(h_ref)[keep]
    np.testing.assert_array_equal(out5["y"], want)


def test_ffn_chain_gate_and_up_are_not_interchangeable():
    # SiLU applies to the gate projection's output only: swapping the two
    # handles changes h (a wiring mistake this pin catches)
    n = 8
    x = np.linspace(-2, 2, n).astype(np.float32)
    Wg = np.eye(n, dtype=np.float32)
    Wu = 3 * np.eye(n, dtype=np.float32)
    Wd = np.eye(n, dtype=np.float32)
    c = oracle.column_norms
    dense = dict(mode="topk", K=n)
    a = ffn.ffn_chain(Wg, c(Wg), dense, Wu, c(Wu), dense, Wd, c(Wd), dense, x)
    b = ffn.ffn_chain(Wu, c(Wu), dense, Wg, c(Wg), dense, Wd, c(Wd), dense, x)
    np.testing.assert_array_equal(a["h"], ffn.silu_mul(x.astype(np.float64), 3.0 * x))
    assert not np.array_equal(a["h"], b["h"])
