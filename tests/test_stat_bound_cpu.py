"""The statistical gate's first threshold, checked on the CPU.

The gate sums the scores and their squares in plain fp64 (any order), takes
t0 = mu + sigma z from those sums and decides the kept set with t0 whenever no
score lies within del = 2^-32 (mu + |z| sigma + |z| E[s^2] / sigma) of it; the
exact threshold t (the oracle's: moments as exact rationals rounded once to
fp64, Spark Transformer article, section 2.2) must then lie within del of t0.
These tests repeat that fp64 arithmetic on the host, in the same operation
order (per-thread sequential sums, then a tree of pairwise sums, 1/n rounded
and multiplied, no fused multiply-add), over score vectors of several shapes
and summation orders, and check that t0 is far closer to t than del (a
margin of 2^8 and more), and that the cases the gate leaves to the exact
moments (near-constant scores, t not safely positive) are flagged."""
import math

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _tree(vals):
    vals = list(vals)
    while len(vals) > 1:
        vals = [vals[i] + vals[i + 1] if i + 1 < len(vals) else vals[i] for i in range(0, len(vals), 2)]
    return vals[0]


def first_threshold(s32, z, order, per_thread=8):
    """(ok, t0, del) as the gate computes them from the plain sums."""
    s = [float(v) for v in np.asarray(s32, np.float32)[order]]
    n = len(s)
    f1, f2 = [], []
    for i in range(0, n, per_thread):
        a, b = 0.0, 0.0
        for v in s[i:i + per_thread]:
            a += v
            b += v * v
        f1.append(a)
        f2.append(b)
    F1, F2 = _tree(f1), _tree(f2)
    inv_n = 1.0 / n
    mu, e2 = F1 * inv_n, F2 * inv_n
    v = e2 - mu * mu
    ok = min(s) != max(s) and v > 2.0 ** -20 * e2
    sg = math.sqrt(v) if ok else 1.0
    t0 = mu + sg * z
    az = abs(z)
    dl = 2.0 ** -32 * (mu + az * sg + az * (e2 / sg))
    ok = ok and (t0 - dl) > 0.0
    return ok, t0, dl


def _vectors():
    rng = np.random.default_rng(7)
    out = []
    for n in (7, 100, 5120, 17920):
        x = rng.laplace(0.0, 1.0, n)
        out.append(("laplace", np.abs(x).astype(np.float32)))
        out.append(("half-normal", np.abs(rng.standard_normal(n)).astype(np.float32)))
        g, u = rng.standard_normal(n), rng.standard_normal(n)
        out.append(("silu-u", np.abs(g / (1 + np.exp(-g)) * u).astype(np.float32)))
        out.append(("lognormal", rng.lognormal(0.0, 2.0, n).astype(np.float32)))
        out.append(("scaled-tiny", (np.abs(rng.standard_normal(n)) * 1e-30).astype(np.float32)))
        two = np.ones(n, np.float32)
        two[: n // 3] = 2.0
        out.append(("two-valued", two))
    return out


@pytest.mark.parametrize("s_keep", [0.02, 0.1, 0.3, 0.5])
def test_first_threshold_within_bound(s_keep):
    z = oracle.normal_quantile(1.0 - s_keep)
    rng = np.random.default_rng(11)
    checked = 0
    for name, s in _vectors():
        t = oracle.stat_threshold(s, s_keep)
        for trial in range(3):
            order = rng.permutation(s.shape[0]) if trial else np.arange(s.shape[0])
            ok, t0, dl = first_threshold(s, z, order)
            if not ok:
                continue
            checked += 1
            assert abs(t0 - t) <= dl * 2.0 ** -8, (name, s.shape[0], trial, t0, t, dl)
    assert checked >= 40


def test_fallback_cases_are_flagged():
    z = oracle.normal_quantile(1.0 - 0.1)
    const = np.full(1000, 0.75, np.float32)
    assert not first_threshold(const, z, np.arange(1000))[0]
    near = np.full(1000, 1.0, np.float32)
    near[0] = np.nextafter(np.float32(1.0), np.float32(2.0))  # sigma / rms ~ 2^-28
    assert not first_threshold(near, z, np.arange(1000))[0]
    # keep fraction above one half: t below the mean, here below zero
    lap = np.abs(np.random.default_rng(3).laplace(0.0, 1.0, 2000)).astype(np.float32)
    z9 = oracle.normal_quantile(1.0 - 0.9)
    ok, t0, _ = first_threshold(lap, z9, np.arange(2000))
    assert t0 < 0.0 and not ok


def test_bound_catches_a_planted_mistake():
    """A first threshold that forgets the squares' weight in the variance
    (sigma^2 = E[s^2] - mu instead of E[s^2] - mu^2) lands far outside del."""
    s = np.abs(np.random.default_rng(5).laplace(0.0, 1.0, 5120)).astype(np.float32)
    z = oracle.normal_quantile(0.9)
    t = oracle.stat_threshold(s, 0.1)
    ok, t0, dl = first_threshold(s, z, np.arange(5120))
    assert ok and abs(t0 - t) <= dl
    mu = float(np.mean(s.astype(np.float64)))
    e2 = float(np.mean(s.astype(np.float64) ** 2))
    wrong = mu + math.sqrt(e2 - mu) * z
    assert abs(wrong - t) > dl
