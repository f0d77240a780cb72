"""Planted mistakes in the oracle must fail its pins.

Each case swaps one oracle function for a copy with a plausible mistake (on
the CPU, through pytest's monkeypatch; the oracle's files are untouched) and
runs a pin from tests/test_oracle_*.py against it: the pin has to raise.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import double_sparse as ods
from oracle import ffn
from oracle import sparse_linear as osl

import test_oracle_double_sparse as pins_ds
import test_oracle_ffn as pins_ffn
import test_oracle_gate as pins_gate


def _fixed_gate(cmp, round_tau=True, report_rounded=True):
    """oracle.gate for mode 'fixed' with a chosen comparison and tau rounding."""
    real = osl.gate

    def gate(x, c, mode, K=None, s_keep=None, tau=None):
        if mode != "fixed":
            return real(x, c, mode, K=K, s_keep=s_keep, tau=tau)
        s = osl.scores(x, c)
        t = float(np.float32(tau)) if round_tau else float(tau)
        mask = cmp(s.astype(np.float64), t)
        idx = osl.active_indices(mask)
        th = float(np.float32(tau)) if report_rounded else float(tau)
        return {"scores": s, "mask": mask, "idx": idx, "count": int(idx.size), "thresh": th}
    return gate


@pytest.mark.parametrize("mutant, pin", [
    (_fixed_gate(lambda s, t: s >= t), pins_gate.test_fixed_gate_strict_comparison),
    (_fixed_gate(lambda s, t: s > t, round_tau=False), pins_gate.test_fixed_gate_rounds_tau_to_fp32_first),
    (_fixed_gate(lambda s, t: s > t, report_rounded=False), pins_gate.test_fixed_gate_rounds_tau_to_fp32_first),
    (_fixed_gate(lambda s, t: s >= t), pins_gate.test_fixed_gate_zero_and_huge_tau),
    (_fixed_gate(lambda s, t: s >= t), pins_gate.test_fixed_gate_matches_sorted_count),
])
def test_fixed_gate_mutants_fail(monkeypatch, mutant, pin):
    monkeypatch.setattr(oracle, "gate", mutant)
    with pytest.raises(AssertionError):
        pin()


def _bf16_truncate(v):
    v = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def _bf16_half_away(v):
    v = np.asarray(v, dtype=np.float64)
    out = []
    for a in v.reshape(-1).tolist():
        if a == 0 or not math.isfinite(a):
            out.append(a)
            continue
        e = math.frexp(abs(a))[1]
        q = 2.0 ** max(e - 8, -133)
        r = math.floor(abs(a) / q + 0.5) * q
        out.append(math.copysign(r, a))
    bits = np.array(out, dtype=np.float64).reshape(v.shape).astype(np.float32).view(np.uint32)
    return (bits >> 16).astype(np.uint16)


def _silu_mul_via_fp32(g, u):
    # double rounding: fp64 -> fp32 -> bf16
    v = (ffn.silu(np.asarray(g, np.float64)) * np.asarray(u, np.float64)).astype(np.float32)
    bits = v.view(np.uint32).astype(np.uint64)
    return ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)


def _chain_silu_on_up(Wg, cg, gate_kw, Wu, cu, up_kw, Wd, cd, down_kw, x, rows=None):
    def kw(d):
        d = dict(d)
        return d.pop("mode"), d
    (mg, kg), (mu, ku), (md, kd) = kw(gate_kw), kw(up_kw), kw(down_kw)
    g = osl.forward(Wg, cg, x, mg, **kg)["y"]
    u = osl.forward(Wu, cu, x, mu, **ku)["y"]
    h = ffn.bf16_round(ffn.silu(u) * g)
    d = osl.forward(Wd, cd, h, md, rows=rows, **kd)
    return {"g": g, "u": u, "h": h, "y": d["y"], "down": d}


@pytest.mark.parametrize("attr, mutant, pin", [
    ("bf16_round", _bf16_truncate, pins_ffn.test_bf16_round_ties_to_even),
    ("bf16_round", _bf16_half_away, pins_ffn.test_bf16_round_ties_to_even),
    ("bf16_round", _bf16_half_away, pins_ffn.test_bf16_round_subnormals_and_overflow),
    ("silu_mul", _silu_mul_via_fp32, pins_ffn.test_silu_mul_rounds_once),
    ("silu", lambda v: 1.0 / (1.0 + np.exp(-np.asarray(v, np.float64))), pins_ffn.test_silu_zero_and_limits),
    # v sigma(-v) (like any v F(v) with F(v) + F(-v) = 1) satisfies the odd-part
    # identity too; scipy's logistic function and the limits catch it
    ("silu", lambda v: np.asarray(v, np.float64) / (1.0 + np.exp(np.asarray(v, np.float64))),
     pins_ffn.test_silu_matches_scipy_expit),
    ("silu", lambda v: np.asarray(v, np.float64) / (1.0 + np.exp(np.asarray(v, np.float64))),
     pins_ffn.test_silu_zero_and_limits),
    ("ffn_chain", _chain_silu_on_up, pins_ffn.test_ffn_chain_gate_and_up_are_not_interchangeable),
    ("ffn_chain", _chain_silu_on_up, pins_ffn.test_ffn_chain_diagonal_weights),
])
def test_ffn_mutants_fail(monkeypatch, attr, mutant, pin):
    monkeypatch.setattr(ffn, attr, mutant)
    with pytest.raises(AssertionError):
        with np.errstate(over="ignore"):
            pin()


def _scores_wrong_channel_order(q, label, channels, n):
    # sums the label columns against the query gathered in reversed order
    qf = ods._as_f32(q)
    lf = ods._as_f32(label)[:n]
    acc = np.zeros(n, np.float32)
    ch = np.asarray(channels).tolist()[::-1]
    for j, c in enumerate(ch):
        acc = acc + np.float32(qf[c]) * lf[:, j]
    return acc


def _scores_fp16_accumulate(q, label, channels, n):
    qf = ods._as_f32(q)
    lf = ods._as_f32(label)[:n]
    acc = np.zeros(n, np.float16)
    for j, c in enumerate(np.asarray(channels).tolist()):
        acc = (acc + np.float32(qf[c]) * lf[:, j]).astype(np.float16)
    return acc.astype(np.float32)


@pytest.mark.parametrize("mutant", [_scores_wrong_channel_order, _scores_fp16_accumulate])
@pytest.mark.parametrize("r", [8, 16, 32])
def test_ds_score_mutants_fail(monkeypatch, mutant, r):
    monkeypatch.setattr(ods, "approx_scores", mutant)
    with pytest.raises(AssertionError):
        pins_ds.test_label_scores_exact_on_integer_inputs(r)
