"""The C-ABI library without a GPU: it loads, exports every declared symbol,
validates arguments before touching a device, reports a missing device
cleanly, and evaluates AS241 on the host bit for bit like the stdlib."""
import ctypes
import math
import os
import re
import statistics

import numpy as np
import pytest

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")
HEADERS = [os.path.join(INCLUDE, "sparse_linear.h"), os.path.join(INCLUDE, "double_sparse.h")]


def _declared():
    names = set()
    for hp in HEADERS:
        names |= set(re.findall(r"\b((?:sparse_linear|ds)_\w+)\s*\(", open(hp).read()))
    return sorted(names)


def test_exports_every_declared_symbol(slib):
    L = slib.lib()
    names = _declared()
    assert len(names) >= 10
    for name in names:
        assert hasattr(L, name), name
    assert sorted(slib.EXPORTED) == names


@pytest.mark.parametrize("p", [1e-300, 1e-30, 1e-12, 1e-4, 0.001, 0.01, 0.02425, 0.05, 0.075, 0.0749,
                               0.0751, 0.1, 0.2, 0.3, 0.45, 0.5, 0.55, 0.7, 0.8, 0.9, 0.9249, 0.925,
                               0.9251, 0.95, 0.975, 0.99, 0.9999, 1 - 1e-12])
def test_host_quantile_bitwise_stdlib(slib, p):
    got = slib.sparse_linear_normal_quantile(p)
    want = statistics.NormalDist().inv_cdf(p)
    assert got.hex() == want.hex()


def test_host_quantile_dense_sweep(slib):
    g = np.random.default_rng(41)
    ps = np.concatenate([g.random(4000), np.exp(-g.uniform(0, 700, 1000)), 1 - np.exp(-g.uniform(2, 36, 500))])
    nd = statistics.NormalDist()
    bad = [p for p in ps.tolist() if 0 < p < 1 and slib.sparse_linear_normal_quantile(p) != nd.inv_cdf(p)]
    assert bad == []
    # the STAT gate's z for the keep fractions used by the workloads
    for s in (0.05, 0.1, 0.15, 0.3, 0.5):
        assert slib.sparse_linear_normal_quantile(1.0 - s) == nd.inv_cdf(1.0 - s)


def test_host_quantile_outside_domain(slib):
    for p in (0.0, 1.0, -0.5, 2.0, float("nan")):
        assert math.isnan(slib.sparse_linear_normal_quantile(p))


def _init(slib, W=1, dt=1, lay=0, m=64, n=32, c=0, gate=0, K=8, s=0.0, mb=1):
    h = ctypes.c_void_p()
    st = slib.lib().sparse_linear_init(ctypes.byref(h), W or None, dt, lay, m, n, c or None, gate, K, s, mb, None)
    return st, h


@pytest.mark.parametrize("kw,status", [
    (dict(W=0), 1),
    (dict(dt=7), 1),
    (dict(lay=5), 1),
    (dict(m=0), 1),
    (dict(n=0), 1),
    (dict(n=32769), 2),
    (dict(m=12), 2),            # bf16 needs m % 8 == 0
    (dict(dt=0, m=6), 2),       # fp32 needs m % 4 == 0
    (dict(K=-1), 1),
    (dict(K=33), 1),
    (dict(gate=1, s=0.0), 1),
    (dict(gate=1, s=1.0), 1),
    (dict(gate=1, s=float("nan")), 1),
    (dict(gate=2, s=-1.0), 1),
    (dict(gate=9), 1),
    (dict(mb=0), 1),
    (dict(mb=17), 1),
])
def test_init_rejects_bad_arguments(slib, kw, status):
    st, h = _init(slib, **kw)
    assert st == status, slib.sparse_linear_last_error()
    assert h.value is None
    assert slib.sparse_linear_last_error() != ""


def test_init_without_device_reports_hip_error(slib):
    torch = pytest.importorskip("torch")
    if torch.cuda.device_count() > 0:
        pytest.skip("a device is present")
    st, h = _init(slib)
    assert st == 4
    assert h.value is None


def test_forward_rejects_null_handle_and_pointers(slib):
    L = slib.lib()
    assert L.sparse_linear_forward(None, 1, 1, 1, 0, None, None, None, None) == 1
    assert L.sparse_linear_forward_dense(None, 1, 1, 1, 0, None) == 1
    assert L.sparse_linear_get_norms(None, 1, None) == 1
    assert L.sparse_linear_destroy(None) == 0
    assert L.sparse_linear_set_plan(None, 0, 0) == 1
    assert L.sparse_linear_set_union_plan(None, 0, 0) == 1
    assert L.sparse_linear_set_deterministic(None, 1) == 1
    assert L.sparse_linear_set_fused(None, 1) == 1
    assert L.sparse_linear_sync_status(None, None) == 1
    assert L.sparse_linear_gather_ceiling(None, 1, 1, 1, None) == 1


def test_forward_ffn_rejects_bad_arguments(slib):
    L = slib.lib()
    assert L.sparse_linear_ffn_workspace_bytes(None) == 0
    assert L.sparse_linear_forward_ffn(None, None, None, 1, 1, 0, 1, 1 << 20, None) == 1
    assert "NULL" in slib.sparse_linear_last_error()


def test_forward_group_rejects_bad_arguments(slib):
    L = slib.lib()
    hs = (ctypes.c_void_p * 2)(None, None)
    ys = (ctypes.c_void_p * 2)(1, 1)
    assert L.sparse_linear_forward_group(None, 1, 1, ys, 0, None) == 1      # NULL handle array
    assert L.sparse_linear_forward_group(hs, 1, 1, None, 0, None) == 1      # NULL y array
    assert L.sparse_linear_forward_group(hs, 1, None, ys, 0, None) == 1     # NULL x
    assert L.sparse_linear_forward_group(hs, 0, 1, ys, 0, None) == 1        # count < 1
    assert L.sparse_linear_forward_group(hs, 9, 1, ys, 0, None) == 1        # count > 8
    assert L.sparse_linear_forward_group(hs, 2, 1, ys, 0, None) == 1        # NULL handles
    assert L.sparse_linear_forward_group(hs, 1, 1, ys, 7, None) == 1        # bad y dtype
    assert "handle" in slib.sparse_linear_last_error() or "dtype" in slib.sparse_linear_last_error()


def test_forward_group_batch_rejects_bad_arguments(slib):
    L = slib.lib()
    hs = (ctypes.c_void_p * 2)(None, None)
    ys = (ctypes.c_void_p * 2)(1, 1)
    assert L.sparse_linear_forward_group_batch(None, 1, 1, 2, ys, 0, None) == 1  # NULL handle array
    assert L.sparse_linear_forward_group_batch(hs, 1, 1, 2, None, 0, None) == 1  # NULL y array
    assert L.sparse_linear_forward_group_batch(hs, 1, None, 2, ys, 0, None) == 1  # NULL x
    assert L.sparse_linear_forward_group_batch(hs, 9, 1, 2, ys, 0, None) == 1    # count > 8
    assert L.sparse_linear_forward_group_batch(hs, 1, 1, 0, ys, 0, None) == 1    # B < 1
    assert L.sparse_linear_forward_group_batch(hs, 2, 1, 2, ys, 0, None) == 1    # NULL handles
    assert "B=" in slib.sparse_linear_last_error() or "handle" in slib.sparse_linear_last_error()


def test_strerror(slib):
    assert slib.sparse_linear_strerror(0) == "success"
    assert slib.sparse_linear_strerror(2) == "unsupported shape or alignment"
    assert slib.sparse_linear_strerror(99) == "unknown status"


# ------------------------------------------------ Double Sparsity entry points
_P = 1 << 20  # a 1 MiB-aligned stand-in address: checks reject before any device access


def _ds(slib, q=_P, key=_P, value=_P, label=_P, ch=_P, sl=_P, B=2, H=4, S=128, d=128, r=16, k=8, scale=0.1,
        out=_P, toks=0):
    return slib.lib().ds_decode_attention(q or None, key or None, value or None, label or None, ch or None,
                                          sl or None, B, H, S, d, r, k, scale, out or None, toks or None, None)


@pytest.mark.parametrize("kw, status", [
    (dict(q=0), 1), (dict(key=0), 1), (dict(value=0), 1), (dict(ch=0), 1), (dict(sl=0), 1), (dict(out=0), 1),
    (dict(label=0), 1),                       # label needed while k < max_seq
    (dict(B=0), 1), (dict(H=0), 1), (dict(S=0), 1), (dict(S=32769), 1),
    (dict(d=96), 2), (dict(d=256), 2), (dict(r=12), 2), (dict(r=64), 2),
    (dict(k=0), 1), (dict(k=-3), 1), (dict(S=20000, k=8193), 2),
    (dict(scale=float("inf")), 1), (dict(scale=float("nan")), 1),
    (dict(label=_P + 8), 2), (dict(q=_P + 8), 2), (dict(d=64, q=_P + 4), 2), (dict(out=_P + 2), 1),
    (dict(toks=_P + 2), 1), (dict(B=1 << 16, H=1 << 16), 1),
    (dict(toks=_P, k=40000), 1),                                  # tokens_out with k above DS_MAX_SEQ
])
def test_ds_decode_rejects(slib, kw, status):
    assert _ds(slib, **kw) == status
    assert slib.lib().sparse_linear_last_error()


def test_ds_label_update_rejects(slib):
    L = slib.lib()
    f = lambda **kw: L.ds_label_cache_update(kw.get("key", _P) or None, kw.get("label", _P) or None,
                                             kw.get("ch", _P) or None, kw.get("start", 0) or None,
                                             kw.get("B", 2), kw.get("H", 4), kw.get("S", 128), kw.get("d", 128),
                                             kw.get("r", 16), kw.get("span", 128), None)
    assert f(key=0) == 1 and f(label=0) == 1 and f(ch=0) == 1
    assert f(d=32) == 2 and f(r=4) == 2 and f(S=0) == 1 and f(span=-1) == 1
    assert f(label=_P + 4) == 2 and f(start=_P + 2) == 1
    assert f(span=0) == 0          # nothing to do: no device access


def test_timeline_setter_unsupported_in_regular_build(slib):
    """The regular library has no timestamp points: installing a buffer is
    refused without touching a device."""
    st = slib.lib().sparse_linear_set_timeline(None)
    assert st == slib.SL_ERR_UNSUPPORTED
    assert "timestamps" in slib.sparse_linear_last_error()


def test_timeline_library_exports_every_declared_symbol(slib):
    """The timeline build (fused.hip with its timestamp points) is the same
    ABI; it loads without a device."""
    from free_activation_sparse_amd import build as _build
    if not os.path.exists(_build.LIB_TIMELINE):
        _build.build()
    L = ctypes.CDLL(_build.LIB_TIMELINE)
    for name in _declared():
        assert hasattr(L, name), name
