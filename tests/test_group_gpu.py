"""GPU parity of the grouped single-token forward (sparse_linear_forward_group):
linears that share their input x (the q/k/v and gate/up projections of a
decoder block, each with its own weights, norms and per-component K or keep
fraction) run in one launch; every linear's y must match the oracle run on
that linear alone (relative L2 2e-3) and the linear's own single forward up
to summation order."""
import numpy as np
import pytest

import oracle
import workloads as wl
from parity_util import REL_L2_TOL, gate_kwargs, rel_l2, tile_rows, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def fas(slib):
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return slib


def _layer(fas, W, c, mode, **g):
    return fas.SparseLinear(to_dev(W, torch), c=to_dev(c, torch), **gate_kwargs(mode, **g))


def _check_group(fas, layers, Ws, cs, gs, mode, x, ctx, rows_per=64):
    xd = to_dev(x, torch)
    ys = fas.SparseLinear.forward_group(layers, xd)
    for l in layers:
        l.sync_status()
    for i, (layer, W, c, g) in enumerate(zip(layers, Ws, cs, gs)):
        rows = np.random.default_rng(i).choice(W.shape[0], min(rows_per, W.shape[0]), replace=False)
        ref = oracle.forward(W, c, x, mode, rows=rows, **g)
        got = ys[i].cpu().numpy()[rows]
        err = rel_l2(got, ref["y"])
        if np.linalg.norm(ref["y"]) == 0:
            assert np.count_nonzero(got) == 0, f"{ctx} linear {i}: y must be exactly 0"
        else:
            assert err <= REL_L2_TOL, f"{ctx} linear {i}: rel L2 {err:.3e}"
        single = layer.forward(xd[None, :])["y"][0]
        layer.sync_status()
        assert rel_l2(ys[i].cpu().numpy(), single.cpu().numpy()) <= 1e-5, f"{ctx} linear {i}: vs single forward"
    return ys


def test_group_llama3_block_inputs(fas):
    """q, k, v (4096, 1024, 1024 rows) and gate, up (14336 rows) of the
    Llama-3-8B block take the same hidden state; per-component sparsity."""
    ps = wl.component_sparsities(3)
    lins = wl.CONFIGS[3].linears
    idx = [li for li, l in enumerate(lins) if l.name in ("q", "k", "v", "gate", "up")]
    Ws = [wl.weight(3, li) for li in idx]
    cs = [oracle.column_norms(W) for W in Ws]
    gs = [dict(K=wl.k_from_sparsity(lins[li].n, round(ps[li], 6))) for li in idx]
    layers = [_layer(fas, W, c, "topk", **g) for W, c, g in zip(Ws, cs, gs)]
    for t in range(3):
        x = wl.token(3, idx[0], t)
        for sel, name in (([0, 1, 2], "qkv"), ([3, 4], "gate/up"), ([0, 1, 2, 3, 4], "all five")):
            print(f"[group {name}] token {t}", flush=True)
            _check_group(fas, [layers[i] for i in sel], [Ws[i] for i in sel], [cs[i] for i in sel],
                         [gs[i] for i in sel], "topk", x, f"{name} token {t}")
    for l in layers:
        l.close()


def test_group_stat_and_fixed(fas):
    """Statistical gates (one gate workgroup per linear, each summing its own
    token's scores, inside one launch) and fixed thresholds, on ragged row
    counts sharing n."""
    n = 5120
    ms = [1024, 2056, 520]
    Ws = [wl.random_matrix(150 + i, m, n, "bf16") for i, m in enumerate(ms)]
    cs = [oracle.column_norms(W) for W in Ws]
    for mode, gs in (("stat", [dict(s_keep=s) for s in (0.1, 0.3, 0.05)]),
                     ("fixed", [dict(tau=t) for t in (0.02, 0.05, 0.0)])):
        layers = [_layer(fas, W, c, mode, **g) for W, c, g in zip(Ws, cs, gs)]
        for t, kind in enumerate(["laplace", "normal", "laplace"]):
            x = wl.random_tokens(160 + t, 1, n, "bf16", kind)[0]
            print(f"[group {mode}] token {t}", flush=True)
            _check_group(fas, layers, Ws, cs, gs, mode, x, f"{mode} token {t}")
        for l in layers:
            l.close()


def test_group_fallbacks_and_single(fas):
    """bf16 outputs, a deterministic handle or mixed gate modes run the
    linears one after another; a group of one is a plain forward."""
    n = 2048
    Ws = [wl.random_matrix(170 + i, m, n, "bf16") for i, m in enumerate((512, 1032))]
    cs = [oracle.column_norms(W) for W in Ws]
    x = wl.random_tokens(171, 1, n, "bf16", "laplace")[0]
    xd = to_dev(x, torch)
    layers = [_layer(fas, Ws[0], cs[0], "topk", K=700), _layer(fas, Ws[1], cs[1], "stat", s_keep=0.2)]
    refs = [oracle.forward(Ws[0], cs[0], x, "topk", K=700)["y"],
            oracle.forward(Ws[1], cs[1], x, "stat", s_keep=0.2)["y"]]
    for y_dtype in (torch.float32, torch.bfloat16):
        ys = fas.SparseLinear.forward_group(layers, xd, y_dtype=y_dtype)
        torch.cuda.synchronize()
        for y, ref in zip(ys, refs):
            assert rel_l2(y.float().cpu().numpy(), ref) <= REL_L2_TOL
    layers[0].set_deterministic(True)
    ys = fas.SparseLinear.forward_group(layers[:1], xd)
    torch.cuda.synchronize()
    assert rel_l2(ys[0].cpu().numpy(), refs[0]) <= REL_L2_TOL
    for l in layers:
        l.close()


def test_group_graph_replays(fas):
    """Grouped launches captured in a graph re-arm every linear's hand-off
    and advance its generation on the device: replays match eager runs."""
    n = 4096
    Ws = [wl.random_matrix(180 + i, m, n, "bf16") for i, m in enumerate((2048, 1024))]
    cs = [oracle.column_norms(W) for W in Ws]
    layers = [_layer(fas, Ws[0], cs[0], "topk", K=1500), _layer(fas, Ws[1], cs[1], "stat", s_keep=0.15)]
    for l in layers:
        l.set_deterministic(False)
    xs = [to_dev(wl.random_tokens(181 + t, 1, n, "bf16", "laplace")[0], torch) for t in range(4)]
    # same gate mode inside a group: one group per mode, two linears each
    pairs = [[layers[0], _layer(fas, Ws[1], cs[1], "topk", K=900)],
             [layers[1], _layer(fas, Ws[0], cs[0], "stat", s_keep=0.25)]]
    eager = [[y.clone() for y in fas.SparseLinear.forward_group(pairs[i % 2], x)] for i, x in enumerate(xs)]
    torch.cuda.synchronize()
    outs = [[torch.empty_like(y) for y in e] for e in eager]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i, x in enumerate(xs):
            fas.SparseLinear.forward_group(pairs[i % 2], x, ys=outs[i])
    for rep in range(3):
        for o in outs:
            for y in o:
                y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for pair in pairs:
            for l in pair:
                l.sync_status()
        for i in range(len(xs)):
            for y, e in zip(outs[i], eager[i]):
                assert rel_l2(y.cpu().numpy(), e.cpu().numpy()) <= 1e-5, f"replay {rep} group {i}"
    for pair in pairs:
        for l in pair:
            l.close()


def test_group_and_ffn_reject_duplicate_handles(fas):
    # one handle twice would share its hand-off state and scratch between two
    # linears of one launch: rejected before anything is enqueued
    n, m = 512, 1024
    Ws = [wl.random_matrix(240 + i, *s, "bf16") for i, s in enumerate(((m, n), (m, n), (n, m)))]
    cs = [oracle.column_norms(W) for W in Ws]
    ls = [_layer(fas, W, c, "topk", K=k) for W, c, k in zip(Ws, cs, (300, 300, 500))]
    x = to_dev(wl.random_tokens(241, 1, n, "bf16")[0], torch)
    ys = [torch.full((m,), 7.0, device="cuda:0") for _ in range(2)]
    torch.cuda.synchronize()
    with pytest.raises(fas.SparseLinearError) as e:
        fas.SparseLinear.forward_group([ls[0], ls[0]], x, ys)
    assert e.value.status == fas.SL_ERR_ARG and "same handle" in str(e.value)
    with pytest.raises(fas.SparseLinearError) as e:
        fas.SparseLinear.forward_group([ls[0], ls[1], ls[0]], x, ys + [torch.empty(m, device="cuda:0")])
    assert e.value.status == fas.SL_ERR_ARG
    torch.cuda.synchronize()
    assert bool((ys[0] == 7.0).all()) and bool((ys[1] == 7.0).all())  # nothing ran
    for args in ((ls[0], ls[0], ls[2]), (ls[0], ls[1], ls[0]), (ls[1], ls[1], ls[1])):
        with pytest.raises(fas.SparseLinearError) as e:
            fas.SparseLinear.forward_ffn(*args, x)
        assert e.value.status == fas.SL_ERR_ARG
    # distinct handles still run
    ys = fas.SparseLinear.forward_group([ls[0], ls[1]], x)
    for l in ls:
        l.sync_status()
    for l in ls:
        l.close()


def _layer_b(fas, W, c, mode, B, **g):
    return fas.SparseLinear(to_dev(W, torch), c=to_dev(c, torch), max_batch=B, **gate_kwargs(mode, **g))


@pytest.mark.parametrize("cfg,mode,B,g", [(5, "topk", 16, 0.65), (5, "topk", 3, 0.9), (4, "stat", 4, 0.10),
                                          (4, "stat", 2, 0.10)])
def test_group_batch_gate_up(fas, cfg, mode, B, g):
    """A batch through the gate and up projections of the Qwen-2.5-7B and
    Phi-4 FFNs (sparse_linear_forward_group_batch: both linears' gates for
    every token in one launch, then each linear's union product): every
    token's y of every linear matches the oracle on that token and linear
    (rows of every 256-row tile), and the linear's own batched forward up to
    summation order; twice, the second time with the first call's
    thresholds as the gates' prior."""
    lins = wl.CONFIGS[cfg].linears
    idx = [li for li, l in enumerate(lins) if l.name in ("gate", "up")]
    Ws = [wl.weight(cfg, li) for li in idx]
    cs = [oracle.column_norms(W) for W in Ws]
    if mode == "topk":
        gs = [dict(K=wl.k_from_sparsity(lins[li].n, g)) for li in idx]
    else:
        gs = [dict(s_keep=g) for _ in idx]
    layers = [_layer_b(fas, W, c, mode, B, **gg) for W, c, gg in zip(Ws, cs, gs)]
    m = Ws[0].shape[0]
    rows = tile_rows(m, 5)
    for call in range(2):
        X = wl.tokens(cfg, idx[0], 200 + 16 * call, B)
        xd = to_dev(X, torch)
        print(f"[group batch cfg {cfg} {mode} B={B}] call {call}", flush=True)
        ys = fas.SparseLinear.forward_group(layers, xd)
        for l in layers:
            l.sync_status()
        for i, (layer, W, c, gg) in enumerate(zip(layers, Ws, cs, gs)):
            single = layer.forward(xd)["y"]
            layer.sync_status()
            got = ys[i].cpu().numpy()
            assert rel_l2(got, single.cpu().numpy()) <= 1e-5, f"linear {i} call {call}: vs batched forward"
            for b in range(B):
                ref = oracle.forward(W, c, X[b], mode, rows=rows, **gg)
                err = rel_l2(got[b][rows], ref["y"])
                assert err <= REL_L2_TOL, f"linear {i} call {call} token {b}: rel L2 {err:.3e}"
    for l in layers:
        l.close()


def test_group_batch_falls_back(fas):
    """Mixed gate modes in one batch call run the linears one after another
    (same results as their own forwards); B above a handle's max_batch is
    rejected."""
    m, n, B = 512, 2048, 4
    W1, W2 = wl.random_matrix(150, m, n, "bf16"), wl.random_matrix(151, m, n, "bf16")
    c1, c2 = oracle.column_norms(W1), oracle.column_norms(W2)
    a = _layer_b(fas, W1, c1, "topk", B, K=700)
    b = _layer_b(fas, W2, c2, "stat", B, s_keep=0.2)
    X = wl.random_tokens(152, B, n, "bf16", "laplace")
    xd = to_dev(X, torch)
    ys = fas.SparseLinear.forward_group([a, b], xd)
    for layer, y in ((a, ys[0]), (b, ys[1])):
        single = layer.forward(xd)["y"]
        layer.sync_status()
        assert rel_l2(y.cpu().numpy(), single.cpu().numpy()) <= 1e-5
    small = _layer_b(fas, W2, c2, "topk", 2, K=100)
    with pytest.raises(fas.SparseLinearError):
        fas.SparseLinear.forward_group([a, small], xd)
    for l in (a, b, small):
        l.close()
