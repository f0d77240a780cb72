"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Masks, counts and thresholds must match bit for bit; y within relative L2
2e-3 of the fp64 oracle. Inputs are the seeded workloads (full layer sizes
where the oracle can follow, sampled output rows where it cannot compute
every row quickly) plus ragged and degenerate edge cases.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from parity_util import REL_L2_TOL, check_token, gate_kwargs, rel_l2, tile_rows, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def fas(slib):
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return slib


def _layer(fas, W, c, mode, K=None, s_keep=None, tau=None, layout="rowmajor", max_batch=1, pass_c=True):
    Wd = to_dev(W if layout == "rowmajor" else np.ascontiguousarray(W.T), torch)
    cd = to_dev(c, torch) if pass_c else None
    return fas.SparseLinear(Wd, c=cd, layout=layout, max_batch=max_batch,
                            **gate_kwargs(mode, K=K, s_keep=s_keep, tau=tau))


def _fwd(layer, x, **kw):
    out = layer.forward(to_dev(x, torch)[None, :], mask=True, count=True, thresh=True, **kw)
    layer.sync_status()  # synchronizes; raises if a fused hand-off timed out
    return out


# ---------------------------------------------------------------- config 1
def test_tiny_config_all_tokens(fas):
    cfg = wl.CONFIGS[1]
    W = wl.weight(1, 0)
    c = oracle.column_norms(W)
    K = wl.k_from_sparsity(256, 0.5)
    layer = _layer(fas, W, c, "topk", K=K)
    for t in range(cfg.tokens):
        x = wl.token(1, 0, t)
        print(f"[tiny] token {t}", flush=True)
        check_token(_fwd(layer, x), 0, W, c, x, "topk", K=K, ctx="tiny")


def test_tiny_bf16_output(fas):
    W = wl.weight(1, 0)
    c = oracle.column_norms(W)
    layer = _layer(fas, W, c, "topk", K=128)
    x = wl.token(1, 0, 3)
    out = _fwd(layer, x, y_dtype=torch.bfloat16)
    assert out["y"].dtype == torch.bfloat16
    # bf16 rounding of y adds up to 2^-9 relative per element
    check_token(out, 0, W, c, x, "topk", K=128, tol=REL_L2_TOL, ctx="tiny-bf16y")


# ---------------------------------------------------------------- config 2
@pytest.fixture(scope="module")
def llama_down():
    W = wl.weight(2, 0)
    return W, oracle.column_norms(W)


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("sparsity", [0.5, 0.65])
def test_llama7b_down_full_size(fas, llama_down, sparsity, fused):
    W, c = llama_down
    K = wl.k_from_sparsity(W.shape[1], sparsity)
    layer = _layer(fas, W, c, "topk", K=K)
    layer.set_fused(fused)
    rows = tile_rows(W.shape[0], 7)
    for t in range(12):
        x = wl.token(2, 0, t)
        print(f"[llama-down p={sparsity}] token {t}", flush=True)
        full = t < 2  # the whole y for two tokens, a row of every tile for the rest
        check_token(_fwd(layer, x), 0, W, c, x, "topk", K=K, rows=None if full else rows, ctx="llama-down")
    layer.close()


def test_llama7b_down_plans(fas, llama_down):
    """Every launch shape gives the same masks and an oracle-close y."""
    W, c = llama_down
    K = wl.k_from_sparsity(W.shape[1], 0.65)
    layer = _layer(fas, W, c, "topk", K=K)
    x = wl.token(2, 0, 100)
    rows = np.arange(0, W.shape[0], 37)
    for rpt in (128, 256, 512):
        for splits in (1, 7, 64, 300):
            print(f"[plan] rows {rpt} splits {splits}", flush=True)
            layer.set_plan(rpt, splits)
            check_token(_fwd(layer, x), 0, W, c, x, "topk", K=K, rows=rows, ctx=f"plan {rpt}/{splits}")
    layer.close()


# ---------------------------------------------------------------- STAT gate (config 4 shapes)
@pytest.mark.parametrize("linear", [0, 1, 2])
def test_phi4_stat_gate_full_size(fas, linear):
    W = wl.weight(4, linear)
    c = oracle.column_norms(W)
    layer = _layer(fas, W, c, "stat", s_keep=0.10)
    rows = tile_rows(W.shape[0], 9 + linear)
    for t in range(8):
        x = wl.token(4, linear, t)
        print(f"[phi4 stat linear {linear}] token {t}", flush=True)
        check_token(_fwd(layer, x), 0, W, c, x, "stat", s_keep=0.10, rows=None if t == 0 else rows,
                    ctx="phi4-stat")
    layer.close()


# ---------------------------------------------------------------- config 3 (seven linears)
def test_llama3_block_linears(fas):
    ps = wl.component_sparsities(3)
    for li, lin in enumerate(wl.CONFIGS[3].linears):
        W = wl.weight(3, li)
        c = oracle.column_norms(W)
        K = wl.k_from_sparsity(lin.n, round(ps[li], 6))
        layer = _layer(fas, W, c, "topk", K=K)
        rows = tile_rows(lin.m, li)
        for t in range(3):
            x = wl.token(3, li, t)
            print(f"[llama3 {lin.name}] token {t} K={K}", flush=True)
            check_token(_fwd(layer, x), 0, W, c, x, "topk", K=K, rows=None if t == 0 else rows,
                        ctx=f"llama3-{lin.name}")
        layer.close()
        del W


# ---------------------------------------------------------------- edge cases
EDGE_SHAPES = [(8, 1), (136, 1000), (520, 2049), (1032, 300), (64, 4100)]


@pytest.mark.parametrize("m,n", EDGE_SHAPES)
@pytest.mark.parametrize("dtype,fused", [("bf16", True), ("bf16", False), ("f32", False)])
def test_ragged_shapes_topk(fas, m, n, dtype, fused):
    W = wl.random_matrix(m * 7 + n, m, n, dtype)
    c = oracle.column_norms(W)
    g = np.random.default_rng(m + n)
    for K in sorted({0, 1, n // 3, n - 1, n}):
        if K < 0:
            continue
        layer = _layer(fas, W, c, "topk", K=K)
        layer.set_fused(fused)
        for t, kind in enumerate(["normal", "ties"]):
            x = wl.random_tokens(m + n + t, 1, n, dtype, kind)[0]
            print(f"[ragged {dtype} {m}x{n} fused={fused}] K={K} {kind}", flush=True)
            check_token(_fwd(layer, x), 0, W, c, x, "topk", K=K, ctx=f"ragged {m}x{n} K={K} {kind}")
        layer.close()
    del g


@pytest.mark.parametrize("s_keep", [0.02, 0.1, 0.5, 0.9])
def test_stat_gate_small(fas, s_keep):
    m, n = 264, 3000
    W = wl.random_matrix(5, m, n, "bf16")
    c = oracle.column_norms(W)
    layer = _layer(fas, W, c, "stat", s_keep=s_keep)
    for t, kind in enumerate(["laplace", "normal", "ties"]):
        x = wl.random_tokens(50 + t, 1, n, "bf16", kind)[0]
        check_token(_fwd(layer, x), 0, W, c, x, "stat", s_keep=s_keep, ctx=f"stat s={s_keep} {kind}")
    layer.close()


@pytest.mark.parametrize("dtype,fused", [("f32", False), ("bf16", False), ("bf16", True)])
def test_stat_gate_constant_scores(fas, dtype, fused):
    # every score equal: sigma = 0, t = mu, nothing kept, y = 0
    m, n = 64, 500
    W = wl.random_matrix(6, m, n, dtype)
    c = np.ones(n, np.float32)
    layer = _layer(fas, W, c, "stat", s_keep=0.1)
    layer.set_fused(fused)
    x = np.full(n, -0.75, np.float32)
    if dtype == "bf16":
        x = wl.f32_to_bf16_bits(x)
    out = _fwd(layer, x)
    check_token(out, 0, W, c, x, "stat", s_keep=0.1, ctx="stat-constant")
    assert int(out["count"][0]) == 0 and float(out["thresh"][0]) == 0.75
    assert torch.count_nonzero(out["y"]).item() == 0


@pytest.mark.parametrize("p,s_keep", [(0.5, 0.15865525393145707), (0.2, 0.02275013194817921)])
@pytest.mark.parametrize("fused", [True, False])
def test_stat_threshold_on_a_score(fas, p, s_keep, fused):
    """Two score values a > b, a fraction p of the inputs at a, and s_keep =
    1 - Phi(sqrt((1 - p) / p)): then t = a up to the last bits of z, so a
    score lies within any rounding bound of t. The first threshold from plain
    sums cannot decide such a token; the exact moments must, bit for bit (all
    inputs at a kept or none, as the exact t falls)."""
    m, n = 1024, 6000
    W = wl.random_matrix(140, m, n, "bf16")
    c = np.ones(n, np.float32)
    layer = _layer(fas, W, c, "stat", s_keep=s_keep)
    layer.set_fused(fused)
    rng = np.random.default_rng(141)
    for t in range(3):
        x = np.ones(n, np.float32)
        x[rng.permutation(n)[: int(round(p * n))]] = 2.0
        x *= np.float32(1.0 + 0.25 * t)  # a, b exact in bf16
        xb = wl.f32_to_bf16_bits(x)
        out = _fwd(layer, xb)
        check_token(out, 0, W, c, xb, "stat", s_keep=s_keep, ctx=f"stat on a score p={p} token {t}")
    layer.close()


def test_stat_fused_plans(fas):
    """Fused statistical gate under every launch shape (row tiles of 128, 256
    and 512 rows; 1 to 150 input chunks, including more workgroups than the
    device holds at once and chunks of 34 inputs): the gate workgroup sums the
    token's scores itself, so masks, counts and thresholds must equal the
    oracle's and the two-launch path's whatever the product's layout."""
    m, n = 2048, 5000
    W = wl.random_matrix(130, m, n, "bf16")
    c = oracle.column_norms(W)
    layer = _layer(fas, W, c, "stat", s_keep=0.15)
    xs = [wl.random_tokens(131 + t, 1, n, "bf16", kind)[0] for t, kind in enumerate(["laplace", "normal", "ties"])]
    layer.set_fused(False)
    ref = [{k: v.clone() for k, v in _fwd(layer, x).items()} for x in xs]
    layer.set_fused(True)
    rows = np.arange(0, m, 29)
    for rpt in (128, 256, 512):
        for splits in (1, 5, 64, 150):
            layer.set_plan(rpt, splits)
            for t, x in enumerate(xs):
                print(f"[stat plan] rows {rpt} splits {splits} token {t}", flush=True)
                out = _fwd(layer, x)
                for k in ("mask", "count", "thresh"):
                    assert torch.equal(out[k], ref[t][k]), (rpt, splits, t, k)
                check_token(out, 0, W, c, x, "stat", s_keep=0.15, rows=rows, ctx=f"stat plan {rpt}/{splits}")
    layer.close()


@pytest.mark.parametrize("tau", [0.0, 0.01, 0.05, 1e9])
def test_fixed_threshold(fas, tau):
    m, n = 128, 2000
    W = wl.random_matrix(8, m, n, "bf16")
    c = oracle.column_norms(W)
    layer = _layer(fas, W, c, "fixed", tau=tau)
    x = wl.random_tokens(9, 1, n, "bf16", "laplace")[0]
    check_token(_fwd(layer, x), 0, W, c, x, "fixed", tau=tau, ctx=f"fixed tau={tau}")
    # without requested outputs the gate kernel is skipped; y must not change
    y2 = layer.forward(to_dev(x, torch)[None, :])["y"]
    torch.cuda.synchronize()
    ref = oracle.forward(W, c, x, "fixed", tau=tau)
    assert rel_l2(y2[0].cpu().numpy(), ref["y"]) <= REL_L2_TOL
    layer.close()


@pytest.mark.parametrize("det", [False, True])
def test_fixed_threshold_fused_full_size(fas, llama_down, det):
    """Fixed (calibrated) threshold on the Llama-2-7B down projection: the
    fused launch, where the product workgroups stream the kept set without
    waiting for a selection, against the oracle, with and without requested
    outputs, for a threshold near the median score (about half kept), 0
    (every nonzero score kept) and one above every score (y exactly 0)."""
    W, c = llama_down
    x0 = wl.token(2, 0, 200)
    tau_mid = float(np.median(oracle.scores(x0, c)))
    rows = np.random.default_rng(11).choice(W.shape[0], 64, replace=False)
    for tau in (tau_mid, 0.0, 1e30):
        layer = _layer(fas, W, c, "fixed", tau=tau)
        layer.set_deterministic(det)
        for t in range(4):
            x = wl.token(2, 0, 200 + t)
            print(f"[fixed fused det={det}] tau={tau:.4g} token {t}", flush=True)
            check_token(_fwd(layer, x), 0, W, c, x, "fixed", tau=tau, rows=rows, ctx=f"fixed tau={tau:.3g}")
            y2 = layer.forward(to_dev(x, torch)[None, :])["y"]
            layer.sync_status()
            ref = oracle.forward(W, c, x, "fixed", tau=tau)["y"]
            if tau == 1e30:
                assert torch.count_nonzero(y2).item() == 0
            else:
                assert rel_l2(y2[0].cpu().numpy()[rows], ref[rows]) <= REL_L2_TOL
        layer.close()


# ---------------------------------------------------------------- identities
def test_topk_all_equals_dense_kernel(fas):
    m, n = 1024, 4096
    W = wl.random_matrix(10, m, n, "bf16")
    c = oracle.column_norms(W)
    layer = _layer(fas, W, c, "topk", K=n)
    layer.set_deterministic(True)  # ordered reduction: same kernel, same bits
    x = to_dev(wl.random_tokens(11, 1, n, "bf16")[0], torch)[None, :]
    yf = layer.forward(x)["y"].clone()  # fused launch: its own split plan
    layer.set_fused(False)
    ys = layer.forward(x)["y"]
    yd = layer.forward_dense(x)
    layer.sync_status()
    assert torch.equal(ys, yd)
    assert rel_l2(yf[0].cpu().numpy(), yd[0].cpu().numpy()) <= 1e-6
    ref = oracle.sparse_product(W, wl.random_tokens(11, 1, n, "bf16")[0], np.arange(n))
    assert rel_l2(yd[0].cpu().numpy(), ref) <= REL_L2_TOL
    layer.close()


def test_one_hot_input_returns_column(fas):
    m, n = 512, 777
    W = wl.random_matrix(12, m, n, "bf16")
    c = oracle.column_norms(W)
    layer = _layer(fas, W, c, "topk", K=5)
    for j in (0, 1, 400, n - 1):
        x = np.zeros(n, np.float32)
        x[j] = 1.0
        xb = wl.f32_to_bf16_bits(x)
        out = _fwd(layer, xb)
        want = oracle.as_f64(W)[:, j]
        np.testing.assert_array_equal(out["y"][0].cpu().numpy().astype(np.float64), want)
        assert out["mask"][0].cpu().numpy().sum() == 5
    layer.close()


def test_orthogonal_error_identity_on_gpu(fas):
    g = np.random.default_rng(13)
    m, n, K = 512, 256, 100
    Q, _ = np.linalg.qr(g.standard_normal((m, n)))
    d = np.exp(g.uniform(np.log(0.1), np.log(10.0), n))
    W = (Q * d).astype(np.float32)
    c = oracle.column_norms(W)
    layer = _layer(fas, W, c, "topk", K=K)
    x = g.standard_normal(n).astype(np.float32)
    out = _fwd(layer, x)
    yd = layer.forward_dense(to_dev(x, torch)[None, :])
    torch.cuda.synchronize()
    diff = (yd[0].double() - out["y"][0].double()).cpu().numpy()
    mask = out["mask"][0].cpu().numpy().astype(bool)
    s = oracle.scores(x, c).astype(np.float64)
    closed = np.sum(s[~mask] ** 2)
    assert abs(np.sum(diff ** 2) - closed) <= 1e-4 * closed
    layer.close()


def test_library_norms_and_colmajor_layout(fas):
    m, n = 2056, 1500
    W = wl.random_matrix(14, m, n, "bf16")
    c = oracle.column_norms(W)
    for layout in ("rowmajor", "colmajor"):
        layer = _layer(fas, W, c, "topk", K=600, layout=layout, pass_c=False)
        got = layer.norms().cpu().numpy()
        ulp = np.spacing(c)
        assert np.all(np.abs(got.astype(np.float64) - c) <= ulp), layout
        x = wl.random_tokens(15, 1, n, "bf16")[0]
        out = _fwd(layer, x)
        # the library's own c differs from the oracle's in at most an ulp; compare with its own c
        check_token(out, 0, W, got, x, "topk", K=600, ctx=f"lib-norms {layout}")
        layer.close()


def test_forward_is_deterministic(fas, llama_down):
    """With the ordered split reduction repeated forwards agree to the bit; the
    default atomic reduction agrees to fp32 summation-order rounding."""
    W, c = llama_down
    layer = _layer(fas, W, c, "topk", K=3853)
    x = to_dev(wl.token(2, 0, 5), torch)[None, :]
    ya = [layer.forward(x)["y"].clone() for _ in range(5)]
    layer.set_deterministic(True)
    ys = [layer.forward(x)["y"].clone() for _ in range(5)]
    ys.append(layer.forward(x, y_dtype=torch.bfloat16)["y"].float())
    torch.cuda.synchronize()
    for y in ys[1:5]:
        assert torch.equal(y, ys[0])
    for y in ya:
        assert rel_l2(y.cpu().numpy(), ys[0].cpu().numpy()) <= 1e-6
    assert rel_l2(ys[5].cpu().numpy(), ys[0].cpu().numpy()) <= 4e-3
    layer.close()


def test_graph_replay_matches_eager(fas, llama_down):
    """Forwards captured in a HIP graph give the eager results on every replay,
    with eager work and synchronizations between the replays."""
    W, c = llama_down
    m = W.shape[0]
    layers = [_layer(fas, W, c, "topk", K=3853), _layer(fas, W, c, "topk", K=5504)]
    for l in layers:
        l.set_deterministic(True)
    xs = [to_dev(wl.token(2, 0, t), torch)[None, :] for t in range(6)]
    eager = [layers[i % 2].forward(x)["y"].clone() for i, x in enumerate(xs)]
    torch.cuda.synchronize()
    ys = [torch.empty((1, m), dtype=torch.float32, device="cuda:0") for _ in xs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i, (x, y) in enumerate(zip(xs, ys)):
            layers[i % 2].forward(x, y=y)
    for rep in range(4):
        for y in ys:
            y.fill_(float("nan"))
        layers[0].forward(xs[rep])  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (y, e) in enumerate(zip(ys, eager)):
            assert torch.equal(y, e), f"replay {rep} forward {i}"
    for l in layers:
        l.close()


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("det", [False, True])
def test_reduction_modes_match_oracle(fas, llama_down, det, fused):
    """Both split reductions (atomic fp32, ordered) and the bf16 output, at
    several launch shapes, on the full Llama-7B down projection, for the fused
    launch and the gate + product launches."""
    W, c = llama_down
    K = wl.k_from_sparsity(W.shape[1], 0.5)
    layer = _layer(fas, W, c, "topk", K=K)
    layer.set_deterministic(det)
    layer.set_fused(fused)
    rows = np.arange(0, W.shape[0], 41)
    for rpt, splits in ((128, 16), (256, 32), (512, 0), (128, 1)):
        layer.set_plan(rpt, splits)
        for t in range(2):
            x = wl.token(2, 0, 40 + t)
            print(f"[reduction det={det} fused={fused}] {rpt}/{splits} token {t}", flush=True)
            check_token(_fwd(layer, x), 0, W, c, x, "topk", K=K, rows=rows, ctx=f"det={det} {rpt}/{splits}")
            check_token(_fwd(layer, x, y_dtype=torch.bfloat16), 0, W, c, x, "topk", K=K, rows=rows,
                        ctx=f"det={det} bf16 {rpt}/{splits}")
    layer.close()


def test_dense_forward_modes(fas, llama_down):
    W, c = llama_down
    layer = _layer(fas, W, c, "topk", K=10)
    x = wl.token(2, 0, 7)
    xd = to_dev(x, torch)[None, :]
    ref = oracle.sparse_product(W, x, np.arange(W.shape[1]))
    for det in (False, True):
        layer.set_deterministic(det)
        y = layer.forward_dense(xd)
        yb = layer.forward_dense(xd, y_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert rel_l2(y[0].cpu().numpy(), ref) <= REL_L2_TOL
        assert rel_l2(yb[0].float().cpu().numpy(), ref) <= REL_L2_TOL
    layer.close()


# ---------------------------------------------------------------- fused launch vs gate + product launches
@pytest.mark.parametrize("mode", ["topk", "stat"])
def test_fused_matches_two_launch(fas, mode):
    """The fused launch and the gate kernel + product kernel give identical
    masks, counts and thresholds, and the same y up to summation order, over
    shapes that take every gate register variant (n up to 32768)."""
    for m, n in ((256, 4096), (1024, 8200), (512, 16384), (256, 20480), (128, 32768)):
        W = wl.random_matrix(90 + n, m, n, "bf16")
        c = oracle.column_norms(W)
        g = dict(K=n // 3) if mode == "topk" else dict(s_keep=0.1)
        layer = _layer(fas, W, c, mode, **g)
        x = wl.random_tokens(91 + n, 1, n, "bf16", "laplace")[0]
        print(f"[fused vs two-launch {mode}] {m}x{n}", flush=True)
        layer.set_fused(True)
        a = _fwd(layer, x)
        a = {k: v.clone() for k, v in a.items()}
        layer.set_fused(False)
        b = _fwd(layer, x)
        assert torch.equal(a["mask"], b["mask"])
        assert torch.equal(a["count"], b["count"])
        assert torch.equal(a["thresh"], b["thresh"])
        assert rel_l2(a["y"][0].cpu().numpy(), b["y"][0].cpu().numpy()) <= 1e-6
        layer.set_fused(True)
        check_token(a, 0, W, c, x, mode, rows=np.arange(0, m, 5), ctx=f"fused {m}x{n}", **g)
        layer.close()


def test_fused_graph_replays_rearm(fas):
    """The fused launch re-arms its hand-off word itself: many captured
    forwards of two layers, replayed repeatedly, give the eager results."""
    m, n = 2048, 5120
    W = wl.random_matrix(95, m, n, "bf16")
    c = oracle.column_norms(W)
    layers = [_layer(fas, W, c, "topk", K=1500), _layer(fas, W, c, "stat", s_keep=0.2)]
    for l in layers:
        l.set_deterministic(True)
    xs = [to_dev(wl.random_tokens(96 + t, 1, n, "bf16", "laplace")[0], torch)[None, :] for t in range(8)]
    eager = [layers[i % 2].forward(x)["y"].clone() for i, x in enumerate(xs)]
    ys = [torch.empty((1, m), dtype=torch.float32, device="cuda:0") for _ in xs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i, (x, y) in enumerate(zip(xs, ys)):
            layers[i % 2].forward(x, y=y)
    for rep in range(5):
        for y in ys:
            y.fill_(float("nan"))
        layers[1].forward(xs[rep])
        torch.cuda.synchronize()
        g.replay()
        for l in layers:
            l.sync_status()
        for i, (y, e) in enumerate(zip(ys, eager)):
            assert torch.equal(y, e), f"replay {rep} forward {i}"
    for l in layers:
        l.close()


def test_fused_speculation_paths(fas):
    """The fused launch streams, ahead of its gate, the inputs whose score is
    well above the handle's previous threshold, and checks that bound against
    the exact threshold. Token scales jumping between calls make the
    speculation fail (dropped and redone), hold, or be empty; every call must
    still match the oracle exactly in mask, count and threshold."""
    m, n = 1024, 6144
    W = wl.random_matrix(120, m, n, "bf16")
    c = oracle.column_norms(W)
    base = [wl.bf16_bits_to_f32(wl.random_tokens(121 + i, 1, n, "bf16", "laplace")[0]) for i in range(4)]
    scales = [1.0, 1.0, 0.1, 1.0, 10.0, 10.0, 1e-3, 1.0, 1.0, 1.05, 0.95]
    for K in (1, 700, n // 2, n - 1, n):
        layer = _layer(fas, W, c, "topk", K=K)
        for i, sc in enumerate(scales):
            x = wl.f32_to_bf16_bits(base[i % 4] * np.float32(sc))
            print(f"[speculation] K={K} call {i} scale {sc}", flush=True)
            check_token(_fwd(layer, x), 0, W, c, x, "topk", K=K, rows=np.arange(0, m, 3),
                        ctx=f"speculation K={K} call {i}")
        layer.close()
    layer = _layer(fas, W, c, "stat", s_keep=0.2)
    for i, sc in enumerate(scales):
        x = wl.f32_to_bf16_bits(base[i % 4] * np.float32(sc))
        check_token(_fwd(layer, x), 0, W, c, x, "stat", s_keep=0.2, rows=np.arange(0, m, 3),
                    ctx=f"speculation stat call {i}")
    layer.close()
