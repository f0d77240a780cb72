"""GPU parity of batched forwards (B > 1): each token's mask, count and
threshold bit-exact against the oracle run on that token alone, and each
token's y within relative L2 2e-3. For bf16 weights the library runs one
matrix-core pass over the union of the B kept sets; the union is invisible in
the results, which is what these tests check."""
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


def _layer(fas, W, c, mode, max_batch, K=None, s_keep=None, tau=None):
    return fas.SparseLinear(to_dev(W, torch), c=to_dev(c, torch), max_batch=max_batch,
                            **gate_kwargs(mode, K=K, s_keep=s_keep, tau=tau))


def _fwd(layer, X, **kw):
    out = layer.forward(to_dev(X, torch), mask=True, count=True, thresh=True, **kw)
    torch.cuda.synchronize()
    return out


def _check_all(out, W, c, X, mode, rows=None, ctx="", full=(), **g):
    """Every token of the batch; tokens listed in `full` compare their whole y."""
    for b in range(X.shape[0]):
        check_token(out, b, W, c, X[b], mode, rows=None if b in full else rows, ctx=f"{ctx} b={b}", **g)


# ---------------------------------------------------------------- config 4: Phi-4 FFN, STAT gate
@pytest.mark.parametrize("linear", [0, 1, 2])
def test_phi4_stat_batched(fas, linear):
    W = wl.weight(4, linear)
    c = oracle.column_norms(W)
    layer = _layer(fas, W, c, "stat", 8, s_keep=0.10)
    rows = tile_rows(W.shape[0], linear)
    first = 0
    for B in (2, 4, 8):
        X = wl.tokens(4, linear, first, B)
        first += B
        print(f"[phi4 stat linear {linear}] B={B}", flush=True)
        _check_all(_fwd(layer, X), W, c, X, "stat", rows=rows, ctx=f"phi4 B={B}", full=(0,) if B == 8 else (),
                   s_keep=0.10)
    layer.close()


# ---------------------------------------------------------------- config 5: Qwen2.5-7B FFN, B = 16
@pytest.mark.parametrize("linear", [0, 1, 2])
@pytest.mark.parametrize("sparsity", [0.65, 0.90])
def test_qwen_b16_topk(fas, linear, sparsity):
    W = wl.weight(5, linear)
    c = oracle.column_norms(W)
    K = wl.k_from_sparsity(W.shape[1], sparsity)
    layer = _layer(fas, W, c, "topk", 16, K=K)
    rows = tile_rows(W.shape[0], linear + 7)
    # two batches of the 16 x 16 tokens: the first and the tenth
    for batch in (0, 9):
        X = wl.tokens(5, linear, 16 * batch, 16)
        print(f"[qwen linear {linear} p={sparsity}] K={K} batch {batch}", flush=True)
        _check_all(_fwd(layer, X), W, c, X, "topk", rows=rows, ctx=f"qwen p={sparsity} batch {batch}",
                   full=(0,) if batch == 0 else (), K=K)
    layer.close()


# ---------------------------------------------------------------- ragged shapes and modes
@pytest.mark.parametrize("m,n", [(8, 5), (136, 1000), (520, 2049), (264, 300), (1032, 4100)])
@pytest.mark.parametrize("B", [2, 3, 16])
def test_union_ragged_topk(fas, m, n, B):
    W = wl.random_matrix(31 * m + n, m, n, "bf16")
    c = oracle.column_norms(W)
    for K in sorted({0, 1, n // 5, n - 1, n}):
        layer = _layer(fas, W, c, "topk", 16, K=K)
        kinds = ["normal", "ties"]
        X = np.concatenate([wl.random_tokens(m + n + B + i, 1, n, "bf16", kinds[i % 2]) for i in range(B)])
        print(f"[union ragged {m}x{n}] B={B} K={K}", flush=True)
        _check_all(_fwd(layer, X), W, c, X, "topk", ctx=f"union {m}x{n} B={B} K={K}", K=K)
        layer.close()


def test_union_speculative_first_steps(fas):
    """A batch whose expected union is near-dense makes the union product load
    its first steps before the union is known, assuming each chunk starts
    with a dense run of columns. Inputs that no token keeps (x = 0 in every
    token at chosen columns, with K below the count of nonzero inputs) break
    that run at different depths in different chunks: in the first, second
    and third 32-column step of chunk 0, the last column of another chunk's
    third step, and nowhere in the rest. Every token must still match the
    oracle exactly in mask, count and threshold."""
    m, n, B = 512, 4096, 16
    W = wl.random_matrix(140, m, n, "bf16")
    c = oracle.column_norms(W)
    X = wl.random_tokens(141, B, n, "bf16", "laplace")
    holes = [5, 40, 70, 512 + 95, 2048 + 33]
    Xf = wl.bf16_bits_to_f32(X)
    Xf[:, holes] = 0.0
    X = wl.f32_to_bf16_bits(Xf)
    for K in (n // 2, n - 2 * len(holes)):
        layer = _layer(fas, W, c, "topk", 16, K=K)
        print(f"[union speculation] K={K}", flush=True)
        out = _fwd(layer, X)
        _check_all(out, W, c, X, "topk", rows=np.arange(0, m, 7), ctx=f"spec K={K}", K=K)
        assert not out["mask"][:, holes].any().item()
        layer.close()


@pytest.mark.parametrize("det", [False, True])
def test_union_reduction_modes_and_bf16(fas, det):
    m, n, B = 2056, 3000, 5
    W = wl.random_matrix(77, m, n, "bf16")
    c = oracle.column_norms(W)
    layer = _layer(fas, W, c, "stat", 8, s_keep=0.3)
    layer.set_deterministic(det)
    X = wl.random_tokens(78, B, n, "bf16", "laplace")
    _check_all(_fwd(layer, X), W, c, X, "stat", ctx=f"det={det}", s_keep=0.3)
    _check_all(_fwd(layer, X, y_dtype=torch.bfloat16), W, c, X, "stat", ctx=f"det={det} bf16", s_keep=0.3)
    if det:
        y1 = _fwd(layer, X)["y"].clone()
        y2 = _fwd(layer, X)["y"]
        assert torch.equal(y1, y2)
    layer.close()


def test_union_dense_and_fixed(fas):
    m, n, B = 1024, 2000, 4
    W = wl.random_matrix(79, m, n, "bf16")
    c = oracle.column_norms(W)
    X = wl.random_tokens(80, B, n, "bf16", "laplace")
    layer = _layer(fas, W, c, "fixed", 4, tau=0.03)
    _check_all(_fwd(layer, X), W, c, X, "fixed", ctx="fixed", tau=0.03)
    y2 = layer.forward(to_dev(X, torch))["y"]  # no outputs requested: no gate kernel
    yd = layer.forward_dense(to_dev(X, torch))
    torch.cuda.synchronize()
    for b in range(B):
        ref = oracle.forward(W, c, X[b], "fixed", tau=0.03)["y"]
        assert rel_l2(y2[b].cpu().numpy(), ref) <= REL_L2_TOL
        dref = oracle.sparse_product(W, X[b], np.arange(n))
        assert rel_l2(yd[b].cpu().numpy(), dref) <= REL_L2_TOL
    layer.close()


def test_fp32_weights_batched(fas):
    """fp32 weights take the single-token kernel once per token."""
    W = wl.weight(1, 0)
    c = oracle.column_norms(W)
    layer = _layer(fas, W, c, "topk", 4, K=128)
    X = np.stack([wl.token(1, 0, t) for t in range(4)])
    _check_all(_fwd(layer, X), W, c, X, "topk", ctx="fp32 batched", K=128)
    layer.close()


def test_union_graph_replay(fas):
    m, n, B = 3584, 4096, 16
    W = wl.random_matrix(81, m, n, "bf16")
    c = oracle.column_norms(W)
    layer = _layer(fas, W, c, "topk", 16, K=1400)
    layer.set_deterministic(True)
    Xs = [to_dev(wl.random_tokens(82 + i, B, n, "bf16"), torch) for i in range(3)]
    eager = [layer.forward(X)["y"].clone() for X in Xs]
    ys = [torch.empty((B, m), dtype=torch.float32, device="cuda:0") for _ in Xs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for X, y in zip(Xs, ys):
            layer.forward(X, y=y)
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        layer.forward(Xs[rep])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (y, e) in enumerate(zip(ys, eager)):
            assert torch.equal(y, e), f"replay {rep} forward {i}"
    layer.close()
