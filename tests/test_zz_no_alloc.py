"""GPU test of the allocation-free FFN entry point
(sparse_linear_forward_ffn_noalloc), called through the C ABI: its y must
equal that of sparse_linear_forward_ffn (caller workspace) on the same
handles and token, on two calls in a row, the second with a smaller layer.
The handles use the ordered split reduction, so both entry points are
bit-reproducible and the comparison is exact; widths above the static
workspace are rejected before anything is enqueued."""
import numpy as np
import pytest

import oracle
import workloads as wl
from parity_util import REL_L2_TOL, gate_kwargs, rel_l2, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def fas(slib):
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return slib


def _chain(fas, n, m, seed, Ks):
    shapes = ((m, n), (m, n), (n, m))
    Ws = [wl.random_matrix(seed + i, a, b, "bf16") for i, (a, b) in enumerate(shapes)]
    cs = [oracle.column_norms(W) for W in Ws]
    ls = [fas.SparseLinear(to_dev(W, torch), c=to_dev(c, torch), **gate_kwargs("topk", K=K))
          for W, c, K in zip(Ws, cs, Ks)]
    for l in ls:
        l.set_deterministic(True)
    return Ws, cs, ls


def _noalloc(fas, ls, x, y):
    fas.sparse_linear_forward_ffn_noalloc(ls[0].handle, ls[1].handle, ls[2].handle, x.data_ptr(), y.data_ptr(),
                                          fas.SL_F32, torch.cuda.current_stream().cuda_stream)


def test_noalloc_matches_workspace_entry_point(fas):
    big = _chain(fas, 1024, 4096, 500, (400, 350, 1500))
    small = _chain(fas, 512, 1536, 510, (200, 180, 700))
    xb = to_dev(wl.random_tokens(520, 1, 1024, "bf16")[0], torch)
    xs = to_dev(wl.random_tokens(521, 1, 512, "bf16")[0], torch)
    yb = torch.full((1024,), float("nan"), device="cuda:0")
    ys = torch.full((512,), float("nan"), device="cuda:0")
    print("[noalloc] call 1: 4096-wide intermediate", flush=True)
    _noalloc(fas, big[2], xb, yb)
    print("[noalloc] call 2: 1536-wide intermediate", flush=True)
    _noalloc(fas, small[2], xs, ys)
    for l in big[2] + small[2]:
        l.sync_status()
    ref_b, _ = fas.SparseLinear.forward_ffn(*big[2], xb)
    ref_s, _ = fas.SparseLinear.forward_ffn(*small[2], xs)
    torch.cuda.synchronize()
    assert torch.isfinite(yb).all().item() and torch.isfinite(ys).all().item()
    assert torch.equal(yb, ref_b), "first call differs from the workspace entry point"
    assert torch.equal(ys, ref_s), "second (smaller) call differs from the workspace entry point"
    # and a repeat of the large call after the small one (the array keeps the
    # small call's contents, which the large call must overwrite)
    _noalloc(fas, big[2], xb, yb)
    torch.cuda.synchronize()
    assert torch.equal(yb, ref_b)
    # the down projection's product against the oracle on the entry point's
    # own intermediate: h from the workspace entry point (identical bits)
    _, ws = fas.SparseLinear.forward_ffn(*small[2], xs)
    torch.cuda.synchronize()
    p = (4 * 1536 + 255) // 256 * 256
    h = ws.cpu().numpy()[2 * p:2 * p + 2 * 1536].view(np.uint16)
    Ws, cs, _ = small
    want = oracle.forward(Ws[2], cs[2], h, "topk", K=700)["y"]
    assert rel_l2(ys.cpu().numpy(), want) <= REL_L2_TOL
    for l in big[2] + small[2]:
        l.close()


def test_noalloc_rejects_width_above_static_workspace(fas):
    n, m = 64, 20480 + 8  # the static workspace holds intermediate widths up to 20480
    _, _, ls = _chain(fas, n, m, 530, (32, 32, 1000))
    x = to_dev(wl.random_tokens(531, 1, n, "bf16")[0], torch)
    y = torch.full((n,), 3.0, device="cuda:0")
    torch.cuda.synchronize()
    with pytest.raises(fas.SparseLinearError) as e:
        _noalloc(fas, ls, x, y)
    assert e.value.status == fas.SL_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())  # nothing ran
    for l in ls:
        l.close()
