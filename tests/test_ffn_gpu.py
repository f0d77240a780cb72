"""GPU parity of the sparse FFN chain (sparse_linear_forward_ffn): g and u
(sparse gate and up projections of one token, one grouped launch), the
epilogue h = bf16(SiLU(g) * u), and the sparse down projection with its own
gate on h.

Per stage, on the stage's actual input: g and u against the oracle on x; h
against oracle.silu_mul of the device's g and u (fp32 SiLU on the device, one
fp64 rounding in the oracle: equal except for rare one-ulp ties); y against the
oracle on the device's h, with the down projection's mask, count and
threshold bit-exact.

End to end, from x alone: y against oracle.ffn_chain (fp64 g and u, one bf16
rounding of h, the down gate on the oracle's own h). The device's fp32 g and u
put a few h values on the other side of a bf16 rounding boundary, so the two
down gates may disagree on inputs whose score lies within that rounding of the
threshold; where they do, every differing input must be such a borderline
input, and y must match the oracle's product over the device's kept set."""
import numpy as np
import pytest

import oracle
import workloads as wl
from parity_util import REL_L2_TOL, check_token, gate_kwargs, rel_l2, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def fas(slib):
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return slib


def _layer(fas, W, c, mode, **g):
    return fas.SparseLinear(to_dev(W, torch), c=to_dev(c, torch), **gate_kwargs(mode, **g))


def _bf16_value(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _split_ws(ws, m):
    p = (4 * m + 255) // 256 * 256
    b = ws.cpu().numpy()
    g = b[:4 * m].view(np.float32).astype(np.float64)
    u = b[p:p + 4 * m].view(np.float32).astype(np.float64)
    h = b[2 * p:2 * p + 2 * m].view(np.uint16)
    return g, u, h


@pytest.mark.parametrize("mode", ["topk", "stat"])
def test_ffn_chain_llama2_shapes(fas, mode):
    n, m = 4096, 11008  # Llama-2-7B FFN: gate/up 11008 x 4096, down 4096 x 11008
    Wg = wl.random_matrix(200, m, n, "bf16")
    Wu = wl.random_matrix(201, m, n, "bf16")
    Wd = wl.random_matrix(202, n, m, "bf16")
    cg, cu, cd = (oracle.column_norms(W) for W in (Wg, Wu, Wd))
    if mode == "topk":
        gg, gu, gd = dict(K=2048), dict(K=2048), dict(K=5504)
    else:
        gg, gu, gd = dict(s_keep=0.3), dict(s_keep=0.3), dict(s_keep=0.2)
    lg, lu, ld = _layer(fas, Wg, cg, mode, **gg), _layer(fas, Wu, cu, mode, **gu), _layer(fas, Wd, cd, mode, **gd)
    rows = np.random.default_rng(3).choice(n, 96, replace=False)
    strict = 0
    for t in range(3):
        x = wl.random_tokens(210 + t, 1, n, "bf16", "normal")[0]
        print(f"[ffn {mode}] token {t}", flush=True)
        y, ws = fas.SparseLinear.forward_ffn(lg, lu, ld, to_dev(x, torch))
        for l in (lg, lu, ld):
            l.sync_status()
        g, u, h = _split_ws(ws, m)
        # 1. gate and up
        for name, got, W, c, gk in (("gate", g, Wg, cg, gg), ("up", u, Wu, cu, gu)):
            ref = oracle.forward(W, c, x, mode, **gk)["y"]
            assert rel_l2(got, ref) <= REL_L2_TOL, f"{name} token {t}"
        # 2. epilogue: fp32 SiLU on the device vs the oracle's fp64 SiLU and
        #    single rounding, on the device's g and u: equal except at rare
        #    rounding ties, by one ulp
        want = oracle.silu_mul(g, u)
        diff = np.abs(h.astype(np.int64) - want.astype(np.int64))
        assert diff.max() <= 1 and np.count_nonzero(diff) <= m // 1000, f"h token {t}: {np.count_nonzero(diff)}"
        # 3. down on the device's h: y against the oracle, and the mask,
        #    count and threshold of a forward with outputs bit-exact
        ref = oracle.forward(Wd, cd, h, mode, rows=rows, **gd)["y"]
        assert rel_l2(y.cpu().numpy()[rows], ref) <= REL_L2_TOL, f"y token {t}"
        out = ld.forward(torch.from_numpy(h.view(np.int16)).to("cuda:0").view(torch.bfloat16)[None, :],
                         mask=True, count=True, thresh=True)
        ld.sync_status()
        check_token(out, 0, Wd, cd, h, mode, rows=rows, ctx=f"ffn down token {t}", **gd)
        # 4. end to end from x
        e2e = oracle.ffn_chain(Wg, cg, dict(mode=mode, **gg), Wu, cu, dict(mode=mode, **gu),
                               Wd, cd, dict(mode=mode, **gd), x)
        hv, ho = _bf16_value(h), _bf16_value(e2e["h"])
        # one bf16 ulp, plus an absolute slack for h near zero, where the fp32
        # g and u of the device may differ from fp64 in more than the last bit
        ulp = np.maximum(np.abs(hv), np.abs(ho)) * 2.0 ** -7 + 1e-4 * np.sqrt(np.mean(ho * ho))
        assert np.all(np.abs(hv - ho) <= ulp), f"h end to end token {t}"
        assert np.count_nonzero(hv != ho) <= m // 50, f"h end to end token {t}: {np.count_nonzero(hv != ho)}"
        mask_dev = out["mask"][0].cpu().numpy().astype(bool)
        mask_or = e2e["down"]["mask"]
        y_dev = y.cpu().numpy().astype(np.float64)
        if np.array_equal(mask_dev, mask_or):
            strict += 1
            err = rel_l2(y_dev, e2e["y"])
            assert err <= REL_L2_TOL, f"y end to end token {t}: rel L2 {err:.3e}"
        else:
            # borderline inputs only: scores within two bf16 roundings of the threshold
            sc = e2e["down"]["scores"].astype(np.float64)
            th = float(e2e["down"]["thresh"])
            d = np.flatnonzero(mask_dev != mask_or)
            assert np.all(np.abs(sc[d] - th) <= 2.0 ** -6 * th), f"token {t}: non-borderline gate difference {d}"
            want_y = oracle.sparse_product(Wd, e2e["h"], np.flatnonzero(mask_dev))
            err = rel_l2(y_dev, want_y)
            assert err <= REL_L2_TOL, f"y end to end (device kept set) token {t}: rel L2 {err:.3e}"
        print(f"[ffn {mode}] token {t}: h differs from the end-to-end oracle in {np.count_nonzero(hv != ho)} of {m}; "
              f"down gates {'agree' if np.array_equal(mask_dev, mask_or) else 'differ at borderline inputs'}", flush=True)
    assert strict >= 1, "no token had identical down gates end to end"
    for l in (lg, lu, ld):
        l.close()


def test_ffn_chain_rejects_bad_workspace(fas):
    n, m = 512, 1024
    Ws = [wl.random_matrix(220 + i, *s, "bf16") for i, s in enumerate(((m, n), (m, n), (n, m)))]
    cs = [oracle.column_norms(W) for W in Ws]
    ls = [_layer(fas, W, c, "topk", K=k) for W, c, k in zip(Ws, cs, (300, 300, 500))]
    x = to_dev(wl.random_tokens(221, 1, n, "bf16")[0], torch)
    nb = fas.sparse_linear_ffn_workspace_bytes(ls[1].handle)
    assert nb >= 10 * m
    short = torch.empty((nb - 256,), dtype=torch.uint8, device="cuda:0")
    with pytest.raises(fas.SparseLinearError):
        fas.SparseLinear.forward_ffn(ls[0], ls[1], ls[2], x, workspace=short)
    with pytest.raises(fas.SparseLinearError):  # shapes that do not chain
        fas.SparseLinear.forward_ffn(ls[0], ls[1], ls[0], x)
    y, _ = fas.SparseLinear.forward_ffn(ls[0], ls[1], ls[2], x)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all().item()
    for l in ls:
        l.close()
