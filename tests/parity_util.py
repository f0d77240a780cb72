"""Helpers for the GPU parity tests: moving seeded inputs to the device and
comparing the library's outputs with the CPU oracle."""
import numpy as np

import oracle

REL_L2_TOL = 2e-3  # relative L2 error bound on y against the fp64 oracle


def to_dev(a, torch, device="cuda:0"):
    """numpy fp32 or bf16-bits (uint16) array -> device tensor of that dtype."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def tile_rows(m, seed, block=128):
    """Sampled output rows that cover every row tile of the kernels' launch
    shapes: one random row from each block of `block` rows (the kernels use
    128-, 256- and 512-row tiles, so every tile of any of them gets at least
    one), plus the last row."""
    g = np.random.default_rng(seed)
    rows = [int(g.integers(b, min(m, b + block))) for b in range(0, m, block)]
    rows.append(m - 1)
    return np.unique(np.asarray(rows, dtype=np.int64))


def gate_kwargs(mode, K=None, s_keep=None, tau=None):
    if mode == "topk":
        return dict(gate="topk", K=K)
    if mode == "stat":
        return dict(gate="stat", s_keep=s_keep)
    return dict(gate="fixed", tau=tau)


def rel_l2(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    nw = np.linalg.norm(want)
    if nw == 0.0:
        return 0.0 if np.all(got == 0) else np.inf
    return float(np.linalg.norm(got - want) / nw)


def check_token(out_gpu, b, W, c, x, mode, K=None, s_keep=None, tau=None, rows=None, tol=REL_L2_TOL,
                ctx=""):
    """Compare token b of a forward's outputs with the oracle. ``rows`` limits
    the product check to sampled output rows."""
    ref = oracle.forward(W, c, x, mode, K=K, s_keep=s_keep, tau=tau, rows=rows)
    y = out_gpu["y"][b].float().cpu().numpy().astype(np.float64)
    if rows is not None:
        y = y[np.asarray(rows)]
    if out_gpu.get("mask") is not None:
        mask = out_gpu["mask"][b].cpu().numpy().astype(bool)
        if not np.array_equal(mask, ref["mask"]):
            diff = np.flatnonzero(mask != ref["mask"])
            raise AssertionError(f"{ctx} token {b}: mask differs at {diff[:10]} (count {diff.size})")
    if out_gpu.get("count") is not None:
        assert int(out_gpu["count"][b]) == ref["count"], f"{ctx} token {b}: count"
    if out_gpu.get("thresh") is not None:
        th = float(out_gpu["thresh"][b])
        assert th == ref["thresh"] or (np.isinf(th) and np.isinf(ref["thresh"])), \
            f"{ctx} token {b}: thresh {th!r} vs {ref['thresh']!r}"
    err = rel_l2(y, ref["y"])
    assert err <= tol, f"{ctx} token {b}: rel L2 {err:.3e} > {tol}"
    return ref, err
