"""Pins for the oracle's sparse product (Spark Transformer article, section 3.1:
the index-list product y += x_j * W[j] over the active indices) and the
single-layer error bound of the WINA article, section 二.

Checks: exact integer brute force in pure Python, one-hot inputs, the dense
case against correctly rounded sums (math.fsum), the Pythagorean error
identity for orthogonal columns and the WINA <= TEAL error inequality.
"""
import math

import numpy as np

import oracle
from workloads import f32_to_bf16_bits


def test_product_integer_brute_force():
    g = np.random.default_rng(21)
    for _ in range(20):
        m, n = int(g.integers(1, 9)), int(g.integers(1, 12))
        W = g.integers(-50, 51, (m, n)).astype(np.float32)
        x = g.integers(-9, 10, n).astype(np.float32)
        idx = np.sort(g.choice(n, int(g.integers(0, n + 1)), replace=False))
        want = [sum(int(W[i, j]) * int(x[j]) for j in idx.tolist()) for i in range(m)]
        got = oracle.sparse_product(W, x, idx)
        assert got.tolist() == [float(v) for v in want]


def test_product_one_hot():
    g = np.random.default_rng(22)
    W = f32_to_bf16_bits(g.standard_normal((33, 17), dtype=np.float32))
    Wf = oracle.as_f64(W)
    x = np.zeros(17, np.float32)
    x[5] = 1.0
    np.testing.assert_array_equal(oracle.sparse_product(W, x, np.array([5])), Wf[:, 5])
    np.testing.assert_array_equal(oracle.sparse_product(W, x, np.array([4, 6])), np.zeros(33))
    np.testing.assert_array_equal(oracle.sparse_product(W, x, np.array([], np.int64)), np.zeros(33))


def test_product_dense_vs_fsum():
    g = np.random.default_rng(23)
    W = g.standard_normal((40, 300), dtype=np.float32)
    x = g.standard_normal(300, dtype=np.float32)
    got = oracle.sparse_product(W, x, np.arange(300))
    for i in range(40):
        exact = math.fsum(float(W[i, j]) * float(x[j]) for j in range(300))  # products exact
        assert abs(got[i] - exact) <= 1e-12 * max(1.0, abs(exact))


def test_product_rows_subset():
    g = np.random.default_rng(24)
    W = g.standard_normal((50, 20), dtype=np.float32)
    x = g.standard_normal(20, dtype=np.float32)
    idx = np.array([1, 4, 9, 19])
    rows = [0, 7, 49]
    np.testing.assert_array_equal(oracle.sparse_product_rows(W, x, idx, rows),
                                  oracle.sparse_product(W, x, idx)[rows])


def _orthogonal_scaled(g, m, n):
    Q, _ = np.linalg.qr(g.standard_normal((m, n)))
    d = np.exp(g.uniform(np.log(0.1), np.log(10.0), n))
    return (Q * d)


def test_orthogonal_error_identity():
    """For orthogonal columns, ||Wx - y_sparse||^2 = sum_dropped x_j^2 ||W_j||^2
    (W kept in fp64 so the columns stay orthogonal to rounding level)."""
    g = np.random.default_rng(25)
    m, n, K = 128, 64, 24
    W = _orthogonal_scaled(g, m, n)
    c = oracle.column_norms(W)
    for _ in range(20):
        x = g.standard_normal(n).astype(np.float32)
        out = oracle.forward(W, c, x, "topk", K=K)
        xf = x.astype(np.float64)
        dense = W @ xf
        err = np.sum((dense - out["y"]) ** 2)
        dropped = np.setdiff1d(np.arange(n), out["idx"])
        closed = np.sum(xf[dropped] ** 2 * np.sum(W[:, dropped] ** 2, axis=0))
        assert abs(err - closed) <= 1e-11 * max(closed, 1e-30)
        # and the dropped energy equals the sum of squared dropped scores, to fp32 rounding
        s = out["scores"].astype(np.float64)
        assert abs(closed - np.sum(s[dropped] ** 2)) <= 1e-6 * closed


def test_wina_error_not_above_teal():
    """WINA article, section 二: with column-orthogonal W (here W = Q D, the
    form the SVD transform of section 五 produces), keeping the K largest
    |x_j| ||W_j|| never leaves more output error than keeping the K largest |x_j|."""
    g = np.random.default_rng(26)
    viol = 0
    for trial in range(200):
        m, n = 64, 48
        K = int(g.integers(1, n))
        W = _orthogonal_scaled(g, m, n).astype(np.float32)
        x = g.standard_normal(n).astype(np.float32)
        c = oracle.column_norms(W)
        dense = oracle.sparse_product(W, x, np.arange(n))
        wina = oracle.forward(W, c, x, "topk", K=K)["y"]
        teal = oracle.forward(W, np.ones(n, np.float32), x, "topk", K=K)["y"]
        e_w = np.sum((dense - wina) ** 2)
        e_t = np.sum((dense - teal) ** 2)
        if e_w > e_t * (1 + 1e-6) + 1e-12:
            viol += 1
    assert viol == 0
