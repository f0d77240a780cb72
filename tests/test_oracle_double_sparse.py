"""Pins for the Double Sparsity decode-attention oracle (CPU only).

The pages print no numeric example for Double Sparsity, so the oracle is
pinned to a hand-derived case with closed-form outputs, to torch's
scaled_dot_product_attention where the selection keeps every token, to exact
q.k scores when the label holds every channel, to brute-force dominance of the
kept set, and to invariances of the output under changes of unkept cache rows.
"""
import math

import numpy as np
import pytest

from oracle import double_sparse as ds
from workloads import decode_attention as wda
from workloads import f32_to_bf16_bits

LN2 = math.log(2.0)
E = math.e


def _tiny():
    # d = 4 (scale 1/2), q = [2, 0, 1, 0], label channels [2, 0] -> sparse query [1, 2]
    q = np.array([2.0, 0.0, 1.0, 0.0])
    K = np.array([[LN2, 9, 1, 9],    # approx 1 + 2 ln2, full logit ln2 + 1/2
                  [0, 9, 1, 9],      # approx 1,  full logit 1/2
                  [-5, 0, 0, 0],     # approx -10 (largest magnitude, smallest value), logit -5
                  [0, -9, 3, 0],     # approx 3,  full logit 3/2
                  [0, 9, 1, 9]])     # approx 1 (ties token 1), full logit 1/2
    V = np.array([[1.0, 0, 0, 0], [0, 1, 0, 0], [0, 0, 1, 0], [0, 0, 0, 1], [1, 1, 1, 1]])
    ch = np.array([[2, 0]])
    return q, K, V, ch


def test_tiny_label_cache():
    q, K, V, ch = _tiny()
    L = ds.label_cache(K[None], ch)[0]
    assert np.array_equal(L, np.array([[1, LN2], [1, 0], [0, -5], [3, 0], [1, 0]]))


def test_tiny_scores_and_selection():
    q, K, V, ch = _tiny()
    L = ds.label_cache(K[None], ch)[0]
    s = ds.approx_scores(q, L, ch[0], 5)
    want = np.array([np.float32(1) + np.float32(2) * np.float32(LN2), 1, -10, 3, 1], np.float32)
    assert np.array_equal(s, want)
    assert ds.heavy_tokens(s, 1).tolist() == [3]          # largest value, not magnitude (-10)
    assert ds.heavy_tokens(s, 2).tolist() == [0, 3]
    assert ds.heavy_tokens(s, 3).tolist() == [0, 1, 3]    # tie 1 vs 4: lower index
    assert ds.heavy_tokens(s, 4).tolist() == [0, 1, 3, 4]
    assert ds.heavy_tokens(s, 9).tolist() == [0, 1, 2, 3, 4]


@pytest.mark.parametrize("k, want", [
    (1, [0, 0, 0, 1]),
    # weights relative to e^(1/2): token 0 -> 2, token 3 -> e
    (2, [2 / (2 + E), 0, 0, E / (2 + E)]),
    (3, [2 / (3 + E), 1 / (3 + E), 0, E / (3 + E)]),
    (4, [3 / (4 + E), 2 / (4 + E), 1 / (4 + E), (E + 1) / (4 + E)]),
    (5, [3 / (4 + E + math.exp(-5.5)), 2 / (4 + E + math.exp(-5.5)),
         (1 + math.exp(-5.5)) / (4 + E + math.exp(-5.5)), (E + 1) / (4 + E + math.exp(-5.5))]),
])
def test_tiny_attention_closed_form(k, want):
    q, K, V, ch = _tiny()
    out, kept = ds.decode(q[None, None], K[None, None], V[None, None], ch, np.array([5]), k)
    np.testing.assert_allclose(out[0, 0], want, rtol=1e-14, atol=1e-15)


def _bf16(a):
    return f32_to_bf16_bits(np.asarray(a, np.float32))


def _case(B, H, S, d, r, k, seed, ragged=True):
    c = wda.DecodeCase("t", B, H, d, S, r, k, ragged=ragged, seed=seed)
    return c, wda.make_inputs(c)


@pytest.mark.parametrize("seed", [0, 1])
def test_dense_matches_torch_sdpa(seed):
    torch = pytest.importorskip("torch")
    c, inp = _case(3, 4, 90, 64, 8, 10_000, seed)
    out, kept = ds.decode(inp.q, inp.key, inp.value, inp.channels, inp.seq_len, c.k)
    f = lambda a: torch.from_numpy(ds.as_f64(a))
    for b in range(c.batch):
        n = int(inp.seq_len[b])
        assert all(len(x) == n for x in kept[b])
        ref = torch.nn.functional.scaled_dot_product_attention(
            f(inp.q[b])[:, None, :], f(inp.key[b, :, :n]), f(inp.value[b, :, :n]), scale=1.0 / math.sqrt(64))
        np.testing.assert_allclose(out[b], ref[:, 0].numpy(), rtol=1e-10, atol=1e-12)


def test_full_channel_scores_match_exact_dot_products():
    # r = d with a permuted channel list: the approximate score is q.k itself
    # up to fp32 rounding; it must lie within the sequential-sum error bound of
    # the exact fp64 product, and the kept set must equal the exact top-k
    # wherever the k-th/(k+1)-th gap exceeds twice that bound.
    c, inp = _case(2, 6, 300, 64, 64, 37, 5, ragged=False)
    gamma = 64 * 2.0 ** -24 / (1 - 64 * 2.0 ** -24)
    decided = 0
    for b in range(2):
        for h in range(6):
            qd = ds.as_f64(inp.q[b, h])
            Kd = ds.as_f64(inp.key[b, h])
            exact = Kd @ qd
            bound = gamma * (np.abs(Kd) @ np.abs(qd))
            L = ds.label_cache(inp.key[b:b + 1], inp.channels)[0, h]
            s = ds.approx_scores(inp.q[b, h], L, inp.channels[h], 300).astype(np.float64)
            assert np.all(np.abs(s - exact) <= bound)
            srt = np.sort(exact)[::-1]
            if srt[36] - srt[37] > 2 * bound.max():
                decided += 1
                want = np.sort(np.argsort(-exact, kind="stable")[:37])
                assert np.array_equal(ds.heavy_tokens(s.astype(np.float32), 37), want)
    assert decided >= 6


@pytest.mark.parametrize("r", [8, 16, 32])
def test_label_scores_exact_on_integer_inputs(r):
    # integer query and keys in [-60, 60] (exact in bf16): every partial sum is
    # an integer below 2^24, so fp32 accumulation is exact and the approximate
    # score must equal the exact dot product of q and k over the r label
    # channels, whatever the summation order; the kept set is then the exact
    # top-k of those integers (ties to the lower index)
    g = np.random.default_rng(100 + r)
    H, S, d, k = 3, 200, 128, 23
    q = g.integers(-60, 61, (H, d)).astype(np.float32)
    key = g.integers(-60, 61, (H, S, d)).astype(np.float32)
    ch = np.stack([g.permutation(d)[:r] for _ in range(H)]).astype(np.int32)
    label = ds.label_cache(_bf16(key)[None], ch)[0]
    for h in range(H):
        exact = key[h][:, ch[h]].astype(np.int64) @ q[h][ch[h]].astype(np.int64)
        s = ds.approx_scores(_bf16(q[h]), label[h], ch[h], S)
        assert np.array_equal(s.astype(np.int64), exact) and np.all(s == exact)
        order = sorted(range(S), key=lambda t: (-exact[t], t))
        assert ds.heavy_tokens(s, k).tolist() == sorted(order[:k])


@pytest.mark.parametrize("r", [8, 16, 32])
def test_label_scores_within_bound_of_exact(r):
    # Gaussian bf16 data (the benchmark's distribution): the fp32 score lies
    # within the sequential-sum error bound of the exact fp64 dot product over
    # the label channels, and the kept set equals the exact top-k wherever the
    # gap at the k-th score exceeds twice that bound
    c, inp = _case(2, 8, 400, 128, r, 40, 50 + r, ragged=False)
    gamma = r * 2.0 ** -24 / (1 - r * 2.0 ** -24)
    decided = 0
    for b in range(2):
        for h in range(8):
            chh = inp.channels[h]
            qd = ds.as_f64(inp.q[b, h])[chh]
            Kd = ds.as_f64(inp.key[b, h])[:, chh]
            exact = Kd @ qd
            bound = gamma * (np.abs(Kd) @ np.abs(qd))
            L = ds.label_cache(inp.key[b:b + 1], inp.channels)[0, h]
            s = ds.approx_scores(inp.q[b, h], L, chh, 400).astype(np.float64)
            assert np.all(np.abs(s - exact) <= bound)
            srt = np.sort(exact)[::-1]
            if srt[39] - srt[40] > 2 * bound.max():
                decided += 1
                want = np.sort(np.lexsort((np.arange(400), -exact))[:40])
                assert np.array_equal(ds.heavy_tokens(s.astype(np.float32), 40), want)
    assert decided >= 4


@pytest.mark.parametrize("seed", range(6))
def test_heavy_tokens_pairwise_dominance(seed):
    g = np.random.default_rng(seed)
    for n in (1, 2, 7, 40):
        s = g.integers(-3, 4, n).astype(np.float32)      # many exact ties, signed
        for k in range(0, n + 2):
            idx = ds.heavy_tokens(s, k).tolist()
            assert len(idx) == min(k, n) and idx == sorted(set(idx))
            kept = set(idx)
            for i in kept:
                for j in set(range(n)) - kept:
                    assert s[i] > s[j] or (s[i] == s[j] and i < j)


def test_output_ignores_unkept_rows():
    c, inp = _case(2, 3, 120, 64, 8, 17, 3)
    label = ds.label_cache(inp.key, inp.channels)
    out, kept = ds.decode(inp.q, inp.key, inp.value, inp.channels, inp.seq_len, c.k, label=label)
    K2, V2, L2 = inp.key.copy(), inp.value.copy(), label.copy()
    g = np.random.default_rng(9)
    for b in range(2):
        n = int(inp.seq_len[b])
        L2[b, :, n:] = _bf16(g.standard_normal(L2[b, :, n:].shape) * 100)
        for h in range(3):
            drop = np.setdiff1d(np.arange(120), kept[b][h])
            K2[b, h, drop] = _bf16(g.standard_normal((drop.size, 64)) * 50)
            V2[b, h, drop] = _bf16(g.standard_normal((drop.size, 64)) * 50)
    out2, kept2 = ds.decode(inp.q, K2, V2, inp.channels, inp.seq_len, c.k, label=L2)
    assert all(np.array_equal(a, b) for ra, rb in zip(kept, kept2) for a, b in zip(ra, rb))
    assert np.array_equal(out, out2)


def test_output_is_convex_combination_of_kept_values():
    c, inp = _case(2, 4, 200, 128, 16, 25, 4)
    out, kept = ds.decode(inp.q, inp.key, inp.value, inp.channels, inp.seq_len, c.k)
    for b in range(2):
        for h in range(4):
            Vk = ds.as_f64(inp.value[b, h, kept[b][h]])
            assert np.all(out[b, h] >= Vk.min(0) - 1e-12) and np.all(out[b, h] <= Vk.max(0) + 1e-12)


def test_token_permutation_maps_selection():
    c, inp = _case(1, 2, 150, 64, 8, 20, 6, ragged=False)
    out, kept = ds.decode(inp.q, inp.key, inp.value, inp.channels, inp.seq_len, c.k)
    perm = np.random.default_rng(2).permutation(150)
    out2, kept2 = ds.decode(inp.q, inp.key[:, :, perm], inp.value[:, :, perm], inp.channels, inp.seq_len, c.k)
    for h in range(2):
        s = ds.approx_scores(inp.q[0, h], ds.label_cache(inp.key, inp.channels)[0, h], inp.channels[h], 150)
        if np.unique(s).size == s.size:   # without ties the kept set is order-free
            assert np.array_equal(np.sort(perm[kept2[0][h]]), kept[0][h])
            np.testing.assert_allclose(out2[0, h], out[0, h], rtol=1e-12, atol=1e-14)


def test_empty_sequence_gives_zeros():
    c, inp = _case(1, 2, 16, 64, 8, 4, 7, ragged=False)
    out, kept = ds.decode(inp.q, inp.key, inp.value, inp.channels, np.array([0]), 4)
    assert not out.any() and all(len(x) == 0 for x in kept[0])
