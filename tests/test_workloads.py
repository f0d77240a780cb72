"""The seeded input module: bf16 rounding, the K-from-sparsity rule, seeding."""
import numpy as np
import torch

import workloads as wl


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(31)
    a = (g.standard_normal(100000) * np.exp2(g.integers(-30, 30, 100000))).astype(np.float32)
    # exact halfway cases between bf16 neighbours, both parities
    half = (np.arange(1, 2001, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    a = np.concatenate([a, half, -half, np.array([0.0, -0.0, 1e-40, -1e-40], np.float32)])
    want = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(wl.f32_to_bf16_bits(a), want)
    back = wl.bf16_bits_to_f32(want)
    np.testing.assert_array_equal(back, torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_k_from_sparsity_values():
    assert wl.k_from_sparsity(256, 0.5) == 128
    assert wl.k_from_sparsity(11008, 0.5) == 5504
    assert wl.k_from_sparsity(11008, 0.65) == 3853
    assert wl.k_from_sparsity(3584, 0.65) == 1255
    assert wl.k_from_sparsity(3584, 0.90) == 359
    assert wl.k_from_sparsity(18944, 0.65) == 6631
    assert wl.k_from_sparsity(18944, 0.90) == 1895
    assert wl.k_from_sparsity(100, 0.0) == 100
    assert wl.k_from_sparsity(100, 1.0) == 0


def test_draws_are_seeded_and_shaped():
    a = wl.weight(2, 0, m=64, n=32)
    b = wl.weight(2, 0, m=64, n=32)
    assert a.dtype == np.uint16 and a.shape == (64, 32)
    np.testing.assert_array_equal(a, b)
    t0 = wl.token(2, 0, 0, n=100)
    t1 = wl.token(2, 0, 1, n=100)
    assert not np.array_equal(t0, t1)
    assert wl.weight(1, 0).dtype == np.float32 and wl.weight(1, 0).shape == (512, 256)
    p = wl.component_sparsities(3)
    assert len(p) == 7 and all(0.3 <= v < 0.7 for v in p)
    assert p == wl.component_sparsities(3)


def test_config3_shared_inputs():
    # q, k, v, gate and up read one hidden state per token
    q = wl.token(3, 0, 5)
    k = wl.token(3, 1, 5)
    up = wl.token(3, 5, 5)
    o = wl.token(3, 3, 5)
    np.testing.assert_array_equal(q, k)
    np.testing.assert_array_equal(q, up)
    assert not np.array_equal(q, o)


# ------------------------------------------- Double Sparsity decode inputs
def test_decode_inputs_seeded_and_prefix_stable():
    from workloads import decode_attention as wda
    c = wda.DecodeCase("t", 3, 4, 64, 50, 8, 5, ragged=True, seed=7)
    a, b = wda.make_inputs(c), wda.make_inputs(c)
    for f in ("q", "key", "value", "channels", "seq_len"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    p = wda.make_inputs(c, batch=2)          # the first sequences of the full case
    assert np.array_equal(p.key, a.key[:2]) and np.array_equal(p.q, a.q[:2])
    assert np.all((a.seq_len >= 1) & (a.seq_len <= 50))
    assert a.key.dtype == np.uint16 and a.channels.dtype == np.int32


def test_decode_inputs_outlier_channels():
    # the channel list starts with the heavy channels, whose keys are scaled up
    from workloads import decode_attention as wda
    c = wda.DecodeCase("t", 2, 3, 128, 4000, 16, 10, seed=8)
    inp = wda.make_inputs(c)
    kf = (inp.key.astype(np.uint32) << 16).view(np.float32)
    std = kf.std(axis=(0, 2))                # per (head, channel)
    for h in range(3):
        heavy = inp.channels[h, :c.heavy]
        rest = np.setdiff1d(np.arange(128), heavy)
        assert np.all(np.abs(std[h, heavy] - c.outlier_scale) < 0.2)
        assert np.all(np.abs(std[h, rest] - 1.0) < 0.1)
        assert len(set(inp.channels[h].tolist())) == 16
