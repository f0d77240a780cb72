"""Double Sparsity decode attention on the GPU against the CPU oracle.

The label cache must match the oracle's bit for bit, the kept token set must
equal the oracle's exactly (both take it from fp32 scores summed in channel
order; see the oracle's precision reading), and the attention output (fp32
on the GPU, fp64 in the oracle over the same bf16 inputs) must agree within
rel L2 <= 2e-3 per (sequence, head) -- the parity bar used for every
floating-point output of this library.
"""
import math

import numpy as np
import pytest

from oracle import double_sparse as ds
from workloads import decode_attention as wda
from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.fixture(scope="module")
def fas(slib):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return slib


def _dev(a, torch):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _host_bits(t):
    return t.cpu().view(__import__("torch").int16).numpy().view(np.uint16)


def _run(fas, inp, k, label=None, scale=None, check_label=True):
    import torch
    B, H, S, d = inp.key.shape
    r = inp.channels.shape[1]
    q, K, V = _dev(inp.q, torch), _dev(inp.key, torch), _dev(inp.value, torch)
    ch, sl = _dev(inp.channels.astype(np.int32), torch), _dev(inp.seq_len.astype(np.int32), torch)
    if label is None:
        L = torch.empty((B, H, S, r), dtype=torch.bfloat16, device="cuda")
        fas.label_cache_update(K, L, ch)
        want_label = ds.label_cache(inp.key, inp.channels)
        if check_label:
            torch.cuda.synchronize()
            assert np.array_equal(_host_bits(L), want_label)
    else:
        L = _dev(label, torch)
    out, toks = fas.decode_attention(q, K, V, L, ch, sl, k, scale=scale, tokens_out=True)
    torch.cuda.synchronize()
    return out.cpu().numpy(), toks.cpu().numpy()


def _check(inp, k, out, toks, label=None, scale=None):
    want, kept = ds.decode(inp.q, inp.key, inp.value, inp.channels, inp.seq_len, k, scale=scale, label=label)
    B, H, d = inp.q.shape
    worst = 0.0
    for b in range(B):
        for h in range(H):
            idx = kept[b][h]
            got = toks[b, h]
            assert np.array_equal(got[:len(idx)], idx), (b, h)
            assert np.all(got[len(idx):] == -1), (b, h)
            den = np.linalg.norm(want[b, h])
            err = np.linalg.norm(out[b, h] - want[b, h])
            if den == 0.0:
                assert err == 0.0, (b, h)
            else:
                worst = max(worst, err / den)
    assert worst <= TOL, worst
    return worst


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("r", [8, 16, 32])
@pytest.mark.parametrize("k", [1, 37, 300, 5000])
def test_decode_small_ragged(fas, d, r, k):
    print(f"[ds] small ragged d={d} r={r} k={k}", flush=True)
    c = wda.DecodeCase("t", 3, 4, d, 1000, r, k, ragged=True, seed=11)
    inp = wda.make_inputs(c)
    out, toks = _run(fas, inp, k)
    _check(inp, k, out, toks)


@pytest.mark.parametrize("kind", ["ties", "constant"])
def test_decode_tie_heavy_labels(fas, kind):
    # labels with few distinct values: the pivot bin holds far more than 64
    # keys, so the radix-select path with index tie-breaking decides
    print(f"[ds] ties {kind}", flush=True)
    c = wda.DecodeCase("t", 2, 3, 128, 3000, 16, 400, ragged=True, seed=12)
    inp = wda.make_inputs(c)
    g = np.random.default_rng(5)
    shape = (2, 3, 3000, 16)
    lab = g.integers(-2, 3, shape) if kind == "ties" else np.ones(shape)
    label = f32_to_bf16_bits(lab.astype(np.float32))
    out, toks = _run(fas, inp, 400, label=label)
    _check(inp, 400, out, toks, label=label)


def test_decode_single_token_and_empty(fas):
    print("[ds] single token / empty", flush=True)
    c = wda.DecodeCase("t", 3, 2, 128, 64, 8, 4, seed=13)
    inp = wda.make_inputs(c)
    inp.seq_len[:] = [1, 0, 64]
    out, toks = _run(fas, inp, 4)
    _check(inp, 4, out, toks)
    # one token: softmax weight 1, out is its value row exactly
    assert np.array_equal(out[0], ds.as_f64(inp.value[0, :, 0]).astype(np.float32))
    assert not out[1].any() and np.all(toks[1] == -1)


def test_decode_max_sequence(fas):
    # DS_MAX_SEQ tokens (the 32-slot register layout) and DS_MAX_K kept
    print("[ds] max sequence", flush=True)
    c = wda.DecodeCase("t", 1, 2, 128, 32768, 16, 8192, seed=14)
    inp = wda.make_inputs(c)
    inp.seq_len[:] = [32768]
    out, toks = _run(fas, inp, 8192)
    _check(inp, 8192, out, toks)
    out, toks = _run(fas, inp, 100)
    _check(inp, 100, out, toks)


@pytest.mark.parametrize("r", [8, 16, 32])
def test_decode_sixteen_slot_layout(fas, r):
    # 8192 < max_seq <= 16384: 16 scores per thread, two workgroups per CU
    print(f"[ds] 16-slot layout r={r}", flush=True)
    c = wda.DecodeCase("t", 2, 4, 128, 12000, r, 700, ragged=True, seed=21)
    inp = wda.make_inputs(c)
    inp.seq_len[0] = 12000
    out, toks = _run(fas, inp, 700)
    _check(inp, 700, out, toks)


def test_decode_clamped_lengths_and_wrapped_channels(fas):
    # documented error behaviour: lengths are clamped to [0, max_seq] and a
    # channel index outside [0, head_dim) is taken modulo head_dim
    import torch
    print("[ds] clamped lengths / wrapped channels", flush=True)
    c = wda.DecodeCase("t", 3, 2, 64, 200, 8, 30, seed=22)
    inp = wda.make_inputs(c)
    lens = np.array([500, -5, 150], np.int32)
    wrapped = inp.channels + 64 * np.array([[0, 1, 2, 0, 3, 0, 1, 0]], np.int32)
    q, K, V = _dev(inp.q, torch), _dev(inp.key, torch), _dev(inp.value, torch)
    L = torch.empty((3, 2, 200, 8), dtype=torch.bfloat16, device="cuda")
    chw = _dev(wrapped, torch)
    fas.label_cache_update(K, L, chw)
    out, toks = fas.decode_attention(q, K, V, L, chw, _dev(lens, torch), 30, tokens_out=True)
    torch.cuda.synchronize()
    inp.seq_len = np.clip(lens, 0, 200)
    _check(inp, 30, out.cpu().numpy(), toks.cpu().numpy())


@pytest.mark.parametrize("k", [999, 1000])
def test_decode_boundary_k(fas, k):
    # n = 1000 for every sequence: k = n - 1 drops exactly one token (the
    # smallest score, ties to the highest index); k = n is the dense path
    print(f"[ds] boundary k={k}", flush=True)
    c = wda.DecodeCase("t", 2, 4, 128, 1000, 16, k, seed=24)
    inp = wda.make_inputs(c)
    out, toks = _run(fas, inp, k)
    _check(inp, k, out, toks)


def test_label_cache_append(fas):
    # decode-style update: one token per sequence at a ragged position
    import torch
    print("[ds] label append", flush=True)
    c = wda.DecodeCase("t", 4, 3, 64, 500, 16, 10, seed=15)
    inp = wda.make_inputs(c)
    K = _dev(inp.key, torch)
    ch = _dev(inp.channels.astype(np.int32), torch)
    L = torch.zeros((4, 3, 500, 16), dtype=torch.bfloat16, device="cuda")
    pos = np.array([0, 17, 498, 499], np.int32)
    fas.label_cache_update(K, L, ch, start=_dev(pos, torch), span=2)
    torch.cuda.synchronize()
    got = _host_bits(L)
    want = ds.label_cache(inp.key, inp.channels)
    mask = np.zeros((4, 500), bool)
    for b, p in enumerate(pos):
        mask[b, p:min(p + 2, 500)] = True
    for b in range(4):
        assert np.array_equal(got[b][:, mask[b]], want[b][:, mask[b]])
        assert not got[b][:, ~mask[b]].any()


def test_decode_deterministic_and_graph_replay(fas):
    import torch
    print("[ds] determinism + graph", flush=True)
    c = wda.DecodeCase("t", 4, 8, 128, 2048, 16, 128, ragged=True, seed=16)
    inp = wda.make_inputs(c)
    q, K, V = _dev(inp.q, torch), _dev(inp.key, torch), _dev(inp.value, torch)
    ch, sl = _dev(inp.channels.astype(np.int32), torch), _dev(inp.seq_len.astype(np.int32), torch)
    L = torch.empty((4, 8, 2048, 16), dtype=torch.bfloat16, device="cuda")
    fas.label_cache_update(K, L, ch)
    ref = fas.decode_attention(q, K, V, L, ch, sl, 128)
    again = fas.decode_attention(q, K, V, L, ch, sl, 128)
    torch.cuda.synchronize()
    assert torch.equal(ref, again)
    out = torch.zeros_like(ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        fas.decode_attention(q, K, V, L, ch, sl, 128, out=out)  # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            fas.decode_attention(q, K, V, L, ch, sl, 128, out=out)
    for i in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), i


@pytest.mark.parametrize("name", sorted(wda.CASES))
def test_decode_full_size(fas, name):
    # the benchmark's Llama-2-7B decode batch: every (sequence, head) checked
    print(f"[ds] full size {name}", flush=True)
    c = wda.CASES[name]
    inp = wda.make_inputs(c)
    out, toks = _run(fas, inp, c.k, check_label=True)
    worst = _check(inp, c.k, out, toks)
    print(f"[ds] {name}: worst rel L2 {worst:.3e}", flush=True)


def test_bad_arguments_leave_outputs(fas):
    import torch
    c = wda.DecodeCase("t", 1, 2, 128, 64, 16, 8, seed=17)
    inp = wda.make_inputs(c)
    q, K, V = _dev(inp.q, torch), _dev(inp.key, torch), _dev(inp.value, torch)
    ch, sl = _dev(inp.channels.astype(np.int32), torch), _dev(inp.seq_len.astype(np.int32), torch)
    L = torch.empty((1, 2, 64, 16), dtype=torch.bfloat16, device="cuda")
    out = torch.full((1, 2, 128), 7.0, device="cuda")
    with pytest.raises(fas.SparseLinearError):
        fas.ds_decode_attention(q.data_ptr(), K.data_ptr(), V.data_ptr(), L.data_ptr() + 2, ch.data_ptr(),
                                sl.data_ptr(), 1, 2, 64, 128, 16, 8, 0.1, out.data_ptr())
    with pytest.raises(fas.SparseLinearError):
        fas.ds_decode_attention(q.data_ptr(), K.data_ptr(), V.data_ptr(), L.data_ptr(), ch.data_ptr(),
                                sl.data_ptr(), 1, 2, 64, 96, 16, 8, 0.1, out.data_ptr())
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
