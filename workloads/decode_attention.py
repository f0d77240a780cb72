"""Seeded synthetic inputs for the Double Sparsity decode-attention workload.

Random draws and bf16 rounding only: no scores, no selection, no attention.
The CPU oracle and the HIP path's tests and benchmark both take their inputs
from here.

Shapes are Llama-2-7B's attention (32 heads of 128 channels, multi-head, one
key/value head per query head). The pages' models and their offline
calibration are not available, so the cache is drawn with the structure the
calibration finds: a few outlier channels per head carry most of q.k. Per head
h a seeded permutation ``order[h]`` of the channels is drawn; its first
``heavy`` entries are the outlier channels, scaled by ``outlier_scale`` in both
q and the keys. The channel list handed to the method for r label channels is
``order[h][:r]``: the outlier channels first, then the next channels of the
permutation (the stand-in for the calibration's channel file).

Every draw comes from ``numpy.random.default_rng(SeedSequence([2000, seed,
role, b]))`` with role 0 for the channel permutations, 1 for keys, 2 for
values, 3 for queries and 4 for sequence lengths.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from . import f32_to_bf16_bits

ROLE_ORDER, ROLE_K, ROLE_V, ROLE_Q, ROLE_LEN = 0, 1, 2, 3, 4


def _rng(seed: int, role: int, b: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([2000, seed, role, b]))


@dataclasses.dataclass(frozen=True)
class DecodeCase:
    """One decode step of one attention layer over a key/value cache."""
    name: str
    batch: int
    heads: int
    head_dim: int
    max_seq: int
    r: int                 # label channels per head
    k: int                 # heavy tokens kept per sequence and head
    ragged: bool = False   # sequence lengths drawn in [1, max_seq] instead of all max_seq
    heavy: int = 8         # outlier channels per head in the synthetic cache
    outlier_scale: float = 4.0
    seed: int = 0


# The pages' headline setting keeps 1/16 of the tokens and 1/16 of the channels
# (Double Sparsity article, introduction); the SGLang example runs 8192-token
# prompts with 16 label channels and 256 heavy tokens (section on SGLang).
CASES = {
    "llama2_7b_b16_s8192_r8_k512": DecodeCase("llama2_7b_b16_s8192_r8_k512", 16, 32, 128, 8192, 8, 512),
    "llama2_7b_b16_s8192_r16_k256": DecodeCase("llama2_7b_b16_s8192_r16_k256", 16, 32, 128, 8192, 16, 256),
}


@dataclasses.dataclass
class DecodeInputs:
    q: np.ndarray          # [B][H][d] bf16 bits
    key: np.ndarray        # [B][H][S][d] bf16 bits
    value: np.ndarray      # [B][H][S][d] bf16 bits
    channels: np.ndarray   # [H][r] int32
    seq_len: np.ndarray    # [B] int32


def channel_order(case: DecodeCase) -> np.ndarray:
    """[H][d] int32: per head, a seeded permutation of the channels."""
    g = _rng(case.seed, ROLE_ORDER)
    return np.stack([g.permutation(case.head_dim) for _ in range(case.heads)]).astype(np.int32)


def make_inputs(case: DecodeCase, batch: Optional[int] = None) -> DecodeInputs:
    """Draw q, the key and value caches, the channel list and the lengths.

    Sequence b's draws depend only on (seed, b), so a smaller ``batch`` gives
    the first sequences of the full case."""
    B = case.batch if batch is None else batch
    H, d, S = case.heads, case.head_dim, case.max_seq
    order = channel_order(case)
    scale = np.ones((H, d), np.float32)
    for h in range(H):
        scale[h, order[h, :case.heavy]] = np.float32(case.outlier_scale)
    key = np.empty((B, H, S, d), np.uint16)
    value = np.empty((B, H, S, d), np.uint16)
    q = np.empty((B, H, d), np.uint16)
    lens = np.empty(B, np.int32)
    for b in range(B):
        kb = _rng(case.seed, ROLE_K, b).standard_normal((H, S, d), dtype=np.float32)
        kb *= scale[:, None, :]
        key[b] = f32_to_bf16_bits(kb)
        value[b] = f32_to_bf16_bits(_rng(case.seed, ROLE_V, b).standard_normal((H, S, d), dtype=np.float32))
        qb = _rng(case.seed, ROLE_Q, b).standard_normal((H, d), dtype=np.float32) * scale
        q[b] = f32_to_bf16_bits(qb)
        lens[b] = int(_rng(case.seed, ROLE_LEN, b).integers(1, S + 1)) if case.ragged else S
    return DecodeInputs(q, key, value, np.ascontiguousarray(order[:, :case.r]), lens)
