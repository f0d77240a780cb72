"""Seeded synthetic inputs for the sparse-linear workloads.

This module draws random numbers and rounds them to the storage dtypes; it
holds none of the method's arithmetic (no norms, scores, selection or
products). Both the CPU oracle (``oracle/``) and the HIP path's tests and
benchmark take their inputs from here, so the two sides see identical bits.

Every draw comes from ``numpy.random.default_rng(SeedSequence([config,
linear, role, index]))`` with ``role`` 0 for a weight matrix, 1 for an input
token and 2 for a per-component sparsity draw, and ``index`` the token number
(0 for weights and sparsity draws).

Shapes are those of the decoder layers the pages name (Llama-2-7B, Llama-3-8B,
Phi-4-14B, Qwen-2.5-7B linears); the pages' real activations come from
Alpaca-calibrated models that are not available, so the distributions below
stand in for them (see the workload table in each ``CONFIGS`` entry).
"""
from __future__ import annotations

import dataclasses
from fractions import Fraction
from typing import Dict, List, Optional, Tuple

import numpy as np

ROLE_W, ROLE_X, ROLE_P = 0, 1, 2


def rng(config: int, linear: int, role: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([config, linear, role, index]))


# --------------------------------------------------------------------------
# bf16 storage (round-to-nearest-even from fp32); arrays are numpy uint16 bits
# --------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (RNE) and return the 16-bit patterns.

    Finite inputs only (the generators never produce NaN/Inf)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# Workload descriptions
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Linear:
    name: str
    m: int          # output rows
    n: int          # input columns
    x_kind: str     # 'normal' | 'silu_gu' | 'laplace'


@dataclasses.dataclass(frozen=True)
class Config:
    cid: int
    name: str
    dtype: str                      # 'f32' | 'bf16' (weights and inputs)
    w_std: float
    linears: Tuple[Linear, ...]
    tokens: int
    gate: str                       # 'topk' | 'stat'
    sparsities: Tuple[float, ...] = ()   # fraction dropped (TOPK)
    s_keep: Optional[float] = None       # keep fraction (STAT)
    batches: Tuple[int, ...] = (1,)
    sparsity_range: Optional[Tuple[float, float]] = None  # per-component draw


CONFIGS: Dict[int, Config] = {
    1: Config(1, "tiny_512x256_f32", "f32", 1.0 / 16.0,
              (Linear("tiny", 512, 256, "normal"),), 64, "topk", sparsities=(0.5,)),
    2: Config(2, "llama7b_down_4096x11008_bf16", "bf16", 0.02,
              (Linear("down", 4096, 11008, "silu_gu"),), 256, "topk",
              sparsities=(0.5, 0.65)),
    3: Config(3, "llama3_8b_block_bf16", "bf16", 0.02,
              (Linear("q", 4096, 4096, "normal"),
               Linear("k", 1024, 4096, "normal"),
               Linear("v", 1024, 4096, "normal"),
               Linear("o", 4096, 4096, "normal"),
               Linear("gate", 14336, 4096, "normal"),
               Linear("up", 14336, 4096, "normal"),
               Linear("down", 4096, 14336, "silu_gu")), 256, "topk",
              sparsity_range=(0.3, 0.7)),
    4: Config(4, "phi4_ffn_stat_bf16", "bf16", 0.02,
              (Linear("gate", 17920, 5120, "laplace"),
               Linear("up", 17920, 5120, "laplace"),
               Linear("down", 5120, 17920, "laplace")), 256, "stat",
              s_keep=0.10, batches=(1, 2, 4, 8)),
    5: Config(5, "qwen25_7b_ffn_b16_bf16", "bf16", 0.02,
              (Linear("gate", 18944, 3584, "normal"),
               Linear("up", 18944, 3584, "normal"),
               Linear("down", 3584, 18944, "normal")), 256, "topk",
              sparsities=(0.65, 0.90), batches=(16,)),
}

# In config 3 the q, k, v, gate and up projections read the same hidden state;
# o reads the attention output and down reads the SiLU(g)*u intermediate.
_SHARED_INPUT_GROUP = {"q": 0, "k": 0, "v": 0, "gate": 0, "up": 0, "o": 1, "down": 2}


def k_from_sparsity(n: int, p: float) -> int:
    """Number of kept inputs for a dropped fraction p: K = n - floor(p*n),
    with p taken as the exact decimal it is written as."""
    return n - int(Fraction(str(p)) * n // 1)


def component_sparsities(config: int = 3) -> List[float]:
    """Seeded per-component dropped fractions, one U[lo, hi) draw per linear in
    the config's order (a WAS-style heterogeneous schedule)."""
    cfg = CONFIGS[config]
    lo, hi = cfg.sparsity_range
    out = []
    for li, _ in enumerate(cfg.linears):
        g = rng(config, li, ROLE_P, 0)
        out.append(float(lo + (hi - lo) * g.random()))
    return out


# --------------------------------------------------------------------------
# Draws
# --------------------------------------------------------------------------
def weight(config: int, linear: int, m: Optional[int] = None, n: Optional[int] = None) -> np.ndarray:
    """Weight matrix in the nn.Linear layout [m][n] (row i = output i).

    Returns float32 for fp32 configs and uint16 bf16 bits otherwise. ``m``/``n``
    override the config shape (used for scaled-down parity cases)."""
    cfg = CONFIGS[config]
    lin = cfg.linears[linear]
    m = lin.m if m is None else m
    n = lin.n if n is None else n
    g = rng(config, linear, ROLE_W, 0)
    w = g.standard_normal((m, n), dtype=np.float32)
    w *= np.float32(cfg.w_std)
    if cfg.dtype == "f32":
        return w
    return f32_to_bf16_bits(w)


def token(config: int, linear: int, index: int, n: Optional[int] = None) -> np.ndarray:
    """One input token x[n]: float32 for fp32 configs, bf16 bits otherwise."""
    cfg = CONFIGS[config]
    lin = cfg.linears[linear]
    n = lin.n if n is None else n
    group = _SHARED_INPUT_GROUP.get(lin.name, linear) if config == 3 else linear
    g = rng(config, group, ROLE_X, index)
    if lin.x_kind == "normal":
        x = g.standard_normal(n, dtype=np.float32)
    elif lin.x_kind == "laplace":
        x = g.laplace(0.0, 1.0, n).astype(np.float32)
    elif lin.x_kind == "silu_gu":
        gg = g.standard_normal(n)
        uu = g.standard_normal(n)
        x = (gg / (1.0 + np.exp(-gg)) * uu).astype(np.float32)
    else:
        raise ValueError(lin.x_kind)
    if cfg.dtype == "f32":
        return x
    return f32_to_bf16_bits(x)


def tokens(config: int, linear: int, first: int, count: int, n: Optional[int] = None) -> np.ndarray:
    """``count`` consecutive tokens stacked as [count][n]."""
    return np.stack([token(config, linear, first + i, n) for i in range(count)])


def random_matrix(seed: int, m: int, n: int, dtype: str, std: float = 0.02) -> np.ndarray:
    """Free-form seeded matrix for edge-case tests (ragged shapes)."""
    g = np.random.default_rng(np.random.SeedSequence([1000, seed, ROLE_W, 0]))
    w = g.standard_normal((m, n), dtype=np.float32) * np.float32(std)
    return w if dtype == "f32" else f32_to_bf16_bits(w)


def random_tokens(seed: int, count: int, n: int, dtype: str, kind: str = "normal") -> np.ndarray:
    """Free-form seeded tokens for edge-case tests."""
    out = []
    for i in range(count):
        g = np.random.default_rng(np.random.SeedSequence([1000, seed, ROLE_X, i]))
        if kind == "normal":
            x = g.standard_normal(n, dtype=np.float32)
        elif kind == "laplace":
            x = g.laplace(0.0, 1.0, n).astype(np.float32)
        elif kind == "ties":
            # few distinct magnitudes, many exact ties, signed, some zeros
            x = (g.integers(-3, 4, n)).astype(np.float32)
        else:
            raise ValueError(kind)
        out.append(x if dtype == "f32" else f32_to_bf16_bits(x))
    return np.stack(out)
