"""Plain fp64 reference of the sparse FFN chain (one token).

TEST INFRASTRUCTURE ONLY: the product path never imports, calls or links
anything here; only tests, the smoke check and the benchmark's CPU leg do. It
shares no code with the HIP library.

Definitions followed (pages cited by title and section):

* ``silu`` -- the SwiGLU FFN of the Llama models whose layer shapes the
  workloads use: SiLU(v) = v / (1 + e^(-v)). The Spark Transformer article,
  section 2.1, describes the FFN as score -> select -> compute over the
  intermediate; it does not print the activation, so this is a reading.
* ``bf16_round`` -- one rounding of a real value (held in fp64) to the
  nearest bfloat16 (8 significant bits, fp32's exponent range, gradual
  underflow down to 2^-133), ties to the even significand; values at or past
  the rounding midpoint above the largest finite bf16 become infinity.
* ``silu_mul`` -- the FFN's intermediate h = bf16(SiLU(g) * u): the product is
  formed in fp64 and rounded once to bf16, the down projection's input dtype.
* ``ffn_chain`` -- g = gate(x), u = up(x), each the sparse linear of
  ``oracle.sparse_linear.forward`` with its own gate (WINA article, section
  一: every projection keeps its inputs by |x_j c_j|); h = silu_mul(g, u);
  y = down(h) with the down projection's own gate on h.

Parity pins (tests/test_oracle_ffn.py): SiLU(0) = 0, its large-|v| limits,
the exact odd-part identity SiLU(v) - SiLU(-v) = v, agreement with scipy's
logistic function; bf16 rounding at hand-built halfway cases (ties to even,
both signs, the subnormal range, overflow) and the nearest-value property on
random inputs; the chain's wiring with diagonal weights, where each stage
reduces to scalar arithmetic on one input.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .sparse_linear import forward

_BF16_MIN_EXP = -133          # quantum of the bf16 subnormals: 2^-133
_BF16_OVERFLOW = 2.0 ** 128   # the first value past the largest finite bf16


def silu(v: np.ndarray) -> np.ndarray:
    """SiLU(v) = v / (1 + exp(-v)) in fp64 (exp overflows to inf for very
    negative v, giving -0)."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def bf16_round(v: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 to each fp64 value (ties to even), as uint16 bit
    patterns. The significand keeps 8 bits: for |v| in [2^(e-1), 2^e) the
    quantum is 2^(e-8), but never below the subnormal quantum 2^-133."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.float64)
    flat_v, flat_o = v.reshape(-1), out.reshape(-1)
    for i, a in enumerate(flat_v.tolist()):
        if a != a:  # NaN stays NaN
            flat_o[i] = a
            continue
        mag = abs(a)
        if mag == 0.0 or mag == float("inf"):
            flat_o[i] = a
            continue
        _, e = np.frexp(mag)               # mag = f * 2^e, f in [0.5, 1)
        qexp = max(int(e) - 8, _BF16_MIN_EXP)
        q = float(np.ldexp(1.0, qexp))
        r = float(np.rint(mag / q)) * q    # rint: round half to even
        if r >= _BF16_OVERFLOW:
            r = float("inf")
        flat_o[i] = -r if a < 0 or (a == 0.0 and np.signbit(a)) else r
    bits = out.astype(np.float32).view(np.uint32)  # bf16 values are exact in fp32
    return (bits >> 16).astype(np.uint16)


def silu_mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """h = bf16(SiLU(g) * u) with one rounding; g and u are real values (fp32
    or fp64 arrays); returns bf16 bit patterns."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    return bf16_round(silu(g) * u)


def ffn_chain(Wg: np.ndarray, cg: np.ndarray, gate_kw: dict, Wu: np.ndarray, cu: np.ndarray, up_kw: dict,
              Wd: np.ndarray, cd: np.ndarray, down_kw: dict, x: np.ndarray,
              rows: Optional[np.ndarray] = None) -> Dict[str, object]:
    """The sparse FFN chain for one token x (W in the [m][n] layout, bf16 bit
    patterns or fp32). Each *_kw holds the gate of that projection: mode
    ('topk', 'stat', 'fixed') and its K, s_keep or tau. ``rows`` limits the
    down projection's product to sampled output rows."""
    def kw(d):
        d = dict(d)
        return d.pop("mode"), d
    mg, kg = kw(gate_kw)
    mu, ku = kw(up_kw)
    md, kd = kw(down_kw)
    g = forward(Wg, cg, x, mg, **kg)
    u = forward(Wu, cu, x, mu, **ku)
    h = silu_mul(g["y"], u["y"])
    d = forward(Wd, cd, h, md, rows=rows, **kd)
    return {"g": g["y"], "u": u["y"], "h": h, "y": d["y"], "down": d, "gate": g, "up": u}
