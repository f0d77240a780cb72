"""Writes the stored expected values under tests/golden/ from the CPU oracle.

Calls only ``oracle`` (and ``workloads`` for the seeded inputs). Run from the
repository root: ``python tests/golden/make_golden.py``.
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads as wl  # noqa: E402


def main():
    W = wl.weight(1, 0)
    c = oracle.column_norms(W)
    K = wl.k_from_sparsity(256, 0.5)
    cases = []
    for t in range(4):
        x = wl.token(1, 0, t)
        out = oracle.forward(W, c, x, "topk", K=K)
        cases.append({
            "token": t,
            "idx": out["idx"].tolist(),
            "thresh": out["thresh"].hex() if hasattr(out["thresh"], "hex") else float(out["thresh"]).hex(),
            "y_hex": [float(v).hex() for v in out["y"]],
        })
    doc = {
        "what": "tiny 512x256 fp32 linear, WINA top-K K=128, tokens 0-3 (seeded), oracle outputs",
        "c_hex": [float(v).hex() for v in c.astype(np.float64)],
        "K": K,
        "cases": cases,
    }
    with open(os.path.join(HERE, "tiny_topk_oracle.json"), "w") as f:
        json.dump(doc, f, indent=0)
        f.write("\n")


if __name__ == "__main__":
    main()
