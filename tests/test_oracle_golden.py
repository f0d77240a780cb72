"""The oracle reproduces its stored outputs for the tiny config (a drift guard;
the stored values were written by tests/golden/make_golden.py from oracle/)."""
import json
import os

import numpy as np

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_topk_oracle.json")


def test_oracle_matches_stored_tiny():
    doc = json.load(open(GOLDEN))
    W = wl.weight(1, 0)
    c = oracle.column_norms(W)
    assert [float.fromhex(h) for h in doc["c_hex"]] == c.astype(np.float64).tolist()
    for case in doc["cases"]:
        out = oracle.forward(W, c, wl.token(1, 0, case["token"]), "topk", K=doc["K"])
        assert out["idx"].tolist() == case["idx"]
        assert out["thresh"] == float.fromhex(case["thresh"])
        assert out["y"].tolist() == [float.fromhex(h) for h in case["y_hex"]]
