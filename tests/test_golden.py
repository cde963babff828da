"""Regression anchors: stored oracle outputs (written by tests/golden/make_golden.py)."""
import hashlib
import json
import os

import numpy as np

from rank_router_top_amd import configs as CF

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_f32_seed0.json")


def _digest(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        if a is not None:
            h.update(a.tobytes())
    return h.hexdigest()


def test_tiny_inputs_and_oracle_unchanged(oracle_lib):
    doc = json.load(open(GOLDEN))
    cfg = CF.TINY
    X = cfg.x_rows(0)
    R1, R2, b = cfg.weights(0)
    assert _digest(X, R1, R2, b) == doc["input_sha256"]
    out = oracle_lib.route_lowrank(X, R1, R2, b, cfg.k, oracle_lib.GATE_TOPK)
    assert np.array_equal(out["idx"], np.array(doc["idx"], np.int32))
    assert np.allclose(out["gate"], np.array(doc["gate"]), rtol=0, atol=1e-15)
    assert np.allclose(out["logit"], np.array(doc["logit"]), rtol=0, atol=1e-14)
