"""Write the stored oracle outputs under tests/golden/ (calls only oracle/).

The paper ("MoRE: Scaling mixture of experts with hardware-aware low-rank
routing") prints no worked router example, so these files are regression
anchors written by the fp64 oracle on seeded synthetic inputs, not values from
the paper.  Run:  python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from rank_router_top_amd import configs as CF  # noqa: E402


def digest(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        if a is not None:
            h.update(a.tobytes())
    return h.hexdigest()


def main():
    oracle.build(force=False)
    cfg = CF.TINY
    X = cfg.x_rows(0)
    R1, R2, b = cfg.weights(0)
    out = oracle.route_lowrank(X, R1, R2, b, cfg.k, oracle.GATE_TOPK, nthreads=1)
    doc = {
        "what": "fp64 oracle on the tiny fp32 low-rank router workload, seed 0",
        "config": {"N": cfg.N, "h": cfg.h, "M": cfg.M, "r": cfg.r, "k": cfg.k, "dtype": cfg.dtype,
                   "gate": "topk_softmax"},
        "input_sha256": digest(X, R1, R2, b),
        "idx": out["idx"].tolist(),
        "gate": [[float(v) for v in row] for row in out["gate"]],
        "logit": [[float(v) for v in row] for row in out["logit"]],
    }
    with open(os.path.join(HERE, "tiny_f32_seed0.json"), "w") as f:
        json.dump(doc, f)
        f.write("\n")


if __name__ == "__main__":
    main()
