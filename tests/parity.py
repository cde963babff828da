"""Shared comparison rules for GPU-vs-oracle parity tests (test infrastructure).

Rule (stated for this router): for every token whose oracle gap between the
k-th and (k+1)-th logit exceeds 1e-3 * max_j |l_j|, the selected index sets
must be identical; gate weights, compared by rank position after both sides
are sorted by (logit desc, index asc), must agree within 1e-3 absolute for
every token.  Extra checks: the returned logits match the oracle's within a
bound derived from fp32 accumulation of ~2^-17-accurate bf16 hi+lo products,
and in full-softmax mode the probabilities and log-sum-exp are checked
relative to their size (at large M every probability is far below 1e-3).
"""
from __future__ import annotations

import numpy as np

GAP_REL = 1e-3
GATE_ABS = 1e-3


def gap_clear(ora: dict) -> np.ndarray:
    return (ora["kth"] - ora["kp1"]) > GAP_REL * ora["maxabs"]


def compare(ora: dict, gpu: dict, k: int, full: bool, logit_tol: float = 2e-4, label: str = "") -> dict:
    """Assert the parity rule; return counts for reporting."""
    idx_g = gpu["idx"]
    gate_g = gpu["gate"]
    N = idx_g.shape[0]
    assert idx_g.shape == (N, k) and gate_g.shape == (N, k)
    clear = gap_clear(ora)
    # index sets on gap-clear tokens
    so = np.sort(ora["idx"], axis=1)
    sg = np.sort(idx_g, axis=1)
    bad_set = np.nonzero(clear & np.any(so != sg, axis=1))[0]
    assert bad_set.size == 0, (f"{label}: {bad_set.size} gap-clear tokens select different experts; "
                               f"first {bad_set[:5]} oracle {ora['idx'][bad_set[:2]]} gpu {idx_g[bad_set[:2]]}")
    # every returned index is a valid expert, without repeats
    assert np.all(idx_g >= 0)
    assert np.all(np.diff(np.sort(idx_g, axis=1), axis=1) != 0), f"{label}: repeated expert in a row"
    # gates by rank position, all tokens
    gerr = np.abs(gate_g.astype(np.float64) - ora["gate"])
    assert np.max(gerr) <= GATE_ABS, f"{label}: max gate error {np.max(gerr):.3g}"
    # logits by rank position
    if gpu.get("logit") is not None:
        lerr = np.abs(gpu["logit"].astype(np.float64) - ora["logit"])
        scale = np.maximum(1.0, ora["maxabs"])[:, None]
        assert np.max(lerr / scale) <= logit_tol, f"{label}: max logit error {np.max(lerr / scale):.3g}"
        # output order: logits non-increasing
        assert np.all(np.diff(gpu["logit"], axis=1) <= 0), f"{label}: output not sorted by logit"
    if full:
        p_o = ora["gate"]
        p_g = gate_g.astype(np.float64)
        assert np.all(np.abs(p_g - p_o) <= 1e-3 * p_o + 1e-7), f"{label}: full-softmax probability off"
        if gpu.get("lse") is not None:
            lerr = np.abs(gpu["lse"].astype(np.float64) - ora["lse"])
            assert np.all(lerr <= 1e-4 * np.maximum(1.0, np.abs(ora["lse"]))), f"{label}: lse off"
    else:
        assert np.allclose(gate_g.sum(1), 1.0, atol=1e-5)
    return dict(tokens=int(N), gap_clear=int(clear.sum()), excluded=int((~clear).sum()))
