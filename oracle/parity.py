"""The comparison rule between a GPU routing result and the fp64 oracle
(TEST INFRASTRUCTURE, like the rest of this package).

Rule stated for this router:
  * for every token whose oracle gap between the k-th and (k+1)-th logit
    exceeds 1e-3 * max_j |l_j| (per token, over all M logits, bias included),
    the selected index sets must be identical;
  * gate weights, compared by rank position after both sides are sorted by
    (logit desc, index asc), must agree within 1e-3 absolute for every token.
Checks that tie every returned index to its own numbers, on every token
(``at`` = the oracle's fp64 logits at the GPU's own indices, from
``oracle.logits_at``):
  * every index lies in [0, M) and no expert repeats in a row;
  * every selected expert is a valid member of a top-k up to the tolerance:
    l[n, idx[n, j]] >= l_(k) - tol, so a token the gap rule excuses may swap
    only near-equal experts;
  * the returned logit of slot j is the oracle's logit of expert idx[n, j]
    within tol = logit_tol * max(1, max|l|), and the logits are non-increasing;
  * the gate of slot j is the gate of expert idx[n, j]: the softmax over the
    oracle logits of the GPU's own k experts (Fig. 12) within 1e-3, or in the
    full-softmax mode exp(l[n, idx[n, j]] - lse) within 1e-3 relative.
In the full-softmax mode the probabilities and the log-sum-exp are also
checked relative to their size (at large M every probability is far below
1e-3, so the absolute rule alone would say little).
"""
from __future__ import annotations

import numpy as np

GAP_REL = 1e-3
GATE_ABS = 1e-3


def gap_clear(ora: dict) -> np.ndarray:
    return (ora["kth"] - ora["kp1"]) > GAP_REL * ora["maxabs"]


def mismatches(ora: dict, gpu_idx: np.ndarray) -> int:
    """Gap-clear tokens whose selected set differs from the oracle's."""
    clear = gap_clear(ora)
    so = np.sort(ora["idx"], axis=1)
    sg = np.sort(gpu_idx, axis=1)
    return int(np.count_nonzero(clear & np.any(so != sg, axis=1)))


def compare(ora: dict, gpu: dict, k: int, full: bool, logit_tol: float, label: str, at: np.ndarray) -> dict:
    """Assert the rule for the rows of `gpu` against `ora` (same rows); return counts.

    at: the oracle's fp64 logits at the GPU's indices, at[n, j] = l[n, gpu idx[n, j]]
    (NaN for an index outside [0, M))."""
    idx_g = gpu["idx"]
    gate_g = gpu["gate"].astype(np.float64)
    N = idx_g.shape[0]
    assert idx_g.shape == (N, k) and gate_g.shape == (N, k), f"{label}: output shape"
    assert at.shape == (N, k), f"{label}: logits-at shape"
    # every index is an expert (logits_at gives NaN outside [0, M)), no repeats
    bad_range = np.nonzero(~np.all(np.isfinite(at), axis=1))[0]
    assert bad_range.size == 0, f"{label}: {bad_range.size} tokens with an index outside [0, M); first {bad_range[:5]}"
    assert np.all(np.diff(np.sort(idx_g, axis=1), axis=1) != 0), f"{label}: repeated expert in a row"
    clear = gap_clear(ora)
    # index sets on gap-clear tokens
    so = np.sort(ora["idx"], axis=1)
    sg = np.sort(idx_g, axis=1)
    bad_set = np.nonzero(clear & np.any(so != sg, axis=1))[0]
    assert bad_set.size == 0, (f"{label}: {bad_set.size} gap-clear tokens select different experts; "
                               f"first {bad_set[:5]} oracle {ora['idx'][bad_set[:2]]} gpu {idx_g[bad_set[:2]]}")
    tol = logit_tol * np.maximum(1.0, ora["maxabs"])
    # every token: each selected expert is within tol of the top-k boundary
    short = at - (ora["kth"] - tol)[:, None]
    bad_sel = np.nonzero(np.any(short < 0, axis=1))[0]
    assert bad_sel.size == 0, (f"{label}: {bad_sel.size} tokens select an expert below the k-th logit by more "
                               f"than the tolerance; first {bad_sel[:5]}")
    # gates by rank position, all tokens
    gerr = np.abs(gate_g - ora["gate"])
    assert np.max(gerr) <= GATE_ABS, f"{label}: max gate error {np.max(gerr):.3g}"
    # logits: slot j carries the logit of expert idx[n, j]; by rank position too
    if gpu.get("logit") is not None:
        lg = gpu["logit"].astype(np.float64)
        perr = np.abs(lg - at) / tol[:, None]
        assert np.max(perr) <= 1.0, (f"{label}: a returned logit differs from the oracle logit of its own "
                                     f"expert by {np.max(perr):.3g} x tol")
        rerr = np.abs(lg - ora["logit"]) / tol[:, None]
        assert np.max(rerr) <= 1.0, f"{label}: max logit error by rank {np.max(rerr):.3g} x tol"
        assert np.all(np.diff(gpu["logit"], axis=1) <= 0), f"{label}: output not sorted by logit"
    # gates: slot j carries the gate of expert idx[n, j]
    if full:
        lse_o = ora["lse"]
        expect = np.exp(at - lse_o[:, None])
        assert np.all(np.abs(gate_g - expect) <= 1e-3 * expect + 1e-7), \
            f"{label}: full-softmax probability of a slot's own expert off"
        p_o = ora["gate"]
        assert np.all(np.abs(gate_g - p_o) <= 1e-3 * p_o + 1e-7), f"{label}: full-softmax probability off"
        if gpu.get("lse") is not None:
            lerr = np.abs(gpu["lse"].astype(np.float64) - lse_o)
            assert np.all(lerr <= 1e-4 * np.maximum(1.0, np.abs(lse_o))), f"{label}: lse off"
    else:
        e = np.exp(at - at.max(axis=1, keepdims=True))
        expect = e / e.sum(axis=1, keepdims=True)
        perr = np.abs(gate_g - expect)
        assert np.max(perr) <= GATE_ABS, (f"{label}: a gate differs from the softmax over its own experts' "
                                          f"logits by {np.max(perr):.3g}")
        assert np.allclose(gate_g.sum(1), 1.0, atol=1e-5), f"{label}: gates do not sum to 1"
    return dict(tokens=int(N), gap_clear=int(clear.sum()), excluded=int((~clear).sum()))


def properties(gpu: dict, k: int, M: int, full: bool, label: str) -> None:
    """Checks that hold for every row at any size, without the oracle: indices
    in [0, M) without repeats, logits non-increasing, and the gates those
    logits imply (Fig. 12 softmax over the k returned logits, or
    exp(l - lse) of eq. (6) with lse >= the largest returned logit)."""
    idx = gpu["idx"]
    N = idx.shape[0]
    assert idx.shape == (N, k), f"{label}: index shape"
    assert np.all((idx >= 0) & (idx < M)), f"{label}: index outside [0, M)"
    assert np.all(np.diff(np.sort(idx, axis=1), axis=1) != 0), f"{label}: repeated expert in a row"
    gate = gpu["gate"].astype(np.float64)
    assert np.all(np.isfinite(gate)) and np.all(gate > 0), f"{label}: gate not positive and finite"
    lg = gpu.get("logit")
    if lg is None:
        return
    lg = lg.astype(np.float64)
    assert np.all(np.isfinite(lg)), f"{label}: non-finite logit"
    assert np.all(np.diff(lg, axis=1) <= 0), f"{label}: logits not non-increasing"
    if full:
        lse = gpu["lse"].astype(np.float64)
        assert np.all(lse >= lg[:, 0] - 1e-5 * np.maximum(1.0, np.abs(lse))), f"{label}: lse below a logit"
        expect = np.exp(lg - lse[:, None])
        assert np.all(np.abs(gate - expect) <= 1e-4 * expect + 1e-9), f"{label}: gate != exp(logit - lse)"
    else:
        e = np.exp(lg - lg[:, :1])
        expect = e / e.sum(axis=1, keepdims=True)
        assert np.max(np.abs(gate - expect)) <= 1e-5, f"{label}: gate != softmax of the returned logits"
        assert np.allclose(gate.sum(1), 1.0, atol=1e-5), f"{label}: gates do not sum to 1"
