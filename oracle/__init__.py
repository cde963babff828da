"""fp64 CPU oracle for the fused low-rank MoE router -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP product path never imports,
calls or links anything here.

Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank routing",
§2 (standard and low-rank router), App. F eq. (5) (logits), App. F.1
Algorithm 1 and Fig. 12 (exact top-k, softmax over the k selected logits),
App. F.2.1 eq. (6) (full softmax / log-sum-exp), eq. (7) and (9) (column sums
of the full softmax and the Switch balancing loss), App. G.1 (normalised
routing entropy), App. F.2.2 eq. (10)-(12) and Algorithm 3 (the backward
pass), App. E Fig. 9 (expert dispatch: sort + count).  The router
arithmetic lives in ``more_oracle.c`` (plain C, fp64, OpenMP over tokens),
which this package builds with gcc and calls through ctypes; the balancing
statistics' final formulas and the dispatch sort are plain numpy in
``oracle.py``.
"""
from .oracle import (DT_BF16, DT_F32, DT_F64, GATE_FULL, GATE_TOPK, backward_lowrank, balance_lowrank,
                     balance_stats, build, dispatch_sort, library_path, logits, logits_at, max_threads, route_fullrank, route_lowrank,
                     softmax_colsum)

__all__ = ["DT_BF16", "DT_F32", "DT_F64", "GATE_FULL", "GATE_TOPK", "backward_lowrank", "balance_lowrank", "balance_stats",
           "build", "dispatch_sort", "library_path", "logits", "logits_at", "max_threads", "route_fullrank", "route_lowrank",
           "softmax_colsum"]
