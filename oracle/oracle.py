"""ctypes marshalling for the C oracle (TEST INFRASTRUCTURE; see package docstring)."""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

DT_BF16, DT_F32, DT_F64 = 0, 1, 2
GATE_TOPK, GATE_FULL = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "more_oracle.c")
_LIB = os.path.join(_HERE, "libmore_oracle.so")
_lock = threading.Lock()
_lib = None

_ERRORS = {1: "bad argument", 2: "non-finite input", 3: "out of memory"}


def library_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP).  Plain C, no GPU code."""
    global _lib
    with _lock:
        if force or not os.path.exists(_LIB):
            tmp = _LIB + ".tmp%d" % os.getpid()
            subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                                   "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
            os.replace(tmp, _LIB)
            _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = C.CDLL(_LIB)
        p, i64, i32 = C.c_void_p, C.c_int64, C.c_int
        lib.oracle_route_lowrank.argtypes = [i32, p, i64, i64, p, i64, p, i64, p, i32, i32,
                                             p, p, p, p, p, p, p, i32]
        lib.oracle_route_fullrank.argtypes = [i32, p, i64, i64, p, i64, p, i32, i32,
                                              p, p, p, p, p, p, p, i32]
        lib.oracle_logits.argtypes = [i32, p, i64, i64, p, i64, p, i64, p, i32, p]
        lib.oracle_logits_at.argtypes = [i32, p, i64, i64, p, i64, p, i64, p, i32, i32, p, p, i32]
        lib.oracle_softmax_colsum.argtypes = [i32, p, i64, i64, p, i64, p, i64, p, i32, p, i32]
        lib.oracle_backward_lowrank.argtypes = [i32, p, i64, i64, p, i64, p, i64, p, i32, p, p, p,
                                                p, p, p, p, i32]
        for f in (lib.oracle_route_lowrank, lib.oracle_route_fullrank, lib.oracle_logits, lib.oracle_logits_at,
                  lib.oracle_softmax_colsum, lib.oracle_backward_lowrank):
            f.restype = C.c_int
        lib.oracle_max_threads.restype = C.c_int
        _lib = lib
    return _lib


def _dt_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return DT_BF16
    if a.dtype == np.float32:
        return DT_F32
    if a.dtype == np.float64:
        return DT_F64
    raise TypeError(f"unsupported storage dtype {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _check(rc: int):
    if rc != 0:
        raise RuntimeError(f"oracle error {rc}: {_ERRORS.get(rc, 'unknown')}")


def _outputs(N: int, k: int):
    return dict(idx=np.empty((N, k), np.int32), gate=np.empty((N, k), np.float64),
                logit=np.empty((N, k), np.float64), lse=np.empty(N, np.float64),
                kth=np.empty(N, np.float64), kp1=np.empty(N, np.float64),
                maxabs=np.empty(N, np.float64))


def route_lowrank(X, R1, R2, bias, k: int, gate: int = GATE_TOPK, nthreads: int = 0) -> dict:
    """Exact top-k of (x R1) R2 + b per token; returns idx, gate, logit, lse, kth, kp1, maxabs."""
    X, R1, R2 = (np.ascontiguousarray(a) for a in (X, R1, R2))
    dt = _dt_code(X)
    assert _dt_code(R1) == dt and _dt_code(R2) == dt
    N, h = X.shape
    h2, r = R1.shape
    r2, M = R2.shape
    assert h2 == h and r2 == r
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = _outputs(N, k)
    _check(_load().oracle_route_lowrank(dt, _ptr(X), N, h, _ptr(R1), r, _ptr(R2), M, _ptr(b), k, gate,
                                        _ptr(out["idx"]), _ptr(out["gate"]), _ptr(out["logit"]),
                                        _ptr(out["lse"]), _ptr(out["kth"]), _ptr(out["kp1"]),
                                        _ptr(out["maxabs"]), nthreads))
    return out


def route_fullrank(X, W, bias, k: int, gate: int = GATE_TOPK, nthreads: int = 0) -> dict:
    """Exact top-k of x W + b per token (the standard router of §2)."""
    X, W = np.ascontiguousarray(X), np.ascontiguousarray(W)
    dt = _dt_code(X)
    assert _dt_code(W) == dt
    N, h = X.shape
    h2, M = W.shape
    assert h2 == h
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = _outputs(N, k)
    _check(_load().oracle_route_fullrank(dt, _ptr(X), N, h, _ptr(W), M, _ptr(b), k, gate,
                                         _ptr(out["idx"]), _ptr(out["gate"]), _ptr(out["logit"]),
                                         _ptr(out["lse"]), _ptr(out["kth"]), _ptr(out["kp1"]),
                                         _ptr(out["maxabs"]), nthreads))
    return out


def logits(X, A, B, bias, fullrank: bool = False) -> np.ndarray:
    """All N x M fp64 logits: (x A) B + b, or x A + b when fullrank (A = W)."""
    X, A = np.ascontiguousarray(X), np.ascontiguousarray(A)
    dt = _dt_code(X)
    N, h = X.shape
    if fullrank:
        M, r = A.shape[1], 0
    else:
        B = np.ascontiguousarray(B)
        r, M = B.shape
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty((N, M), np.float64)
    _check(_load().oracle_logits(dt, _ptr(X), N, h, _ptr(A), r, _ptr(None if fullrank else B), M,
                                 _ptr(b), int(fullrank), _ptr(out)))
    return out


def logits_at(X, A, B, bias, idx, fullrank: bool = False, nthreads: int = 0) -> np.ndarray:
    """fp64 logits of the experts named by idx (N x k): out[n, j] = l[n, idx[n, j]]
    with l = (x A) B + b, or x A + b when fullrank (A = W).  NaN where an
    index lies outside [0, M)."""
    X, A = np.ascontiguousarray(X), np.ascontiguousarray(A)
    dt = _dt_code(X)
    N, h = X.shape
    if fullrank:
        M, r = A.shape[1], 0
    else:
        B = np.ascontiguousarray(B)
        r, M = B.shape
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    assert idx.ndim == 2 and idx.shape[0] == N
    k = idx.shape[1]
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty((N, k), np.float64)
    if N == 0 or k == 0:
        return out
    _check(_load().oracle_logits_at(dt, _ptr(X), N, h, _ptr(A), r, _ptr(None if fullrank else B), M,
                                    _ptr(b), int(fullrank), k, _ptr(idx), _ptr(out), nthreads))
    return out


def softmax_colsum(X, A, B, bias, fullrank: bool = False, nthreads: int = 0) -> np.ndarray:
    """psum_i = sum over tokens of the full-softmax probability of expert i (eq. 6, 7)."""
    X, A = np.ascontiguousarray(X), np.ascontiguousarray(A)
    dt = _dt_code(X)
    N, h = X.shape
    if fullrank:
        M, r = A.shape[1], 0
    else:
        B = np.ascontiguousarray(B)
        r, M = B.shape
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty(M, np.float64)
    _check(_load().oracle_softmax_colsum(dt, _ptr(X), N, h, _ptr(A), r, _ptr(None if fullrank else B), M,
                                         _ptr(b), int(fullrank), _ptr(out), nthreads))
    return out


def balance_stats(psum, counts, N: int, k: int) -> tuple[float, float]:
    """Switch balancing loss (eq. 9) and normalised routing entropy (App. G.1).

    L_bal = M * sum_i f_i p_i with f_i = counts_i / (N k) (the share of the
    N k dispatch slots) and p_i = psum_i / N.  H_norm = -sum_a q_a log q_a /
    log M with q_a = counts_a / sum_b counts_b and 0 log 0 = 0; for M = 1
    (one expert carries everything, which is also an even load) H_norm = 1.
    """
    psum = np.asarray(psum, np.float64)
    counts = np.asarray(counts, np.int64)
    M = psum.shape[0]
    f = counts.astype(np.float64) / (N * k)
    p = psum / N
    lbal = float(M * np.dot(f, p))
    if M == 1:
        return lbal, 1.0
    q = counts[counts > 0].astype(np.float64) / counts.sum()
    return lbal, float(-(q * np.log(q)).sum() / np.log(M))


def balance_lowrank(X, R1, R2, bias, k: int, gate: int = GATE_TOPK, nthreads: int = 0) -> dict:
    """Training-forward outputs (App. F.2.1, Algorithm 2 and eq. 7, 9): the
    routing results of route_lowrank, plus psum (eq. 7), the dispatch counts
    per expert (bincount of the selected indices) and (L_bal, H_norm)."""
    out = route_lowrank(X, R1, R2, bias, k, gate, nthreads)
    # lse of every token (the full-softmax normaliser is an output of the training forward)
    full = route_lowrank(X, R1, R2, bias, k, GATE_FULL, nthreads) if gate != GATE_FULL else out
    out["lse"] = full["lse"]
    N = X.shape[0]
    M = R2.shape[1]
    out["psum"] = softmax_colsum(X, R1, R2, bias, False, nthreads)
    out["counts"] = np.bincount(out["idx"].reshape(-1), minlength=M).astype(np.int64)
    out["lbal"], out["hnorm"] = balance_stats(out["psum"], out["counts"], N, k) if N > 0 else (0.0, 0.0)
    return out


def backward_lowrank(X, R1, R2, bias, idx, tvbar, pbar, nthreads: int = 0) -> dict:
    """Gradients of F = sum tvbar * l[n, idx] + sum pbar * psum (App. F.2.2,
    eq. 10-12, Algorithm 3) with the selection idx held fixed: dict(xbar
    N x h, r1bar h x r, r2bar r x M, bbar M), all fp64."""
    X, R1, R2 = (np.ascontiguousarray(a) for a in (X, R1, R2))
    dt = _dt_code(X)
    N, h = X.shape
    r, M = R2.shape
    k = idx.shape[1]
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    tv = np.ascontiguousarray(tvbar, dtype=np.float64)
    pb = None if pbar is None else np.ascontiguousarray(pbar, dtype=np.float64)
    out = dict(xbar=np.empty((N, h)), r1bar=np.empty((h, r)), r2bar=np.empty((r, M)), bbar=np.empty(M))
    _check(_load().oracle_backward_lowrank(dt, _ptr(X), N, h, _ptr(R1), r, _ptr(R2), M, _ptr(b), k, _ptr(idx),
                                           _ptr(tv), _ptr(pb), _ptr(out["xbar"]), _ptr(out["r1bar"]),
                                           _ptr(out["r2bar"]), _ptr(out["bbar"]), nthreads))
    return out


def dispatch_sort(idx, M: int) -> dict:
    """Expert dispatch after the router (App. E, Fig. 9: "sort + count",
    (N, k) -> N k sorted indices + offsets).  The N k selected slots, numbered
    s = n k + j in row-major order of idx, are ordered by expert, slots of the
    same expert in increasing s (a stable sort: a library sort is the step);
    offsets[e] is where expert e's run starts, offsets[M] = N k."""
    keys = np.ascontiguousarray(idx).astype(np.int64).reshape(-1)
    if keys.size and (keys.min() < 0 or keys.max() >= M):
        raise ValueError("expert index outside [0, M)")
    order = np.argsort(keys, kind="stable")
    offsets = np.zeros(M + 1, np.int64)
    offsets[1:] = np.cumsum(np.bincount(keys, minlength=M))
    return dict(sorted_expert=keys[order].astype(np.int32), sorted_slot=order.astype(np.int32),
                offsets=offsets.astype(np.int32))


def max_threads() -> int:
    return int(_load().oracle_max_threads())
