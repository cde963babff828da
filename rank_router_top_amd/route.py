"""Thin ctypes binding of libmore_route.so (C ABI in include/more_route.h).

Argument marshalling only: every step of routing runs in the HIP kernels of the
library.  torch supplies device memory and the current stream.  There is no
fallback: if the library is missing, or a call returns an error code, a
RuntimeError is raised.
"""
from __future__ import annotations

import ctypes as C
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmore_route.so")

MORE_DT_BF16, MORE_DT_F32 = 0, 1
MORE_GATE_TOPK_SOFTMAX, MORE_GATE_FULL_SOFTMAX = 0, 1
MORE_OK = 0
MORE_ERR_WORKSPACE = 6
MORE_ERR_UNSUPPORTED = 7
STATUS_NAMES = {0: "MORE_OK", 1: "MORE_ERR_NULL_ARG", 2: "MORE_ERR_BAD_SHAPE", 3: "MORE_ERR_BAD_K",
                4: "MORE_ERR_BAD_DTYPE", 5: "MORE_ERR_BAD_GATE", 6: "MORE_ERR_WORKSPACE",
                7: "MORE_ERR_UNSUPPORTED", 8: "MORE_ERR_HIP", 9: "MORE_ERR_ALIGNMENT", 10: "MORE_ERR_STALLED",
                11: "MORE_ERR_SCRATCH_LIMIT"}
MORE_ERR_STALLED = 10
MORE_ERR_SCRATCH_LIMIT = 11
EXPORTS = ("more_route_lowrank", "more_route_fullrank", "more_route_workspace_bytes",
           "more_status_str", "more_abi_version", "more_lowrank_pack", "more_lowrank_route_packed",
           "more_lowrank_balance_packed", "more_balance_workspace_bytes", "more_dispatch_sort",
           "more_dispatch_workspace_bytes", "more_lowrank_backward_packed", "more_backward_workspace_bytes",
           "more_topk_merge", "more_set_route_paths", "more_route_status", "more_set_spin_limit",
           "more_dispatch_sort_noalloc")

_lock = threading.Lock()
_lib = None


class MoreError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} -> {STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


def lib() -> C.CDLL:
    """Load libmore_route.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                                   "`python -m rank_router_top_amd.build` (no CPU fallback exists)")
            L = C.CDLL(LIB_PATH)
            p, i64, i32 = C.c_void_p, C.c_int64, C.c_int32
            L.more_route_lowrank.argtypes = [i32, p, i64, i64, p, i64, p, i64, p, i32, i32,
                                             p, p, p, p, p, C.c_size_t, p]
            L.more_route_lowrank.restype = C.c_int
            L.more_route_fullrank.argtypes = [i32, p, i64, i64, p, i64, p, i32, i32,
                                              p, p, p, p, p, C.c_size_t, p]
            L.more_route_fullrank.restype = C.c_int
            L.more_lowrank_pack.argtypes = [i32, p, i64, i64, p, i64, p, p, C.c_size_t, p]
            L.more_lowrank_pack.restype = C.c_int
            L.more_lowrank_route_packed.argtypes = [i32, p, i64, i64, i64, i64, i32, i32,
                                                    p, p, p, p, p, C.c_size_t, p]
            L.more_lowrank_route_packed.restype = C.c_int
            L.more_lowrank_balance_packed.argtypes = [i32, p, i64, i64, i64, i64, i32, i32,
                                                      p, p, p, p, p, p, p, p, C.c_size_t, p]
            L.more_lowrank_balance_packed.restype = C.c_int
            L.more_balance_workspace_bytes.argtypes = [i32, i64, i64, i64, i64, i32]
            L.more_dispatch_sort.argtypes = [p, i64, i32, i64, p, p, p, p, C.c_size_t, p]
            L.more_dispatch_sort.restype = C.c_int
            L.more_dispatch_sort_noalloc.argtypes = [p, i64, i32, i64, p, p, p, p]
            L.more_dispatch_sort_noalloc.restype = C.c_int
            L.more_dispatch_workspace_bytes.argtypes = [i64, i32, i64]
            L.more_lowrank_backward_packed.argtypes = [i32, p, i64, i64, p, i64, p, i64, i32, p, p, p, p,
                                                       p, p, p, p, p, C.c_size_t, p]
            L.more_lowrank_backward_packed.restype = C.c_int
            L.more_backward_workspace_bytes.argtypes = [i32, i64, i64, i64, i64, i32]
            L.more_backward_workspace_bytes.restype = C.c_size_t
            L.more_dispatch_workspace_bytes.restype = C.c_size_t
            L.more_balance_workspace_bytes.restype = C.c_size_t
            L.more_route_workspace_bytes.argtypes = [C.c_int, i32, i64, i64, i64, i64, i32, i32, C.c_int]
            L.more_route_workspace_bytes.restype = C.c_size_t
            L.more_topk_merge.argtypes = [i64, i64, i64, i32, i32, p, p, p, p, p, p, p, p]
            L.more_topk_merge.restype = C.c_int
            L.more_status_str.argtypes = [C.c_int]
            L.more_status_str.restype = C.c_char_p
            L.more_abi_version.restype = C.c_int
            _lib = L
    return _lib


def set_route_paths(names: str | None) -> None:
    """more_set_route_paths: restrict the kernel forms (testing aid; None = all)."""
    L = lib()
    L.more_set_route_paths.argtypes = [C.c_char_p]
    L.more_set_route_paths.restype = None
    L.more_set_route_paths(None if names is None else names.encode())


def set_spin_limit(polls: int) -> None:
    """more_set_spin_limit: polls before a kernel's bounded wait gives up (testing aid; 0 = default)."""
    L = lib()
    L.more_set_spin_limit.argtypes = [C.c_int]
    L.more_set_spin_limit.restype = None
    L.more_set_spin_limit(int(polls))


def route_status(workspace, stream=None) -> int:
    """more_route_status: synchronise the stream, read and clear the workspace's stall word.
    Returns MORE_OK or MORE_ERR_STALLED (other codes raise)."""
    L = lib()
    L.more_route_status.argtypes = [C.c_void_p, C.c_void_p]
    L.more_route_status.restype = C.c_int
    code = L.more_route_status(_ptr(workspace), _stream(stream))
    if code not in (MORE_OK, MORE_ERR_STALLED):
        _check("more_route_status", code)
    return code


def status_str(code: int) -> str:
    return lib().more_status_str(code).decode()


def _check(fn: str, code: int):
    if code != MORE_OK:
        raise MoreError(fn, code, status_str(code))


def workspace_bytes(fullrank: bool, dt: int, N: int, h: int, r: int, M: int, k: int, gate: int,
                    has_bias: bool) -> int:
    return int(lib().more_route_workspace_bytes(int(fullrank), dt, N, h, r, M, k, gate, int(has_bias)))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return MORE_DT_BF16
    if t.dtype == torch.float32:
        return MORE_DT_F32
    raise TypeError(f"unsupported tensor dtype {t.dtype}: bfloat16 or float32 expected")


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _outputs(X, k, want_logit, want_lse, out):
    import torch
    N = X.shape[0]
    if out is not None:
        return out
    dev = X.device
    return dict(idx=torch.empty((N, k), dtype=torch.int32, device=dev),
                gate=torch.empty((N, k), dtype=torch.float32, device=dev),
                logit=torch.empty((N, k), dtype=torch.float32, device=dev) if want_logit else None,
                lse=torch.empty((N,), dtype=torch.float32, device=dev) if want_lse else None)


def _workspace(nbytes, workspace, device):
    import torch
    if workspace is not None:
        return workspace
    return torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=device)


def route_lowrank(X, R1, R2, bias, k: int, gate: int = MORE_GATE_TOPK_SOFTMAX, *, out=None,
                  workspace=None, want_logit: bool = True, want_lse: bool = True, stream=None) -> dict:
    """more_route_lowrank on torch device tensors.  Returns dict(idx, gate, logit, lse)."""
    dt = _dtype_code(X)
    N, h = X.shape
    r, M = R2.shape
    want_lse = want_lse and gate == MORE_GATE_FULL_SOFTMAX
    o = _outputs(X, k, want_logit, want_lse, out)
    nb = workspace_bytes(False, dt, N, h, r, M, k, gate, bias is not None)
    ws = _workspace(nb, workspace, X.device)
    _check("more_route_lowrank", lib().more_route_lowrank(
        dt, _ptr(X), N, h, _ptr(R1), r, _ptr(R2), M, _ptr(bias), k, gate,
        _ptr(o["idx"]), _ptr(o["gate"]), _ptr(o.get("logit")), _ptr(o.get("lse")),
        _ptr(ws), ws.numel(), _stream(stream)))
    return o


def pack_lowrank(R1, R2, bias, workspace, stream=None):
    """more_lowrank_pack: pack static low-rank weights into `workspace` (uint8 device tensor)."""
    dt = _dtype_code(R1)
    h, r = R1.shape
    M = R2.shape[1]
    _check("more_lowrank_pack", lib().more_lowrank_pack(
        dt, _ptr(R1), h, r, _ptr(R2), M, _ptr(bias), _ptr(workspace), workspace.numel(), _stream(stream)))


def route_lowrank_packed(X, r: int, M: int, k: int, gate: int, workspace, *, out=None,
                         want_logit: bool = True, want_lse: bool = True, stream=None) -> dict:
    """more_lowrank_route_packed: route X against weights packed by pack_lowrank."""
    dt = _dtype_code(X)
    N, h = X.shape
    want_lse = want_lse and gate == MORE_GATE_FULL_SOFTMAX
    o = _outputs(X, k, want_logit, want_lse, out)
    _check("more_lowrank_route_packed", lib().more_lowrank_route_packed(
        dt, _ptr(X), N, h, r, M, k, gate, _ptr(o["idx"]), _ptr(o["gate"]), _ptr(o.get("logit")),
        _ptr(o.get("lse")), _ptr(workspace), workspace.numel(), _stream(stream)))
    return o


def balance_workspace_bytes(dt: int, N: int, h: int, r: int, M: int, k: int) -> int:
    return int(lib().more_balance_workspace_bytes(dt, N, h, r, M, k))


def balance_lowrank_packed(X, r: int, M: int, k: int, gate: int, workspace, *, out=None,
                           want_logit: bool = True, stream=None) -> dict:
    """more_lowrank_balance_packed: the routing results plus lse, psum (M),
    counts (M) and stats = (L_bal, H_norm), against weights packed by
    pack_lowrank into `workspace` (sized by balance_workspace_bytes)."""
    import torch
    dt = _dtype_code(X)
    N, h = X.shape
    o = _outputs(X, k, want_logit, True, out)
    if "psum" not in o:
        o["psum"] = torch.empty((M,), dtype=torch.float32, device=X.device)
        o["counts"] = torch.empty((M,), dtype=torch.int32, device=X.device)
        o["stats"] = torch.empty((4,), dtype=torch.float32, device=X.device)
    _check("more_lowrank_balance_packed", lib().more_lowrank_balance_packed(
        dt, _ptr(X), N, h, r, M, k, gate, _ptr(o["idx"]), _ptr(o["gate"]), _ptr(o.get("logit")),
        _ptr(o["lse"]), _ptr(o["psum"]), _ptr(o["counts"]), _ptr(o["stats"]), _ptr(workspace),
        workspace.numel(), _stream(stream)))
    return o


def dispatch_workspace_bytes(N: int, k: int, M: int) -> int:
    return int(lib().more_dispatch_workspace_bytes(N, k, M))


def topk_merge(cand_logit, cand_idx, shard_lse, M: int, shard_width: int, gate: int = MORE_GATE_TOPK_SOFTMAX, *,
               want_logit: bool = True, want_lse: bool = True, stream=None) -> dict:
    """more_topk_merge: cand_logit / cand_idx are (G, N, k) device tensors
    (fp32 / int32, shard-local indices), shard_lse (G, N) fp32 or None.
    Returns dict(idx, gate, logit, lse) with global expert indices."""
    import torch
    G, N, k = cand_logit.shape
    dev = cand_logit.device
    full = gate == MORE_GATE_FULL_SOFTMAX
    o = {"idx": torch.empty((N, k), dtype=torch.int32, device=dev),
         "gate": torch.empty((N, k), dtype=torch.float32, device=dev),
         "logit": torch.empty((N, k), dtype=torch.float32, device=dev) if want_logit else None,
         "lse": torch.empty(N, dtype=torch.float32, device=dev) if (want_lse and full) else None}
    _check("more_topk_merge", lib().more_topk_merge(
        N, M, shard_width, k, gate, _ptr(cand_logit.contiguous()), _ptr(cand_idx.contiguous()),
        _ptr(None if shard_lse is None else shard_lse.contiguous()),
        _ptr(o["idx"]), _ptr(o["gate"]), _ptr(o["logit"]), _ptr(o["lse"]), _stream(stream)))
    return o


def dispatch_sort(idx, M: int, *, out=None, workspace=None, stream=None) -> dict:
    """more_dispatch_sort on an N x k int32 device tensor: returns
    dict(sorted_expert, sorted_slot, offsets)."""
    import torch
    N, k = idx.shape
    if out is None:
        out = dict(sorted_expert=torch.empty((N * k,), dtype=torch.int32, device=idx.device),
                   sorted_slot=torch.empty((N * k,), dtype=torch.int32, device=idx.device),
                   offsets=torch.empty((M + 1,), dtype=torch.int32, device=idx.device))
    ws = _workspace(dispatch_workspace_bytes(N, k, M), workspace, idx.device)
    _check("more_dispatch_sort", lib().more_dispatch_sort(
        _ptr(idx), N, k, M, _ptr(out["sorted_expert"]), _ptr(out["sorted_slot"]), _ptr(out["offsets"]),
        _ptr(ws), ws.numel(), _stream(stream)))
    return out


def dispatch_sort_noalloc(idx, M: int, *, out=None, stream=None) -> dict:
    """more_dispatch_sort_noalloc: as dispatch_sort, with the library's static
    scratch instead of a workspace (outputs allocated here unless given)."""
    import torch
    N, k = idx.shape
    if out is None:
        out = dict(sorted_expert=torch.empty((N * k,), dtype=torch.int32, device=idx.device),
                   sorted_slot=torch.empty((N * k,), dtype=torch.int32, device=idx.device),
                   offsets=torch.empty((M + 1,), dtype=torch.int32, device=idx.device))
    _check("more_dispatch_sort_noalloc", lib().more_dispatch_sort_noalloc(
        _ptr(idx), N, k, M, _ptr(out["sorted_expert"]), _ptr(out["sorted_slot"]), _ptr(out["offsets"]),
        _stream(stream)))
    return out


def backward_workspace_bytes(dt: int, N: int, h: int, r: int, M: int, k: int) -> int:
    return int(lib().more_backward_workspace_bytes(dt, N, h, r, M, k))


def backward_lowrank_packed(X, R1, R2, idx, logit_grad, psum_grad, lse, workspace, *, out=None,
                            want_bias_grad: bool = True, stream=None) -> dict:
    """more_lowrank_backward_packed: gradients of the selected-logit and psum
    losses with the selection held fixed, against weights packed by
    pack_lowrank into `workspace` (sized by backward_workspace_bytes).
    Returns dict(X_grad bf16 N x h, R1_grad, R2_grad, bias_grad)."""
    import torch
    dt = _dtype_code(X)
    N, h = X.shape
    r, M = R2.shape
    k = idx.shape[1]
    if out is None:
        out = dict(X_grad=torch.empty((N, h), dtype=torch.bfloat16, device=X.device),
                   R1_grad=torch.empty((h, r), dtype=torch.float32, device=X.device),
                   R2_grad=torch.empty((r, M), dtype=torch.float32, device=X.device),
                   bias_grad=torch.empty((M,), dtype=torch.float32, device=X.device) if want_bias_grad else None)
    _check("more_lowrank_backward_packed", lib().more_lowrank_backward_packed(
        dt, _ptr(X), N, h, _ptr(R1), r, _ptr(R2), M, k, _ptr(idx), _ptr(logit_grad), _ptr(psum_grad), _ptr(lse),
        _ptr(out["X_grad"]), _ptr(out["R1_grad"]), _ptr(out["R2_grad"]), _ptr(out.get("bias_grad")),
        _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def route_fullrank(X, W, bias, k: int, gate: int = MORE_GATE_TOPK_SOFTMAX, *, out=None,
                   workspace=None, want_logit: bool = True, want_lse: bool = True, stream=None) -> dict:
    """more_route_fullrank on torch device tensors.  Returns dict(idx, gate, logit, lse)."""
    dt = _dtype_code(X)
    N, h = X.shape
    M = W.shape[1]
    want_lse = want_lse and gate == MORE_GATE_FULL_SOFTMAX
    o = _outputs(X, k, want_logit, want_lse, out)
    nb = workspace_bytes(True, dt, N, h, 0, M, k, gate, bias is not None)
    ws = _workspace(nb, workspace, X.device)
    _check("more_route_fullrank", lib().more_route_fullrank(
        dt, _ptr(X), N, h, _ptr(W), M, _ptr(bias), k, gate,
        _ptr(o["idx"]), _ptr(o["gate"]), _ptr(o.get("logit")), _ptr(o.get("lse")),
        _ptr(ws), ws.numel(), _stream(stream)))
    return o


def to_device(a, device):
    """numpy input (bf16 bits as uint16, or fp32) -> torch tensor on `device`."""
    import numpy as np
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)
