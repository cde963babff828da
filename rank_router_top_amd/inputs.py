"""Seeded synthetic inputs for the fused low-rank router.

This module only draws numbers: it holds none of the router's arithmetic.  Both
the fp64 CPU oracle (``oracle/``) and the HIP path take their inputs from here,
so the two sides always see bit-identical operands.

Value distributions (MoRE: Scaling mixture of experts with hardware-aware
low-rank routing, App. D, Lemma 1 and App. F benchmarks):

* X rows are N(0, 1), optionally RMS-normalised per row (x <- x / sqrt(mean(x^2)),
  fp64, no epsilon and no gain), then rounded to the storage dtype.
* R1 (h x r) ~ N(0, 1/h) and R2 (r x M) ~ N(0, 1/r).  With unit-RMS rows the
  logits then have unit variance, which is the variance-matching condition of
  Lemma 1 (the second argument of N(., .) is read as a variance).
* W (h x M, full-rank router) ~ N(0, 1/h).
* bias (M, fp32) ~ N(0, 0.5).

Rounding: fp64 -> fp32 (round to nearest even, numpy) and, for bf16 storage,
fp32 -> bf16 round to nearest even done here in integer arithmetic.  bf16
tensors are returned as ``uint16`` arrays of raw bf16 bits.

Every tensor has its own stream: ``SeedSequence([seed, cfg_id, tensor_id])``
with tensor ids X=0, R1=1, R2=2, bias=3, W=4.  X is drawn in fixed row chunks,
so any prefix of rows is reproducible without drawing the rest
(``make_x(..., n_rows=...)``).
"""
from __future__ import annotations

import numpy as np

DT_BF16 = "bf16"
DT_F32 = "f32"

TENSOR_X, TENSOR_R1, TENSOR_R2, TENSOR_BIAS, TENSOR_W = 0, 1, 2, 3, 4

# X is drawn in chunks of this many rows; chunk c uses its own child stream,
# so a row prefix never depends on how many rows follow.
X_CHUNK_ROWS = 4096


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return raw bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of raw bf16 bits to fp32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _rng(seed: int, cfg_id: int, tensor_id: int, chunk: int | None = None) -> np.random.Generator:
    key = [seed, cfg_id, tensor_id] if chunk is None else [seed, cfg_id, tensor_id, chunk]
    return np.random.default_rng(np.random.SeedSequence(key))


def _store(a64: np.ndarray, dtype: str) -> np.ndarray:
    a32 = a64.astype(np.float32)
    if dtype == DT_F32:
        return a32
    if dtype == DT_BF16:
        return f32_to_bf16_bits(a32)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_x(seed: int, cfg_id: int, N: int, h: int, dtype: str, rms_norm: bool,
           row0: int = 0, n_rows: int | None = None) -> np.ndarray:
    """Rows [row0, row0+n_rows) of the N x h token matrix (default: all N rows)."""
    if n_rows is None:
        n_rows = N - row0
    if row0 < 0 or n_rows < 0 or row0 + n_rows > N:
        raise ValueError("row range outside [0, N)")
    out = np.empty((n_rows, h), dtype=np.float32 if dtype == DT_F32 else np.uint16)
    r = row0
    while r < row0 + n_rows:
        c = r // X_CHUNK_ROWS
        c0 = c * X_CHUNK_ROWS
        c1 = min(c0 + X_CHUNK_ROWS, N)
        block = _rng(seed, cfg_id, TENSOR_X, c).standard_normal((c1 - c0, h))
        lo, hi = r - c0, min(c1, row0 + n_rows) - c0
        block = block[lo:hi]
        if rms_norm:
            block = block / np.sqrt(np.mean(block * block, axis=1, keepdims=True))
        out[r - row0:r - row0 + (hi - lo)] = _store(block, dtype)
        r += hi - lo
    return out


def make_r1(seed: int, cfg_id: int, h: int, r: int, dtype: str) -> np.ndarray:
    """Down-projection R1 (h x r, row-major) ~ N(0, 1/h)."""
    return _store(_rng(seed, cfg_id, TENSOR_R1).standard_normal((h, r)) / np.sqrt(h), dtype)


def make_r2(seed: int, cfg_id: int, r: int, M: int, dtype: str) -> np.ndarray:
    """Up-projection R2 (r x M, row-major) ~ N(0, 1/r)."""
    return _store(_rng(seed, cfg_id, TENSOR_R2).standard_normal((r, M)) / np.sqrt(r), dtype)


def make_w(seed: int, cfg_id: int, h: int, M: int, dtype: str) -> np.ndarray:
    """Full-rank router weight W (h x M, row-major) ~ N(0, 1/h)."""
    return _store(_rng(seed, cfg_id, TENSOR_W).standard_normal((h, M)) / np.sqrt(h), dtype)


def make_bias(seed: int, cfg_id: int, M: int, var: float = 0.5) -> np.ndarray:
    """Per-expert bias (M, fp32) ~ N(0, var)."""
    return (_rng(seed, cfg_id, TENSOR_BIAS).standard_normal(M) * np.sqrt(var)).astype(np.float32)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 view of a stored tensor (bf16 bits or fp32)."""
    if dtype == DT_BF16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


TENSOR_SETS = 5


def make_expert_sets(seed: int, cfg_id: int, N: int, M: int, k: int, skew: float = 0.7) -> np.ndarray:
    """N x k int32 rows of k distinct experts in [0, M), in drawn order: the
    shape of a router's selected indices.  Experts are drawn from a skewed
    categorical distribution, p_e proportional to exp(skew * g_e) with
    g_e ~ N(0, 1) (a biased router concentrates load the same way), and rows
    that drew an expert twice are drawn again until every row is distinct."""
    if not (1 <= k <= M):
        raise ValueError("need 1 <= k <= M")
    rng = _rng(seed, cfg_id, TENSOR_SETS)
    p = np.exp(skew * rng.standard_normal(M))
    cdf = np.cumsum(p / p.sum())
    cdf[-1] = 1.0

    def draw(n):
        return np.minimum(np.searchsorted(cdf, rng.random((n, k)), side="right"), M - 1).astype(np.int32)

    out = draw(N)
    while True:
        s = np.sort(out, axis=1)
        bad = np.nonzero(np.any(s[:, 1:] == s[:, :-1], axis=1))[0] if k > 1 else np.zeros(0, np.int64)
        if bad.size == 0:
            return out
        if k > M // 2:
            # dense rows: a uniformly random k-subset per offending row
            for i in bad:
                out[i] = rng.permutation(M)[:k]
        else:
            out[bad] = draw(bad.size)


TENSOR_GRAD = 6


def make_grads(seed: int, cfg_id: int, N: int, k: int, M: int) -> tuple[np.ndarray, np.ndarray]:
    """Incoming gradients of a backward pass: tvbar (N x k fp32) ~ N(0, 1) on
    the selected logits, and pbar (M fp32) = (M / N) f + N(0, 0.1 M / N): the
    Switch-loss gradient of a skewed dispatch (f drawn like make_expert_sets'
    loads) plus noise."""
    rng = _rng(seed, cfg_id, TENSOR_GRAD)
    tv = rng.standard_normal((N, k)).astype(np.float32)
    f = np.exp(0.7 * rng.standard_normal(M))
    f = f / f.sum()
    pb = ((M / max(N, 1)) * (f + 0.1 * rng.standard_normal(M) / M)).astype(np.float32)
    return tv, pb
