"""The router workloads: shapes, dtypes, gate modes and input recipes.

Shapes follow the router-alone measurements of "MoRE: Scaling mixture of
experts with hardware-aware low-rank routing" (§4.2 Fig. 3, App. H.6 Fig. 24:
N = B*T tokens with T = 1024) plus a many-expert setting.  Each config names
the generator streams it draws from (``x_cfg`` for X and bias, ``w_cfg`` for
R1/R2/W), so the rank sweep reuses the headline's X and bias exactly.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

from . import inputs as I

GATE_TOPK_SOFTMAX = 0
GATE_FULL_SOFTMAX = 1


@dataclass(frozen=True)
class RouterConfig:
    name: str
    N: int
    h: int
    M: int
    r: int            # 0 for the full-rank router
    k: int
    dtype: str
    rms_norm: bool
    bias_var: float   # 0 -> no bias
    gates: tuple      # gate modes exercised on this workload
    x_cfg: int
    w_cfg: int
    fullrank: bool = False

    @property
    def has_bias(self) -> bool:
        return self.bias_var > 0

    def with_n(self, n: int) -> "RouterConfig":
        """Same workload at fewer tokens (the first n rows of the same X)."""
        return replace(self, N=n)

    def x_rows(self, seed: int, row0: int = 0, n_rows: int | None = None, n_total: int | None = None):
        return I.make_x(seed, self.x_cfg, n_total or self.N, self.h, self.dtype, self.rms_norm,
                        row0=row0, n_rows=n_rows)

    def weights(self, seed: int):
        """(R1, R2, bias) for the low-rank router or (W, None, bias) for full rank."""
        bias = I.make_bias(seed, self.x_cfg, self.M, self.bias_var) if self.has_bias else None
        if self.fullrank:
            return I.make_w(seed, self.w_cfg, self.h, self.M, self.dtype), None, bias
        return (I.make_r1(seed, self.w_cfg, self.h, self.r, self.dtype),
                I.make_r2(seed, self.w_cfg, self.r, self.M, self.dtype), bias)

    def x_bytes(self) -> int:
        return self.N * self.h * (2 if self.dtype == I.DT_BF16 else 4)

    def flops(self) -> int:
        """Algorithmic MFMA work: 2N(hr + rM) low-rank, 2NhM full-rank."""
        if self.fullrank:
            return 2 * self.N * self.h * self.M
        return 2 * self.N * (self.h * self.r + self.r * self.M)


TINY = RouterConfig("tiny_f32", N=256, h=128, M=192, r=16, k=4, dtype=I.DT_F32, rms_norm=False,
                    bias_var=0.0, gates=(GATE_TOPK_SOFTMAX,), x_cfg=1, w_cfg=1)
PREFILL_H512 = RouterConfig("prefill_h512", N=262144, h=512, M=4096, r=32, k=8, dtype=I.DT_BF16,
                            rms_norm=True, bias_var=0.0,
                            gates=(GATE_TOPK_SOFTMAX, GATE_FULL_SOFTMAX), x_cfg=2, w_cfg=2)
HEADLINE = RouterConfig("headline", N=262144, h=2048, M=4096, r=32, k=8, dtype=I.DT_BF16,
                        rms_norm=True, bias_var=0.5, gates=(GATE_TOPK_SOFTMAX,), x_cfg=3, w_cfg=3)
RANK16 = replace(HEADLINE, name="rank16", r=16, w_cfg=4)
RANK64 = replace(HEADLINE, name="rank64", r=64, w_cfg=4)
RANK128 = replace(HEADLINE, name="rank128", r=128, w_cfg=4)
FULLRANK = replace(HEADLINE, name="fullrank", r=0, w_cfg=4, fullrank=True)
MANY_PREFILL = RouterConfig("many_experts_prefill", N=65536, h=4096, M=65536, r=64, k=16,
                            dtype=I.DT_BF16, rms_norm=True, bias_var=0.0,
                            gates=(GATE_FULL_SOFTMAX,), x_cfg=5, w_cfg=5)
# Decode: the first 256 tokens of the prefill batch, same weights.
MANY_DECODE = replace(MANY_PREFILL, name="many_experts_decode", N=256)

ALL = {c.name: c for c in (TINY, PREFILL_H512, HEADLINE, RANK16, RANK64, RANK128, FULLRANK,
                           MANY_PREFILL, MANY_DECODE)}


def decode_x(seed: int, cfg: RouterConfig) -> np.ndarray:
    """Decode X is the row prefix of the prefill batch (same generator streams)."""
    return I.make_x(seed, cfg.x_cfg, MANY_PREFILL.N, cfg.h, cfg.dtype, cfg.rms_norm, 0, cfg.N)
