"""GPU parity of the expert-sharded top-k: every shard routed by the library
over its own experts, the shards' candidate lists merged by more_topk_merge,
against the fp64 oracle routing over all M experts at once.

Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
routing", App. E.3 (top-k over expert shards), Fig. 12 and eq. (6) / (8)."""
import math
import sys

import numpy as np
import pytest
import torch

from rank_router_top_amd import configs as CF
from rank_router_top_amd import inputs as I
from rank_router_top_amd import route as R

from oracle.parity import compare, gap_clear

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"


def say(msg):
    print(f"[merge] {msg}", flush=True)
    sys.stdout.flush()


def sharded_route(X, R1, R2, b, k, gate, width):
    """Route every shard of `width` consecutive experts, then merge."""
    M = R2.shape[1]
    Xd, R1d = R.to_device(X, DEV), R.to_device(R1, DEV)
    G = (M + width - 1) // width
    logits, idxs, lses = [], [], []
    for g in range(G):
        cols = slice(g * width, min(M, (g + 1) * width))
        R2g = R.to_device(np.ascontiguousarray(R2[:, cols]), DEV)
        bg = None if b is None else R.to_device(np.ascontiguousarray(b[cols]), DEV)
        o = R.route_lowrank(Xd, R1d, R2g, bg, k, gate)
        logits.append(o["logit"])
        idxs.append(o["idx"])
        if gate == CF.GATE_FULL_SOFTMAX:
            lses.append(o["lse"])
    cl = torch.stack(logits).contiguous()
    ci = torch.stack(idxs).contiguous()
    sl = torch.stack(lses).contiguous() if lses else None
    out = R.topk_merge(cl, ci, sl, M, width, gate)
    torch.cuda.synchronize()
    return {key: (None if v is None else v.cpu().numpy()) for key, v in out.items()}


# the last two have 41 and 64 shards: the merge takes one wave per token there
CASES = [(CF.HEADLINE, 1024 + 19, 512), (CF.HEADLINE, 700, 2048), (CF.PREFILL_H512, 900, 1000),
         (CF.HEADLINE, 300, 100), (CF.HEADLINE, 200, 64)]


@pytest.mark.parametrize("cfg,n,width", CASES, ids=[f"{c.name}-{n}-w{w}" for c, n, w in CASES])
@pytest.mark.parametrize("gate", [CF.GATE_TOPK_SOFTMAX, CF.GATE_FULL_SOFTMAX])
def test_sharded_equals_full_route(oracle_lib, cfg, n, width, gate):
    X = cfg.x_rows(0, 0, n, n_total=cfg.N)
    R1, R2, b = cfg.weights(0)
    say(f"{cfg.name} N={n} M={cfg.M} shard width {width} gate={gate}")
    g = sharded_route(X, R1, R2, b, cfg.k, gate, width)
    o = oracle_lib.route_lowrank(X, R1, R2, b, cfg.k, gate)
    at = oracle_lib.logits_at(X, R1, R2, b, g["idx"])
    say(f"ok {compare(o, g, cfg.k, gate == CF.GATE_FULL_SOFTMAX, 2e-4, 'sharded', at)}")


def test_sharded_ties_lower_index_wins(oracle_lib):
    """Experts copied into other shards (same column of R2, same bias) give
    bitwise-equal logits in different shards; the merged, ordered lists must
    put the lower global index first, as the oracle does."""
    rng = np.random.default_rng(17)
    h, r, M, N, width = 256, 32, 1200, 600, 256
    X = I.make_x(4, 51, N, h, I.DT_BF16, True)
    R1 = I.f32_to_bf16_bits((rng.standard_normal((h, r)) / math.sqrt(h)).astype(np.float32))
    R2f = (rng.standard_normal((r, M)) / math.sqrt(r)).astype(np.float32)
    bf = (rng.standard_normal(M) * math.sqrt(0.5)).astype(np.float32)
    dup = rng.choice(np.arange(width, M), M // 8, replace=False)
    src = (rng.random(dup.size) * (dup - width)).astype(np.int64)   # in an earlier shard
    R2f[:, dup] = R2f[:, src]
    bf[dup] = bf[src]
    R2 = I.f32_to_bf16_bits(R2f)
    for k in (1, 5, 8, 16):   # 5: the scalar form with filler slots; 8, 16: the 16-byte form
        for gate in (CF.GATE_TOPK_SOFTMAX, CF.GATE_FULL_SOFTMAX):
            say(f"ties k={k} gate={gate}")
            g = sharded_route(X, R1, R2, bf, k, gate, width)
            o = oracle_lib.route_lowrank(X, R1, R2, bf, k, gate)
            compare(o, g, k, gate == CF.GATE_FULL_SOFTMAX, 2e-4, "sharded-ties",
                    oracle_lib.logits_at(X, R1, R2, bf, g["idx"]))
            lo = o["logit"]
            d = np.abs(np.diff(lo, axis=1)) if k > 1 else np.zeros((N, 0))
            sep = np.all((d == 0) | (d > 1e-3), axis=1) & gap_clear(o)
            assert np.array_equal(g["idx"][sep], o["idx"][sep]), "tie rule violated"


def test_merge_of_one_shard_is_identity():
    """G = 1: the merge returns the shard's own list, gates recomputed from
    its logits (and lse) exactly as the routing call forms them."""
    cfg = CF.HEADLINE
    X = R.to_device(cfg.x_rows(0, 0, 333, n_total=cfg.N), DEV)
    R1, R2, b = (R.to_device(a, DEV) for a in cfg.weights(0))
    for gate in (CF.GATE_TOPK_SOFTMAX, CF.GATE_FULL_SOFTMAX):
        o = R.route_lowrank(X, R1, R2, b, cfg.k, gate)
        m = R.topk_merge(o["logit"][None].contiguous(), o["idx"][None].contiguous(),
                         None if gate == 0 else o["lse"][None].contiguous(), cfg.M, cfg.M, gate)
        torch.cuda.synchronize()
        assert torch.equal(m["idx"], o["idx"])
        assert torch.equal(m["logit"], o["logit"])
        assert torch.allclose(m["gate"], o["gate"], rtol=0, atol=1e-6)
        if gate:
            assert torch.allclose(m["lse"], o["lse"], rtol=0, atol=1e-6)
