"""GPU parity of the fused full-rank router (more_route_fullrank) against the
fp64 oracle: the LDS-tiled kernel (bf16, k <= 8, h a multiple of 64) at
ragged shapes, exact ties, degenerate logits and the full benchmark size, and
the plain kernel that covers the other shapes.

Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
routing", §2 (the standard router), Fig. 12 and eq. (6) (gates)."""
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
    print(f"[fullrank] {msg}", flush=True)
    sys.stdout.flush()


def to_np(o):
    return {k: (None if v is None else v.cpu().numpy()) for k, v in o.items()}


def run(X, W, b, k, gate):
    d = [R.to_device(a, DEV) for a in (X, W, b)]
    out = R.route_fullrank(*d, k, gate)
    torch.cuda.synchronize()
    return to_np(out)


def gaussian_case(seed, N, h, M, with_bias):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((N, h))
    X /= np.sqrt(np.mean(X * X, axis=1, keepdims=True))
    W = rng.standard_normal((h, M)) / math.sqrt(h)
    b = (rng.standard_normal(M) * math.sqrt(0.5)).astype(np.float32) if with_bias else None
    return I.f32_to_bf16_bits(X.astype(np.float32)), I.f32_to_bf16_bits(W.astype(np.float32)), b


# (N, h, M, k, bias): tiled kernel at ragged token tails, M past a 512-expert
# slab, M below one slab, a single token, k = 1; then two shapes of the plain
# kernel (h not a multiple of 64, k > 8)
SHAPES = [
    (300, 128, 1000, 8, True),
    (129, 64, 192, 4, False),
    (1, 256, 513, 1, True),
    (257, 512, 4096, 8, True),
    (200, 96, 300, 8, True),
    (150, 128, 700, 16, False),
]


@pytest.mark.parametrize("N,h,M,k,bias", SHAPES, ids=[f"{n}x{h}x{m}-k{k}-b{int(b)}" for n, h, m, k, b in SHAPES])
def test_fullrank_shapes(oracle_lib, N, h, M, k, bias):
    X, W, b = gaussian_case(N * 3 + M, N, h, M, bias)
    for gate in (CF.GATE_TOPK_SOFTMAX, CF.GATE_FULL_SOFTMAX):
        say(f"N={N} h={h} M={M} k={k} bias={bias} gate={gate}")
        g = run(X, W, b, k, gate)
        o = oracle_lib.route_fullrank(X, W, b, k, gate)
        at = oracle_lib.logits_at(X, W, None, b, g["idx"], fullrank=True)
        say(f"ok {compare(o, g, k, gate == CF.GATE_FULL_SOFTMAX, 2e-4, 'fullrank-shape', at)}")


def test_fullrank_exact_ties(oracle_lib):
    """A tenth of the experts copy the column and bias of a lower-index expert
    (some in another slab or expert quarter), so their logits are bitwise
    equal; the ordered index lists must match the oracle's (lower index
    first) wherever the distinct logits are well separated."""
    rng = np.random.default_rng(21)
    N, h, M = 400, 128, 1536
    X = I.make_x(4, 41, N, h, I.DT_BF16, True)
    Wf = (rng.standard_normal((h, M)) / math.sqrt(h)).astype(np.float32)
    bf = (rng.standard_normal(M) * math.sqrt(0.5)).astype(np.float32)
    dup = rng.choice(np.arange(1, M), M // 10, replace=False)
    src = (rng.random(dup.size) * dup).astype(np.int64)
    Wf[:, dup] = Wf[:, src]
    bf[dup] = bf[src]
    W = I.f32_to_bf16_bits(Wf)
    for b in (None, bf):
        for k in (1, 5, 8):
            for gate in (CF.GATE_TOPK_SOFTMAX, CF.GATE_FULL_SOFTMAX):
                say(f"ties k={k} bias={b is not None} gate={gate}")
                g = run(X, W, b, k, gate)
                o = oracle_lib.route_fullrank(X, W, b, k, gate)
                at = oracle_lib.logits_at(X, W, None, b, g["idx"], fullrank=True)
                compare(o, g, k, gate == CF.GATE_FULL_SOFTMAX, 2e-4, "fullrank-ties", at)
                lo = o["logit"]
                d = np.abs(np.diff(lo, axis=1)) if k > 1 else np.zeros((N, 0))
                sep = np.all((d == 0) | (d > 1e-3), axis=1) & gap_clear(o)
                assert np.array_equal(g["idx"][sep], o["idx"][sep]), "tie rule violated"


def test_fullrank_all_equal_logits():
    """Zero tokens and no bias: every logit is 0, so the top k are experts
    0..k-1 with uniform gates, and the full-softmax gates are 1/M with
    lse = log M."""
    N, h, M = 130, 64, 1100
    X = np.zeros((N, h), np.uint16)
    rng = np.random.default_rng(3)
    W = I.f32_to_bf16_bits(rng.standard_normal((h, M)).astype(np.float32))
    for k in (1, 8):
        say(f"all-equal k={k}")
        g = run(X, W, None, k, 0)
        assert np.array_equal(g["idx"], np.tile(np.arange(k, dtype=np.int32), (N, 1)))
        assert np.allclose(g["gate"], 1.0 / k, atol=1e-6)
        gf = run(X, W, None, k, 1)
        assert np.array_equal(gf["idx"], np.tile(np.arange(k, dtype=np.int32), (N, 1)))
        assert np.allclose(gf["gate"], 1.0 / M, rtol=1e-5)
        assert np.allclose(gf["lse"], math.log(M), atol=1e-5)


@pytest.mark.parametrize("gate", [CF.GATE_TOPK_SOFTMAX, CF.GATE_FULL_SOFTMAX])
def test_fullrank_full_size(oracle_lib, gate):
    """The full-rank workload at full size (N = 262144, h = 2048, M = 4096,
    k = 8, bias) as the benchmark launches it.  The batch is 128 copies of one
    2048-row block of the seeded tokens: the oracle checks the block, and every
    copy of a row must give bitwise the same outputs."""
    cfg = CF.FULLRANK
    base_n, reps = 2048, cfg.N // 2048
    Xb = cfg.x_rows(0, 0, base_n, n_total=cfg.N)
    W, _, b = cfg.weights(0)
    say(f"full size gate={gate}: oracle on the base block")
    o = oracle_lib.route_fullrank(Xb, W, b, cfg.k, gate)
    say(f"full size gate={gate}: GPU on the tiled batch")
    X = R.to_device(np.tile(Xb, (reps, 1)), DEV)
    d = [R.to_device(a, DEV) for a in (W, b)]
    g = to_np(R.route_fullrank(X, *d, cfg.k, gate))
    torch.cuda.synchronize()
    for key in ("idx", "gate", "logit") + (("lse",) if gate else ()):
        v = g[key].reshape((reps, base_n) + g[key].shape[1:])
        assert all(np.array_equal(v[c], v[0]) for c in range(1, reps)), key
    first = {key: (None if v is None else v[:base_n]) for key, v in g.items()}
    at = oracle_lib.logits_at(Xb, W, None, b, first["idx"], fullrank=True)
    say(f"full size gate={gate}: ok {compare(o, first, cfg.k, gate == CF.GATE_FULL_SOFTMAX, 2e-4, 'fullrank-full', at)}")
