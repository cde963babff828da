"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every case prints its name before running so that a failing GPU step can be
identified from the log.  Sizes are reduced from the full workloads so the
oracle finishes in seconds, while still spanning many expert tiles, several
workgroups and a ragged token tail.
"""
import math
import sys

import numpy as np
import pytest
import torch

from rank_router_top_amd import configs as CF
from rank_router_top_amd import inputs as I
from rank_router_top_amd import route as R

from oracle.parity import compare, gap_clear, properties

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"


def say(msg):
    print(f"[parity] {msg}", flush=True)
    sys.stdout.flush()


def to_np(o):
    return {k: (None if v is None else v.cpu().numpy()) for k, v in o.items()}


def run_lowrank(X, R1, R2, b, k, gate):
    d = [R.to_device(a, DEV) for a in (X, R1, R2, b)]
    out = R.route_lowrank(*d, k, gate)
    torch.cuda.synchronize()
    return to_np(out)


def run_fullrank(X, W, b, k, gate):
    d = [R.to_device(a, DEV) for a in (X, W, b)]
    out = R.route_fullrank(*d, k, gate)
    torch.cuda.synchronize()
    return to_np(out)


def check_lowrank(oracle_lib, X, R1, R2, b, k, gate, label, logit_tol=2e-4):
    say(f"{label}: N={X.shape[0]} h={X.shape[1]} r={R1.shape[1]} M={R2.shape[1]} k={k} gate={gate}")
    g = run_lowrank(X, R1, R2, b, k, gate)
    o = oracle_lib.route_lowrank(X, R1, R2, b, k, gate)
    at = oracle_lib.logits_at(X, R1, R2, b, g["idx"])
    res = compare(o, g, k, gate == R.MORE_GATE_FULL_SOFTMAX, logit_tol, label, at)
    say(f"{label}: ok {res}")
    return o, g


# --------------------------------------------------------------------------- configs
CASES = [
    (CF.TINY, 256, CF.GATE_TOPK_SOFTMAX),
    (CF.PREFILL_H512, 4096 + 37, CF.GATE_TOPK_SOFTMAX),
    (CF.PREFILL_H512, 2048 + 99, CF.GATE_FULL_SOFTMAX),
    (CF.HEADLINE, 2048 + 5, CF.GATE_TOPK_SOFTMAX),
    (CF.HEADLINE, 1024 + 77, CF.GATE_FULL_SOFTMAX),
    (CF.RANK16, 1024 + 1, CF.GATE_TOPK_SOFTMAX),
    (CF.RANK64, 1024 + 31, CF.GATE_TOPK_SOFTMAX),
    (CF.RANK128, 1024 + 64, CF.GATE_TOPK_SOFTMAX),
    (CF.MANY_DECODE, 256, CF.GATE_FULL_SOFTMAX),
    (CF.MANY_PREFILL, 2048 + 19, CF.GATE_FULL_SOFTMAX),
]


@pytest.mark.parametrize("cfg,n,gate", CASES, ids=[f"{c.name}-{n}-g{g}" for c, n, g in CASES])
def test_lowrank_configs(oracle_lib, cfg, n, gate):
    X = cfg.x_rows(0, 0, n, n_total=cfg.N)
    R1, R2, b = cfg.weights(0)
    check_lowrank(oracle_lib, X, R1, R2, b, cfg.k, gate, cfg.name)


@pytest.mark.parametrize("seed", [1, 2])
def test_headline_other_seeds(oracle_lib, seed):
    cfg = CF.HEADLINE
    X = cfg.x_rows(seed, 0, 1024, n_total=cfg.N)
    R1, R2, b = cfg.weights(seed)
    check_lowrank(oracle_lib, X, R1, R2, b, cfg.k, CF.GATE_TOPK_SOFTMAX, f"headline-seed{seed}")


@pytest.mark.parametrize("gate", [CF.GATE_TOPK_SOFTMAX, CF.GATE_FULL_SOFTMAX])
def test_fullrank_baseline(oracle_lib, gate):
    cfg = CF.FULLRANK
    n = 512 + 3
    X = cfg.x_rows(0, 0, n, n_total=cfg.N)
    W, _, b = cfg.weights(0)
    say(f"fullrank: N={n} gate={gate}")
    g = run_fullrank(X, W, b, cfg.k, gate)
    o = oracle_lib.route_fullrank(X, W, b, cfg.k, gate)
    at = oracle_lib.logits_at(X, W, None, b, g["idx"], fullrank=True)
    say(f"fullrank: ok {compare(o, g, cfg.k, gate == CF.GATE_FULL_SOFTMAX, 2e-4, 'fullrank', at)}")


def test_fullrank_tiny_fp32(oracle_lib):
    rng = np.random.default_rng(4)
    X = rng.standard_normal((200, 64)).astype(np.float32)
    W = (rng.standard_normal((64, 77)) / 8).astype(np.float32)
    b = rng.standard_normal(77).astype(np.float32)
    say("fullrank fp32 tiny")
    g = run_fullrank(X, W, b, 5, 0)
    o = oracle_lib.route_fullrank(X, W, b, 5, 0)
    compare(o, g, 5, False, 1e-5, "fullrank-f32", oracle_lib.logits_at(X, W, None, b, g["idx"], fullrank=True))


# ------------------------------------------------------------------------ edge cases
@pytest.mark.parametrize("N,h,r,M,k,dt", [
    (1, 64, 16, 40, 3, "bf16"),        # single token
    (33, 8, 16, 32, 32, "bf16"),       # k = M = 32, h = 8 (half a K-step)
    (40, 8, 16, 33, 30, "bf16"),       # M one past a tile, k close to M
    (70, 136, 32, 100, 1, "bf16"),     # k = 1, h % 16 = 8, ragged M
    (130, 256, 48, 1000, 32, "bf16"),  # k = 32 (largest list), r = 48 padded to 64
    (97, 96, 16, 257, 16, "f32"),      # fp32 path, k = 16
    (64, 64, 128, 64, 32, "f32"),      # fp32, r = 128, k = M/2
    (2048 + 40, 256, 32, 4096 + 700, 8, "bf16"),   # two-kernel path, 3 chunks of the bias order, last one ragged
    (120, 128, 16, 16384 - 3, 8, "bf16"),          # largest M with the bias-descending order (8 chunks)
    (2048 + 50, 1024, 64, 4096, 8, "bf16"),        # two-kernel path at r = 64, the largest h whose R1 fits its LDS
])
def test_edge_shapes(oracle_lib, N, h, r, M, k, dt):
    rng = np.random.default_rng(N * 7 + M)
    X = rng.standard_normal((N, h))
    X /= np.sqrt(np.mean(X * X, axis=1, keepdims=True))
    R1 = rng.standard_normal((h, r)) / math.sqrt(h)
    R2 = rng.standard_normal((r, M)) / math.sqrt(r)
    b = (rng.standard_normal(M) * 0.7).astype(np.float32)
    conv = (lambda a: I.f32_to_bf16_bits(a.astype(np.float32))) if dt == "bf16" else (lambda a: a.astype(np.float32))
    X, R1, R2 = conv(X), conv(R1), conv(R2)
    for gate in (0, 1):
        check_lowrank(oracle_lib, X, R1, R2, b, k, gate, f"edge-{N}x{h}x{r}x{M}-k{k}-{dt}",
                      logit_tol=2e-4 if dt == "bf16" else 1e-5)


# Few tokens, many experts: the expert range split over (block, shard) waves and
# the shards' candidate lists merged (App. E.3; eq. (8) across shards).  The
# shapes cover one token, a ragged M with the largest k, the largest block
# count the form takes (64 blocks), r = 128 and a shard whose tiles hold a
# single real expert (M = 32 t + 1).
@pytest.mark.parametrize("N,h,r,M,k", [
    (1, 4096, 64, 65536, 16),
    (100, 512, 32, 8192 + 5, 32),
    (2048, 2048, 32, 4096, 8),
    (300, 1024, 128, 20000, 4),
    (77, 256, 16, 32 * 260 + 1, 8),
    (77, 256, 16, 32 * 260 + 1, 16),     # two-pass shards at k = 16, the last shard with one real expert
    (100, 512, 32, 8192 + 5, 12),        # k below the 16-wide lists (their +inf pads)
])
def test_splitm_shapes(oracle_lib, route_paths, N, h, r, M, k):
    route_paths("splitm")
    rng = np.random.default_rng(N * 3 + M)
    X = rng.standard_normal((N, h))
    X /= np.sqrt(np.mean(X * X, axis=1, keepdims=True))
    R1 = rng.standard_normal((h, r)) / math.sqrt(h)
    R2 = rng.standard_normal((r, M)) / math.sqrt(r)
    b = (rng.standard_normal(M) * 0.7).astype(np.float32)
    X, R1, R2 = (I.f32_to_bf16_bits(a.astype(np.float32)) for a in (X, R1, R2))
    for gate in (0, 1):
        check_lowrank(oracle_lib, X, R1, R2, b, k, gate, f"splitm-{N}x{h}x{r}x{M}-k{k}")


def test_exact_ties_lower_index_wins(oracle_lib):
    """Duplicated R2 columns (and equal biases) give bitwise-equal logits; the
    lower expert index must win, with and without the bias-ordered sweep."""
    rng = np.random.default_rng(9)
    h, r, M = 64, 16, 256
    X = I.f32_to_bf16_bits(rng.standard_normal((300, h)).astype(np.float32))
    R1 = I.f32_to_bf16_bits((rng.standard_normal((h, r)) / 8).astype(np.float32))
    base = rng.standard_normal((r, 16)).astype(np.float32)
    cols = rng.integers(0, 16, M)
    R2 = I.f32_to_bf16_bits(base[:, cols])
    bias_base = rng.standard_normal(16).astype(np.float32)
    for b in (None, bias_base[cols]):
        for k in (1, 5, 8, 20):
            say(f"ties k={k} bias={b is not None}")
            g = run_lowrank(X, R1, R2, b, k, 0)
            o = oracle_lib.route_lowrank(X, R1, R2, b, k, 0)
            # logits of equal columns are bitwise equal on both sides, so the full
            # ordered index lists must agree wherever the oracle's distinct values
            # are separated by more than the GPU's rounding
            assert np.array_equal(g["idx"], o["idx"]), "tie rule violated"


def test_bias_ties_across_order_chunks(oracle_lib):
    """Biases on a coarse grid (many exact ties, -0 and +0 among them) across
    the 2048-expert chunks the sweep order is built from: the order must still
    be a permutation, so the result matches the oracle."""
    rng = np.random.default_rng(11)
    N, h, r, M, k = 2048 + 17, 128, 32, 6000, 8
    X = rng.standard_normal((N, h))
    X /= np.sqrt(np.mean(X * X, axis=1, keepdims=True))
    R1 = rng.standard_normal((h, r)) / math.sqrt(h)
    R2 = rng.standard_normal((r, M)) / math.sqrt(r)
    b = (np.round(rng.standard_normal(M) * 2) / 4).astype(np.float32)
    b[::7] = -0.0
    conv = lambda a: I.f32_to_bf16_bits(a.astype(np.float32))
    check_lowrank(oracle_lib, conv(X), conv(R1), conv(R2), b, k, 0, "bias-ties-6000")


def test_all_equal_logits(oracle_lib):
    """Zero tokens and no bias: every logit is 0.  The top-k must be experts
    0..k-1 with uniform gates (stresses the log's tie pruning)."""
    N, h, r, M = 64, 32, 16, 4096
    X = np.zeros((N, h), np.uint16)
    rng = np.random.default_rng(0)
    R1 = I.f32_to_bf16_bits(rng.standard_normal((h, r)).astype(np.float32))
    R2 = I.f32_to_bf16_bits(rng.standard_normal((r, M)).astype(np.float32))
    for k in (1, 8, 32):
        say(f"all-equal k={k}")
        g = run_lowrank(X, R1, R2, None, k, 0)
        assert np.array_equal(g["idx"], np.tile(np.arange(k, dtype=np.int32), (N, 1)))
        assert np.allclose(g["gate"], 1.0 / k, atol=1e-6)
        gf = run_lowrank(X, R1, R2, None, k, 1)
        assert np.allclose(gf["gate"], 1.0 / M, rtol=1e-5)
        assert np.allclose(gf["lse"], math.log(M), atol=1e-5)


def test_planted_set_fp32(oracle_lib):
    """Thm. 4 construction (App. J) at r = M: top-k = S exactly, equal logits
    inside S listed by ascending index, gates 1/k."""
    M, k, N = 64, 6, 40
    rho = math.sqrt(1 / k + 1 / (M - k))
    rng = np.random.default_rng(1)
    X = np.full((N, M), -1.0 / ((M - k) * rho), np.float32)
    sets = []
    for n in range(N):
        S = np.sort(rng.choice(M, k, replace=False))
        X[n, S] = np.float32(1.0 / (k * rho))
        sets.append(S)
    eye = np.eye(M, dtype=np.float32)
    say("planted set")
    g = run_lowrank(X, eye, eye, None, k, 0)
    assert np.array_equal(g["idx"], np.array(sets, np.int32))
    assert np.allclose(g["gate"], 1.0 / k, atol=1e-6)


def test_hypercube_router(oracle_lib):
    """Prop. 1 construction: sign-vector experts (exact in bf16); top-1 is the
    sign pattern of z."""
    r, h, N = 8, 64, 512
    M = 2 ** r
    R1 = np.zeros((h, 16), np.float32)
    R1[:r, :r] = np.eye(r)
    bits = (np.arange(M)[None, :] >> np.arange(r)[:, None]) & 1
    R2 = np.zeros((16, M), np.float32)
    R2[:r] = np.where(bits == 1, 1.0, -1.0)
    X = I.make_x(3, 30, N, h, I.DT_BF16, False)
    z = I.to_f64(X, I.DT_BF16)[:, :r]
    say("hypercube")
    g = run_lowrank(X, I.f32_to_bf16_bits(R1), I.f32_to_bf16_bits(R2), None, 4, 0)
    top1 = ((z > 0).astype(np.int64) << np.arange(r)).sum(1)
    assert np.array_equal(g["idx"][:, 0], top1.astype(np.int32))
    o = oracle_lib.route_lowrank(X, I.f32_to_bf16_bits(R1), I.f32_to_bf16_bits(R2), None, 4, 0)
    at = oracle_lib.logits_at(X, I.f32_to_bf16_bits(R1), I.f32_to_bf16_bits(R2), None, g["idx"])
    compare(o, g, 4, False, 2e-4, "hypercube", at)


def test_hypercube_loads_within_bernstein_bound_gpu(oracle_lib):
    """Prop. 1 / Lemma 4 on the GPU's selection: under the hypercube router each
    expert is chosen with probability exactly k/M (the sign symmetry survives
    the bf16 rounding of the Gaussian tokens); over n tokens every load lies
    within sqrt(2 n k L / M) + 2L/3 of n k / M with probability >= 1 - delta,
    L = log(2M/delta).  Seeded: one fixed draw that must satisfy the bound; the
    selection is also held to the oracle's by the parity rule."""
    r, h, k, n, delta = 8, 64, 4, 1 << 16, 1e-3
    M = 2 ** r
    R1 = np.zeros((h, 16), np.float32)
    R1[:r, :r] = np.eye(r)
    bits = (np.arange(M)[None, :] >> np.arange(r)[:, None]) & 1
    R2 = np.zeros((16, M), np.float32)
    R2[:r] = np.where(bits == 1, 1.0, -1.0)
    rng = np.random.default_rng(2025)
    X = I.f32_to_bf16_bits(rng.standard_normal((n, h)).astype(np.float32))
    R1b, R2b = I.f32_to_bf16_bits(R1), I.f32_to_bf16_bits(R2)
    say("hypercube loads")
    g = run_lowrank(X, R1b, R2b, None, k, 0)
    loads = np.bincount(g["idx"].ravel(), minlength=M)
    L = math.log(2 * M / delta)
    bound = math.sqrt(2 * n * k * L / M) + 2 * L / 3
    assert loads.sum() == n * k
    assert np.max(np.abs(loads - n * k / M)) <= bound, (np.max(np.abs(loads - n * k / M)), bound)
    o = oracle_lib.route_lowrank(X, R1b, R2b, None, k, 0)
    compare(o, g, k, False, 2e-4, "hypercube-loads", oracle_lib.logits_at(X, R1b, R2b, None, g["idx"]))


def test_expert_permutation_equivariance():
    """Lemma 3: permuting R2's columns and the bias permutes the indices; gates unchanged."""
    cfg = CF.HEADLINE
    X = cfg.x_rows(0, 0, 1024, n_total=cfg.N)
    R1, R2, b = cfg.weights(0)
    perm = np.random.default_rng(5).permutation(cfg.M)
    say("equivariance")
    a = run_lowrank(X, R1, R2, b, cfg.k, 0)
    c = run_lowrank(X, R1, np.ascontiguousarray(R2[:, perm]), b[perm], cfg.k, 0)
    assert np.array_equal(np.sort(perm[c["idx"]], 1), np.sort(a["idx"], 1))
    assert np.allclose(a["gate"], c["gate"], atol=1e-6)


def test_deterministic_bitwise():
    """Two runs are bit-identical (candidates may be logged in a different
    order from run to run; the results may not differ)."""
    cfg = CF.HEADLINE
    X = cfg.x_rows(0, 0, 4096 + 3, n_total=cfg.N)
    R1, R2, b = cfg.weights(0)
    say("determinism")
    a = run_lowrank(X, R1, R2, b, cfg.k, 0)
    c = run_lowrank(X, R1, R2, b, cfg.k, 0)
    for key in ("idx", "gate", "logit"):
        assert np.array_equal(a[key], c[key])


def test_gap_rule_excludes_few_tokens(oracle_lib):
    """Sanity of the comparison itself on the headline shape: the gap rule
    excludes a minority of tokens, so parity is tested on most of them."""
    cfg = CF.HEADLINE
    X = cfg.x_rows(0, 0, 2048, n_total=cfg.N)
    R1, R2, b = cfg.weights(0)
    o = oracle_lib.route_lowrank(X, R1, R2, b, cfg.k, 0)
    assert gap_clear(o).mean() > 0.8


# ------------------------------------------------------------- every kernel path
# The library takes the fastest kernel whose envelope fits; MORE_ROUTE_PATHS
# restricts the candidates so that the slower paths are checked on the same
# shapes ("none" leaves only the plain kernel, which fits every shape).
PATH_CASES = [
    (CF.HEADLINE, 1024 + 77, CF.GATE_TOPK_SOFTMAX),
    (CF.PREFILL_H512, 512 + 9, CF.GATE_FULL_SOFTMAX),
    (CF.RANK16, 512 + 3, CF.GATE_TOPK_SOFTMAX),
]


@pytest.fixture
def route_paths():
    """Restrict the kernel forms for one test; every form is allowed again after it."""
    yield R.set_route_paths
    R.set_route_paths(None)


@pytest.mark.parametrize("path", ["split", "ring", "splitm", "pc", "lock", "stream", "none"])
@pytest.mark.parametrize("cfg,n,gate", PATH_CASES, ids=[f"{c.name}-{n}-g{g}" for c, n, g in PATH_CASES])
def test_kernel_paths(oracle_lib, route_paths, path, cfg, n, gate):
    route_paths(path)
    X = cfg.x_rows(0, 0, n, n_total=cfg.N)
    R1, R2, b = cfg.weights(0)
    check_lowrank(oracle_lib, X, R1, R2, b, cfg.k, gate, f"{cfg.name}-path-{path}")


def test_packed_workspace_sizes(oracle_lib):
    """Pack once, route batches of different sizes against one workspace: one
    sized for the largest batch (the two-kernel path, token scratch present)
    and one sized for no tokens at all (no scratch: a one-kernel path)."""
    cfg = CF.HEADLINE
    R1, R2, b = (R.to_device(a, DEV) for a in cfg.weights(0))
    sizes = [1024 + 77, 300]
    for n_ws in (max(sizes), 0):
        nbytes = R.workspace_bytes(False, 0, n_ws, cfg.h, cfg.r, cfg.M, cfg.k, 0, True)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
        R.pack_lowrank(R1, R2, b, ws)
        for n in sizes:
            say(f"packed workspace for {n_ws} tokens, batch of {n}")
            Xn = cfg.x_rows(0, 0, n, n_total=cfg.N)
            g = to_np(R.route_lowrank_packed(R.to_device(Xn, DEV), cfg.r, cfg.M, cfg.k, 0, ws))
            torch.cuda.synchronize()
            o = oracle_lib.route_lowrank(Xn, *cfg.weights(0), cfg.k, 0)
            at = oracle_lib.logits_at(Xn, *cfg.weights(0), g["idx"])
            compare(o, g, cfg.k, False, 2e-4, f"packed-{n_ws}-{n}", at)


def test_ties_many_experts(oracle_lib):
    """M = 4096 with exact ties: a tenth of the experts copy the column and
    bias of a lower-index expert, so their logits are bitwise equal; the
    ordered index lists must match the oracle's (lower index first)."""
    rng = np.random.default_rng(11)
    h, r, M, N = 256, 32, 4096, 700
    X = I.make_x(4, 31, N, h, I.DT_BF16, True)
    R1 = I.f32_to_bf16_bits((rng.standard_normal((h, r)) / math.sqrt(h)).astype(np.float32))
    R2f = (rng.standard_normal((r, M)) / math.sqrt(r)).astype(np.float32)
    b = (rng.standard_normal(M) * math.sqrt(0.5)).astype(np.float32)
    dup = rng.choice(np.arange(1, M), M // 10, replace=False)
    src = (rng.random(dup.size) * dup).astype(np.int64)   # a lower index
    R2f[:, dup] = R2f[:, src]
    b[dup] = b[src]
    R2 = I.f32_to_bf16_bits(R2f)
    for gate in (0, 1):
        say(f"ties M=4096 gate={gate}")
        g = run_lowrank(X, R1, R2, b, 8, gate)
        o = oracle_lib.route_lowrank(X, R1, R2, b, 8, gate)
        compare(o, g, 8, gate == 1, 2e-4, "ties-4096", oracle_lib.logits_at(X, R1, R2, b, g["idx"]))
        # where the oracle's distinct logits are well separated, the full
        # ordered lists (ties included) must agree
        lo = o["logit"]
        sep = np.all((np.abs(np.diff(lo, axis=1)) == 0) | (np.abs(np.diff(lo, axis=1)) > 1e-3), axis=1)
        sep &= gap_clear(o)
        assert np.array_equal(g["idx"][sep], o["idx"][sep]), "tie rule violated"


def sample_rows(N, extra, seed):
    """One row of every 32-token block (at a position that walks through the
    block from one block to the next) plus `extra` seeded random rows."""
    nb = (N + 31) // 32
    per_block = np.minimum(np.arange(nb) * 32 + (np.arange(nb) * 13 + 5) % 32, N - 1)
    rnd = np.random.default_rng(seed).choice(N, size=min(extra, N), replace=False)
    return np.unique(np.concatenate([per_block, rnd]))


def route_packed_full(X_np, cfg, gate):
    """Route all rows of X in the launch configuration the benchmark times:
    weights packed once, workspace for all N tokens."""
    X = R.to_device(X_np, DEV)
    d = [R.to_device(a, DEV) for a in cfg.weights(0)]
    nbytes = R.workspace_bytes(False, R.MORE_DT_BF16, X_np.shape[0], cfg.h, cfg.r, cfg.M, cfg.k, gate,
                               d[2] is not None)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    R.pack_lowrank(*d, ws)
    g = to_np(R.route_lowrank_packed(X, cfg.r, cfg.M, cfg.k, gate, ws))
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("gate", [CF.GATE_TOPK_SOFTMAX, CF.GATE_FULL_SOFTMAX])
def test_headline_full_size(oracle_lib, full_tokens, gate):
    """Headline workload at full size (N = 262144 seeded tokens, h = 2048,
    M = 4096, r = 32, k = 8, bias) in the launch configuration the benchmark
    times.  Every row is checked for the properties that need no oracle; the
    oracle checks one row of every 32-token block plus 8192 random rows, so an
    error in which block a wave reads or writes shows up wherever it falls."""
    cfg = CF.HEADLINE
    say(f"full size gate={gate}: generating the {cfg.N} seeded tokens")
    X = full_tokens(cfg)
    say(f"full size gate={gate}: GPU on all tokens")
    g = route_packed_full(X, cfg, gate)
    properties(g, cfg.k, cfg.M, gate == CF.GATE_FULL_SOFTMAX, "full-size")
    rows = sample_rows(cfg.N, 8192, 17)
    R1, R2, b = cfg.weights(0)
    say(f"full size gate={gate}: oracle on {rows.size} sampled rows")
    o = oracle_lib.route_lowrank(X[rows], R1, R2, b, cfg.k, gate)
    sub = {key: (None if v is None else v[rows]) for key, v in g.items()}
    at = oracle_lib.logits_at(X[rows], R1, R2, b, sub["idx"])
    res = compare(o, sub, cfg.k, gate == CF.GATE_FULL_SOFTMAX, 2e-4, "full-size", at)
    say(f"full size gate={gate}: ok {res}")


def test_many_experts_prefill_full_size(oracle_lib, full_tokens):
    """Many-expert prefill at full size (N = 65536, h = 4096, M = 65536, r = 64,
    k = 16, full-softmax gate): enough 32-token blocks that every wave of the
    persistent grid routes several of them.  Properties on every row; the
    oracle on one row of every 8th block plus 512 random rows."""
    cfg = CF.MANY_PREFILL
    say("many-expert prefill full size: generating tokens")
    X = full_tokens(cfg)
    say("many-expert prefill full size: GPU on all tokens")
    g = route_packed_full(X, cfg, CF.GATE_FULL_SOFTMAX)
    properties(g, cfg.k, cfg.M, True, "many-prefill-full")
    rows = np.unique(np.concatenate([sample_rows(cfg.N, 512, 23)[::8], [cfg.N - 1]]))
    R1, R2, b = cfg.weights(0)
    say(f"many-expert prefill full size: oracle on {rows.size} rows")
    o = oracle_lib.route_lowrank(X[rows], R1, R2, b, cfg.k, CF.GATE_FULL_SOFTMAX)
    sub = {key: (None if v is None else v[rows]) for key, v in g.items()}
    at = oracle_lib.logits_at(X[rows], R1, R2, b, sub["idx"])
    res = compare(o, sub, cfg.k, True, 2e-4, "many-prefill-full", at)
    say(f"many-expert prefill full size: ok {res}")
