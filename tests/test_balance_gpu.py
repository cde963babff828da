"""GPU parity of the balancing statistics (more_lowrank_balance_packed)
against the fp64 oracle.

Paper: "MoRE: Scaling mixture of experts with hardware-aware low-rank routing",
App. F.2.1 (Algorithm 2; eq. 6, 7, 9) and App. G.1 (H_norm).

Tolerances, derived from the arithmetic of the HIP path:
  * routing outputs (indices, gates, logits, lse): the parity rule of
    tests/parity.py, as for the routing call.
  * psum: each P_{n,i} = exp(l - lse) carries the logit and lse errors (about
    1e-5 absolute: fp32 accumulation of exact bf16 products, z at ~2^-17)
    plus a few ulp of exp2, so each term is within ~2e-5 relative, and fp32
    accumulation of at most N terms adds < N * 2^-24 relative in the worst
    case (the per-slot sums hold N / 256 terms): |d psum_i| <= 2e-4 psum_i
    + 1e-7 N.
  * counts: bit-exact on tokens the gap rule calls clear; a token the rule
    excludes may move up to k entries between experts on each side, so
    sum |d counts| <= 2 k * (excluded tokens).  The counts are always exactly
    the bincount of the returned indices.
  * L_bal, H_norm: within what the psum tolerance and the count freedom above
    allow (derived in check_stats), plus fp32 output rounding.
"""
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
PSUM_REL = 2e-4
PSUM_ABS_PER_TOKEN = 1e-7


def say(msg):
    print(f"[balance] {msg}", flush=True)
    sys.stdout.flush()


def run_balance(X, R1, R2, b, k, gate, n_ws=None):
    """Pack the weights, then one balancing call on a workspace sized for
    n_ws tokens (default: the batch)."""
    N, h = X.shape
    r, M = R2.shape
    n_ws = N if n_ws is None else n_ws
    nbytes = R.balance_workspace_bytes(R.MORE_DT_BF16, n_ws, h, r, M, k)
    assert nbytes > 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    d = [R.to_device(a, DEV) for a in (X, R1, R2, b)]
    R.pack_lowrank(d[1], d[2], d[3], ws)
    out = R.balance_lowrank_packed(d[0], r, M, k, gate, ws)
    torch.cuda.synchronize()
    return {key: (None if v is None else v.cpu().numpy()) for key, v in out.items()}


def check_psum(ps_o, ps_g, N, label):
    err = np.abs(ps_g.astype(np.float64) - ps_o)
    tol = PSUM_REL * ps_o + PSUM_ABS_PER_TOKEN * N
    worst = int(np.argmax(err - tol))
    assert np.all(err <= tol), (f"{label}: psum off at expert {worst}: gpu {ps_g[worst]} oracle {ps_o[worst]}")
    assert abs(float(ps_g.astype(np.float64).sum()) - N) <= PSUM_REL * N + 1e-3, f"{label}: sum psum != N"


def check_counts(cnt_o, cnt_g, idx_g, k, excluded, label):
    M = cnt_o.shape[0]
    assert np.array_equal(cnt_g, np.bincount(idx_g.reshape(-1), minlength=M)), f"{label}: counts != bincount(idx)"
    diff = int(np.abs(cnt_g.astype(np.int64) - cnt_o).sum())
    assert diff <= 2 * k * excluded, f"{label}: counts differ by {diff} with {excluded} excluded tokens"
    return diff


def check_stats(o, g, N, k, count_diff, label):
    """L_bal = M/(N^2 k) sum c_i psum_i: the psum tolerance moves it by at most
    PSUM_REL L + M/(N^2 k) sum c_i 1e-7 N, and each moved count by at most
    M/(N^2 k) max psum.  H_norm = (log C - (1/C) sum c log c)/log M, C = N k:
    one count moved by one changes it by at most (log C + 1)/(C log M)."""
    M = o["psum"].shape[0]
    C = N * k
    l_tol = (PSUM_REL * o["lbal"] + M / (N * N * k) * (C * PSUM_ABS_PER_TOKEN * N
             + count_diff * float(o["psum"].max())) + 2e-6 * max(1.0, o["lbal"]))
    assert abs(float(g["stats"][0]) - o["lbal"]) <= l_tol, f"{label}: L_bal {g['stats'][0]} vs {o['lbal']}"
    h_tol = (count_diff * (math.log(C) + 1) / (C * math.log(M)) if M > 1 else 0.0) + 2e-6
    assert abs(float(g["stats"][1]) - o["hnorm"]) <= h_tol, f"{label}: H_norm {g['stats'][1]} vs {o['hnorm']}"


def check_balance(oracle_lib, X, R1, R2, b, k, gate, label, n_ws=None):
    say(f"{label}: N={X.shape[0]} h={X.shape[1]} r={R1.shape[1]} M={R2.shape[1]} k={k} gate={gate} "
        f"bias={b is not None}")
    g = run_balance(X, R1, R2, b, k, gate, n_ws)
    o = oracle_lib.balance_lowrank(X, R1, R2, b, k, gate)
    N = X.shape[0]
    at = oracle_lib.logits_at(X, R1, R2, b, g["idx"])
    res = compare(o, g, k, gate == R.MORE_GATE_FULL_SOFTMAX, 2e-4, label, at)
    lerr = np.abs(g["lse"].astype(np.float64) - o["lse"])
    assert np.all(lerr <= 1e-4 * np.maximum(1.0, np.abs(o["lse"]))), f"{label}: lse off"
    check_psum(o["psum"], g["psum"], N, label)
    diff = check_counts(o["counts"], g["counts"], g["idx"], k, res["excluded"], label)
    check_stats(o, g, N, k, diff, label)
    say(f"{label}: ok {res} count moves {diff} L_bal {g['stats'][0]:.6f} H_norm {g['stats'][1]:.6f}")
    return o, g


CASES = [
    (CF.HEADLINE, 2048 + 5, CF.GATE_TOPK_SOFTMAX),
    (CF.HEADLINE, 1024 + 77, CF.GATE_FULL_SOFTMAX),
    (CF.PREFILL_H512, 2048 + 99, CF.GATE_TOPK_SOFTMAX),
    (CF.RANK16, 1024 + 1, CF.GATE_TOPK_SOFTMAX),
    (CF.PREFILL_H512, 1024 + 31, CF.GATE_FULL_SOFTMAX),
]


@pytest.mark.parametrize("cfg,n,gate", CASES, ids=[f"{c.name}-{n}-g{g}" for c, n, g in CASES])
def test_balance_configs(oracle_lib, cfg, n, gate):
    X = cfg.x_rows(0, 0, n, n_total=cfg.N)
    R1, R2, b = cfg.weights(0)
    check_balance(oracle_lib, X, R1, R2, b, cfg.k, gate, cfg.name)


@pytest.mark.parametrize("N,h,r,M,k,bias", [
    (1, 256, 32, 4096, 8, True),       # a single token
    (300, 256, 32, 6000, 8, True),     # M past the earlier LDS-staged bias limit, ragged last tile
    (200, 256, 16, 20000, 4, True),    # M past the bias-descending order's limit (index order)
    (33, 512, 16, 1000, 4, True),      # ragged block, ragged expert tiles (padding positions)
    (700, 256, 32, 1000, 8, False),    # no bias: plain two passes
    (64, 128, 16, 8, 8, True),         # k = M: every expert selected by every token
    (300, 128, 48, 200, 1, True),      # r = 48 (three 16-rank blocks, padded to four), k = 1
    (96, 256, 64, 5888, 8, True),      # the largest M of the envelope at k = 8
    (200, 1024, 64, 4096, 8, True),    # r = 64 at the largest h of the envelope
    (96, 256, 32, 14720, 4, True),     # the largest M of the envelope at k = 4
])
def test_balance_edge_shapes(oracle_lib, N, h, r, M, k, bias):
    seed = 7
    X = I.make_x(seed, 41, N, h, I.DT_BF16, True)
    R1 = I.make_r1(seed, 41, h, r, I.DT_BF16)
    R2 = I.make_r2(seed, 41, r, M, I.DT_BF16)
    b = I.make_bias(seed, 41, M) if bias else None
    for gate in (CF.GATE_TOPK_SOFTMAX, CF.GATE_FULL_SOFTMAX):
        check_balance(oracle_lib, X, R1, R2, b, k, gate, f"edge-N{N}-r{r}-M{M}-k{k}-b{int(bias)}")


def test_balance_planted_dispatch():
    """Thm. 4 planted construction (r = M = 64, R1 = R2 = I on the first 64
    input dimensions): each expert is selected by exactly k tokens, so counts
    are k, H_norm = 1 and every psum_i = 1 (closed form, no oracle)."""
    M, k, h = 64, 8, 64
    rho = math.sqrt(1.0 / k + 1.0 / (M - k))
    a, c = 1.0 / (k * rho), -1.0 / ((M - k) * rho)
    Xf = np.full((M, h), c, np.float32)
    for n in range(M):
        Xf[n, [(n + j) % M for j in range(k)]] = a
    eye = np.eye(h, M, dtype=np.float32)
    g = run_balance(I.f32_to_bf16_bits(Xf), I.f32_to_bf16_bits(eye), I.f32_to_bf16_bits(np.eye(M, dtype=np.float32)),
                    None, k, CF.GATE_TOPK_SOFTMAX)
    assert np.array_equal(g["counts"], np.full(M, k))
    # the bf16 inputs are the rounded a and c: P depends on them only through
    # the two-valued logits, so psum_i = 1 still holds exactly in real numbers
    assert np.allclose(g["psum"], 1.0, rtol=0, atol=1e-5)
    assert abs(float(g["stats"][1]) - 1.0) < 1e-6
    assert abs(float(g["stats"][0]) - 1.0) < 1e-5


def test_balance_deterministic_bitwise():
    """Fixed summation order: two calls on the same inputs give the same bits."""
    cfg = CF.HEADLINE
    X = cfg.x_rows(0, 0, 3000, n_total=cfg.N)
    R1, R2, b = cfg.weights(0)
    g1 = run_balance(X, R1, R2, b, cfg.k, 0)
    g2 = run_balance(X, R1, R2, b, cfg.k, 0)
    for key in ("idx", "gate", "lse", "psum", "counts", "stats"):
        assert np.array_equal(g1[key], g2[key]), key


def test_balance_rejects_outside_envelope():
    cfg = CF.HEADLINE
    X = torch.zeros((64, 256), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    with pytest.raises(R.MoreError) as e:
        R.balance_lowrank_packed(X, 32, 4096, 16, 0, ws)          # k = 16 > 8
    assert e.value.code == R.MORE_ERR_UNSUPPORTED
    with pytest.raises(R.MoreError) as e:
        R.balance_lowrank_packed(X, 128, 4096, 8, 0, ws)          # r = 128 > 64
    assert e.value.code == R.MORE_ERR_UNSUPPORTED
    X2 = torch.zeros((64, 2048), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(R.MoreError) as e:
        R.balance_lowrank_packed(X2, 64, 4096, 8, 0, ws)          # r = 64 at h = 2048: R1 too large
    assert e.value.code == R.MORE_ERR_UNSUPPORTED
    small = torch.empty(4096, dtype=torch.uint8, device=DEV)
    with pytest.raises(R.MoreError) as e:
        R.balance_lowrank_packed(X, 32, 4096, 8, 0, small)        # workspace too small
    assert e.value.code == R.MORE_ERR_WORKSPACE
    assert cfg.k == 8


def test_balance_full_size_headline(oracle_lib):
    """Headline shape at full size (N = 262144, h = 2048, M = 4096, r = 32,
    k = 8, bias), in the launch configuration the benchmark times (workspace
    for all N tokens).  The batch repeats one 8191-row block of the seeded
    tokens (an odd period, so no copy lines up with the 32-token blocks or the
    persistent grid's strides; the last copy is cut at N).  The oracle on that
    block fixes the whole result: psum and counts are 32 x the block's plus
    those of its first 32 rows, L_bal and H_norm follow from them; every copy
    of a row must give the same indices, gates and lse."""
    cfg = CF.HEADLINE
    base_n = 8191
    reps = -(-cfg.N // base_n)
    tail = cfg.N - (reps - 1) * base_n
    Xb = cfg.x_rows(0, 0, base_n, n_total=cfg.N)
    R1, R2, b = cfg.weights(0)
    say("full size: oracle on the base block")
    o = oracle_lib.balance_lowrank(Xb, R1, R2, b, cfg.k, 0)
    ot = oracle_lib.balance_lowrank(Xb[:tail], R1, R2, b, cfg.k, 0)
    say("full size: GPU on the tiled batch")
    g = run_balance(np.tile(Xb, (reps, 1))[:cfg.N], R1, R2, b, cfg.k, 0)
    N = cfg.N
    for key in ("idx", "gate", "lse", "logit"):
        v = g[key]
        for c in range(1, reps):
            n0 = c * base_n
            n1 = min(n0 + base_n, N)
            assert np.array_equal(v[n0:n1], v[:n1 - n0]), f"copy {c} differs in {key}"
    first = {key: v[:base_n] for key, v in g.items() if key in ("idx", "gate", "logit", "lse")}
    res = compare(o, first, cfg.k, False, 2e-4, "full-size block", oracle_lib.logits_at(Xb, R1, R2, b, first["idx"]))
    full_copies = reps - 1
    ps_o = full_copies * o["psum"] + ot["psum"]
    cnt_o = full_copies * o["counts"] + ot["counts"]
    check_psum(ps_o, g["psum"], N, "full-size")
    excl_tail = int((~gap_clear(ot)).sum())
    diff = check_counts(cnt_o, g["counts"], g["idx"], cfg.k, full_copies * res["excluded"] + excl_tail, "full-size")
    lbal, hnorm = oracle_lib.balance_stats(ps_o, cnt_o, N, cfg.k)
    ob = dict(o, psum=ps_o, counts=cnt_o, lbal=lbal, hnorm=hnorm)
    check_stats(ob, g, N, cfg.k, diff, "full-size")
    say(f"full size: ok {res} count moves {diff}")


@pytest.mark.parametrize("spread", [30.0, 90.0])
def test_balance_wide_bias_spread(oracle_lib, spread):
    """Biases spread over +-spread/2 (natural log units): at 90 the spread of
    a wave's experts exceeds the range where the psum sweep factors the bias
    out of the exponentials (100 log2 units), so that wave takes the
    unfactored form; both must match the oracle."""
    N, h, r, M, k = 500, 256, 32, 4096, 8
    X = I.make_x(5, 42, N, h, I.DT_BF16, True)
    R1 = I.make_r1(5, 42, h, r, I.DT_BF16)
    R2 = I.make_r2(5, 42, r, M, I.DT_BF16)
    rng = np.random.default_rng(17)
    b = (rng.uniform(-0.5, 0.5, M) * spread).astype(np.float32)
    for gate in (CF.GATE_TOPK_SOFTMAX, CF.GATE_FULL_SOFTMAX):
        check_balance(oracle_lib, X, R1, R2, b, k, gate, f"bias-spread-{spread:g}")
