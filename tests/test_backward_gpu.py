"""GPU parity of the backward pass (more_lowrank_backward_packed) against the
fp64 oracle.

Paper: "MoRE: Scaling mixture of experts with hardware-aware low-rank routing",
App. F.2.2 (eq. 10-12) and Algorithm 3.  The forward runs on the GPU first
(the balancing call, which returns lse); the selection fed to both sides is a
seeded synthetic one, so it does not come from the HIP path.

Tolerance per output tensor T: |T - T_oracle| <= rtol |T_oracle| + atol
max|T_oracle|.  X_grad is stored as bf16 (rtol 2^-8 covers its rounding);
R1_grad, R2_grad and bias_grad are fp32 sums of products whose operands enter
the MFMAs as bf16 hi + lo pairs (~2^-17 relative) with fp32 accumulation over
up to N terms of both signs: rtol 1e-3 and atol 1e-4 bound those errors with
a wide margin at the sizes tested.
"""
import sys

import numpy as np
import pytest
import torch

from rank_router_top_amd import configs as CF
from rank_router_top_amd import inputs as I
from rank_router_top_amd import route as R

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"
TOL = {"xbar": (2.0 ** -8, 1e-3), "r1bar": (1e-3, 1e-4), "r2bar": (1e-3, 1e-4), "bbar": (1e-3, 1e-4)}


def say(msg):
    print(f"[backward] {msg}", flush=True)
    sys.stdout.flush()


def run_gpu(X, R1, R2, b, idx, tv, pb, k):
    """Forward (balancing call, for lse) then backward on one packed workspace."""
    N, h = X.shape
    r, M = R2.shape
    nbytes = max(R.backward_workspace_bytes(R.MORE_DT_BF16, N, h, r, M, k),
                 R.balance_workspace_bytes(R.MORE_DT_BF16, N, h, r, M, min(k, 8)))
    assert nbytes > 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    d = [R.to_device(a, DEV) for a in (X, R1, R2, b)]
    R.pack_lowrank(d[1], d[2], d[3], ws)
    fwd = R.balance_lowrank_packed(d[0], r, M, min(k, 8), 0, ws)
    t_idx = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).to(DEV)
    t_tv = torch.from_numpy(np.ascontiguousarray(tv, dtype=np.float32)).to(DEV)
    t_pb = None if pb is None else torch.from_numpy(np.ascontiguousarray(pb, dtype=np.float32)).to(DEV)
    out = R.backward_lowrank_packed(d[0], d[1], d[2], t_idx, t_tv, t_pb, fwd["lse"], ws)
    torch.cuda.synchronize()
    return dict(xbar=out["X_grad"].float().cpu().numpy().astype(np.float64),
                r1bar=out["R1_grad"].cpu().numpy().astype(np.float64),
                r2bar=out["R2_grad"].cpu().numpy().astype(np.float64),
                bbar=out["bias_grad"].cpu().numpy().astype(np.float64))


def compare(o, g, label, scale=1.0):
    for key, (rtol, atol) in TOL.items():
        ref = scale * o[key] if key != "xbar" else o[key]
        err = np.abs(g[key] - ref)
        lim = rtol * np.abs(ref) + atol * np.max(np.abs(ref))
        worst = np.unravel_index(np.argmax(err - lim), err.shape)
        assert np.all(err <= lim), (f"{label}: {key} off at {worst}: gpu {g[key][worst]} oracle {ref[worst]} "
                                    f"(max rel err {np.max(err / np.maximum(np.abs(ref), 1e-30)):.3g})")
    say(f"{label}: ok (max |err| / max|ref|: " + ", ".join(
        f"{key} {np.max(np.abs(g[key] - (scale * o[key] if key != 'xbar' else o[key]))) / np.max(np.abs(o[key] if key == 'xbar' else scale * o[key])):.2e}"
        for key in TOL) + ")")


def check(oracle_lib, cfg_id, N, h, r, M, k, bias, pbar=True, label=""):
    X = I.make_x(0, cfg_id, N, h, I.DT_BF16, True)
    R1 = I.make_r1(0, cfg_id, h, r, I.DT_BF16)
    R2 = I.make_r2(0, cfg_id, r, M, I.DT_BF16)
    b = I.make_bias(0, cfg_id, M) if bias else None
    idx = I.make_expert_sets(0, cfg_id, N, M, k)
    tv, pb = I.make_grads(0, cfg_id, N, k, M)
    pb = pb if pbar else None
    say(f"{label}: N={N} h={h} r={r} M={M} k={k} bias={bias} pbar={pbar}")
    g = run_gpu(X, R1, R2, b, idx, tv, pb, k)
    o = oracle_lib.backward_lowrank(X, R1, R2, b, idx, tv, pb)
    compare(o, g, label)


@pytest.mark.parametrize("N,h,r,M,k,bias,pbar", [
    (2048 + 5, 2048, 32, 4096, 8, True, True),     # headline shape, reduced N
    (1024 + 77, 512, 32, 4096, 8, False, True),    # prefill h = 512, no bias
    (1024 + 1, 2048, 16, 4096, 8, True, True),     # rank 16
    (33, 256, 32, 1000, 4, True, True),            # ragged block and ragged expert tiles
    (1, 512, 32, 4096, 8, True, True),             # one token
    (700, 256, 32, 300, 32, True, False),          # k = 32, no balancing gradient
])
def test_backward_shapes(oracle_lib, N, h, r, M, k, bias, pbar):
    check(oracle_lib, 70, N, h, r, M, k, bias, pbar, f"N{N}-h{h}-r{r}-M{M}-k{k}")


def test_backward_full_size_headline(oracle_lib):
    """N = 262144 tokens at the headline shape, as 32 copies of one 8192-row
    block (with its selection and incoming gradients): the oracle on the block
    fixes everything -- every copy of a row has the block row's X_grad, and the
    weight and bias gradients are 32 times the block's."""
    cfg = CF.HEADLINE
    base, reps = 8192, cfg.N // 8192
    X = cfg.x_rows(0, 0, base, n_total=cfg.N)
    R1, R2, b = cfg.weights(0)
    idx = I.make_expert_sets(0, 71, base, cfg.M, cfg.k)
    tv, pb = I.make_grads(0, 71, base, cfg.k, cfg.M)
    say("full size: oracle on the base block")
    o = oracle_lib.backward_lowrank(X, R1, R2, b, idx, tv, pb)
    say("full size: GPU on the tiled batch")
    g = run_gpu(np.tile(X, (reps, 1)), R1, R2, b, np.tile(idx, (reps, 1)), np.tile(tv, (reps, 1)), pb, cfg.k)
    xb = g["xbar"].reshape(reps, base, -1)
    assert all(np.array_equal(xb[c], xb[0]) for c in range(1, reps))
    g["xbar"] = xb[0]
    compare(o, g, "full-size", scale=float(reps))


def test_backward_deterministic_bitwise(oracle_lib):
    X = I.make_x(0, 72, 3000, 512, I.DT_BF16, True)
    R1 = I.make_r1(0, 72, 512, 32, I.DT_BF16)
    R2 = I.make_r2(0, 72, 32, 4096, I.DT_BF16)
    b = I.make_bias(0, 72, 4096)
    idx = I.make_expert_sets(0, 72, 3000, 4096, 8)
    tv, pb = I.make_grads(0, 72, 3000, 8, 4096)
    g1 = run_gpu(X, R1, R2, b, idx, tv, pb, 8)
    g2 = run_gpu(X, R1, R2, b, idx, tv, pb, 8)
    for key in g1:
        assert np.array_equal(g1[key], g2[key]), key
