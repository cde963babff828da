"""GPU parity of the expert dispatch (more_dispatch_sort) against the oracle.

Paper: "MoRE: Scaling mixture of experts with hardware-aware low-rank routing",
App. E, Fig. 9 (sort + count after the router).  Integer work: the sorted
experts, the slot order (stable, hence unique) and the offsets must equal the
oracle's bit for bit.
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


def say(msg):
    print(f"[dispatch] {msg}", flush=True)
    sys.stdout.flush()


def run_sort(idx, M):
    t = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).to(DEV)
    out = R.dispatch_sort(t, M)
    torch.cuda.synchronize()
    return {key: v.cpu().numpy() for key, v in out.items()}


def check(oracle_lib, idx, M, label):
    say(f"{label}: N={idx.shape[0]} k={idx.shape[1]} M={M}")
    g = run_sort(idx, M)
    o = oracle_lib.dispatch_sort(idx, M)
    for key in ("sorted_expert", "sorted_slot", "offsets"):
        assert np.array_equal(g[key], o[key]), f"{label}: {key} differs at {np.nonzero(g[key] != o[key])[0][:5]}"
    say(f"{label}: ok")


@pytest.mark.parametrize("N,M,k", [
    (1, 4096, 8),          # a single token
    (1000, 4096, 8),       # one pass, one block
    (8192 // 8 + 3, 4096, 8),   # just over one block of 8192 entries
    (5000, 64, 4),         # one pass, few experts: repeated digits in every round
    (5000, 65, 4),         # one pass, M not a power of two
    (5000, 4097, 4),       # two passes, the second with one live bit
    (3000, 1, 1),          # a single expert
    (20000, 65536, 16),    # two passes, 40 blocks (blocks spread over the XCDs)
    (777, 1 << 24, 3),     # two full 12-bit passes, the largest M
    (4096 + 1, 300, 7),    # ragged
    (16384, 4096, 4),      # 8 blocks: one per XCD
])
def test_dispatch_shapes(oracle_lib, N, M, k):
    idx = I.make_expert_sets(2, 61, N, M, k)
    check(oracle_lib, idx, M, f"N{N}-M{M}-k{k}")


def test_dispatch_one_set_for_every_token(oracle_lib):
    """Degenerate load: every token picks the same k experts."""
    N, M, k = 30000, 4096, 8
    row = np.array([4000, 3, 17, 2048, 5, 4095, 0, 99], np.int32)
    check(oracle_lib, np.tile(row, (N, 1)), M, "one-set")


def test_dispatch_full_size_headline(oracle_lib):
    """The headline workload's shape: N = 262144 tokens, k = 8, M = 4096, with
    the skewed expert load of a biased router."""
    cfg = CF.HEADLINE
    idx = I.make_expert_sets(0, 62, cfg.N, cfg.M, cfg.k)
    check(oracle_lib, idx, cfg.M, "headline")


def test_dispatch_of_router_output():
    """The router's own indices (headline shape, 8192 tokens) go straight in:
    the result is a stable expert ordering of exactly those slots, and the
    offsets delimit each expert's run (properties that fix it uniquely)."""
    cfg = CF.HEADLINE
    X = R.to_device(cfg.x_rows(0, 0, 8192, n_total=cfg.N), DEV)
    R1, R2, b = (R.to_device(a, DEV) for a in cfg.weights(0))
    routed = R.route_lowrank(X, R1, R2, b, cfg.k, 0)
    out = R.dispatch_sort(routed["idx"], cfg.M)
    torch.cuda.synchronize()
    flat = routed["idx"].cpu().numpy().reshape(-1)
    se, ss, off = (out[key].cpu().numpy() for key in ("sorted_expert", "sorted_slot", "offsets"))
    assert np.array_equal(np.sort(ss), np.arange(flat.size))
    assert np.array_equal(se, flat[ss])
    assert np.all(np.diff(se) >= 0)
    assert np.all(np.diff(ss)[np.diff(se) == 0] > 0)
    assert off[0] == 0 and off[-1] == flat.size
    assert np.array_equal(np.diff(off), np.bincount(flat, minlength=cfg.M))


def test_dispatch_rejects_bad_arguments():
    t = torch.zeros((4, 2), dtype=torch.int32, device=DEV)
    with pytest.raises(R.MoreError):
        R.dispatch_sort(t, 1)                     # k = 2 > M = 1
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(R.MoreError) as e:
        R.dispatch_sort(t, 4096, workspace=small)
    assert e.value.code == R.MORE_ERR_WORKSPACE


@pytest.mark.parametrize("M", [300, 5000])
def test_dispatch_out_of_range_entries_stay_in_bounds(M):
    """Entries outside [0, M) have no defined place in the order (the header
    says so), but the call must still write only inside its outputs: the
    slots stay a permutation of 0 .. N k - 1.  With one pass (M <= 4096) the
    offsets come from the digit counts (such entries count in the last
    expert), so they stay a non-decreasing cover of 0 .. N k and every
    in-range entry is still found under its own expert, in increasing slot
    order."""
    N, k = 3000, 4
    idx = I.make_expert_sets(2, 65, N, M, k)
    rng = np.random.default_rng(7)
    bad = rng.random(idx.shape) < 0.05
    idx = np.where(bad, np.where(rng.random(idx.shape) < 0.5, -3, M + 5), idx).astype(np.int32)
    say(f"out-of-range entries: N={N} k={k} M={M} bad={int(bad.sum())}")
    g = run_sort(idx, M)
    flat = idx.reshape(-1)
    ss, off = g["sorted_slot"], g["offsets"]
    assert np.array_equal(np.sort(ss), np.arange(flat.size))
    if M > 4096:
        say("ok (several passes: slots only)")
        return
    assert off[0] == 0 and off[-1] == flat.size and np.all(np.diff(off) >= 0)
    ok = (flat >= 0) & (flat < M)
    for e in np.unique(flat[ok])[:50]:
        run = ss[off[e]:off[e + 1]]
        mine = np.nonzero(flat == e)[0]
        assert np.all(np.isin(mine, run)), f"expert {e}: a slot is missing from its run"
        assert np.all(np.diff(run[np.isin(run, mine)]) > 0)
    say("ok")
