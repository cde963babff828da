"""A bounded wait that gives up must surface as an error, never as MORE_OK
with stale outputs.

The persistent routing kernels hand work between their waves through bounded
waits.  A tiny spin limit set from the host (more_set_spin_limit, a testing
aid) makes those waits give up on the first miss: every wave still exits
normally, and more_route_status must report MORE_ERR_STALLED for the
workspace.  With the default limit the same call must report MORE_OK and
match the oracle.  (App. F.1, Algorithm 1: the top-k values and indices are
the kernel's contract, so a call that could not compute them must say so.)
"""
import sys

import numpy as np
import pytest
import torch

from rank_router_top_amd import configs as CF
from rank_router_top_amd import route as R

from oracle.parity import compare

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"


def say(msg):
    print(f"[stall] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture
def spin_limit():
    yield R.set_spin_limit
    R.set_spin_limit(0)


@pytest.fixture
def route_paths():
    yield R.set_route_paths
    R.set_route_paths(None)


@pytest.mark.parametrize("path", ["split", "ring", "pc"])
def test_tiny_spin_limit_reports_stall(oracle_lib, spin_limit, route_paths, path):
    route_paths(path)
    cfg = CF.HEADLINE
    n = 32 * 1024 + 7
    Xn = cfg.x_rows(0, 0, n, n_total=cfg.N)
    R1, R2, b = cfg.weights(0)
    X = R.to_device(Xn, DEV)
    d = [R.to_device(a, DEV) for a in (R1, R2, b)]
    nbytes = R.workspace_bytes(False, R.MORE_DT_BF16, n, cfg.h, cfg.r, cfg.M, cfg.k, 0, True)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    R.pack_lowrank(*d, ws)
    assert R.route_status(ws) == R.MORE_OK
    say(f"tiny spin limit: path {path}, N={n}")
    spin_limit(1)
    R.route_lowrank_packed(X, cfg.r, cfg.M, cfg.k, 0, ws)
    assert R.route_status(ws) == R.MORE_ERR_STALLED
    # the word is cleared by the check
    assert R.route_status(ws) == R.MORE_OK
    say("default spin limit")
    spin_limit(0)
    g = R.route_lowrank_packed(X, cfg.r, cfg.M, cfg.k, 0, ws)
    assert R.route_status(ws) == R.MORE_OK
    g = {key: (None if v is None else v.cpu().numpy()) for key, v in g.items()}
    o = oracle_lib.route_lowrank(Xn, R1, R2, b, cfg.k, 0)
    at = oracle_lib.logits_at(Xn, R1, R2, b, g["idx"])
    say(f"ok {compare(o, g, cfg.k, False, 2e-4, 'after-stall', at)}")


def test_whole_call_tiny_spin_limit_reports_stall(oracle_lib, spin_limit):
    """The whole routing call (more_route_lowrank): the sweep operands are
    packed on a side stream and the routing kernel waits for their ready word
    with a bounded wait.  With a tiny spin limit the call's waits give up and
    the stall word says so; with the default limit the call is exact."""
    cfg = CF.HEADLINE
    n = 32 * 1024 + 7
    Xn = cfg.x_rows(0, 0, n, n_total=cfg.N)
    R1, R2, b = cfg.weights(0)
    X = R.to_device(Xn, DEV)
    d = [R.to_device(a, DEV) for a in (R1, R2, b)]
    nbytes = R.workspace_bytes(False, R.MORE_DT_BF16, n, cfg.h, cfg.r, cfg.M, cfg.k, 0, True)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    say(f"whole call, tiny spin limit: N={n}")
    spin_limit(1)
    R.route_lowrank(X, *d, cfg.k, 0, workspace=ws)
    assert R.route_status(ws) == R.MORE_ERR_STALLED
    say("whole call, default spin limit")
    spin_limit(0)
    g = R.route_lowrank(X, *d, cfg.k, 0, workspace=ws)
    assert R.route_status(ws) == R.MORE_OK
    g = {key: (None if v is None else v.cpu().numpy()) for key, v in g.items()}
    o = oracle_lib.route_lowrank(Xn, R1, R2, b, cfg.k, 0)
    at = oracle_lib.logits_at(Xn, R1, R2, b, g["idx"])
    say(f"ok {compare(o, g, cfg.k, False, 2e-4, 'whole-call', at)}")
