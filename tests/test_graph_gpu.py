"""The whole routing call (more_route_lowrank) captured in a HIP graph.

Under capture the call forks the packing of the sweep operands onto a side
stream and joins it back with events (a per-call ready token would be
replayed unchanged).  The graph is replayed several times, with the
program's own eager work and synchronisations between the replays, and every
replay must give the eager call's outputs bit for bit (integer indices and
the same floating-point arithmetic in the same order).  (App. F.1,
Algorithm 1: the top-k values and indices are the call's contract.)
"""
import sys

import pytest
import torch

from rank_router_top_amd import configs as CF
from rank_router_top_amd import route as R

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"


def say(msg):
    print(f"[graph] {msg}", flush=True)
    sys.stdout.flush()


def test_whole_call_graph_replays_match_eager():
    cfg = CF.HEADLINE
    n = 32 * 1024 + 7
    X = R.to_device(cfg.x_rows(0, 0, n, n_total=cfg.N), DEV)
    d = [R.to_device(a, DEV) for a in cfg.weights(0)]
    nbytes = R.workspace_bytes(False, R.MORE_DT_BF16, n, cfg.h, cfg.r, cfg.M, cfg.k, 0, True)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    say(f"eager call: N={n}")
    ref = R.route_lowrank(X, *d, cfg.k, 0, workspace=ws)
    torch.cuda.synchronize()
    assert R.route_status(ws) == R.MORE_OK
    ref = {key: v.clone() for key, v in ref.items() if v is not None}
    out = {key: torch.empty_like(v) for key, v in ref.items()}
    out.setdefault("logit", None)
    say("capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        R.route_lowrank(X, *d, cfg.k, 0, out=out, workspace=ws, stream=s)
    torch.cuda.synchronize()
    for rep in range(4):
        for v in out.values():
            if v is not None:
                v.fill_(-7)              # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert R.route_status(ws) == R.MORE_OK
        for key, v in ref.items():
            assert torch.equal(out[key], v), f"replay {rep}: {key} differs"
        say(f"replay {rep}: ok")
