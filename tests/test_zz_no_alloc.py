"""The allocation-free dispatch sort (more_dispatch_sort_noalloc, for callers
that cannot allocate device memory) against more_dispatch_sort with a
workspace, through the C ABI.

Three calls in a row on the library's one static scratch, each smaller than
the one before, so every call after the first runs on scratch that an earlier
call left behind: the headline shape (N = 262144, k = 8, M = 4096, one pass),
a ragged shape, and one with M > 4096 (two passes through the key and slot
buffers).
Integer work: every output must equal the workspace variant's bit for bit.
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
KEYS = ("sorted_expert", "sorted_slot", "offsets")


def say(msg):
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


def test_noalloc_sort_matches_workspace_sort():
    cfg = CF.HEADLINE
    cases = [(cfg.N, cfg.k, cfg.M, 62), (4096 + 1, 7, 300, 63), (3000, 4, 65536, 64)]
    for N, k, M, stream_id in cases:
        say(f"N={N} k={k} M={M}")
        idx = torch.from_numpy(np.ascontiguousarray(I.make_expert_sets(3, stream_id, N, M, k), np.int32)).to(DEV)
        ref = R.dispatch_sort(idx, M)
        got = R.dispatch_sort_noalloc(idx, M)
        torch.cuda.synchronize()
        for key in KEYS:
            a, b = ref[key].cpu().numpy(), got[key].cpu().numpy()
            assert np.array_equal(a, b), f"N={N} k={k} M={M}: {key} differs at {np.nonzero(a != b)[0][:5]}"
        say(f"N={N} k={k} M={M}: ok")


def test_noalloc_sort_rejects_beyond_its_scratch():
    """N k = 2^22 entries at M = 65536 (two passes: counts plus the key and
    slot buffers) need more than the 32 MiB scratch: the call returns
    MORE_ERR_SCRATCH_LIMIT and enqueues nothing."""
    N, k, M = 1 << 19, 8, 65536
    assert R.dispatch_workspace_bytes(N, k, M) > 32 << 20
    idx = torch.zeros((N, k), dtype=torch.int32, device=DEV)
    with pytest.raises(R.MoreError) as e:
        R.dispatch_sort_noalloc(idx, M)
    assert e.value.code == R.MORE_ERR_SCRATCH_LIMIT
