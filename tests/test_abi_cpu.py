"""The C-ABI library: loads without a GPU, exports what include/more_route.h
declares, and rejects bad arguments on the host before any HIP call."""
import ctypes as C
import os
import re

import pytest

from rank_router_top_amd import route as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "more_route.h")

pytestmark = pytest.mark.skipif(not os.path.exists(R.LIB_PATH),
                                reason="libmore_route.so not built (python -m rank_router_top_amd.build)")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(more_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(R.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = C.CDLL(R.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


def test_version_and_status_strings():
    assert R.lib().more_abi_version() == 1
    for code in range(10):
        s = R.status_str(code)
        assert s and s != "unknown status"
    assert R.status_str(99) == "unknown status"


def test_workspace_size_is_pure_host_and_rejects_bad_args():
    packed = R.workspace_bytes(False, R.MORE_DT_BF16, 0, 2048, 32, 4096, 8, 0, True)
    # packed R1 in two operand layouts (2 x 128 KiB) + packed R2 (256 KiB) + bias
    # operands + sweep order
    assert 2 * 128 * 1024 + 256 * 1024 <= packed < 2 * 128 * 1024 + 256 * 1024 + 128 * 1024
    # plus token scratch: z of every 32-token block as bf16 hi + lo (4 bytes per token and rank)
    ws = R.workspace_bytes(False, R.MORE_DT_BF16, 262144, 2048, 32, 4096, 8, 0, True)
    assert ws == packed + 262144 * 32 * 4
    # few tokens (at most 64 blocks of 32): the split-M form's scratch instead,
    # when larger: 8 K-part partial sums of z (fp32, 4 KiB per block and 32
    # ranks) and, per shard of 4 expert tiles (32 shards at M = 4096), k
    # candidate logits, indices and gates and one log-sum-exp per token
    parts = 8 * 2 * 4096
    cand = 32 * 33 * 8 * 4
    lse = (32 * 33 * 4 + 255) // 256 * 256
    assert R.workspace_bytes(False, R.MORE_DT_BF16, 33, 2048, 32, 4096, 8, 0, True) == packed + parts + 3 * cand + lse
    assert R.workspace_bytes(False, R.MORE_DT_F32, 1000, 2048, 32, 4096, 8, 0, True) == \
        R.workspace_bytes(False, R.MORE_DT_F32, 0, 2048, 32, 4096, 8, 0, True)   # fp32: no two-kernel path
    assert ws % 256 == 0 and packed % 256 == 0
    assert R.workspace_bytes(True, R.MORE_DT_BF16, 100, 2048, 0, 4096, 8, 0, True) >= 2048 * 4096 * 2
    assert R.workspace_bytes(False, R.MORE_DT_BF16, 1, 2048, 24, 4096, 8, 0, False) == 0   # r % 16
    assert R.workspace_bytes(False, R.MORE_DT_BF16, 1, 2044, 32, 4096, 8, 0, False) == 0   # h % 8
    assert R.workspace_bytes(False, R.MORE_DT_BF16, 1, 2048, 32, 4096, 33, 0, False) == 0  # k
    assert R.workspace_bytes(False, 7, 1, 2048, 32, 4096, 8, 0, False) == 0                # dtype


FAKE = C.c_void_p(0x1000)     # aligned non-null host address: never dereferenced on error paths
ODD = C.c_void_p(0x1004)


def call_lowrank(dt=0, X=FAKE, N=64, h=64, R1=FAKE, r=16, R2=FAKE, M=32, bias=None, k=4, gate=0,
                 idx=FAKE, g=FAKE, logit=None, lse=None, ws=FAKE, ws_bytes=1 << 20):
    return R.lib().more_route_lowrank(dt, X, N, h, R1, r, R2, M, bias, k, gate, idx, g, logit, lse,
                                      ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=5), 4), (dict(gate=3), 5), (dict(N=-1), 2), (dict(h=0), 2), (dict(M=0), 2),
    (dict(r=0), 2), (dict(k=0), 3), (dict(k=33), 3), (dict(k=40, M=39), 3), (dict(k=5, M=4), 3),
    (dict(h=60), 7), (dict(r=24), 7), (dict(r=144), 7), (dict(X=None), 1), (dict(R1=None), 1),
    (dict(R2=None), 1), (dict(idx=None), 1), (dict(g=None), 1), (dict(X=ODD), 9),
    (dict(idx=ODD), 9), (dict(ws=None), 6), (dict(ws_bytes=100), 6),
    (dict(ws=C.c_void_p(0x1010)), 6),
])
def test_lowrank_rejects_bad_arguments_before_any_hip_call(kw, code):
    assert call_lowrank(**kw) == code


def test_empty_batch_is_a_noop():
    assert call_lowrank(N=0, X=None, idx=None, g=None) == 0


def test_fullrank_workspace_covers_the_tiled_layout():
    """bf16 with k <= 8 and h a multiple of 64 runs the LDS-tiled kernel: W
    packed per 256-expert slab (h x 256 bf16 each) plus the bias in
    accumulator layout (256 fp32 per slab), past the plain layout's size."""
    bf = R.MORE_DT_BF16
    for h, M in ((2048, 4096), (128, 1000), (64, 192), (256, 513)):
        nslab = (M + 255) // 256
        need = nslab * 256 * h * 2 + nslab * 256 * 4
        for k in (1, 8):
            assert R.workspace_bytes(True, bf, 100, h, 0, M, k, 0, True) >= need
    # shapes of the plain kernel keep its own size
    assert R.workspace_bytes(True, bf, 100, 96, 0, 300, 8, 0, True) > 0
    assert R.workspace_bytes(True, bf, 100, 128, 0, 700, 16, 0, True) > 0


def test_topk_merge_validation():
    """The shard merge checks its arguments on the host: gate, shapes, k
    against the shard width and the last shard, and required pointers; N = 0
    is a no-op (no HIP call)."""
    f = R.lib().more_topk_merge
    FK = FAKE
    assert f(10, 4096, 512, 8, 7, FK, FK, None, FK, FK, None, None, None) == 5          # gate
    assert f(-1, 4096, 512, 8, 0, FK, FK, None, FK, FK, None, None, None) == 2          # N
    assert f(10, 4096, 0, 8, 0, FK, FK, None, FK, FK, None, None, None) == 2            # width
    assert f(10, 4096, 4, 8, 0, FK, FK, None, FK, FK, None, None, None) == 3            # k > width
    assert f(10, 1000, 300, 200, 0, FK, FK, None, FK, FK, None, None, None) == 3        # last shard 100 < k
    assert f(10, 4096, 512, 33, 0, FK, FK, None, FK, FK, None, None, None) == 3         # k > MORE_MAX_K
    assert f(10, 4096, 512, 8, 0, None, FK, None, FK, FK, None, None, None) == 1        # candidates
    assert f(10, 4096, 512, 8, 1, FK, FK, None, FK, FK, None, None, None) == 1          # full gate needs lse
    assert f(0, 4096, 512, 8, 0, None, None, None, None, None, None, None, None) == 0   # N = 0


def test_fullrank_rejects_bad_arguments():
    L = R.lib()
    f = L.more_route_fullrank
    assert f(0, FAKE, 64, 64, FAKE, 32, None, 33, 0, FAKE, FAKE, None, None, FAKE, 1 << 20, None) == 3
    assert f(0, FAKE, 64, 63, FAKE, 32, None, 4, 0, FAKE, FAKE, None, None, FAKE, 1 << 20, None) == 7
    assert f(0, None, 64, 64, FAKE, 32, None, 4, 0, FAKE, FAKE, None, None, FAKE, 1 << 20, None) == 1
    assert f(0, FAKE, 64, 64, FAKE, 32, None, 4, 0, FAKE, FAKE, None, None, FAKE, 16, None) == 6


def call_balance(dt=0, N=64, h=256, r=32, M=4096, k=8, gate=0, idx=FAKE, g=FAKE, logit=None, lse=FAKE,
                 psum=FAKE, counts=FAKE, stats=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return R.lib().more_lowrank_balance_packed(dt, FAKE, N, h, r, M, k, gate, idx, g, logit, lse, psum,
                                               counts, stats, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(k=16), 7), (dict(r=128), 7), (dict(dt=1), 7), (dict(M=65537), 7), (dict(M=65537, k=4), 7), (dict(M=14720, k=4, ws_bytes=100), 6),
    (dict(lse=None), 1), (dict(psum=None), 1), (dict(counts=None), 1), (dict(stats=None), 1),
    (dict(psum=ODD), 9), (dict(ws_bytes=100), 6), (dict(gate=2), 5), (dict(k=0), 3), (dict(h=60), 7),
])
def test_balance_rejects_bad_arguments_before_any_hip_call(kw, code):
    assert call_balance(**kw) == code


def test_balance_empty_batch_is_a_noop():
    assert call_balance(N=0, idx=None, g=None, lse=None, psum=None, counts=None, stats=None) == 0


def test_balance_workspace_bytes():
    """Packed weights + z scratch (4 bytes per token and rank) + per-slot
    partial sums: fp32 by sweep position and int32 by expert, one row per
    token slot (at most 256 slots, one per 32-token block below that)."""
    bf = R.MORE_DT_BF16
    route = R.workspace_bytes(False, bf, 262144, 2048, 32, 4096, 8, 0, True)
    assert R.balance_workspace_bytes(bf, 262144, 2048, 32, 4096, 8) == route + 2 * 256 * 4096 * 4
    packed = R.workspace_bytes(False, bf, 0, 2048, 32, 4096, 8, 0, True)
    # 33 tokens: z of 2 blocks (4 KiB each) and 2 partial-sum slots
    assert R.balance_workspace_bytes(bf, 33, 2048, 32, 4096, 8) == packed + 2 * 4096 + 2 * 2 * 4096 * 4
    assert R.balance_workspace_bytes(bf, 10, 2048, 32, 65535, 8) > 0
    assert R.balance_workspace_bytes(bf, 10, 2048, 32, 65537, 8) == 0    # 16-bit sweep positions
    assert R.balance_workspace_bytes(bf, 10, 2048, 32, 65535, 4) > 0
    assert R.balance_workspace_bytes(bf, 10, 2048, 32, 65537, 4) == 0
    assert R.balance_workspace_bytes(R.MORE_DT_F32, 10, 2048, 32, 4096, 8) == 0
    assert R.balance_workspace_bytes(bf, 10, 2048, 128, 4096, 8) == 0
    assert R.balance_workspace_bytes(bf, 10, 4608, 16, 4096, 8) > 0       # R1 resident in LDS
    assert R.balance_workspace_bytes(bf, 10, 4864, 16, 4096, 8) == 0
    assert R.balance_workspace_bytes(bf, 10, 1024, 64, 4096, 8) > 0       # R1 (128 KiB) + 3 z slots fit
    assert R.balance_workspace_bytes(bf, 10, 1056, 64, 4096, 8) == 0
    assert R.balance_workspace_bytes(bf, 10, 2048, 32, 4096, 9) == 0


def test_dispatch_workspace_and_validation():
    """Digit counts (min(M, 4096) per block of 8192 entries, plus one row of
    digit totals, 256-byte aligned) and, for more than one pass (M > 4096), a
    key and a slot buffer of N k entries."""
    assert R.dispatch_workspace_bytes(262144, 8, 4096) == 257 * 4096 * 4
    assert R.dispatch_workspace_bytes(1000, 4, 64) == 512
    assert R.dispatch_workspace_bytes(1000, 4, 300) == 2560                       # 2 x 300 ints, aligned
    assert R.dispatch_workspace_bytes(262144, 8, 4097) == 257 * 4096 * 4 + 2 * 262144 * 8 * 4
    assert R.dispatch_workspace_bytes(1000, 5, 4) == 0          # k > M
    assert R.dispatch_workspace_bytes(1 << 28, 8, 4096) == 0     # N k >= 2^31 - 1
    f = R.lib().more_dispatch_sort
    assert f(FAKE, 10, 4, 2, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == 3      # k > M
    assert f(None, 10, 4, 64, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == 1
    assert f(ODD, 10, 4, 64, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == 9
    assert f(FAKE, 10, 4, 64, FAKE, FAKE, FAKE, FAKE, 16, None) == 6
    assert f(FAKE, 0, 4, 64, None, None, None, None, 0, None) == 0            # N = 0: no-op
    assert f(FAKE, -1, 4, 64, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == 2


def test_dispatch_noalloc_rejects_before_any_hip_call():
    """The allocation-free sort checks its arguments like more_dispatch_sort,
    then its 32 MiB static scratch, before any HIP call."""
    f = R.lib().more_dispatch_sort_noalloc
    assert f(FAKE, 10, 4, 2, FAKE, FAKE, FAKE, None) == 3                   # k > M
    assert f(None, 10, 4, 64, FAKE, FAKE, FAKE, None) == 1
    assert f(ODD, 10, 4, 64, FAKE, FAKE, FAKE, None) == 9
    assert f(FAKE, 0, 4, 64, None, None, None, None) == 0                   # N = 0: no-op
    assert f(FAKE, -1, 4, 64, FAKE, FAKE, FAKE, None) == 2
    assert R.dispatch_workspace_bytes(1 << 19, 8, 65536) > 32 << 20
    assert f(FAKE, 1 << 19, 8, 65536, FAKE, FAKE, FAKE, None) == R.MORE_ERR_SCRATCH_LIMIT
    assert R.dispatch_workspace_bytes(1 << 22, 8, 4096) > 32 << 20
    assert f(FAKE, 1 << 22, 8, 4096, FAKE, FAKE, FAKE, None) == R.MORE_ERR_SCRATCH_LIMIT
    assert R.status_str(R.MORE_ERR_SCRATCH_LIMIT) != "unknown status"


def call_backward(dt=0, N=64, h=256, r=32, M=4096, k=8, idx=FAKE, tv=FAKE, pb=None, lse=FAKE, xg=FAKE,
                  r1g=FAKE, r2g=FAKE, bg=None, ws=FAKE, ws_bytes=100):
    return R.lib().more_lowrank_backward_packed(dt, FAKE, N, h, FAKE, r, FAKE, M, k, idx, tv, pb, lse, xg, r1g, r2g,
                                                bg, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(r=64), 7), (dict(r=128), 7), (dict(dt=1), 7), (dict(h=240), 7), (dict(M=20000), 7),
    (dict(lse=None), 1), (dict(xg=None), 1), (dict(r1g=None), 1), (dict(r2g=None), 1), (dict(idx=None), 1),
    (dict(tv=None), 1), (dict(xg=ODD), 9), (dict(pb=ODD), 9), (dict(k=33), 3), (dict(ws_bytes=100), 6),
])
def test_backward_rejects_bad_arguments_before_any_hip_call(kw, code):
    assert call_backward(**kw) == code


def test_backward_workspace_bytes():
    bf = R.MORE_DT_BF16
    assert R.backward_workspace_bytes(bf, 262144, 2048, 32, 4096, 8) > R.workspace_bytes(
        False, bf, 262144, 2048, 32, 4096, 8, 0, True)
    assert R.backward_workspace_bytes(bf, 100, 2048, 16, 4096, 32) > 0
    assert R.backward_workspace_bytes(bf, 100, 2048, 64, 4096, 8) == 0      # r > 32
    assert R.backward_workspace_bytes(bf, 100, 2048, 32, 16384, 8) > 0
    assert R.backward_workspace_bytes(bf, 100, 2048, 32, 16385, 8) == 0     # M > 16384
    assert R.backward_workspace_bytes(R.MORE_DT_F32, 100, 2048, 32, 4096, 8) == 0
