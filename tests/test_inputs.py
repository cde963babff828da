"""The seeded input generator: determinism, row-prefix stability, distributions, rounding."""
import numpy as np
import pytest
import torch

from rank_router_top_amd import configs as CF
from rank_router_top_amd import inputs as I


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(7)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40], np.float32)]).astype(np.float32)
    # include exact halfway cases: low 16 bits == 0x8000
    u = rng.integers(0, 2 ** 31, 1000, dtype=np.uint32) & np.uint32(0xFFFF0000) | np.uint32(0x8000)
    u = u[((u >> 23) & 0xFF) != 0xFF]          # finite values only
    a = np.concatenate([a, u.view(np.float32), -u.view(np.float32)])
    ours = I.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = I.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_x_is_deterministic_and_prefix_stable():
    a = I.make_x(0, 9, 10000, 64, I.DT_BF16, True)
    b = I.make_x(0, 9, 10000, 64, I.DT_BF16, True)
    assert np.array_equal(a, b)
    # a row prefix or a window never depends on the rest of the batch
    assert np.array_equal(I.make_x(0, 9, 300, 64, I.DT_BF16, True), a[:300])
    assert np.array_equal(I.make_x(0, 9, 10000, 64, I.DT_BF16, True, row0=4000, n_rows=5000), a[4000:9000])
    # other seed / config / tensor -> other values
    assert not np.array_equal(I.make_x(1, 9, 300, 64, I.DT_BF16, True), a[:300])
    assert not np.array_equal(I.make_x(0, 8, 300, 64, I.DT_BF16, True), a[:300])


def test_decode_rows_are_prefill_prefix():
    dec = CF.MANY_DECODE.x_rows(0)
    pre = CF.MANY_PREFILL.x_rows(0, 0, 256)
    assert dec.shape == (256, 4096) and np.array_equal(dec, pre)


def test_rms_normalised_rows():
    x = I.to_f64(I.make_x(3, 9, 512, 2048, I.DT_BF16, True), I.DT_BF16)
    ms = np.mean(x * x, axis=1)
    assert np.all(np.abs(ms - 1.0) < 5e-3)   # bf16 rounding only
    xr = I.to_f64(I.make_x(3, 9, 512, 2048, I.DT_F32, False), I.DT_F32)
    assert abs(np.mean(xr * xr) - 1.0) < 0.01 and abs(np.mean(xr)) < 0.01


@pytest.mark.parametrize("h,r,M", [(512, 32, 4096), (2048, 16, 1024)])
def test_weight_variances(h, r, M):
    R1 = I.to_f64(I.make_r1(0, 9, h, r, I.DT_BF16), I.DT_BF16)
    R2 = I.to_f64(I.make_r2(0, 9, r, M, I.DT_BF16), I.DT_BF16)
    assert abs(R1.var() * h - 1.0) < 0.05
    assert abs(R2.var() * r - 1.0) < 0.05
    b = I.make_bias(0, 9, 65536)
    assert b.dtype == np.float32 and abs(b.var() - 0.5) < 0.02


def test_config_table():
    h = CF.HEADLINE
    assert (h.N, h.h, h.M, h.r, h.k) == (262144, 2048, 4096, 32, 8) and h.has_bias
    assert CF.TINY.dtype == I.DT_F32 and not CF.TINY.rms_norm and CF.TINY.k == 4
    assert CF.RANK64.x_cfg == h.x_cfg and CF.FULLRANK.fullrank
    assert CF.MANY_PREFILL.gates == (CF.GATE_FULL_SOFTMAX,) and CF.MANY_DECODE.N == 256
    assert h.flops() == 2 * 262144 * (2048 * 32 + 32 * 4096)
