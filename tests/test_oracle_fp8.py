"""Pins for the FP8 (E4M3) cache oracle: the encoding against torch's own float8_e4m3fn
conversion, the rounding bound, scale invariance, and lossless attention for values on the
E4M3 grid.  CPU only."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8
from tests.helpers import paged_from_contiguous


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_encode(y):
    return torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_of_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = fp8.e4m3_decode(codes), _torch_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref)) and np.isnan(ours).sum() == 2
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_encode_matches_torch_inside_the_range():
    rng = np.random.default_rng(11)
    grid = fp8.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))          # 0 .. 448, ascending
    mids = (grid[:-1] + grid[1:]) / 2                                     # exact ties
    y = np.concatenate([
        grid, mids, np.nextafter(mids.astype(np.float32), np.float32(0)), np.nextafter(mids.astype(np.float32), np.float32(1e9)),
        rng.standard_normal(20000) * 3, rng.standard_normal(5000) * 0.004,   # typical and subnormal range
        rng.uniform(-448, 448, 5000), [0.0, -0.0, 1e-30, -1e-30],
    ]).astype(np.float32)
    y = np.concatenate([y, -y])
    y = y[np.abs(y) <= 448]
    np.testing.assert_array_equal(fp8.e4m3_encode(y), _torch_encode(y))


def test_encode_saturates_and_keeps_nan():
    codes = fp8.e4m3_encode(np.array([448.0, 460.0, 1e6, np.inf, -1e6, -np.inf, np.nan], np.float32))
    np.testing.assert_array_equal(codes[:6], [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE])
    assert codes[6] & 0x7F == 0x7F


def test_round_trip_error_bound():
    rng = np.random.default_rng(12)
    y = np.concatenate([rng.uniform(2.0 ** -6, 448, 20000), -rng.uniform(2.0 ** -6, 448, 2000)]).astype(np.float32)
    back = fp8.e4m3_decode(fp8.e4m3_encode(y))
    assert (np.abs(back - y) <= 2.0 ** -4 * np.abs(y)).all()          # half a unit in the last place
    sub = rng.uniform(-2.0 ** -6, 2.0 ** -6, 5000).astype(np.float32)
    assert (np.abs(fp8.e4m3_decode(fp8.e4m3_encode(sub)) - sub) <= 2.0 ** -10).all()


@pytest.mark.parametrize("k", [-3, -1, 0, 2, 4])
def test_power_of_two_scales_are_exact(k):
    rng = np.random.default_rng(13)
    x = (rng.uniform(-20, 20, 4000)).astype(np.float32)
    np.testing.assert_array_equal(fp8.quantize(x * np.float32(2.0 ** k), 2.0 ** k), fp8.quantize(x, 1.0))


@pytest.mark.parametrize("scale", [0.25, 1.0, 8.0])
def test_attention_over_grid_values_is_lossless(scale):
    """K/V on the E4M3 grid times kv_scale store exactly; attention over the stored codes then
    equals plain attention over the original values (the read undoes the store)."""
    rng = np.random.default_rng(14)
    H, Hkv, D, BS = 4, 2, 16, 4
    grid = fp8.e4m3_decode(rng.integers(0, 0x7F, size=(2, 2, 40, Hkv, D)).astype(np.uint8))
    grid *= np.where(rng.random(grid.shape) < 0.5, -1.0, 1.0) * scale
    ks = [grid[0, 0, :23], grid[0, 1, :40]]
    vs = [grid[1, 0, :23], grid[1, 1, :40]]
    cache, table = paged_from_contiguous(ks, vs, BS, rng, extra_blocks=2)
    codes = fp8.quantize(cache, scale)
    np.testing.assert_array_equal(fp8.dequantize(codes, scale), cache)
    q = rng.standard_normal((2, H, D)) * 0.05
    lens = np.array([23, 40])
    np.testing.assert_array_equal(oracle.decode(q, fp8.dequantize(codes, scale), table, lens, 0.3, Hkv),
                                  oracle.decode(q, cache, table, lens, 0.3, Hkv))


def test_store_writes_quantized_rows_and_skips_negative_slots():
    rng = np.random.default_rng(15)
    codes = np.zeros((2, 3, 4, 2, 8), np.uint8)
    k = rng.standard_normal((3, 2, 8)).astype(np.float32)
    v = rng.standard_normal((3, 2, 8)).astype(np.float32)
    out = fp8.store_kv_fp8(codes, k, v, np.array([5, -1, 11]), 0.5)
    np.testing.assert_array_equal(out[0, 1, 1], fp8.quantize(k[0], 0.5))
    np.testing.assert_array_equal(out[1, 2, 3], fp8.quantize(v[2], 0.5))
    assert out.sum() == out[:, 1, 1].sum() + out[:, 2, 3].sum()
    # the stored value is x / kv_scale up to rounding: decode * kv_scale is back near x
    np.testing.assert_allclose(fp8.dequantize(out[0, 1, 1], 0.5), k[0], rtol=2.0 ** -4, atol=2.0 ** -10)
