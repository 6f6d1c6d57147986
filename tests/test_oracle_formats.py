"""Pins for the oracle's number-format decoders and the e4m3 quantiser,
checked against sources other than the oracle itself: torch's own
float8_e4m3fn / bfloat16 casts (every code), the OCP E2M1 value table, and
the defining inequalities of round-to-nearest."""

import numpy as np
import pytest
import torch

from oracle import formats as fm


def test_e4m3_decode_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = fm.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert fm.e4m3_decode(np.uint8(0x7E)) == 448.0
    assert np.isnan(fm.e4m3_decode(np.uint8(0x7F)))


def test_e2m1_decode_matches_ocp_table():
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    ours = fm.e2m1_decode(np.arange(16))
    assert list(ours[:8]) == table
    assert list(ours[8:]) == [-v for v in table]


def test_e8m0_decode():
    assert fm.e8m0_decode(np.uint8(127)) == 1.0
    assert fm.e8m0_decode(np.uint8(0)) == 2.0 ** -127
    assert fm.e8m0_decode(np.uint8(254)) == 2.0 ** 127
    assert np.isnan(fm.e8m0_decode(np.uint8(255)))


def test_unpack_fp4_low_nibble_first():
    packed = np.array([[0x21, 0x8F]], dtype=np.uint8)
    assert fm.unpack_fp4(packed).tolist() == [[1, 2, 15, 8]]


def test_bf16_bits_roundtrip_matches_torch():
    g = torch.Generator().manual_seed(1)
    v = torch.randn(4096, generator=g, dtype=torch.float32) * 10
    bits = v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours_bits = fm.f64_to_bf16_bits(v.numpy().astype(np.float64))
    assert np.array_equal(bits, ours_bits)
    assert np.array_equal(fm.bf16_bits_to_f64(bits), v.to(torch.bfloat16).to(torch.float64).numpy())


def test_e4m3_round_matches_torch_in_range():
    g = torch.Generator().manual_seed(2)
    v = (torch.randn(20000, generator=g, dtype=torch.float64) * 60).clamp(-448, 448)
    # include exact midpoints between neighbouring codes (ties)
    grid = fm.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (grid[:-1] + grid[1:]) / 2
    v = np.concatenate([v.numpy(), mids, -mids])
    ours = fm.e4m3_round(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_round_saturates():
    assert fm.e4m3_round(np.array([1e6, -1e6, 449.0, 470.0])).tolist() == [448.0, -448.0, 448.0, 448.0]


def test_e4m3_round_is_nearest():
    v = np.linspace(-448, 448, 100001)
    r = fm.e4m3_round(v)
    grid = fm.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    full = np.concatenate([-grid[::-1], grid])
    best = np.abs(v[:, None] - full[None, :]).min(axis=1)
    assert np.allclose(np.abs(r - v), best, rtol=0, atol=1e-12)


@pytest.mark.parametrize("v,expect", [(1.0, 1.0), (1.5, 2.0), (0.3, 0.5), (448.0, 512.0),
                                      (2.0 ** -20, 2.0 ** -20), (3.0 * 2 ** -30, 2.0 ** -28)])
def test_pow2_at_least(v, expect):
    assert fm.pow2_at_least(v) == expect
