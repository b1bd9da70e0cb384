"""Pins for the oracle's storage decoders and the generator's encoders."""
import math

import numpy as np
import pytest
import torch

from oracle.formats import bf16_bits_to_f64, e4m3_bits_to_f64
from workloads.generate import f32_to_bf16_bits, f32_to_e4m3_bits


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_bits_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan_ours, nan_ref = np.isnan(ours), np.isnan(ref)
    assert (nan_ours == nan_ref).all()
    assert nan_ours.sum() == 2  # S.1111.111 only
    np.testing.assert_array_equal(ours[~nan_ours], ref[~nan_ref])
    # signed zeros are kept
    assert math.copysign(1.0, ours[0x80]) == -1.0


@pytest.mark.parametrize("code,value", [
    (0x7E, 448.0), (0xFE, -448.0), (0x38, 1.0), (0xB8, -1.0), (0x08, 2.0 ** -6),
    (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x40, 2.0), (0x3C, 1.5), (0x00, 0.0),
])
def test_e4m3_hand_values(code, value):
    assert e4m3_bits_to_f64(np.array([code], np.uint8))[0] == value


def test_bf16_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    assert bf16_bits_to_f64(np.array([0x3F80], np.uint16))[0] == 1.0
    assert bf16_bits_to_f64(np.array([0xC000], np.uint16))[0] == -2.0


def test_generator_bf16_is_round_nearest_even():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200000).astype(np.float32)
    # exact ties: values halfway between two bf16 neighbours
    base = np.array([1.0, 1.0078125, -3.0, 0.5], np.float32).view(np.uint32)
    ties = (base + np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties])
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins
    assert f32_to_bf16_bits(np.array([1.0 + 2.0 ** -8], np.float32))[0] == 0x3F80


def test_generator_e4m3_roundtrip_and_saturation():
    grid = e4m3_bits_to_f64(np.arange(256, dtype=np.uint8))
    finite = grid[np.isfinite(grid)].astype(np.float32)
    back = e4m3_bits_to_f64(f32_to_e4m3_bits(finite))
    np.testing.assert_array_equal(back, finite.astype(np.float64))
    assert e4m3_bits_to_f64(f32_to_e4m3_bits(np.array([1e6, -1e6], np.float32))).tolist() == [448.0, -448.0]
    # nearest rounding: 1.0625 lies halfway between 1.0 and 1.125 -> even (1.0)
    assert e4m3_bits_to_f64(f32_to_e4m3_bits(np.array([1.0625, 1.07], np.float32))).tolist() == [1.0, 1.125]
