"""Pins of the oracle's storage-format decoding against library casts and the
OCP FP8 definition (tests/golden/e4m3fn_spot_values.json)."""
import json
import os

import numpy as np
import torch

from oracle import E4M3FN_TABLE, bf16_to_f64, e4m3fn_to_f64, dequant, FP8
from synthetic.gen import to_bf16_bits, to_e4m3fn_bits

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_decode_matches_torch_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3fn_table_matches_torch_all_patterns():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(E4M3FN_TABLE), nan)
    assert np.array_equal(E4M3FN_TABLE[~nan], ref[~nan])
    assert np.array_equal(np.signbit(E4M3FN_TABLE[~nan]), np.signbit(ref[~nan]))


def test_e4m3fn_spot_values_from_the_format_definition():
    g = json.load(open(os.path.join(GOLD, "e4m3fn_spot_values.json")))
    for hexbyte, val in g["values"].items():
        got = e4m3fn_to_f64(np.array([int(hexbyte, 16)], dtype=np.uint8))[0]
        assert got == val and np.signbit(got) == np.signbit(val), hexbyte
    for hexbyte in g["nan"]:
        assert np.isnan(e4m3fn_to_f64(np.array([int(hexbyte, 16)], dtype=np.uint8))[0])


def test_fp8_dequant_applies_per_head_scale():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 3, 16)).astype(np.float32) * np.array([1.0, 10.0, 0.01], np.float32)[None, :, None]
    bits, scale = to_e4m3fn_bits(x, head_axis=1)
    v = dequant(bits, FP8, scale, head_axis=1)
    # every head's amax maps to the largest finite code
    for h in range(3):
        assert np.isclose(np.abs(v[:, h]).max(), float(np.float32(scale[h])) * 448.0)
    # relative error of e4m3 rounding is at most 2^-4 for normal values
    rel = np.abs(v - x) / np.maximum(np.abs(x), 1e-30)
    normal = np.abs(x) / scale[None, :, None] >= 2.0 ** -6
    assert rel[normal].max() <= 2.0 ** -4 + 1e-12


def test_bf16_rounding_is_nearest_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1.0
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.0], dtype=np.float32)
    got = bf16_to_f64(to_bf16_bits(x))
    assert got.tolist() == [1.0, 1.0 + 2.0 ** -6, -2.0]
