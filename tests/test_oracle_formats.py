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


# ----------------------------------------------------------------------------
# MXFP4 (OCP microscaling: E2M1 elements, one E8M0 scale per 32 elements)
# ----------------------------------------------------------------------------
def test_e2m1_table_matches_the_format_value_list():
    """The OCP MX specification lists the E2M1 magnitudes for codes 0..7 as
    0, 0.5, 1, 1.5, 2, 3, 4, 6; codes 8..15 are their negatives."""
    from oracle import E2M1_TABLE
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert E2M1_TABLE[:8].tolist() == mags
    assert (-E2M1_TABLE[8:]).tolist() == mags
    assert np.signbit(E2M1_TABLE[8])


def test_e2m1_table_matches_torch_through_e4m3fn():
    """Every E2M1 value is an e4m3fn value: move the sign, exponent (bias 1 ->
    bias 7) and mantissa (1 bit -> top of 3) fields into an e4m3fn byte and
    let torch decode it."""
    from oracle import E2M1_TABLE
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        if e == 0:      # subnormal E2M1: 0 or 0.5 = 2^-1 (e4m3 exponent field 6)
            byte = (s << 7) | ((6 << 3) if m else 0)
        else:
            byte = (s << 7) | ((e - 1 + 7) << 3) | (m << 2)
        ref = torch.tensor([byte], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).item()
        assert E2M1_TABLE[c] == ref, c


def test_e8m0_decode_matches_torch_all_codes():
    from oracle import e8m0_to_f64
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    ours = e8m0_to_f64(codes)
    nan = np.isnan(ref)
    assert nan.tolist() == [False] * 255 + [True]
    assert np.array_equal(np.isnan(ours), nan) and np.array_equal(ours[~nan], ref[~nan])


def test_mxfp4_record_layout_by_hand():
    """Slot 5 of a hand-built record: element i has code i % 16 (element 2j
    in the low nibble of byte j), the four 32-element groups have scale codes
    127, 128, 126, 130."""
    from oracle import mxfp4_record_rows
    rec = np.zeros(128 * 64 + 128 * 4, dtype=np.uint8)
    codes = np.arange(128) % 16
    rec[5 * 64:6 * 64] = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    rec[128 * 64 + 5 * 4:128 * 64 + 6 * 4] = [127, 128, 126, 130]
    vals = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    vals = vals + [-v for v in vals]
    exp = np.array([vals[i % 16] * [1.0, 2.0, 0.5, 8.0][i // 32] for i in range(128)])
    got = mxfp4_record_rows(rec[None, :], [5])[0]
    assert np.array_equal(got, exp)
    assert np.array_equal(mxfp4_record_rows(rec[None, :], [4])[0], np.zeros(128) * 2.0 ** 0)


def test_mxfp4_quantizer_round_trip_and_error_bound():
    """The generator's MXFP4 conversion, decoded by the oracle: values already
    on the grid come back exactly; others are within the grid spacing."""
    from oracle import mxfp4_record_rows, E2M1_TABLE
    from synthetic.gen import to_mxfp4_rows, mxfp4_pool_to_records
    rng = np.random.default_rng(3)
    # exact: random codes with one +-4 or +-6 per 32-group, random shared exponents
    codes = rng.integers(0, 16, size=(128, 128))
    codes[:, ::32] = rng.choice([6, 7, 14, 15], size=(128, 4))
    X = rng.integers(-20, 20, size=(128, 4))
    vals = E2M1_TABLE[codes] * np.repeat(np.ldexp(1.0, X), 32, axis=1)
    rec = mxfp4_pool_to_records(to_mxfp4_rows(vals.astype(np.float32))[None, None])[0, 0]
    got = mxfp4_record_rows(np.repeat(rec[None], 128, axis=0), np.arange(128))
    assert np.array_equal(got, vals)
    # bound: |x - q(x)| <= 2^X (half the largest spacing, 2) below saturation,
    # < 2^(X+1) in the saturated range (6, 8) x 2^X
    x = (rng.standard_normal((128, 128)) * rng.choice([1e-3, 1.0, 50.0], size=(128, 1))).astype(np.float32)
    rec = mxfp4_pool_to_records(to_mxfp4_rows(x)[None, None])[0, 0]
    got = mxfp4_record_rows(np.repeat(rec[None], 128, axis=0), np.arange(128))
    amax = np.abs(x.reshape(128, 4, 32)).max(axis=2)
    Xs = np.floor(np.log2(amax)) - 2
    bound = np.repeat(np.ldexp(1.0, Xs.astype(int) + 1), 32, axis=1)
    assert (np.abs(got - x) < bound).all()
    assert (np.abs(got) <= np.repeat(6.0 * np.ldexp(1.0, Xs.astype(int)), 32, axis=1)).all()


def test_mxfp4_q_row_layout_by_hand():
    """An MXFP4 proxy q row: 64 code bytes (element 2j in the low nibble of
    byte j), then the four scale bytes of its 32-element groups."""
    from oracle import mxfp4_q_rows
    codes = (np.arange(128) * 7) % 16
    row = np.concatenate([(codes[0::2] | (codes[1::2] << 4)).astype(np.uint8),
                          np.array([125, 127, 129, 131], np.uint8)])
    vals = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    vals = vals + [-v for v in vals]
    exp = np.array([vals[codes[i]] * [0.25, 1.0, 4.0, 16.0][i // 32] for i in range(128)])
    got = mxfp4_q_rows(np.stack([row, row])[None])      # [1, 2, 68] -> [1, 2, 128]
    assert got.shape == (1, 2, 128) and np.array_equal(got[0, 1], exp)
