"""Pins for the oracle's number-format decoding (CPU only).

Each test compares the oracle against something other than itself: a table
typed by hand, torch's float8 / bfloat16 casts (library routines), or a
structural property of the definition.
"""

import math

import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle import formats as F


def _golden_e2m1():
    return {int(c): float(v) for c, v in read_golden("e2m1_values.txt")}


def test_e2m1_definition_matches_hand_table():
    table = _golden_e2m1()
    assert sorted(table) == list(range(16))
    for code, want in table.items():
        got = F.e2m1_value(code)
        assert got == want
        assert math.copysign(1.0, got) == math.copysign(1.0, want), code  # -0 for code 8


def test_e2m1_magnitudes_monotone_and_symmetric():
    mags = [F.e2m1_value(c) for c in range(8)]
    assert all(a < b for a, b in zip(mags, mags[1:]))
    for c in range(8):
        assert F.e2m1_value(c + 8) == -F.e2m1_value(c)


def test_e4m3_matches_torch_on_all_256_bytes():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([F.e4m3_value(i) for i in range(256)])
    nan_ref, nan_got = np.isnan(ref), np.isnan(got)
    assert (nan_ref == nan_got).all()
    assert list(np.nonzero(nan_got)[0]) == [0x7F, 0xFF]
    assert (ref[~nan_ref] == got[~nan_got]).all()
    assert (np.signbit(ref[~nan_ref]) == np.signbit(got[~nan_got])).all()


def test_e4m3_spot_values():
    for hexbyte, want in read_golden("e4m3_spot_values.txt"):
        got = F.e4m3_value(int(hexbyte, 16))
        if want == "nan":
            assert math.isnan(got)
        else:
            assert got == float(want), hexbyte
            assert math.copysign(1, got) == math.copysign(1, float(want))


def test_e4m3_positive_bytes_strictly_increasing():
    vals = [F.e4m3_value(b) for b in range(0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:]))


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = F.bf16_bits_to_f64(bits)
    same = (ref == got) | (np.isnan(ref) & np.isnan(got))
    assert same.all()


def test_nibble_order_low_nibble_first():
    # byte 0x21 holds element 0 = code 1 (low nibble) and element 1 = code 2
    codes = F.unpack_nibbles(np.array([[0x21, 0xF0]], dtype=np.uint8))
    assert codes.tolist() == [[1, 2, 0, 15]]


@pytest.mark.parametrize("g", [1.0, 2.0, 0.5, 0.7])
def test_dequant_brute_force_all_code_scale_pairs(g):
    """Every (code, scale byte) product, against the hand e2m1 table times
    torch's e4m3 decode times the tensor scale."""
    e2m1 = _golden_e2m1()
    # one row per scale byte; 16 columns = codes 0..15 in element order
    row_codes = np.array([(2 * j) | ((2 * j + 1) << 4) for j in range(8)], dtype=np.uint8)
    codes = np.tile(row_codes, (256, 1))
    scales = np.arange(256, dtype=np.uint8).reshape(256, 1)
    w = F.dequant_nvfp4(codes, scales, g)
    s_ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()
    g32 = float(np.float32(g))
    for sb in range(256):
        for c in range(16):
            want = e2m1[c] * s_ref[sb] * g32
            got = w[sb, c]
            if math.isnan(want):
                assert math.isnan(got)
            else:
                assert got == want, (sb, c)


def test_dequant_block_index_runs_along_columns():
    # codes all 1.0 (nibble 2 -> byte 0x22); 4 blocks with distinct scales
    codes = np.full((3, 32), 0x22, dtype=np.uint8)   # K = 64
    scales = np.array([[0x38, 0x40, 0x30, 0x00]] * 3, dtype=np.uint8)  # 1, 2, 0.5, 0
    w = F.dequant_nvfp4(codes, scales, 1.0)
    want = np.repeat(np.array([1.0, 2.0, 0.5, 0.0]), 16)
    assert (w == want[None, :]).all()


def test_dequant_rejects_bad_scale_shape():
    with pytest.raises(ValueError):
        F.dequant_nvfp4(np.zeros((2, 8), np.uint8), np.zeros((2, 2), np.uint8), 1.0)
