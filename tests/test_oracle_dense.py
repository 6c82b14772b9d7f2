"""The dense NVFP4 GEMV oracle against values fixed independently of it.

Pins: a matrix built value by value from the golden e2m1 / e4m3 tables
(tests/golden, typed from the formats' definitions) and packed by hand in
the canonical byte order, multiplied with numpy; a closed form (every weight
1.0 gives the row sums of x); the tensor scale's linearity; brute-force
loops on a tiny case; the sign bit.
"""

import numpy as np
import pytest

from conftest import read_golden

import oracle



def _e2m1_table():
    return {int(c): float(v) for c, v in read_golden("e2m1_values.txt")}


def _e4m3_spots():
    out = {}
    for hexbyte, v in read_golden("e4m3_spot_values.txt"):
        f = float(v)
        if np.isfinite(f):
            out[int(hexbyte, 16)] = f
    return out


def _pack_nibbles(codes):
    """Canonical order, written out here: element 2j -> low nibble of byte j."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def _bf16_bits(x):
    """Round-to-nearest-even float -> bf16 bits (test helper, numpy only)."""
    f = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((f + 0x7FFF + ((f >> 16) & 1)) >> 16).astype(np.uint16)
    return r


def _random_case(rng, n, k, b, scale_bytes):
    table = _e2m1_table()
    codes = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    sbytes = rng.choice(scale_bytes, size=(n, k // 16)).astype(np.uint8)
    spots = _e4m3_spots()
    w = np.array([[table[int(c)] for c in row] for row in codes], dtype=np.float64)
    w *= np.repeat(np.array([[spots[int(s)] for s in row] for row in sbytes]), 16, axis=1)
    x_bits = _bf16_bits(rng.standard_normal((b, k)))
    x = (x_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return codes, sbytes, w, x_bits, x


def test_hand_built_matrix_matches_numpy_matmul():
    rng = np.random.default_rng(1)
    scale_bytes = [b for b in _e4m3_spots() if b not in (0x00, 0x80)]
    codes, sbytes, w, x_bits, x = _random_case(rng, 24, 96, 3, scale_bytes)
    ts = 0.375
    y = oracle.dense_gemv(_pack_nibbles(codes), sbytes, ts, x_bits)
    want = x @ (w * ts).T
    np.testing.assert_allclose(y, want, rtol=1e-13, atol=1e-13 * np.abs(want).max())


def test_unit_weights_give_row_sums():
    rng = np.random.default_rng(2)
    n, k, b = 8, 64, 4
    codes = np.full((n, k), 2, dtype=np.uint8)             # e2m1 code 2 = 1.0
    sbytes = np.full((n, k // 16), 0x38, dtype=np.uint8)   # e4m3 0x38 = 1.0
    x_bits = _bf16_bits(rng.standard_normal((b, k)))
    x = (x_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    y = oracle.dense_gemv(_pack_nibbles(codes), sbytes, 1.0, x_bits)
    np.testing.assert_allclose(y, np.repeat(x.sum(axis=1, keepdims=True), n, axis=1), rtol=1e-14, atol=1e-12)


def test_tensor_scale_is_linear_and_sign_bit_negates():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 8, size=(6, 32), dtype=np.uint8)      # non-negative codes
    sbytes = np.full((6, 2), 0x40, dtype=np.uint8)
    x_bits = _bf16_bits(rng.standard_normal((2, 32)))
    y1 = oracle.dense_gemv(_pack_nibbles(codes), sbytes, 1.5, x_bits)
    y2 = oracle.dense_gemv(_pack_nibbles(codes), sbytes, 3.0, x_bits)
    np.testing.assert_array_equal(y2, 2.0 * y1)
    yneg = oracle.dense_gemv(_pack_nibbles(codes | 8), sbytes, 1.5, x_bits)
    np.testing.assert_array_equal(yneg, -y1)


def test_brute_force_tiny():
    rng = np.random.default_rng(4)
    table, spots = _e2m1_table(), _e4m3_spots()
    scale_bytes = sorted(b for b in spots if b not in (0x00, 0x80))
    n, k, b = 3, 32, 2
    codes = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    sbytes = rng.choice(scale_bytes, size=(n, k // 16)).astype(np.uint8)
    x_bits = _bf16_bits(rng.standard_normal((b, k)))
    xv = (x_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    y = oracle.dense_gemv(_pack_nibbles(codes), sbytes, 2.0, x_bits)
    for bb in range(b):
        for r in range(n):
            s = 0.0
            for c in range(k):
                s += table[int(codes[r, c])] * spots[int(sbytes[r, c // 16])] * 2.0 * xv[bb, c]
            assert abs(y[bb, r] - s) <= 1e-12 * max(1.0, abs(s))
