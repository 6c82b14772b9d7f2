"""Exact decoding of the stored number formats (oracle; test infrastructure).

Sources
  * "Frontier MoE on consumer Blackwell (SM120)", section "GLM-5.2 (753B) --
    the headline model": an NVFP4 tensor is e2m1 values times an e4m3 scale
    per 16-element block times one per-tensor fp32 scale ("scale_2").
  * "vLLM adds day-0 support for Recursive's Flint ...", section "A 40B MoE
    that activates 2.5B parameters": the checkpoint runs weight-only
    (W4A16) with BF16 activations.

Readings adopted where the pages name a format but do not spell it out
  * e2m1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; exponent
    field 0 is subnormal (0 or 0.5).  Code 8 is negative zero.
  * e4m3: the "FN" variant -- bias 7, no infinities, S.1111.111 is NaN,
    largest finite 448, smallest subnormal 2^-9.
  * block of 16 runs along the reduction (column) dimension of each row.
  * canonical byte order: element 2j of a row sits in the low nibble of
    byte j of that row, element 2j+1 in the high nibble; block scales are
    row-major [rows, cols/16].

All decoders return float64 and are exact (every value they produce is a
dyadic rational that float64 represents exactly).
"""

from __future__ import annotations

import numpy as np


def e2m1_value(code: int) -> float:
    """Value of one 4-bit e2m1 code, from its bit fields.

    sign = bit 3, exponent = bits 2..1 (bias 1), mantissa = bit 0.
    Exponent 0 is subnormal: value = mantissa * 0.5.
    """
    code = int(code)
    if not 0 <= code <= 15:
        raise ValueError("e2m1 code out of range")
    sign = -1.0 if (code >> 3) & 1 else 1.0
    exp = (code >> 1) & 3
    man = code & 1
    if exp == 0:
        mag = man * 0.5
    else:
        mag = (1.0 + 0.5 * man) * 2.0 ** (exp - 1)
    return sign * mag  # code 8 gives -0.0


def e4m3_value(byte: int) -> float:
    """Value of one e4m3 (FN variant) byte, from its bit fields.

    sign = bit 7, exponent = bits 6..3 (bias 7), mantissa = bits 2..0.
    Exponent 0 is subnormal: value = mantissa/8 * 2^-6.
    Exponent 15 with mantissa 7 is NaN; there are no infinities.
    """
    byte = int(byte)
    if not 0 <= byte <= 255:
        raise ValueError("e4m3 byte out of range")
    sign = -1.0 if (byte >> 7) & 1 else 1.0
    exp = (byte >> 3) & 15
    man = byte & 7
    if exp == 15 and man == 7:
        return float("nan")
    if exp == 0:
        mag = (man / 8.0) * 2.0 ** -6
    else:
        mag = (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return sign * mag


# Lookup arrays built by evaluating the bit-field definitions above on every
# possible code; the decoders below index them.
_E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
_E4M3 = np.array([e4m3_value(b) for b in range(256)], dtype=np.float64)

# Value pair of every code byte in canonical order: (low nibble, high nibble).
_E2M1_PAIR = np.stack([_E2M1[np.arange(256) & 15], _E2M1[np.arange(256) >> 4]], axis=1)

# The magnitudes codes 0..7 take under the definition, kept only so tests can
# compare the definition against a table typed by hand.
E2M1_MAGNITUDES_BY_DEFINITION = tuple(float(v) for v in _E2M1[:8])


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64.

    A bf16 number is the upper half of an IEEE binary32 number, so shifting
    the 16 bits into the top of a 32-bit word gives the same value.
    """
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):     # NaN patterns stay NaN
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def unpack_nibbles(packed) -> np.ndarray:
    """Canonical nibble order: byte j of a row holds element 2j (low nibble)
    and element 2j+1 (high nibble).  Returns uint8 codes [..., 2*n]."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def dequant_nvfp4(codes, scales, tensor_scale: float) -> np.ndarray:
    """Dequantise one NVFP4 matrix to float64.

    codes  : uint8 [R, K/2]  (canonical nibble order)
    scales : uint8 [R, K/16] e4m3 block scales, block b covers columns
             16b .. 16b+15 of its row
    tensor_scale : the matrix's fp32 per-tensor scale

    W[r, c] = e2m1(code[r, c]) * e4m3(scales[r, c // 16]) * tensor_scale
    ("Frontier MoE on consumer Blackwell (SM120)", section "GLM-5.2").
    """
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    R, half_k = codes.shape
    K = 2 * half_k
    if scales.shape != (R, K // 16) or K % 16:
        raise ValueError("scale shape does not match codes")
    vals = _E2M1_PAIR[codes].reshape(R, K // 16, 16)        # element values, by block
    blk = _E4M3[scales][:, :, None]                         # one scale per block
    return (vals * blk * float(np.float32(tensor_scale))).reshape(R, K)


def dequant_bf16(bits) -> np.ndarray:
    """BF16 weight matrix (uint16 bit patterns) to float64, exactly."""
    return bf16_bits_to_f64(bits)
