"""The sign-symmetric 2-bit expert codec (oracle; test infrastructure).

Source: "Frontier MoE on consumer Blackwell (SM120)", section "How it fits --
2-bit experts at FP4 quality": the routed experts are stored as 2-bit planes
whose codebook is forced to be sign-symmetric, {-4, -1, 1, 4}, and NVFP4
checkpoints are re-quantised to it at load after an exact float64
dequantisation; section "GLM-5.2 (753B)": an NVFP4 tensor is e2m1 codes times
an e4m3 scale per 16-element block times a per-tensor fp32 scale.

Readings (the page gives the codebook and the exact re-quantisation, not the
plane layout or how a block's scale is chosen):
  * A 2-bit matrix keeps NVFP4's scale structure and only narrows the codes:
    W[r, c] = LEVELS[q[r, c]] * e4m3(s[r, c // 16]) * tensor_scale with
    LEVELS = (-4, -1, 1, 4) for q = 0, 1, 2, 3.
  * Canonical byte order: byte j of a row holds elements 4j .. 4j+3, element
    4j+i in bits 2i, 2i+1.
  * Re-quantising an NVFP4 matrix keeps its tensor scale.  Each 16-element
    block is dequantised exactly without it (v = e2m1 * e4m3) and gets the
    non-negative finite e4m3 scale (bytes 0x00 .. 0x7E) whose levels fit it
    with the least squared error sum_i (v_i - LEVELS[q_i] * s)^2, summed in
    element order in float64; every q_i is the level nearest to v_i / s, an
    element exactly halfway between 1 and 4 (|v| = 2.5 s) takes 1, and the
    sign of the level is the sign bit of v (+0 -> +1, -0 -> -1; with s = 0
    every level gives 0 and the sign bit alone picks q).  Equal errors go to
    the smaller scale.
"""

from __future__ import annotations

import numpy as np

from .formats import e4m3_value, unpack_nibbles, e2m1_value

LEVELS = (-4.0, -1.0, 1.0, 4.0)
_LEVELS = np.array(LEVELS)
_E4M3_FINITE_NONNEG = np.array([e4m3_value(b) for b in range(0x7F)])   # bytes 0x00 .. 0x7E, increasing
_E2M1 = np.array([e2m1_value(c) for c in range(16)])


def unpack_2bit(packed) -> np.ndarray:
    """Canonical order: byte j holds elements 4j+i in bits 2i..2i+1.
    Returns uint8 codes [..., 4*n]."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (4 * p.shape[-1],), dtype=np.uint8)
    for i in range(4):
        out[..., i::4] = (p >> (2 * i)) & 3
    return out


def pack_2bit(codes) -> np.ndarray:
    """Inverse of unpack_2bit: codes [..., 4*n] in 0..3 -> bytes [..., n]."""
    c = np.asarray(codes, dtype=np.uint8)
    if c.shape[-1] % 4 or np.any(c > 3):
        raise ValueError("2-bit codes must be 0..3, a multiple of 4 per row")
    out = np.zeros(c.shape[:-1] + (c.shape[-1] // 4,), dtype=np.uint8)
    for i in range(4):
        out |= (c[..., i::4] << (2 * i)).astype(np.uint8)
    return out


def dequant_2bit(codes, scales, tensor_scale: float) -> np.ndarray:
    """One 2-bit matrix to float64: codes uint8 [R, K/4] (canonical order),
    scales e4m3 [R, K/16], W = LEVELS[q] * e4m3(scale of the block) * tensor_scale."""
    q = unpack_2bit(codes)
    R, K = q.shape
    scales = np.asarray(scales, dtype=np.uint8)
    if scales.shape != (R, K // 16) or K % 16:
        raise ValueError("scale shape does not match codes")
    blk = np.array([e4m3_value(b) for b in range(256)])[scales]
    vals = _LEVELS[q].reshape(R, K // 16, 16)
    return (vals * blk[:, :, None] * float(np.float32(tensor_scale))).reshape(R, K)


def nearest_codes(v: np.ndarray, s: float) -> np.ndarray:
    """Index of the level nearest to v / s (the reading's tie and sign rules),
    decided without dividing: |v| <= 2.5 s  <=>  2 |v| <= 5 s, both exact."""
    neg = np.signbit(v)
    big = (2.0 * np.abs(v) > 5.0 * s) if s > 0 else np.zeros(v.shape, dtype=bool)
    return np.where(neg, np.where(big, 0, 1), np.where(big, 3, 2)).astype(np.uint8)


def requant_from_nvfp4(codes4, scales4):
    """Re-quantise one NVFP4 matrix (codes uint8 [R, K/2], e4m3 scales
    [R, K/16]) to the 2-bit planes: returns (codes uint8 [R, K/4], e4m3 scales
    uint8 [R, K/16]); the tensor scale is unchanged.

    For every block the squared error of each candidate scale byte is summed
    element by element in float64 and the first (smallest) scale with the
    least error wins."""
    c4 = unpack_nibbles(np.asarray(codes4, dtype=np.uint8))
    R, K = c4.shape
    s4 = np.asarray(scales4, dtype=np.uint8)
    if s4.shape != (R, K // 16):
        raise ValueError("scale shape does not match codes")
    blk = np.array([e4m3_value(b) for b in range(256)])[s4]
    v = (_E2M1[c4].reshape(R, K // 16, 16) * blk[:, :, None])          # exact, without the tensor scale
    best_err = np.full((R, K // 16), np.inf)
    best_sb = np.zeros((R, K // 16), dtype=np.uint8)
    best_q = np.zeros((R, K // 16, 16), dtype=np.uint8)
    for sb in range(0x7F):
        s = float(_E4M3_FINITE_NONNEG[sb])
        q = nearest_codes(v, s)
        rec = _LEVELS[q] * s
        err = np.zeros((R, K // 16))
        for i in range(16):                  # element order
            d = v[:, :, i] - rec[:, :, i]
            err = err + d * d
        better = err < best_err              # ties keep the smaller scale found first
        best_err = np.where(better, err, best_err)
        best_sb = np.where(better, np.uint8(sb), best_sb)
        best_q = np.where(better[:, :, None], q, best_q)
    return pack_2bit(best_q.reshape(R, K)), best_sb
