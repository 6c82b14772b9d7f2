"""Pins of the oracle's 2-bit codec (decoding and re-quantisation from NVFP4).

SM120 page, section "How it fits -- 2-bit experts at FP4 quality": the
sign-symmetric codebook {-4, -1, 1, 4} and the exact float64 re-quantisation
from NVFP4.  The re-quantiser is checked against an exhaustive search written
as plainly as possible (every scale byte, every level of every element), and
against closed forms: blocks the codebook holds exactly, mirror symmetry,
doubling, all-zero blocks.
"""

import numpy as np
import pytest

import oracle
from oracle.codec2 import LEVELS


def test_levels_are_the_sign_symmetric_codebook():
    assert LEVELS == (-4.0, -1.0, 1.0, 4.0)
    assert [-v for v in LEVELS] == list(reversed(LEVELS))


def test_unpack_every_byte():
    b = np.arange(256, dtype=np.uint8)[None, :]
    q = oracle.unpack_2bit(b)
    for j in range(256):
        assert q[0, 4 * j:4 * j + 4].tolist() == [j & 3, (j >> 2) & 3, (j >> 4) & 3, (j >> 6) & 3]
    assert np.array_equal(oracle.pack_2bit(q), b)


def test_dequant_hand_matrix():
    # one row of 32 elements: codes 0,1,2,3 repeated; block 0 scale 0.5 (0x30), block 1 scale 2 (0x40)
    codes = oracle.pack_2bit(np.array([[0, 1, 2, 3] * 8], dtype=np.uint8))
    scales = np.array([[0x30, 0x40]], dtype=np.uint8)
    w = oracle.dequant_2bit(codes, scales, 0.75)
    want = np.array([-4, -1, 1, 4] * 8, dtype=np.float64) * np.repeat([0.5, 2.0], 16) * 0.75
    assert np.array_equal(w[0], want)


def _brute_block(v):
    """Exhaustive: every non-negative finite e4m3 scale, every level of every
    element; least error, then the smaller scale; per element the least
    |v - L s|, then (tie between 1 and 4) the smaller magnitude, the sign from
    the sign bit when all levels tie (s = 0)."""
    best = None
    for sb in range(0x7F):
        s = oracle.e4m3_value(sb)
        qs, err = [], 0.0
        for x in v:
            cands = []
            for qi, L in enumerate(LEVELS):
                d = abs(x - L * s)
                # preference: distance, then smaller |L|, then the sign agreeing with x's sign bit
                cands.append((d, abs(L), (L < 0) != bool(np.signbit(x)), qi))
            d, _, _, qi = min(cands)
            qs.append(qi)
        for x, qi in zip(v, qs):
            err = err + (x - LEVELS[qi] * s) ** 2
        if best is None or err < best[0]:
            best = (err, sb, qs)
    return best[1], best[2]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_requant_matches_exhaustive_search(seed):
    rng = np.random.default_rng(seed)
    rows = 3
    codes4 = rng.integers(0, 256, size=(rows, 16), dtype=np.uint8)          # 32 elements per row: 2 blocks
    scales4 = rng.integers(0x01, 0x7F, size=(rows, 2), dtype=np.uint8)
    q2, s2 = oracle.requant_from_nvfp4(codes4, scales4)
    v = oracle.dequant_nvfp4(codes4, scales4, 1.0)
    qu = oracle.unpack_2bit(q2)
    for r in range(rows):
        for b in range(2):
            sb, qs = _brute_block(v[r, 16 * b:16 * b + 16].tolist())
            assert s2[r, b] == sb, (r, b)
            assert qu[r, 16 * b:16 * b + 16].tolist() == qs, (r, b)


def test_exactly_representable_blocks_come_back_exactly():
    """A block holding both magnitudes (so no other scale reproduces it) of
    L * s for an e4m3 s: the requantiser returns s and the codes, error 0."""
    rng = np.random.default_rng(7)
    for sb in (0x28, 0x30, 0x33, 0x38, 0x3B, 0x45):      # 0.25, 0.5, 0.6875, 1, 1.375, 2.5
        s = oracle.e4m3_value(sb)
        q = rng.integers(0, 4, size=16).astype(np.uint8)
        q[0], q[1] = 0, 2                                   # both magnitudes present
        # as NVFP4: L*s = e2m1 * scale with e2m1 in {+-1, +-4} and the same scale byte
        e2m1_code = {0: 0xE, 1: 0xA, 2: 0x2, 3: 0x6}
        nib = np.array([e2m1_code[int(x)] for x in q], dtype=np.uint8)
        codes4 = (nib[0::2] | (nib[1::2] << 4))[None, :]
        q2, s2 = oracle.requant_from_nvfp4(codes4, np.array([[sb]], dtype=np.uint8))
        assert s2[0, 0] == sb
        assert oracle.unpack_2bit(q2)[0].tolist() == q.tolist()
        assert np.array_equal(oracle.dequant_2bit(q2, s2, 1.0), oracle.dequant_nvfp4(codes4, [[sb]], 1.0))


def test_mirror_and_doubling():
    rng = np.random.default_rng(11)
    codes4 = rng.integers(0, 256, size=(8, 64), dtype=np.uint8)
    scales4 = rng.integers(0x30, 0x58, size=(8, 8), dtype=np.uint8)   # 0.5 .. 30: doubled scales stay normal
    q2, s2 = oracle.requant_from_nvfp4(codes4, scales4)
    # every code's sign bit flipped: the same scales, mirrored codes (q -> 3 - q)
    qm, sm = oracle.requant_from_nvfp4(codes4 ^ 0x88, scales4)
    assert np.array_equal(sm, s2)
    assert np.array_equal(oracle.unpack_2bit(qm), 3 - oracle.unpack_2bit(q2))
    # every block scale doubled (e4m3 exponent + 1): new scales doubled, same codes
    qd, sd = oracle.requant_from_nvfp4(codes4, scales4 + 8)
    nz = s2 != 0
    assert np.array_equal(sd[nz], s2[nz] + 8)
    assert np.array_equal(oracle.unpack_2bit(qd), oracle.unpack_2bit(q2))


def test_zero_blocks_and_signed_zeros():
    # codes 0 (+0) and 8 (-0) alternating: the scale 0 fits exactly; +0 -> level +1, -0 -> level -1
    codes4 = np.full((1, 8), 0x80, dtype=np.uint8)            # low nibble +0, high nibble -0
    q2, s2 = oracle.requant_from_nvfp4(codes4, np.array([[0x38]], dtype=np.uint8))
    assert s2[0, 0] == 0
    assert oracle.unpack_2bit(q2)[0].tolist() == [2, 1] * 8


def test_error_is_minimal_over_scales():
    """The chosen scale's error is at most that of every other scale byte
    (evaluated here as the sum over elements of the least per-level error)."""
    rng = np.random.default_rng(3)
    codes4 = rng.integers(0, 256, size=(4, 32), dtype=np.uint8)
    scales4 = rng.integers(0x10, 0x60, size=(4, 4), dtype=np.uint8)
    q2, s2 = oracle.requant_from_nvfp4(codes4, scales4)
    v = oracle.dequant_nvfp4(codes4, scales4, 1.0).reshape(4, 4, 16)
    w = oracle.dequant_2bit(q2, s2, 1.0).reshape(4, 4, 16)
    got = np.sum((v - w) ** 2, axis=-1)
    for sb in range(0x7F):
        s = oracle.e4m3_value(sb)
        e = np.min([(v - L * s) ** 2 for L in LEVELS], axis=0).sum(axis=-1)
        assert np.all(got <= e * (1 + 1e-12) + 1e-300)


def test_layer_with_2bit_experts_equals_bf16_experts_of_the_same_values():
    """The layer's 2-bit branch against its BF16 branch: experts whose 2-bit
    values (levels x e4m3 scales, tensor scale 1) are exact in bf16."""
    from types import SimpleNamespace
    rng = np.random.default_rng(5)
    H, I, E, k = 64, 32, 4, 2

    def two_bit(rows, cols):
        q = rng.integers(0, 4, size=(rows, cols), dtype=np.uint8)
        s = rng.integers(0x30, 0x40, size=(rows, cols // 16), dtype=np.uint8)
        return oracle.pack_2bit(q), s

    experts = []
    for _ in range(E):
        c13, s13 = two_bit(2 * I, H)
        c2, s2 = two_bit(H, I)
        experts.append({"codes13": c13, "scales13": s13, "g13": 1.0, "codes2": c2, "scales2": s2, "g2": 1.0})

    def bf16_bits(a):
        f = np.asarray(a, dtype=np.float32).view(np.uint32)
        assert np.all(f & 0xFFFF == 0)                      # exact in bf16
        return (f >> 16).astype(np.uint16)

    shared = {"w13": bf16_bits(rng.standard_normal((2 * I, H)) * 0 + 0.5),
              "w2": bf16_bits(np.full((H, I), 0.25))}
    router = bf16_bits(np.round(rng.standard_normal((E, H)) * 8) / 8)
    base = dict(hidden=H, inter=I, n_routed=E, top_k=k, n_shared=1, route="sigmoid", shared_wtype="bf16",
                router_w=router, router_bias=None, gamma=None, eps=1e-6, residual=False,
                shared_expert=lambda s: shared)
    l2 = SimpleNamespace(**base, routed_wtype="2bit", routed_expert=lambda e: experts[e])
    as_bf16 = [{"w13": bf16_bits(oracle.dequant_2bit(x["codes13"], x["scales13"], 1.0)),
                "w2": bf16_bits(oracle.dequant_2bit(x["codes2"], x["scales2"], 1.0))} for x in experts]
    lb = SimpleNamespace(**base, routed_wtype="bf16", routed_expert=lambda e: as_bf16[e])
    x = bf16_bits(np.round(rng.standard_normal((3, H)) * 16) / 16)
    a, b = oracle.moe_layer(l2, x), oracle.moe_layer(lb, x)
    assert np.array_equal(a["ids"], b["ids"])
    assert np.array_equal(a["out"], b["out"])
