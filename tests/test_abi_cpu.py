"""The C-ABI library on the CPU: it loads, exports what the header declares,
validates descriptions, and its packers are lossless.  No kernel runs here."""

import os
import re

import numpy as np
import pytest

from conftest import ROOT
from quantized_expert_gemv_amd import binding as B
from quantized_expert_gemv_amd.synth import WORKLOADS

HEADER = os.path.join(ROOT, "include", "moe_decode.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(moe_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(B.lib, n), n
    assert set(names) == set(B.EXPORTED)


def test_bench_header_symbols_are_exported():
    text = open(os.path.join(ROOT, "include", "moe_bench.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"^\s*int\s+(moe_\w+)\s*\(", text, flags=re.M)))
    assert set(names) == set(B.BENCH_EXPORTED)
    for n in names:
        assert hasattr(B.lib, n), n
    assert B.lib.moe_bench_read_stream(None, 65536, None, None) == -1
    assert B.lib.moe_bench_fill(None, 16, 0, None) == -1
    assert B.lib.moe_bench_empty(0, None) == -1


def test_binding_follows_the_header_abi_version():
    with open(HEADER) as f:
        m = re.search(r"#define MOE_ABI_VERSION (\d+)", f.read())
    assert m and int(m.group(1)) == B.ABI_VERSION


def test_abi_version_and_status_strings():
    assert B.moe_abi_version() == 4 == B.ABI_VERSION
    for code in B.STATUS:
        assert B.moe_status_str(code)
    assert B.moe_status_str(0) == "ok"


def _desc_for(wl, **over):
    kw = dict(hidden=wl.hidden, inter=wl.inter, n_routed=wl.n_routed, top_k=wl.top_k, n_shared=wl.n_shared,
              max_batch=max(wl.batch, 1), routed_wtype=wl.routed_wtype, shared_wtype=wl.shared_wtype,
              route=wl.route)
    kw.update(over)
    return B.make_desc(**kw)


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_all_workloads_validate(name):
    assert B.moe_layer_validate(_desc_for(WORKLOADS[name])) == B.MOE_OK


@pytest.mark.parametrize("over,status", [
    (dict(hidden=0), -1), (dict(top_k=300), -1), (dict(n_shared=-1), -1), (dict(route=7), -1),
    (dict(routed_wtype=5), -1), (dict(max_batch=0), -1),
    (dict(max_batch=9), -2), (dict(hidden=2050), -2), (dict(inter=4096), -2), (dict(n_routed=600, top_k=6), -2),
    (dict(top_k=17), -2), (dict(n_shared=5), -2), (dict(routed_wtype="bf16", shared_wtype="nvfp4"), -2),
    (dict(route="sink", router_bias=16), -2), (dict(hidden=2048 + 32 * 3), -2),
    (dict(prenorm_gamma=8), -3),
])
def test_validation_error_codes(over, status):
    assert B.moe_layer_validate(_desc_for(WORKLOADS["flint_b1"], **over)) == status


def test_null_description_and_handle():
    assert B.lib.moe_layer_validate(None) == -1
    assert B.lib.moe_decode_layer(None, None, None, None, None, None, None, 1, None) == -1
    assert B.lib.moe_layer_routing(None, None, None, None, None) == -1
    assert B.lib.moe_layer_destroy(None) == -1
    assert B.lib.moe_layer_set_path(None, B.MOE_PATH_AUTO, None) == -1
    assert B.lib.moe_decode_chain(None, 1, None, None, None, None, None, None, 1, None) == -1
    n = B.C.c_size_t(7)
    assert B.lib.moe_prefill_workspace_bytes(None, 1, B.C.byref(n)) == -1
    assert B.lib.moe_prefill_layer(None, None, None, None, None, None, None, 1, None, 0, None, None, None) == -1


def test_layout_sizes_flint():
    lay = B.moe_expert_layout_query(_desc_for(WORKLOADS["flint_b1"]), B.MOE_SET_ROUTED)
    assert lay["w13_code_bytes"] == 1024 * 2048 // 2
    assert lay["w2_code_bytes"] == 2048 * 512 // 2
    assert lay["w13_scale_bytes"] == 1024 * 2048 // 16
    assert lay["w2_scale_bytes"] == 2048 * 512 // 16
    per_expert = lay["code_stride"] + lay["scale_stride"]
    assert per_expert == 1_769_472          # bytes of one Flint expert in NVFP4
    assert lay["scale_region_bytes"] == lay["tensor_scale_offset"] + 256 * 8
    bf = B.moe_expert_layout_query(_desc_for(WORKLOADS["flint_bf16_b1"]), B.MOE_SET_SHARED)
    assert bf["code_stride"] == 3 * 2048 * 512 * 2 and bf["scale_region_bytes"] == 0


SHAPES = [(256, 256), (256, 128), (1024, 2048), (2048, 512), (4096, 7168), (7168, 2048), (128, 32), (128, 1536)]


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_nvfp4_pack_roundtrip_is_lossless(rows, cols):
    rng = np.random.default_rng(rows * 7 + cols)
    codes = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, size=(rows, cols // 16), dtype=np.uint8)   # incl. NaN / -0 bytes
    cp, sp = B.moe_pack_nvfp4(codes, scales)
    # a permutation of 16-byte code units and 2-byte scale pairs
    assert sorted(map(bytes, cp.reshape(-1, 16))) == sorted(map(bytes, codes.reshape(-1, 16)))
    assert sorted(map(bytes, sp.reshape(-1, 2))) == sorted(map(bytes, scales.reshape(-1, 2)))
    c2, s2 = B.moe_unpack_nvfp4(rows, cols, cp, sp)
    assert (c2 == codes).all() and (s2 == scales).all()


def test_nvfp4_pack_exhaustive_bytes():
    rows, cols = 256, 512            # every code byte and every scale byte value appears
    codes = (np.arange(rows * cols // 2) % 256).astype(np.uint8).reshape(rows, cols // 2)
    scales = (np.arange(rows * cols // 16) * 7 % 256).astype(np.uint8).reshape(rows, cols // 16)
    cp, sp = B.moe_pack_nvfp4(codes, scales)
    assert np.bincount(cp, minlength=256).tolist() == np.bincount(codes.ravel(), minlength=256).tolist()
    c2, s2 = B.moe_unpack_nvfp4(rows, cols, cp, sp)
    assert (c2 == codes).all() and (s2 == scales).all()


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_bf16_pack_roundtrip_is_lossless(rows, cols):
    rng = np.random.default_rng(rows + cols)
    w = rng.integers(0, 1 << 16, size=(rows, cols), dtype=np.uint32).astype(np.uint16)
    wp = B.moe_pack_bf16(w)
    assert sorted(map(bytes, wp.view(np.uint8).reshape(-1, 16))) == \
        sorted(map(bytes, w.view(np.uint8).reshape(-1, 16)))
    assert (B.moe_unpack_bf16(rows, cols, wp) == w).all()


def test_packer_rejects_unsupported_shapes():
    with pytest.raises(B.MoeError):
        B.moe_pack_nvfp4(np.zeros((3, 16), np.uint8), np.zeros((3, 2), np.uint8))     # rows % rpw
    with pytest.raises(B.MoeError):
        B.moe_pack_bf16(np.zeros((4, 48), np.uint16))                                  # cols % 32


def test_create_fails_cleanly_without_gpu():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present")
    h = B.C.c_void_p()
    st = B.lib.moe_layer_create(B.C.byref(_desc_for(WORKLOADS["tiny"])), B.C.byref(h))
    assert st == -6 and not h.value


# ---- whole-set packers -------------------------------------------------------------------

def _rand_expert(rng, wtype, H, I):
    if wtype == "nvfp4":
        return {"codes13": rng.integers(0, 256, (2 * I, H // 2), dtype=np.uint8),
                "scales13": rng.integers(0, 256, (2 * I, H // 16), dtype=np.uint8),
                "codes2": rng.integers(0, 256, (H, I // 2), dtype=np.uint8),
                "scales2": rng.integers(0, 256, (H, I // 16), dtype=np.uint8),
                "g13": np.float32(rng.choice([0.37, 0.7, 1.3, 2.0])),
                "g2": np.float32(rng.choice([0.37, 0.7, 1.3, 2.0]))}
    return {"w13": rng.integers(0, 1 << 16, (2 * I, H), dtype=np.uint32).astype(np.uint16),
            "w2": rng.integers(0, 1 << 16, (H, I), dtype=np.uint32).astype(np.uint16)}


def _small_desc(rwt="nvfp4", swt="nvfp4", E=5, S=2):
    return B.make_desc(hidden=256, inter=128, n_routed=E, top_k=2, n_shared=S, max_batch=1,
                       routed_wtype=rwt, shared_wtype=swt)


@pytest.mark.parametrize("wtype,set_", [("nvfp4", 0), ("nvfp4", 1), ("bf16", 0), ("bf16", 1)])
def test_expert_set_pack_roundtrip_and_placement(wtype, set_):
    """moe_pack_experts places every expert (codes, block scales, tensor scales) where
    moe_expert_layout_query says, packed in pieces; moe_unpack_experts inverts it."""
    rng = np.random.default_rng(5 + set_)
    H, I = 256, 128
    desc = _small_desc(wtype, wtype)
    n = desc.n_routed if set_ == 0 else desc.n_shared
    exps = [_rand_expert(rng, wtype, H, I) for _ in range(n)]
    lay = B.moe_expert_layout_query(desc, set_)
    if set_ == 1:
        code = np.zeros(lay["shared_total_bytes"], np.uint8)
        scale = None
    else:
        code = np.zeros(lay["code_region_bytes"], np.uint8)
        scale = np.zeros(max(lay["scale_region_bytes"], 1), np.uint8)
    B.moe_pack_experts(desc, set_, 0, exps[:1], code, scale)      # in two pieces
    B.moe_pack_experts(desc, set_, 1, exps[1:], code, scale)
    back = B.moe_unpack_experts(desc, set_, 0, n, code, scale)
    for a, b in zip(exps, back):
        for key in a:
            assert np.array_equal(np.asarray(a[key]), np.asarray(b[key])), key
    # each expert matches the single-matrix packer at the documented offsets
    sreg = code[lay["shared_scale_offset"]:] if set_ == 1 else scale
    for e, ex in enumerate(exps):
        c0 = e * lay["code_stride"]
        if wtype == "nvfp4":
            cp, sp = B.moe_pack_nvfp4(ex["codes13"], ex["scales13"])
            s0 = e * lay["scale_stride"]
            assert np.array_equal(code[c0:c0 + cp.size], cp) and np.array_equal(sreg[s0:s0 + sp.size], sp)
            cp2, sp2 = B.moe_pack_nvfp4(ex["codes2"], ex["scales2"])
            assert np.array_equal(code[c0 + cp.size:c0 + cp.size + cp2.size], cp2)
            ts = sreg[lay["tensor_scale_offset"] + 8 * e:][:8].view(np.float32)
            assert ts.tolist() == [np.float32(ex["g13"]), np.float32(ex["g2"])]
        else:
            wp = B.moe_pack_bf16(ex["w13"])
            assert np.array_equal(code[c0:c0 + wp.nbytes].view(np.uint16), wp)


def test_expert_set_pack_rejects_bad_ranges():
    desc = _small_desc(E=2)
    lay = B.moe_expert_layout_query(desc, 0)
    code = np.zeros(lay["code_region_bytes"], np.uint8)
    scale = np.zeros(lay["scale_region_bytes"], np.uint8)
    ex = _rand_expert(np.random.default_rng(1), "nvfp4", 256, 128)
    with pytest.raises(B.MoeError):
        B.moe_pack_experts(desc, 0, 2, [ex], code, scale)          # first == n
    with pytest.raises(B.MoeError):
        B.moe_pack_experts(desc, 0, 1, [ex, ex], code, scale)      # past the end
    with pytest.raises(B.MoeError):
        B.moe_pack_experts(desc, 0, 0, [ex], code, None)           # scale region missing
    with pytest.raises(B.MoeError):
        B.moe_pack_experts(desc, 2, 0, [ex], code, scale)          # no such set


# ---- validate agrees with create on every weight-type pair --------------------------------

@pytest.mark.parametrize("shape", ["flint", "generic"])
@pytest.mark.parametrize("rwt,swt,want", [("nvfp4", "nvfp4", 0), ("bf16", "bf16", 0), ("nvfp4", "bf16", 0),
                                          ("bf16", "nvfp4", -2)])
def test_validate_accepts_exactly_the_compiled_type_pairs(shape, rwt, swt, want):
    """Every pair validate accepts has a compiled kernel at every batch bucket (the
    Flint shape falls back to the argument-shaped kernel for mixed pairs), so
    create cannot fail for lack of a variant; the GPU test checks create itself."""
    kw = dict(hidden=2048, inter=512, n_routed=256, top_k=6, n_shared=1) if shape == "flint" else \
        dict(hidden=1024, inter=256, n_routed=64, top_k=4, n_shared=2)
    for mb in (1, 2, 4, 8):
        d = B.make_desc(max_batch=mb, routed_wtype=rwt, shared_wtype=swt, **kw)
        assert B.moe_layer_validate(d) == want, (mb, rwt, swt)


def test_static_entry_rejects_oversize_workspace_before_the_device():
    """The handle-less call's workspace must fit the static scratch array: the
    largest shapes at batch 8 do not, and are refused on the host."""
    big = B.make_desc(hidden=2048, inter=2048, n_routed=512, top_k=16, n_shared=4, max_batch=8)
    assert B.moe_layer_validate(big) == 0
    st = B.lib.moe_decode_layer_static(B.C.byref(big), None, None, None, None, None, None, 1, None, None)
    assert st == -2
    ok = _desc_for(WORKLOADS["flint_b8"])
    st = B.lib.moe_decode_layer_static(B.C.byref(ok), None, None, None, None, None, None, 1, None, None)
    assert st == -1                  # fits; the missing buffers are the error


# ---- dense NVFP4 GEMV packing ------------------------------------------------------

@pytest.mark.parametrize("rows,cols", [(1, 32), (7, 96), (100, 96), (333, 512), (2560, 2048), (64, 2048)])
def test_dense_pack_round_trip(rows, cols):
    rng = np.random.default_rng(rows * 7 + cols)
    codes = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, size=(rows, cols // 16), dtype=np.uint8)
    cr, sr = B.moe_pack_dense(codes, scales, 0.625)
    lay = B.moe_dense_layout_query(rows, cols)
    assert lay["packed_rows"] >= rows and lay["code_bytes"] == lay["packed_rows"] * cols // 2
    assert cr.nbytes == lay["code_bytes"] and sr.nbytes == lay["scale_region_bytes"]
    c2, s2, ts = B.moe_unpack_dense(rows, cols, cr, sr)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales) and ts == 0.625
    # every canonical byte appears in the packed region (a permutation plus zero padding)
    assert np.array_equal(np.sort(cr)[-codes.size:], np.sort(codes.ravel()))


@pytest.mark.parametrize("rows,cols", [(0, 64), (8, 0), (8, 48), (8, 4096), (8, 2080)])
def test_dense_bad_shapes(rows, cols):
    lay = B.moe_dense_layout()
    assert B.lib.moe_dense_layout_query(rows, cols, B.C.byref(lay)) == -1
    assert B.lib.moe_dense_gemv(rows, cols, None, None, None, None, 1, None) == -1


def test_dense_gemv_rejects_without_a_device_call():
    # null pointers and batch outside 1..8 are refused before any launch
    assert B.lib.moe_dense_gemv(64, 64, None, None, None, None, 1, None) == -1
    x = np.zeros(256, dtype=np.uint8)
    p = x.ctypes.data
    assert B.lib.moe_dense_gemv(64, 64, p, p, p, p + 128, 9, None) == -4
    assert B.lib.moe_dense_gemv(64, 64, p, p, p, p + 128, 0, None) == -4
    assert B.lib.moe_dense_gemv(64, 64, p + 1, p, p, p + 128, 1, None) == -3


# ---- the 2-bit expert planes (host side) -----------------------------------------------------

@pytest.mark.parametrize("seed,rows,cols", [(0, 8, 64), (1, 3, 256), (2, 16, 2048)])
def test_library_requant_matches_the_oracle_bit_for_bit(seed, rows, cols):
    """moe_requant_2bit (C++, float64 with no fused multiply-adds) against the
    oracle's re-quantisation: the same scale bytes and codes, every block."""
    import oracle
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0x00, 0x7F, size=(rows, cols // 16), dtype=np.uint8)
    scales[0, 0] = 0x00                                           # a zero block scale
    q_lib, s_lib = B.moe_requant_2bit(codes, scales)
    q_ref, s_ref = oracle.requant_from_nvfp4(codes, scales)
    assert np.array_equal(s_lib, s_ref)
    assert np.array_equal(q_lib, q_ref)


def test_requant_argument_checks():
    assert B.lib.moe_requant_2bit(1, 24, None, None, None, None) == -1
    z = np.zeros(64, np.uint8)
    assert B.lib.moe_requant_2bit(1, 24, B._ptr(z), B._ptr(z), B._ptr(z), B._ptr(z)) == -1   # cols % 16


def test_2bit_layer_validation_rules():
    """2-bit routed experts: the Flint shape at batch 1 to 8 with an NVFP4
    shared expert and sigmoid routing; anything else is unsupported."""
    flint = dict(hidden=2048, inter=512, n_routed=256, top_k=6, n_shared=1, routed_wtype="2bit")
    assert B.moe_layer_validate(B.make_desc(max_batch=1, **flint)) == 0
    assert B.moe_layer_validate(B.make_desc(max_batch=2, **flint)) == 0
    assert B.moe_layer_validate(B.make_desc(max_batch=8, **flint)) == 0
    assert B.moe_layer_validate(B.make_desc(max_batch=9, **flint)) == -2
    assert B.moe_layer_validate(B.make_desc(max_batch=1, shared_wtype="bf16", **flint)) == -2
    assert B.moe_layer_validate(B.make_desc(max_batch=1, route="sink", **flint)) == -2
    assert B.moe_layer_validate(B.make_desc(hidden=1024, inter=256, n_routed=64, top_k=4, n_shared=1, max_batch=1,
                                            routed_wtype="2bit")) == -2


def test_2bit_expert_pack_round_trip_and_layout():
    d = B.make_desc(hidden=2048, inter=512, n_routed=256, top_k=6, n_shared=1, max_batch=1, routed_wtype="2bit")
    lay = B.moe_expert_layout_query(d, B.MOE_SET_ROUTED)
    assert lay["w13_code_bytes"] == 2 * 512 * 2048 // 4 and lay["w2_code_bytes"] == 2048 * 512 // 4
    assert lay["w13_scale_bytes"] == 2 * 512 * 2048 // 16 and lay["w2_scale_bytes"] == 2048 * 512 // 16
    rng = np.random.default_rng(4)
    ex = {"codes13": rng.integers(0, 256, size=(1024, 512), dtype=np.uint8),
          "scales13": rng.integers(0, 256, size=(1024, 128), dtype=np.uint8),
          "codes2": rng.integers(0, 256, size=(2048, 128), dtype=np.uint8),
          "scales2": rng.integers(0, 256, size=(2048, 32), dtype=np.uint8),
          "g13": np.float32(0.7), "g2": np.float32(1.3)}
    code = np.zeros(lay["code_region_bytes"], np.uint8)
    scale = np.zeros(lay["scale_region_bytes"], np.uint8)
    B.moe_pack_experts(d, B.MOE_SET_ROUTED, 5, [ex], code, scale)
    back = B.moe_unpack_experts(d, B.MOE_SET_ROUTED, 5, 1, code, scale)[0]
    for k in ("codes13", "scales13", "codes2", "scales2"):
        assert np.array_equal(back[k], ex[k]), k
    assert back["g13"] == np.float32(0.7) and back["g2"] == np.float32(1.3)
    # the packed chunk (row r, 32-column chunk j) of W13 is the row's canonical bytes 8 j .. 8 j + 8
    base = 5 * lay["code_stride"]
    assert np.array_equal(code[base + (3 * 64 + 7) * 8: base + (3 * 64 + 7) * 8 + 8], ex["codes13"][3, 56:64])
