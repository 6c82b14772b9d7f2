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


def test_abi_version_and_status_strings():
    assert B.moe_abi_version() == 2
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


def test_layout_sizes_flint():
    lay = B.moe_expert_layout_query("nvfp4", 2048, 512, 256)
    assert lay["w13_code_bytes"] == 1024 * 2048 // 2
    assert lay["w2_code_bytes"] == 2048 * 512 // 2
    assert lay["w13_scale_bytes"] == 1024 * 2048 // 16
    assert lay["w2_scale_bytes"] == 2048 * 512 // 16
    per_expert = lay["code_stride"] + lay["scale_stride"]
    assert per_expert == 1_769_472          # bytes of one Flint expert in NVFP4
    assert lay["scale_region_bytes"] == lay["tensor_scale_offset"] + 256 * 8
    bf = B.moe_expert_layout_query("bf16", 2048, 512, 1)
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
