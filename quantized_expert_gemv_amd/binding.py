"""ctypes binding of libmoe_decode.so (argument marshalling only).

The function names mirror the C ABI in include/moe_decode.h.  Every step of
the layer runs in the library's HIP kernels; PyTorch is used only to own
device memory and to supply the current HIP stream.  Importing this module
loads the library and raises if it has not been built: there is no fallback.
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_decode.so")

MOE_OK = 0
STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED", -3: "MOE_ERR_ALIGNMENT",
          -4: "MOE_ERR_BATCH", -5: "MOE_ERR_LAUNCH", -6: "MOE_ERR_DEVICE", -7: "MOE_ERR_STATE"}
MOE_W_NVFP4, MOE_W_BF16, MOE_W_2BIT = 0, 1, 2
MOE_ROUTE_SIGMOID_TOPK, MOE_ROUTE_SOFTMAX_SINK = 0, 1
MOE_SET_ROUTED, MOE_SET_SHARED = 0, 1
WTYPES = {"nvfp4": MOE_W_NVFP4, "bf16": MOE_W_BF16, "2bit": MOE_W_2BIT}
ROUTES = {"sigmoid": MOE_ROUTE_SIGMOID_TOPK, "sink": MOE_ROUTE_SOFTMAX_SINK}

EXPORTED = ("moe_abi_version", "moe_status_str", "moe_layer_validate", "moe_expert_layout_query",
            "moe_pack_experts", "moe_unpack_experts",
            "moe_pack_nvfp4", "moe_unpack_nvfp4", "moe_pack_bf16", "moe_unpack_bf16",
            "moe_layer_create", "moe_layer_destroy", "moe_decode_layer", "moe_decode_layer_static",
            "moe_layer_routing",
            "moe_layer_set_profiling", "moe_layer_debug_h", "moe_layer_set_path", "moe_decode_chain", "moe_layer_error", "moe_layer_reset",
            "moe_layer_grid", "moe_dense_layout_query", "moe_pack_dense", "moe_unpack_dense",
            "moe_dense_gemv", "moe_prefill_workspace_bytes", "moe_prefill_layer", "moe_requant_2bit")


BENCH_EXPORTED = ("moe_bench_read_stream", "moe_bench_fill", "moe_bench_empty")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({status})")
        self.status = status


class moe_layer_desc(C.Structure):
    _fields_ = [("hidden", C.c_int), ("inter", C.c_int), ("n_routed", C.c_int), ("top_k", C.c_int),
                ("n_shared", C.c_int), ("max_batch", C.c_int), ("routed_wtype", C.c_int),
                ("shared_wtype", C.c_int), ("route", C.c_int), ("router_bias", C.c_void_p),
                ("prenorm_gamma", C.c_void_p), ("rms_eps", C.c_float), ("add_residual", C.c_int)]


class moe_expert_layout(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in (
        "w13_code_bytes", "w2_code_bytes", "code_stride", "code_region_bytes", "w13_scale_bytes",
        "w2_scale_bytes", "scale_stride", "tensor_scale_offset", "scale_region_bytes",
        "shared_scale_offset", "shared_total_bytes")]

    def as_dict(self) -> dict:
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


class moe_dense_layout(C.Structure):
    _fields_ = [("rows", C.c_int), ("cols", C.c_int), ("packed_rows", C.c_int)] + [(n, C.c_size_t) for n in (
        "code_bytes", "scale_bytes", "tensor_scale_offset", "scale_region_bytes")]

    def as_dict(self) -> dict:
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


def _load() -> C.CDLL:
    # torch ships its own HIP runtime whose SONAME equals the system one's.
    # Importing torch first makes the library's libamdhip64.so.7 dependency
    # resolve to that already-loaded runtime, so the process has a single HIP
    # runtime and torch's allocations and streams are valid in our calls.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m quantized_expert_gemv_amd.build` "
                          "(there is no CPU fallback)")
    lib = C.CDLL(LIB_PATH)
    vp, i32, sz = C.c_void_p, C.c_int, C.c_size_t
    sig = {
        "moe_abi_version": ([], i32),
        "moe_status_str": ([i32], C.c_char_p),
        "moe_layer_validate": ([C.POINTER(moe_layer_desc)], i32),
        "moe_expert_layout_query": ([C.POINTER(moe_layer_desc), i32, C.POINTER(moe_expert_layout)], i32),
        "moe_pack_experts": ([C.POINTER(moe_layer_desc), i32, i32, i32, vp, vp, vp, vp, vp, vp, vp], i32),
        "moe_unpack_experts": ([C.POINTER(moe_layer_desc), i32, i32, i32, vp, vp, vp, vp, vp, vp, vp], i32),
        "moe_pack_nvfp4": ([i32, i32, vp, vp, vp, vp], i32),
        "moe_unpack_nvfp4": ([i32, i32, vp, vp, vp, vp], i32),
        "moe_pack_bf16": ([i32, i32, vp, vp], i32),
        "moe_unpack_bf16": ([i32, i32, vp, vp], i32),
        "moe_layer_create": ([C.POINTER(moe_layer_desc), C.POINTER(vp)], i32),
        "moe_layer_destroy": ([vp], i32),
        "moe_decode_layer": ([vp, vp, vp, vp, vp, vp, vp, i32, vp], i32),
        "moe_decode_layer_static": ([C.POINTER(moe_layer_desc), vp, vp, vp, vp, vp, vp, i32, vp, vp], i32),
        "moe_layer_routing": ([vp, vp, vp, vp, vp], i32),
        "moe_layer_set_profiling": ([vp, vp, i32], i32),
        "moe_layer_debug_h": ([vp, vp, vp, vp], i32),
        "moe_layer_set_path": ([vp, i32, vp], i32),
        "moe_decode_chain": ([vp, i32, vp, vp, vp, vp, vp, vp, i32, vp], i32),
        "moe_layer_error": ([vp, C.POINTER(C.c_uint), i32], i32),
        "moe_layer_reset": ([vp], i32),
        "moe_layer_grid": ([vp, C.POINTER(i32), C.POINTER(i32)], i32),
        "moe_dense_layout_query": ([i32, i32, C.POINTER(moe_dense_layout)], i32),
        "moe_pack_dense": ([i32, i32, vp, vp, C.c_float, vp, vp], i32),
        "moe_unpack_dense": ([i32, i32, vp, vp, vp, vp, C.POINTER(C.c_float)], i32),
        "moe_dense_gemv": ([i32, i32, vp, vp, vp, vp, i32, vp], i32),
        "moe_prefill_workspace_bytes": ([vp, i32, C.POINTER(sz)], i32),
        "moe_prefill_layer": ([vp, vp, vp, vp, vp, vp, vp, i32, vp, sz, vp, vp, vp], i32),
        "moe_requant_2bit": ([i32, i32, vp, vp, vp, vp], i32),
    }
    sig.update({
        "moe_bench_read_stream": ([vp, sz, vp, vp], i32),
        "moe_bench_fill": ([vp, sz, C.c_uint, vp], i32),
        "moe_bench_empty": ([i32, vp], i32),
    })
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes, f.restype = args, res
    return lib


lib = _load()


def _check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status)


def _ptr(a) -> int | None:
    """Device pointer of a torch tensor, host pointer of a numpy array, or an int."""
    if a is None:
        return None
    if isinstance(a, int):
        return a
    if isinstance(a, np.ndarray):
        return a.ctypes.data
    return a.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---- host-only entry points ---------------------------------------------------------

ABI_VERSION = 4   # MOE_ABI_VERSION of the header these wrappers follow


def moe_abi_version() -> int:
    return lib.moe_abi_version()


def moe_status_str(status: int) -> str:
    return lib.moe_status_str(status).decode()


def make_desc(*, hidden, inter, n_routed, top_k, n_shared, max_batch, routed_wtype="nvfp4",
              shared_wtype="nvfp4", route="sigmoid", router_bias=None, prenorm_gamma=None,
              rms_eps=1e-6, add_residual=False) -> moe_layer_desc:
    return moe_layer_desc(hidden, inter, n_routed, top_k, n_shared, max_batch,
                          WTYPES.get(routed_wtype, routed_wtype), WTYPES.get(shared_wtype, shared_wtype),
                          ROUTES.get(route, route), _ptr(router_bias), _ptr(prenorm_gamma),
                          float(rms_eps), int(bool(add_residual)))


def moe_layer_validate(desc: moe_layer_desc) -> int:
    return lib.moe_layer_validate(C.byref(desc))


def moe_expert_layout_query(desc: "moe_layer_desc", set_: int = MOE_SET_ROUTED) -> dict:
    out = moe_expert_layout()
    _check("moe_expert_layout_query", lib.moe_expert_layout_query(C.byref(desc), int(set_), C.byref(out)))
    return out.as_dict()


def _canon(ex: dict, wtype: str):
    """Canonical arrays of one expert dict (codes13/scales13/codes2/scales2/g13/g2 for
    NVFP4 and the 2-bit planes, or w13/w2)."""
    if wtype in ("nvfp4", "2bit"):
        return (np.ascontiguousarray(ex["codes13"], np.uint8), np.ascontiguousarray(ex["scales13"], np.uint8),
                np.ascontiguousarray(ex["codes2"], np.uint8), np.ascontiguousarray(ex["scales2"], np.uint8),
                np.array([ex["g13"], ex["g2"]], np.float32))
    return (np.ascontiguousarray(ex["w13"], np.uint16), None, np.ascontiguousarray(ex["w2"], np.uint16), None, None)


def _wtype_of(desc, set_):
    return desc.routed_wtype if set_ == MOE_SET_ROUTED else desc.shared_wtype


def moe_pack_experts(desc: "moe_layer_desc", set_: int, first: int, experts: list, region: np.ndarray,
                     scale_region=None) -> None:
    """Packs the expert dicts `experts` as experts first.. of one set of the layer
    `desc` describes into the set's host buffers (the library places every byte)."""
    wt = _wtype_of(desc, set_)
    parts = [_canon(ex, "bf16" if wt == MOE_W_BF16 else "nvfp4") for ex in experts]
    stack = [np.ascontiguousarray(np.stack([p[i] for p in parts])) if parts[0][i] is not None else None
             for i in range(5)]
    _check("moe_pack_experts", lib.moe_pack_experts(C.byref(desc), int(set_), first, len(experts),
                                                    *[_ptr(a) for a in stack], _ptr(region), _ptr(scale_region)))


def moe_unpack_experts(desc: "moe_layer_desc", set_: int, first: int, count: int, region: np.ndarray,
                       scale_region=None) -> list:
    """Inverse of moe_pack_experts: the canonical expert dicts of experts first..first+count-1."""
    H, I = desc.hidden, desc.inter
    wt = _wtype_of(desc, set_)
    if wt != MOE_W_BF16:
        per = 2 if wt == MOE_W_NVFP4 else 4        # codes per byte
        arrs = [np.empty((count, 2 * I, H // per), np.uint8), np.empty((count, 2 * I, H // 16), np.uint8),
                np.empty((count, H, I // per), np.uint8), np.empty((count, H, I // 16), np.uint8),
                np.empty((count, 2), np.float32)]
    else:
        arrs = [np.empty((count, 2 * I, H), np.uint16), None, np.empty((count, H, I), np.uint16), None, None]
    _check("moe_unpack_experts", lib.moe_unpack_experts(C.byref(desc), int(set_), first, count, _ptr(region),
                                                        _ptr(scale_region), *[_ptr(a) for a in arrs]))
    if arrs[1] is not None:
        return [{"codes13": arrs[0][i], "scales13": arrs[1][i], "codes2": arrs[2][i], "scales2": arrs[3][i],
                 "g13": arrs[4][i, 0], "g2": arrs[4][i, 1]} for i in range(count)]
    return [{"w13": arrs[0][i], "w2": arrs[2][i]} for i in range(count)]


def moe_pack_nvfp4(codes: np.ndarray, scales: np.ndarray, codes_out=None, scales_out=None):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, half = codes.shape
    codes_out = np.empty(codes.size, np.uint8) if codes_out is None else codes_out
    scales_out = np.empty(scales.size, np.uint8) if scales_out is None else scales_out
    assert codes_out.nbytes >= codes.nbytes and scales_out.nbytes >= scales.nbytes
    _check("moe_pack_nvfp4", lib.moe_pack_nvfp4(rows, 2 * half, _ptr(codes), _ptr(scales),
                                                _ptr(codes_out), _ptr(scales_out)))
    return codes_out, scales_out


def moe_unpack_nvfp4(rows: int, cols: int, codes_p: np.ndarray, scales_p: np.ndarray):
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 16), np.uint8)
    _check("moe_unpack_nvfp4", lib.moe_unpack_nvfp4(rows, cols, _ptr(np.ascontiguousarray(codes_p)),
                                                    _ptr(np.ascontiguousarray(scales_p)),
                                                    _ptr(codes), _ptr(scales)))
    return codes, scales


def moe_pack_bf16(w: np.ndarray, w_out=None):
    w = np.ascontiguousarray(w, dtype=np.uint16)
    rows, cols = w.shape
    w_out = np.empty(w.size, np.uint16) if w_out is None else w_out
    assert w_out.nbytes >= w.nbytes
    _check("moe_pack_bf16", lib.moe_pack_bf16(rows, cols, _ptr(w), _ptr(w_out)))
    return w_out


def moe_unpack_bf16(rows: int, cols: int, w_p: np.ndarray):
    w = np.empty((rows, cols), np.uint16)
    _check("moe_unpack_bf16", lib.moe_unpack_bf16(rows, cols, _ptr(np.ascontiguousarray(w_p)), _ptr(w)))
    return w


# ---- device entry points --------------------------------------------------------------

def moe_layer_create(desc: moe_layer_desc) -> int:
    h = C.c_void_p()
    _check("moe_layer_create", lib.moe_layer_create(C.byref(desc), C.byref(h)))
    return h.value


def moe_layer_destroy(handle: int) -> None:
    _check("moe_layer_destroy", lib.moe_layer_destroy(handle))


def moe_decode_layer(handle, x, router_w, expert_packed, scales, shared_w, out, batch, stream=None) -> None:
    _check("moe_decode_layer", lib.moe_decode_layer(handle, _ptr(x), _ptr(router_w), _ptr(expert_packed),
                                                    _ptr(scales), _ptr(shared_w), _ptr(out), int(batch),
                                                    _stream(stream)))


def moe_decode_layer_static(desc: moe_layer_desc, x, router_w, expert_packed, scales, shared_w, out, batch,
                            err_flags=None, stream=None) -> None:
    _check("moe_decode_layer_static",
           lib.moe_decode_layer_static(C.byref(desc), _ptr(x), _ptr(router_w), _ptr(expert_packed), _ptr(scales),
                                       _ptr(shared_w), _ptr(out), int(batch), _ptr(err_flags), _stream(stream)))


def moe_layer_routing(handle, ids=None, w=None, c=None, stream=None) -> None:
    _check("moe_layer_routing", lib.moe_layer_routing(handle, _ptr(ids), _ptr(w), _ptr(c), _stream(stream)))


def moe_layer_set_profiling(handle, events, n_events: int) -> None:
    """events: a ctypes array of hipEvent_t pointers (or None to turn profiling off)."""
    _check("moe_layer_set_profiling", lib.moe_layer_set_profiling(handle, events, int(n_events)))


def moe_layer_debug_h(handle, h_routed=None, h_shared=None, stream=None) -> None:
    _check("moe_layer_debug_h", lib.moe_layer_debug_h(handle, _ptr(h_routed), _ptr(h_shared), _stream(stream)))


MOE_PATH_AUTO, MOE_PATH_GENERAL, MOE_PATH_DEDICATED = 0, 1, 2
MOE_MAX_CHAIN = 16


def moe_decode_chain(handles, x, router_w, expert_packed, scales, shared_w, out, batch: int, stream=None) -> None:
    """handles and the four weight arguments: sequences of one entry per layer."""
    n = len(handles)
    arr = lambda items: (C.c_void_p * n)(*[_ptr(t) for t in items])   # noqa: E731
    hs = (C.c_void_p * n)(*handles)
    _check("moe_decode_chain", lib.moe_decode_chain(hs, n, _ptr(x), arr(router_w), arr(expert_packed), arr(scales),
                                                    arr(shared_w), _ptr(out), int(batch), _stream(stream)))


def moe_requant_2bit(codes, scales):
    """NVFP4 canonical (codes uint8 [R, K/2], e4m3 scales [R, K/16]) -> the 2-bit
    planes (codes uint8 [R, K/4], e4m3 scales [R, K/16]), on the host."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    R, K = codes.shape[0], 2 * codes.shape[1]
    q = np.empty((R, K // 4), dtype=np.uint8)
    s2 = np.empty((R, K // 16), dtype=np.uint8)
    _check("moe_requant_2bit", lib.moe_requant_2bit(R, K, _ptr(codes), _ptr(scales), _ptr(q), _ptr(s2)))
    return q, s2


MOE_PREFILL_MAX_TOKENS = 65536


def moe_prefill_workspace_bytes(handle, tokens: int) -> int:
    n = C.c_size_t(0)
    _check("moe_prefill_workspace_bytes", lib.moe_prefill_workspace_bytes(handle, int(tokens), C.byref(n)))
    return int(n.value)


def moe_prefill_layer(handle, x, router_w, expert_packed, scales, shared_w, out, tokens: int, workspace,
                      workspace_bytes: int, topk_ids=None, topk_w=None, stream=None) -> None:
    _check("moe_prefill_layer",
           lib.moe_prefill_layer(handle, _ptr(x), _ptr(router_w), _ptr(expert_packed), _ptr(scales), _ptr(shared_w),
                                 _ptr(out), int(tokens), _ptr(workspace), int(workspace_bytes), _ptr(topk_ids),
                                 _ptr(topk_w), _stream(stream)))


def moe_layer_set_path(handle, path: int) -> int:
    """Kernels of the handle's calls (MOE_PATH_AUTO or MOE_PATH_GENERAL);
    returns the path in force (MOE_PATH_DEDICATED or MOE_PATH_GENERAL)."""
    active = C.c_int(-1)
    _check("moe_layer_set_path", lib.moe_layer_set_path(handle, int(path), C.byref(active)))
    return active.value


def moe_layer_error(handle, clear: bool = False) -> int:
    """Sticky error bits of the handle (waits for the device)."""
    flags = C.c_uint(0)
    _check("moe_layer_error", lib.moe_layer_error(handle, C.byref(flags), int(bool(clear))))
    return int(flags.value)


def moe_layer_reset(handle) -> None:
    _check("moe_layer_reset", lib.moe_layer_reset(handle))


def moe_layer_grid(handle) -> tuple[int, int]:
    """(workgroups of the layer kernel, shared-memory bytes per workgroup at max_batch)."""
    g, l = C.c_int(0), C.c_int(0)
    _check("moe_layer_grid", lib.moe_layer_grid(handle, C.byref(g), C.byref(l)))
    return int(g.value), int(l.value)


# ---- measurement utilities (include/moe_bench.h) -----------------------------------------

def moe_bench_read_stream(buf, sink, stream=None) -> None:
    _check("moe_bench_read_stream", lib.moe_bench_read_stream(_ptr(buf), buf.numel() * buf.element_size(),
                                                              _ptr(sink), _stream(stream)))


def moe_bench_fill(buf, value: int = 0, stream=None) -> None:
    _check("moe_bench_fill", lib.moe_bench_fill(_ptr(buf), buf.numel() * buf.element_size(), int(value),
                                                _stream(stream)))


def moe_bench_empty(workgroups: int, stream=None) -> None:
    _check("moe_bench_empty", lib.moe_bench_empty(int(workgroups), _stream(stream)))


# ---- small-batch dense NVFP4 GEMV ----------------------------------------------------

def moe_dense_layout_query(rows: int, cols: int) -> dict:
    lay = moe_dense_layout()
    _check("moe_dense_layout_query", lib.moe_dense_layout_query(int(rows), int(cols), C.byref(lay)))
    return lay.as_dict()


def moe_pack_dense(codes: np.ndarray, scales: np.ndarray, tensor_scale: float):
    """Canonical NVFP4 matrix (codes uint8 [rows][cols/2], scales uint8 [rows][cols/16])
    -> (code_region, scale_region) host arrays."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, cols = codes.shape[0], 2 * codes.shape[1]
    lay = moe_dense_layout_query(rows, cols)
    cr = np.zeros(lay["code_bytes"], dtype=np.uint8)
    sr = np.zeros(lay["scale_region_bytes"], dtype=np.uint8)
    _check("moe_pack_dense", lib.moe_pack_dense(rows, cols, _ptr(codes), _ptr(scales), float(tensor_scale),
                                                _ptr(cr), _ptr(sr)))
    return cr, sr


def moe_unpack_dense(rows: int, cols: int, code_region: np.ndarray, scale_region: np.ndarray):
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    scales = np.zeros((rows, cols // 16), dtype=np.uint8)
    ts = C.c_float(0.0)
    _check("moe_unpack_dense", lib.moe_unpack_dense(int(rows), int(cols), _ptr(code_region), _ptr(scale_region),
                                                    _ptr(codes), _ptr(scales), C.byref(ts)))
    return codes, scales, ts.value


def moe_dense_gemv(rows: int, cols: int, code_region, scale_region, x, y, batch: int, stream=None) -> None:
    _check("moe_dense_gemv", lib.moe_dense_gemv(int(rows), int(cols), _ptr(code_region), _ptr(scale_region),
                                                _ptr(x), _ptr(y), int(batch), _stream(stream)))
