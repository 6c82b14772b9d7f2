"""Load a layer's canonical bytes onto the GPU and call it through the C ABI.

``DeviceLayer(layer, max_batch)`` takes any object with the canonical-layer
attributes (see ``synth.SynthLayer`` / ``synth.ArrayLayer``), repacks every
expert with the library's lossless packers on the host, copies the packed
buffers to device memory owned by torch tensors, and creates a layer handle.
Calling it runs ``moe_decode_layer`` on the current torch stream.
"""

from __future__ import annotations

import numpy as np
import torch

from . import binding as B


def bits_to_bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def bf16_tensor_to_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def pack_expert_set(desc, set_: int, get_expert, n: int):
    """Host-side packing of one expert set of the layer `desc` describes, one
    expert at a time, by the library's set packer.

    Returns (region, scale region or None, layout): the routed set's code and
    scale regions, or the shared set's one buffer."""
    lay = B.moe_expert_layout_query(desc, set_)
    if set_ == B.MOE_SET_SHARED:
        region = np.zeros(max(lay["shared_total_bytes"], 16), np.uint8)
        scales = None
    else:
        region = np.zeros(max(lay["code_region_bytes"], 16), np.uint8)
        scales = np.zeros(max(lay["scale_region_bytes"], 16), np.uint8)
    for e in range(n):
        B.moe_pack_experts(desc, set_, e, [get_expert(e)], region, scales)
    return region, scales, lay


class DeviceLayer:
    def __init__(self, layer, max_batch: int, device="cuda"):
        self.layer = layer
        self.device = torch.device(device)
        H, I, E, S = layer.hidden, layer.inter, layer.n_routed, layer.n_shared
        self.H, self.I, self.E, self.S, self.k = H, I, E, S, layer.top_k
        self.max_batch = max_batch

        self.router_w = bits_to_bf16_tensor(layer.router_w, self.device)
        self.router_bias = (torch.from_numpy(np.asarray(layer.router_bias, np.float32)).to(self.device)
                            if layer.router_bias is not None else None)
        self.gamma = bits_to_bf16_tensor(layer.gamma, self.device) if layer.gamma is not None else None
        self.desc = B.make_desc(hidden=H, inter=I, n_routed=E, top_k=layer.top_k, n_shared=S,
                                max_batch=max_batch, routed_wtype=layer.routed_wtype,
                                shared_wtype=layer.shared_wtype, route=layer.route,
                                router_bias=self.router_bias, prenorm_gamma=self.gamma,
                                rms_eps=layer.eps, add_residual=layer.residual)
        codes, scales, self.layout_r = pack_expert_set(self.desc, B.MOE_SET_ROUTED, layer.routed_expert, E)
        self.expert_packed = torch.from_numpy(codes).to(self.device)
        self.scales = torch.from_numpy(scales).to(self.device) if layer.routed_wtype != "bf16" else None
        del codes, scales
        if S > 0:
            blob, _, self.layout_s = pack_expert_set(self.desc, B.MOE_SET_SHARED, layer.shared_expert, S)
            self.shared_w = torch.from_numpy(blob).to(self.device)
        else:
            self.layout_s, self.shared_w = None, None
        self.handle = B.moe_layer_create(self.desc)

    # buffers of this layer as the C ABI takes them (may be swapped for copies)
    def buffers(self) -> dict:
        return {"router_w": self.router_w, "expert_packed": self.expert_packed,
                "scales": self.scales, "shared_w": self.shared_w}

    def __call__(self, x: torch.Tensor, out: torch.Tensor | None = None, stream=None, bufs: dict | None = None):
        b = bufs or self.buffers()
        batch = x.shape[0]
        if out is None:
            out = torch.empty((batch, self.H), dtype=torch.bfloat16, device=self.device)
        B.moe_decode_layer(self.handle, x, b["router_w"], b["expert_packed"], b["scales"], b["shared_w"],
                           out, batch, stream)
        return out

    def prefill(self, x: torch.Tensor, out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                routing: bool = False, stream=None, bufs: dict | None = None):
        """The prefill path on x [T, H]: returns out (and the selection ids,
        weights [T, k] if routing).  workspace: a uint8 device tensor of at
        least moe_prefill_workspace_bytes, or None to allocate one here."""
        b = bufs or self.buffers()
        T = x.shape[0]
        if out is None:
            out = torch.empty((T, self.H), dtype=torch.bfloat16, device=self.device)
        need = B.moe_prefill_workspace_bytes(self.handle, T)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
        ids = torch.empty((T, self.k), dtype=torch.int32, device=self.device) if routing else None
        w = torch.empty((T, self.k), dtype=torch.float32, device=self.device) if routing else None
        B.moe_prefill_layer(self.handle, x, b["router_w"], b["expert_packed"], b["scales"], b["shared_w"], out, T,
                            workspace, workspace.numel(), ids, w, stream)
        return (out, ids, w) if routing else out

    def routing(self, batch: int):
        ids = torch.empty((batch, self.k), dtype=torch.int32, device=self.device)
        w = torch.empty((batch, self.k), dtype=torch.float32, device=self.device)
        c = torch.empty((batch, max(self.S, 1)), dtype=torch.float32, device=self.device)
        B.moe_layer_routing(self.handle, ids, w, c)
        return ids, w, c[:, :self.S]

    def debug_h(self, batch: int):
        hr = torch.empty((batch, self.k, self.I), dtype=torch.bfloat16, device=self.device)
        hs = torch.empty((batch, max(self.S, 1), self.I), dtype=torch.bfloat16, device=self.device)
        B.moe_layer_debug_h(self.handle, hr, hs)
        return hr, hs[:, :self.S]

    def set_path(self, path: str) -> str:
        """Kernels of later calls: "auto" or "general"; returns the path in force ("dedicated" or "general")."""
        code = {"auto": B.MOE_PATH_AUTO, "general": B.MOE_PATH_GENERAL}[path]
        return "dedicated" if B.moe_layer_set_path(self.handle, code) == B.MOE_PATH_DEDICATED else "general"

    def error(self, clear: bool = False) -> int:
        return B.moe_layer_error(self.handle, clear)

    def grid(self) -> tuple[int, int]:
        return B.moe_layer_grid(self.handle)

    def close(self):
        if getattr(self, "handle", None):
            B.moe_layer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
