"""Seeded synthetic MoE decode layers (inputs for tests and benchmarks).

This module only draws random inputs and stores them in the canonical
byte formats; it holds none of the layer's arithmetic, and neither the
oracle nor the HIP library imports it.  Both sides receive the same arrays
from it.

Canonical stored formats (what both sides read)
  * bf16 tensors: uint16 bit patterns.
  * NVFP4 matrix [R, K]: codes uint8 [R, K/2] (element 2j in the low nibble
    of byte j, 2j+1 in the high nibble), e4m3 block scales uint8 [R, K/16]
    (block b = columns 16b..16b+15), one fp32 tensor scale.
  * expert: gate/up matrix W13 [2I, H] (gate rows first) and down matrix
    W2 [H, I].

Workloads (shapes from the Flint page, "A 40B MoE that activates 2.5B
parameters", and the Inkling page, "Model Architecture"; value
distributions as stated with each entry of WORKLOADS).  Every tensor is
drawn from numpy's default_rng seeded with
SeedSequence([1234, workload_id, slot, tensor_id, index]), so any expert of
any slot can be regenerated on its own without holding the layer in memory.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

_ROOT_SEED = 1234

# tensor ids inside a seed sequence
_T_ROUTER, _T_BIAS, _T_X = 0, 1, 3
_T_CODES13, _T_SCALES13, _T_CODES2, _T_SCALES2 = 10, 11, 12, 13
_T_BF13, _T_BF2 = 14, 15
_T_TSCALE = 16
_SHARED_OFFSET = 100  # shared expert s uses index _SHARED_OFFSET + s


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    hidden: int
    inter: int
    n_routed: int
    top_k: int
    n_shared: int
    batch: int
    route: str = "sigmoid"            # "sigmoid" | "sink"
    routed_wtype: str = "nvfp4"       # "nvfp4" | "bf16" | "2bit"
    shared_wtype: str = "nvfp4"
    router_std: float = 0.02          # None -> 1/sqrt(hidden)
    bias_std: float | None = None     # per-expert router bias, fp32
    prenorm: bool = False             # RMSNorm prologue + residual
    eps: float = 1e-6
    bf16_std: float = 0.02            # bf16 expert weights
    scale_mult: float = 0.05          # e4m3 block scale = |N(0,1)| * scale_mult
    description: str = field(default="", compare=False)


WORKLOADS = {
    "tiny": Workload(0, "tiny", 256, 128, 16, 2, 1, 1,
                     description="tiny: H=256 I=128 E=16 top-2 + 1 shared, NVFP4, b1"),
    "flint_b1": Workload(1, "flint_b1", 2048, 512, 256, 6, 1, 1,
                         description="Flint-shaped: H=2048 I=512 E=256 top-6 + 1 shared, NVFP4, b1"),
    "flint_b8": Workload(2, "flint_b8", 2048, 512, 256, 6, 1, 8,
                         router_std=None, bias_std=0.5,
                         description="Flint-shaped NVFP4, b8, router N(0,1/sqrt(H)) + bias N(0,0.5)"),
    "flint_bf16_b1": Workload(3, "flint_bf16_b1", 2048, 512, 256, 6, 1, 1,
                              routed_wtype="bf16", shared_wtype="bf16",
                              description="Flint-shaped, BF16 experts N(0,0.02), b1"),
    "flint_bf16_b8": Workload(3, "flint_bf16_b8", 2048, 512, 256, 6, 1, 8,
                              routed_wtype="bf16", shared_wtype="bf16",
                              description="Flint-shaped, BF16 experts N(0,0.02), b8"),
    "flint_chain": Workload(5, "flint_chain", 2048, 512, 256, 6, 1, 1,
                            prenorm=True,
                            description="Flint-shaped NVFP4 layer with pre-norm RMSNorm and residual, b1"),
    "flint_2bit_b1": Workload(10, "flint_2bit_b1", 2048, 512, 256, 6, 1, 1, routed_wtype="2bit",
                              description="Flint-shaped: H=2048 I=512 E=256 top-6, routed experts in 2-bit "
                                          "sign-symmetric planes, 1 NVFP4 shared, b1"),
    "flint_2bit_b8": Workload(11, "flint_2bit_b8", 2048, 512, 256, 6, 1, 8, routed_wtype="2bit",
                              router_std=None, bias_std=0.5,
                              description="Flint-shaped: H=2048 I=512 E=256 top-6, routed experts in 2-bit "
                                          "sign-symmetric planes, 1 NVFP4 shared, b8, router N(0,1/sqrt(H)) + "
                                          "bias N(0,0.5)"),
    "sink_b4": Workload(4, "sink_b4", 7168, 2048, 256, 6, 2, 4,
                        route="sink", shared_wtype="bf16",
                        description="expert sink: H=7168 I=2048 E=256 NVFP4 top-6 + 2 BF16 shared in a 258-way softmax, b4"),
}


def _rng(wid: int, slot: int, tensor: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([_ROOT_SEED, wid, slot, tensor, index]))


def to_bf16_bits(a) -> np.ndarray:
    """float -> bf16 bit patterns, round to nearest even (torch's cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_e4m3_bytes(a) -> np.ndarray:
    """float -> e4m3 (FN) bytes, round to nearest even (torch's cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


class ArrayLayer:
    """A layer given by explicit canonical arrays (used for crafted cases).

    routed: list of per-expert dicts, shared: list of per-expert dicts; each
    dict holds codes13/scales13/codes2/scales2/g13/g2 (nvfp4) or w13/w2
    (bf16).
    """

    def __init__(self, *, hidden, inter, top_k, router_w, routed, shared,
                 route="sigmoid", routed_wtype="nvfp4", shared_wtype="nvfp4",
                 router_bias=None, gamma=None, eps=1e-6, residual=False):
        self.hidden, self.inter, self.top_k = hidden, inter, top_k
        self.n_routed, self.n_shared = len(routed), len(shared)
        self.route, self.routed_wtype, self.shared_wtype = route, routed_wtype, shared_wtype
        self.router_w = np.asarray(router_w, dtype=np.uint16)
        self.router_bias = None if router_bias is None else np.asarray(router_bias, np.float32)
        self.gamma = None if gamma is None else np.asarray(gamma, dtype=np.uint16)
        self.eps, self.residual = eps, residual
        self._routed, self._shared = routed, shared

    def routed_tensor_scales(self, e: int) -> tuple:
        """(W13, W2) fp32 tensor scales of routed expert e (NVFP4), without drawing its codes."""
        return self._tscale(e, 0), self._tscale(e, 1)

    def shared_tensor_scales(self, s: int) -> tuple:
        return self._tscale(_SHARED_OFFSET + s, 0), self._tscale(_SHARED_OFFSET + s, 1)

    def routed_expert(self, e: int) -> dict:
        return self._routed[e]

    def shared_expert(self, s: int) -> dict:
        return self._shared[s]


class SynthLayer:
    """One seeded synthetic layer of a workload; experts are drawn on demand."""

    def __init__(self, workload: Workload | str, slot: int = 0, tscale_set=None):
        """tscale_set: optional values from which each NVFP4 expert's two fp32
        tensor scales (W13, W2) are drawn, seeded per expert; default 1.0 (the
        workloads' stated distribution)."""
        if isinstance(workload, str):
            workload = WORKLOADS[workload]
        wl = workload
        self.wl, self.slot = wl, slot
        self.tscale_set = None if tscale_set is None else np.asarray(tscale_set, np.float32)
        self.hidden, self.inter = wl.hidden, wl.inter
        self.n_routed, self.top_k, self.n_shared = wl.n_routed, wl.top_k, wl.n_shared
        self.route = wl.route
        self.routed_wtype, self.shared_wtype = wl.routed_wtype, wl.shared_wtype
        self.eps, self.residual = wl.eps, wl.prenorm
        n_rows = wl.n_routed + (wl.n_shared if wl.route == "sink" else 0)
        std = wl.router_std if wl.router_std is not None else 1.0 / np.sqrt(wl.hidden)
        r = _rng(wl.wid, slot, _T_ROUTER)
        self.router_w = to_bf16_bits(r.normal(0.0, std, size=(n_rows, wl.hidden)))
        if wl.bias_std is not None:
            self.router_bias = _rng(wl.wid, slot, _T_BIAS).normal(
                0.0, wl.bias_std, size=wl.n_routed).astype(np.float32)
        else:
            self.router_bias = None
        self.gamma = (np.full(wl.hidden, 0x3F80, dtype=np.uint16) if wl.prenorm else None)

    # -- experts ------------------------------------------------------------
    def _nvfp4_expert(self, index: int) -> dict:
        wl, H, I = self.wl, self.hidden, self.inter
        w = wl.wid

        def scales(tid, shape):
            a = np.abs(_rng(w, self.slot, tid, index).standard_normal(size=shape, dtype=np.float32))
            a *= np.float32(wl.scale_mult)
            return to_e4m3_bytes(a)

        return {
            "codes13": _rng(w, self.slot, _T_CODES13, index).integers(
                0, 256, size=(2 * I, H // 2), dtype=np.uint8),
            "scales13": scales(_T_SCALES13, (2 * I, H // 16)),
            "codes2": _rng(w, self.slot, _T_CODES2, index).integers(
                0, 256, size=(H, I // 2), dtype=np.uint8),
            "scales2": scales(_T_SCALES2, (H, I // 16)),
            "g13": self._tscale(index, 0),
            "g2": self._tscale(index, 1),
        }

    def _2bit_expert(self, index: int) -> dict:
        """The sign-symmetric 2-bit planes: codes uniform over the four levels,
        e4m3 block scales drawn as for NVFP4."""
        wl, H, I = self.wl, self.hidden, self.inter
        w = wl.wid

        def scales(tid, shape):
            a = np.abs(_rng(w, self.slot, tid, index).standard_normal(size=shape, dtype=np.float32))
            a *= np.float32(wl.scale_mult)
            return to_e4m3_bytes(a)

        return {
            "codes13": _rng(w, self.slot, _T_CODES13, index).integers(0, 256, size=(2 * I, H // 4), dtype=np.uint8),
            "scales13": scales(_T_SCALES13, (2 * I, H // 16)),
            "codes2": _rng(w, self.slot, _T_CODES2, index).integers(0, 256, size=(H, I // 4), dtype=np.uint8),
            "scales2": scales(_T_SCALES2, (H, I // 16)),
            "g13": self._tscale(index, 0),
            "g2": self._tscale(index, 1),
        }

    def _tscale(self, index: int, which: int) -> np.float32:
        if self.tscale_set is None:
            return np.float32(1.0)
        pick = _rng(self.wl.wid, self.slot, _T_TSCALE, index).integers(0, self.tscale_set.size, size=2)
        return np.float32(self.tscale_set[pick[which]])

    def _bf16_expert(self, index: int) -> dict:
        wl, H, I = self.wl, self.hidden, self.inter
        r13 = _rng(wl.wid, self.slot, _T_BF13, index)
        r2 = _rng(wl.wid, self.slot, _T_BF2, index)
        return {
            "w13": to_bf16_bits(r13.standard_normal(size=(2 * I, H), dtype=np.float32) * np.float32(wl.bf16_std)),
            "w2": to_bf16_bits(r2.standard_normal(size=(H, I), dtype=np.float32) * np.float32(wl.bf16_std)),
        }

    def routed_tensor_scales(self, e: int) -> tuple:
        """(W13, W2) fp32 tensor scales of routed expert e (NVFP4), without drawing its codes."""
        return self._tscale(e, 0), self._tscale(e, 1)

    def shared_tensor_scales(self, s: int) -> tuple:
        return self._tscale(_SHARED_OFFSET + s, 0), self._tscale(_SHARED_OFFSET + s, 1)

    def routed_expert(self, e: int) -> dict:
        if not 0 <= e < self.n_routed:
            raise IndexError(e)
        if self.routed_wtype == "2bit":
            return self._2bit_expert(e)
        return (self._nvfp4_expert(e) if self.routed_wtype == "nvfp4"
                else self._bf16_expert(e))

    def shared_expert(self, s: int) -> dict:
        if not 0 <= s < self.n_shared:
            raise IndexError(s)
        idx = _SHARED_OFFSET + s
        return (self._nvfp4_expert(idx) if self.shared_wtype == "nvfp4"
                else self._bf16_expert(idx))

    # -- activations --------------------------------------------------------
    def x(self, step: int = 0, batch: int | None = None) -> np.ndarray:
        """bf16 bits [batch, H] of N(0,1) activations for one step."""
        b = self.wl.batch if batch is None else batch
        r = _rng(self.wl.wid, self.slot, _T_X, step)
        return to_bf16_bits(r.standard_normal(size=(b, self.hidden)))
