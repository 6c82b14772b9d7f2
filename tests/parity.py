"""Comparison of the HIP layer against the oracle (used by the GPU tests,
smoke() and bench.py's spot checks).

Acceptance (for every layer output):
  * the selected expert set of each token matches the oracle's exactly,
    except for tokens whose oracle k-th/(k+1)-th score gap is below 1e-5;
    such tokens are reported and compared against the oracle re-run with
    the GPU's selection forced;
  * max |gpu - oracle| <= 1e-2 * max |oracle| over the [batch, hidden]
    output of the layer.
"""

from __future__ import annotations

import numpy as np

import oracle
from quantized_expert_gemv_amd.device_layer import bf16_tensor_to_bits, bits_to_bf16_tensor

GAP_EPS = 1e-5
OUT_TOL = 1e-2


def bf16_bits_f64(bits) -> np.ndarray:
    return oracle.bf16_bits_to_f64(bits)


def compare_layer(dev, layer, x_bits: np.ndarray, tokens=None, tol: float = OUT_TOL) -> dict:
    """Run the device layer on x_bits and compare with the oracle.

    tokens: optional subset of token rows for the oracle (the GPU still runs
    the whole batch); tokens are independent, so the oracle on a subset of
    rows gives exactly those rows' outputs.
    """
    import torch
    B = x_bits.shape[0]
    x = bits_to_bf16_tensor(x_bits, dev.device)
    out = dev(x)
    ids, w, c = dev.routing(B)
    torch.cuda.synchronize()
    flags = dev.error()
    assert flags == 0, f"layer kernel reported error bits {flags:#x} (a wait for another workgroup timed out)"
    out_f = bf16_bits_f64(bf16_tensor_to_bits(out))
    ids_g, w_g, c_g = ids.cpu().numpy(), w.cpu().numpy(), c.cpu().numpy()

    rows = list(range(B)) if tokens is None else list(tokens)
    ref = oracle.moe_layer(layer, x_bits[rows])
    exempt, mismatched = [], []
    for i, b in enumerate(rows):
        if set(ids_g[b].tolist()) != set(ref["ids"][i].tolist()):
            if ref["gaps"][i] < GAP_EPS:
                exempt.append(b)
            else:
                mismatched.append(b)
    if exempt:
        forced = np.array([ids_g[b] for b in rows])
        ref_out = oracle.moe_layer(layer, x_bits[rows], force_ids=forced)["out"]
    else:
        ref_out = ref["out"]
    got = out_f[rows]
    scale = float(np.max(np.abs(ref_out)))
    err = float(np.max(np.abs(got - ref_out)))
    row_err = np.max(np.abs(got - ref_out), axis=1) / np.maximum(np.max(np.abs(ref_out), axis=1), 1e-30)

    # routing weights of matched tokens, in the GPU's selection order
    w_err = 0.0
    for i, b in enumerate(rows):
        if b in exempt or b in mismatched:
            continue
        ref_w = dict(zip(ref["ids"][i].tolist(), ref["w"][i].tolist()))
        for e, wv in zip(ids_g[b].tolist(), w_g[b].tolist()):
            w_err = max(w_err, abs(wv - ref_w[e]))
        if ref["c"].shape[1]:
            w_err = max(w_err, float(np.max(np.abs(c_g[b] - ref["c"][i]))))
    return {
        "out": out, "out_f": out_f, "ids": ids_g, "w": w_g, "c": c_g, "ref": ref, "ref_out": ref_out,
        "rows": rows, "exempt": exempt, "mismatched": mismatched, "max_err": err, "max_ref": scale,
        "rel_err": err / max(scale, 1e-30), "row_rel_err": row_err, "w_err": w_err,
        "ok": (not mismatched) and err <= tol * scale,
    }
