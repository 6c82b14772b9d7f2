"""The MoE decode layer, evaluated from its definition in float64 (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources
  * "vLLM adds day-0 support for Recursive's Flint ...", section "A 40B MoE
    that activates 2.5B parameters": a pre-norm MoE, hidden 2048, 256
    experts with sigmoid top-6 routing plus one shared expert; weight-only
    NVFP4 with BF16 activations.
  * same page, section "From 1,096 kernels to 346": the router and expert
    GEMVs fetch no bytes of experts outside the top-k; routing and the expert
    combine sit next to the GEMVs.
  * "TML Inkling on vLLM ...", section "Model Architecture" (MoE paragraph):
    the two shared experts take part in the routing-score computation and
    absorb probability mass, but are never candidates for the top-6.

Readings adopted where the pages are silent
  * sigmoid mode: s = sigmoid(l + bias); the top-k is taken on l + bias
    (sigmoid is strictly increasing, so the set is the same), exact ties go
    to the lower expert index; the weights are renormalised,
    w = s_T / sum(s_T); no extra scaling factor; the shared expert's
    coefficient is 1.
  * sink mode: p = softmax over all E + S router logits; the top-k is taken
    over the routed part only; routed weights are the selected
    probabilities (no renormalisation); shared expert s is weighted by its
    own probability p[E + s].
  * expert MLP: rows [0, I) of the fused gate/up matrix are the gate, rows
    [I, 2I) the up projection; h = SiLU(gate) * up with SiLU(g) = g*sigmoid(g)
    and no clamp; y = W2 h.
  * pre-norm (2-layer chain only): xhat = x / sqrt(mean(x^2) + eps) * gamma,
    and the layer output is x + MoE(xhat).
  * every token of a batch is independent of the others.

No rounding is applied anywhere: inputs are the exact values of the stored
bytes and every step is float64.
"""

from __future__ import annotations

import math

import numpy as np

from .codec2 import dequant_2bit
from .formats import bf16_bits_to_f64, dequant_bf16, dequant_nvfp4


def rmsnorm(x: np.ndarray, gamma: np.ndarray | None, eps: float) -> np.ndarray:
    """Pre-norm RMSNorm of each row of x (float64).

    Flint page, section "A 40B MoE ...": the model is a pre-norm MoE.
    xhat = x / sqrt(mean(x^2) + eps) * gamma.
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    y = x / np.sqrt(ms + eps)
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64)
    return y


def router_logits(xhat: np.ndarray, router_w: np.ndarray,
                  bias: np.ndarray | None = None) -> np.ndarray:
    """Router GEMV: l[b, e] = sum_h xhat[b, h] * R[e, h] (+ bias[e]).

    Flint page, section "From 1,096 kernels to 346" (router GEMV).
    router_w is float64 [E_r, H]; a bias of length E is added to the first E
    logits (the routed experts).
    """
    l = np.asarray(xhat, dtype=np.float64) @ np.asarray(router_w, dtype=np.float64).T
    if bias is not None:
        b = np.asarray(bias, dtype=np.float64)
        l[..., : b.shape[0]] += b
    return l


def _topk_desc(keys: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest keys, largest first; equal keys in
    ascending index order."""
    keys = np.asarray(keys, dtype=np.float64)
    order = np.lexsort((np.arange(keys.shape[0]), -keys))
    return order[:k]


def _sigmoid(v):
    """Logistic function 1 / (1 + exp(-v)), written so that exp never
    overflows: for v < 0 it is evaluated as exp(v) / (1 + exp(v))."""
    v = np.asarray(v, dtype=np.float64)
    e = np.exp(-np.abs(v))
    return np.where(v >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def route_sigmoid_topk(logits: np.ndarray, k: int, n_shared: int):
    """Sigmoid top-k with renormalised weights, for one token.

    Flint page, section "A 40B MoE ...": "sigmoid top-6 routing plus a
    shared expert".  Returns (ids in selection order, weights, shared
    coefficients, scores) where scores = sigmoid(logits).
    """
    logits = np.asarray(logits, dtype=np.float64)
    ids = _topk_desc(logits, k)
    s = _sigmoid(logits)
    w = s[ids] / np.sum(s[ids])
    c = np.ones(n_shared, dtype=np.float64)
    return ids, w, c, s


def route_softmax_sink(logits: np.ndarray, n_routed: int, k: int):
    """Expert-sink routing for one token.

    Inkling page, section "Model Architecture": the shared experts join the
    routing-score computation but are excluded from the top-k.  The softmax
    runs over all E + S logits; the top-k is taken over the first E.
    Returns (ids, weights = selected probabilities, shared coefficients =
    the shared experts' probabilities, routed probabilities).
    """
    logits = np.asarray(logits, dtype=np.float64)
    z = np.exp(logits - np.max(logits))
    p = z / np.sum(z)
    ids = _topk_desc(logits[:n_routed], k)
    return ids, p[ids], p[n_routed:].copy(), p[:n_routed]


def selection_gap(scores: np.ndarray, k: int) -> float:
    """Gap between the k-th and (k+1)-th largest score (inf if k == E).

    Used to exempt near-tied tokens from the exact-selection check.
    """
    s = np.sort(np.asarray(scores, dtype=np.float64))[::-1]
    if k >= s.shape[0]:
        return math.inf
    return float(s[k - 1] - s[k])


def expert_mlp(w13: np.ndarray, w2: np.ndarray, xhat: np.ndarray):
    """SiLU-gated expert MLP on one token.

    w13 : float64 [2I, H] (gate rows then up rows), w2 : float64 [H, I].
    gate = w13[:I] x, up = w13[I:] x, h = SiLU(gate) * up, y = w2 h.
    Returns (h, y).
    """
    I2 = w13.shape[0]
    I = I2 // 2
    gu = w13 @ np.asarray(xhat, dtype=np.float64)
    g, u = gu[:I], gu[I:]
    h = g * _sigmoid(g) * u
    y = w2 @ h
    return h, y


def _dequant_expert(mats: dict, wtype: str):
    if wtype == "nvfp4":
        w13 = dequant_nvfp4(mats["codes13"], mats["scales13"], mats["g13"])
        w2 = dequant_nvfp4(mats["codes2"], mats["scales2"], mats["g2"])
    elif wtype == "bf16":
        w13 = dequant_bf16(mats["w13"])
        w2 = dequant_bf16(mats["w2"])
    elif wtype == "2bit":
        w13 = dequant_2bit(mats["codes13"], mats["scales13"], mats["g13"])
        w2 = dequant_2bit(mats["codes2"], mats["scales2"], mats["g2"])
    else:
        raise ValueError(f"unknown weight type {wtype!r}")
    return w13, w2


def moe_layer(layer, x_bits, force_ids=None) -> dict:
    """Evaluate one MoE decode layer for a batch of tokens.

    ``layer`` supplies: hidden, inter, n_routed, top_k, n_shared, route
    ("sigmoid" or "sink"), routed_wtype / shared_wtype ("nvfp4", "bf16", or
    for the routed set "2bit", the sign-symmetric planes of codec2),
    router_w (uint16 bf16 bits [E_r, H]), router_bias (float32 [E] or None),
    gamma (uint16 bf16 bits [H] or None), eps, residual (bool), and the
    accessors routed_expert(e) / shared_expert(s) returning the canonical
    stored arrays of one expert.

    x_bits: uint16 bf16 bits [B, H].
    force_ids: optional [B, k] selection to use instead of the top-k (the
    re-run for near-tied tokens).

    Returns a dict with out [B, H] (float64, unrounded), logits, ids, w, c,
    scores, gaps, xhat and the per-(token, expert) h and y vectors.
    """
    x = bf16_bits_to_f64(x_bits)
    B, H = x.shape
    k, E, S = layer.top_k, layer.n_routed, layer.n_shared
    if layer.gamma is not None:
        xhat = rmsnorm(x, bf16_bits_to_f64(layer.gamma), layer.eps)
    else:
        xhat = x
    R = bf16_bits_to_f64(layer.router_w)
    logits = router_logits(xhat, R, layer.router_bias)

    ids = np.zeros((B, k), dtype=np.int64)
    w = np.zeros((B, k))
    c = np.zeros((B, S))
    gaps = np.zeros(B)
    scores = []
    for b in range(B):
        if layer.route == "sigmoid":
            i_b, w_b, c_b, s_b = route_sigmoid_topk(logits[b], k, S)
        elif layer.route == "sink":
            i_b, w_b, c_b, s_b = route_softmax_sink(logits[b], E, k)
        else:
            raise ValueError(f"unknown routing {layer.route!r}")
        gaps[b] = selection_gap(s_b, k)
        if force_ids is not None:
            i_b = np.asarray(force_ids[b], dtype=np.int64)
            if layer.route == "sigmoid":
                w_b = s_b[i_b] / np.sum(s_b[i_b])
            else:
                w_b = s_b[i_b]
        ids[b], w[b], c[b] = i_b, w_b, c_b
        scores.append(s_b)

    # Dequantise each distinct expert once, apply it to every token that uses
    # it, and release it before the next (only selected experts are touched).
    uses: dict = {}
    for b in range(B):
        for j in range(k):
            uses.setdefault(int(ids[b, j]), []).append((b, j))
    y_routed = np.zeros((B, k, H))
    y_shared = np.zeros((B, S, H))
    h_pairs, y_pairs = {}, {}
    for e in sorted(uses):
        w13, w2 = _dequant_expert(layer.routed_expert(e), layer.routed_wtype)
        for b, j in uses[e]:
            h, y = expert_mlp(w13, w2, xhat[b])
            h_pairs[(b, e)], y_pairs[(b, e)] = h, y
            y_routed[b, j] = y
        del w13, w2
    for s in range(S):
        w13, w2 = _dequant_expert(layer.shared_expert(s), layer.shared_wtype)
        for b in range(B):
            h, y = expert_mlp(w13, w2, xhat[b])
            h_pairs[(b, "shared", s)], y_pairs[(b, "shared", s)] = h, y
            y_shared[b, s] = y
        del w13, w2

    # weighted combine: routed slots in selection order, then shared experts
    out = np.zeros((B, H))
    for b in range(B):
        acc = np.zeros(H)
        for j in range(k):
            acc = acc + w[b, j] * y_routed[b, j]
        for s in range(S):
            acc = acc + c[b, s] * y_shared[b, s]
        out[b] = acc + (x[b] if layer.residual else 0.0)

    return {
        "out": out, "logits": logits, "ids": ids, "w": w, "c": c,
        "scores": np.stack(scores), "gaps": gaps, "xhat": xhat,
        "h": h_pairs, "y": y_pairs,
    }
