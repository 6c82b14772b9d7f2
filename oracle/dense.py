"""Small-batch dense NVFP4 GEMV, evaluated from its definition in float64 (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources
  * "vLLM adds day-0 support for Recursive's Flint ...", section "From 1,096
    kernels to 346": a small-batch dense GEMV runs on the same packed NVFP4
    weights as the large-batch kernel; the model runs weight-only (W4A16)
    with BF16 activations (section "A 40B MoE that activates 2.5B
    parameters").
  * same page, section "A 40B MoE that activates 2.5B parameters": GQA with
    32 query and 4 KV heads at hidden size 2048, and a dense MLP in layers 0
    and 1 -- the dense GEMVs of a decode step.
  * "Frontier MoE on consumer Blackwell (SM120)", section "GLM-5.2 (753B) --
    the headline model": an NVFP4 weight is an e2m1 value times an e4m3
    scale per 16-element block times a per-tensor fp32 scale.

Readings adopted where the pages are silent
  * y[b, n] = sum_k W[n, k] * x[b, k]: the rows of W are the outputs, the
    block-16 scales run along k (the reduction), no bias.
  * the kernel stores y in bf16, one rounding of the exact sum (as every
    activation the layer stores); the oracle returns the exact float64 sum.
  * the tokens of a batch are independent.
"""

from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64, dequant_nvfp4


def dense_gemv(codes, scales, tensor_scale: float, x_bits) -> np.ndarray:
    """y = x W^T for one NVFP4 matrix W [N, K] and bf16 activations x [B, K].

    codes  : uint8 [N, K/2] e2m1 nibbles (canonical order), scales : uint8
    [N, K/16] e4m3 block scales, tensor_scale : fp32 per-tensor scale,
    x_bits : uint16 [B, K] bf16 bit patterns.  Returns float64 [B, N].
    """
    w = dequant_nvfp4(codes, scales, tensor_scale)          # [N, K], exact
    x = bf16_bits_to_f64(np.atleast_2d(x_bits))              # [B, K], exact
    if x.shape[1] != w.shape[1]:
        raise ValueError("x and W disagree on the reduction size")
    return x @ w.T
