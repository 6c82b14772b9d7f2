"""CPU fp64 oracle for the small-batch NVFP4 MoE decode layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import this
package: only the tests, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant with the HIP library; it reads the canonical stored bytes of a
layer (bf16 bit patterns, e2m1 nibbles, e4m3 scale bytes, fp32 tensor
scales) and evaluates the layer's plain definition in float64.

Modules
  formats  -- exact decoding of bf16, e2m1 (FP4) and e4m3 (FP8) bytes and
              NVFP4 dequantisation.
  layer    -- RMSNorm, router GEMV, the two routing rules, the SiLU-gated
              expert MLP and the weighted combine.
  dense    -- the small-batch dense NVFP4 GEMV y = x W^T.
  codec2   -- the sign-symmetric 2-bit expert planes: decoding and the
              re-quantisation from NVFP4.

Every function cites the page passage it follows.  Readings adopted where
the pages are silent are listed in the module docstrings.
"""

from .formats import (  # noqa: F401
    E2M1_MAGNITUDES_BY_DEFINITION,
    bf16_bits_to_f64,
    dequant_bf16,
    dequant_nvfp4,
    e2m1_value,
    e4m3_value,
    unpack_nibbles,
)
from .codec2 import dequant_2bit, nearest_codes, pack_2bit, requant_from_nvfp4, unpack_2bit  # noqa: F401
from .dense import dense_gemv  # noqa: F401
from .layer import (  # noqa: F401
    expert_mlp,
    moe_layer,
    rmsnorm,
    route_sigmoid_topk,
    route_softmax_sink,
    router_logits,
    selection_gap,
)
