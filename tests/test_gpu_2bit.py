"""GPU parity of the layer with routed experts in the sign-symmetric 2-bit
planes (moe_decode_layer, through the C ABI) against the fp64 oracle, at
batch 1 and at batch 2-8.

The layer is the Flint shape (H=2048, I=512, 256 routed experts, top-6, one
NVFP4 shared expert); the routed experts' codes are uniform over the four
levels {-4, -1, 1, 4} with e4m3 block scales drawn as for NVFP4.  Acceptance
is the decode path's: selection exact except near ties (gap < 1e-5), weights
within 1e-4, max |gpu - oracle| <= 1e-2 max |oracle|; plus the per-pair h of
the selected experts against the oracle's, distinct per-expert tensor scales,
bitwise repetition and the handle-less entry point.  At batch 2-8 the
workload is the batch-8 one (router N(0, 1/sqrt(H)) + bias N(0, 0.5), so the
tokens share some experts): batches 8, 3 and 2, distinct tensor scales, and
bitwise repetition.
"""

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from parity import compare_layer  # noqa: E402

TS_SET = (0.37, 0.7, 1.3, 2.0)
_DEVS = {}


def _note(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_expert_gemv_amd import device_layer  # noqa: F401  (raises if the library is not built)
    yield
    for _, d in _DEVS.values():
        d.close()
    _DEVS.clear()
    torch.cuda.synchronize()


def dev_of(tscales=False):
    from quantized_expert_gemv_amd.device_layer import DeviceLayer
    from quantized_expert_gemv_amd.synth import SynthLayer
    if tscales not in _DEVS:
        _note(f"[upload] flint_2bit_b1 tensor_scales={'distinct' if tscales else 'unit'}")
        layer = SynthLayer("flint_2bit_b1", tscale_set=TS_SET if tscales else None)
        dev = DeviceLayer(layer, 1)
        if dev.set_path("auto") != "dedicated":
            pytest.skip("2-bit experts run on the batch-1 kernel of the Flint shape (256 CUs)")
        _DEVS[tscales] = (layer, dev)
    return _DEVS[tscales]


def dev_b8(tscales=False):
    from quantized_expert_gemv_amd.device_layer import DeviceLayer
    from quantized_expert_gemv_amd.synth import SynthLayer
    key = ("b8", tscales)
    if key not in _DEVS:
        _note(f"[upload] flint_2bit_b8 tensor_scales={'distinct' if tscales else 'unit'}")
        layer = SynthLayer("flint_2bit_b8", tscale_set=TS_SET if tscales else None)
        dev = DeviceLayer(layer, 8)
        if dev.set_path("auto") != "dedicated":
            pytest.skip("2-bit experts run on the dedicated kernels of the Flint shape (256 CUs)")
        _DEVS[key] = (layer, dev)
    return _DEVS[key]


@pytest.mark.parametrize("step,batch", [(0, 8), (1, 8), (2, 3), (3, 2)])
def test_2bit_b8_meets_the_oracle(step, batch):
    layer, dev = dev_b8()
    r = compare_layer(dev, layer, layer.x(step, batch=batch))
    _note(f"[2bit b{batch}] step {step}: rel_err={r['rel_err']:.3e} w_err={r['w_err']:.2e} "
          f"mismatched={r['mismatched']} exempt={r['exempt']}")
    assert not r["mismatched"] and r["rel_err"] <= 1e-2 and r["w_err"] <= 1e-4


def test_2bit_b8_distinct_tensor_scales_and_repeats_bitwise():
    from quantized_expert_gemv_amd.device_layer import bits_to_bf16_tensor
    layer, dev = dev_b8(tscales=True)
    x_bits = layer.x(4, batch=8)
    r = compare_layer(dev, layer, x_bits)
    _note(f"[2bit b8 ts] rel_err={r['rel_err']:.3e} mismatched={r['mismatched']}")
    assert not r["mismatched"] and r["rel_err"] <= 1e-2 and r["w_err"] <= 1e-4
    x = bits_to_bf16_tensor(x_bits, dev.device)
    first = dev(x).clone()
    for _ in range(3):
        again = dev(x)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16), first.view(torch.int16))
    assert dev.error() == 0


@pytest.mark.parametrize("step", [0, 1, 2, 3])
def test_2bit_layer_meets_the_oracle(step):
    layer, dev = dev_of()
    r = compare_layer(dev, layer, layer.x(step))
    _note(f"[2bit] step {step}: rel_err={r['rel_err']:.3e} w_err={r['w_err']:.2e} mismatched={r['mismatched']} "
          f"exempt={r['exempt']}")
    assert not r["mismatched"] and r["rel_err"] <= 1e-2 and r["w_err"] <= 1e-4


def test_2bit_layer_h_per_pair():
    layer, dev = dev_of()
    x = layer.x(5)
    r = compare_layer(dev, layer, x)
    hr, hs = dev.debug_h(1)
    torch.cuda.synchronize()
    hr = hr.float().cpu().numpy()
    ids = r["ids"][0].tolist()
    for j, e in enumerate(ids):
        want = r["ref"]["h"][(0, e)]
        err = np.max(np.abs(hr[0, j] - want))
        assert err <= 1e-2 * np.max(np.abs(want)), (j, e, err)
    want = r["ref"]["h"][(0, "shared", 0)]
    assert np.max(np.abs(hs[0, 0].float().cpu().numpy() - want)) <= 1e-2 * np.max(np.abs(want))


def test_2bit_layer_distinct_tensor_scales():
    layer, dev = dev_of(tscales=True)
    for step in (0, 1):
        r = compare_layer(dev, layer, layer.x(step))
        _note(f"[2bit ts] step {step}: rel_err={r['rel_err']:.3e} mismatched={r['mismatched']}")
        assert not r["mismatched"] and r["rel_err"] <= 1e-2 and r["w_err"] <= 1e-4


def test_2bit_layer_repeats_bitwise_and_static_entry_agrees():
    from quantized_expert_gemv_amd import binding as B
    from quantized_expert_gemv_amd.device_layer import bits_to_bf16_tensor
    layer, dev = dev_of()
    x = bits_to_bf16_tensor(layer.x(9), dev.device)
    first = dev(x).clone()
    b = dev.buffers()
    for _ in range(3):
        again = dev(x)
        out = torch.empty_like(x)
        B.moe_decode_layer_static(dev.desc, x, b["router_w"], b["expert_packed"], b["scales"], b["shared_w"],
                                  out, 1)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16), first.view(torch.int16))
        assert torch.equal(out.view(torch.int16), first.view(torch.int16))
    assert dev.error() == 0


def test_2bit_layer_refuses_what_it_cannot_run():
    from quantized_expert_gemv_amd import binding as B
    layer, dev = dev_of()
    with pytest.raises(B.MoeError) as e:
        B.moe_layer_set_path(dev.handle, B.MOE_PATH_GENERAL)
    assert e.value.status == -2
    from quantized_expert_gemv_amd.device_layer import bits_to_bf16_tensor
    x = bits_to_bf16_tensor(layer.x(0), dev.device)
    bufs = dev.buffers()
    with pytest.raises(B.MoeError) as e:
        B.moe_decode_chain([dev.handle], x, [bufs["router_w"]], [bufs["expert_packed"]], [bufs["scales"]],
                           [bufs["shared_w"]], torch.empty_like(x), 1)
    assert e.value.status == -2
    assert B.moe_prefill_workspace_bytes(dev.handle, 4) > 0   # the prefill path takes 2-bit layers
