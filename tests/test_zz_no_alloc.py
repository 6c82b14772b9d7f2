"""The handle-less, allocation-free layer call (moe_decode_layer_static)
against the handle call (moe_decode_layer) on the same inputs: the same
kernels, so the outputs must be bitwise equal; also checked against the
oracle, and under HIP graph capture."""

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _note(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def flint8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_expert_gemv_amd.device_layer import DeviceLayer
    from quantized_expert_gemv_amd.synth import SynthLayer
    layer = SynthLayer("flint_b8")
    dev = DeviceLayer(layer, 8)
    yield layer, dev
    dev.close()
    torch.cuda.synchronize()


def _static(dev, x, out, err, stream=None):
    from quantized_expert_gemv_amd import binding as B
    b = dev.buffers()
    B.moe_decode_layer_static(dev.desc, x, b["router_w"], b["expert_packed"], b["scales"], b["shared_w"], out,
                              x.shape[0], err, stream)


def test_static_call_equals_handle_call_twice_second_smaller(flint8):
    from parity import compare_layer  # noqa: F401  (oracle comparison below)
    import oracle
    from quantized_expert_gemv_amd.device_layer import bf16_tensor_to_bits, bits_to_bf16_tensor
    layer, dev = flint8
    err = torch.zeros(1, dtype=torch.int32, device=dev.device)
    for n, step in ((8, 0), (3, 1)):
        _note(f"[no-alloc] flint_b8 batch {n} step {step}")
        xb = layer.x(step, batch=n)
        x = bits_to_bf16_tensor(xb, dev.device)
        ref = dev(x).clone()
        out = torch.full_like(ref, float("nan"))
        _static(dev, x, out, err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), n
        got = oracle.bf16_bits_to_f64(bf16_tensor_to_bits(out))
        want = oracle.moe_layer(layer, xb)["out"]
        rel = np.max(np.abs(got - want)) / np.max(np.abs(want))
        _note(f"[no-alloc] batch {n}: bitwise equal to the handle call; rel_err vs oracle {rel:.3e}")
        assert rel <= 1e-2


def test_static_call_in_a_replayed_graph(flint8):
    from quantized_expert_gemv_amd.device_layer import bits_to_bf16_tensor
    layer, dev = flint8
    xs = [bits_to_bf16_tensor(layer.x(20 + i, batch=n), dev.device) for i, n in enumerate((8, 2))]
    err = torch.zeros(1, dtype=torch.int32, device=dev.device)
    eager = []
    for x in xs:
        o = torch.empty((x.shape[0], layer.hidden), dtype=torch.bfloat16, device=dev.device)
        _static(dev, x, o, err)
        eager.append(o)
    torch.cuda.synchronize()
    outs = [torch.empty_like(e) for e in eager]
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for x, o in zip(xs, outs):
                _static(dev, x, o, err, stream=cap)
    torch.cuda.current_stream().wait_stream(cap)
    for rep in range(3):
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for e, o in zip(eager, outs):
            assert torch.equal(e.view(torch.int16), o.view(torch.int16)), rep
        mid = dev(xs[1])                 # eager handle work between replays
        torch.cuda.synchronize()
        assert torch.equal(mid.view(torch.int16), eager[1].view(torch.int16))
    assert int(err.item()) == 0
