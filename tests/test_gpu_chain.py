"""GPU tests of the layer chain: one launch for several pre-norm residual MoE
layers (moe_decode_chain), through the C ABI.

Each layer of the chain computes what a single call of the same layer
computes, on the same bf16 input, so the chain's output must equal, bit for
bit, the output of the layers called one after another; each of those calls
is checked against the fp64 oracle with its GPU input (teacher forcing), and
the last output end to end.  The layers are the seeded Flint-shaped chain
workload (H=2048, I=512, 256 experts, top-6 + 1 shared, NVFP4, pre-norm and
residual), one weight set per layer.
"""

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from parity import compare_layer  # noqa: E402


def _note(msg):
    print(msg, file=sys.stderr, flush=True)


_LAYERS = []


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_expert_gemv_amd import device_layer  # noqa: F401  (raises if the library is not built)
    yield
    _LAYERS.clear()
    torch.cuda.synchronize()


def layers(n):
    from quantized_expert_gemv_amd.device_layer import DeviceLayer
    from quantized_expert_gemv_amd.synth import SynthLayer
    while len(_LAYERS) < n:
        slot = len(_LAYERS)
        _note(f"[upload] flint_chain slot={slot}")
        layer = SynthLayer("flint_chain", slot)
        _LAYERS.append((layer, DeviceLayer(layer, 1)))
    return _LAYERS[:n]


def _chain(devs, x, out=None):
    from quantized_expert_gemv_amd import binding as B
    if out is None:
        out = torch.empty_like(x)
    bufs = [d.buffers() for d in devs]
    B.moe_decode_chain([d.handle for d in devs], x, [b["router_w"] for b in bufs], [b["expert_packed"] for b in bufs],
                       [b["scales"] for b in bufs], [b["shared_w"] for b in bufs], out, 1)
    return out


def _one_by_one(devs, x):
    y = x
    for d in devs:
        y = d(y).clone()
    return y


@pytest.mark.parametrize("n", [1, 2, 5])
def test_chain_equals_layers_one_by_one(n):
    from quantized_expert_gemv_amd.device_layer import bits_to_bf16_tensor
    ls = layers(n)
    devs = [d for _, d in ls]
    if devs[0].set_path("auto") != "dedicated":
        pytest.skip("the chain runs on the batch-1 kernel dedicated to the Flint shape (256 CUs)")
    x = bits_to_bf16_tensor(ls[0][0].x(3), devs[0].device)
    got = _chain(devs, x).clone()
    ids_chain = [d.routing(1)[0].clone() for d in devs]
    want = _one_by_one(devs, x)
    ids_single = [d.routing(1)[0].clone() for d in devs]
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    for a, b in zip(ids_chain, ids_single):
        assert torch.equal(a, b)
    for _, d in ls:
        assert d.error() == 0


def test_chain_layers_meet_the_oracle():
    """Each layer of a 4-layer chain against the oracle (teacher forcing: the
    oracle gets the GPU's bf16 input of that layer), and end to end.

    End to end, the oracle runs the four layers on its own outputs with the
    chain's expert selection forced at every layer: a layer's rounding moves
    the next layer's router scores by about 1e-3, more than the gap between
    the 6th and 7th score of some tokens, so an unforced oracle chain may pick
    another expert there and the two chains then differ by that expert's
    whole contribution.  Such flips are reported with the oracle's gap, not
    failed.  With the selection shared, each layer adds at most its own
    bound (1e-2 of its output's max), so 4 layers stay within 4e-2."""
    import oracle
    from quantized_expert_gemv_amd.device_layer import bf16_tensor_to_bits, bits_to_bf16_tensor
    from quantized_expert_gemv_amd.synth import to_bf16_bits
    ls = layers(4)
    devs = [d for _, d in ls]
    if devs[0].set_path("auto") != "dedicated":
        pytest.skip("the chain runs on the batch-1 kernel dedicated to the Flint shape (256 CUs)")
    x_bits = ls[0][0].x(7)
    x = bits_to_bf16_tensor(x_bits, devs[0].device)
    got = _chain(devs, x).clone()
    chain_ids = [d.routing(1)[0].cpu().numpy().copy() for d in devs]
    torch.cuda.synchronize()
    h = x_bits
    for i, (layer, d) in enumerate(ls):
        r = compare_layer(d, layer, h)
        _note(f"[chain layer {i}] rel_err={r['rel_err']:.3e} mismatched={r['mismatched']}")
        assert not r["mismatched"] and r["rel_err"] <= 1e-2
        assert np.array_equal(np.sort(r["ids"][0]), np.sort(chain_ids[i][0]))
        h = bf16_tensor_to_bits(r["out"])
    assert np.array_equal(bf16_tensor_to_bits(got), h)   # the chain's output is the last layer's
    ref = x_bits
    for i, (layer, _) in enumerate(ls):
        free = oracle.moe_layer(layer, ref)
        if set(free["ids"][0].tolist()) != set(chain_ids[i][0].tolist()):
            _note(f"[chain layer {i}] oracle chain selects {sorted(free['ids'][0].tolist())}, GPU chain "
                  f"{sorted(chain_ids[i][0].tolist())}; oracle 6th/7th gap {free['gaps'][0]:.2e}")
        ref = to_bf16_bits(oracle.moe_layer(layer, ref, force_ids=chain_ids[i])["out"])
    ref_f = oracle.bf16_bits_to_f64(ref)
    e2e = np.max(np.abs(oracle.bf16_bits_to_f64(h) - ref_f)) / np.max(np.abs(ref_f))
    _note(f"[chain end-to-end, 4 layers, selection shared] rel_err={e2e:.3e}")
    assert e2e <= 4e-2


def test_longest_chain_repeated_and_interleaved():
    """MOE_MAX_CHAIN layers (the weight sets cycle), called repeatedly, with
    single calls on the first handle in between: every repetition gives the
    same bits, and the single calls are unaffected."""
    from quantized_expert_gemv_amd import binding as B
    from quantized_expert_gemv_amd.device_layer import bits_to_bf16_tensor
    ls = layers(4)
    devs = [d for _, d in ls]
    if devs[0].set_path("auto") != "dedicated":
        pytest.skip("the chain runs on the batch-1 kernel dedicated to the Flint shape (256 CUs)")
    chain = [devs[i % 4] for i in range(B.MOE_MAX_CHAIN)]
    x = bits_to_bf16_tensor(ls[0][0].x(11), devs[0].device)
    first = _chain(chain, x).clone()
    single = devs[0](x).clone()
    for _ in range(3):
        again = _chain(chain, x)
        s2 = devs[0](x)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16), first.view(torch.int16))
        assert torch.equal(s2.view(torch.int16), single.view(torch.int16))
    assert torch.equal(first.view(torch.int16), _one_by_one(chain, x).view(torch.int16))
    for d in devs:
        assert d.error() == 0


def test_chain_in_a_replayed_graph():
    from quantized_expert_gemv_amd.device_layer import bits_to_bf16_tensor
    ls = layers(3)
    devs = [d for _, d in ls]
    if devs[0].set_path("auto") != "dedicated":
        pytest.skip("the chain runs on the batch-1 kernel dedicated to the Flint shape (256 CUs)")
    xs = [bits_to_bf16_tensor(ls[0][0].x(20 + i), devs[0].device) for i in range(2)]
    eager = [_chain(devs, x).clone() for x in xs]
    outs = [torch.empty_like(e) for e in eager]
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for x, o in zip(xs, outs):
                _chain(devs, x, out=o)
    torch.cuda.current_stream().wait_stream(cap)
    for rep in range(3):
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for e, o in zip(eager, outs):
            assert torch.equal(e.view(torch.int16), o.view(torch.int16)), rep
        _chain(devs, xs[0])   # eager work between replays
        torch.cuda.synchronize()
    for d in devs:
        assert d.error() == 0


def test_chain_argument_errors():
    from quantized_expert_gemv_amd import binding as B
    from quantized_expert_gemv_amd.device_layer import bits_to_bf16_tensor
    ls = layers(2)
    devs = [d for _, d in ls]
    x = bits_to_bf16_tensor(ls[0][0].x(1), devs[0].device)
    out = torch.empty_like(x)
    bufs = [d.buffers() for d in devs]
    args = lambda n: ([bufs[i % 2]["router_w"] for i in range(n)],   # noqa: E731
                      [bufs[i % 2]["expert_packed"] for i in range(n)],
                      [bufs[i % 2]["scales"] for i in range(n)], [bufs[i % 2]["shared_w"] for i in range(n)])
    with pytest.raises(B.MoeError) as e:
        B.moe_decode_chain([], x, [], [], [], [], out, 1)
    assert e.value.status == -1
    with pytest.raises(B.MoeError) as e:
        B.moe_decode_chain([devs[i % 2].handle for i in range(17)], x, *args(17), out, 1)
    assert e.value.status == -1
    with pytest.raises(B.MoeError) as e:
        B.moe_decode_chain([d.handle for d in devs], x, *args(2), x, 1)     # out == x
    assert e.value.status == -1
    with pytest.raises(B.MoeError) as e:
        B.moe_decode_chain([d.handle for d in devs], x, *args(2), out, 2)   # batch above the handles' max
    assert e.value.status in (-2, -4)
    devs[0].set_path("general")
    try:
        with pytest.raises(B.MoeError) as e:
            B.moe_decode_chain([d.handle for d in devs], x, *args(2), out, 1)
        assert e.value.status == -2
    finally:
        devs[0].set_path("auto")
