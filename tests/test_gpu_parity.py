"""GPU parity: the HIP layer (through the C ABI) against the fp64 oracle.

Workloads are the seeded synthetic layers of quantized_expert_gemv_amd.synth
at their full sizes (the oracle evaluates only the selected experts, so it
finishes in seconds even at Flint size; for the expert-sink layer it is
evaluated on sampled tokens).  The bar: selected sets identical except
near-ties (oracle gap < 1e-5, reported and re-checked with the GPU's
selection forced), max|gpu - oracle| <= 1e-2 * max|oracle| per layer output.
"""

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from parity import compare_layer  # noqa: E402
from quantized_expert_gemv_amd.synth import WORKLOADS, ArrayLayer, SynthLayer, to_bf16_bits, to_e4m3_bytes  # noqa: E402


def _note(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_expert_gemv_amd import device_layer  # noqa: F401  (loads the library; raises if not built)
    yield
    _CACHE.clear()
    torch.cuda.synchronize()


_CACHE = {}


def dev_layer(name, max_batch=None, slot=0):
    from quantized_expert_gemv_amd.device_layer import DeviceLayer
    key = (name, max_batch, slot)
    if key not in _CACHE:
        _note(f"[upload] {name} slot={slot} max_batch={max_batch}")
        layer = SynthLayer(name, slot)
        _CACHE[key] = (layer, DeviceLayer(layer, max_batch or WORKLOADS[name].batch))
    return _CACHE[key]


def _report(tag, r):
    _note(f"[{tag}] rel_err={r['rel_err']:.3e} max_ref={r['max_ref']:.3e} w_err={r['w_err']:.2e} "
          f"exempt={r['exempt']} mismatched={r['mismatched']}")


@pytest.mark.parametrize("name,steps", [("tiny", 6), ("flint_b1", 4), ("flint_b8", 4),
                                        ("flint_bf16_b1", 2), ("flint_bf16_b8", 2)])
def test_layer_parity(name, steps):
    layer, dev = dev_layer(name)
    for step in range(steps):
        r = compare_layer(dev, layer, layer.x(step))
        _report(f"{name} step {step} D={len(set(r['ids'].ravel().tolist()))}", r)
        assert not r["mismatched"], r["mismatched"]
        assert r["rel_err"] <= 1e-2
        assert r["w_err"] <= 1e-4


@pytest.mark.parametrize("path", ["auto", "general"])
def test_ragged_batches_on_a_batch8_handle(path):
    """Every batch size on one handle, through the kernels dedicated to the
    Flint shape (batch 1: a wavefront per expert; batch 2-8: the small-batch
    kernel) and through the general kernel."""
    layer, dev = dev_layer("flint_b8")
    active = dev.set_path(path)
    try:
        if path == "general":
            assert active == "general"
        elif torch.cuda.get_device_properties(0).multi_processor_count >= 256:
            assert active == "dedicated"
        for n in (1, 2, 3, 5, 7, 8):
            r = compare_layer(dev, layer, layer.x(100 + n, batch=n))
            _report(f"flint_b8 {active} batch {n}", r)
            assert not r["mismatched"] and r["rel_err"] <= 1e-2 and r["w_err"] <= 1e-4
        assert dev.error() == 0
    finally:
        dev.set_path("auto")


# Shapes other than Flint's run the kernel variants that read the shape from
# the arguments; these two cover every batch bucket (1, 2, 4, 8) of them, with
# one wave step per row (H=1024) and four rows per step (H=512) in gate/up.
_GENERIC = {
    "generic_h1024": dict(hidden=1024, inter=256, n_routed=64, top_k=4, n_shared=2),
    "generic_h512": dict(hidden=512, inter=128, n_routed=32, top_k=3, n_shared=1),
}


@pytest.mark.parametrize("name", sorted(_GENERIC))
def test_generic_shape_every_batch_bucket(name):
    from quantized_expert_gemv_amd.device_layer import DeviceLayer
    from quantized_expert_gemv_amd.synth import Workload
    wl = Workload(6, name, batch=8, router_std=None, bias_std=0.5, description=name, **_GENERIC[name])
    layer = SynthLayer(wl)
    dev = DeviceLayer(layer, 8)
    for n in (1, 2, 3, 5, 8):
        r = compare_layer(dev, layer, layer.x(200 + n, batch=n))
        _report(f"{name} batch {n} D={len(set(r['ids'].ravel().tolist()))}", r)
        assert not r["mismatched"] and r["rel_err"] <= 1e-2 and r["w_err"] <= 1e-4


def test_sink_parity_every_token():
    layer, dev = dev_layer("sink_b4")
    r = compare_layer(dev, layer, layer.x(0), tokens=[0, 1, 2, 3])
    _report("sink_b4", r)
    assert not r["mismatched"] and r["rel_err"] <= 1e-2 and r["w_err"] <= 1e-5
    # the shared experts' coefficients are their softmax probabilities
    assert np.all(r["c"] > 0) and np.all(r["c"] < 1)
    # per-pair activations of token 0, including the BF16 shared experts
    hr, hs = dev.debug_h(4)
    hr, hs = hr.float().cpu().numpy(), hs.float().cpu().numpy()
    ref = r["ref"]
    for j, e in enumerate(r["ids"][0].tolist()):
        want = ref["h"][(0, e)]
        assert np.max(np.abs(hr[0, j] - want)) <= 1e-2 * np.max(np.abs(want))
    for s in range(2):
        want = ref["h"][(0, "shared", s)]
        assert np.max(np.abs(hs[0, s] - want)) <= 1e-2 * np.max(np.abs(want))


def test_sink_shared_path_with_routed_scales_zeroed():
    """The shared term is ~1e-3 of the routed term, so it is checked on its
    own: zero every routed block scale, leaving out = sum_s p_s y_s."""
    layer, dev = dev_layer("sink_b4")
    lay = dev.layout_r
    saved = dev.scales.clone()
    try:
        dev.scales[:lay["tensor_scale_offset"]].zero_()

        class Zeroed:
            def __getattr__(self, n):
                return getattr(layer, n)

            def routed_expert(self, e):
                ex = dict(layer.routed_expert(e))
                ex["scales13"] = np.zeros_like(ex["scales13"])
                ex["scales2"] = np.zeros_like(ex["scales2"])
                return ex
        r = compare_layer(dev, Zeroed(), layer.x(1), tokens=[1])
        _report("sink shared-only", r)
        assert not r["mismatched"] and r["rel_err"] <= 1e-2
        assert r["max_ref"] > 0
    finally:
        dev.scales.copy_(saved)
        torch.cuda.synchronize()


def test_two_layer_prenorm_chain():
    (l1, d1), (l2, d2) = dev_layer("flint_chain", slot=0), dev_layer("flint_chain", slot=1)
    import oracle
    from quantized_expert_gemv_amd.device_layer import bf16_tensor_to_bits
    x = l1.x(0)
    r1 = compare_layer(d1, l1, x)
    _report("chain layer 1", r1)
    assert not r1["mismatched"] and r1["rel_err"] <= 1e-2
    h1 = bf16_tensor_to_bits(r1["out"])
    r2 = compare_layer(d2, l2, h1)          # teacher forcing: oracle fed the GPU's layer-1 output
    _report("chain layer 2", r2)
    assert not r2["mismatched"] and r2["rel_err"] <= 1e-2
    # end to end (oracle rounds its layer-1 output to bf16 like the stored activations)
    ref1 = oracle.moe_layer(l1, x)["out"]
    ref2 = oracle.moe_layer(l2, to_bf16_bits(ref1))["out"]
    e2e = np.max(np.abs(r2["out_f"] - ref2)) / np.max(np.abs(ref2))
    _note(f"[chain end-to-end] rel_err={e2e:.3e}")
    assert e2e <= 2e-2


@pytest.mark.parametrize("path", ["auto", "general"])
def test_h_per_pair_flint(path):
    """SiLU*up activations of every selection and of the shared expert at
    batch 1, from both batch-1 kernels: the role-split one (one wavefront per
    expert; the automatic choice on a device with 256 compute units) and the
    general kernel (split-K gate/up on 256 workgroups).  Both write the same
    words, and each output must meet the oracle."""
    layer, dev = dev_layer("flint_b1")
    active = dev.set_path(path)
    try:
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        G, _ = dev.grid()
        _note(f"[h per pair] flint_b1 path={path} -> {active} kernel; general grid {G} workgroups, {cus} CUs")
        if path == "general":
            assert active == "general"
        elif cus >= 256:
            assert active == "dedicated"
        for step in (7, 11, 19):
            r = compare_layer(dev, layer, layer.x(step))
            _report(f"flint_b1 {active} step {step}", r)
            assert not r["mismatched"] and r["rel_err"] <= 1e-2 and r["w_err"] <= 1e-4
            hr, hs = dev.debug_h(1)
            hr, hs = hr.float().cpu().numpy(), hs.float().cpu().numpy()
            for j, e in enumerate(r["ids"][0].tolist()):
                want = r["ref"]["h"][(0, e)]
                assert np.max(np.abs(hr[0, j] - want)) <= 1e-2 * np.max(np.abs(want)), (step, j, e)
            want = r["ref"]["h"][(0, "shared", 0)]
            assert np.max(np.abs(hs[0, 0] - want)) <= 1e-2 * np.max(np.abs(want)), step
        assert dev.error() == 0
    finally:
        dev.set_path("auto")


def test_batch1_kernels_agree_and_alternate():
    """The two batch-1 kernels share the handle's call counter and words:
    alternating them call by call keeps every output equal, bit for bit, to
    the same kernel's output for that input, and within the parity bar of the
    other kernel's."""
    layer, dev = dev_layer("flint_b1")
    from quantized_expert_gemv_amd.device_layer import bits_to_bf16_tensor
    xs = [bits_to_bf16_tensor(layer.x(300 + i), dev.device) for i in range(3)]
    ref = {}
    try:
        for rep in range(2):
            for path in ("auto", "general"):
                dev.set_path(path)
                for i, x in enumerate(xs):
                    o = dev(x).clone()
                    if (path, i) in ref:
                        assert torch.equal(o.view(torch.int16), ref[(path, i)].view(torch.int16)), (rep, path, i)
                    ref[(path, i)] = o
        torch.cuda.synchronize()
        for i in range(len(xs)):
            a, b = ref[("auto", i)].float(), ref[("general", i)].float()
            assert (a - b).abs().max().item() <= 1e-2 * b.abs().max().item(), i
        assert dev.error() == 0
    finally:
        dev.set_path("auto")


def test_deterministic_bitwise():
    layer, dev = dev_layer("flint_b8")
    from quantized_expert_gemv_amd.device_layer import bits_to_bf16_tensor
    x = bits_to_bf16_tensor(layer.x(3), dev.device)
    a = dev(x).clone()
    b = dev(x).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_unselected_experts_are_not_read():
    """Poison every expert the routing did not pick (NaN scale bytes, 0xFF
    codes): the output must not change by a single bit."""
    layer, dev = dev_layer("flint_b1")
    from quantized_expert_gemv_amd.device_layer import bits_to_bf16_tensor
    x = bits_to_bf16_tensor(layer.x(11), dev.device)
    a = dev(x).clone()
    ids, _, _ = dev.routing(1)
    sel = set(ids.cpu().numpy().ravel().tolist())
    lay = dev.layout_r
    saved_c, saved_s = dev.expert_packed.clone(), dev.scales.clone()
    try:
        for e in range(layer.n_routed):
            if e in sel:
                continue
            dev.expert_packed[e * lay["code_stride"]:(e + 1) * lay["code_stride"]].fill_(0xFF)
            dev.scales[e * lay["scale_stride"]:(e + 1) * lay["scale_stride"]].fill_(0x7F)
        b = dev(x).clone()
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    finally:
        dev.expert_packed.copy_(saved_c)
        dev.scales.copy_(saved_s)
        torch.cuda.synchronize()


def test_doubling_down_tensor_scales_doubles_output_bitwise():
    layer, dev = dev_layer("flint_b1")
    from quantized_expert_gemv_amd.device_layer import bits_to_bf16_tensor
    x = bits_to_bf16_tensor(layer.x(12), dev.device)
    a = dev(x).clone().float()
    lay_r, lay_s = dev.layout_r, dev.layout_s
    saved_s, saved_sh = dev.scales.clone(), dev.shared_w.clone()
    try:
        ts = dev.scales[lay_r["tensor_scale_offset"]:].view(torch.float32).view(-1, 2)
        ts[:, 1] *= 2
        o = lay_s["shared_scale_offset"] + lay_s["tensor_scale_offset"]
        tss = dev.shared_w[o:o + 8 * layer.n_shared].view(torch.float32).view(-1, 2)
        tss[:, 1] *= 2
        b = dev(x).clone().float()
        torch.cuda.synchronize()
        assert torch.equal(b, 2 * a)
    finally:
        dev.scales.copy_(saved_s)
        dev.shared_w.copy_(saved_sh)
        torch.cuda.synchronize()


def test_token_in_batch8_matches_token_alone():
    layer, dev = dev_layer("flint_b8")
    from quantized_expert_gemv_amd.device_layer import bits_to_bf16_tensor
    xb = layer.x(5)
    full = dev(bits_to_bf16_tensor(xb, dev.device)).float()
    ids8, _, _ = dev.routing(8)
    ids8 = ids8.cpu().numpy()
    for b in (0, 4, 7):
        one = dev(bits_to_bf16_tensor(xb[b:b + 1], dev.device)).float()
        ids1, _, _ = dev.routing(1)
        assert ids1.cpu().numpy()[0].tolist() == ids8[b].tolist()   # router logits are batch-independent
        err = (one[0] - full[b]).abs().max().item()
        assert err <= 1e-2 * full[b].abs().max().item()


# ---------------------------------------------------------------------------
# crafted layers
# ---------------------------------------------------------------------------

def _tiny_arrays(rng, E=16, H=256, I=128, scale_fn=None):
    def ex():
        d = {"codes13": rng.integers(0, 256, (2 * I, H // 2), dtype=np.uint8),
             "codes2": rng.integers(0, 256, (H, I // 2), dtype=np.uint8),
             "g13": np.float32(1.0), "g2": np.float32(1.0)}
        if scale_fn is None:
            d["scales13"] = to_e4m3_bytes(np.abs(rng.standard_normal((2 * I, H // 16))) * 0.05)
            d["scales2"] = to_e4m3_bytes(np.abs(rng.standard_normal((H, I // 16))) * 0.05)
        else:
            d["scales13"], d["scales2"] = scale_fn((2 * I, H // 16)), scale_fn((H, I // 16))
        return d
    return [ex() for _ in range(E)]


def test_every_finite_e4m3_scale_byte():
    from quantized_expert_gemv_amd.device_layer import DeviceLayer
    rng = np.random.default_rng(77)
    finite = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], dtype=np.uint8)
    counter = [0]

    def cyc(shape):
        n = int(np.prod(shape))
        out = finite[(np.arange(n) + counter[0]) % finite.size].reshape(shape)
        counter[0] += 37
        return out
    H, I = 256, 128
    layer = ArrayLayer(hidden=H, inter=I, top_k=2, router_w=to_bf16_bits(rng.normal(0, 0.05, (16, H))),
                       routed=_tiny_arrays(rng, scale_fn=cyc), shared=_tiny_arrays(rng, E=1, scale_fn=cyc))
    dev = DeviceLayer(layer, 2)
    for step in range(3):
        x = to_bf16_bits(rng.standard_normal((2, H)))
        r = compare_layer(dev, layer, x)
        _report(f"all-scale-bytes step {step}", r)
        assert not r["mismatched"] and r["rel_err"] <= 1e-2
    dev.close()


def test_exact_ties_and_k_equals_E():
    from quantized_expert_gemv_amd.device_layer import DeviceLayer
    rng = np.random.default_rng(78)
    H, I = 256, 128
    # zero router: every logit is 0 -> ties broken to the lowest indices
    layer = ArrayLayer(hidden=H, inter=I, top_k=3, router_w=np.zeros((8, H), np.uint16),
                       routed=_tiny_arrays(rng, E=8), shared=_tiny_arrays(rng, E=1))
    dev = DeviceLayer(layer, 4)
    r = compare_layer(dev, layer, to_bf16_bits(rng.standard_normal((4, H))))
    assert r["ids"].tolist() == [[0, 1, 2]] * 4
    assert np.allclose(r["w"], 1 / 3, atol=1e-7)
    assert r["rel_err"] <= 1e-2
    dev.close()
    # k == E: every expert selected for every token
    layer = ArrayLayer(hidden=H, inter=I, top_k=4, router_w=to_bf16_bits(rng.normal(0, 0.1, (4, H))),
                       routed=_tiny_arrays(rng, E=4), shared=[])
    dev = DeviceLayer(layer, 3)
    r = compare_layer(dev, layer, to_bf16_bits(rng.standard_normal((3, H))))
    assert all(sorted(row) == [0, 1, 2, 3] for row in r["ids"].tolist())
    assert np.allclose(r["w"].sum(axis=1), 1.0, atol=1e-6)
    assert not r["mismatched"] and r["rel_err"] <= 1e-2
    dev.close()


def test_error_paths_on_device():
    from quantized_expert_gemv_amd import binding as B
    layer, dev = dev_layer("tiny")
    x = torch.zeros((2, layer.hidden), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(x)
    bufs = dev.buffers()
    call = lambda xx, oo, n: B.lib.moe_decode_layer(  # noqa: E731
        dev.handle, xx.data_ptr(), bufs["router_w"].data_ptr(), bufs["expert_packed"].data_ptr(),
        bufs["scales"].data_ptr(), bufs["shared_w"].data_ptr(), oo.data_ptr(), n,
        torch.cuda.current_stream().cuda_stream)
    assert call(x, out, 0) == -4
    assert call(x, out, 2) == -4                   # this handle's max_batch is 1
    assert call(x, x, 1) == -1                     # out aliases x
    xm = torch.zeros(2 * layer.hidden + 8, dtype=torch.bfloat16, device="cuda")[1:1 + layer.hidden]
    assert B.lib.moe_decode_layer(dev.handle, xm.data_ptr(), bufs["router_w"].data_ptr(),
                                  bufs["expert_packed"].data_ptr(), bufs["scales"].data_ptr(),
                                  bufs["shared_w"].data_ptr(), out.data_ptr(), 1, None) == -3
    fresh = B.moe_layer_create(dev.desc)
    try:
        assert B.lib.moe_layer_routing(fresh, None, None, None, None) == -7
    finally:
        B.moe_layer_destroy(fresh)


def test_grid_plan_one_workgroup_per_cu():
    from quantized_expert_gemv_amd import binding as B
    layer, dev = dev_layer("flint_b1")
    G, lds = dev.grid()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    _note(f"[grid] flint_b1: {G} workgroups, {lds} B shared memory; device has {cus} CUs")
    assert G == min(cus, layer.n_routed)
    assert B.moe_layer_error(dev.handle) == 0


def test_graph_replays_match_eager_calls():
    """The call counter that tags cross-workgroup words lives on the device, so
    replaying a captured sequence of calls must give the eager results every time."""
    layer, dev = dev_layer("flint_b8")
    from quantized_expert_gemv_amd.device_layer import bits_to_bf16_tensor
    xs = [bits_to_bf16_tensor(layer.x(40 + i, batch=n), dev.device) for i, n in enumerate((8, 3, 1))]
    eager = [dev(x).clone() for x in xs]
    torch.cuda.synchronize()
    outs = [torch.empty_like(e) for e in eager]
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for x, o in zip(xs, outs):
                dev(x, out=o)
    torch.cuda.current_stream().wait_stream(cap)
    for rep in range(3):
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for e, o in zip(eager, outs):
            assert torch.equal(e.view(torch.int16), o.view(torch.int16)), rep
        # eager work between replays
        again = dev(xs[1])
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16), eager[1].view(torch.int16))
    assert dev.error() == 0


def test_many_calls_alternating_batches():
    layer, dev = dev_layer("flint_b8")
    from quantized_expert_gemv_amd.device_layer import bits_to_bf16_tensor
    ref = {}
    for rep in range(3):
        for n in (8, 1, 5):
            x = bits_to_bf16_tensor(layer.x(60 + n, batch=n), dev.device)
            o = dev(x).clone()
            if n in ref:
                assert torch.equal(o.view(torch.int16), ref[n].view(torch.int16)), (rep, n)
            ref[n] = o
    torch.cuda.synchronize()
    assert dev.error() == 0


# ---------------------------------------------------------------------------
# per-expert tensor scales (NVFP4's third factor), other shapes, invariants
# ---------------------------------------------------------------------------

TS_SET = (0.37, 0.7, 1.3, 2.0)   # distinct, mostly not powers of two


def _put_tensor_scales(dev, lt):
    """Write lt's per-expert fp32 tensor scales into dev's packed buffers in
    place (the code and block-scale bytes are those of the same seeded layer);
    returns the saved buffers."""
    saved = (dev.scales.clone() if dev.scales is not None else None,
             dev.shared_w.clone() if dev.shared_w is not None else None)
    if lt.routed_wtype == "nvfp4":
        o = dev.layout_r["tensor_scale_offset"]
        ts = torch.tensor([lt.routed_tensor_scales(e) for e in range(lt.n_routed)], dtype=torch.float32)
        dev.scales[o:o + ts.numel() * 4].view(torch.float32).copy_(ts.view(-1).to(dev.device))
    if lt.n_shared and lt.shared_wtype == "nvfp4":
        o = dev.layout_s["shared_scale_offset"] + dev.layout_s["tensor_scale_offset"]
        ts = torch.tensor([lt.shared_tensor_scales(q) for q in range(lt.n_shared)], dtype=torch.float32)
        dev.shared_w[o:o + ts.numel() * 4].view(torch.float32).copy_(ts.view(-1).to(dev.device))
    torch.cuda.synchronize()
    return saved


def _restore(dev, saved):
    if saved[0] is not None:
        dev.scales.copy_(saved[0])
    if saved[1] is not None:
        dev.shared_w.copy_(saved[1])
    torch.cuda.synchronize()


def _check_h_token(dev, r, batch, b=0):
    hr, hs = dev.debug_h(batch)
    hr, hs = hr.float().cpu().numpy(), hs.float().cpu().numpy()
    i = r["rows"].index(b)
    for j, e in enumerate(r["ids"][b].tolist()):
        want = r["ref"]["h"][(i, e)]
        assert np.max(np.abs(hr[b, j] - want)) <= 1e-2 * np.max(np.abs(want)), (b, j, e)
    for q in range(hs.shape[1]):
        want = r["ref"]["h"][(i, "shared", q)]
        assert np.max(np.abs(hs[b, q] - want)) <= 1e-2 * np.max(np.abs(want)), (b, q)


@pytest.mark.parametrize("name,tokens,steps", [("flint_b1", None, (0, 1, 2)), ("flint_b8", None, (0, 1)),
                                               ("sink_b4", [1, 2], (2,))])
def test_parity_with_distinct_tensor_scales(name, tokens, steps):
    """Every routed and shared NVFP4 expert carries its own W13 and W2 tensor
    scales drawn from {0.37, 0.7, 1.3, 2.0}: a scale read for the wrong expert,
    slot or matrix moves the output or h far beyond the tolerance."""
    layer, dev = dev_layer(name)
    lt = SynthLayer(name, tscale_set=TS_SET)
    saved = _put_tensor_scales(dev, lt)
    try:
        for step in steps:
            x = lt.x(step)
            r = compare_layer(dev, lt, x, tokens=tokens)
            _report(f"{name} tensor scales step {step}", r)
            assert not r["mismatched"] and r["rel_err"] <= 1e-2 and r["w_err"] <= 1e-4
            _check_h_token(dev, r, x.shape[0], b=r["rows"][0])
    finally:
        _restore(dev, saved)


def test_more_than_256_routed_experts_with_distinct_tensor_scales():
    """E = 384: the routed tensor-scale table covers experts beyond the first 256."""
    from quantized_expert_gemv_amd.device_layer import DeviceLayer
    from quantized_expert_gemv_amd.synth import Workload
    wl = Workload(8, "e384", 256, 128, 384, 4, 1, 8, router_std=None, bias_std=0.5, description="E=384")
    layer = SynthLayer(wl, tscale_set=TS_SET)
    dev = DeviceLayer(layer, 8)
    try:
        seen = set()
        for n, step in ((1, 0), (3, 1), (8, 2), (8, 3)):
            r = compare_layer(dev, layer, layer.x(step, batch=n))
            seen |= set(r["ids"].ravel().tolist())
            _report(f"E=384 batch {n}", r)
            assert not r["mismatched"] and r["rel_err"] <= 1e-2 and r["w_err"] <= 1e-4
        assert max(seen) >= 256, sorted(seen)       # experts past 256 were exercised
    finally:
        dev.close()


def test_flint_shape_nvfp4_routed_bf16_shared():
    """The precision split of the Inkling page (NVFP4 routed, BF16 shared
    experts) at the Flint shape: validate accepts it, create runs it."""
    from quantized_expert_gemv_amd import binding as B
    from quantized_expert_gemv_amd.device_layer import DeviceLayer
    from quantized_expert_gemv_amd.synth import Workload
    wl = Workload(9, "flint_mixed", 2048, 512, 256, 6, 1, 2, shared_wtype="bf16", description="mixed")
    layer = SynthLayer(wl)
    dev = DeviceLayer(layer, 2)
    try:
        assert B.moe_layer_validate(dev.desc) == 0
        for n in (1, 2):
            r = compare_layer(dev, layer, layer.x(n, batch=n))
            _report(f"flint mixed batch {n}", r)
            assert not r["mismatched"] and r["rel_err"] <= 1e-2
    finally:
        dev.close()


class _Permuted:
    """The same layer with routed expert ids relabelled: new expert e is old
    expert perm[e] (router row and bias move with it)."""

    def __init__(self, base, perm):
        self._b, self.perm = base, np.asarray(perm)
        self.router_w = base.router_w[self.perm]
        self.router_bias = None if base.router_bias is None else base.router_bias[self.perm]

    def __getattr__(self, n):
        return getattr(self._b, n)

    def routed_expert(self, e):
        return self._b.routed_expert(int(self.perm[e]))


@pytest.mark.parametrize("name", ["flint_b1", "flint_b8"])
def test_expert_permutation_permutes_ids_only(name):
    from quantized_expert_gemv_amd.device_layer import DeviceLayer, bits_to_bf16_tensor
    layer, dev = dev_layer(name)
    perm = np.random.default_rng(31).permutation(layer.n_routed)
    lp = _Permuted(layer, perm)
    dp = DeviceLayer(lp, dev.max_batch)
    try:
        for step in (0, 1):
            x = bits_to_bf16_tensor(layer.x(step), dev.device)
            a, b = dev(x).clone(), dp(x).clone()
            ia, _, _ = dev.routing(x.shape[0])
            ib, _, _ = dp.routing(x.shape[0])
            torch.cuda.synchronize()
            assert (perm[ib.cpu().numpy()] == ia.cpu().numpy()).all()
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    finally:
        dp.close()
