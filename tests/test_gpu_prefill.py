"""GPU parity of the prefill path (moe_prefill_layer, through the C ABI)
against the fp64 oracle.

The prefill path computes the same layer as the decode kernels for T tokens
at once (grouped GEMMs on the matrix cores), so the oracle is the same layer
definition, evaluated token by token.  Acceptance is the decode path's:
  * each token's selected set equals the oracle's, except tokens whose
    oracle k-th/(k+1)-th score gap is below 1e-5 (then the oracle is re-run
    with the GPU's selection forced);
  * routing weights within 1e-4 of the oracle's;
  * max |gpu - oracle| <= 1e-2 * max |oracle| over the compared rows.
Cases: the tiny shape (every token compared, ragged T; T = 1500 with
128-row tiles), the Flint shape at T = 64 (every token), T = 1000 and
T = 8192 (sampled tokens, several tiles per expert; 128-row tiles at 8192),
pre-norm + residual, distinct per-expert tensor scales, routed experts in
the 2-bit planes (T = 64 and T = 8192 sampled, and with distinct tensor
scales), T = 1, and run-to-run / graph-replay bit equality.
"""

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

GAP_EPS = 1e-5
TS_SET = (0.37, 0.7, 1.3, 2.0)


def _note(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_expert_gemv_amd import device_layer  # noqa: F401  (raises if the library is not built)
    yield
    _DEVS.clear()
    torch.cuda.synchronize()


_DEVS = {}


def dev_of(name, tscales=False):
    from quantized_expert_gemv_amd.device_layer import DeviceLayer
    from quantized_expert_gemv_amd.synth import SynthLayer
    key = (name, tscales)
    if key not in _DEVS:
        _note(f"[upload] {name} tensor_scales={'distinct' if tscales else 'unit'}")
        layer = SynthLayer(name, tscale_set=TS_SET if tscales else None)
        _DEVS[key] = (layer, DeviceLayer(layer, 1))
    return _DEVS[key]


def check_prefill(name, T, step, sample=None, tscales=False):
    import oracle
    from quantized_expert_gemv_amd.device_layer import bf16_tensor_to_bits, bits_to_bf16_tensor
    layer, dev = dev_of(name, tscales)
    x_bits = layer.x(step, batch=T)
    _note(f"[prefill] {name} T={T} step={step} tensor_scales={tscales}")
    x = bits_to_bf16_tensor(x_bits, dev.device)
    out, ids, w = dev.prefill(x, routing=True)
    torch.cuda.synchronize()
    got = oracle.bf16_bits_to_f64(bf16_tensor_to_bits(out))
    ids, w = ids.cpu().numpy(), w.cpu().numpy()
    rows = list(range(T)) if sample is None else sorted(set(sample))
    ref = oracle.moe_layer(layer, x_bits[rows])
    exempt, mismatched, w_err = [], [], 0.0
    for i, t in enumerate(rows):
        if set(ids[t].tolist()) != set(ref["ids"][i].tolist()):
            (exempt if ref["gaps"][i] < GAP_EPS else mismatched).append(t)
            continue
        ref_w = dict(zip(ref["ids"][i].tolist(), ref["w"][i].tolist()))
        w_err = max(w_err, max(abs(float(wv) - ref_w[e]) for e, wv in zip(ids[t].tolist(), w[t].tolist())))
    ref_out = ref["out"]
    if exempt:
        ref_out = oracle.moe_layer(layer, x_bits[rows], force_ids=ids[rows])["out"]
    err = float(np.max(np.abs(got[rows] - ref_out)))
    scale = float(np.max(np.abs(ref_out)))
    _note(f"[prefill] {name} T={T}: rel_err={err / scale:.3e} w_err={w_err:.2e} exempt={exempt} "
          f"mismatched={mismatched}")
    assert np.all(np.isfinite(got))
    assert not mismatched
    assert w_err <= 1e-4
    assert err <= 1e-2 * scale
    return out, ids


@pytest.mark.parametrize("T", [1, 5, 33, 100])
def test_prefill_tiny_every_token(T):
    check_prefill("tiny", T, step=T)


def test_prefill_flint_every_token():
    check_prefill("flint_b1", 64, step=3)


def test_prefill_flint_many_tokens_sampled():
    """T = 1000: ~23 rows per expert on average, each routed group in one
    64-row tile; the shared expert spans 16 tiles."""
    rng = np.random.default_rng(5)
    sample = [0, 1, 999] + rng.choice(1000, size=21, replace=False).tolist()
    check_prefill("flint_b1", 1000, step=4, sample=sample)


def test_prefill_tiny_long_tiles_every_token():
    """T = 1500 on the tiny shape (E = 16, top-2): the routed groups average
    more than 128 rows, so the call runs 128-row tiles: full ones, partial
    ones of 65..127 rows (8 row blocks) and remainders of <= 64 rows (4 row
    blocks); the shared expert spans 12 tiles."""
    out, ids = check_prefill("tiny", 1500, step=11)
    counts = np.bincount(ids.ravel(), minlength=16)
    assert counts.min() > 128 and np.any(counts % 128 > 64) and np.any((counts % 128 > 0) & (counts % 128 <= 64))


def test_prefill_flint_long_tiles_sampled():
    """T = 8192 at the Flint shape (the benchmarked size): ~192 rows per
    routed expert, 128-row tiles; sampled tokens."""
    rng = np.random.default_rng(9)
    sample = [0, 8191] + rng.choice(8192, size=14, replace=False).tolist()
    check_prefill("flint_b1", 8192, step=12, sample=sample)


def test_prefill_2bit_every_token():
    """Routed experts in the 2-bit planes (widened to e2m1 as they are
    staged; the shared expert stays NVFP4), 64-row tiles."""
    check_prefill("flint_2bit_b1", 64, step=13)


def test_prefill_2bit_long_tiles_sampled_and_tensor_scales():
    rng = np.random.default_rng(14)
    sample = [0, 8191] + rng.choice(8192, size=10, replace=False).tolist()
    check_prefill("flint_2bit_b1", 8192, step=14, sample=sample)
    check_prefill("flint_2bit_b1", 100, step=15, tscales=True)


def test_prefill_prenorm_residual():
    check_prefill("flint_chain", 40, step=6)


def test_prefill_distinct_tensor_scales():
    check_prefill("flint_b1", 48, step=7, tscales=True)


def test_prefill_is_deterministic_and_graph_safe():
    from quantized_expert_gemv_amd import binding as B
    from quantized_expert_gemv_amd.device_layer import bits_to_bf16_tensor
    layer, dev = dev_of("tiny")
    T = 77
    x = bits_to_bf16_tensor(layer.x(9, batch=T), dev.device)
    ws = torch.empty(B.moe_prefill_workspace_bytes(dev.handle, T), dtype=torch.uint8, device=dev.device)
    first = dev.prefill(x, workspace=ws).clone()
    again = dev.prefill(x, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), again.view(torch.int16))
    out = torch.empty_like(first)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            dev.prefill(x, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(cap)
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), first.view(torch.int16)), rep
        dev.prefill(x, workspace=ws)   # eager work between the replays
        torch.cuda.synchronize()


def test_prefill_argument_errors():
    from quantized_expert_gemv_amd import binding as B
    from quantized_expert_gemv_amd.device_layer import bits_to_bf16_tensor
    layer, dev = dev_of("tiny")
    T = 8
    x = bits_to_bf16_tensor(layer.x(0, batch=T), dev.device)
    out = torch.empty_like(x)
    need = B.moe_prefill_workspace_bytes(dev.handle, T)
    ws = torch.empty(need, dtype=torch.uint8, device=dev.device)
    b = dev.buffers()
    args = (b["router_w"], b["expert_packed"], b["scales"], b["shared_w"])
    with pytest.raises(B.MoeError) as e:
        B.moe_prefill_layer(dev.handle, x, *args, out, T, ws, need - 1)
    assert e.value.status == -1
    with pytest.raises(B.MoeError) as e:
        B.moe_prefill_layer(dev.handle, x, *args, x, T, ws, need)     # out == x
    assert e.value.status == -1
    with pytest.raises(B.MoeError) as e:
        B.moe_prefill_layer(dev.handle, x, *args, out, 0, ws, need)
    assert e.value.status == -4
    with pytest.raises(B.MoeError) as e:
        B.moe_prefill_workspace_bytes(dev.handle, B.MOE_PREFILL_MAX_TOKENS + 1)
    assert e.value.status == -4
    # a shape the path does not take: the expert-sink routing
    desc = B.make_desc(hidden=256, inter=128, n_routed=16, top_k=2, n_shared=1, max_batch=1, route="sink",
                       shared_wtype="bf16")
    h = B.moe_layer_create(desc)
    try:
        with pytest.raises(B.MoeError) as e:
            B.moe_prefill_workspace_bytes(h, 4)
        assert e.value.status == -2
    finally:
        B.moe_layer_destroy(h)
    torch.cuda.synchronize()
