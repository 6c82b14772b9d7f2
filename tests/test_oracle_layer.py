"""Pins for the oracle's layer evaluation (CPU only).

Closed forms, special cases, invariants and a brute-force scalar evaluation
of tiny layers.  Chosen so that a dropped term, a swapped gate/up half, a
transposed matrix, a wrong combine weight or a missing residual fails one
of them.
"""

import math

import numpy as np
import pytest

from oracle import formats as F
from oracle import layer as L
from quantized_expert_gemv_amd.synth import ArrayLayer, SynthLayer, to_bf16_bits, to_e4m3_bytes

E2M1 = {0: 0.0, 1: 0.5, 2: 1.0, 3: 1.5, 4: 2.0, 5: 3.0, 6: 4.0, 7: 6.0}


def _silu(v):
    return v / (1.0 + math.exp(-v))


def _const_nvfp4(R, K, code_byte, scale_byte, g=1.0):
    return (np.full((R, K // 2), code_byte, np.uint8),
            np.full((R, K // 16), scale_byte, np.uint8), np.float32(g))


def _const_expert(H, I, code13=0x22, code_up=None, code2=0x22, sc13=0x38, sc2=0x38, g13=1.0, g2=1.0):
    c13, s13, _ = _const_nvfp4(2 * I, H, code13, sc13)
    if code_up is not None:
        c13[I:] = code_up
    c2, s2, _ = _const_nvfp4(H, I, code2, sc2)
    return {"codes13": c13, "scales13": s13, "codes2": c2, "scales2": s2,
            "g13": np.float32(g13), "g2": np.float32(g2)}


def _random_nvfp4_expert(rng, H, I):
    def sc(shape):
        return to_e4m3_bytes(np.abs(rng.standard_normal(shape)) * 0.05)
    return {"codes13": rng.integers(0, 256, (2 * I, H // 2), dtype=np.uint8),
            "scales13": sc((2 * I, H // 16)),
            "codes2": rng.integers(0, 256, (H, I // 2), dtype=np.uint8),
            "scales2": sc((H, I // 16)),
            "g13": np.float32(rng.choice([1.0, 0.7, 2.0])),
            "g2": np.float32(rng.choice([1.0, 0.5, 1.3]))}


def _tiny_random_layer(rng, H=32, I=32, E=5, k=2, S=1, route="sigmoid", bias=False, gamma=False):
    n_rows = E + (S if route == "sink" else 0)
    router = to_bf16_bits(rng.normal(0, 0.3, size=(n_rows, H)))
    return ArrayLayer(hidden=H, inter=I, top_k=k, router_w=router,
                      routed=[_random_nvfp4_expert(rng, H, I) for _ in range(E)],
                      shared=[_random_nvfp4_expert(rng, H, I) for _ in range(S)],
                      route=route,
                      router_bias=(rng.normal(0, 0.5, E).astype(np.float32) if bias else None),
                      gamma=(to_bf16_bits(rng.uniform(0.5, 1.5, H)) if gamma else None),
                      residual=gamma)


# ---------------------------------------------------------------------------
# brute force: scalar Python loops straight from the definitions
# ---------------------------------------------------------------------------

def _scalar_dequant(codes, scales, g, r, c):
    byte = int(codes[r][c // 2])
    code = (byte & 0xF) if c % 2 == 0 else (byte >> 4)
    mag = E2M1[code & 7]
    val = -mag if code & 8 else mag
    sb = int(scales[r][c // 16])
    sgn = -1.0 if sb & 0x80 else 1.0
    e, m = (sb >> 3) & 15, sb & 7
    sv = sgn * ((m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return val * sv * float(g)


def _bf16(bits):
    import struct
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def _brute_layer(layer, x_bits, forced=None):
    """forced: optional per-token list of experts used instead of the top-k
    (their weights still follow the routing rule's definition)."""
    H, I, E, k, S = layer.hidden, layer.inter, layer.n_routed, layer.top_k, layer.n_shared
    outs = []
    for b_row, row in enumerate(x_bits):
        x = [_bf16(v) for v in row]
        if layer.gamma is not None:
            ms = math.fsum(v * v for v in x) / H
            x_hat = [x[i] / math.sqrt(ms + layer.eps) * _bf16(layer.gamma[i]) for i in range(H)]
        else:
            x_hat = list(x)
        n_rows = E + (S if layer.route == "sink" else 0)
        logit = [math.fsum(x_hat[h] * _bf16(layer.router_w[e][h]) for h in range(H)) for e in range(n_rows)]
        if layer.router_bias is not None:
            for e in range(E):
                logit[e] += float(layer.router_bias[e])
        order = sorted(range(E), key=lambda e: (-logit[e], e))[:k]
        if forced is not None:
            order = [int(e) for e in forced[b_row]]
        if layer.route == "sigmoid":
            s = [1 / (1 + math.exp(-v)) for v in logit]
            tot = math.fsum(s[e] for e in order)
            coef = {e: s[e] / tot for e in order}
            cs = [1.0] * S
        else:
            mx = max(logit)
            z = [math.exp(v - mx) for v in logit]
            tot = math.fsum(z)
            coef = {e: z[e] / tot for e in order}
            cs = [z[E + s_] / tot for s_ in range(S)]

        def mlp(ex):
            gate = [math.fsum(_scalar_dequant(ex["codes13"], ex["scales13"], ex["g13"], r, c) * x_hat[c]
                              for c in range(H)) for r in range(I)]
            up = [math.fsum(_scalar_dequant(ex["codes13"], ex["scales13"], ex["g13"], I + r, c) * x_hat[c]
                            for c in range(H)) for r in range(I)]
            h = [_silu(gate[r]) * up[r] for r in range(I)]
            return [math.fsum(_scalar_dequant(ex["codes2"], ex["scales2"], ex["g2"], n, i) * h[i]
                              for i in range(I)) for n in range(H)]

        out = [0.0] * H
        terms = [(coef[e], layer.routed_expert(e)) for e in order] + \
                [(cs[s_], layer.shared_expert(s_)) for s_ in range(S)]
        for cf, ex in terms:
            y = mlp(ex)
            out = [out[n] + cf * y[n] for n in range(H)]
        if layer.residual:
            out = [out[n] + x[n] for n in range(H)]
        outs.append(out)
    return np.array(outs)


@pytest.mark.parametrize("seed,route,bias,gamma", [(1, "sigmoid", False, False), (2, "sigmoid", True, False),
                                                   (3, "sink", False, False), (4, "sigmoid", False, True)])
def test_layer_matches_scalar_brute_force(seed, route, bias, gamma):
    rng = np.random.default_rng(seed)
    layer = _tiny_random_layer(rng, route=route, bias=bias, gamma=gamma,
                               S=2 if route == "sink" else 1)
    x = to_bf16_bits(rng.standard_normal((2, layer.hidden)))
    got = L.moe_layer(layer, x)["out"]
    want = _brute_layer(layer, x)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-11 * np.abs(want).max())


def test_expert_mlp_matches_scalar_loops():
    rng = np.random.default_rng(3)
    H, I = 48, 16
    w13 = rng.normal(size=(2 * I, H))
    w2 = rng.normal(size=(H, I))
    x = rng.normal(size=H)
    h, y = L.expert_mlp(w13, w2, x)
    for r in range(I):
        g = math.fsum(w13[r, c] * x[c] for c in range(H))
        u = math.fsum(w13[I + r, c] * x[c] for c in range(H))
        assert h[r] == pytest.approx(_silu(g) * u, rel=1e-12, abs=1e-12)
    for n in range(H):
        assert y[n] == pytest.approx(math.fsum(w2[n, i] * h[i] for i in range(I)), rel=1e-11, abs=1e-11)


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def _const_layer(H, I, E, k, S, expert_fn, shared_fn=None, route="sigmoid", shared_wtype="nvfp4"):
    rng = np.random.default_rng(11)
    n_rows = E + (S if route == "sink" else 0)
    router = to_bf16_bits(rng.normal(0, 0.5, size=(n_rows, H)))
    shared_fn = shared_fn or expert_fn
    return ArrayLayer(hidden=H, inter=I, top_k=k, router_w=router,
                      routed=[expert_fn(e) for e in range(E)],
                      shared=[shared_fn(s) for s in range(S)], route=route,
                      shared_wtype=shared_wtype)


def test_closed_form_all_ones_sigmoid():
    H, I = 256, 128
    layer = _const_layer(H, I, 16, 2, 1, lambda e: _const_expert(H, I))
    x = to_bf16_bits(np.random.default_rng(5).standard_normal((3, H)))
    r = L.moe_layer(layer, x)
    xs = F.bf16_bits_to_f64(x).sum(axis=1)
    want = 2 * I * np.array([_silu(v) * v for v in xs])   # renormalised w sum to 1, c = 1
    np.testing.assert_allclose(r["out"], np.repeat(want[:, None], H, axis=1), rtol=1e-12)


def test_closed_form_gate_and_up_are_distinct_halves():
    # gate rows all 1.0 (code 2), up rows all 0.5 (code 1): h = silu(S) * S/2
    H, I = 64, 32
    layer = _const_layer(H, I, 4, 1, 1, lambda e: _const_expert(H, I, code13=0x22, code_up=0x11))
    x = to_bf16_bits(np.random.default_rng(6).standard_normal((2, H)))
    r = L.moe_layer(layer, x)
    xs = F.bf16_bits_to_f64(x).sum(axis=1)
    want = 2 * I * np.array([_silu(v) * v / 2 for v in xs])
    np.testing.assert_allclose(r["out"], np.repeat(want[:, None], H, axis=1), rtol=1e-12)


def test_closed_form_down_rows_follow_output_index():
    # W2 row n uses scale byte 0x38 (1.0) for even n and 0x40 (2.0) for odd n
    H, I = 64, 32

    def ex(e):
        d = _const_expert(H, I)
        d["scales2"][1::2, :] = 0x40
        return d
    layer = _const_layer(H, I, 4, 2, 1, ex)
    x = to_bf16_bits(np.random.default_rng(8).standard_normal((1, H)))
    r = L.moe_layer(layer, x)
    v = F.bf16_bits_to_f64(x).sum()
    base = 2 * I * _silu(v) * v
    want = np.where(np.arange(H) % 2 == 1, 2 * base, base)
    np.testing.assert_allclose(r["out"][0], want, rtol=1e-12)


def test_closed_form_sink_all_ones():
    H, I, E, S, k = 64, 32, 8, 2, 3

    def shared_bf16(s):
        return {"w13": np.full((2 * I, H), 0x3F80, np.uint16), "w2": np.full((H, I), 0x3F80, np.uint16)}
    layer = _const_layer(H, I, E, k, S, lambda e: _const_expert(H, I), shared_bf16,
                         route="sink", shared_wtype="bf16")
    x = to_bf16_bits(np.random.default_rng(9).standard_normal((2, H)))
    r = L.moe_layer(layer, x)
    xs = F.bf16_bits_to_f64(x).sum(axis=1)
    for b in range(2):
        mass = r["w"][b].sum() + r["c"][b].sum()
        assert mass < 1.0
        want = mass * I * _silu(xs[b]) * xs[b]
        np.testing.assert_allclose(r["out"][b], want, rtol=1e-12)


def test_zero_routed_scales_leave_only_shared_term():
    H, I = 64, 32
    layer = _const_layer(H, I, 6, 2, 1, lambda e: _const_expert(H, I, sc13=0x00, sc2=0x00),
                         lambda s: _const_expert(H, I))
    x = to_bf16_bits(np.random.default_rng(10).standard_normal((2, H)))
    r = L.moe_layer(layer, x)
    xs = F.bf16_bits_to_f64(x).sum(axis=1)
    want = I * np.array([_silu(v) * v for v in xs])   # shared only, c = 1
    np.testing.assert_allclose(r["out"], np.repeat(want[:, None], H, axis=1), rtol=1e-12)


def test_rmsnorm_closed_form():
    x = np.full((1, 16), 3.0)
    got = L.rmsnorm(x, np.full(16, 2.0), 1e-6)
    assert got[0, 0] == pytest.approx(3.0 / math.sqrt(9.0 + 1e-6) * 2.0, rel=1e-15)
    y = np.random.default_rng(1).normal(size=(2, 32))
    # scale invariance (up to eps)
    np.testing.assert_allclose(L.rmsnorm(4 * y, None, 0.0), L.rmsnorm(y, None, 0.0), rtol=1e-14)
    assert np.mean(L.rmsnorm(y, None, 0.0) ** 2, axis=1) == pytest.approx([1.0, 1.0], rel=1e-14)


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def test_doubling_down_tensor_scales_doubles_output_exactly():
    rng = np.random.default_rng(21)
    layer = _tiny_random_layer(rng, E=6, k=2)
    x = to_bf16_bits(rng.standard_normal((2, layer.hidden)))
    a = L.moe_layer(layer, x)["out"]
    for ex in layer._routed + layer._shared:
        ex["g2"] = np.float32(ex["g2"] * 2)
    b = L.moe_layer(layer, x)["out"]
    assert (b == 2 * a).all()


def test_expert_permutation_permutes_ids_only():
    rng = np.random.default_rng(22)
    layer = _tiny_random_layer(rng, E=6, k=3)
    x = to_bf16_bits(rng.standard_normal((2, layer.hidden)))
    a = L.moe_layer(layer, x)
    perm = rng.permutation(6)            # new expert j is old expert perm[j]
    inv = np.argsort(perm)
    layer2 = ArrayLayer(hidden=layer.hidden, inter=layer.inter, top_k=3,
                        router_w=layer.router_w[perm], routed=[layer._routed[p] for p in perm],
                        shared=layer._shared)
    b = L.moe_layer(layer2, x)
    np.testing.assert_allclose(b["out"], a["out"], rtol=1e-12, atol=1e-12)
    for bt in range(2):
        assert sorted(perm[b["ids"][bt]].tolist()) == sorted(a["ids"][bt].tolist())
        assert sorted(inv[a["ids"][bt]].tolist()) == sorted(b["ids"][bt].tolist())


def test_tokens_are_independent():
    rng = np.random.default_rng(23)
    layer = _tiny_random_layer(rng, E=6, k=2)
    x = to_bf16_bits(rng.standard_normal((3, layer.hidden)))
    full = L.moe_layer(layer, x)["out"]
    for b in range(3):
        one = L.moe_layer(layer, x[b:b + 1])["out"]
        np.testing.assert_array_equal(one[0], full[b])


def test_residual_adds_input():
    rng = np.random.default_rng(24)
    layer = _tiny_random_layer(rng, gamma=True)
    x = to_bf16_bits(rng.standard_normal((2, layer.hidden)))
    with_res = L.moe_layer(layer, x)["out"]
    layer.residual = False
    without = L.moe_layer(layer, x)["out"]
    np.testing.assert_array_equal(with_res, without + F.bf16_bits_to_f64(x))


def test_forced_selection_recomputes_weights():
    rng = np.random.default_rng(25)
    layer = _tiny_random_layer(rng, E=6, k=2)
    x = to_bf16_bits(rng.standard_normal((1, layer.hidden)))
    a = L.moe_layer(layer, x)
    forced = np.array([[int(a["ids"][0, 1]), int(a["ids"][0, 0])]])
    b = L.moe_layer(layer, x, force_ids=forced)
    np.testing.assert_allclose(b["out"], a["out"], rtol=1e-13)   # same set, other order


@pytest.mark.parametrize("route", ["sigmoid", "sink"])
def test_forced_selection_of_another_set_follows_the_routing_rule(route):
    """The re-run used for near-tied tokens: a selection that is NOT the
    top-k.  Sigmoid mode: w = s_T / sum s_T over the forced set T.  Sink
    mode: w = p_T, the forced experts' own softmax probabilities, not
    renormalised.  Checked against hand-written scalar formulas and the
    scalar brute-force layer."""
    rng = np.random.default_rng(26 if route == "sigmoid" else 27)
    layer = _tiny_random_layer(rng, E=6, k=2, S=2 if route == "sink" else 1, route=route)
    x = to_bf16_bits(rng.standard_normal((2, layer.hidden)))
    a = L.moe_layer(layer, x)
    # the two lowest-scoring routed experts of each token, lowest first
    forced = np.array([sorted(range(6), key=lambda e: (a["logits"][b, e], e))[:2] for b in range(2)])
    for b in range(2):
        assert not set(forced[b].tolist()) & set(a["ids"][b].tolist())
    r = L.moe_layer(layer, x, force_ids=forced)
    assert r["ids"].tolist() == forced.tolist()
    for b in range(2):
        lg = [float(v) for v in a["logits"][b]]
        if route == "sigmoid":
            s = [1.0 / (1.0 + math.exp(-v)) for v in lg]
            tot = s[forced[b, 0]] + s[forced[b, 1]]
            want = [s[forced[b, 0]] / tot, s[forced[b, 1]] / tot]
            assert abs(sum(r["w"][b]) - 1.0) < 1e-12
        else:
            mx = max(lg)
            z = [math.exp(v - mx) for v in lg]
            tot = math.fsum(z)
            want = [z[forced[b, 0]] / tot, z[forced[b, 1]] / tot]
            assert sum(r["w"][b]) < 0.5          # not renormalised: two low-probability experts
            np.testing.assert_allclose(r["c"][b], [z[6] / tot, z[7] / tot], rtol=1e-12)
        np.testing.assert_allclose(r["w"][b], want, rtol=1e-12)
    np.testing.assert_allclose(r["out"], _brute_layer(layer, x, forced=forced), rtol=1e-9, atol=1e-9)
    assert np.max(np.abs(r["out"] - a["out"])) > 1e-3 * np.max(np.abs(a["out"]))


def test_sigmoid_is_finite_and_exact_at_large_arguments():
    import warnings
    with warnings.catch_warnings():
        warnings.simplefilter("error")
        v = L._sigmoid(np.array([-1000.0, -40.0, 0.0, 40.0, 1000.0]))
    assert v[0] == 0.0 and v[-1] == 1.0 and v[2] == 0.5
    np.testing.assert_allclose(v[1], math.exp(-40.0) / (1.0 + math.exp(-40.0)), rtol=1e-15)


def test_synth_layer_is_deterministic_and_distributed_as_stated():
    a = SynthLayer("tiny")
    b = SynthLayer("tiny")
    assert (a.router_w == b.router_w).all()
    ea, eb = a.routed_expert(3), b.routed_expert(3)
    assert all((ea[key] == eb[key]).all() for key in ("codes13", "scales13", "codes2", "scales2"))
    assert not (a.routed_expert(4)["codes13"] == ea["codes13"]).all()
    assert (a.x(0) == b.x(0)).all() and not (a.x(1) == a.x(0)).all()
    # scale bytes |N(0,1)|*0.05 in e4m3: some exact zeros, many subnormals
    fl = SynthLayer("flint_b1")
    sc = np.concatenate([fl.routed_expert(e)["scales13"].ravel() for e in range(4)])
    zero_frac = np.mean(sc == 0)
    sub_frac = np.mean((sc >> 3) == 0)
    assert 0.005 < zero_frac < 0.03
    assert 0.15 < sub_frac < 0.30
    codes = fl.routed_expert(0)["codes13"]
    nib = np.concatenate([codes & 15, codes >> 4]).ravel()
    counts = np.bincount(nib, minlength=16)
    assert counts.min() > 0.9 * nib.size / 16
