"""Pins for the oracle's routing rules (CPU only): hand-checked cases and
brute force over all subsets."""

import itertools
import math

import numpy as np
import pytest

from oracle import layer as L


def _sig(v):
    return 1.0 / (1.0 + math.exp(-v))


def test_sigmoid_top2_hand_case_with_tie():
    logits = np.array([0.1, 2.0, -1.0, 3.0, 0.5, 2.0, -3.0, 0.0])
    ids, w, c, s = L.route_sigmoid_topk(logits, 2, 1)
    # 3.0 first; 2.0 appears at indices 1 and 5 -> the lower index wins
    assert ids.tolist() == [3, 1]
    s3, s1 = _sig(3.0), _sig(2.0)
    assert w[0] == pytest.approx(s3 / (s3 + s1), rel=1e-15)
    assert w[1] == pytest.approx(s1 / (s3 + s1), rel=1e-15)
    assert c.tolist() == [1.0]
    assert s[6] == pytest.approx(_sig(-3.0), rel=1e-15)


def test_exact_ties_go_to_lower_index():
    ids, _, _, _ = L.route_sigmoid_topk(np.zeros(10), 4, 1)
    assert ids.tolist() == [0, 1, 2, 3]
    ids, _, _, _ = L.route_softmax_sink(np.zeros(12), 10, 3)
    assert ids.tolist() == [0, 1, 2]


def test_k_equals_E_selects_all_and_renormalises():
    logits = np.array([0.3, -0.2, 1.7, 0.0, -2.5])
    ids, w, _, s = L.route_sigmoid_topk(logits, 5, 1)
    assert sorted(ids.tolist()) == [0, 1, 2, 3, 4]
    want = np.array([_sig(v) for v in logits])
    want = want / want.sum()
    for j, e in enumerate(ids):
        assert w[j] == pytest.approx(want[e], rel=1e-14)
    assert w.sum() == pytest.approx(1.0, rel=1e-15)


@pytest.mark.parametrize("E", [3, 6, 9, 10])
def test_sigmoid_topk_brute_force(E):
    rng = np.random.default_rng(E)
    for _ in range(20):
        logits = rng.normal(size=E)
        for k in range(1, E + 1):
            ids, w, _, s = L.route_sigmoid_topk(logits, k, 1)
            best = max(itertools.combinations(range(E), k),
                       key=lambda sub: sum(_sig(logits[i]) for i in sub))
            assert set(ids.tolist()) == set(best)
            sel = set(ids.tolist())
            if k < E:
                assert min(s[i] for i in sel) >= max(s[i] for i in range(E) if i not in sel)
            assert abs(sum(w) - 1.0) < 1e-12
            # selection order is by descending score
            assert all(s[a] >= s[b] for a, b in zip(ids, ids[1:]))


def test_sink_probabilities_and_exclusion():
    E, S, k = 8, 2, 3
    logits = np.array([0.5, 1.0, -0.3, 2.0, 0.0, 1.5, -1.0, 0.2, 5.0, 4.0])
    ids, w, c, p_routed = L.route_softmax_sink(logits, E, k)
    z = [math.exp(v) for v in logits]
    tot = math.fsum(z)
    p = [v / tot for v in z]
    # the two shared logits are the largest but are never candidates
    assert ids.tolist() == [3, 5, 1]
    for j, e in enumerate(ids):
        assert w[j] == pytest.approx(p[e], rel=1e-14)
    assert c[0] == pytest.approx(p[8], rel=1e-14) and c[1] == pytest.approx(p[9], rel=1e-14)
    assert math.fsum(p_routed) + math.fsum(c) == pytest.approx(1.0, rel=1e-15)
    # routed weights are not renormalised
    assert w.sum() < 1.0 - 0.5


@pytest.mark.parametrize("E", [4, 7, 10])
def test_sink_topk_brute_force(E):
    rng = np.random.default_rng(100 + E)
    for _ in range(10):
        logits = rng.normal(size=E + 2)
        for k in range(1, E + 1):
            ids, w, c, p = L.route_softmax_sink(logits, E, k)
            best = max(itertools.combinations(range(E), k), key=lambda sub: sum(p[i] for i in sub))
            assert set(ids.tolist()) == set(best)
            assert (ids < E).all()


def test_selection_gap():
    assert L.selection_gap(np.array([0.9, 0.1, 0.5, 0.7]), 2) == pytest.approx(0.2)
    assert L.selection_gap(np.array([0.3, 0.3, 0.1]), 1) == 0.0
    assert L.selection_gap(np.array([0.3, 0.2]), 2) == math.inf


def test_router_logits_bias_applies_to_routed_only():
    xh = np.array([[1.0, 2.0]])
    R = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    l = L.router_logits(xh, R, np.array([0.5, -0.5]))
    assert l.tolist() == [[1.5, 1.5, 3.0]]
