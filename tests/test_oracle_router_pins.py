"""Pins of the oracle's baseline routers (oracle_route_with), against things
other than itself.

Sources: the MoE architecture blog (intelliparadigm.com) §2.1, the Switch
Transformer router, a softmax over x W_r with TOP-K selection (K usually 2);
§5.1, ReMoE, G(x) = ReLU(x W_g) with the output divided by the sum of G.
The reading taken: the top-k router keeps each selected expert's softmax
probability (no renormalisation over the k), ties go to the lower index;
ReMoE's division by sum(G) is folded into the gates.

Pins: numpy argsort / scipy softmax on an independently computed z; a
hand-worked tie; stability for huge logits; sum(g) = 1 identities; exact
invariance of ReMoE gates under scaling (W_r, b) by 2.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from workload import make_layer, make_tokens

HERE = os.path.dirname(os.path.abspath(__file__))


def _z_numpy(x, w_r, b):
    return x.astype(np.float64) @ w_r.astype(np.float64).T + b.astype(np.float64)


@pytest.mark.parametrize("E,k", [(8, 1), (8, 2), (64, 2), (65, 4), (128, 8), (128, 128), (5, 5)])
def test_topk_softmax_matches_library(E, k):
    rng = np.random.default_rng(100 + E + k)
    d = 48
    layer = make_layer(d, E, 16, "f32", 0.3, rng)
    x = make_tokens(d, 6, 4, 0.5, "f32", rng).x
    z, g, m = oracle.route_with(x, layer.w_router, layer.b_router, oracle.ROUTER_TOPK_SOFTMAX, k)
    zn = _z_numpy(x, layer.w_router, layer.b_router)
    np.testing.assert_allclose(z, zn, rtol=1e-12, atol=1e-12)
    p = softmax(zn, axis=1)
    for t in range(x.shape[0]):
        sel = np.sort(np.argsort(-zn[t], kind="stable")[:k])
        bits = [i for i in range(E) if (int(m[t, i // 64]) >> (i % 64)) & 1]
        assert bits == sel.tolist()
        expect = np.zeros(E)
        expect[sel] = p[t, sel]
        np.testing.assert_allclose(g[t], expect, rtol=1e-12, atol=1e-15)
    if k == E:
        np.testing.assert_allclose(g.sum(axis=1), 1.0, rtol=1e-14)


def test_topk_ties_go_to_the_lower_index():
    ex = json.load(open(os.path.join(HERE, "golden", "router_baselines.json")))["topk_tie"]
    x = np.array(ex["x"], np.float32)[None, :]
    w = np.array(ex["w_router"], np.float32)
    b = np.zeros(w.shape[0], np.float32)
    for k_str, want in ex["selected"].items():
        z, g, m = oracle.route_with(x, w, b, oracle.ROUTER_TOPK_SOFTMAX, int(k_str))
        np.testing.assert_array_equal(z[0], ex["z"])
        bits = [i for i in range(w.shape[0]) if (int(m[0, 0]) >> i) & 1]
        assert bits == want
        for i, v in ex["gates"][k_str].items():
            assert abs(g[0, int(i)] - v) <= 1e-15


def test_topk_softmax_is_stable_for_huge_logits():
    rng = np.random.default_rng(7)
    d, E = 16, 32
    w = (rng.standard_normal((E, d)) * 200.0).astype(np.float32)
    x = rng.standard_normal((5, d)).astype(np.float32)
    z, g, m = oracle.route_with(x, w, np.zeros(E, np.float32), oracle.ROUTER_TOPK_SOFTMAX, E)
    assert np.isfinite(g).all() and np.abs(z).max() > 500
    np.testing.assert_allclose(g.sum(axis=1), 1.0, rtol=1e-14)


def test_relu_sum_router_identities():
    rng = np.random.default_rng(17)
    d, E = 40, 70
    layer = make_layer(d, E, 16, "f32", 0.8, rng)
    x = make_tokens(d, 8, 3, 0.6, "f32", rng).x
    z, g, m = oracle.route_with(x, layer.w_router, layer.b_router, oracle.ROUTER_RELU_SUM)
    zn = _z_numpy(x, layer.w_router, layer.b_router)
    a = np.maximum(zn, 0.0)
    on = (z > 0).any(axis=1)
    assert on.any()
    np.testing.assert_allclose(g[on].sum(axis=1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(g[on], a[on] / a[on].sum(axis=1, keepdims=True), rtol=1e-12, atol=1e-15)
    assert np.all(g[~on] == 0)
    for t in range(x.shape[0]):
        bits = [i for i in range(E) if (int(m[t, i // 64]) >> (i % 64)) & 1]
        assert bits == np.nonzero(z[t] > 0)[0].tolist()
    # scaling (W_r, b) by 2 is exact in binary and leaves every gate unchanged
    z2, g2, m2 = oracle.route_with(x, (layer.w_router * 2).astype(np.float32),
                                   (layer.b_router * 2).astype(np.float32), oracle.ROUTER_RELU_SUM)
    np.testing.assert_array_equal(g2, g)
    np.testing.assert_array_equal(m2, m)


def test_relu_sum_router_without_active_expert():
    d, E = 8, 4
    x = np.ones((2, d), np.float32)
    w = -np.ones((E, d), np.float32)
    z, g, m = oracle.route_with(x, w, np.zeros(E, np.float32), oracle.ROUTER_RELU_SUM)
    assert np.all(g == 0) and np.all(m == 0)


def test_bad_router_arguments_are_rejected():
    x = np.ones((1, 8), np.float32)
    w = np.ones((4, 8), np.float32)
    with pytest.raises(RuntimeError):
        oracle.route_with(x, w, None, oracle.ROUTER_TOPK_SOFTMAX, 0)
    with pytest.raises(RuntimeError):
        oracle.route_with(x, w, None, oracle.ROUTER_TOPK_SOFTMAX, 5)
    with pytest.raises(RuntimeError):
        oracle.route_with(x, w, None, 3, 1)
