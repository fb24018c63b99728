"""Pins of the oracle's FFF tree layer (oracle_fff_forward), against things
other than itself.

Source: "Dynamic sparsity in tree-structured feed-forward layers at scale"
(write-up on gist.science), §2 methodology: P parallel perfect binary trees
of depth D; per token, hard routing from the root, one root-to-leaf path per
tree; the visited nodes' activations, concatenated over the trees, go
through a final projection; GELU as the node activation; the FFFpost variant
moves the nonlinearity after the sparse output aggregation.  §4: depth 6 is
about 94% sparse, depth 13 above 99%.

Readings taken (the write-up gives no formulas): heap-ordered nodes (children
of n at 2n + 1, 2n + 2); right iff the node's pre-activation c > 0; a depth-D
tree has levels 0..D (2^(D+1) - 1 nodes, D + 1 visited); each node owns an
output row (its column of the final projection); GELU is the exact
c Phi(c); FFFpost applies GELU to the summed output.

Pins: a hand-worked two-tree example (tests/golden/fff_hand_tree.json) with
a pre-activation of exactly 0; the dense evaluation and the depth-0 layer
against a numpy matmul MLP with scipy's normal CDF; brute force over every
leaf of small trees; the all-right and all-left closed forms; the sparsity
figures the write-up quotes; additivity over trees; bf16 inputs against the
same values in f32.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import ndtr

import oracle
from workload import bf16_bits_to_f32, make_fff_layer, make_fff_tokens

HERE = os.path.dirname(os.path.abspath(__file__))


def _gelu(c):
    return c * ndtr(c)


def _f64(a):
    return (bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


def _hand():
    ex = json.load(open(os.path.join(HERE, "golden", "fff_hand_tree.json")))
    P, N = len(ex["w_node_col0"]), len(ex["w_node_col0"][0])
    w = np.zeros((P, N, 2), np.float32)
    w[:, :, 0] = ex["w_node_col0"]
    w[:, :, 1] = ex["w_node_col1"]
    o = np.zeros((P, N, 2), np.float32)
    for p in range(P):
        for n in range(N):
            v = 10 * p + n + 1
            o[p, n] = (v, v * v / 16.0)
    return ex, np.array([ex["x"]], np.float32), w, np.array(ex["b_node"], np.float32), o


def test_hand_worked_tree():
    ex, x, w, b, o = _hand()
    paths, pre, y = oracle.fff_forward(x, w, b, o)
    assert paths[0].tolist() == ex["paths"]
    np.testing.assert_array_equal(pre[0], ex["preact"])
    want = np.zeros(2)
    for p, path in enumerate(ex["paths"]):
        for n, c in zip(path, ex["preact"][p]):
            want += _gelu(c) * o[p, n].astype(np.float64)
    np.testing.assert_allclose(y[0], want, rtol=1e-14, atol=1e-14)
    # FFFpost: linear node activations, GELU on the summed output
    _, _, yp = oracle.fff_forward(x, w, b, o, post=True)
    lin = np.zeros(2)
    for p, path in enumerate(ex["paths"]):
        for n, c in zip(path, ex["preact"][p]):
            lin += c * o[p, n].astype(np.float64)
    np.testing.assert_allclose(yp[0], _gelu(lin), rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("dtype,post", [("f32", False), ("bf16", False), ("f32", True)])
def test_dense_evaluation_is_the_plain_mlp(dtype, post):
    rng = np.random.default_rng(21)
    d, P, D = 24, 3, 3
    layer = make_fff_layer(d, P, D, dtype, rng)
    x = make_fff_tokens(d, 9, dtype, rng)
    _, pre, y = oracle.fff_forward(x, layer.w_node, layer.b_node, layer.w_out, post=post, dense=True)
    N = (1 << (D + 1)) - 1
    X = _f64(x)
    Wn = _f64(layer.w_node).reshape(P * N, d)
    Wo = _f64(layer.w_out).reshape(P * N, d)
    C = X @ Wn.T + layer.b_node.reshape(-1).astype(np.float64)
    np.testing.assert_allclose(pre.reshape(len(x), P * N), C, rtol=1e-12, atol=1e-12)
    want = _gelu(C @ Wo) if post else _gelu(C) @ Wo
    np.testing.assert_allclose(y, want, rtol=1e-11, atol=1e-12)


def test_depth_zero_is_an_mlp_of_p_units():
    rng = np.random.default_rng(22)
    d, P = 40, 7
    layer = make_fff_layer(d, P, 0, "f32", rng)
    x = make_fff_tokens(d, 11, "f32", rng)
    paths, _, y = oracle.fff_forward(x, layer.w_node, layer.b_node, layer.w_out)
    assert np.all(paths == 0)
    _, _, yd = oracle.fff_forward(x, layer.w_node, layer.b_node, layer.w_out, dense=True)
    np.testing.assert_array_equal(y, yd)
    C = _f64(x) @ _f64(layer.w_node)[:, 0, :].T + layer.b_node[:, 0]
    np.testing.assert_allclose(y, _gelu(C) @ _f64(layer.w_out)[:, 0, :], rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("post", [False, True])
def test_paths_by_brute_force_over_every_leaf(post):
    rng = np.random.default_rng(23)
    d, P, D = 16, 3, 3
    layer = make_fff_layer(d, P, D, "f32", rng)
    x = make_fff_tokens(d, 20, "f32", rng)
    paths, pre, y = oracle.fff_forward(x, layer.w_node, layer.b_node, layer.w_out, post=post)
    X, Wn, Wo = _f64(x), _f64(layer.w_node), _f64(layer.w_out)
    B = layer.b_node.astype(np.float64)
    for t in range(len(x)):
        acc = np.zeros(d)
        for p in range(P):
            C = Wn[p] @ X[t] + B[p]          # every node's pre-activation
            consistent = []
            for leaf in range(1 << D):      # the root-to-leaf path ending at this leaf
                nodes = [0]
                for lev in range(D):
                    right = (leaf >> (D - 1 - lev)) & 1
                    nodes.append(2 * nodes[-1] + 1 + right)
                if all((C[nodes[i]] > 0) == (nodes[i + 1] == 2 * nodes[i] + 2) for i in range(D)):
                    consistent.append(nodes)
            assert len(consistent) == 1
            assert paths[t, p].tolist() == consistent[0]
            np.testing.assert_allclose(pre[t, p], C[consistent[0]], rtol=1e-12, atol=1e-13)
            for n in consistent[0]:
                acc += (C[n] if post else _gelu(C[n])) * Wo[p, n]
        np.testing.assert_allclose(y[t], _gelu(acc) if post else acc, rtol=1e-11, atol=1e-12)


def test_all_right_and_all_left_closed_forms():
    rng = np.random.default_rng(24)
    d, P, D = 8, 2, 5
    layer = make_fff_layer(d, P, D, "f32", rng)
    x = make_fff_tokens(d, 4, "f32", rng)
    N = (1 << (D + 1)) - 1
    right, _, _ = oracle.fff_forward(x, layer.w_node, np.full((P, N), 100.0, np.float32), layer.w_out)
    left, _, _ = oracle.fff_forward(x, layer.w_node, np.full((P, N), -100.0, np.float32), layer.w_out)
    assert np.all(right == np.array([(1 << (lv + 1)) - 2 for lv in range(D + 1)]))
    assert np.all(left == np.array([(1 << lv) - 1 for lv in range(D + 1)]))


def test_visited_fraction_matches_the_quoted_sparsity():
    # depth 6 is quoted as about 94% sparse and depth 13 as above 99%: with
    # levels 0..D a tree holds 2^(D+1) - 1 nodes and a token visits D + 1
    for D, lo, hi in ((6, 0.94, 0.95), (13, 0.99, 1.0)):
        rng = np.random.default_rng(25 + D)
        P = 2
        w = np.zeros((P, oracle.fff_nodes(D), 4), np.float32)
        w[..., 0] = rng.standard_normal(w.shape[:2])
        paths, _, _ = oracle.fff_forward(np.ones((3, 4), np.float32), w, None, w)
        visited = len(set(paths[0, 0].tolist()))
        assert visited == D + 1
        assert lo <= 1 - visited / oracle.fff_nodes(D) <= hi


def test_output_is_additive_over_trees_and_tokens():
    rng = np.random.default_rng(26)
    d, P, D = 20, 4, 2
    layer = make_fff_layer(d, P, D, "f32", rng)
    x = make_fff_tokens(d, 6, "f32", rng)
    _, _, y = oracle.fff_forward(x, layer.w_node, layer.b_node, layer.w_out)
    parts = sum(oracle.fff_forward(x, layer.w_node[p:p + 1], layer.b_node[p:p + 1], layer.w_out[p:p + 1])[2]
                for p in range(P))
    np.testing.assert_allclose(y, parts, rtol=1e-12, atol=1e-13)
    one = np.stack([oracle.fff_forward(x[t:t + 1], layer.w_node, layer.b_node, layer.w_out)[2][0]
                    for t in range(len(x))])
    np.testing.assert_array_equal(y, one)


def test_bf16_inputs_equal_their_f32_values():
    rng = np.random.default_rng(27)
    d, P, D = 32, 3, 3
    layer = make_fff_layer(d, P, D, "bf16", rng)
    x = make_fff_tokens(d, 5, "bf16", rng)
    a = oracle.fff_forward(x, layer.w_node, layer.b_node, layer.w_out)
    b = oracle.fff_forward(bf16_bits_to_f32(x), bf16_bits_to_f32(layer.w_node), layer.b_node,
                           bf16_bits_to_f32(layer.w_out))
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_bad_arguments_are_rejected():
    w = np.zeros((1, 3, 4), np.float32)
    with pytest.raises(AssertionError):
        oracle.fff_forward(np.zeros((1, 5), np.float32), w, None, w)   # width mismatch
    with pytest.raises(AssertionError):
        oracle.fff_forward(np.zeros((1, 4), np.float32), np.zeros((1, 4, 4), np.float32), None,
                           np.zeros((1, 4, 4), np.float32))             # not a perfect tree
