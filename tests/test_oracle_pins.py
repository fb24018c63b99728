"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against a hand-worked example, a closed form, an
invariant, brute force, or a special case that reduces to a library routine
(numpy matmul, scipy's logistic function).  Sources of the definitions: the
BlockFFN write-up (lsdiaocha.cn) §2 and §4, and the BlockFFN abstract
(arXiv 2507.08771).
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle
from workload import bf16_round_bits, bf16_bits_to_f32


def _f64(a):
    a = np.asarray(a)
    return bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def _rand_layer(rng, d, E, de, dtype="f32", bias=0.0):
    wr = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    wi = (rng.standard_normal((E, de, d)) / np.sqrt(d)).astype(np.float32)
    wo = (rng.standard_normal((E, d, de)) / np.sqrt(de)).astype(np.float32)
    b = (np.full(E, bias) + 0.3 * rng.standard_normal(E)).astype(np.float32)
    if dtype == "bf16":
        wr, wi, wo = bf16_round_bits(wr), bf16_round_bits(wi), bf16_round_bits(wo)
    return wr, b, wi, wo


def _rand_x(rng, T, d, dtype="f32"):
    x = rng.standard_normal((T, d)).astype(np.float32)
    return bf16_round_bits(x) if dtype == "bf16" else x


# ---------------------------------------------------------------- hand-worked example

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hand_example_router_and_expert(golden, dtype):
    ex = golden["router_expert"]
    conv = (lambda a: bf16_round_bits(np.asarray(a, np.float32))) if dtype == "bf16" else \
        (lambda a: np.asarray(a, np.float32))
    x, wr, wi, wo = conv(ex["x"]), conv(ex["w_router"]), conv(ex["w_in"]), conv(ex["w_out"])
    b = np.asarray(ex["b_router"], np.float32)
    z, g, m = oracle.route(x, wr, b, None, 1e-6)
    np.testing.assert_array_equal(z, np.asarray(ex["expected_z"]))
    np.testing.assert_allclose(g, np.asarray(ex["expected_g"]), rtol=1e-15, atol=0)
    assert m[:, 0].tolist() == ex["expected_mask"]
    y = oracle.forward_tokens(x, wi, wo, g, m)
    np.testing.assert_allclose(y, np.asarray(ex["expected_y"]), rtol=1e-14, atol=0)
    um, cnt, lst = oracle.chunk_union(m, 4, 1)
    np.testing.assert_array_equal(oracle.forward_chunks(x, wi, wo, g, 1, cnt, lst), y)
    np.testing.assert_array_equal(oracle.forward_dense(x, wi, wo, g), y)


def test_hand_example_union_and_stats(golden):
    ex = golden["masks_union_stats"]
    E, L = ex["n_experts"], ex["chunk_len"]
    sets = ex["active_sets"]
    m = np.zeros((len(sets), 2), np.uint64)
    for t, s in enumerate(sets):
        for i in s:
            m[t, i // 64] |= np.uint64(1) << np.uint64(i % 64)
    um, cnt, lst = oracle.chunk_union(m, E, L)
    for c, want in enumerate(ex["expected_union_lists"]):
        assert cnt[c] == len(want)
        assert lst[c, : cnt[c]].tolist() == want
        assert (lst[c, cnt[c]:] == -1).all()
    st = oracle.stats(m, E, L)
    assert st["active_pairs"] == ex["expected_active_pairs"]
    assert st["union_sum"] == ex["expected_union_sum"]
    assert st["tls"] == pytest.approx(ex["expected_tls"], abs=1e-15)
    assert st["cls"] == pytest.approx(ex["expected_cls"], abs=1e-15)
    assert st["hist"][:4].tolist() == ex["expected_hist_prefix"]
    assert st["hist"][4:].sum() == 0
    assert (st["reuse_num"], st["reuse_den"]) == (ex["expected_reuse_num"], ex["expected_reuse_den"])


def test_bf16_widening_known_patterns():
    # bf16 is the upper half of a binary32: 0x3F80 = 1.0, 0xC000 = -2.0,
    # 0x3F81 = 1 + 2^-7, 0x0001 = the smallest bf16 subnormal 2^-133.
    w = np.array([[0x3F80]], np.uint16)
    for bits, val in [(0x3F80, 1.0), (0xC000, -2.0), (0x3F81, 1.0078125), (0x0001, 2.0 ** -133)]:
        z, _, _ = oracle.route(np.array([[bits]], np.uint16), w, None, None, 1e-6)
        assert z[0, 0] == val


# ---------------------------------------------------------------- router

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_router_preactivation_equals_matmul(dtype):
    rng = np.random.default_rng(11)
    d, E, T = 96, 70, 13
    wr, b, _, _ = _rand_layer(rng, d, E, 16, dtype)
    x = _rand_x(rng, T, d, dtype)
    z, g, m = oracle.route(x, wr, b, None, 1e-6)
    ref = _f64(x) @ _f64(wr).T + b.astype(np.float64)
    np.testing.assert_allclose(z, ref, rtol=1e-12, atol=1e-13)


def test_router_pattern_gates_and_rms():
    rng = np.random.default_rng(12)
    d, E, T = 64, 37, 50
    wr, b, _, _ = _rand_layer(rng, d, E, 16, bias=-0.5)
    x = _rand_x(rng, T, d)
    eps = 1e-6
    z, g, m = oracle.route(x, wr, b, None, eps)
    for t in range(T):
        want = {i for i in range(E) if z[t, i] > 0}
        got = {i for i in range(E) if (int(m[t, i // 64]) >> (i % 64)) & 1}
        assert got == want
        assert (g[t] >= 0).all()
        assert {i for i in range(E) if g[t, i] > 0} == want
        a = np.maximum(z[t], 0)
        ms = float((a * a).mean())
        # closed form: with unit scale, mean(g^2) = ms / (ms + eps)
        assert float((g[t] ** 2).mean()) == pytest.approx(ms / (ms + eps), rel=1e-12, abs=1e-300)


def test_router_eps_zero_normalises_exactly():
    rng = np.random.default_rng(13)
    wr, b, _, _ = _rand_layer(rng, 32, 16, 16, bias=0.5)
    x = _rand_x(rng, 20, 32)
    _, g, m = oracle.route(x, wr, b, None, 0.0)
    active = m[:, 0] != 0
    assert active.all()
    np.testing.assert_allclose(np.sqrt((g ** 2).mean(axis=1)), 1.0, rtol=1e-14)


def test_router_pattern_and_magnitude_separate():
    # write-up §2: RMSNorm separates the activation pattern from its strength.
    # Scaling (W_r, b) by c > 0 keeps the pattern; with eps = 0 the gates are
    # unchanged (bit-for-bit for c = 2, where every product scales exactly).
    rng = np.random.default_rng(14)
    wr, b, _, _ = _rand_layer(rng, 48, 24, 16, bias=-0.3)
    x = _rand_x(rng, 30, 48)
    z1, g1, m1 = oracle.route(x, wr, b, None, 0.0)
    z2, g2, m2 = oracle.route(x, wr * 2, b * 2, None, 0.0)
    np.testing.assert_array_equal(m1, m2)
    np.testing.assert_array_equal(g1, g2)
    # c = 3 rounds the stored fp32 weights, so the gates move by fp32 rounding only
    z3, g3, m3 = oracle.route(x, wr * 3, b * 3, None, 0.0)
    np.testing.assert_array_equal(m1, m3)
    np.testing.assert_allclose(g1, g3, rtol=2e-6, atol=1e-7)


def test_router_scale_vector_and_no_bias():
    rng = np.random.default_rng(15)
    wr, b, _, _ = _rand_layer(rng, 40, 12, 16)
    x = _rand_x(rng, 9, 40)
    s = rng.uniform(0.5, 2.0, 12).astype(np.float32)
    _, g1, _ = oracle.route(x, wr, b, None, 1e-6)
    _, gs, _ = oracle.route(x, wr, b, s, 1e-6)
    np.testing.assert_allclose(gs, g1 * s.astype(np.float64), rtol=1e-15)
    z0, _, _ = oracle.route(x, wr, None, None, 1e-6)
    np.testing.assert_allclose(z0, _f64(x) @ _f64(wr).T, rtol=1e-12, atol=1e-13)


def test_router_tie_and_no_active_token():
    # z = 0 exactly is inactive; a token with no active expert gets zero gates
    # and a zero output.
    wr = np.array([[1.0, -1.0], [0.0, 0.0], [-1.0, -1.0]], np.float32)
    x = np.array([[2.0, 2.0], [1.0, 1.0]], np.float32)
    z, g, m = oracle.route(x, wr, None, None, 1e-6)
    assert (z[0] == [0.0, 0.0, -4.0]).all()
    assert (m == 0).all() and (g == 0).all()
    wi = np.ones((3, 4, 2), np.float32)
    wo = np.ones((3, 2, 4), np.float32)
    y = oracle.forward_tokens(x, wi, wo, g, m)
    assert (y == 0).all()


# ---------------------------------------------------------------- experts and layer

def _dense_mlp_reference(x, wi, wo, g):
    """y = W_out_cat (g_rep * SiLU(W_in_cat x)): numpy matmul + scipy logistic."""
    x64, wi64, wo64 = _f64(x), _f64(wi), _f64(wo)
    E, de, d = wi64.shape
    w_in_cat = wi64.reshape(E * de, d)                      # [E d_e][d]
    w_out_cat = wo64.transpose(1, 0, 2).reshape(d, E * de)  # [d][E d_e]
    u = x64 @ w_in_cat.T                                    # [T][E d_e]
    h = u * expit(u)
    g_rep = np.repeat(g, de, axis=1)
    return (g_rep * h) @ w_out_cat.T


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bias", [10.0, -0.8])
def test_layer_equals_dense_mlp_over_concatenated_experts(dtype, bias):
    rng = np.random.default_rng(21)
    d, E, de, T = 72, 9, 24, 17
    wr, b, wi, wo = _rand_layer(rng, d, E, de, dtype, bias=bias)
    x = _rand_x(rng, T, d, dtype)
    z, g, m = oracle.route(x, wr, b, None, 1e-6)
    if bias > 0:
        assert (z > 0).all()
    y = oracle.forward_tokens(x, wi, wo, g, m)
    ref = _dense_mlp_reference(x, wi, wo, g)
    scale = np.sqrt((ref ** 2).mean())
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12 * scale)


def test_single_expert_matches_library_mlp():
    rng = np.random.default_rng(22)
    d, de, T = 50, 20, 8
    wr, b, wi, wo = _rand_layer(rng, d, 1, de, bias=0.0)
    x = _rand_x(rng, T, d)
    z, g, m = oracle.route(x, wr, b, None, 1e-6)
    for t in range(T):
        if z[t, 0] > 0:
            a = z[t, 0]
            assert g[t, 0] == pytest.approx(a / np.sqrt(a * a + 1e-6), rel=1e-15)
            u = _f64(wi[0]) @ _f64(x[t])
            ref = g[t, 0] * (_f64(wo[0]) @ (u * expit(u)))
            e = oracle.expert(x, t, wi, wo, 0)
            np.testing.assert_allclose(g[t, 0] * e, ref, rtol=1e-12, atol=1e-14)
        else:
            assert g[t, 0] == 0.0
    y = oracle.forward_tokens(x, wi, wo, g, m)
    np.testing.assert_allclose(y, _dense_mlp_reference(x, wi, wo, g), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dense_and_chunk_evaluations_are_bit_identical(dtype):
    # Zero-gate experts contribute exactly nothing (write-up §4: compute over
    # the union, mask the rest), so evaluating every expert, or every expert of
    # the chunk's union, gives the per-token sparse result bit for bit.
    rng = np.random.default_rng(23)
    d, E, de, L, C = 64, 20, 16, 4, 6
    wr, b, wi, wo = _rand_layer(rng, d, E, de, dtype, bias=-1.0)
    x = _rand_x(rng, L * C, d, dtype)
    z, g, m = oracle.route(x, wr, b, None, 1e-6)
    um, cnt, lst = oracle.chunk_union(m, E, L)
    y_tok = oracle.forward_tokens(x, wi, wo, g, m)
    np.testing.assert_array_equal(oracle.forward_chunks(x, wi, wo, g, L, cnt, lst), y_tok)
    np.testing.assert_array_equal(oracle.forward_dense(x, wi, wo, g), y_tok)
    assert (cnt < E).any()  # the case really is sparse


# ---------------------------------------------------------------- union and stats, brute force

def _random_masks(rng, T, E, p):
    act = rng.random((T, E)) < p
    W = (E + 63) // 64
    m = np.zeros((T, W), np.uint64)
    for t in range(T):
        for i in np.nonzero(act[t])[0]:
            m[t, i // 64] |= np.uint64(1) << np.uint64(int(i) % 64)
    return act, m


@pytest.mark.parametrize("E,L,C,p", [(1, 1, 5, 0.5), (8, 4, 16, 0.2), (63, 3, 7, 0.1),
                                     (64, 8, 9, 0.15), (65, 2, 11, 0.3), (128, 32, 3, 0.05),
                                     (128, 8, 10, 0.0), (100, 5, 4, 1.0)])
def test_union_and_stats_brute_force(E, L, C, p):
    rng = np.random.default_rng(E * 1000 + L)
    T = L * C
    act, m = _random_masks(rng, T, E, p)
    sets = [set(np.nonzero(act[t])[0].tolist()) for t in range(T)]
    um, cnt, lst = oracle.chunk_union(m, E, L)
    union_sum = 0
    for c in range(C):
        u = set().union(*sets[c * L:(c + 1) * L])
        union_sum += len(u)
        assert cnt[c] == len(u)
        assert lst[c, :cnt[c]].tolist() == sorted(u)
        assert (lst[c, cnt[c]:] == -1).all()
        assert cnt[c] >= max(len(s) for s in sets[c * L:(c + 1) * L])
        for w in range(um.shape[1]):
            bits = {i for i in range(E) if i // 64 == w and (int(um[c, w]) >> (i % 64)) & 1}
            assert bits == {i for i in u if i // 64 == w}
    st = oracle.stats(m, E, L)
    pairs = sum(len(s) for s in sets)
    assert st["active_pairs"] == pairs and st["union_sum"] == union_sum
    assert st["tls"] == pytest.approx(1 - pairs / (T * E), abs=1e-15)
    assert st["cls"] == pytest.approx(1 - union_sum / (C * E), abs=1e-15)
    hist = np.zeros(E + 1, np.int64)
    for s in sets:
        hist[len(s)] += 1
    np.testing.assert_array_equal(st["hist"], hist)
    num = sum(len(sets[t] & sets[t - 1]) for t in range(1, T))
    den = sum(len(sets[t - 1]) for t in range(1, T))
    assert (st["reuse_num"], st["reuse_den"]) == (num, den)


def test_chunk_sparsity_relations():
    # CLS_1 = TLS, CLS_L <= TLS, CLS_2L <= CLS_L for aligned chunks.
    rng = np.random.default_rng(31)
    act, m = _random_masks(rng, 64, 40, 0.15)
    tls = oracle.stats(m, 40, 1)["tls"]
    assert oracle.stats(m, 40, 1)["cls"] == pytest.approx(tls, abs=1e-15)
    prev = tls
    for L in (2, 4, 8, 16, 32, 64):
        cls = oracle.stats(m, 40, L)["cls"]
        assert cls <= prev + 1e-15
        prev = cls


def test_ragged_tail_rejected():
    m = np.zeros((10, 1), np.uint64)
    with pytest.raises(RuntimeError):
        oracle.chunk_union(m, 8, 4)
