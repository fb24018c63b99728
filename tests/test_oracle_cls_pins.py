"""Pins of the oracle's CLS-aware objectives (oracle_cls_losses) and of the
backward's extra router gradient, against things other than themselves.

Source: the BlockFFN write-up (lsdiaocha.cn) §3.  The activation-locality
loss is a binary cross-entropy between neighbouring tokens' activation
patterns: the pattern sequence is shifted left by one token and the
activation pattern is approximated by a sharp sigmoid.  The
chunk-sparsification loss is the probability that an expert fires for at
least one token of an L-token chunk.  Readings (the pages give no formulas):
p = sigmoid(alpha z); the locality target is the next token's hard pattern
(no gradient through it), over every consecutive pair of the stream; both
losses are means (over pairs x experts, chunks x experts).

Pins: torch's binary_cross_entropy_with_logits and autodiff on the same
definition; central finite differences; chunk length 1 (L_CS = mean p); a
hand-worked two-token chunk; the sharp limit, where L_CS equals the union
fraction the sparsity statistics count; linearity of the backward in the
extra router gradient (checked with numpy matmuls).
"""
import numpy as np
import pytest
import torch

import oracle
from workload import make_layer, make_tokens


def _z(seed, T=24, E=10, margin=0.05):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((T, E)) * 0.6
    z = np.where(np.abs(z) < margin, np.sign(z + 1e-12) * margin * 2, z)  # keep away from the kink
    return z


@pytest.mark.parametrize("L,alpha", [(1, 5.0), (4, 10.0), (8, 3.0), (3, 25.0)])
def test_losses_match_torch_autodiff(L, alpha):
    z = _z(3 + L)
    w_al, w_cs = 0.7, 1.9
    al, cs, dz = oracle.cls_losses(z, L, alpha, w_al, w_cs)
    tz = torch.tensor(z, dtype=torch.float64, requires_grad=True)
    y = (tz[1:] > 0).double().detach()
    t_al = torch.nn.functional.binary_cross_entropy_with_logits(alpha * tz[:-1], y, reduction="mean")
    p = torch.sigmoid(alpha * tz)
    T, E = z.shape
    q = torch.prod(1 - p.reshape(T // L, L, E), dim=1)
    t_cs = (1 - q).mean()
    (w_al * t_al + w_cs * t_cs).backward()
    assert abs(al - t_al.item()) <= 1e-12 * max(1.0, abs(al))
    assert abs(cs - t_cs.item()) <= 1e-12
    np.testing.assert_allclose(dz, tz.grad.numpy(), rtol=1e-9, atol=1e-14)


def test_gradient_matches_finite_differences():
    z = _z(41, T=12, E=6)
    L, alpha, w_al, w_cs = 4, 6.0, 1.3, 0.8
    _, _, dz = oracle.cls_losses(z, L, alpha, w_al, w_cs)
    rng = np.random.default_rng(2)
    h = 1e-6
    for _ in range(12):
        t, i = int(rng.integers(z.shape[0])), int(rng.integers(z.shape[1]))
        zp, zm = z.copy(), z.copy()
        zp[t, i] += h
        zm[t, i] -= h
        fp = np.dot([w_al, w_cs], oracle.cls_losses(zp, L, alpha, want_grad=False)[:2])
        fm = np.dot([w_al, w_cs], oracle.cls_losses(zm, L, alpha, want_grad=False)[:2])
        assert abs((fp - fm) / (2 * h) - dz[t, i]) <= 1e-6 * max(1.0, abs(dz[t, i]))


def test_chunk_length_one_and_hand_worked_chunk():
    z = _z(5)
    _, cs, _ = oracle.cls_losses(z, 1, 4.0)
    assert abs(cs - np.mean(1 / (1 + np.exp(-4.0 * z)))) <= 1e-14
    # one chunk of two tokens, one expert: 1 - (1 - p1)(1 - p2), p = sigmoid(alpha z)
    z2 = np.array([[np.log(3.0)], [-np.log(3.0)]])  # alpha = 1: p1 = 3/4, p2 = 1/4
    al, cs, dz = oracle.cls_losses(z2, 2, 1.0)
    assert abs(cs - (1 - 0.25 * 0.75)) <= 1e-15
    # locality: the single pair's target is token 2's pattern (z < 0 -> 0): BCE(3/4, 0) = log 4
    assert abs(al - np.log(4.0)) <= 1e-15
    # dL_CS/dz1 = p1 (1 - p1) (1 - p2) = 3/16 * 3/4; dL_AL/dz1 = p1 - 0
    assert abs(dz[0, 0] - (0.75 + 3 / 16 * 0.75)) <= 1e-15


def test_sharp_limit_counts_the_union():
    rng = np.random.default_rng(9)
    d, E, L = 32, 20, 4
    layer = make_layer(d, E, 16, "f32", 0.7, rng)
    x = make_tokens(d, 6, L, 0.6, "f32", rng).x
    z, g, m = oracle.route(x, layer.w_router, layer.b_router, None, 1e-6)
    assert np.abs(z).min() > 1e-3  # alpha |z| > 100: every p is within e^-100 of 0 or 1
    _, cs, _ = oracle.cls_losses(z, L, 1e5, want_grad=False)
    st = oracle.stats(m, E, L)
    assert abs(cs - st["union_sum"] / (st["n_chunks"] * E)) <= 1e-12


def test_backward_is_linear_in_the_extra_router_gradient():
    rng = np.random.default_rng(77)
    d, E, de = 24, 6, 8
    layer = make_layer(d, E, de, "f32", 0.4, rng)
    x = make_tokens(d, 4, 3, 0.6, "f32", rng).x
    dy = rng.standard_normal(x.shape).astype(np.float32)
    extra = rng.standard_normal((x.shape[0], E))
    args = (x, layer.w_router, layer.b_router, layer.rms_scale, layer.rms_eps, layer.w_in, layer.w_out, dy)
    base = oracle.backward(*args)
    both = oracle.backward(*args, dz_extra=extra)
    X = x.astype(np.float64)
    Wr = layer.w_router.astype(np.float64)
    np.testing.assert_allclose(both["dz"] - base["dz"], extra, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(both["db"] - base["db"], extra.sum(axis=0), rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(both["dw_router"] - base["dw_router"], extra.T @ X, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(both["dx"] - base["dx"], extra @ Wr, rtol=1e-10, atol=1e-10)
    for k in ("dw_in", "dw_out", "ds", "dg"):
        np.testing.assert_array_equal(both[k], base[k])
