"""Pins of the oracle's layer backward, against things other than itself.

* central finite differences of the loss sum(y * dy), computed by the
  oracle's forward, on sampled coordinates of every input and parameter;
* reverse-mode autodiff (torch, float64, CPU) of the layer written from its
  definition, compared on whole gradient tensors;
* identities the definition fixes: y is linear in the RMS scale s and in
  W_out, so sum(ds * s) = sum(dW_out * W_out) = loss; with eps = 0 the gates
  are scale-free in (W_r, b), so sum(dW_r * W_r) + sum(db * b) = 0; with one
  expert and eps = 0 the gate is constant, so dz = 0;
* restricting the computed blocks (expert / token selections) changes no
  selected value.
Sources: the BlockFFN write-up (lsdiaocha.cn) §2 core design (ReLU + RMSNorm
router, non-gated Swish experts; the router is differentiable end to end) and
the abstract of arXiv 2507.08771.
"""
import numpy as np
import pytest
import torch

import oracle
from workload import make_layer, make_tokens


def _loss(layer, x0, dy, **over):
    p = dict(x=x0, w_router=layer.w_router, b_router=layer.b_router, rms_scale=layer.rms_scale,
             w_in=layer.w_in, w_out=layer.w_out)
    p.update(over)
    z, g, m = oracle.route(p["x"], p["w_router"], p["b_router"], p["rms_scale"], layer.rms_eps)
    y = oracle.forward_tokens(p["x"], p["w_in"], p["w_out"], g, m)
    return float(np.sum(y * dy.astype(np.float64)))


def _case(seed=0, d=24, E=6, de=8, C=4, L=2, margin=0.05, scale=True):
    """An fp32 layer whose pre-activations all sit at least `margin` from 0
    (finite differences never cross the ReLU kink), with a random scale s and
    at least one active expert per token."""
    for s in range(seed, seed + 200):
        rng = np.random.default_rng(s)
        layer = make_layer(d, E, de, "f32", 0.4, rng)
        if scale:
            layer.rms_scale = (0.5 + rng.random(E)).astype(np.float32)
        x = make_tokens(d, C, L, 0.6, "f32", rng).x
        z, g, m = oracle.route(x, layer.w_router, layer.b_router, layer.rms_scale, layer.rms_eps)
        if np.abs(z).min() > margin and (z > 0).any(axis=1).all() and (z <= 0).any():
            dy = rng.standard_normal(x.shape).astype(np.float32)
            return layer, x, dy
    raise AssertionError("no seed gives a kink-free case")


def _fd(layer, x, dy, name, idx, h_rel=1e-3):
    """Central difference of the loss in one float32 coordinate; the step is
    the exact float32 difference of the two perturbed values."""
    base = {"x": x, "w_router": layer.w_router, "b_router": layer.b_router, "rms_scale": layer.rms_scale,
            "w_in": layer.w_in, "w_out": layer.w_out}[name]
    v = float(base[idx])
    h = h_rel * max(1.0, abs(v))
    plus, minus = base.copy(), base.copy()
    plus[idx] = np.float32(v + h)
    minus[idx] = np.float32(v - h)
    step = float(plus[idx]) - float(minus[idx])
    return (_loss(layer, x, dy, **{name: plus}) - _loss(layer, x, dy, **{name: minus})) / step


GRAD_OF = {"x": "dx", "w_router": "dw_router", "b_router": "db", "rms_scale": "ds", "w_in": "dw_in",
           "w_out": "dw_out"}


@pytest.mark.parametrize("name", sorted(GRAD_OF))
def test_backward_matches_finite_differences(name):
    layer, x, dy = _case(seed=11)
    gr = oracle.backward(x, layer.w_router, layer.b_router, layer.rms_scale, layer.rms_eps, layer.w_in,
                         layer.w_out, dy)[GRAD_OF[name]]
    rng = np.random.default_rng(5)
    shape = gr.shape
    scale = np.abs(gr).max()
    assert scale > 0
    for _ in range(8):
        idx = tuple(int(rng.integers(n)) for n in shape)
        if name in ("w_in", "w_out"):
            # sample inside an expert some token activates, so the gradient is not trivially 0
            z, g, m = oracle.route(x, layer.w_router, layer.b_router, layer.rms_scale, layer.rms_eps)
            on = np.nonzero((z > 0).any(axis=0))[0]
            idx = (int(on[rng.integers(len(on))]),) + idx[1:]
        fd = _fd(layer, x, dy, name, idx)
        assert abs(fd - gr[idx]) <= 2e-4 * scale + 1e-4 * abs(fd), (name, idx, fd, gr[idx])


def _torch_reference(layer, x, dy, eps):
    """The layer written from its definition in float64 torch, all experts
    dense (inactive pairs have gate 0); autodiff gives every gradient."""
    f = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)  # noqa: E731
    tx, wr, b, s, wi, wo = (f(x), f(layer.w_router), f(layer.b_router), f(layer.rms_scale), f(layer.w_in),
                            f(layer.w_out))
    z = tx @ wr.T + b
    a = torch.relu(z)
    g = s * a / torch.sqrt((a * a).mean(dim=1, keepdim=True) + eps)
    u = torch.einsum("td,ejd->tej", tx, wi)
    h = u * torch.sigmoid(u)
    e = torch.einsum("tej,edj->ted", h, wo)
    y = (g[:, :, None] * e).sum(dim=1)
    (y * torch.tensor(dy, dtype=torch.float64)).sum().backward()
    return dict(dx=tx.grad, dw_router=wr.grad, db=b.grad, ds=s.grad, dw_in=wi.grad, dw_out=wo.grad)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_matches_autodiff(dtype):
    rng = np.random.default_rng(21)
    d, E, de = 32, 10, 12
    layer = make_layer(d, E, de, dtype, 0.5, rng)
    layer.rms_scale = (0.5 + rng.random(E)).astype(np.float32)
    x = make_tokens(d, 5, 3, 0.6, dtype, rng).x
    dy = rng.standard_normal((x.shape[0], d)).astype(np.float32)
    o = oracle.backward(x, layer.w_router, layer.b_router, layer.rms_scale, layer.rms_eps, layer.w_in,
                        layer.w_out, dy)

    def widen(a):
        a = np.asarray(a)
        return (a.astype(np.uint32) << 16).view(np.float32) if a.dtype == np.uint16 else a

    wl = type("L", (), {})()
    wl.w_router, wl.b_router, wl.rms_scale = widen(layer.w_router), layer.b_router, layer.rms_scale
    wl.w_in, wl.w_out = widen(layer.w_in), widen(layer.w_out)
    ref = _torch_reference(wl, widen(x), dy, layer.rms_eps)
    for k, v in ref.items():
        r = v.detach().numpy()
        assert np.abs(o[k] - r).max() <= 1e-9 * max(1.0, np.abs(r).max()), k


def test_linear_parameter_identities():
    layer, x, dy = _case(seed=31)
    loss = _loss(layer, x, dy)
    o = oracle.backward(x, layer.w_router, layer.b_router, layer.rms_scale, layer.rms_eps, layer.w_in,
                        layer.w_out, dy)
    # y is linear in s and in W_out (degree-1 homogeneous): Euler's identity
    assert np.isclose(np.sum(o["ds"] * layer.rms_scale), loss, rtol=1e-10, atol=1e-12)
    assert np.isclose(np.sum(o["dw_out"] * layer.w_out), loss, rtol=1e-10, atol=1e-12)


def test_router_scale_invariance():
    # eps = 0: g depends on z only through z / |relu(z)|, so scaling (W_r, b)
    # leaves the loss unchanged and its directional derivative vanishes
    layer, x, dy = _case(seed=41)
    layer.rms_eps = 0.0
    o = oracle.backward(x, layer.w_router, layer.b_router, layer.rms_scale, 0.0, layer.w_in, layer.w_out, dy)
    euler = np.sum(o["dw_router"] * layer.w_router) + np.sum(o["db"] * layer.b_router)
    size = np.abs(o["dw_router"] * layer.w_router).sum() + np.abs(o["db"] * layer.b_router).sum()
    assert size > 1e-3
    assert abs(euler) <= 1e-10 * size


def test_single_expert_gate_is_constant():
    # E = 1, eps = 0: g = s * a / |a| = s whenever the expert fires, so the
    # router receives no gradient at all
    rng = np.random.default_rng(51)
    layer = make_layer(16, 1, 8, "f32", -1.0, rng)
    x = make_tokens(16, 4, 2, 0.5, "f32", rng).x
    dy = rng.standard_normal(x.shape).astype(np.float32)
    z, _, _ = oracle.route(x, layer.w_router, layer.b_router, None, 0.0)
    assert (z > 0).sum() >= 4
    o = oracle.backward(x, layer.w_router, layer.b_router, None, 0.0, layer.w_in, layer.w_out, dy)
    assert np.abs(o["dz"]).max() <= 1e-12 * max(1.0, np.abs(o["dg"]).max())
    assert np.abs(o["dw_router"]).max() <= 1e-10 and np.abs(o["db"]).max() <= 1e-10
    assert np.abs(o["dw_in"]).max() > 0 and np.abs(o["dx"]).max() > 0


def test_inactive_pairs_get_nothing():
    layer, x, dy = _case(seed=61)
    o = oracle.backward(x, layer.w_router, layer.b_router, layer.rms_scale, layer.rms_eps, layer.w_in,
                        layer.w_out, dy)
    z, g, m = oracle.route(x, layer.w_router, layer.b_router, layer.rms_scale, layer.rms_eps)
    off = z <= 0
    assert np.all(o["dz"][off] == 0) and np.all(o["dg"][off] == 0)
    never = ~(z > 0).any(axis=0)
    assert np.all(o["dw_in"][never] == 0) and np.all(o["dw_out"][never] == 0)


def test_selection_leaves_selected_values_unchanged():
    layer, x, dy = _case(seed=71)
    args = (x, layer.w_router, layer.b_router, layer.rms_scale, layer.rms_eps, layer.w_in, layer.w_out, dy)
    full = oracle.backward(*args)
    es = np.zeros(layer.w_in.shape[0], bool)
    es[1::2] = True
    ts = np.zeros(x.shape[0], bool)
    ts[::3] = True
    part = oracle.backward(*args, expert_sel=es, token_sel=ts)
    for k in ("dw_router", "db", "ds", "dz", "dg"):
        np.testing.assert_array_equal(part[k], full[k])
    np.testing.assert_array_equal(part["dw_in"][es], full["dw_in"][es])
    np.testing.assert_array_equal(part["dw_out"][es], full["dw_out"][es])
    assert np.all(part["dw_in"][~es] == 0)
    np.testing.assert_array_equal(part["dx"][ts], full["dx"][ts])
    assert np.all(part["dx"][~ts] == 0)
