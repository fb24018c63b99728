"""GPU parity of the layer backward (through the C ABI) against the CPU oracle.

The GPU runs blockffn_route (for z) and blockffn_backward on seeded inputs;
the oracle recomputes everything in fp64 from the same inputs.  Bars, per
gradient tensor G, derived from the arithmetic: every product takes bf16
operands, and dy, the hidden gradients, g * Swish(u) and dz are rounded to
bf16 (unit roundoff 2^-9 ~ 2e-3 per rounded operand), with fp32 sums.  So
  ||G_gpu - G||_F <= 1e-2 ||G||_F   and   max |G_gpu - G| <= 1e-2 max |G|,
about five times that roundoff.  (A bar relative to RMS(G), as for the
forward's y, does not fit weight gradients: they are sums over the few pairs
of one expert, with max |G| up to 25 x RMS(G), and bf16 rounding alone then
puts max |err| near 0.1 x RMS.)  Pairs whose oracle pre-activation is
within 1e-3 of zero may legitimately flip between fp32 and fp64; a flipped
pair moves its token's dz and so that token's dx and its expert's router
row, so those tokens (dx) and experts (dW_r, db) are left out and counted.
Expert weight gradients and ds are compared in full: a flipped pair's share
of them scales with its gate, which is within 1e-3 of zero.
"""
import numpy as np
import pytest
import torch

import oracle
from activation_sparse_moe_amd import binding as B
from activation_sparse_moe_amd._capi import BF16
from gpu_parity_util import BAND, check_backward as _check, check_grad as _compare, say
from workload import CONFIGS, make_layer, make_tokens, make_workload

pytestmark = pytest.mark.gpu

# name: (d, E, d_e, T-chunks, L, bias_k, alpha, seed, scale)   scale: None | "pos" | "signed"
CASES = {
    "d512_E64_de128_T96": (512, 64, 128, 12, 8, 0.9, 0.7, 601, "pos"),
    "d256_E80_de256_T70": (256, 80, 256, 14, 5, 0.8, 0.6, 602, None),      # E not /16, two hidden tiles, ragged
    "d384_E8_de128_T40": (384, 8, 128, 5, 8, -0.5, 0.5, 603, "pos"),       # most pairs active, long groups
    "d512_E128_de128_T33": (512, 128, 128, 33, 1, 1.8, 0.0, 604, None),    # rare experts, some never active
    "d256_E16_de128_T48_signed": (256, 16, 128, 6, 8, 0.3, 0.6, 605, "signed"),  # negative RMS scales
}


def _layer_and_tokens(name):
    d, E, de, C, L, k, a, seed, scale = CASES[name]
    rng = np.random.default_rng(seed)
    layer = make_layer(d, E, de, "bf16", k, rng)
    if scale == "pos":
        layer.rms_scale = (0.5 + rng.random(E)).astype(np.float32)
    elif scale == "signed":
        layer.rms_scale = (rng.random(E) * 2.0 - 0.7).astype(np.float32)
    x = make_tokens(d, C, L, a, "bf16", rng).x
    dy = rng.standard_normal((x.shape[0], d)).astype(np.float32)
    return layer, x, dy


def _gpu_backward(layer, x, dy):
    dl = B.DeviceLayer.from_workload(layer)
    xd = B.tokens_to_device(x, BF16)
    _, _, z = B.blockffn_route(dl, xd, 1, want_preact=True)
    out = B.blockffn_backward(dl, xd, z, torch.from_numpy(dy).cuda())
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy().astype(np.float64) for k, v in out.items()}
    res["z"] = z.cpu().numpy()
    return res


@pytest.mark.parametrize("name", sorted(CASES))
def test_backward_matches_oracle(name):
    layer, x, dy = _layer_and_tokens(name)
    say(f"[gpu] backward {name} T={x.shape[0]}")
    gpu = _gpu_backward(layer, x, dy)
    ref = oracle.backward(x, layer.w_router, layer.b_router, layer.rms_scale, layer.rms_eps, layer.w_in,
                          layer.w_out, dy)
    z_ref, _, _ = oracle.route(x, layer.w_router, layer.b_router, layer.rms_scale, layer.rms_eps)
    rel, nt, ne = _check(gpu, ref, gpu["z"], z_ref, gpu["dx"], ref["dx"])
    # experts no token activates get exactly zero weight gradients
    never = ~(z_ref > 0).any(axis=0) & ~(np.abs(z_ref) < BAND).any(axis=0)
    assert np.all(gpu["d_w_in"][never] == 0) and np.all(gpu["d_w_out"][never] == 0)
    say(f"  {name}: " + ", ".join(f"{k} {v:.1e}" for k, v in rel.items()) + f"; band tokens {nt}, experts {ne}")


def test_backward_is_reproducible_and_zero_tokens_is_a_no_op():
    layer, x, dy = _layer_and_tokens("d512_E64_de128_T96")
    a = _gpu_backward(layer, x, dy)
    b = _gpu_backward(layer, x, dy)
    for k in ("dx", "d_w_router", "d_b_router", "d_rms_scale", "d_w_in", "d_w_out"):
        np.testing.assert_array_equal(a[k], b[k])
    dl = B.DeviceLayer.from_workload(layer)
    xd = B.tokens_to_device(x[:0], BF16)
    z = torch.empty((0, layer.w_router.shape[0]), dtype=torch.float32, device="cuda")
    dx = torch.full((1, layer.w_router.shape[1]), 7.0, device="cuda")
    B.blockffn_backward(dl, xd, z, torch.empty((0, layer.w_router.shape[1]), device="cuda"), dx=dx)
    torch.cuda.synchronize()
    assert torch.all(dx == 7.0)


def test_backward_full_size_sampled():
    """The batched workload (4096 tokens, d 4096, 128 experts) in one call, as
    the benchmark runs it; the oracle checks 288 tokens' dx, 32 experts'
    weight gradients (over every token that activates them) and the router
    gradients over all tokens."""
    cfg = CONFIGS["batched_L8_d4096_E128"]
    layer, tok = make_workload(cfg)
    x = tok.x
    T, d = x.shape
    dy = np.random.default_rng(cfg.seed + 100).standard_normal((T, d)).astype(np.float32)
    say(f"[gpu] backward full size {cfg.name} T={T}")
    gpu = _gpu_backward(layer, x, dy)
    tok_idx = np.unique(np.r_[np.linspace(0, T - 1, 256).astype(int), np.arange(1, 17), np.arange(T - 16, T)])
    experts = sorted(set(np.linspace(0, cfg.n_experts - 1, 32).astype(int).tolist()))
    assert len(experts) == 32 and len(tok_idx) >= 256
    tsel = np.zeros(T, bool)
    tsel[tok_idx] = True
    esel = np.zeros(cfg.n_experts, bool)
    esel[experts] = True
    ref = oracle.backward(x, layer.w_router, layer.b_router, layer.rms_scale, layer.rms_eps, layer.w_in,
                          layer.w_out, dy, expert_sel=esel, token_sel=tsel)
    z_ref, _, _ = oracle.route(x, layer.w_router, layer.b_router, layer.rms_scale, layer.rms_eps)
    rel, nt, _ = _check(gpu, ref, gpu["z"][tok_idx], z_ref[tok_idx], gpu["dx"][tok_idx], ref["dx"][tok_idx],
                        experts=experts, router=False)
    # router gradients over all tokens: experts with a band pair are left out
    band_e = (np.abs(z_ref) < BAND).any(axis=0)
    rel["d_w_router"] = _compare("d_w_router", gpu["d_w_router"], ref["dw_router"], ~band_e)
    rel["d_b_router"] = _compare("d_b_router", gpu["d_b_router"], ref["db"], ~band_e)
    assert (~band_e).sum() >= 4
    say(f"  {cfg.name}: " + ", ".join(f"{k} {v:.1e}" for k, v in rel.items()) +
        f"; band tokens {nt} of {len(tok_idx)}, router rows compared {(~band_e).sum()}")


# ---------------------------------------------------------------- CLS-aware objectives
CLS_ALPHA, CLS_W_AL, CLS_W_CS = 8.0, 0.5, 2.0
E_MIN_COMPARED = 32


def _cls_gpu(layer, x, L):
    dl = B.DeviceLayer.from_workload(layer)
    xd = B.tokens_to_device(x, BF16)
    _, _, z = B.blockffn_route(dl, xd, L, want_preact=True)
    losses, dz = B.blockffn_cls_losses(layer.w_router.shape[0], z, L, CLS_ALPHA, CLS_W_AL, CLS_W_CS)
    torch.cuda.synchronize()
    return dl, xd, z, losses.cpu().numpy().astype(np.float64), dz


@pytest.mark.parametrize("name", ["d512_E64_de128_T96", "d256_E80_de256_T70", "d384_E8_de128_T40"])
def test_cls_losses_match_oracle(name):
    """Bars: losses within 1e-4 relative, plus the share of targets the fp32
    and fp64 pre-activations may disagree on (pairs with |z| < 1e-3, each
    moving L_AL by at most alpha |z_t| / ((T-1) E)); dz within 1e-4 x max|dz|
    on tokens whose next token has no such pair."""
    layer, x, _ = _layer_and_tokens(name)
    L = CASES[name][4]
    say(f"[gpu] cls losses {name} T={x.shape[0]} L={L}")
    _, _, z, losses, dz = _cls_gpu(layer, x, L)
    z_ref, _, _ = oracle.route(x, layer.w_router, layer.b_router, layer.rms_scale, layer.rms_eps)
    al, cs, dz_ref = oracle.cls_losses(z_ref, L, CLS_ALPHA, CLS_W_AL, CLS_W_CS)
    T, E = z_ref.shape
    band_next = np.zeros(T, bool)
    band_next[:-1] = (np.abs(z_ref[1:]) < BAND).any(axis=1)
    slack = CLS_ALPHA * np.abs(z_ref[:-1][(np.abs(z_ref[1:]) < BAND)]).sum() / ((T - 1) * E)
    assert abs(losses[0] - al) <= 1e-4 * abs(al) + slack, (losses[0], al, slack)
    assert abs(losses[1] - cs) <= 1e-4 * abs(cs)
    g = dz.cpu().numpy()
    keep = ~band_next
    assert np.abs(g[keep] - dz_ref[keep]).max() <= 1e-4 * np.abs(dz_ref).max()
    say(f"  {name}: L_AL {losses[0]:.6f} (oracle {al:.6f}), L_CS {losses[1]:.6f} (oracle {cs:.6f})")


# E = 80: the router term's contraction runs over expert rows padded to 96 with zeros; T = 70 and 96:
# token tiles of 64 with a ragged tail
@pytest.mark.parametrize("name", ["d512_E64_de128_T96", "d256_E80_de256_T70"])
def test_backward_with_cls_gradient_matches_oracle(name):
    layer, x, dy = _layer_and_tokens(name)
    L = CASES[name][4]
    say(f"[gpu] backward + cls gradient {name}")
    dl, xd, z, _, dz = _cls_gpu(layer, x, L)
    out = B.blockffn_backward(dl, xd, z, torch.from_numpy(dy).cuda(), dz_extra=dz)
    torch.cuda.synchronize()
    gpu = {k: v.cpu().numpy().astype(np.float64) for k, v in out.items()}
    z_ref, _, _ = oracle.route(x, layer.w_router, layer.b_router, layer.rms_scale, layer.rms_eps)
    _, _, dz_ref = oracle.cls_losses(z_ref, L, CLS_ALPHA, CLS_W_AL, CLS_W_CS)
    ref = oracle.backward(x, layer.w_router, layer.b_router, layer.rms_scale, layer.rms_eps, layer.w_in,
                          layer.w_out, dy, dz_extra=dz_ref)
    # a target flip in the next token moves this token's extra gradient: leave those tokens out of dx
    band_rows = (np.abs(z_ref) < BAND).any(axis=1)
    band_rows[:-1] |= band_rows[1:]
    rel = {"dx": _compare("dx", gpu["dx"], ref["dx"], ~band_rows)}
    for k, r in (("d_w_in", "dw_in"), ("d_w_out", "dw_out"), ("d_rms_scale", "ds")):
        rel[k] = _compare(k, gpu[k], ref[r])
    # a band pair (t, i) moves dz[t][i] and the target of dz_extra[t-1][i]: both stay in expert i's router row
    bad_e = (np.abs(z_ref) < BAND).any(axis=0)
    assert (~bad_e).sum() >= E_MIN_COMPARED
    rel["d_w_router"] = _compare("d_w_router", gpu["d_w_router"], ref["dw_router"], ~bad_e)
    rel["d_b_router"] = _compare("d_b_router", gpu["d_b_router"], ref["db"], ~bad_e)
    say("  " + ", ".join(f"{k} {v:.1e}" for k, v in rel.items()) +
        f"; band rows {int(band_rows.sum())}, router rows compared {int((~bad_e).sum())}")
