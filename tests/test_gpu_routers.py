"""GPU parity of the baseline routers (blockffn_route_with) against the oracle,
and the rest of the path (union, forward) run on their gates.

Bars: pre-activations as for the BlockFFN router; masks bit-exact except
tokens whose decision sits within 1e-3 of its threshold in the oracle's fp64
z (for top-k: the gap between the k-th and (k+1)-th largest z; for the
ReLU-sum router: some |z_i| < 1e-3), which are counted and left out; gates
within 1e-4 (bf16) / 1e-5 (fp32) x RMS of the oracle's; y within 2e-2 (bf16)
/ 1e-5 (fp32) x RMS.
"""
import numpy as np
import pytest
import torch

import oracle
from activation_sparse_moe_amd import binding as B
from activation_sparse_moe_amd._capi import BF16, F32
from gpu_parity_util import BAND, GATE_TOL, Y_TOL, bits, say
from workload import make_layer, make_tokens

pytestmark = pytest.mark.gpu

# name: (d, E, d_e, dtype, L, chunks, bias_k, alpha, seed)
SHAPES = {
    "bf16_d512_E64_L8": (512, 64, 128, "bf16", 8, 10, 0.9, 0.8, 701),    # MFMA router
    "bf16_d640_E70_L3": (640, 70, 128, "bf16", 3, 11, 0.9, 0.6, 702),    # VALU router, two mask words
    "f32_d128_E24_L4": (128, 24, 32, "f32", 4, 6, 0.5, 0.7, 703),        # fp32
}
ROUTERS = [("topk_softmax", 1), ("topk_softmax", 2), ("topk_softmax", 8), ("relu_sum", 0)]


def _band_tokens(z, kind, k):
    if kind == "relu_sum":
        return (np.abs(z) < BAND).any(axis=1)
    zs = -np.sort(-z, axis=1)
    return (zs[:, k - 1] - zs[:, k]) < BAND if k < z.shape[1] else np.zeros(z.shape[0], bool)


@pytest.mark.parametrize("router,k", ROUTERS, ids=[f"{r}{k}" for r, k in ROUTERS])
@pytest.mark.parametrize("shape", sorted(SHAPES))
def test_router_matches_oracle(shape, router, k):
    d, E, de, dt, L, C, bias_k, a, seed = SHAPES[shape]
    rng = np.random.default_rng(seed)
    layer = make_layer(d, E, de, dt, bias_k, rng)
    x = make_tokens(d, C, L, a, dt, rng).x
    say(f"[gpu] router {router}{k} {shape} T={x.shape[0]}")
    dl = B.DeviceLayer.from_workload(layer)
    xd = B.tokens_to_device(x, F32 if dt == "f32" else BF16)
    g, m, z = B.blockffn_route_with(dl, xd, L, router=router, top_k=k, want_preact=True)
    um, cnt, lst = B.blockffn_chunk_union(E, m, L)
    y = B.blockffn_forward(dl, xd, L, g, cnt, lst)
    torch.cuda.synchronize()
    kind = oracle.ROUTER_TOPK_SOFTMAX if router == "topk_softmax" else oracle.ROUTER_RELU_SUM
    z_ref, g_ref, m_ref = oracle.route_with(x, layer.w_router, layer.b_router, kind, k)
    gz, gg, gm = z.cpu().numpy(), g.cpu().numpy(), B.masks_to_u64(m)
    scale = np.sqrt((z_ref ** 2).mean())
    assert np.abs(gz - z_ref).max() <= (1e-5 if dt == "f32" else 1e-4) * scale
    band = _band_tokens(z_ref, router, k)
    ob, gb = bits(m_ref, E), bits(gm, E)
    diff = (ob != gb).any(axis=1)
    assert not (diff & ~band).any(), f"mask mismatch outside the band at tokens {np.nonzero(diff & ~band)[0][:8]}"
    keep = ~band
    if router == "topk_softmax":
        assert np.all(gb.sum(axis=1) == k)
    rms = np.sqrt((g_ref[keep] ** 2).mean())
    assert np.abs(gg[keep] - g_ref[keep]).max() <= GATE_TOL[dt] * rms
    y_ref = oracle.forward_tokens(x, layer.w_in, layer.w_out, g_ref, m_ref)
    yr = y.cpu().numpy()
    yrms = np.sqrt((y_ref[keep] ** 2).mean())
    err = np.abs(yr[keep] - y_ref[keep]).max()
    assert err <= Y_TOL[dt] * yrms, f"y error {err:.3e} > {Y_TOL[dt]} x RMS {yrms:.3e}"
    say(f"  {router}{k} {shape}: max|dy|/rms {err / yrms:.2e}, band tokens {int(band.sum())}")
