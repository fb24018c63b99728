"""GPU parity on seeded, drawn shapes: every forward mode a shape allows, the
one-call layer step and (for matrix-core shapes) the backward, each against
the CPU oracle with the bars of gpu_parity_util.

The fixed cases elsewhere pick shapes for the tiles and tails they exercise;
these draw d, E, d_e, chunk length, chunk count, dtype, bias and token
correlation from the whole supported range (1 <= E <= 128, d a multiple of 64,
d_e a multiple of 16, chunks of 1..32 tokens), so that combinations nobody
chose are covered too, and do the same for the baseline routers (top-k
softmax with k drawn from 1..E, and the ReLU-sum router) and the CLS-aware
objectives.  Each draw is a pure function of its seed.
"""
import numpy as np
import pytest
import torch

import oracle
from activation_sparse_moe_amd import binding as B
from activation_sparse_moe_amd._capi import BF16
from gpu_parity_util import (check_backward, check_baseline_router, check_route, check_union, check_y,
                              conditioned_tols, oracle_full, run_gpu, say)
from workload import make_layer, make_tokens
from workload.gen import bf16_bits_to_f32, bf16_round_bits

pytestmark = pytest.mark.gpu

FORWARD_SEEDS = range(40)
ROUTER_SEEDS = range(16)
BACKWARD_SEEDS = range(10)


def _draw_forward(seed: int):
    r = np.random.default_rng(7000 + seed)
    dt = "f32" if r.random() < 0.2 else "bf16"
    if dt == "bf16" and r.random() < 0.7:  # matrix-core shapes
        d = 128 * int(r.integers(1, 9))
        de = int(r.choice([128, 256]))
    else:
        d = 64 * int(r.integers(1, 17))
        de = 16 * int(r.integers(1, 17))
    E = int(r.choice([1, 2, 7, 16, 24, 33, 48, 64, 65, 80, 100, 127, 128]))
    L = int(r.choice([1, 2, 3, 5, 8, 9, 13, 16, 17, 24, 31, 32]))
    C = int(r.integers(1, 25))
    return d, E, de, dt, L, C, float(r.uniform(-0.3, 1.6)), float(r.uniform(0.0, 0.9))


def _draw_backward(seed: int):
    r = np.random.default_rng(8000 + seed)
    d = 128 * int(r.integers(1, 9))
    de = int(r.choice([128, 256]))
    E = int(r.choice([1, 3, 8, 17, 40, 64, 96, 128]))
    T = int(r.integers(1, 200))
    return d, E, de, T, float(r.uniform(-0.3, 1.6)), float(r.uniform(0.0, 0.9)), int(r.integers(0, 3))


def _checks(layer, x, L, gpu, z, g, m, um, y_ref, st, what):
    E, dt = layer.n_experts, layer.dtype
    flipped, keep = check_route(gpu, z, g, m, E, dt, layer=layer)
    check_union(gpu, um, z, E, L)
    check_y(gpu["y"], y_ref, keep, dt, what)
    if gpu.get("stats") is not None and not flipped:
        for key in ("active_pairs", "union_sum", "reuse_num", "reuse_den"):
            assert gpu["stats"][key] == st[key], f"{what}: {key}"
        np.testing.assert_array_equal(gpu["stats"]["hist"], st["hist"])


@pytest.mark.parametrize("seed", FORWARD_SEEDS)
def test_forward_on_drawn_shapes(seed):
    d, E, de, dt, L, C, k, a = _draw_forward(seed)
    say(f"[gpu] drawn forward {seed}: d={d} E={E} d_e={de} {dt} L={L} chunks={C}")
    rng = np.random.default_rng(9000 + seed)
    layer = make_layer(d, E, de, dt, k, rng)
    x = make_tokens(d, C, L, a, dt, rng).x
    dl = B.DeviceLayer.from_workload(layer)
    xd = B.tokens_to_device(x, dl.dtype)
    z, g, m, um, _, _ = oracle_full(layer, x, L)
    y_ref = oracle.forward_tokens(x, layer.w_in, layer.w_out, g, m)
    st = oracle.stats(m, E, L)
    modes = ["auto", "gemv", "dense"]
    if dt == "bf16" and d % 128 == 0 and de % 128 == 0:
        modes += ["chunk_mfma", "chunk_split"]
    if dt == "bf16" and d % 128 == 0 and de in (128, 256):
        modes.append("grouped")
    for mode in modes:
        say(f"  mode {mode}")
        gpu = run_gpu(dl, xd, L, mode=mode)
        _checks(layer, x, L, gpu, z, g, m, um, y_ref, st, f"seed {seed}/{mode}")
    say("  one-call layer step")
    out = B.blockffn_layer_forward(dl, xd, L, want_preact=True)
    torch.cuda.synchronize()
    gpu = dict(g=out["gates"].cpu().numpy(), mask=B.masks_to_u64(out["token_masks"]),
               umask=B.masks_to_u64(out["chunk_masks"]), count=out["active_count"].cpu().numpy(),
               list=out["active_list"].cpu().numpy(), y=out["y"].cpu().numpy(), z=out["preact"].cpu().numpy(),
               stats=B.stats_dict(out["stats"]))
    _checks(layer, x, L, gpu, z, g, m, um, y_ref, st, f"seed {seed}/layer step")


@pytest.mark.parametrize("seed", ROUTER_SEEDS)
def test_baseline_routers_on_drawn_shapes(seed):
    d, E, de, dt, L, C, k, a = _draw_forward(100 + seed)
    r = np.random.default_rng(7500 + seed)
    router = "relu_sum" if seed % 3 == 2 else "topk_softmax"
    top_k = int(r.integers(1, E + 1)) if router == "topk_softmax" else 0
    say(f"[gpu] drawn router {seed}: {router}{top_k} d={d} E={E} d_e={de} {dt} L={L} chunks={C}")
    rng = np.random.default_rng(9200 + seed)
    layer = make_layer(d, E, de, dt, k, rng)
    x = make_tokens(d, C, L, a, dt, rng).x
    check_baseline_router(layer, x, L, router, top_k, f"seed {seed}")


@pytest.mark.parametrize("seed", BACKWARD_SEEDS)
def test_backward_on_drawn_shapes(seed):
    d, E, de, T, k, a, scale = _draw_backward(seed)
    say(f"[gpu] drawn backward {seed}: d={d} E={E} d_e={de} T={T} scale={scale}")
    rng = np.random.default_rng(9500 + seed)
    layer = make_layer(d, E, de, "bf16", k, rng)
    if scale == 1:
        layer.rms_scale = (0.5 + rng.random(E)).astype(np.float32)
    elif scale == 2:
        layer.rms_scale = (rng.random(E) * 2.0 - 0.7).astype(np.float32)
    x = make_tokens(d, T, 1, a, "bf16", rng).x
    dy = rng.standard_normal((T, d)).astype(np.float32)
    dl = B.DeviceLayer.from_workload(layer)
    xd = B.tokens_to_device(x, BF16)
    _, _, zd = B.blockffn_route(dl, xd, 1, want_preact=True)
    out = B.blockffn_backward(dl, xd, zd, torch.from_numpy(dy).cuda())
    torch.cuda.synchronize()
    gpu = {key: v.cpu().numpy().astype(np.float64) for key, v in out.items()}
    gz = zd.cpu().numpy()
    args = (x, layer.w_router, layer.b_router, layer.rms_scale, layer.rms_eps, layer.w_in, layer.w_out)
    ref = oracle.backward(*args, dy)
    # drawn shapes include ill-conditioned ones (few tokens, one active expert of three): the bars
    # follow how far the oracle's own gradients move when dy is rounded as the kernels round it
    tols = conditioned_tols(ref, oracle.backward(*args, bf16_bits_to_f32(bf16_round_bits(dy))))
    z_ref, _, _ = oracle.route(x, layer.w_router, layer.b_router, layer.rms_scale, layer.rms_eps)
    rel, nt, ne = check_backward(gpu, ref, gz, z_ref, gpu["dx"], ref["dx"], tols=tols)
    say("  " + ", ".join(f"{key} {v:.1e} (bar {tols[key][0]:.1e})" for key, v in rel.items())
        + f"; band tokens {nt}, experts {ne}")


@pytest.mark.parametrize("seed", range(12))
def test_cls_losses_on_drawn_inputs(seed):
    """The CLS-aware objectives on drawn pre-activations (E, chunk length, chunks, scale, shift,
    alpha, weights).  Both sides take the same fp32 z, so every target [z > 0] agrees: the losses
    must match within 1e-4 relative and dz within 1e-4 x max |dz| (fp32 against fp64 arithmetic)."""
    r = np.random.default_rng(7700 + seed)
    E = int(r.choice([1, 2, 7, 16, 33, 64, 100, 128]))
    L = int(r.choice([1, 2, 5, 8, 16, 17, 32]))
    C = int(r.integers(1, 41))
    alpha = float(r.uniform(1.0, 16.0))
    w_al, w_cs = float(r.uniform(0.0, 2.0)), float(r.uniform(0.0, 2.0))
    z = (r.standard_normal((C * L, E)) * r.uniform(0.1, 3.0) + r.uniform(-2.0, 1.0)).astype(np.float32)
    say(f"[gpu] drawn cls losses {seed}: E={E} L={L} chunks={C} alpha={alpha:.2f} w=({w_al:.2f}, {w_cs:.2f})")
    losses, dz = B.blockffn_cls_losses(E, torch.from_numpy(z).cuda(), L, alpha, w_al, w_cs)
    torch.cuda.synchronize()
    al, cs, dz_ref = oracle.cls_losses(z, L, alpha, w_al, w_cs)
    got = losses.cpu().numpy()
    assert abs(got[0] - al) <= 1e-4 * abs(al) + 1e-7, (got[0], al)
    assert abs(got[1] - cs) <= 1e-4 * abs(cs) + 1e-7, (got[1], cs)
    top = np.abs(dz_ref).max()
    assert np.abs(dz.cpu().numpy() - dz_ref).max() <= 1e-4 * top + 1e-12
