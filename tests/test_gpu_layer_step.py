"""GPU parity of blockffn_layer_forward, the one-call layer step (router,
chunk union, expert forward and statistics).

Short calls (at most 64 tokens and 16 chunks, bf16, E a multiple of 16)
run the three-kernel step; the rest run the separate calls.  Every output is
compared with the oracle element by element (bars in gpu_parity_util), and
with the separate calls where those are bit-for-bit comparable.  The step
must also be reproducible bit for bit, across calls and under graph replay.
"""
import numpy as np
import pytest
import torch

import oracle
from activation_sparse_moe_amd import binding as B
from activation_sparse_moe_amd._capi import BF16
from gpu_parity_util import check_route, check_union, check_y, oracle_full, say
from workload import make_layer, make_tokens

pytestmark = pytest.mark.gpu

# name: (d, E, d_e, dtype, L, chunks, bias_k, alpha, seed)
CASES = {
    "d2048_E64_L8_one_chunk": (2048, 64, 128, "bf16", 8, 1, 0.887, 0.8, 901),    # the verify step
    "d2048_E64_L1_16_tokens": (2048, 64, 128, "bf16", 1, 16, 0.887, 0.0, 902),   # 16 decode tokens
    "d512_E80_de256_L8_x8": (512, 80, 256, "bf16", 8, 8, 0.9, 0.8, 903),         # two mask words, 64 tokens
    "d1024_E128_L32_x2": (1024, 128, 128, "bf16", 32, 2, 1.0, 0.65, 904),        # two token tiles, E = 128
    "d640_E48_L17_x3": (640, 48, 128, "bf16", 17, 3, 0.9, 0.7, 905),             # padded tile (d/128 = 5)
    "d256_E16_de128_L5_x3": (256, 16, 128, "bf16", 5, 3, 0.5, 0.6, 906),         # few experts
    "d4096_E128_L32_x2": (4096, 128, 128, "bf16", 32, 2, 1.0364, 0.647, 910),     # the largest d, 64 tokens
    "d4096_E128_de256_L8_x1": (4096, 128, 256, "bf16", 8, 1, 1.0364, 0.647, 911), # d_e 256
    # the separate-call regime: too many tokens; fp32; E not a multiple of 16
    "d512_E64_L8_x12_separate": (512, 64, 128, "bf16", 8, 12, 0.9, 0.8, 907),
    "f32_d128_E24_de32_L8_separate": (128, 24, 32, "f32", 8, 4, 0.8, 0.7, 908),
    "d512_E70_L8_separate": (512, 70, 128, "bf16", 8, 2, 0.9, 0.8, 909),
}


def _case(name):
    d, E, de, dt, L, C, k, a, seed = CASES[name]
    rng = np.random.default_rng(seed)
    layer = make_layer(d, E, de, dt, k, rng)
    tok = make_tokens(d, C, L, a, dt, rng)
    return layer, tok.x, L


def _numpy(out):
    o = {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items() if k != "workspace"}
    return dict(g=o["gates"], mask=B.masks_to_u64(out["token_masks"]), umask=B.masks_to_u64(out["chunk_masks"]),
                count=o["active_count"], list=o["active_list"], y=o["y"], z=o["preact"],
                stats=B.stats_dict(out["stats"]))


def _compare(layer, x, L, gpu, name):
    E, dt = layer.n_experts, layer.dtype
    z, g, m, um, cnt, lst = oracle_full(layer, x, L)
    flipped, keep = check_route(gpu, z, g, m, E, dt, layer=layer)
    nflip_u = check_union(gpu, um, z, E, L)
    y_ref = oracle.forward_tokens(x, layer.w_in, layer.w_out, g, m)
    rel = check_y(gpu["y"], y_ref, keep, dt, name)
    # statistics: exact on the GPU's own masks, and on the oracle's when no pattern bit flipped
    st_own = oracle.stats(gpu["mask"], E, L)
    st_ref = oracle.stats(m, E, L) if not flipped else st_own
    for st in (st_own, st_ref):
        for key in ("active_pairs", "union_sum", "reuse_num", "reuse_den"):
            assert gpu["stats"][key] == st[key], key
        np.testing.assert_array_equal(gpu["stats"]["hist"], st["hist"])
    T = x.shape[0]
    assert (gpu["stats"]["n_tokens"], gpu["stats"]["n_chunks"], gpu["stats"]["n_experts"],
            gpu["stats"]["chunk_len"]) == (T, T // L, E, L)
    say(f"  {name}: max|dy|/rms {rel:.2e}, band flips {len(flipped)} tokens / {nflip_u} union bits")


@pytest.mark.parametrize("name", sorted(CASES))
def test_layer_step_matches_oracle(name):
    layer, x, L = _case(name)
    say(f"[gpu] layer step {name} T={x.shape[0]}")
    dl = B.DeviceLayer.from_workload(layer)
    xd = B.tokens_to_device(x, dl.dtype)
    out = B.blockffn_layer_forward(dl, xd, L, want_preact=True)
    torch.cuda.synchronize()
    _compare(layer, x, L, _numpy(out), name)


@pytest.mark.parametrize("name", ["d2048_E64_L8_one_chunk", "d512_E80_de256_L8_x8", "d640_E48_L17_x3"])
def test_layer_step_agrees_with_separate_calls(name):
    """Masks and unions as the separate calls' outside the rounding band of z; with equal masks, outputs
    within the output bar of each other; statistics exact on each side's own masks."""
    layer, x, L = _case(name)
    say(f"[gpu] layer step vs separate calls {name}")
    dl = B.DeviceLayer.from_workload(layer)
    xd = B.tokens_to_device(x, dl.dtype)
    step = _numpy(B.blockffn_layer_forward(dl, xd, L, want_preact=True))
    g, m, z = B.blockffn_route(dl, xd, L, want_preact=True)
    um, cnt, lst = B.blockffn_chunk_union(layer.n_experts, m, L)
    y = B.blockffn_forward(dl, xd, L, g, cnt, lst, mode="chunk_split")
    torch.cuda.synchronize()
    z_sep = z.cpu().numpy()
    assert np.abs(step["z"].astype(np.float64) - z_sep).max() <= 1e-4 * max(1.0, np.sqrt((z_sep ** 2).mean()))
    m_sep = B.masks_to_u64(m)
    same = (m_sep == step["mask"]).all(axis=1)
    near = (np.abs(z_sep) < 1e-3).any(axis=1)
    assert (same | near).all(), "masks differ away from the band"
    if same.all():
        np.testing.assert_array_equal(step["umask"], B.masks_to_u64(um))
        np.testing.assert_array_equal(step["count"], cnt.cpu().numpy())
        np.testing.assert_array_equal(step["list"], lst.cpu().numpy())
    check_y(step["y"], y.cpu().numpy().astype(np.float64), same, "bf16", name)


@pytest.mark.parametrize("name", ["d2048_E64_L8_one_chunk", "d2048_E64_L1_16_tokens", "d1024_E128_L32_x2"])
def test_layer_step_is_reproducible(name):
    layer, x, L = _case(name)
    say(f"[gpu] layer step reproducibility {name}")
    dl = B.DeviceLayer.from_workload(layer)
    xd = B.tokens_to_device(x, dl.dtype)
    out = B.alloc_layer_forward(dl, x.shape[0], L, want_preact=True)
    first = None
    for rep in range(4):
        for k, v in out.items():
            if v is not None and k != "workspace":
                v.fill_(7 if v.dtype != torch.float32 else 3.0)
        out["workspace"].fill_(0xA5)   # stale scratch must not matter
        B.blockffn_layer_forward(dl, xd, L, out=out)
        torch.cuda.synchronize()
        got = {k: v.cpu().clone() for k, v in out.items() if v is not None and k != "workspace"}
        if first is None:
            first = got
            continue
        for k in first:
            assert torch.equal(got[k], first[k]), f"call {rep}: {k} differs"


def test_layer_step_distinct_layers_per_chunk():
    """layers[c % n_layers] for chunk c, each layer in its own allocations."""
    d, E, de, L, C = 1024, 64, 128, 8, 6
    rng = np.random.default_rng(910)
    layers = [make_layer(d, E, de, "bf16", 0.9, rng) for _ in range(2)]
    x = make_tokens(d, C, L, 0.8, "bf16", rng).x
    say("[gpu] layer step, two layers in separate allocations")
    dls = [B.DeviceLayer.from_workload(ly) for ly in layers]
    xd = B.tokens_to_device(x, BF16)
    gpu = _numpy(B.blockffn_layer_forward(dls, xd, L, want_preact=True))
    for li, ly in enumerate(layers):
        chunks = [c for c in range(C) if c % 2 == li]
        tok = np.concatenate([np.arange(c * L, (c + 1) * L) for c in chunks])
        sub = dict(g=gpu["g"][tok], mask=gpu["mask"][tok], umask=gpu["umask"][chunks], count=gpu["count"][chunks],
                   list=gpu["list"][chunks], y=gpu["y"][tok], z=gpu["z"][tok])
        z, g, m, um, cnt, lst = oracle_full(ly, x[tok], L)
        flipped, keep = check_route(sub, z, g, m, E, "bf16", layer=ly)
        check_union(sub, um, z, E, L)
        check_y(sub["y"], oracle.forward_tokens(x[tok], ly.w_in, ly.w_out, g, m), keep, "bf16", f"layer {li}")
    st = oracle.stats(gpu["mask"], E, L)
    assert gpu["stats"]["union_sum"] == st["union_sum"]


def test_layer_step_no_expert_and_every_expert():
    """A bias far below zero activates nothing (y = 0, empty unions); far above, every expert."""
    d, E, de, L, C = 512, 64, 128, 8, 2
    rng = np.random.default_rng(911)
    x = make_tokens(d, C, L, 0.8, "bf16", rng).x
    for label, shift in (("none", -1e4), ("all", 1e4)):
        layer = make_layer(d, E, de, "bf16", 0.9, np.random.default_rng(912))
        layer.b_router = (layer.b_router + shift).astype(np.float32)
        say(f"[gpu] layer step, {label} active")
        dl = B.DeviceLayer.from_workload(layer)
        xd = B.tokens_to_device(x, BF16)
        gpu = _numpy(B.blockffn_layer_forward(dl, xd, L, want_preact=True))
        if label == "none":
            assert (gpu["count"] == 0).all() and (gpu["list"] == -1).all()
            assert (gpu["y"] == 0).all() and (gpu["g"] == 0).all()
            assert gpu["stats"]["active_pairs"] == 0 and gpu["stats"]["hist"][0] == C * L
        else:
            assert (gpu["count"] == E).all()
            assert gpu["stats"]["hist"][E] == C * L
        _compare(layer, x, L, gpu, f"{label} active")


def test_layer_step_graph_replays_match_eager():
    d, E, de, L, C = 2048, 64, 128, 8, 1
    rng = np.random.default_rng(913)
    layer = make_layer(d, E, de, "bf16", 0.887, rng)
    x = make_tokens(d, C, L, 0.8, "bf16", rng).x
    say("[gpu] layer step graph replay")
    dl = B.DeviceLayer.from_workload(layer)
    xd = B.tokens_to_device(x, BF16)
    out = B.alloc_layer_forward(dl, C * L, L, want_preact=True)
    B.blockffn_layer_forward(dl, xd, L, out=out)
    torch.cuda.synchronize()
    eager = {k: v.cpu().clone() for k, v in out.items() if v is not None and k != "workspace"}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.blockffn_layer_forward(dl, xd, L, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(3):  # three steps in one graph: the counters must be cleared by every step
            B.blockffn_layer_forward(dl, xd, L, out=out)
    for rep in range(3):
        for k, v in out.items():
            if v is not None and k != "workspace":
                v.fill_(0)
        noise = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in eager:
            assert torch.equal(out[k].cpu(), eager[k]), f"replay {rep}: {k} differs from the eager run"
        del noise
