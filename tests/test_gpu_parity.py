"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every case draws its inputs from the seeded generator, runs router -> chunk
union -> expert forward -> stats on the GPU, runs the oracle on the same
inputs, and compares element by element (bars in gpu_parity_util).  Shapes
span several tiles and ragged tails: E not a multiple of 64 (and of 16),
an odd number of 128-element steps, chunk lengths that pad a 16-token tile,
single tokens, fp32 and bf16.
"""
import numpy as np
import pytest
import torch

import oracle
from activation_sparse_moe_amd import binding as B
from activation_sparse_moe_amd._capi import BF16, F32
from gpu_parity_util import (bits, check_route, check_union, check_y, oracle_full, run_gpu, say)
from workload import CONFIGS, make_layer, make_tokens, make_workload

pytestmark = pytest.mark.gpu

# name: (d, E, d_e, dtype, L, chunks, bias_k, alpha, seed)
CASES = {
    "bf16_d512_E80_de256_L8": (512, 80, 256, "bf16", 8, 12, 0.9, 0.8, 101),     # MFMA router, 2 mask words
    "bf16_d640_E70_de128_L8": (640, 70, 128, "bf16", 8, 10, 0.9, 0.8, 102),     # VALU router, 5 MFMA steps
    "bf16_d512_E64_de128_L32": (512, 64, 128, "bf16", 32, 4, 1.0, 0.65, 103),   # two token tiles
    "bf16_d512_E48_de128_L17": (512, 48, 128, "bf16", 17, 3, 0.9, 0.7, 104),    # second tile padded
    "bf16_d1024_E64_de128_L1": (1024, 64, 128, "bf16", 1, 40, 0.887, 0.0, 105), # single-token GEMV
    "bf16_d256_E128_de64_L3": (256, 128, 64, "bf16", 3, 9, 1.0, 0.6, 106),      # short chunk GEMV, E = 128
    "f32_d128_E24_de32_L8": (128, 24, 32, "f32", 8, 6, 0.8, 0.7, 107),          # fp32 chunk -> GEMV
}


def _case(name):
    d, E, de, dt, L, C, k, a, seed = CASES[name]
    rng = np.random.default_rng(seed)
    layer = make_layer(d, E, de, dt, k, rng)
    tok = make_tokens(d, C, L, a, dt, rng)
    return layer, tok.x, L


def _compare_all(layer, x, L, gpu, name, check_stats=True):
    E, dt = layer.n_experts, layer.dtype
    z, g, m, um, cnt, lst = oracle_full(layer, x, L)
    flipped, keep = check_route(gpu, z, g, m, E, dt, layer=layer)
    nflip_u = check_union(gpu, um, z, E, L)
    y_ref = oracle.forward_tokens(x, layer.w_in, layer.w_out, g, m)
    rel = check_y(gpu["y"], y_ref, keep, dt, name)
    if check_stats and not flipped:
        st = oracle.stats(m, E, L)
        for key in ("active_pairs", "union_sum", "reuse_num", "reuse_den"):
            assert gpu["stats"][key] == st[key], key
        np.testing.assert_array_equal(gpu["stats"]["hist"], st["hist"])
    say(f"  {name}: max|dy|/rms {rel:.2e}, band flips {len(flipped)} tokens / {nflip_u} union bits")
    return y_ref, keep


@pytest.mark.parametrize("name", sorted(CASES))
def test_layer_parity(name):
    layer, x, L = _case(name)
    say(f"[gpu] layer parity {name} T={x.shape[0]}")
    dl = B.DeviceLayer.from_workload(layer)
    xd = B.tokens_to_device(x, dl.dtype)
    gpu = run_gpu(dl, xd, L)
    _compare_all(layer, x, L, gpu, name)


@pytest.mark.parametrize("name", sorted(CASES))
def test_every_mode_matches_oracle(name):
    layer, x, L = _case(name)
    dl = B.DeviceLayer.from_workload(layer)
    xd = B.tokens_to_device(x, dl.dtype)
    modes = ["gemv", "dense"]
    if layer.dtype == "bf16" and layer.d % 128 == 0 and layer.d_expert % 128 == 0:
        modes += ["chunk_mfma", "chunk_split"]
    z, g, m, um, cnt, lst = oracle_full(layer, x, L)
    y_ref = oracle.forward_dense(x, layer.w_in, layer.w_out, g)
    for mode in modes:
        say(f"[gpu] mode {mode} {name}")
        gpu = run_gpu(dl, xd, L, mode=mode, stats=False)
        flipped, keep = check_route(gpu, z, g, m, layer.n_experts, layer.dtype, layer=layer)
        check_y(gpu["y"], y_ref, keep, layer.dtype, f"{name}/{mode}")


def _separate_layer(ly):
    """A layer whose five tensors are each their own torch allocation, as a model's parameters are."""
    dev = torch.device("cuda")
    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return B.DeviceLayer.from_tensors(bf(ly.w_router), bf(ly.w_in), bf(ly.w_out),
                                      b_router=torch.from_numpy(ly.b_router).to(dev), rms_eps=ly.rms_eps)


@pytest.mark.parametrize("alloc", ["separate", "strided"])
def test_distinct_layers_per_chunk(alloc):
    # chunk c must use layers[c % n_layers]: three different layers in one call, either each in its own
    # allocations (the kernels get their addresses) or as evenly spaced copies in one buffer
    d, E, de, L, C = 512, 64, 128, 8, 9
    rngs = [np.random.default_rng(200 + r) for r in range(3)]
    layers = [make_layer(d, E, de, "bf16", 0.9, rg) for rg in rngs]
    x = make_tokens(d, C, L, 0.8, "bf16", np.random.default_rng(210)).x
    if alloc == "separate":
        dl = [_separate_layer(ly) for ly in layers]
    else:
        dl = B.DeviceLayer.from_workload(layers[0], replicas=3)
        for r in (1, 2):
            t = dl.tensors(r)
            src = B.DeviceLayer.from_workload(layers[r]).tensors(0)
            for key in ("w_router", "b_router", "w_in", "w_out"):
                t[key].copy_(src[key])
    xd = B.tokens_to_device(x, BF16)
    for mode in ("auto", "chunk_mfma", "gemv", "dense"):
        say(f"[gpu] {alloc} layers mode {mode}")
        gpu = run_gpu(dl, xd, L, mode=mode, n_layers=3 if alloc == "strided" else None)
        for r in range(3):
            chunks = np.arange(r, C, 3)
            tok = (chunks[:, None] * L + np.arange(L)[None, :]).ravel()
            ly = layers[r]
            z, g, m = oracle.route(x[tok], ly.w_router, ly.b_router, None, ly.rms_eps)
            flipped, keep = check_route(gpu, z, g, m, E, "bf16", t_idx=tok, layer=ly)
            y_ref = oracle.forward_tokens(x[tok], ly.w_in, ly.w_out, g, m)
            check_y(gpu["y"][tok], y_ref, keep, "bf16", f"{alloc} layer {r}/{mode}")


def test_single_token_units_through_separate_layers():
    # chunk_len 1 (decode): token t uses layers[t % 3]; the router and experts take the GEMV-sized path
    d, E, de, T = 1024, 64, 128, 12
    layers = [make_layer(d, E, de, "bf16", 0.887, np.random.default_rng(220 + r)) for r in range(3)]
    x = make_tokens(d, T, 1, 0.0, "bf16", np.random.default_rng(230)).x
    dl = [_separate_layer(ly) for ly in layers]
    xd = B.tokens_to_device(x, BF16)
    for mode in ("auto", "gemv"):
        say(f"[gpu] decode through separate layers mode {mode}")
        gpu = run_gpu(dl, xd, 1, mode=mode)
        for r in range(3):
            tok = np.arange(r, T, 3)
            ly = layers[r]
            z, g, m = oracle.route(x[tok], ly.w_router, ly.b_router, None, ly.rms_eps)
            flipped, keep = check_route(gpu, z, g, m, E, "bf16", t_idx=tok, layer=ly)
            y_ref = oracle.forward_tokens(x[tok], ly.w_in, ly.w_out, g, m)
            check_y(gpu["y"][tok], y_ref, keep, "bf16", f"decode layer {r}/{mode}")


def test_edge_cases_empty_none_and_all_active():
    d, E, de, L = 512, 64, 128, 8
    rng = np.random.default_rng(300)
    layer = make_layer(d, E, de, "bf16", 0.9, rng)
    x = make_tokens(d, 4, L, 0.8, "bf16", rng).x
    dl = B.DeviceLayer.from_workload(layer)
    # zero tokens: every entry point returns OK and enqueues nothing
    say("[gpu] edge: zero tokens")
    x0 = torch.empty((0, d), dtype=torch.bfloat16, device="cuda")
    g0, m0, _ = B.blockffn_route(dl, x0, L)
    _, c0, l0 = B.blockffn_chunk_union(E, m0, L)
    y0 = B.blockffn_forward(dl, x0, L, g0, c0, l0)
    torch.cuda.synchronize()
    assert y0.shape == (0, d)
    # no expert active anywhere: gates, masks, unions and outputs are exactly zero
    for name, bias in (("none active", -1e4), ("all active", 1e4)):
        say(f"[gpu] edge: {name}")
        t = dl.tensors(0)
        t["b_router"].fill_(bias)
        layer.b_router = np.full(E, bias, np.float32)
        xd = B.tokens_to_device(x, BF16)
        for mode in ("auto", "gemv", "chunk_mfma", "chunk_split"):
            gpu = run_gpu(dl, xd, L, mode=mode)
            if bias < 0:
                assert (gpu["mask"] == 0).all() and (gpu["g"] == 0).all()
                assert (gpu["count"] == 0).all() and (gpu["list"] == -1).all()
                assert (gpu["y"] == 0).all()
                assert gpu["stats"]["active_pairs"] == 0 and gpu["stats"]["hist"][0] == x.shape[0]
            else:
                assert (gpu["count"] == E).all()
                np.testing.assert_array_equal(gpu["list"], np.tile(np.arange(E), (4, 1)))
            _compare_all(layer, x, L, gpu, f"{name}/{mode}")


@pytest.mark.parametrize("L", [8, 32])
def test_empty_unions_among_busy_chunks(L):
    """Chunks whose tokens are all zero activate nothing (z = b < 0): their y must be exactly zero
    while their neighbours' are right, on the batched chunk path (more than 16 chunks)."""
    d, E, de, C = 1024, 64, 128, 40
    rng = np.random.default_rng(310 + L)
    layer = make_layer(d, E, de, "bf16", 0.9, rng)
    x = make_tokens(d, C, L, 0.8, "bf16", rng).x.copy()
    empty = [0, 3, 4, 17, 39]
    for c in empty:
        x[c * L:(c + 1) * L] = 0
    say(f"[gpu] empty unions among {C} chunks, L={L}")
    dl = B.DeviceLayer.from_workload(layer)
    xd = B.tokens_to_device(x, BF16)
    gpu = run_gpu(dl, xd, L)
    assert all(gpu["count"][c] == 0 for c in empty)
    assert (gpu["count"][[c for c in range(C) if c not in empty]] > 0).all()
    for c in empty:
        assert (gpu["y"][c * L:(c + 1) * L] == 0).all()
    _compare_all(layer, x, L, gpu, f"empty unions L={L}")


def test_many_chunks():
    # more than 1024 chunks: each thread of the plan kernel owns several chunks,
    # and the stats kernel takes several rounds of tokens per thread
    d, E, de, L, C = 256, 16, 128, 8, 1300
    rng = np.random.default_rng(520)
    layer = make_layer(d, E, de, "bf16", 0.9, rng)
    x = make_tokens(d, C, L, 0.7, "bf16", rng).x
    dl = B.DeviceLayer.from_workload(layer)
    xd = B.tokens_to_device(x, BF16)
    say(f"[gpu] many chunks C={C} T={x.shape[0]}")
    gpu = run_gpu(dl, xd, L, mode="chunk_mfma")
    _compare_all(layer, x, L, gpu, "many_chunks/chunk_mfma")
    z, g, m, um, cnt, lst = oracle_full(layer, x, L)
    y_ref = oracle.forward_dense(x, layer.w_in, layer.w_out, g)
    dense = run_gpu(dl, xd, L, mode="dense", stats=False)
    flipped, keep = check_route(dense, z, g, m, E, "bf16", layer=layer)
    check_y(dense["y"], y_ref, keep, "bf16", "many_chunks/dense")


def test_union_and_stats_kernels_on_seeded_masks():
    # masks straight from a seeded generator (not from the router), so the
    # union and statistics kernels are compared bit for bit
    rng = np.random.default_rng(400)
    for E, L, C, p in ((8, 4, 16, 0.2), (64, 8, 512, 0.19), (70, 3, 33, 0.3), (128, 32, 20, 0.15),
                       (128, 1, 100, 0.5), (1, 2, 7, 0.5),
                       (16, 8, 1100, 0.25), (32, 1, 9000, 0.3)):  # several rounds per stats thread
        say(f"[gpu] union/stats E={E} L={L} C={C}")
        T = L * C
        act = rng.random((T, E)) < p
        W = (E + 63) // 64
        m = np.zeros((T, W), np.uint64)
        for w in range(W):
            for b in range(min(64, E - 64 * w)):
                m[:, w] |= act[:, 64 * w + b].astype(np.uint64) << np.uint64(b)
        md = torch.from_numpy(m.view(np.int64)).cuda()
        um, cnt, lst = B.blockffn_chunk_union(E, md, L)
        st = B.stats_dict(B.blockffn_sparsity_stats(E, md, L))
        torch.cuda.synchronize()
        o_um, o_cnt, o_lst = oracle.chunk_union(m, E, L)
        np.testing.assert_array_equal(B.masks_to_u64(um), o_um)
        np.testing.assert_array_equal(cnt.cpu().numpy(), o_cnt)
        np.testing.assert_array_equal(lst.cpu().numpy(), o_lst)
        o_st = oracle.stats(m, E, L)
        for key in ("n_tokens", "n_chunks", "active_pairs", "union_sum", "reuse_num", "reuse_den"):
            assert st[key] == o_st[key], key
        np.testing.assert_array_equal(st["hist"], o_st["hist"])


def test_tiny_fp32_config_full():
    cfg = CONFIGS["tiny_f32_L4"]
    layer, tok = make_workload(cfg)
    say(f"[gpu] {cfg.name} full")
    dl = B.DeviceLayer.from_workload(layer)
    gpu = run_gpu(dl, B.tokens_to_device(tok.x, F32), cfg.chunk_len)
    _compare_all(layer, tok.x, cfg.chunk_len, gpu, cfg.name)
    # the oracle's dense evaluation agrees too (zero-gate experts add nothing)
    z, g, m = oracle.route(tok.x, layer.w_router, layer.b_router, None, layer.rms_eps)
    np.testing.assert_array_equal(oracle.forward_dense(tok.x, layer.w_in, layer.w_out, g),
                                  oracle.forward_tokens(tok.x, layer.w_in, layer.w_out, g, m))


@pytest.mark.parametrize("name", ["decode_L1_d2048_E64", "chunk8_d2048_E64", "large_L8_d4096_E128",
                                  "large_L32_d4096_E128"])
def test_full_size_every_output(name):
    """Full workload in the benchmark's launch configuration (one layer copy
    per chunk where it fits, the same calls); the oracle checks every mask,
    union and gate, the statistics, and every token's output."""
    cfg = CONFIGS[name]
    layer, tok = make_workload(cfg)
    L, E = cfg.chunk_len, cfg.n_experts
    reps = cfg.replicas
    say(f"[gpu] full size {name} T={cfg.n_tokens} replicas={reps}")
    dl = B.DeviceLayer.from_workload(layer, replicas=reps)
    xd = B.tokens_to_device(tok.x, dl.dtype)
    # as the benchmark runs it: calls of at most one unit per layer copy
    parts = []
    sub = min(cfg.units, reps)
    for c0 in range(0, cfg.units, sub):
        parts.append(run_gpu(dl, xd[c0 * L:(c0 + sub) * L], L, n_layers=reps, want_preact=False, stats=False))
    gpu = {k: np.concatenate([p_[k] for p_ in parts]) for k in parts[0]}
    gpu["stats"] = B.stats_dict(B.blockffn_sparsity_stats(E, torch.from_numpy(gpu["mask"].view(np.int64)).cuda(), L))
    del dl, xd
    torch.cuda.empty_cache()
    z, g, m, um, cnt, lst = oracle_full(layer, tok.x, L)
    flipped, keep = check_route(gpu, z, g, m, E, cfg.dtype, layer=layer)
    nflip_u = check_union(gpu, um, z, E, L)
    if not flipped:
        st = oracle.stats(m, E, L)
        assert gpu["stats"]["union_sum"] == st["union_sum"]
        assert gpu["stats"]["active_pairs"] == st["active_pairs"]
    y_ref = oracle.forward_tokens(tok.x, layer.w_in, layer.w_out, g, m)
    rel = check_y(gpu["y"], y_ref, keep, cfg.dtype, name)
    say(f"  {name}: all {cfg.n_tokens} tokens, max|dy|/rms {rel:.2e}, band flips {len(flipped)} tokens / "
        f"{nflip_u} union bits, TLS {gpu['stats']['tls']:.4f} CLS {gpu['stats']['cls']:.4f}")


# ---------------------------------------------------------------- grouped-by-expert batch path

GROUPED_CASES = {
    # name: (d, E, d_e, L, chunks, bias_k, alpha, seed)
    "d512_E64_de128_L8_C40": (512, 64, 128, 8, 40, 1.0, 0.65, 501),      # ragged last tile per expert
    "d768_E80_de256_L4_C33": (768, 80, 256, 4, 33, 0.9, 0.7, 502),       # E not a multiple of 16, 2 hidden tiles
    "d1024_E128_de128_L1_C300": (1024, 128, 128, 1, 300, 1.6, 0.0, 503),  # rarely-active experts, some empty
    "d256_E8_de128_L8_C16": (256, 8, 128, 8, 16, -1.0, 0.5, 504),        # most pairs active, long groups
    "d384_E24_de128_L8_C12": (384, 24, 128, 8, 12, 0.8, 0.6, 505),       # d not a multiple of a down block's 256 columns
}


@pytest.mark.parametrize("name", sorted(GROUPED_CASES))
def test_grouped_mode_matches_oracle(name):
    d, E, de, L, C, k, a, seed = GROUPED_CASES[name]
    rng = np.random.default_rng(seed)
    layer = make_layer(d, E, de, "bf16", k, rng)
    x = make_tokens(d, C, L, a, "bf16", rng).x
    say(f"[gpu] grouped {name} T={x.shape[0]}")
    dl = B.DeviceLayer.from_workload(layer)
    xd = B.tokens_to_device(x, BF16)
    gpu = run_gpu(dl, xd, L, mode="grouped")
    _compare_all(layer, x, L, gpu, f"grouped/{name}")
    # a second call on the same buffers gives the same bits (deterministic combine)
    gpu2 = run_gpu(dl, xd, L, mode="grouped", stats=False)
    np.testing.assert_array_equal(gpu["y"], gpu2["y"])


def test_grouped_full_size_every_output():
    cfg = CONFIGS["batched_L8_d4096_E128"]
    layer, tok = make_workload(cfg)
    L, E = cfg.chunk_len, cfg.n_experts
    say(f"[gpu] grouped full size {cfg.name} T={cfg.n_tokens}")
    dl = B.DeviceLayer.from_workload(layer)
    xd = B.tokens_to_device(tok.x, BF16)
    gpu = run_gpu(dl, xd, L, mode="grouped", want_preact=False)
    del dl, xd
    torch.cuda.empty_cache()
    z, g, m, um, cnt, lst = oracle_full(layer, tok.x, L)
    flipped, keep = check_route(gpu, z, g, m, E, cfg.dtype, layer=layer)
    y_ref = oracle.forward_tokens(tok.x, layer.w_in, layer.w_out, g, m)
    rel = check_y(gpu["y"], y_ref, keep, cfg.dtype, cfg.name)
    say(f"  {cfg.name}: all {cfg.n_tokens} tokens, max|dy|/rms {rel:.2e}, band flips {len(flipped)}")


def test_grouped_mode_signed_scales():
    # a negative RMS scale gives active pairs negative gates; the grouped path
    # must still include them (pairs are the non-zero gates)
    d, E, de, L, C = 256, 16, 128, 8, 6
    rng = np.random.default_rng(506)
    layer = make_layer(d, E, de, "bf16", 0.3, rng)
    layer.rms_scale = (rng.random(E) * 2.0 - 0.7).astype(np.float32)
    x = make_tokens(d, C, L, 0.6, "bf16", rng).x
    say(f"[gpu] grouped signed scales T={x.shape[0]}")
    dl = B.DeviceLayer.from_workload(layer)
    xd = B.tokens_to_device(x, BF16)
    gpu = run_gpu(dl, xd, L, mode="grouped")
    assert (gpu["g"] < 0).any()
    _compare_all(layer, x, L, gpu, "grouped/signed_scales")
