"""FFF tree layer on the GPU (blockffn_fff_forward through the C ABI) against
the CPU oracle, on the same seeded inputs.

Bars:
  * paths: bit-exact, except where the two sides turn differently at a node
    whose oracle pre-activation lies within 1e-4 of zero: fp32 and fp64 sums
    may disagree on the sign there, and the walks then continue on different
    nodes, so that token is left out of the output check and counted (the
    count must stay below 1% of the tokens; with unit-variance
    pre-activations and fp32 errors near 1e-6 it is normally 0);
  * node pre-activations where the paths agree: |dc| <= 1e-4 (c has unit
    variance; an fp32 dot product of length d <= 4096 errs by about 1e-6);
  * outputs: max |dy| <= 1e-5 x RMS(y_oracle) over the compared tokens, for
    fp32 and bf16 layers alike: bf16 inputs are exact in both
    computations and the GPU keeps every intermediate in fp32 (no rounding to
    bf16 between nodes), so the only differences are fp32 summation order
    and the fp32 GELU, a few units in the 7th digit.
"""
import numpy as np
import pytest
import torch

import oracle
from activation_sparse_moe_amd import binding as B
from activation_sparse_moe_amd._capi import BF16, F32
from gpu_parity_util import say
from workload import get_fff_config, make_fff_layer, make_fff_tokens, make_fff_workload

pytestmark = pytest.mark.gpu

BAND = 1e-4
PRE_TOL = 1e-4
Y_TOL = 1e-5


def _dev_layer(layers, post=False, interleave=True, separate=False):
    """One device layer stack from a list of host layers (copy r = layers[r]), or with `separate` a list of
    device layers, each in its own allocation."""
    if separate:
        return [B.DeviceFffLayer.from_workload(lr, post=post, interleave=interleave) for lr in layers]
    dl = B.DeviceFffLayer.from_workload(layers[0], post=post, replicas=len(layers), interleave=interleave)
    for r, lr in enumerate(layers[1:], start=1):
        dl.fill(r, lr)
    return dl


def _oracle(layers, x, post, dense, tokens=None):
    """Oracle outputs for the given tokens (all by default), token t through layers[t % len(layers)]."""
    T = x.shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    n = len(layers)
    P, D = layers[0].n_trees, layers[0].depth
    V = ((1 << (D + 1)) - 1) if dense else D + 1
    paths = np.zeros((len(tokens), P, V), np.int32)
    pre = np.zeros((len(tokens), P, V))
    y = np.zeros((len(tokens), x.shape[1]))
    for r in range(n):
        sel = np.nonzero(tokens % n == r)[0]
        if len(sel) == 0:
            continue
        lr = layers[r]
        p, c, yy = oracle.fff_forward(x[tokens[sel]], lr.w_node, lr.b_node, lr.w_out, post=post, dense=dense)
        if p is not None:
            paths[sel] = p
        pre[sel] = c
        y[sel] = yy
    return paths, pre, y


def _compare(paths_g, pre_g, y_g, paths_o, pre_o, y_o, where):
    T = y_o.shape[0]
    flipped = set()
    if paths_o is not None:
        assert np.all(paths_g[:, :, 0] == 0)
        differ = paths_g != paths_o
        for t, p in zip(*np.nonzero(differ.any(axis=2))):
            lv = int(np.argmax(differ[t, p]))           # first level on a different node (>= 1)
            c = pre_o[t, p, lv - 1]
            assert abs(c) < BAND, f"{where}: token {t} tree {p} turned differently at level {lv - 1}, c = {c}"
            flipped.add(int(t))
        same = np.cumprod(~differ, axis=2).astype(bool)
        dc = np.abs(pre_g.astype(np.float64) - pre_o)[same]
        assert dc.size == 0 or dc.max() <= PRE_TOL, f"{where}: pre-activation error {dc.max():.3e}"
    assert len(flipped) <= max(1, T // 100), f"{where}: {len(flipped)} tokens took a different path"
    keep = np.array([t for t in range(T) if t not in flipped], dtype=np.int64)
    if keep.size == 0:
        return 0
    yo = y_o[keep]
    rms = np.sqrt(np.mean(yo ** 2))
    err = np.abs(y_g[keep].astype(np.float64) - yo).max()
    assert err <= Y_TOL * rms, f"{where}: max |dy| = {err:.3e} > {Y_TOL} x RMS {rms:.3e}"
    return len(flipped)


def _case(d, P, D, dtype, T, seed, post=False, dense=False, n_layers=1, bias=True, interleave=True, split=0,
          separate=False):
    rng = np.random.default_rng(seed)
    layers = [make_fff_layer(d, P, D, dtype, rng, bias=bias) for _ in range(n_layers)]
    x = make_fff_tokens(d, T, dtype, rng)
    where = (f"d={d} P={P} D={D} {dtype} T={T} post={post} dense={dense} layers={n_layers} "
             f"interleave={interleave} split={split} separate={separate}")
    say(f"[gpu] fff {where}")
    dl = _dev_layer(layers, post, interleave, separate)
    xd = B.tokens_to_device(x, F32 if dtype == "f32" else BF16)
    y, paths, pre = B.blockffn_fff_forward(dl, xd, mode="dense" if dense else "sparse", want_paths=not dense,
                                           split=split)
    torch.cuda.synchronize()
    po, co, yo = _oracle(layers, x, post, dense)
    flips = _compare(None if dense else paths.cpu().numpy(), None if dense else pre.cpu().numpy(),
                     y.cpu().numpy(), None if dense else po, co, yo, where)
    return dl, xd, flips


@pytest.mark.parametrize("d,P,D,dtype,T,post,n_layers", [
    (256, 5, 3, "f32", 48, False, 1),
    (256, 5, 3, "f32", 1, False, 1),
    (512, 13, 4, "bf16", 33, False, 1),     # 13 trees: lockstep pairs, then single trees
    (2048, 64, 6, "bf16", 40, False, 3),    # the timed shape, three distinct stacked layers
    (1024, 8, 5, "bf16", 20, True, 1),      # GELU after the aggregation
    (768, 6, 2, "f32", 17, True, 2),
    (512, 16, 0, "bf16", 9, False, 1),      # depth 0: a plain MLP of 16 units
    (512, 2, 15, "bf16", 16, False, 1),     # maximum depth
    (2048, 4, 3, "f32", 12, False, 1),      # widest f32 row (8 pieces)
    (4096, 8, 3, "bf16", 12, False, 1),     # widest bf16 row (8 pieces)
])
def test_fff_sparse_matches_oracle(d, P, D, dtype, T, post, n_layers):
    _case(d, P, D, dtype, T, 900 + d + P + D + T, post=post, n_layers=n_layers)


@pytest.mark.parametrize("d,P,D,dtype,T,post", [
    (256, 3, 3, "f32", 10, False),
    (512, 4, 4, "bf16", 7, False),
    (512, 5, 2, "bf16", 6, True),
])
def test_fff_dense_matches_oracle(d, P, D, dtype, T, post):
    _case(d, P, D, dtype, T, 950 + d + P + D, post=post, dense=True)


@pytest.mark.parametrize("split", [1, 2, 3, 0])
@pytest.mark.parametrize("d,P,D,dtype,T,post", [
    (2048, 64, 6, "bf16", 7, False),        # 64 trees over 1, 2, 3 or (automatically) 16 blocks per token
    (512, 13, 4, "bf16", 5, True),          # uneven groups, GELU after the combine
    (256, 9, 3, "f32", 3, False),
])
def test_fff_blocks_per_token(d, P, D, dtype, T, post, split):
    _case(d, P, D, dtype, T, 970 + P + split, post=post, split=split)


@pytest.mark.parametrize("dense", [False, True])
def test_fff_separately_allocated_layers(dense):
    # token t uses layers[t % 3], each layer in its own allocation: the kernel gets each layer's addresses
    _case(1024, 6, 3, "bf16", 14, 966, dense=dense, n_layers=3, separate=True)


def test_fff_without_bias():
    _case(512, 6, 4, "bf16", 11, 961, bias=False)


@pytest.mark.parametrize("dense", [False, True])
def test_fff_separate_row_arrays(dense):
    # node_stride 0: w_node and w_out as two dense [P][N][d] arrays
    _case(1024, 7, 3, "bf16", 13, 965, dense=dense, n_layers=2, interleave=False)


def test_fff_zero_tokens_and_determinism():
    dl, xd, _ = _case(1024, 9, 4, "bf16", 64, 962)
    y0 = torch.full((0, 1024), 7.0, device="cuda")
    y_empty, _, _ = B.blockffn_fff_forward(dl, xd[:0], y=y0)
    assert y_empty.shape == (0, 1024)
    a = B.blockffn_fff_forward(dl, xd, want_paths=True)
    b = B.blockffn_fff_forward(dl, xd, want_paths=True)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_fff_graph_replays_match_eager():
    rng = np.random.default_rng(963)
    layer = make_fff_layer(512, 8, 4, "bf16", rng)
    x = make_fff_tokens(512, 24, "bf16", rng)
    say("[gpu] fff graph replay")
    dl = B.DeviceFffLayer.from_workload(layer)
    xd = B.tokens_to_device(x, BF16)
    ws = B.alloc_fff_workspace(dl, 24)                      # 24 tokens: several blocks per token
    assert ws is not None
    y, paths, pre = B.blockffn_fff_forward(dl, xd, want_paths=True, workspace=ws)
    torch.cuda.synchronize()
    eager = [v.clone() for v in (y, paths, pre)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.blockffn_fff_forward(dl, xd, y=y, paths=paths, node_preact=pre, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.blockffn_fff_forward(dl, xd, y=y, paths=paths, node_preact=pre, workspace=ws)
    for rep in range(3):
        for v in (y, paths, pre, ws):
            v.zero_()
        noise = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((y, paths, pre), eager):
            assert torch.equal(got, want), f"replay {rep} differs from the eager run"
        del noise


def test_fff_timed_configuration_every_output():
    """The benchmark's configuration and launch: 4096 tokens, each through its
    own copy of the layer (1024 copies), all in one call; every token's paths,
    node pre-activations and output against the oracle (every copy holds the
    same weights)."""
    cfg = get_fff_config("fff_D6_P64_d2048")
    layer, x = make_fff_workload(cfg)
    say(f"[gpu] fff timed configuration {cfg.name}, {cfg.replicas} copies")
    dl = B.DeviceFffLayer.from_workload(layer, replicas=cfg.replicas)
    xd = B.tokens_to_device(x, BF16)
    y, paths, pre = B.blockffn_fff_forward(dl, xd, want_paths=True)
    torch.cuda.synchronize()
    po, co, yo = _oracle([layer], x, False, False)
    _compare(paths.cpu().numpy(), pre.cpu().numpy(), y.cpu().numpy(), po, co, yo, cfg.name)
    del dl
    torch.cuda.empty_cache()


def _draw(seed: int):
    """A seeded shape from the supported range: dtype, d, trees, depth, tokens, layer copies, bias,
    node layout, blocks per token (at most ceil(P / 4)) and, at small depth, the dense mode."""
    r = np.random.default_rng(6000 + seed)
    dtype = "f32" if r.random() < 0.3 else "bf16"
    d = (256 if dtype == "f32" else 512) * int(r.integers(1, 9))
    P = int(r.choice([1, 2, 3, 7, 13, 16, 33, 64]))
    D = int(r.integers(0, 9))
    dense = D <= 6 and r.random() < 0.25
    split = int(r.integers(0, (P + 3) // 4 + 1))  # 0: the library's choice
    return dict(d=d, P=P, D=D, dtype=dtype, T=int(r.integers(1, 65)), dense=bool(dense),
                n_layers=int(r.integers(1, 4)), bias=bool(r.random() < 0.7), interleave=bool(r.random() < 0.5),
                split=split)


@pytest.mark.parametrize("seed", range(16))
def test_fff_drawn_shapes(seed):
    s = _draw(seed)
    _case(s["d"], s["P"], s["D"], s["dtype"], s["T"], 990 + seed, dense=s["dense"], n_layers=s["n_layers"],
          bias=s["bias"], interleave=s["interleave"], split=s["split"])
