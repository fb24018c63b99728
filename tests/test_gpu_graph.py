"""The C-ABI calls under HIP graph capture: one captured step (route, union,
forward, stats; and the grouped forward and the backward) replayed several
times, with eager work and synchronisations between the replays, must give
exactly the eager results every time (the kernels are deterministic, and no
call issues a memset or allocates)."""
import numpy as np
import pytest
import torch

from activation_sparse_moe_amd import binding as B
from activation_sparse_moe_amd._capi import BF16
from gpu_parity_util import say
from workload import make_layer, make_tokens

pytestmark = pytest.mark.gpu


def _bufs(dl, T, L, mode):
    E, d = dl.n_experts, dl.d
    dev = "cuda"
    C = T // L
    return dict(g=torch.empty((T, E), device=dev), m=torch.empty((T, dl.mask_words), dtype=torch.int64, device=dev),
                um=torch.empty((C, dl.mask_words), dtype=torch.int64, device=dev),
                cnt=torch.empty((C,), dtype=torch.int32, device=dev),
                lst=torch.empty((C, E), dtype=torch.int32, device=dev),
                y=torch.empty((T, d), device=dev), st=torch.empty((8 + 129,), dtype=torch.int64, device=dev),
                ws=B.alloc_workspace(dl, T, L, mode))


def _step(dl, xd, L, b, mode):
    B.blockffn_route(dl, xd, L, gates=b["g"], token_masks=b["m"])
    B.blockffn_chunk_union(dl.n_experts, b["m"], L, chunk_masks=b["um"], active_count=b["cnt"],
                           active_list=b["lst"])
    B.blockffn_forward(dl, xd, L, b["g"], b["cnt"], b["lst"], mode=mode, workspace=b["ws"], y=b["y"])
    B.blockffn_sparsity_stats(dl.n_experts, b["m"], L, stats_dev=b["st"])


def _snapshot(b):
    return {k: v.detach().cpu().clone() for k, v in b.items() if k != "ws"}


# (mode, chunk length, chunks): 24 chunks of 8 take the chunk kernels under AUTO, 8 chunks the
# few-unit kernels, 20 chunks of 32 the lockstep two-tile kernels
@pytest.mark.parametrize("mode,L,C", [("auto", 8, 24), ("grouped", 8, 24), ("gemv", 8, 24), ("chunk_split", 8, 24),
                                      ("auto", 8, 8), ("auto", 32, 20)])
def test_forward_step_replays_match_eager(mode, L, C):
    d, E, de = 512, 64, 128
    rng = np.random.default_rng(801)
    layer = make_layer(d, E, de, "bf16", 0.9, rng)
    x = make_tokens(d, C, L, 0.8, "bf16", rng).x
    say(f"[gpu] graph replay, forward mode {mode}, {C} chunks of {L}")
    dl = B.DeviceLayer.from_workload(layer)
    xd = B.tokens_to_device(x, BF16)
    b = _bufs(dl, x.shape[0], L, mode)
    _step(dl, xd, L, b, mode)
    torch.cuda.synchronize()
    eager = _snapshot(b)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm the capture stream
        _step(dl, xd, L, b, mode)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _step(dl, xd, L, b, mode)
    for rep in range(3):
        for v in b.values():  # scribble over the outputs eagerly, then replay
            v.fill_(0) if v.dtype != torch.uint8 else None
        noise = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(b)
        for k in eager:
            assert torch.equal(got[k], eager[k]), f"replay {rep}: {k} differs from the eager run"
        del noise


def test_backward_replays_match_eager():
    d, E, de, L, C = 256, 16, 128, 8, 8
    rng = np.random.default_rng(802)
    layer = make_layer(d, E, de, "bf16", 0.5, rng)
    x = make_tokens(d, C, L, 0.6, "bf16", rng).x
    say("[gpu] graph replay, backward")
    dl = B.DeviceLayer.from_workload(layer)
    xd = B.tokens_to_device(x, BF16)
    _, _, z = B.blockffn_route(dl, xd, L, want_preact=True)
    dy = torch.randn((x.shape[0], d), device="cuda")
    ws = B.alloc_backward_workspace(dl, x.shape[0])
    out = B.blockffn_backward(dl, xd, z, dy, workspace=ws)
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in out.items()}
    grads = {k: v for k, v in out.items() if k != "dx"}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.blockffn_backward(dl, xd, z, dy, workspace=ws, dx=out["dx"], grads=grads)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.blockffn_backward(dl, xd, z, dy, workspace=ws, dx=out["dx"], grads=grads)
    for rep in range(3):
        for v in out.values():
            v.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in eager:
            assert torch.equal(out[k], eager[k]), f"replay {rep}: {k} differs from the eager run"
