"""blockffn_forward_noalloc (the forward with the library's static scratch
array, for callers that cannot allocate) against blockffn_forward with a
caller workspace, through the C ABI.

The two share every kernel, so on the same inputs they must give the same
bits; the results are also held to the oracle's bar (max |dy| <= 2e-2 x RMS
of the oracle output for bf16).  Calls follow one another on one stream with
shrinking inputs, so each call runs on scratch the previous one left behind.
"""
import numpy as np
import pytest
import torch

import oracle
from activation_sparse_moe_amd import _capi
from activation_sparse_moe_amd import binding as B
from activation_sparse_moe_amd._capi import BF16
from gpu_parity_util import check_y, oracle_full, say
from workload import make_layer, make_tokens

pytestmark = pytest.mark.gpu


def _case(d, E, de, L, C, seed):
    rng = np.random.default_rng(seed)
    layer = make_layer(d, E, de, "bf16", 0.887, rng)
    x = make_tokens(d, C, L, 0.8, "bf16", rng).x
    dl = B.DeviceLayer.from_workload(layer)
    xd = B.tokens_to_device(x, BF16)
    g, m, z = B.blockffn_route(dl, xd, L)
    _, cnt, lst = B.blockffn_chunk_union(E, m, L)
    return layer, x, dl, xd, g, cnt, lst


def test_noalloc_matches_forward_on_successive_calls():
    # (d, E, d_e, L, chunks, mode): 28 MiB of scratch on the chunk path, then smaller calls that find the
    # previous call's data in the array: the split path (a few chunks), the grouped and GEMV paths
    calls = [(2048, 64, 128, 8, 224, "auto"), (2048, 64, 128, 8, 6, "auto"), (512, 64, 128, 8, 12, "grouped"),
             (1024, 48, 128, 1, 40, "gemv")]
    runs = []
    for k, (d, E, de, L, C, mode) in enumerate(calls):
        layer, x, dl, xd, g, cnt, lst = _case(d, E, de, L, C, 700 + k)
        need = B.blockffn_workspace_size(dl, x.shape[0], L, mode)
        assert 0 < need <= _capi.NOALLOC_SCRATCH_BYTES
        y_na = torch.full((x.shape[0], d), float("nan"), device="cuda")
        say(f"[gpu] noalloc call {k}: d={d} E={E} L={L} C={C} mode={mode} scratch {need} bytes")
        B.blockffn_forward_noalloc(dl, xd, L, g, cnt, lst, mode=mode, y=y_na)
        runs.append((layer, x, dl, xd, g, cnt, lst, L, mode, y_na))
    torch.cuda.synchronize()
    for k, (layer, x, dl, xd, g, cnt, lst, L, mode, y_na) in enumerate(runs):
        y_ws = B.blockffn_forward(dl, xd, L, g, cnt, lst, mode=mode)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ws), f"call {k}: the static-scratch forward differs from the workspace forward"
        z, og, om, _, _, _ = oracle_full(layer, x, L)
        keep = np.ones(x.shape[0], bool)
        y_ref = oracle.forward_tokens(x, layer.w_in, layer.w_out, og, om)
        # tokens whose activation pattern flipped inside the decision band leave the output check
        gm = B.masks_to_u64(B.blockffn_route(dl, xd, L)[1])
        flips = (gm != om).any(axis=1)
        keep &= ~flips
        rel = check_y(y_na.cpu().numpy(), y_ref, keep, "bf16", f"noalloc call {k}")
        say(f"  call {k}: bit-identical to blockffn_forward, max|dy|/rms {rel:.2e} against the oracle")


def test_noalloc_rejects_calls_beyond_the_array():
    # 4096 chunk-8 tokens at d = 2048, E = 64 need 64 MiB: refused on the host, nothing enqueued
    d, E, de, L, C = 2048, 64, 128, 8, 512
    layer, x, dl, xd, g, cnt, lst = _case(d, E, de, L, C, 720)
    assert B.blockffn_workspace_size(dl, x.shape[0], L) > _capi.NOALLOC_SCRATCH_BYTES
    y = torch.full((x.shape[0], d), 3.0, device="cuda")
    with pytest.raises(_capi.BlockFFNError) as err:
        B.blockffn_forward_noalloc(dl, xd, L, g, cnt, lst, y=y)
    assert err.value.status == _capi.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
    # zero tokens: valid, nothing to do
    B.blockffn_forward_noalloc(dl, xd[:0], L, g[:0], cnt[:0], lst[:0], y=y[:0])
    torch.cuda.synchronize()
