"""The C-ABI library loads, exports what include/blockffn.h declares, matches
the header's struct layout, and rejects bad arguments on the host.

No test here runs GPU work: every call below fails host-side validation,
which runs before any HIP call.  Calls that use placeholder device pointers
are skipped on a machine that shows a GPU, so that no placeholder can ever
reach a kernel.
"""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from activation_sparse_moe_amd import _capi
from activation_sparse_moe_amd._capi import BlockffnFffLayer, BlockffnGrads, BlockffnLayer, BlockffnStats

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "blockffn.h")


@pytest.fixture(scope="module")
def lib():
    return _capi.load()


def _no_gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


cpu_only = pytest.mark.skipif(not _no_gpu_visible(), reason="placeholder pointers are only used without a GPU")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(blockffn_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert set(declared) == set(_capi.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _capi.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(declared) <= exported
    # internal symbols stay hidden
    assert not any(s.startswith("_ZN4bffn") for s in exported)


def test_struct_layout_matches_header():
    prog = r"""
#include <stddef.h>
#include <stdio.h>
#include "blockffn.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu\n", sizeof(blockffn_layer), offsetof(blockffn_layer, reserved),
         offsetof(blockffn_layer, w_router), offsetof(blockffn_layer, w_out), sizeof(blockffn_stats));
  printf("%zu %zu\n", offsetof(blockffn_stats, active_pairs), offsetof(blockffn_stats, hist));
  printf("%zu %zu %zu\n", sizeof(blockffn_grads), offsetof(blockffn_grads, d_rms_scale),
         offsetof(blockffn_grads, d_w_out));
  printf("%zu %zu %zu %zu %zu\n", sizeof(blockffn_fff_layer), offsetof(blockffn_fff_layer, activation),
         offsetof(blockffn_fff_layer, w_node), offsetof(blockffn_fff_layer, b_node),
         offsetof(blockffn_fff_layer, w_out));
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "layout.c")
        exe = os.path.join(tmp, "layout")
        open(src, "w").write(prog)
        subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I",
                        "/opt/rocm/include", src, "-o", exe], check=True)
        lines = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split("\n")
    a = [int(v) for v in lines[0].split()]
    b = [int(v) for v in lines[1].split()]
    assert a == [ctypes.sizeof(BlockffnLayer), BlockffnLayer.reserved.offset, BlockffnLayer.w_router.offset,
                 BlockffnLayer.w_out.offset, ctypes.sizeof(BlockffnStats)]
    assert b == [BlockffnStats.active_pairs.offset, BlockffnStats.hist.offset]
    c = [int(v) for v in lines[2].split()]
    assert c == [ctypes.sizeof(BlockffnGrads), BlockffnGrads.d_rms_scale.offset, BlockffnGrads.d_w_out.offset]
    f = [int(v) for v in lines[3].split()]
    assert f == [ctypes.sizeof(BlockffnFffLayer), BlockffnFffLayer.activation.offset,
                 BlockffnFffLayer.w_node.offset, BlockffnFffLayer.b_node.offset, BlockffnFffLayer.w_out.offset]


def test_version_and_status_strings(lib):
    assert lib.blockffn_version() == 2
    assert lib.blockffn_status_string(0) == b"ok"
    for code in range(-9, 0):
        s = lib.blockffn_status_string(code)
        assert s and s != b"unknown status"
    assert lib.blockffn_status_string(-100) == b"unknown status"


P = 0x10000  # placeholder, 64 KiB aligned; never dereferenced (every call fails validation)


def _layer(**kw):
    f = dict(d=256, n_experts=16, d_expert=128, dtype=1, rms_eps=1e-6, reserved=0,
             w_router=P, b_router=P, rms_scale=None, w_in=P, w_out=P)
    f.update(kw)
    return BlockffnLayer(**f)


def _arr(layers):
    return (BlockffnLayer * len(layers))(*layers)


def _route(lib, layer, n_layers=1, x=P, T=16, L=8, gates=P, masks=P, preact=None):
    ref = None if layer is None else ctypes.byref(layer) if isinstance(layer, BlockffnLayer) else layer
    return lib.blockffn_route(ref, n_layers, x, T, L, gates, masks, preact, None)


@cpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), _capi.ERR_DTYPE),
    (dict(n_experts=0), _capi.ERR_SHAPE),
    (dict(n_experts=129), _capi.ERR_SHAPE),
    (dict(d=100), _capi.ERR_SHAPE),
    (dict(d=0), _capi.ERR_SHAPE),
    (dict(d_expert=24), _capi.ERR_SHAPE),
    (dict(d_expert=2048), _capi.ERR_SHAPE),
    (dict(rms_eps=-1.0), _capi.ERR_SHAPE),
    (dict(rms_eps=float("nan")), _capi.ERR_SHAPE),
    (dict(reserved=1), _capi.ERR_SHAPE),
    (dict(w_in=None), _capi.ERR_NULL),
    (dict(w_router=P + 8), _capi.ERR_ALIGN),
    (dict(b_router=P + 2), _capi.ERR_ALIGN),
])
def test_route_rejects_bad_layer(lib, kw, code):
    assert _route(lib, _layer(**kw)) == code
    assert lib.blockffn_last_error()


@cpu_only
def test_route_rejects_bad_arguments(lib):
    assert _route(lib, None) == _capi.ERR_NULL
    assert _route(lib, _layer(), n_layers=0) == _capi.ERR_LAYERS
    assert _route(lib, _layer(), n_layers=-3) == _capi.ERR_LAYERS
    assert _route(lib, _layer(), L=0) == _capi.ERR_CHUNK
    assert _route(lib, _layer(), L=33) == _capi.ERR_CHUNK
    assert _route(lib, _layer(), T=12, L=8) == _capi.ERR_CHUNK             # ragged tail
    assert _route(lib, _layer(), T=-8) == _capi.ERR_CHUNK
    assert _route(lib, _layer(), x=None) == _capi.ERR_NULL
    assert _route(lib, _layer(), gates=None) == _capi.ERR_NULL
    assert _route(lib, _layer(), x=P + 4) == _capi.ERR_ALIGN
    assert _route(lib, _layer(), masks=P + 4) == _capi.ERR_ALIGN
    assert b"multiple of chunk_len" in (lib.blockffn_route(ctypes.byref(_layer()), 1, P, 12, 8, P, P, None, None)
                                        and lib.blockffn_last_error())


@cpu_only
def test_layer_arrays_are_validated(lib):
    """Every descriptor of a layer array is checked, and they must share one shape."""
    M = 1 << 24
    ok2 = _arr([_layer(), _layer(w_router=P + M, b_router=P + 2 * M, w_in=P + 3 * M, w_out=P + 4 * M)])
    # a valid array passes validation and then fails on the NULL x (nothing is launched)
    assert _route(lib, ok2, n_layers=2, x=None) == _capi.ERR_NULL
    bad = [
        (_arr([_layer(), _layer(d=512)]), _capi.ERR_LAYERS),            # shapes differ
        (_arr([_layer(), _layer(n_experts=32)]), _capi.ERR_LAYERS),
        (_arr([_layer(), _layer(d_expert=256)]), _capi.ERR_LAYERS),
        (_arr([_layer(), _layer(dtype=0)]), _capi.ERR_LAYERS),
        (_arr([_layer(), _layer(rms_eps=1e-5)]), _capi.ERR_LAYERS),
        (_arr([_layer(), _layer(w_in=None)]), _capi.ERR_NULL),          # a later descriptor is checked too
        (_arr([_layer(), _layer(w_out=P + 8)]), _capi.ERR_ALIGN),
        (_arr([_layer(), _layer(reserved=3)]), _capi.ERR_SHAPE),
        (_arr([_layer(), _layer(dtype=9)]), _capi.ERR_DTYPE),
    ]
    for arr, code in bad:
        assert _route(lib, arr, n_layers=2) == code, lib.blockffn_last_error()
        assert _forward(lib, arr, n_layers=2) == code
    # more than 32 scattered layers cannot be listed; evenly spaced ones can be any number, and so can
    # repeats of a few layers
    def scattered(n):
        return _arr([_layer(w_router=P + M * (l * l + 1), w_in=P + M * (l * l + 2), w_out=P + M * (l * l + 3))
                     for l in range(n)])
    assert _route(lib, scattered(32), n_layers=32, x=None) == _capi.ERR_NULL
    assert _route(lib, scattered(33), n_layers=33, x=None) == _capi.ERR_LAYERS
    assert b"evenly spaced" in lib.blockffn_last_error()
    even = _arr([_layer(w_router=P + l * M, b_router=P + l * M + 4096, w_in=P + l * M + 8192,
                        w_out=P + l * M + 16384) for l in range(600)])
    assert _route(lib, even, n_layers=600, x=None) == _capi.ERR_NULL
    # evenly spaced except that one layer's bias is NULL: 40 such layers must be listed, which is too many
    uneven = list(even)[:40]
    uneven[7] = _layer(w_router=P + 7 * M, b_router=None, w_in=P + 7 * M + 8192, w_out=P + 7 * M + 16384)
    assert _route(lib, _arr(uneven), n_layers=40, x=None) == _capi.ERR_LAYERS
    periodic = _arr(list(scattered(2)) * 40)                           # 80 entries, 2 distinct layers
    assert _route(lib, periodic, n_layers=80, x=None) == _capi.ERR_NULL


@cpu_only
def test_union_and_stats_reject_bad_arguments(lib):
    u = lib.blockffn_chunk_union
    assert u(0, P, 16, 8, P, P, P, None) == _capi.ERR_SHAPE
    assert u(200, P, 16, 8, P, P, P, None) == _capi.ERR_SHAPE
    assert u(64, P, 16, 3, P, P, P, None) == _capi.ERR_CHUNK
    assert u(64, None, 16, 8, P, P, P, None) == _capi.ERR_NULL
    assert u(64, P, 16, 8, P, P, None, None) == _capi.ERR_NULL
    assert u(64, P + 4, 16, 8, P, P, P, None) == _capi.ERR_ALIGN
    s = lib.blockffn_sparsity_stats
    assert s(0, P, 16, 8, P, None) == _capi.ERR_SHAPE
    assert s(64, P, 16, 5, P, None) == _capi.ERR_CHUNK
    assert s(64, P, 16, 8, None, None) == _capi.ERR_NULL
    assert s(64, P, 16, 8, P + 4, None) == _capi.ERR_ALIGN


def _forward(lib, layer, mode=0, T=16, L=8, ws=P, ws_bytes=1 << 40, y=P, count=P, lst=P, n_layers=1):
    ref = ctypes.byref(layer) if isinstance(layer, BlockffnLayer) else layer
    return lib.blockffn_forward(ref, n_layers, P, T, L, P, count, lst, mode, ws, ws_bytes, y, None)


@cpu_only
def test_forward_rejects_bad_arguments(lib):
    assert _forward(lib, _layer(), mode=9) == _capi.ERR_MODE
    assert _forward(lib, _layer(dtype=0), mode=_capi.MODE_CHUNK_MFMA) == _capi.ERR_MODE  # MFMA needs bf16
    assert _forward(lib, _layer(d=192), mode=_capi.MODE_CHUNK_MFMA) == _capi.ERR_MODE    # d % 128
    assert _forward(lib, _layer(), ws_bytes=1024) == _capi.ERR_WORKSPACE
    assert _forward(lib, _layer(), ws=None) == _capi.ERR_NULL
    assert _forward(lib, _layer(), ws=P + 64) == _capi.ERR_ALIGN
    assert _forward(lib, _layer(), y=P + 4) == _capi.ERR_ALIGN
    assert _forward(lib, _layer(), count=None) == _capi.ERR_NULL
    assert _forward(lib, _layer(), T=20) == _capi.ERR_CHUNK
    assert _forward(lib, _layer(dtype=0), mode=_capi.MODE_GROUPED) == _capi.ERR_MODE     # GROUPED needs bf16
    assert _forward(lib, _layer(d_expert=64), mode=_capi.MODE_GROUPED) == _capi.ERR_MODE
    assert _forward(lib, _layer(d_expert=384), mode=_capi.MODE_GROUPED) == _capi.ERR_MODE   # d_expert 128 or 256
    two = _arr([_layer(), _layer(w_router=P + (1 << 20), w_in=P + (1 << 20), w_out=P + (1 << 20))])
    assert _forward(lib, two, mode=_capi.MODE_GROUPED, n_layers=2) == _capi.ERR_LAYERS  # one layer only
    assert _forward(lib, _layer(), mode=_capi.MODE_GROUPED, ws_bytes=4096) == _capi.ERR_WORKSPACE


@cpu_only
def test_forward_noalloc_rejects_calls_beyond_its_array(lib):
    f = lib.blockffn_forward_noalloc
    lay = _layer(d=2048, n_experts=64, d_expert=128)
    # 4096 chunk-8 tokens need 64 MiB of scratch: more than the static array holds
    assert f(ctypes.byref(lay), 1, P, 4096, 8, P, P, P, 0, P, None) == _capi.ERR_WORKSPACE
    assert b"static array" in lib.blockffn_last_error()
    assert f(ctypes.byref(lay), 1, P, 20, 8, P, P, P, 0, P, None) == _capi.ERR_CHUNK   # validated like the forward
    assert f(ctypes.byref(lay), 1, P, 16, 8, P, P, P, 9, P, None) == _capi.ERR_MODE
    assert f(ctypes.byref(lay), 0, P, 16, 8, P, P, P, 0, P, None) == _capi.ERR_LAYERS
    assert f(ctypes.byref(lay), 1, None, 0, 8, None, None, None, 0, None, None) == _capi.OK  # no tokens: nothing to do


def test_workspace_size(lib):
    lay = _layer(d=2048, n_experts=64, d_expert=128)
    T = 4096
    r256 = lambda v: (v + 255) // 256 * 256  # noqa: E731
    # hidden activations (bf16 on the chunk path, fp32 on the GEMV path) + the plan: one int64 per
    # chunk plus a total, the down kernel's 8 + 1 XCD range bounds, and 1 + 8 u32 pool counters
    plan = lambda C: r256(8 * (C + 1) + 8 * 9 + 4 * 9)  # noqa: E731
    assert lib.blockffn_workspace_size(ctypes.byref(lay), T, 8, _capi.MODE_CHUNK_MFMA) == \
        T * 64 * 128 * 2 + plan(T // 8)
    assert lib.blockffn_workspace_size(ctypes.byref(lay), T, 1, _capi.MODE_AUTO) == \
        T * 64 * 128 * 2 + plan(T)
    assert lib.blockffn_workspace_size(ctypes.byref(lay), T, 1, _capi.MODE_GEMV) == \
        T * 64 * 128 * 4 + plan(T)
    assert lib.blockffn_workspace_size(ctypes.byref(lay), T, 3, _capi.MODE_AUTO) == 0   # ragged
    assert lib.blockffn_workspace_size(ctypes.byref(lay), T, 8, 99) == 0
    # a few units: AUTO runs blocks of 16 rows over a given union, whose workspace is Swish(W_in x)
    # [C][E][L][d_e] bf16; CHUNK_SPLIT splits each unit's work (8 k-ranges of 4 steps, 8 slot ranges)
    # and adds the fp32 partial tiles of the up items [C][E][d_e/64][8][L][64] and the down items
    # [C][d/64][8][L][64]
    C, L = 2, 8
    split_ws = C * L * 64 * 128 * 2 + plan(C) + r256(C * 64 * 2 * 8 * L * 64 * 4) + r256(C * 32 * 8 * L * 64 * 4)
    assert lib.blockffn_workspace_size(ctypes.byref(lay), C * L, L, _capi.MODE_AUTO) == r256(C * L * 64 * 128 * 2)
    assert lib.blockffn_workspace_size(ctypes.byref(lay), C * L, L, _capi.MODE_CHUNK_SPLIT) == split_ws
    # d above 4096: AUTO splits
    big = _layer(d=8192, n_experts=64, d_expert=128)
    assert lib.blockffn_workspace_size(ctypes.byref(big), C * L, L, _capi.MODE_AUTO) == \
        lib.blockffn_workspace_size(ctypes.byref(big), C * L, L, _capi.MODE_CHUNK_SPLIT)
    assert lib.blockffn_workspace_size(ctypes.byref(lay), C * L, L, _capi.MODE_CHUNK_MFMA) == \
        C * L * 64 * 128 * 2 + plan(C)
    # 17 units: AUTO no longer splits
    assert lib.blockffn_workspace_size(ctypes.byref(lay), 17 * L, L, _capi.MODE_AUTO) == \
        17 * L * 64 * 128 * 2 + plan(17)
    # CHUNK_SPLIT needs the matrix-core shapes
    f32 = _layer(d=2048, n_experts=64, d_expert=128, dtype=_capi.F32)
    assert lib.blockffn_workspace_size(ctypes.byref(f32), C * L, L, _capi.MODE_CHUNK_SPLIT) == 0


def _layer_forward(lib, layer, T=16, L=8, x=P, gates=P, masks=P, preact=None, um=P, count=P, lst=P, stats=P,
                   ws=P, ws_bytes=1 << 40, y=P, n_layers=1):
    ref = ctypes.byref(layer) if isinstance(layer, BlockffnLayer) else layer
    return lib.blockffn_layer_forward(ref, n_layers, x, T, L, gates, masks, preact, um, count, lst, stats, ws,
                                      ws_bytes, y, None)


@cpu_only
def test_layer_forward_rejects_bad_arguments(lib):
    lay = _layer(d=2048, n_experts=64, d_expert=128)
    assert _layer_forward(lib, None) == _capi.ERR_NULL
    assert _layer_forward(lib, lay, n_layers=0) == _capi.ERR_LAYERS
    assert _layer_forward(lib, lay, L=0) == _capi.ERR_CHUNK
    assert _layer_forward(lib, lay, T=12) == _capi.ERR_CHUNK
    for kw in ("x", "gates", "masks", "um", "count", "lst", "y"):
        assert _layer_forward(lib, lay, **{kw: None}) == _capi.ERR_NULL, kw
    assert _layer_forward(lib, lay, ws=None) == _capi.ERR_NULL
    assert _layer_forward(lib, lay, ws=P + 64) == _capi.ERR_ALIGN
    assert _layer_forward(lib, lay, ws_bytes=4096) == _capi.ERR_WORKSPACE
    assert _layer_forward(lib, lay, T=4096, ws_bytes=4096) == _capi.ERR_WORKSPACE   # the separate-call regime
    assert _layer_forward(lib, lay, stats=P + 4) == _capi.ERR_ALIGN
    assert _layer_forward(lib, lay, preact=P + 2) == _capi.ERR_ALIGN
    assert _layer_forward(lib, lay, x=P + 4) == _capi.ERR_ALIGN
    assert _layer_forward(lib, _arr([lay, _layer(d=1024, n_experts=64, d_expert=128)]), n_layers=2) == \
        _capi.ERR_LAYERS
    # no tokens: nothing is read or written
    assert _layer_forward(lib, lay, T=0, x=None, gates=None, masks=None, um=None, count=None, lst=None, stats=None,
                          ws=None, y=None) == _capi.OK


def test_layer_forward_workspace_size(lib):
    lay = _layer(d=2048, n_experts=64, d_expert=128)
    r256 = lambda v: (v + 255) // 256 * 256  # noqa: E731
    # the three-kernel step (at most 64 tokens and 16 chunks, d <= 4096): the router's partial
    # pre-activations [T][E][d/128] fp32, then Swish(W_in x) [T][E][d_e] bf16
    for C, L in ((1, 8), (2, 8), (16, 1), (2, 32)):
        T = C * L
        want = r256(16 * T * 64 * 4) + r256(T * 64 * 128 * 2)
        assert lib.blockffn_layer_forward_workspace_size(ctypes.byref(lay), T, L) == want, (C, L)
    # more tokens, or another shape: the separate calls' AUTO forward workspace
    for T, L, ly in ((4096, 8, lay), (72, 8, lay), (16, 8, _layer(d=2048, n_experts=64, d_expert=128, dtype=0)),
                     (16, 8, _layer(d=2048, n_experts=72, d_expert=128)),
                     (16, 8, _layer(d=8192, n_experts=64, d_expert=128))):
        assert lib.blockffn_layer_forward_workspace_size(ctypes.byref(ly), T, L) == \
            lib.blockffn_workspace_size(ctypes.byref(ly), T, L, _capi.MODE_AUTO), (T, L)
    assert lib.blockffn_layer_forward_workspace_size(ctypes.byref(lay), 12, 8) == 0        # ragged
    assert lib.blockffn_layer_forward_workspace_size(ctypes.byref(_layer(d=100)), 16, 8) == 0


def _grads(**kw):
    f = dict(d_w_router=P, d_b_router=P, d_rms_scale=P, d_w_in=P, d_w_out=P)
    f.update(kw)
    return BlockffnGrads(**f)


def _backward(lib, layer, T=16, x=P, preact=P, dy=P, ws=P, ws_bytes=1 << 40, dx=P, grads=None):
    g = _grads() if grads is None else grads
    return lib.blockffn_backward(ctypes.byref(layer) if layer is not None else None, x, T, preact, dy, None, ws,
                                 ws_bytes, dx, ctypes.byref(g), None)


@cpu_only
def test_backward_validation(lib):
    ok = _layer(d=256, n_experts=16, d_expert=128)
    assert _backward(lib, None) == _capi.ERR_NULL
    assert _backward(lib, _layer(dtype=0)) == _capi.ERR_MODE            # bf16 only
    assert _backward(lib, _layer(d_expert=64)) == _capi.ERR_MODE        # d_expert 128 or 256
    assert _backward(lib, _layer(d=192)) == _capi.ERR_MODE              # d a multiple of 128
    assert _backward(lib, ok, T=-1) == _capi.ERR_SHAPE
    assert _backward(lib, ok, T=1 << 27) == _capi.ERR_SHAPE             # pairs indexed with 32 bits
    assert _backward(lib, ok, T=0, x=None, preact=None, dy=None, ws=None, dx=None) == _capi.OK
    assert _backward(lib, ok, preact=None) == _capi.ERR_NULL
    assert _backward(lib, ok, dx=None) == _capi.ERR_NULL
    assert _backward(lib, ok, grads=_grads(d_w_in=None)) == _capi.ERR_NULL
    assert _backward(lib, ok, dy=P + 4) == _capi.ERR_ALIGN
    assert _backward(lib, ok, grads=_grads(d_w_out=P + 8)) == _capi.ERR_ALIGN
    assert _backward(lib, ok, ws=P + 16) == _capi.ERR_ALIGN
    assert _backward(lib, ok, ws_bytes=4096) == _capi.ERR_WORKSPACE
    assert b"workspace" in lib.blockffn_last_error()


def test_backward_workspace_size(lib):
    lay = _layer(d=4096, n_experts=128, d_expert=128)
    T = 4096
    n = lib.blockffn_backward_workspace_size(ctypes.byref(lay), T)
    P_ = T * 128
    # at least: pair arrays, hidden gradients, partial rows
    need = 3 * 4 * P_ + 2 * (2 * P_ * 128) + 2 * P_ * 4096
    assert n >= need
    # and no copy of a weight (the transposed products read the weights as they lie)
    assert n < need + 2 * 128 * 4096 * 128
    assert lib.blockffn_backward_workspace_size(ctypes.byref(_layer(dtype=0)), T) == 0
    assert lib.blockffn_backward_workspace_size(ctypes.byref(lay), -1) == 0


def _route_with(lib, layer, router=1, top_k=2, T=16, L=8, x=P, gates=P, masks=P):
    return lib.blockffn_route_with(ctypes.byref(layer), 1, x, T, L, router, top_k, gates, masks, None, None)


@cpu_only
def test_route_with_validation(lib):
    ok = _layer()
    assert _route_with(lib, ok, router=3) == _capi.ERR_MODE
    assert _route_with(lib, ok, router=-1) == _capi.ERR_MODE
    assert _route_with(lib, ok, router=1, top_k=0) == _capi.ERR_SHAPE
    assert _route_with(lib, ok, router=1, top_k=17) == _capi.ERR_SHAPE      # E = 16
    assert _route_with(lib, ok, router=1, top_k=2, T=0, x=None, gates=None, masks=None) == _capi.OK
    assert _route_with(lib, ok, router=2, top_k=0, x=None) == _capi.ERR_NULL   # top_k ignored for ReMoE
    assert _route_with(lib, ok, router=1, top_k=2, gates=P + 2) == _capi.ERR_ALIGN


@cpu_only
def test_cls_losses_validation(lib):
    ws_need = lib.blockffn_cls_losses_workspace_size(64, 8)
    assert ws_need >= 8 * 2 * 4
    assert lib.blockffn_cls_losses_workspace_size(63, 8) == 0
    call = lambda **kw: lib.blockffn_cls_losses(*[kw.get(k, v) for k, v in (  # noqa: E731
        ("E", 16), ("z", P), ("T", 64), ("L", 8), ("alpha", ctypes.c_float(10.0)), ("wa", ctypes.c_float(1.0)),
        ("wc", ctypes.c_float(1.0)), ("ws", P), ("nb", 1 << 20), ("loss", P), ("dz", P), ("s", None))])
    assert call(E=0) == _capi.ERR_SHAPE
    assert call(L=7) == _capi.ERR_CHUNK
    assert call(alpha=ctypes.c_float(0.0)) == _capi.ERR_SHAPE
    assert call(wa=ctypes.c_float(float("inf"))) == _capi.ERR_SHAPE
    assert call(loss=None) == _capi.ERR_NULL
    assert call(z=P + 2) == _capi.ERR_ALIGN
    assert call(ws=P + 16) == _capi.ERR_ALIGN
    assert call(nb=8) == _capi.ERR_WORKSPACE


def _fff_layer(**kw):
    v = dict(d=2048, n_trees=64, depth=6, dtype=_capi.BF16, activation=0, node_stride=0,
             w_node=P, b_node=P, w_out=P)
    v.update(kw)
    return BlockffnFffLayer(**v)


@cpu_only
def test_fff_forward_validation(lib):
    def call(layer=None, n_layers=1, x=P, T=4, mode=0, split=1, paths=None, pre=None, ws=None, nb=0, y=P):
        ly = _fff_layer() if layer is None else layer
        ref = ctypes.byref(ly) if isinstance(ly, BlockffnFffLayer) else ly
        return lib.blockffn_fff_forward(ref, n_layers, x, T, mode, split, paths, pre, ws, nb, y, None)

    assert lib.blockffn_fff_forward(None, 1, P, 4, 0, 1, None, None, None, 0, P, None) == _capi.ERR_NULL
    assert call(_fff_layer(dtype=2)) == _capi.ERR_DTYPE
    for d in (0, 256, 2048 + 64, 4608):       # bf16: multiples of 512 up to 4096
        assert call(_fff_layer(d=d)) == _capi.ERR_SHAPE, d
    assert call(_fff_layer(d=256, dtype=_capi.F32), T=0, x=None, y=None) == _capi.OK
    assert call(_fff_layer(d=4096, dtype=_capi.F32)) == _capi.ERR_SHAPE   # f32: up to 2048
    assert call(_fff_layer(n_trees=0)) == _capi.ERR_SHAPE
    assert call(_fff_layer(depth=-1)) == _capi.ERR_SHAPE
    assert call(_fff_layer(depth=16)) == _capi.ERR_SHAPE
    assert call(_fff_layer(activation=2)) == _capi.ERR_SHAPE
    assert call(_fff_layer(node_stride=2048)) == _capi.ERR_SHAPE         # shorter than a bf16 row of 2048
    assert call(_fff_layer(node_stride=4096 + 8)) == _capi.ERR_SHAPE     # not a multiple of 16
    assert call(_fff_layer(node_stride=8192), T=0, x=None, y=None) == _capi.OK   # interleaved rows
    assert call(mode=2) == _capi.ERR_MODE
    assert call(mode=1, paths=P) == _capi.ERR_MODE
    assert call(mode=1, pre=P) == _capi.ERR_MODE
    assert call(n_layers=0) == _capi.ERR_LAYERS
    arr = lambda *ls: (BlockffnFffLayer * len(ls))(*ls)  # noqa: E731
    M = 1 << 26
    assert call(arr(_fff_layer(), _fff_layer(w_node=P + M, b_node=P + M, w_out=P + M)), n_layers=2,
                x=None) == _capi.ERR_NULL                             # a valid array
    assert call(arr(_fff_layer(), _fff_layer(depth=5)), n_layers=2) == _capi.ERR_LAYERS
    assert call(arr(_fff_layer(), _fff_layer(node_stride=8192)), n_layers=2) == _capi.ERR_LAYERS
    assert call(arr(_fff_layer(), _fff_layer(activation=1)), n_layers=2) == _capi.ERR_LAYERS
    assert call(arr(_fff_layer(), _fff_layer(w_out=P + 8)), n_layers=2) == _capi.ERR_ALIGN
    many = arr(*[_fff_layer(w_node=P + M * (l * l + 1), w_out=P + M * (l * l + 2)) for l in range(33)])
    assert call(many, n_layers=33) == _capi.ERR_LAYERS                 # 33 scattered layers
    assert call(T=-1) == _capi.ERR_SHAPE
    assert call(T=1 << 31) == _capi.ERR_SHAPE
    assert call(_fff_layer(w_node=None)) == _capi.ERR_NULL
    assert call(x=None) == _capi.ERR_NULL
    assert call(y=None) == _capi.ERR_NULL
    assert call(x=P + 8) == _capi.ERR_ALIGN
    assert call(_fff_layer(w_out=P + 8)) == _capi.ERR_ALIGN
    assert call(_fff_layer(b_node=P + 2)) == _capi.ERR_ALIGN
    assert call(paths=P + 2) == _capi.ERR_ALIGN
    # blocks per token: 0 (automatic) .. ceil(P / 4) = 16
    assert call(split=-1) == _capi.ERR_SHAPE
    assert call(split=17) == _capi.ERR_SHAPE
    need = 4 * 2 * 2048 * 4                                              # T x G x d fp32 partials
    assert call(split=2) == _capi.ERR_WORKSPACE
    assert call(split=2, ws=P, nb=need - 16) == _capi.ERR_WORKSPACE
    assert call(split=2, ws=P + 8, nb=need) == _capi.ERR_ALIGN
    # a valid call with no tokens enqueues nothing
    assert call(T=0, x=None, y=None) == _capi.OK
    assert call(T=0, x=None, y=None, mode=1) == _capi.OK
    assert call(T=0, x=None, y=None, split=0) == _capi.OK


def test_fff_workspace_size(lib):
    ly = _fff_layer()
    size = lambda T, split: lib.blockffn_fff_workspace_size(ctypes.byref(ly), T, split)  # noqa: E731
    assert size(4096, 0) == 0                       # enough tokens: one block per token
    assert size(64, 1) == 0
    assert size(64, 0) == 64 * 16 * 2048 * 4        # a token's 64 trees over 16 blocks
    assert size(1000, 0) == 1000 * 4 * 2048 * 4     # ceil(3072 / 1000) = 4 blocks per token
    assert size(64, 3) == 64 * 3 * 2048 * 4
    assert size(64, 17) == 0                        # invalid split
    assert lib.blockffn_fff_workspace_size(ctypes.byref(_fff_layer(d=100)), 64, 0) == 0


@cpu_only
def test_read_probe_validation(lib):
    assert lib.blockffn_read_probe(P, 1 << 20, 0, None, None) == _capi.ERR_NULL
    assert lib.blockffn_read_probe(None, 1 << 20, 0, P, None) == _capi.ERR_NULL
    assert lib.blockffn_read_probe(P + 8, 1 << 20, 0, P, None) == _capi.ERR_ALIGN
    assert lib.blockffn_read_probe(P, (1 << 20) + 4, 0, P, None) == _capi.ERR_ALIGN
    assert lib.blockffn_read_probe(P, 1 << 20, -1, P, None) == _capi.ERR_SHAPE
    assert lib.blockffn_read_probe(P, 0, 0, P, None) == _capi.OK     # nothing to read
