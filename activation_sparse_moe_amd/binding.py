"""Python binding of libblockffn with the C ABI's names.

PyTorch supplies device memory and streams only; each function marshals its
arguments into one call of the C ABI, which enqueues HIP kernels on the
current torch stream (or the stream given).  Output tensors are allocated
here when the caller passes none.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np
import torch

from . import _capi
from ._capi import BF16, F32, MODES, ROUTERS, BlockffnFffLayer, BlockffnGrads, BlockffnLayer, check, load

_ALIGN = 256
_STATS_WORDS = 8 + 129


def _torch_dtype(dtype: int) -> torch.dtype:
    return torch.float32 if dtype == F32 else torch.bfloat16


def _elem(dtype: int) -> int:
    return 4 if dtype == F32 else 2


def _round(v: int, a: int = _ALIGN) -> int:
    return (v + a - 1) // a * a


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _to_device(a, dtype: int, device) -> torch.Tensor:
    """numpy float32 / uint16-bf16-bits (or a torch tensor) -> device tensor of the layer dtype."""
    if isinstance(a, torch.Tensor):
        return a.to(device=device, dtype=_torch_dtype(dtype)).contiguous()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        assert dtype == BF16, "bf16 bit patterns given for an fp32 layer"
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    assert a.dtype == np.float32, f"expected float32 or uint16 bf16 bits, got {a.dtype}"
    return torch.from_numpy(a).to(device=device, dtype=_torch_dtype(dtype))


class DeviceLayer:
    """`replicas` copies of one BlockFFN layer in a single device buffer.

    Every copy has the same internal layout, so copy r's tensors sit at
    replica 0's addresses plus r * stride bytes.  Passed to a call, the
    copies become an array of layer descriptors (chunk c uses copy
    c % n_layers), which the library recognises as evenly spaced.  The copies
    are distinct memory, so a stack of them streams from HBM like a stack of
    distinct layers.  A list of DeviceLayer objects (each in its own
    allocation) may be passed wherever one DeviceLayer is accepted.
    """

    def __init__(self, d: int, n_experts: int, d_expert: int, dtype: int, rms_eps: float = 1e-6,
                 device="cuda", replicas: int = 1, has_bias: bool = True, has_scale: bool = False):
        assert dtype in (F32, BF16)
        self.d, self.n_experts, self.d_expert, self.dtype = d, n_experts, d_expert, dtype
        self.rms_eps, self.replicas, self.device = float(rms_eps), int(replicas), torch.device(device)
        es = _elem(dtype)
        E, de = n_experts, d_expert
        sizes = [("w_router", E * d * es), ("b_router", 4 * E if has_bias else 0),
                 ("rms_scale", 4 * E if has_scale else 0), ("w_in", E * de * d * es), ("w_out", E * d * de * es)]
        self._off = {}
        off = 0
        for name, nbytes in sizes:
            self._off[name] = (off, nbytes) if nbytes else None
            off = _round(off + nbytes)
        self.stride = _round(off, 4096)
        self.buffer = torch.empty(self.stride * self.replicas, dtype=torch.uint8, device=self.device)

    # views into copy r
    def _view(self, name: str, r: int, shape, dtype: torch.dtype) -> Optional[torch.Tensor]:
        slot = self._off[name]
        if slot is None:
            return None
        off, nbytes = slot
        base = r * self.stride + off
        return self.buffer[base:base + nbytes].view(dtype).view(*shape)

    def tensors(self, r: int = 0) -> dict:
        if getattr(self, "_own", None) is not None:  # a layer made from the caller's tensors
            assert r == 0, "a layer made from separate tensors has one copy"
            return dict(self._own)
        td = _torch_dtype(self.dtype)
        E, d, de = self.n_experts, self.d, self.d_expert
        return dict(w_router=self._view("w_router", r, (E, d), td),
                    b_router=self._view("b_router", r, (E,), torch.float32),
                    rms_scale=self._view("rms_scale", r, (E,), torch.float32),
                    w_in=self._view("w_in", r, (E, de, d), td),
                    w_out=self._view("w_out", r, (E, d, de), td))

    @classmethod
    def from_arrays(cls, w_router, b_router, rms_scale, w_in, w_out, dtype: int, rms_eps: float = 1e-6,
                    device="cuda", replicas: int = 1) -> "DeviceLayer":
        E, d = w_router.shape
        de = w_in.shape[1]
        self = cls(d, E, de, dtype, rms_eps, device, replicas, has_bias=b_router is not None,
                   has_scale=rms_scale is not None)
        t = self.tensors(0)
        t["w_router"].copy_(_to_device(w_router, dtype, self.device))
        t["w_in"].copy_(_to_device(w_in, dtype, self.device))
        t["w_out"].copy_(_to_device(w_out, dtype, self.device))
        if b_router is not None:
            t["b_router"].copy_(torch.as_tensor(np.asarray(b_router, np.float32)).to(self.device))
        if rms_scale is not None:
            t["rms_scale"].copy_(torch.as_tensor(np.asarray(rms_scale, np.float32)).to(self.device))
        for r in range(1, replicas):
            self.buffer[r * self.stride:(r + 1) * self.stride].copy_(self.buffer[:self.stride])
        return self

    @classmethod
    def from_tensors(cls, w_router: torch.Tensor, w_in: torch.Tensor, w_out: torch.Tensor,
                     b_router: Optional[torch.Tensor] = None, rms_scale: Optional[torch.Tensor] = None,
                     rms_eps: float = 1e-6) -> "DeviceLayer":
        """A layer over existing device tensors (each may be its own allocation, as a model's
        parameters are); nothing is copied and the tensors must outlive the layer's use."""
        E, d = w_router.shape
        de = w_in.shape[1]
        assert w_router.dtype == w_in.dtype == w_out.dtype and w_router.dtype in (torch.float32, torch.bfloat16)
        assert w_in.shape == (E, de, d) and w_out.shape == (E, d, de)
        for t in (w_router, w_in, w_out, b_router, rms_scale):
            assert t is None or (t.is_contiguous() and t.device == w_router.device)
        self = cls.__new__(cls)
        self.d, self.n_experts, self.d_expert = d, E, de
        self.dtype = F32 if w_router.dtype == torch.float32 else BF16
        self.rms_eps, self.replicas, self.device = float(rms_eps), 1, w_router.device
        self.stride, self.buffer, self._off = 0, None, None
        self._own = dict(w_router=w_router, b_router=b_router, rms_scale=rms_scale, w_in=w_in, w_out=w_out)
        return self

    @classmethod
    def from_workload(cls, layer, device="cuda", replicas: int = 1) -> "DeviceLayer":
        return cls.from_arrays(layer.w_router, layer.b_router, layer.rms_scale, layer.w_in, layer.w_out,
                               F32 if layer.dtype == "f32" else BF16, layer.rms_eps, device, replicas)

    def descriptor(self) -> BlockffnLayer:
        # the buffer never moves, so the descriptor is built once
        if getattr(self, "_desc", None) is not None:
            return self._desc
        t = self.tensors(0)
        self._desc = BlockffnLayer(self.d, self.n_experts, self.d_expert, self.dtype, self.rms_eps, 0,
                                   t["w_router"].data_ptr(),
                                   t["b_router"].data_ptr() if t["b_router"] is not None else None,
                                   t["rms_scale"].data_ptr() if t["rms_scale"] is not None else None,
                                   t["w_in"].data_ptr(), t["w_out"].data_ptr())
        return self._desc

    def descriptors(self, n: int):
        """ctypes array of n descriptors: copy l % replicas for l < n (built once per n)."""
        cache = self.__dict__.setdefault("_descs", {})
        if n not in cache:
            base = self.descriptor()
            arr = (BlockffnLayer * n)()
            for l in range(n):
                off = (l % self.replicas) * self.stride
                arr[l] = BlockffnLayer(self.d, self.n_experts, self.d_expert, self.dtype, self.rms_eps, 0,
                                       base.w_router + off, base.b_router + off if base.b_router else None,
                                       base.rms_scale + off if base.rms_scale else None, base.w_in + off,
                                       base.w_out + off)
            cache[n] = arr
        return cache[n]

    @property
    def mask_words(self) -> int:
        return (self.n_experts + 63) // 64

    def single_copy(self, r: int) -> "DeviceLayer":
        """A view of copy r alone (n_layers 1), sharing this buffer: for calls that
        should read one particular copy."""
        import copy as _copy
        v = _copy.copy(self)
        v.__dict__.pop("_descs", None)
        base = self.descriptor()
        off = r * self.stride
        v._desc = BlockffnLayer(self.d, self.n_experts, self.d_expert, self.dtype, self.rms_eps, 0,
                                base.w_router + off, base.b_router + off if base.b_router else None,
                                base.rms_scale + off if base.rms_scale else None, base.w_in + off, base.w_out + off)
        v.replicas = 1
        return v


def tokens_to_device(x, dtype: int, device="cuda") -> torch.Tensor:
    return _to_device(x, dtype, device)


def _layers(layer, n_layers: Optional[int]):
    """(first DeviceLayer, ctypes descriptor array, count) for a call: a DeviceLayer's copies (all of them
    unless n_layers says how many), or one descriptor per DeviceLayer of a sequence (each its copy 0)."""
    if isinstance(layer, (list, tuple)):
        assert n_layers is None or n_layers == len(layer), "n_layers must match the sequence length"
        arr = (BlockffnLayer * len(layer))(*[ly.descriptor() for ly in layer])
        return layer[0], arr, len(layer)
    n = layer.replicas if n_layers is None else int(n_layers)
    if n < 1:  # passed through so that the library reports it
        return layer, ctypes.pointer(layer.descriptor()), n
    return layer, layer.descriptors(n), n


def blockffn_route(layer: DeviceLayer, x: torch.Tensor, chunk_len: int, n_layers: Optional[int] = None,
                   gates: Optional[torch.Tensor] = None, token_masks: Optional[torch.Tensor] = None,
                   preact: Optional[torch.Tensor] = None, want_preact: bool = False, stream=None):
    """Router (ReLU + RMSNorm) -> (gates [T][E] f32, token_masks [T][W] int64 bit patterns, preact or None)."""
    T = x.shape[0]
    layer, descs, nl = _layers(layer, n_layers)
    E = layer.n_experts
    if gates is None:
        gates = torch.empty((T, E), dtype=torch.float32, device=x.device)
    if token_masks is None:
        token_masks = torch.empty((T, layer.mask_words), dtype=torch.int64, device=x.device)
    if want_preact and preact is None:
        preact = torch.empty((T, E), dtype=torch.float32, device=x.device)
    check(load().blockffn_route(descs, nl, _ptr(x), T, chunk_len, _ptr(gates), _ptr(token_masks),
                                _ptr(preact), _stream(stream)), "blockffn_route")
    return gates, token_masks, preact


def blockffn_route_with(layer: DeviceLayer, x: torch.Tensor, chunk_len: int, router="blockffn", top_k: int = 0,
                        n_layers: Optional[int] = None, gates: Optional[torch.Tensor] = None,
                        token_masks: Optional[torch.Tensor] = None, preact: Optional[torch.Tensor] = None,
                        want_preact: bool = False, stream=None):
    """Router with a selectable gate function ("blockffn", "topk_softmax" with top_k, "relu_sum")."""
    T = x.shape[0]
    layer, descs, nl = _layers(layer, n_layers)
    E = layer.n_experts
    kind = ROUTERS[router] if isinstance(router, str) else int(router)
    if gates is None:
        gates = torch.empty((T, E), dtype=torch.float32, device=x.device)
    if token_masks is None:
        token_masks = torch.empty((T, layer.mask_words), dtype=torch.int64, device=x.device)
    if want_preact and preact is None:
        preact = torch.empty((T, E), dtype=torch.float32, device=x.device)
    check(load().blockffn_route_with(descs, nl, _ptr(x), T, chunk_len, kind, top_k, _ptr(gates),
                                     _ptr(token_masks), _ptr(preact), _stream(stream)), "blockffn_route_with")
    return gates, token_masks, preact


def blockffn_chunk_union(n_experts: int, token_masks: torch.Tensor, chunk_len: int,
                         chunk_masks: Optional[torch.Tensor] = None, active_count: Optional[torch.Tensor] = None,
                         active_list: Optional[torch.Tensor] = None, stream=None):
    """Chunk union -> (chunk_masks [C][W] int64, active_count [C] int32, active_list [C][E] int32)."""
    T, W = token_masks.shape
    C = T // chunk_len if chunk_len > 0 else 0
    dev = token_masks.device
    if chunk_masks is None:
        chunk_masks = torch.empty((C, W), dtype=torch.int64, device=dev)
    if active_count is None:
        active_count = torch.empty((C,), dtype=torch.int32, device=dev)
    if active_list is None:
        active_list = torch.empty((C, n_experts), dtype=torch.int32, device=dev)
    check(load().blockffn_chunk_union(n_experts, _ptr(token_masks), T, chunk_len, _ptr(chunk_masks),
                                      _ptr(active_count), _ptr(active_list), _stream(stream)),
          "blockffn_chunk_union")
    return chunk_masks, active_count, active_list


def blockffn_workspace_size(layer: DeviceLayer, n_tokens: int, chunk_len: int, mode="auto") -> int:
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    if isinstance(layer, (list, tuple)):
        layer = layer[0]
    desc = layer.descriptor()
    return int(load().blockffn_workspace_size(ctypes.byref(desc), n_tokens, chunk_len, m))


def alloc_workspace(layer: DeviceLayer, n_tokens: int, chunk_len: int, mode="auto") -> torch.Tensor:
    if isinstance(layer, (list, tuple)):
        layer = layer[0]
    nbytes = blockffn_workspace_size(layer, n_tokens, chunk_len, mode)
    # torch's caching allocator returns 256-byte aligned blocks
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=layer.device)


def blockffn_forward(layer: DeviceLayer, x: torch.Tensor, chunk_len: int, gates: torch.Tensor,
                     active_count: Optional[torch.Tensor], active_list: Optional[torch.Tensor], mode="auto",
                     n_layers: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
                     y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Expert evaluation over each chunk's union -> y [T][d] fp32."""
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    T = x.shape[0]
    layer, descs, nl = _layers(layer, n_layers)
    if y is None:
        y = torch.empty((T, layer.d), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(layer, T, chunk_len, m)
    check(load().blockffn_forward(descs, nl, _ptr(x), T, chunk_len, _ptr(gates), _ptr(active_count),
                                  _ptr(active_list), m, _ptr(workspace), workspace.numel(), _ptr(y),
                                  _stream(stream)), "blockffn_forward")
    return y


def blockffn_forward_noalloc(layer: DeviceLayer, x: torch.Tensor, chunk_len: int, gates: torch.Tensor,
                             active_count: Optional[torch.Tensor], active_list: Optional[torch.Tensor], mode="auto",
                             n_layers: Optional[int] = None, y: Optional[torch.Tensor] = None,
                             stream=None) -> torch.Tensor:
    """blockffn_forward with the library's static scratch array instead of a workspace -> y [T][d] fp32.
    Allocates y here only when none is given."""
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    T = x.shape[0]
    layer, descs, nl = _layers(layer, n_layers)
    if y is None:
        y = torch.empty((T, layer.d), dtype=torch.float32, device=x.device)
    check(load().blockffn_forward_noalloc(descs, nl, _ptr(x), T, chunk_len, _ptr(gates), _ptr(active_count),
                                          _ptr(active_list), m, _ptr(y), _stream(stream)),
          "blockffn_forward_noalloc")
    return y


def blockffn_layer_forward_workspace_size(layer: DeviceLayer, n_tokens: int, chunk_len: int) -> int:
    if isinstance(layer, (list, tuple)):
        layer = layer[0]
    desc = layer.descriptor()
    return int(load().blockffn_layer_forward_workspace_size(ctypes.byref(desc), n_tokens, chunk_len))


def alloc_layer_forward(layer: DeviceLayer, n_tokens: int, chunk_len: int, want_preact: bool = False,
                        want_stats: bool = True, device=None) -> dict:
    """Output buffers and workspace of blockffn_layer_forward, for reuse across calls."""
    if isinstance(layer, (list, tuple)):
        layer = layer[0]
    dev = layer.device if device is None else device
    T, E, W = n_tokens, layer.n_experts, layer.mask_words
    C = T // chunk_len if chunk_len > 0 else 0
    nbytes = blockffn_layer_forward_workspace_size(layer, T, chunk_len)
    return {
        "gates": torch.empty((T, E), dtype=torch.float32, device=dev),
        "token_masks": torch.empty((T, W), dtype=torch.int64, device=dev),
        "preact": torch.empty((T, E), dtype=torch.float32, device=dev) if want_preact else None,
        "chunk_masks": torch.empty((C, W), dtype=torch.int64, device=dev),
        "active_count": torch.empty((C,), dtype=torch.int32, device=dev),
        "active_list": torch.empty((C, E), dtype=torch.int32, device=dev),
        "stats": torch.empty((_STATS_WORDS,), dtype=torch.int64, device=dev) if want_stats else None,
        "workspace": torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev),
        "y": torch.empty((T, layer.d), dtype=torch.float32, device=dev),
    }


def blockffn_layer_forward(layer: DeviceLayer, x: torch.Tensor, chunk_len: int, n_layers: Optional[int] = None,
                           out: Optional[dict] = None, want_preact: bool = False, want_stats: bool = True,
                           stream=None) -> dict:
    """Router, chunk union, forward and statistics in one call -> the dict of alloc_layer_forward, filled."""
    T = x.shape[0]
    layer, descs, nl = _layers(layer, n_layers)
    if out is None:
        out = alloc_layer_forward(layer, T, chunk_len, want_preact, want_stats, x.device)
    ws = out["workspace"]
    check(load().blockffn_layer_forward(descs, nl, _ptr(x), T, chunk_len, _ptr(out["gates"]),
                                        _ptr(out["token_masks"]), _ptr(out["preact"]), _ptr(out["chunk_masks"]),
                                        _ptr(out["active_count"]), _ptr(out["active_list"]), _ptr(out["stats"]),
                                        _ptr(ws), ws.numel(), _ptr(out["y"]), _stream(stream)),
          "blockffn_layer_forward")
    return out


def blockffn_backward_workspace_size(layer: DeviceLayer, n_tokens: int) -> int:
    desc = layer.descriptor()
    return int(load().blockffn_backward_workspace_size(ctypes.byref(desc), n_tokens))


def alloc_backward_workspace(layer: DeviceLayer, n_tokens: int) -> torch.Tensor:
    nbytes = blockffn_backward_workspace_size(layer, n_tokens)
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=layer.device)


def blockffn_backward(layer: DeviceLayer, x: torch.Tensor, preact: torch.Tensor, dy: torch.Tensor,
                      workspace: Optional[torch.Tensor] = None, dx: Optional[torch.Tensor] = None,
                      grads: Optional[dict] = None, dz_extra: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Layer backward -> dict(dx, d_w_router, d_b_router, d_rms_scale, d_w_in, d_w_out), all fp32."""
    T = x.shape[0]
    E, d, de = layer.n_experts, layer.d, layer.d_expert
    dev = x.device
    if dx is None:
        dx = torch.empty((T, d), dtype=torch.float32, device=dev)
    if grads is None:
        grads = dict(d_w_router=torch.empty((E, d), dtype=torch.float32, device=dev),
                     d_b_router=torch.empty((E,), dtype=torch.float32, device=dev),
                     d_rms_scale=torch.empty((E,), dtype=torch.float32, device=dev),
                     d_w_in=torch.empty((E, de, d), dtype=torch.float32, device=dev),
                     d_w_out=torch.empty((E, d, de), dtype=torch.float32, device=dev))
    if workspace is None:
        workspace = alloc_backward_workspace(layer, T)
    g = BlockffnGrads(*[grads[k].data_ptr() for k in ("d_w_router", "d_b_router", "d_rms_scale", "d_w_in",
                                                       "d_w_out")])
    desc = layer.descriptor()
    check(load().blockffn_backward(ctypes.byref(desc), _ptr(x), T, _ptr(preact), _ptr(dy), _ptr(dz_extra),
                                   _ptr(workspace),
                                   workspace.numel(), _ptr(dx), ctypes.byref(g), _stream(stream)),
          "blockffn_backward")
    return dict(dx=dx, **grads)


def blockffn_cls_losses(n_experts: int, preact: torch.Tensor, chunk_len: int, alpha: float, w_locality: float = 1.0,
                        w_chunk: float = 1.0, want_grad: bool = True, losses: Optional[torch.Tensor] = None,
                        dz: Optional[torch.Tensor] = None, stream=None):
    """CLS-aware objectives -> (losses [2] fp32 device tensor, dz [T][E] fp32 or None)."""
    T = preact.shape[0]
    dev = preact.device
    if losses is None:
        losses = torch.empty((2,), dtype=torch.float32, device=dev)
    if want_grad and dz is None:
        dz = torch.empty((T, n_experts), dtype=torch.float32, device=dev)
    lib = load()
    nbytes = int(lib.blockffn_cls_losses_workspace_size(T, chunk_len))
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    check(lib.blockffn_cls_losses(n_experts, _ptr(preact), T, chunk_len, float(alpha), float(w_locality),
                                  float(w_chunk), _ptr(ws), ws.numel(), _ptr(losses), _ptr(dz), _stream(stream)),
          "blockffn_cls_losses")
    return losses, dz


def blockffn_sparsity_stats(n_experts: int, token_masks: torch.Tensor, chunk_len: int,
                            stats_dev: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Sparsity statistics into a device int64 tensor laid out as blockffn_stats."""
    if stats_dev is None:
        stats_dev = torch.empty((_STATS_WORDS,), dtype=torch.int64, device=token_masks.device)
    T = token_masks.shape[0]
    check(load().blockffn_sparsity_stats(n_experts, _ptr(token_masks), T, chunk_len, _ptr(stats_dev),
                                         _stream(stream)), "blockffn_sparsity_stats")
    return stats_dev


def stats_dict(stats_dev: torch.Tensor) -> dict:
    v = stats_dev.cpu().numpy()
    keys = ("n_tokens", "n_chunks", "n_experts", "chunk_len", "active_pairs", "union_sum", "reuse_num", "reuse_den")
    out = {k: int(v[i]) for i, k in enumerate(keys)}
    E = out["n_experts"]
    out["hist"] = v[8:8 + E + 1].astype(np.int64)
    T, C = out["n_tokens"], out["n_chunks"]
    out["tls"] = 1.0 - out["active_pairs"] / (T * E) if T else 0.0
    out["cls"] = 1.0 - out["union_sum"] / (C * E) if C else 0.0
    out["reuse"] = out["reuse_num"] / out["reuse_den"] if out["reuse_den"] else 0.0
    return out


def masks_to_u64(token_masks: torch.Tensor) -> np.ndarray:
    return token_masks.cpu().numpy().view(np.uint64)


class DeviceFffLayer:
    """`replicas` copies of one FFF tree layer in a single device buffer.

    Copy r holds the node rows, then b_node [P][N] (fp32, optional), at
    replica 0's offsets plus r * stride bytes.  Passed to a call, the copies
    become an array of descriptors (token t uses copy t % n_layers), which
    the library recognises as evenly spaced.  With
    `interleave` (the default) each node's input and output rows sit next to
    each other, [P][N][2][d], so a visited node is one contiguous read;
    otherwise w_node [P][N][d] and w_out [P][N][d] are separate arrays."""

    def __init__(self, d: int, n_trees: int, depth: int, dtype: int, post: bool = False, device="cuda",
                 replicas: int = 1, has_bias: bool = True, interleave: bool = True):
        assert dtype in (F32, BF16)
        self.d, self.n_trees, self.depth, self.dtype = d, n_trees, depth, dtype
        self.post, self.replicas, self.device = bool(post), int(replicas), torch.device(device)
        self.interleave = bool(interleave)
        self.nodes = (1 << (depth + 1)) - 1
        self.rows = n_trees * self.nodes
        self.row_bytes = d * _elem(dtype)
        self.node_stride = 2 * self.row_bytes if self.interleave else self.row_bytes
        nb = self.rows * self.row_bytes
        if self.interleave:
            self._w_node_off, self._w_out_off = 0, self.row_bytes
            off = _round(2 * nb)
        else:
            self._w_node_off, self._w_out_off = 0, _round(nb)
            off = _round(self._w_out_off + nb)
        self._b_off = off if has_bias else None
        off = _round(off + (4 * self.rows if has_bias else 0))
        self.stride = _round(off, 4096)
        self.buffer = torch.empty(self.stride * self.replicas, dtype=torch.uint8, device=self.device)
        self._base = 0  # byte offset of copy 0 in the buffer (non-zero for single_copy views)
        self._desc = None

    def rows_view(self, which: str, r: int = 0, n_copies: int = 1) -> torch.Tensor:
        """[n_copies][P N][d] view of the input ("w_node") or output ("w_out") rows of copies r.."""
        td = _torch_dtype(self.dtype)
        es = _elem(self.dtype)
        flat = self.buffer.view(td)
        off = self._base + r * self.stride + (self._w_node_off if which == "w_node" else self._w_out_off)
        return flat.as_strided((n_copies, self.rows, self.d), (self.stride // es, self.node_stride // es, 1), off // es)

    def tensors(self, r: int = 0) -> dict:
        P, N, d = self.n_trees, self.nodes, self.d
        b = None
        if self._b_off is not None:
            base = self._base + r * self.stride + self._b_off
            b = self.buffer[base:base + 4 * self.rows].view(torch.float32).view(P, N)
        return dict(w_node=self.rows_view("w_node", r)[0].view(P, N, d) if not self.interleave
                    else self.rows_view("w_node", r)[0].unflatten(0, (P, N)),
                    b_node=b,
                    w_out=self.rows_view("w_out", r)[0].view(P, N, d) if not self.interleave
                    else self.rows_view("w_out", r)[0].unflatten(0, (P, N)))

    @classmethod
    def from_workload(cls, layer, post: bool = False, device="cuda", replicas: int = 1,
                      interleave: bool = True) -> "DeviceFffLayer":
        dtype = F32 if layer.dtype == "f32" else BF16
        self = cls(layer.d, layer.n_trees, layer.depth, dtype, post, device, replicas,
                   has_bias=layer.b_node is not None, interleave=interleave)
        self.fill(0, layer)
        for r in range(1, self.replicas):
            self.buffer[r * self.stride:(r + 1) * self.stride].copy_(self.buffer[:self.stride])
        return self

    def fill(self, r: int, layer) -> None:
        """Write a host layer (workload.FffLayer) into copy r."""
        t = self.tensors(r)
        t["w_node"].copy_(_to_device(layer.w_node, self.dtype, self.device))
        t["w_out"].copy_(_to_device(layer.w_out, self.dtype, self.device))
        if layer.b_node is not None:
            t["b_node"].copy_(torch.as_tensor(np.asarray(layer.b_node, np.float32)).to(self.device))

    def single_copy(self, r: int) -> "DeviceFffLayer":
        """A view of copy r alone (n_layers 1), sharing this buffer."""
        import copy as _copy
        v = _copy.copy(self)
        v._desc = None
        v.__dict__.pop("_descs", None)
        v._base = self._base + r * self.stride
        v.replicas = 1
        return v

    def descriptor(self) -> BlockffnFffLayer:
        if self._desc is None:
            base = self.buffer.data_ptr() + self._base
            self._desc = BlockffnFffLayer(self.d, self.n_trees, self.depth, self.dtype,
                                          _capi.FFF_GELU_OUTPUT if self.post else _capi.FFF_GELU_NODES,
                                          self.node_stride, base + self._w_node_off,
                                          base + self._b_off if self._b_off is not None else None,
                                          base + self._w_out_off)
        return self._desc

    def descriptors(self, n: int):
        """ctypes array of n descriptors: copy l % replicas for l < n (built once per n)."""
        cache = self.__dict__.setdefault("_descs", {})
        if n not in cache:
            b = self.descriptor()
            arr = (BlockffnFffLayer * n)()
            for l in range(n):
                off = (l % self.replicas) * self.stride
                arr[l] = BlockffnFffLayer(b.d, b.n_trees, b.depth, b.dtype, b.activation, b.node_stride,
                                          b.w_node + off, b.b_node + off if b.b_node else None, b.w_out + off)
            cache[n] = arr
        return cache[n]


def blockffn_fff_workspace_size(layer: DeviceFffLayer, n_tokens: int, split: int = 0) -> int:
    return int(load().blockffn_fff_workspace_size(ctypes.byref(layer.descriptor()), n_tokens, int(split)))


def alloc_fff_workspace(layer: DeviceFffLayer, n_tokens: int, split: int = 0) -> Optional[torch.Tensor]:
    nbytes = blockffn_fff_workspace_size(layer, n_tokens, split)
    return torch.empty(nbytes, dtype=torch.uint8, device=layer.device) if nbytes else None


def blockffn_fff_forward(layer: DeviceFffLayer, x: torch.Tensor, mode: str = "sparse", want_paths: bool = False,
                         split: int = 0, workspace: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                         paths: Optional[torch.Tensor] = None, node_preact: Optional[torch.Tensor] = None,
                         n_layers: Optional[int] = None, stream=None):
    """FFF tree layer -> (y [T][d] f32, paths [T][P][D+1] i32 or None, node_preact [T][P][D+1] f32 or None).
    A workspace is allocated here when the call needs one and none is given."""
    T = x.shape[0]
    if isinstance(layer, (list, tuple)):
        assert n_layers is None or n_layers == len(layer), "n_layers must match the sequence length"
        descs, nl = (BlockffnFffLayer * len(layer))(*[ly.descriptor() for ly in layer]), len(layer)
        layer = layer[0]
    else:
        nl = layer.replicas if n_layers is None else int(n_layers)
        descs = layer.descriptors(nl) if nl >= 1 else ctypes.pointer(layer.descriptor())
    if y is None:
        y = torch.empty((T, layer.d), dtype=torch.float32, device=x.device)
    if want_paths and paths is None:
        paths = torch.empty((T, layer.n_trees, layer.depth + 1), dtype=torch.int32, device=x.device)
    if want_paths and node_preact is None:
        node_preact = torch.empty((T, layer.n_trees, layer.depth + 1), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = alloc_fff_workspace(layer, T, split)
    m = {"sparse": _capi.FFF_SPARSE, "dense": _capi.FFF_DENSE}[mode]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(load().blockffn_fff_forward(descs, nl, _ptr(x), T, m, int(split), _ptr(paths),
                                      _ptr(node_preact), _ptr(workspace), ws_bytes, _ptr(y), _stream(stream)),
          "blockffn_fff_forward")
    return y, paths, node_preact


def blockffn_read_probe(buf: torch.Tensor, sink: torch.Tensor, blocks: int = 0, stream=None) -> None:
    """One streaming read of `buf` (the HBM read-ceiling probe)."""
    check(load().blockffn_read_probe(_ptr(buf), buf.numel() * buf.element_size(), int(blocks), _ptr(sink),
                                     _stream(stream)), "blockffn_read_probe")
