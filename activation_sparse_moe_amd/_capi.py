"""ctypes declarations of libblockffn's C ABI (include/blockffn.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Loading fails loudly if the library has not been built; there is no
fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libblockffn.so")

F32, BF16 = 0, 1
MODE_AUTO, MODE_GEMV, MODE_CHUNK_MFMA, MODE_GROUPED, MODE_DENSE, MODE_CHUNK_SPLIT = 0, 1, 2, 3, 4, 5
ROUTER_BLOCKFFN, ROUTER_TOPK_SOFTMAX, ROUTER_RELU_SUM = 0, 1, 2
ROUTERS = {"blockffn": ROUTER_BLOCKFFN, "topk_softmax": ROUTER_TOPK_SOFTMAX, "relu_sum": ROUTER_RELU_SUM}
MODES = {"auto": MODE_AUTO, "gemv": MODE_GEMV, "chunk_mfma": MODE_CHUNK_MFMA, "chunk_split": MODE_CHUNK_SPLIT,
         "grouped": MODE_GROUPED,
         "dense": MODE_DENSE}

OK = 0
ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_CHUNK, ERR_WORKSPACE = -1, -2, -3, -4, -5
ERR_MODE, ERR_ALIGN, ERR_LAYERS, ERR_HIP = -6, -7, -8, -9

NOALLOC_SCRATCH_BYTES = 32 << 20  # BLOCKFFN_NOALLOC_SCRATCH_BYTES

FFF_GELU_NODES, FFF_GELU_OUTPUT = 0, 1
FFF_SPARSE, FFF_DENSE = 0, 1

# Every symbol include/blockffn.h declares.
EXPORTS = ("blockffn_route", "blockffn_route_with", "blockffn_chunk_union", "blockffn_forward",
           "blockffn_forward_noalloc", "blockffn_sparsity_stats",
           "blockffn_layer_forward", "blockffn_layer_forward_workspace_size",
           "blockffn_backward", "blockffn_backward_workspace_size",
           "blockffn_cls_losses", "blockffn_cls_losses_workspace_size", "blockffn_fff_forward", "blockffn_fff_workspace_size", "blockffn_read_probe",
           "blockffn_set_stage_events", "blockffn_workspace_size", "blockffn_status_string",
           "blockffn_last_error", "blockffn_version", "blockffn_build_digest")


class BlockffnLayer(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("d_expert", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("reserved", ctypes.c_int32),
        ("w_router", ctypes.c_void_p), ("b_router", ctypes.c_void_p), ("rms_scale", ctypes.c_void_p),
        ("w_in", ctypes.c_void_p), ("w_out", ctypes.c_void_p),
    ]


class BlockffnFffLayer(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int32), ("n_trees", ctypes.c_int32), ("depth", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("activation", ctypes.c_int32), ("node_stride", ctypes.c_int32),
        ("w_node", ctypes.c_void_p), ("b_node", ctypes.c_void_p), ("w_out", ctypes.c_void_p),
    ]


class BlockffnStats(ctypes.Structure):
    _fields_ = [
        ("n_tokens", ctypes.c_int64), ("n_chunks", ctypes.c_int64), ("n_experts", ctypes.c_int64),
        ("chunk_len", ctypes.c_int64), ("active_pairs", ctypes.c_int64), ("union_sum", ctypes.c_int64),
        ("reuse_num", ctypes.c_int64), ("reuse_den", ctypes.c_int64), ("hist", ctypes.c_int64 * 129),
    ]


class BlockffnGrads(ctypes.Structure):
    _fields_ = [("d_w_router", ctypes.c_void_p), ("d_b_router", ctypes.c_void_p), ("d_rms_scale", ctypes.c_void_p),
                ("d_w_in", ctypes.c_void_p), ("d_w_out", ctypes.c_void_p)]


class BlockFFNError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where} failed ({status}): {message}")
        self.status = status


_lock = threading.Lock()
_lib = None


def load(path: str = None) -> ctypes.CDLL:
    """Load libblockffn.so (built by `python -m activation_sparse_moe_amd.build`), or the build that
    BLOCKFFN_LIB names (the host-sanitizer build of the CPU tests)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if path is None:
            path = os.environ.get("BLOCKFFN_LIB") or LIB_PATH
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m activation_sparse_moe_amd.build` "
                               "(the BlockFFN path has no fallback)")
        # torch brings its own HIP runtime, which its libraries load under the name "libamdhip64.so"; the
        # library links "libamdhip64.so.7", which that runtime also answers to once it is loaded.  Loaded
        # first, the library would pull in the system runtime, torch would then load its own beside it, and
        # the two runtimes in one process disagree (calls fail with "no ROCm-capable device").  Importing
        # torch first leaves one runtime, shared by torch and the library.
        import torch  # noqa: F401
        lib = ctypes.CDLL(path)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        lp = ctypes.POINTER(BlockffnLayer)
        lib.blockffn_route.argtypes = [lp, i32, vp, i64, i32, vp, vp, vp, vp]
        lib.blockffn_route_with.argtypes = [lp, i32, vp, i64, i32, i32, i32, vp, vp, vp, vp]
        lib.blockffn_chunk_union.argtypes = [i32, vp, i64, i32, vp, vp, vp, vp]
        lib.blockffn_forward.argtypes = [lp, i32, vp, i64, i32, vp, vp, vp, i32, vp, sz, vp, vp]
        lib.blockffn_forward_noalloc.argtypes = [lp, i32, vp, i64, i32, vp, vp, vp, i32, vp, vp]
        lib.blockffn_sparsity_stats.argtypes = [i32, vp, i64, i32, vp, vp]
        lib.blockffn_layer_forward.argtypes = [lp, i32, vp, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp]
        lib.blockffn_layer_forward_workspace_size.argtypes = [lp, i64, i32]
        lib.blockffn_layer_forward_workspace_size.restype = sz
        lib.blockffn_backward.argtypes = [lp, vp, i64, vp, vp, vp, vp, sz, vp, ctypes.POINTER(BlockffnGrads), vp]
        flt = ctypes.c_float
        lib.blockffn_cls_losses.argtypes = [i32, vp, i64, i32, flt, flt, flt, vp, sz, vp, vp, vp]
        lib.blockffn_fff_forward.argtypes = [ctypes.POINTER(BlockffnFffLayer), i32, vp, i64, i32, i32, vp, vp, vp, sz,
                                             vp, vp]
        lib.blockffn_fff_workspace_size.argtypes = [ctypes.POINTER(BlockffnFffLayer), i64, i32]
        lib.blockffn_fff_workspace_size.restype = sz
        lib.blockffn_read_probe.argtypes = [vp, sz, i32, vp, vp]
        lib.blockffn_cls_losses_workspace_size.argtypes = [i64, i32]
        lib.blockffn_cls_losses_workspace_size.restype = sz
        lib.blockffn_backward_workspace_size.argtypes = [lp, i64]
        lib.blockffn_backward_workspace_size.restype = sz
        for f in ("blockffn_route", "blockffn_route_with", "blockffn_chunk_union", "blockffn_forward",
                  "blockffn_forward_noalloc", "blockffn_layer_forward",
                  "blockffn_sparsity_stats", "blockffn_backward", "blockffn_cls_losses", "blockffn_fff_forward",
                  "blockffn_read_probe"):
            getattr(lib, f).restype = ctypes.c_int
        lib.blockffn_set_stage_events.argtypes = [vp, i32]
        lib.blockffn_set_stage_events.restype = ctypes.c_int
        lib.blockffn_workspace_size.argtypes = [lp, i64, i32, i32]
        lib.blockffn_workspace_size.restype = sz
        lib.blockffn_status_string.argtypes = [ctypes.c_int]
        lib.blockffn_status_string.restype = ctypes.c_char_p
        lib.blockffn_last_error.argtypes = []
        lib.blockffn_last_error.restype = ctypes.c_char_p
        lib.blockffn_version.argtypes = []
        lib.blockffn_version.restype = ctypes.c_int
        lib.blockffn_build_digest.argtypes = []
        lib.blockffn_build_digest.restype = ctypes.c_char_p
        _check_digest(lib, path)
        _lib = lib
        return lib


def _check_digest(lib, path: str) -> None:
    """Refuse a library built from other sources than those beside it (a stale build)."""
    from . import build as _build
    if os.path.dirname(os.path.abspath(path)) != PKG or not os.path.isdir(_build.CSRC):
        return  # not an in-tree build, or no sources to compare with
    have = lib.blockffn_build_digest().decode()
    want = _build.library_digest()
    if have != want:
        raise RuntimeError(f"{path} was built from sources with digest {have}, but the sources here have digest "
                           f"{want}: rebuild it with `python -m activation_sparse_moe_amd.build`")


def build_digest() -> str:
    return load().blockffn_build_digest().decode()


def check(status: int, where: str) -> None:
    if status != OK:
        lib = load()
        raise BlockFFNError(status, where, lib.blockffn_last_error().decode(errors="replace"))
