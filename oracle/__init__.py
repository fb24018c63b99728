"""CPU oracle of the BlockFFN layer (forward and backward) and of the FFF tree
layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never loads it and
shares no code with it.

The arithmetic lives in ``blockffn_oracle.c`` and ``fff_oracle.c`` (plain C,
double accumulation, OpenMP over tokens); this module only builds them with
gcc and marshals numpy arrays.  Arrays are float32 (an fp32 layer) or uint16 bfloat16 bit patterns
(a bf16 layer); the C code widens them itself.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = (os.path.join(_HERE, "blockffn_oracle.c"), os.path.join(_HERE, "fff_oracle.c"))
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

F32, BF16 = 0, 1
MAX_HIST = 129


class OracleStats(ctypes.Structure):
    _fields_ = [
        ("n_tokens", ctypes.c_int64), ("n_chunks", ctypes.c_int64),
        ("n_experts", ctypes.c_int64), ("chunk_len", ctypes.c_int64),
        ("active_pairs", ctypes.c_int64), ("union_sum", ctypes.c_int64),
        ("reuse_num", ctypes.c_int64), ("reuse_den", ctypes.c_int64),
        ("hist", ctypes.c_int64 * MAX_HIST),
    ]


SAN_LIB = os.path.join(_HERE, "liboracle_san.so")
# AddressSanitizer and UndefinedBehaviorSanitizer (host code only; any report aborts the process)
SAN_FLAGS = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g"]


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile liboracle.so with gcc (plain -O2, no fast-math, no FMA contraction); with `sanitize`,
    liboracle_san.so, the same code under ASan + UBSan (load it with gcc's libasan preloaded)."""
    lib = SAN_LIB if sanitize else _LIB
    if not force and os.path.exists(lib) and all(os.path.getmtime(lib) >= os.path.getmtime(s) for s in SOURCES):
        return lib
    tmp = lib + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           *(SAN_FLAGS if sanitize else []), "-shared", "-fPIC", "-o", tmp, *SOURCES, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            # BLOCKFFN_ORACLE_LIB points the tests at another build of the
            # oracle: a deliberately broken copy (mutation tests) or the
            # sanitizer build; normally it is unset.
            path = os.environ.get("BLOCKFFN_ORACLE_LIB")
            if not path:
                build(force=False)
                path = _LIB
            lib = ctypes.CDLL(path)
            vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
            lib.oracle_route.argtypes = [i32, i32, i32, vp, i64, vp, vp, vp, dbl, vp, vp, vp]
            lib.oracle_expert.argtypes = [i32, i32, i32, vp, i64, vp, vp, i32, vp]
            lib.oracle_forward_tokens.argtypes = [i32, i32, i32, i32, vp, i64, vp, vp, vp, vp, vp]
            lib.oracle_forward_chunks.argtypes = [i32, i32, i32, i32, vp, i64, i32, vp, vp, vp, vp, vp, vp]
            lib.oracle_forward_dense.argtypes = [i32, i32, i32, i32, vp, i64, vp, vp, vp, vp]
            lib.oracle_union.argtypes = [i32, vp, i64, i32, vp, vp, vp]
            lib.oracle_stats.argtypes = [i32, vp, i64, i32, ctypes.POINTER(OracleStats)]
            lib.oracle_route_with.argtypes = [i32, i32, i32, vp, i64, vp, vp, i32, i32, vp, vp, vp]
            lib.oracle_backward.argtypes = [i32, i32, i32, i32, vp, i64, vp, vp, vp, dbl, vp, vp, vp, vp, vp, vp,
                                            vp, vp, vp, vp, vp, vp, vp, vp]
            lib.oracle_cls_losses.argtypes = [i32, vp, i64, i32, dbl, dbl, dbl, vp, vp]
            lib.oracle_fff_forward.argtypes = [i32, i32, i32, i32, i32, i32, vp, i64, vp, vp, vp, vp, vp, vp]
            lib.oracle_num_threads.argtypes = []
            for name in ("oracle_route", "oracle_expert", "oracle_forward_tokens",
                         "oracle_forward_chunks", "oracle_forward_dense", "oracle_union",
                         "oracle_stats", "oracle_backward", "oracle_route_with", "oracle_cls_losses", "oracle_fff_forward",
                         "oracle_num_threads"):
                getattr(lib, name).restype = ctypes.c_int
            _lib = lib
    return _lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle inputs must be float32 or uint16 (bf16 bits), got {a.dtype}")


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype=None):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype) if dtype is not None else np.ascontiguousarray(a)


def _check(rc: int, name: str):
    if rc != 0:
        raise RuntimeError(f"{name} failed with code {rc}")


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def mask_words(n_experts: int) -> int:
    return (n_experts + 63) // 64


def route(x, w_router, b_router=None, rms_scale=None, eps: float = 1e-6):
    """Router: returns (z[T][E] f64, g[T][E] f64, mask[T][W] u64)."""
    x, w_router = _c(x), _c(w_router)
    code = _dtype_code(x)
    assert _dtype_code(w_router) == code, "x and w_router must share a dtype"
    T, d = x.shape
    E = w_router.shape[0]
    assert w_router.shape == (E, d)
    b = _c(b_router, np.float32)
    s = _c(rms_scale, np.float32)
    z = np.empty((T, E), np.float64)
    g = np.empty((T, E), np.float64)
    m = np.empty((T, mask_words(E)), np.uint64)
    _check(_load().oracle_route(d, E, code, _p(x), T, _p(w_router), _p(b), _p(s), float(eps),
                                _p(z), _p(g), _p(m)), "oracle_route")
    return z, g, m


ROUTER_TOPK_SOFTMAX, ROUTER_RELU_SUM = 1, 2


def route_with(x, w_router, b_router, kind: int, top_k: int = 0):
    """Baseline routers: kind 1 = top-k of a softmax, kind 2 = ReLU divided by its sum.
    Returns (z, g, mask) like route()."""
    x, w_router = _c(x), _c(w_router)
    code = _dtype_code(x)
    assert _dtype_code(w_router) == code
    T, d = x.shape
    E = w_router.shape[0]
    b = _c(b_router, np.float32)
    z = np.empty((T, E), np.float64)
    g = np.empty((T, E), np.float64)
    m = np.empty((T, mask_words(E)), np.uint64)
    _check(_load().oracle_route_with(d, E, code, _p(x), T, _p(w_router), _p(b), int(kind), int(top_k), _p(z), _p(g),
                                     _p(m)), "oracle_route_with")
    return z, g, m


def expert(x, t: int, w_in, w_out, i: int):
    """E_i(x_t) as a float64 vector of length d."""
    x, w_in, w_out = _c(x), _c(w_in), _c(w_out)
    code = _dtype_code(x)
    E, de, d = w_in.shape
    e = np.empty(d, np.float64)
    _check(_load().oracle_expert(d, de, code, _p(x), int(t), _p(w_in), _p(w_out), int(i), _p(e)),
           "oracle_expert")
    return e


def _fwd_common(x, w_in, w_out, g):
    x, w_in, w_out = _c(x), _c(w_in), _c(w_out)
    code = _dtype_code(x)
    assert _dtype_code(w_in) == code and _dtype_code(w_out) == code
    T, d = x.shape
    E, de, d2 = w_in.shape
    assert d2 == d and w_out.shape == (E, d, de)
    g = _c(g, np.float64)
    assert g.shape == (T, E)
    return x, w_in, w_out, g, code, T, d, E, de


def forward_tokens(x, w_in, w_out, g, mask):
    x, w_in, w_out, g, code, T, d, E, de = _fwd_common(x, w_in, w_out, g)
    mask = _c(mask, np.uint64)
    y = np.empty((T, d), np.float64)
    _check(_load().oracle_forward_tokens(d, E, de, code, _p(x), T, _p(w_in), _p(w_out), _p(g),
                                         _p(mask), _p(y)), "oracle_forward_tokens")
    return y


def forward_chunks(x, w_in, w_out, g, chunk_len: int, count, lst):
    x, w_in, w_out, g, code, T, d, E, de = _fwd_common(x, w_in, w_out, g)
    count = _c(count, np.int32)
    lst = _c(lst, np.int32)
    y = np.empty((T, d), np.float64)
    _check(_load().oracle_forward_chunks(d, E, de, code, _p(x), T, int(chunk_len), _p(w_in),
                                         _p(w_out), _p(g), _p(count), _p(lst), _p(y)),
           "oracle_forward_chunks")
    return y


def forward_dense(x, w_in, w_out, g):
    x, w_in, w_out, g, code, T, d, E, de = _fwd_common(x, w_in, w_out, g)
    y = np.empty((T, d), np.float64)
    _check(_load().oracle_forward_dense(d, E, de, code, _p(x), T, _p(w_in), _p(w_out), _p(g), _p(y)),
           "oracle_forward_dense")
    return y


def chunk_union(mask, n_experts: int, chunk_len: int):
    """Returns (umask[C][W] u64, count[C] i32, list[C][E] i32 with -1 tail)."""
    mask = _c(mask, np.uint64)
    T = mask.shape[0]
    W = mask_words(n_experts)
    C = T // chunk_len
    um = np.empty((C, W), np.uint64)
    cnt = np.empty(C, np.int32)
    lst = np.empty((C, n_experts), np.int32)
    _check(_load().oracle_union(n_experts, _p(mask), T, int(chunk_len), _p(um), _p(cnt), _p(lst)),
           "oracle_union")
    return um, cnt, lst


def stats(mask, n_experts: int, chunk_len: int) -> dict:
    mask = _c(mask, np.uint64)
    T = mask.shape[0]
    st = OracleStats()
    _check(_load().oracle_stats(n_experts, _p(mask), T, int(chunk_len), ctypes.byref(st)), "oracle_stats")
    out = {f: getattr(st, f) for f, _ in OracleStats._fields_ if f != "hist"}
    out["hist"] = np.array(st.hist[: n_experts + 1], dtype=np.int64)
    out["tls"] = 1.0 - st.active_pairs / (T * n_experts) if T else 0.0
    out["cls"] = 1.0 - st.union_sum / (st.n_chunks * n_experts) if st.n_chunks else 0.0
    out["reuse"] = st.reuse_num / st.reuse_den if st.reuse_den else 0.0
    return out


def layer_forward(layer, x, chunk_len: int):
    """Full oracle pass on one layer: route, union, per-token forward, stats."""
    z, g, m = route(x, layer.w_router, layer.b_router, layer.rms_scale, layer.rms_eps)
    um, cnt, lst = chunk_union(m, layer.n_experts, chunk_len)
    y = forward_tokens(x, layer.w_in, layer.w_out, g, m)
    return dict(z=z, g=g, mask=m, umask=um, count=cnt, list=lst, y=y)


def backward(x, w_router, b_router, rms_scale, eps, w_in, w_out, dy, expert_sel=None, token_sel=None,
             dz_extra=None) -> dict:
    """Gradients of sum(y * dy) with respect to x and every parameter (float64).

    Returns dx[T][d], dw_router[E][d], db[E], ds[E], dw_in[E][de][d],
    dw_out[E][d][de], and the per-pair dz[T][E] and dg[T][E].  expert_sel /
    token_sel (bool arrays of length E / T) restrict which dw_in / dw_out
    blocks and which dx rows are computed; the rest stay zero.  dz_extra
    ([T][E]) is an extra gradient with respect to z (e.g. of the CLS-aware
    objectives), added to every pair's dz.
    """
    x, w_router, w_in, w_out = _c(x), _c(w_router), _c(w_in), _c(w_out)
    code = _dtype_code(x)
    assert _dtype_code(w_router) == code and _dtype_code(w_in) == code and _dtype_code(w_out) == code
    T, d = x.shape
    E, de, d2 = w_in.shape
    assert d2 == d and w_out.shape == (E, d, de) and w_router.shape == (E, d)
    dy = _c(dy, np.float32)
    assert dy.shape == (T, d)
    b = _c(b_router, np.float32)
    s = _c(rms_scale, np.float32)
    dze = None if dz_extra is None else _c(dz_extra, np.float64)
    es = None if expert_sel is None else _c(np.asarray(expert_sel, dtype=bool).astype(np.uint8))
    ts = None if token_sel is None else _c(np.asarray(token_sel, dtype=bool).astype(np.uint8))
    out = dict(dx=np.empty((T, d)), dw_router=np.empty((E, d)), db=np.empty(E), ds=np.empty(E),
               dw_in=np.empty((E, de, d)), dw_out=np.empty((E, d, de)), dz=np.empty((T, E)), dg=np.empty((T, E)))
    _check(_load().oracle_backward(d, E, de, code, _p(x), T, _p(w_router), _p(b), _p(s), float(eps), _p(w_in),
                                   _p(w_out), _p(dy), _p(dze), _p(es), _p(ts), _p(out["dx"]), _p(out["dw_router"]),
                                   _p(out["db"]), _p(out["ds"]), _p(out["dw_in"]), _p(out["dw_out"]), _p(out["dz"]),
                                   _p(out["dg"])), "oracle_backward")
    return out


def cls_losses(z, chunk_len: int, alpha: float, w_al: float = 1.0, w_cs: float = 1.0, want_grad: bool = True):
    """CLS-aware objectives on pre-activations z[T][E] (float64):
    returns (L_AL, L_CS, dz or None) with dz = w_al dL_AL/dz + w_cs dL_CS/dz."""
    z = _c(z, np.float64)
    T, E = z.shape
    loss = np.empty(2, np.float64)
    dz = np.empty((T, E), np.float64) if want_grad else None
    _check(_load().oracle_cls_losses(E, _p(z), T, int(chunk_len), float(alpha), float(w_al), float(w_cs), _p(loss),
                                      _p(dz)), "oracle_cls_losses")
    return float(loss[0]), float(loss[1]), dz


def fff_nodes(depth: int) -> int:
    """Nodes of one perfect binary tree of depth D (levels 0..D)."""
    return (1 << (depth + 1)) - 1


def fff_forward(x, w_node, b_node, w_out, post: bool = False, dense: bool = False, want_paths: bool = True):
    """FFF tree layer.  x[T][d]; w_node, w_out [P][N][d] with N = 2^(D+1) - 1; b_node [P][N] or None.

    Returns (paths, preact, y): paths [T][P][D+1] int32 node ids (None when dense or not wanted),
    preact [T][P][D+1] float64 ([T][P][N] when dense), y [T][d] float64."""
    x, w_node, w_out = _c(x), _c(w_node), _c(w_out)
    code = _dtype_code(x)
    assert _dtype_code(w_node) == code and _dtype_code(w_out) == code, "x and the node rows must share a dtype"
    T, d = x.shape
    P, N, d2 = w_node.shape
    D = int(N + 1).bit_length() - 2
    assert d2 == d and fff_nodes(D) == N and w_out.shape == (P, N, d)
    b = _c(b_node, np.float32)
    assert b is None or b.shape == (P, N)
    V = N if dense else D + 1
    paths = np.empty((T, P, V), np.int32) if (want_paths and not dense) else None
    preact = np.empty((T, P, V), np.float64)
    y = np.empty((T, d), np.float64)
    _check(_load().oracle_fff_forward(d, P, D, code, int(bool(post)), int(bool(dense)), _p(x), T, _p(w_node), _p(b),
                                      _p(w_out), _p(paths), _p(preact), _p(y)), "oracle_fff_forward")
    return paths, preact, y
