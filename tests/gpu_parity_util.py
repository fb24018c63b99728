"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare it with the CPU oracle on the same seeded inputs.

Bars (element by element):
  * activation patterns and chunk unions: bit-exact, except (token, expert)
    pairs whose oracle pre-activation lies within 1e-3 of zero, where fp32
    and fp64 accumulation may legitimately disagree on the sign; tokens with
    such a flip are left out of the gate and output checks and counted;
  * gates: max |dg| <= 1e-5 (fp32 layers) or 1e-4 (bf16) times RMS of the
    oracle gates, over tokens where RMSNorm is well conditioned
    (mean(a^2) + eps >= 1e-4, so an error in z is amplified at most 100x;
    a token whose only active pre-activation is tiny has mean(a^2) << eps
    and amplifies it about 1/sqrt(eps) = 1000x).  On every token, the gate
    function itself is checked on the GPU's own z: the GPU gates against
    fp64 gates of that z (the oracle router on z with an identity matrix),
    |dg| <= 1e-5 |g| + 1e-6 RMS (the fp32 epilogue's rounding);
  * outputs: a token with no active expert gets an exactly zero row; on the
    other compared tokens max |dy| <= 1e-5 (fp32) or 2e-2 (bf16) times RMS of
    the oracle output over those tokens.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from activation_sparse_moe_amd import binding as B
from activation_sparse_moe_amd._capi import BF16, F32

BAND = 1e-3
GATE_TOL = {"f32": 1e-5, "bf16": 1e-4}
COND_MS = 1e-4       # mean(a^2) + eps below this: RMSNorm amplifies z errors over 100x
GATE_FN_REL = 1e-5   # gate epilogue on the GPU's own z: relative bar
GATE_FN_ABS = 1e-6   # ... plus this times RMS(g)
Y_TOL = {"f32": 1e-5, "bf16": 2e-2}
BWD_TOL = 1e-2     # backward gradients (the bar's derivation heads test_gpu_backward)


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bits(m_u64: np.ndarray, E: int) -> np.ndarray:
    """[T][W] u64 masks -> [T][E] bool."""
    T, W = m_u64.shape
    out = np.zeros((T, E), bool)
    for i in range(E):
        out[:, i] = (m_u64[:, i // 64] >> np.uint64(i % 64)) & np.uint64(1)
    return out


def run_gpu(dev_layer: B.DeviceLayer, x_dev: torch.Tensor, L: int, mode="auto", n_layers=None,
            want_preact=True, stats=True):
    """route -> chunk_union -> forward (-> stats) on the current stream; numpy results."""
    E = (dev_layer[0] if isinstance(dev_layer, (list, tuple)) else dev_layer).n_experts
    g, m, z = B.blockffn_route(dev_layer, x_dev, L, n_layers=n_layers, want_preact=want_preact)
    um, cnt, lst = B.blockffn_chunk_union(E, m, L)
    y = B.blockffn_forward(dev_layer, x_dev, L, g, cnt, lst, mode=mode, n_layers=n_layers)
    st = B.blockffn_sparsity_stats(E, m, L) if stats else None
    torch.cuda.synchronize()
    out = dict(g=g.cpu().numpy(), mask=B.masks_to_u64(m), umask=B.masks_to_u64(um), count=cnt.cpu().numpy(),
               list=lst.cpu().numpy(), y=y.cpu().numpy())
    if z is not None:
        out["z"] = z.cpu().numpy()
    if st is not None:
        out["stats"] = B.stats_dict(st)
    return out


def check_route(gpu: dict, z: np.ndarray, g: np.ndarray, m: np.ndarray, E: int, dtype: str, t_idx=None,
                layer=None):
    """Masks bit-exact outside the band, gates within tolerance where RMSNorm is
    well conditioned, and (given the layer and the GPU's z) the gate function
    on the GPU's own z.  Returns the flipped-token set."""
    gm = gpu["mask"] if t_idx is None else gpu["mask"][t_idx]
    gg = gpu["g"] if t_idx is None else gpu["g"][t_idx]
    ob, gb = bits(m, E), bits(gm, E)
    diff = ob != gb
    if diff.any():
        bad = diff & (np.abs(z) >= BAND)
        assert not bad.any(), f"mask mismatch outside the band at {np.argwhere(bad)[:8].tolist()}"
    flipped = set(np.nonzero(diff.any(axis=1))[0].tolist())
    keep = np.array([t not in flipped for t in range(z.shape[0])], bool)
    rms = np.sqrt((g ** 2).mean())
    eps = layer.rms_eps if layer is not None else 1e-6
    well = keep & ((np.maximum(z, 0.0) ** 2).mean(axis=1) + eps >= COND_MS)
    if well.any():
        err = np.abs(gg[well].astype(np.float64) - g[well]).max()
        assert err <= GATE_TOL[dtype] * rms, f"gate error {err:.3e} > {GATE_TOL[dtype]} x RMS {rms:.3e}"
    if "z" in gpu:
        gz = gpu["z"] if t_idx is None else gpu["z"][t_idx]
        scale = np.sqrt((z ** 2).mean())
        zerr = np.abs(gz.astype(np.float64) - z).max()
        assert zerr <= 1e-4 * max(scale, 1.0), f"pre-activation error {zerr:.3e}"
        if layer is not None:
            # the oracle router on the GPU's z (identity matrix, no bias: z is
            # reproduced exactly) gives fp64 gates of that z
            gz32 = np.ascontiguousarray(gz, dtype=np.float32)
            _, g_of_z, m_of_z = oracle.route(gz32, np.eye(E, dtype=np.float32), None, layer.rms_scale, eps)
            np.testing.assert_array_equal(gm, m_of_z)  # the pattern is the sign of the GPU's own z
            dg = np.abs(gg.astype(np.float64) - g_of_z)
            bar = GATE_FN_REL * np.abs(g_of_z) + GATE_FN_ABS * rms
            assert (dg <= bar).all(), f"gate function error {dg.max():.3e} on the GPU's own z"
    return flipped, keep


def check_union(gpu: dict, o_um: np.ndarray, z: np.ndarray, E: int, L: int, c_idx=None):
    """Union bit-exact except experts with a band flip in the chunk; list/count consistent."""
    gum = gpu["umask"] if c_idx is None else gpu["umask"][c_idx]
    gcnt = gpu["count"] if c_idx is None else gpu["count"][c_idx]
    glst = gpu["list"] if c_idx is None else gpu["list"][c_idx]
    ob, gb = bits(o_um, E), bits(gum, E)
    C = ob.shape[0]
    near = (np.abs(z) < BAND).reshape(C, L, E).any(axis=1)
    diff = ob != gb
    assert not (diff & ~near).any(), f"union mismatch at {np.argwhere(diff & ~near)[:8].tolist()}"
    for c in range(C):
        want = np.nonzero(gb[c])[0]
        assert gcnt[c] == len(want)
        np.testing.assert_array_equal(glst[c, :gcnt[c]], want)
        assert (glst[c, gcnt[c]:] == -1).all()
    return int(diff.sum())


def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, keep: np.ndarray, dtype: str, what=""):
    """Outputs of the compared tokens: a token with no active expert (its oracle row is exactly
    zero) must get an exactly zero row; the other rows must lie within Y_TOL x RMS of those rows.
    Exact zero rows carry no rounding, so they are checked exactly and left out of the RMS that
    scales the bar (with them in, a call whose tokens are mostly silent would hold its few live
    rows to a bar shrunk by the silent share)."""
    if not keep.any():
        return 0.0
    silent = keep & ~np.any(y_ref != 0, axis=1)
    if silent.any():
        assert not np.any(y_gpu[silent] != 0), f"{what}: a token with no active expert has a non-zero output"
    live = keep & ~silent
    if not live.any():
        return 0.0
    ref = y_ref[live]
    rms = np.sqrt((ref ** 2).mean())
    err = np.abs(y_gpu[live].astype(np.float64) - ref).max()
    rel = err / rms
    assert err <= Y_TOL[dtype] * rms, f"{what} output error {err:.3e} > {Y_TOL[dtype]} x RMS {rms:.3e}"
    return rel


def oracle_full(layer, x, L):
    z, g, m = oracle.route(x, layer.w_router, layer.b_router, layer.rms_scale, layer.rms_eps)
    um, cnt, lst = oracle.chunk_union(m, layer.n_experts, L)
    return z, g, m, um, cnt, lst


def router_band_tokens(z, kind, k):
    """Tokens whose baseline-router decision lies within BAND of its threshold in the oracle's z:
    some |z_i| < BAND for the ReLU-sum router, the gap between the k-th and (k+1)-th largest z
    for top-k."""
    if kind == "relu_sum":
        return (np.abs(z) < BAND).any(axis=1)
    zs = -np.sort(-z, axis=1)
    return (zs[:, k - 1] - zs[:, k]) < BAND if k < z.shape[1] else np.zeros(z.shape[0], bool)


def check_baseline_router(layer, x, L, router, k, what=""):
    """blockffn_route_with (top-k softmax or ReLU-sum), the union and the forward on its gates,
    against the oracle: z within 1e-4 (bf16) / 1e-5 (fp32) x RMS(z); masks bit-exact outside the
    band (router_band_tokens); gates within GATE_TOL x RMS(g) and y within Y_TOL x RMS(y) on the
    other tokens.  Returns (max |dy| / RMS(y), band tokens)."""
    E, dt = layer.n_experts, layer.dtype
    dl = B.DeviceLayer.from_workload(layer)
    xd = B.tokens_to_device(x, F32 if dt == "f32" else BF16)
    g, m, z = B.blockffn_route_with(dl, xd, L, router=router, top_k=k, want_preact=True)
    um, cnt, lst = B.blockffn_chunk_union(E, m, L)
    y = B.blockffn_forward(dl, xd, L, g, cnt, lst)
    torch.cuda.synchronize()
    kind = oracle.ROUTER_TOPK_SOFTMAX if router == "topk_softmax" else oracle.ROUTER_RELU_SUM
    z_ref, g_ref, m_ref = oracle.route_with(x, layer.w_router, layer.b_router, kind, k)
    gz, gg, gm = z.cpu().numpy(), g.cpu().numpy(), B.masks_to_u64(m)
    scale = np.sqrt((z_ref ** 2).mean())
    assert np.abs(gz - z_ref).max() <= (1e-5 if dt == "f32" else 1e-4) * scale
    band = router_band_tokens(z_ref, router, k)
    ob, gb = bits(m_ref, E), bits(gm, E)
    diff = (ob != gb).any(axis=1)
    assert not (diff & ~band).any(), f"mask mismatch outside the band at tokens {np.nonzero(diff & ~band)[0][:8]}"
    keep = ~band
    if router == "topk_softmax":
        assert np.all(gb.sum(axis=1) == k)
    if not keep.any():
        return 0.0, int(band.sum())
    rms = np.sqrt((g_ref[keep] ** 2).mean())
    assert np.abs(gg[keep] - g_ref[keep]).max() <= GATE_TOL[dt] * rms
    y_ref = oracle.forward_tokens(x, layer.w_in, layer.w_out, g_ref, m_ref)
    rel = check_y(y.cpu().numpy(), y_ref, keep, dt, what)
    say(f"  {router}{k} {what}: max|dy|/rms {rel:.2e}, band tokens {int(band.sum())}")
    return rel, int(band.sum())


def dtype_code(layer) -> int:
    return F32 if layer.dtype == "f32" else BF16


def check_grad(name, got, ref, rows=None, tol=BWD_TOL, tol_max=None):
    """A backward gradient against the oracle gradient: the norm-wise error within tol of ||G|| and
    the largest element error within tol_max (default tol) of max |G|.  Returns the norm-wise one."""
    tol_max = tol if tol_max is None else tol_max
    if rows is not None:
        got, ref = got[rows], ref[rows]
    if ref.size == 0:
        return 0.0
    top = np.abs(ref).max()
    if top == 0:
        assert np.all(got == 0), f"{name}: expected zeros, max |got| {np.abs(got).max():.3e}"
        return 0.0
    err = np.abs(got - ref).max()
    fro = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert fro <= tol, f"{name}: norm-wise relative error {fro:.3e} > {tol:.3e}"
    assert err <= tol_max * top, f"{name}: max |err| {err:.3e} > {tol_max:.3e} x max |G| {top:.3e}"
    return fro


GRADS = (("dx", "dx"), ("d_w_in", "dw_in"), ("d_w_out", "dw_out"), ("d_rms_scale", "ds"),
         ("d_w_router", "dw_router"), ("d_b_router", "db"))


def conditioned_tols(ref, ref_rounded, factor: float = 5.0):
    """Bars that follow the problem's conditioning.  ref_rounded is the oracle's result with dy
    rounded to bf16, as the kernels round it; how far each gradient moves under that one rounding
    (norm-wise and max-element, relative) measures how much the problem amplifies rounding.  The
    bars are factor times that, and never below BWD_TOL: on well-conditioned inputs the move is
    about 2e-3 and the bars stay at BWD_TOL, but a router gradient that nearly cancels (tokens with
    a single active expert, whose normalised gate hardly depends on z) can move 5x more."""
    tols = {}
    for name, key in GRADS:
        a, b = ref[key], ref_rounded[key]
        n, top = np.linalg.norm(a), np.abs(a).max()
        fro = np.linalg.norm(a - b) / n if n > 0 else 0.0
        mx = np.abs(a - b).max() / top if top > 0 else 0.0
        tols[name] = (max(BWD_TOL, factor * fro), max(BWD_TOL, factor * mx))
    return tols


def check_backward(gpu, ref, gz, z_ref, dx_gpu, dx_ref, experts=None, router=True, tols=None):
    """Compare every gradient.  gz / z_ref are the pre-activations of the
    tokens whose dx rows are compared; experts restricts the expert blocks;
    router=False leaves dW_r and db to the caller; tols (from conditioned_tols)
    replaces the fixed bars per gradient."""
    def t(name):
        return tols[name] if tols is not None else (BWD_TOL, BWD_TOL)
    band = np.abs(z_ref) < BAND
    flips = (gz > 0) != (z_ref > 0)
    assert not (flips & ~band).any(), "activation pattern differs outside the band"
    bad_tok = band.any(axis=1)
    bad_exp = band.any(axis=0)
    rel = {"dx": check_grad("dx", dx_gpu, dx_ref, ~bad_tok, *t("dx"))}
    ex = np.arange(z_ref.shape[1]) if experts is None else np.asarray(experts)
    rel["d_w_in"] = check_grad("d_w_in", gpu["d_w_in"][ex], ref["dw_in"][ex], None, *t("d_w_in"))
    rel["d_w_out"] = check_grad("d_w_out", gpu["d_w_out"][ex], ref["dw_out"][ex], None, *t("d_w_out"))
    rel["d_rms_scale"] = check_grad("d_rms_scale", gpu["d_rms_scale"], ref["ds"], None, *t("d_rms_scale"))
    if router:
        rel["d_w_router"] = check_grad("d_w_router", gpu["d_w_router"], ref["dw_router"], ~bad_exp,
                                       *t("d_w_router"))
        rel["d_b_router"] = check_grad("d_b_router", gpu["d_b_router"], ref["db"], ~bad_exp, *t("d_b_router"))
    return rel, int(bad_tok.sum()), int(bad_exp.sum())
