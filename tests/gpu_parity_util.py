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
  * outputs: max |dy| <= 1e-5 (fp32) or 2e-2 (bf16) times RMS of the oracle
    output over the compared tokens.
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
    E = dev_layer.n_experts
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
    if not keep.any():
        return 0.0
    ref = y_ref[keep]
    rms = np.sqrt((ref ** 2).mean())
    err = np.abs(y_gpu[keep].astype(np.float64) - ref).max()
    rel = err / rms if rms > 0 else err
    assert err <= Y_TOL[dtype] * rms or (rms == 0 and err == 0), \
        f"{what} output error {err:.3e} > {Y_TOL[dtype]} x RMS {rms:.3e}"
    return rel


def oracle_full(layer, x, L):
    z, g, m = oracle.route(x, layer.w_router, layer.b_router, layer.rms_scale, layer.rms_eps)
    um, cnt, lst = oracle.chunk_union(m, layer.n_experts, L)
    return z, g, m, um, cnt, lst


def dtype_code(layer) -> int:
    return F32 if layer.dtype == "f32" else BF16
