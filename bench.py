#!/usr/bin/env python3
"""Benchmark of the BlockFFN layer forward on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic
input: router (ReLU + RMSNorm) -> chunk union -> expert forward over each
chunk's union -> sparsity statistics, all through the C ABI.  The default
workload is the speculative-verify chunk of 8 tokens: d = 2048, E = 64
experts of 2048 -> 128 -> 2048, bf16, 512 chunks (4096 tokens), every chunk
streaming its own copy of the layer so that no weight byte is served from a
cache.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

With --workload fff_D6_P64_d2048 it measures the FFF tree layer instead (64
trees of depth 6, d = 2048, bf16, 4096 independent tokens, each through its
own copy of the layer): one step is one blockffn_fff_forward over the batch.
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "chunk-8 BlockFFN layer tokens/s + active-weight HBM GB/s (% of peak)"
FFF_METRIC = "FFF tree layer tokens/s + visited-node HBM GB/s (% of peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published
DEFAULT_WORKLOAD = "chunk8_d2048_E64"
CSRC = os.path.join(ROOT, "activation_sparse_moe_amd", "csrc")


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--mode", default=None, help="forward mode (default: the workload's)")
    p.add_argument("--dense-steps", type=int, default=5, help="steps of the dense all-experts comparison (0: skip)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--router", default="blockffn", choices=("blockffn", "topk_softmax", "relu_sum"),
                   help="gate function: the BlockFFN router, or a baseline router for comparison")
    p.add_argument("--top-k", type=int, default=2, help="experts per token for --router topk_softmax")
    p.add_argument("--eager", action="store_true",
                   help="time eager launches (default: each step replayed from a HIP graph)")
    p.add_argument("--backward", action="store_true",
                   help="also time blockffn_backward on the batch (grouped workloads: one layer)")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target CPU time (seconds x threads) of the oracle sample")
    p.add_argument("--latency-units", type=int, default=64,
                   help="latency mode: units run one after another, one graph per chain of this many (0: skip)")
    p.add_argument("--fff-split", type=int, default=0,
                   help="FFF workloads: blocks per token (0: the library's choice)")
    p.add_argument("--no-ceilings", action="store_true",
                   help="skip the measured ceilings (HBM read probe, hipBLASLt bf16 GEMM)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a 1 GiB device copy (reference kernel for HBM byte counters)")
    return p.parse_args(argv)


# The sources each profiled kernel is built from: its counter summary stays
# valid while these files are unchanged.
KERNEL_SOURCES = {
    "expert_up": ("expert_mfma.hip", "lds_stream.h", "bffn_internal.h"),
    "expert_down": ("expert_mfma.hip", "lds_stream.h", "bffn_internal.h"),
    "grouped_up": ("grouped.hip", "grouped_kernels.h", "lds_stream.h", "bffn_internal.h"),
    "grouped_down": ("grouped.hip", "grouped_kernels.h", "lds_stream.h", "bffn_internal.h"),
    "fff_walk": ("fff.hip", "fff_probe_launch.h", "bffn_internal.h"),
}


def source_digest(kernel: str = None) -> str:
    """sha256 prefix of the library sources (all of them, or those of one kernel)."""
    h = hashlib.sha256()
    names = KERNEL_SOURCES[kernel] if kernel else [os.path.basename(p) for p in glob.glob(os.path.join(CSRC, "*"))]
    for name in sorted(names):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def _build_digest() -> str:
    """Digest of the sources the loaded library was built from (loading refuses a stale build)."""
    from activation_sparse_moe_amd import _capi
    return _capi.build_digest()


def profiled_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if there is none or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}__hbm_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_digest") != source_digest(kernel):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class StepRunner:
    """Holds the device buffers of one workload and runs steps on the current stream."""

    def __init__(self, cfg, mode: str, router: str = "blockffn", top_k: int = 0):
        import numpy as np
        import torch
        from activation_sparse_moe_amd import binding as B
        from workload import make_workload

        self.B, self.torch, self.np = B, torch, np
        self.cfg, self.mode = cfg, mode
        self.router, self.top_k = router, top_k
        t = time.time()
        self.layer, tok = make_workload(cfg)
        self.x_host = tok.x
        self.gen_s = time.time() - t
        self.dl = B.DeviceLayer.from_workload(self.layer, replicas=cfg.replicas)
        self.xd = B.tokens_to_device(tok.x, self.dl.dtype)
        T, E, L = cfg.n_tokens, cfg.n_experts, cfg.chunk_len
        dev = self.xd.device
        self.gates = torch.empty((T, E), dtype=torch.float32, device=dev)
        self.masks = torch.empty((T, self.dl.mask_words), dtype=torch.int64, device=dev)
        C = T // L
        self.umask = torch.empty((C, self.dl.mask_words), dtype=torch.int64, device=dev)
        self.count = torch.empty((C,), dtype=torch.int32, device=dev)
        self.lst = torch.empty((C, E), dtype=torch.int32, device=dev)
        self.y = torch.empty((T, cfg.d), dtype=torch.float32, device=dev)
        self.stats = torch.empty((8 + 129,), dtype=torch.int64, device=dev)
        # units per call: never more than the layer copies, so no two units of
        # one launch stream the same weights
        self.sub_units = min(C, cfg.replicas) if cfg.replicas > 1 else C
        self.n_sub = (C + self.sub_units - 1) // self.sub_units
        sub_T = self.sub_units * L
        self.ws = {}
        for m in {mode, "dense"}:
            self.ws[m] = B.alloc_workspace(self.dl, sub_T, L, m)
        self.n_stage = 4 if mode == "grouped" else 3
        self.lib = B.load()

    def step(self, mode: str, ev=None, stage_events=None):
        """route -> union -> forward -> stats, in sub-batches of at most one
        unit per layer copy.  ev: 4 torch events recorded after route, union,
        forward and stats of the last sub-batch; stage_events: one ctypes array
        of hipEvent_t per sub-batch, which the library records around that
        sub-batch's forward kernels."""
        B, cfg = self.B, self.cfg
        L, E = cfg.chunk_len, cfg.n_experts
        C = cfg.n_tokens // L
        nb = (C + self.sub_units - 1) // self.sub_units
        for b in range(nb):
            c0, c1 = b * self.sub_units, min(C, (b + 1) * self.sub_units)
            t0, t1 = c0 * L, c1 * L
            last = b == nb - 1
            x, g, m, y = self.xd[t0:t1], self.gates[t0:t1], self.masks[t0:t1], self.y[t0:t1]
            cnt, lst, um = self.count[c0:c1], self.lst[c0:c1], self.umask[c0:c1]
            if self.router == "blockffn":
                B.blockffn_route(self.dl, x, L, gates=g, token_masks=m)
            else:
                B.blockffn_route_with(self.dl, x, L, router=self.router, top_k=self.top_k, gates=g, token_masks=m)
            if ev is not None and last:
                ev[0].record()
            B.blockffn_chunk_union(E, m, L, chunk_masks=um, active_count=cnt, active_list=lst)
            if ev is not None and last:
                ev[1].record()
            if stage_events is not None:
                self.lib.blockffn_set_stage_events(ctypes.cast(stage_events[b], ctypes.c_void_p), self.n_stage)
            B.blockffn_forward(self.dl, x, L, g, cnt, lst, mode=mode, workspace=self.ws[mode], y=y)
            if stage_events is not None:
                self.lib.blockffn_set_stage_events(None, 0)
            if ev is not None and last:
                ev[2].record()
        B.blockffn_sparsity_stats(E, self.masks, L, stats_dev=self.stats)
        if ev is not None:
            ev[3].record()

    def timed(self, mode: str, steps: int, warmup: int):
        torch = self.torch
        for _ in range(warmup):
            self.step(mode)
        torch.cuda.synchronize()
        E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
        evs = [[E() for _ in range(4)] for _ in range(steps)]
        ns = self.n_stage if mode == self.mode else 3
        nb = self.n_sub
        stage = [[[E() for _ in range(ns)] for _ in range(nb)] for _ in range(steps)]
        # record every event once so that its hipEvent exists before the
        # library is handed the raw handles
        for per_step in stage:
            for row in per_step:
                for e in row:
                    e.record()
        torch.cuda.synchronize()
        handles = [[(ctypes.c_void_p * ns)(*[e.cuda_event for e in row]) for row in per_step] for per_step in stage]
        start, end = E(), E()
        torch.cuda.synchronize()
        start.record()
        prev = start
        starts = []
        for k in range(steps):
            starts.append(prev)
            self.step(mode, ev=evs[k], stage_events=handles[k]) if ns == self.n_stage else \
                self._step_n(mode, evs[k], handles[k], ns)
            prev = evs[k][3]
        end.record()
        torch.cuda.synchronize()
        total_ms = start.elapsed_time(end)
        per = {"route": [], "union": [], "up": [], "down": [], "stats": [], "forward": []}
        if ns > 3:
            per["combine"] = []
        for k in range(steps):
            # kernel time per step: the sum over the step's sub-batch launches
            per["up"].append(sum(r[0].elapsed_time(r[1]) for r in stage[k]))
            per["down"].append(sum(r[1].elapsed_time(r[2]) for r in stage[k]))
            if ns > 3:
                per["combine"].append(sum(r[2].elapsed_time(r[3]) for r in stage[k]))
            if nb == 1:
                per["route"].append(starts[k].elapsed_time(evs[k][0]))
                per["union"].append(evs[k][0].elapsed_time(evs[k][1]))
                per["forward"].append(evs[k][1].elapsed_time(evs[k][2]))
                per["stats"].append(evs[k][2].elapsed_time(evs[k][3]))
        avg = {k: sum(v) / len(v) for k, v in per.items() if v}
        return total_ms / steps, avg

    def graph_ms(self, mode: str, steps: int, warmup: int, forward_only: bool = False) -> float:
        """One whole step (every sub-batch) captured in a HIP graph and replayed:
        the step with no host launch overhead.  forward_only: the forward calls
        alone (every sub-batch; route and union results from earlier steps)."""
        torch = self.torch
        run = (lambda: self.forward_calls(mode)) if forward_only else (lambda: self.step(mode))
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for _ in range(max(1, warmup)):
                run()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        for _ in range(max(1, warmup)):
            g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    def forward_calls(self, mode: str):
        """blockffn_forward of every sub-batch, on the gates and unions already in the buffers."""
        B, cfg = self.B, self.cfg
        L = cfg.chunk_len
        C = cfg.n_tokens // L
        for b in range(self.n_sub):
            c0, c1 = b * self.sub_units, min(C, (b + 1) * self.sub_units)
            t0, t1 = c0 * L, c1 * L
            B.blockffn_forward(self.dl, self.xd[t0:t1], L, self.gates[t0:t1], self.count[c0:c1], self.lst[c0:c1],
                               mode=mode, workspace=self.ws[mode], y=self.y[t0:t1])

    def eager_ms(self, mode: str, steps: int, warmup: int) -> float:
        """Eager steps with no events inside the timed loop (instrumented steps
        leave the GPU idle between launches on the larger layers)."""
        torch = self.torch
        for _ in range(warmup):
            self.step(mode)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            self.step(mode)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    def _step_n(self, mode, ev, handle, ns):
        n0 = self.n_stage
        self.n_stage = ns
        try:
            self.step(mode, ev=ev, stage_events=handle)
        finally:
            self.n_stage = n0

    def byte_model(self):
        """Algorithmic bytes per launch of each kernel (what the method must
        move: the router, only the union's expert rows, x, gates, hidden
        activations, y)."""
        np, cfg = self.np, self.cfg
        cnt = self.count.cpu().numpy().astype(np.int64)
        es = 2 if cfg.dtype == "bf16" else 4
        d, E, de, L, T = cfg.d, cfg.n_experts, cfg.d_expert, cfg.chunk_len, cfg.n_tokens
        C = T // L
        W = (E + 63) // 64
        U = int(cnt.sum())
        mfma = cfg.dtype == "bf16" and d % 128 == 0 and de % 128 == 0  # the library's matrix-core path
        hid = 2 if self.mode in ("auto", "chunk_mfma", "dense") and mfma else 4
        b = {
            "route": C * (E * d * es + E * 4) + T * d * es + T * E * 4 + T * W * 8,
            "union": T * W * 8 + C * (W * 8 + 4 + E * 4),
            "up": U * de * d * es + T * d * es + U * L * 4 + U * L * de * hid,
            "down": U * d * de * es + U * L * de * hid + T * d * 4,
            "stats": T * W * 8,
        }
        active_weight = C * E * d * es + U * 2 * d * de * es
        step_alg = C * E * d * es + U * 2 * d * de * es + T * d * es + T * d * 4
        return b, U, active_weight, step_alg

    def flop_model(self):
        """Algorithmic matrix flops of the grouped kernels (token-expert pairs
        x 2 d d_e each) and the bytes they must move."""
        np, cfg = self.np, self.cfg
        g = self.gates.cpu().numpy()
        P = int((g > 0).sum())
        d, de, E, T = cfg.d, cfg.d_expert, cfg.n_experts, cfg.n_tokens
        return {"pairs": P, "up_flops": 2 * P * d * de, "down_flops": 2 * P * de * d,
                "layer_bytes": 2 * (E * d + 2 * E * d * de) + 4 * E, "x_bytes": 2 * T * d, "y_bytes": 4 * T * d,
                "partial_bytes": 2 * P * d}

def cpu_baseline(cfg, layer, x_host, target_s: float):
    """The oracle as it stands, on the host cores, on a bounded sample of chunks."""
    import oracle
    L = cfg.chunk_len
    C = cfg.n_tokens // L

    def run(n_chunks):
        x = x_host[: n_chunks * L]
        t = time.perf_counter()
        z, g, m = oracle.route(x, layer.w_router, layer.b_router, layer.rms_scale, layer.rms_eps)
        oracle.chunk_union(m, layer.n_experts, L)
        oracle.forward_tokens(x, layer.w_in, layer.w_out, g, m)
        oracle.stats(m, layer.n_experts, L)
        return time.perf_counter() - t

    cores = oracle.num_threads()
    n = max(1, min(C, 8 if L > 1 else 64))
    dt = run(n)
    if dt * cores < target_s and n < C:
        n = int(min(C, max(n + 1, n * target_s / max(dt * cores, 1e-3))))
        dt = run(n)
    reps = 1
    while dt * cores < target_s:  # the whole workload is short: repeat it
        dt += run(n)
        reps += 1
    return {"value": round(reps * n * L / dt, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of {C} chunks ({n * L} tokens) of this workload, layer copy 0, x{reps}: route + union "
                      f"+ per-token forward + stats, fp64 C oracle, {dt:.1f} s on {cores} threads "
                      f"({dt * cores:.0f} CPU-s)"}


def torch_dense_reference_ms(runner, steps: int) -> float:
    """Dense all-experts forward of the whole batch as two vendor GEMMs
    (torch.matmul -> hipBLASLt) over the concatenated experts, on the same
    inputs and gates: the comparison for the grouped path."""
    import torch
    t = runner.dl.tensors(0)
    E, d, de = runner.cfg.n_experts, runner.cfg.d, runner.cfg.d_expert
    w_in_t = t["w_in"].reshape(E * de, d).t().contiguous()                      # [d][E d_e]
    w_out_t = t["w_out"].permute(0, 2, 1).reshape(E * de, d).contiguous()      # [E d_e][d]
    g_rep = runner.gates.repeat_interleave(de, dim=1)
    x = runner.xd

    def fwd():
        h = torch.matmul(x, w_in_t).float()
        h = (torch.nn.functional.silu(h) * g_rep).to(torch.bfloat16)
        return torch.matmul(h, w_out_t)

    for _ in range(2):
        fwd()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fwd()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def torch_dense_chunks_reference(runner, steps: int) -> dict:
    """Dense all-experts forward of every unit through its own layer copy as
    vendor GEMMs (torch.bmm -> hipBLASLt): per sub-batch, one batched product
    of each unit's tokens with its copy's concatenated W_in rows, SiLU times
    the gates, and one batched product with the concatenated W_out rows.  The
    transposed, concatenated weights of every copy are laid out once before
    the timed steps (not timed).  Same inputs and gates as the sparse step;
    the comparison for the chunk workloads.  Returns the forward time and the
    largest difference from the DENSE mode's y of the same kernels on the
    first sub-batch (run just before), relative to its RMS."""
    import torch
    cfg, dl = runner.cfg, runner.dl
    E, d, de, L = cfg.n_experts, cfg.d, cfg.d_expert, cfg.chunk_len
    U = runner.sub_units
    copies = max(1, cfg.replicas)
    w_in_t = torch.empty((U, d, E * de), dtype=torch.bfloat16, device="cuda")   # [copy][d][E d_e]
    w_out_t = torch.empty((U, E * de, d), dtype=torch.bfloat16, device="cuda")  # [copy][E d_e][d]
    for r in range(U):
        t = dl.tensors(r % copies)
        w_in_t[r].copy_(t["w_in"].reshape(E * de, d).t())
        w_out_t[r].copy_(t["w_out"].permute(0, 2, 1).reshape(E * de, d))
    C = cfg.n_tokens // L
    subs = []
    for b in range(runner.n_sub):
        c0, c1 = b * U, min(C, (b + 1) * U)
        n = c1 - c0
        x = runner.xd[c0 * L:c1 * L].view(n, L, d)
        g = runner.gates[c0 * L:c1 * L].view(n, L, E).repeat_interleave(de, dim=2)
        subs.append((x, g, n))
    y_ref = runner.y[:subs[0][2] * L].clone()  # the DENSE mode's y of the first sub-batch
    outs = [None] * len(subs)

    def fwd():
        for k, (x, g, n) in enumerate(subs):
            h = torch.bmm(x, w_in_t[:n])
            h = (torch.nn.functional.silu(h.float()) * g).to(torch.bfloat16)
            outs[k] = torch.bmm(h, w_out_t[:n])

    for _ in range(2):
        fwd()
    torch.cuda.synchronize()
    y0 = outs[0].reshape(-1, d).float()
    rms = float(y_ref.pow(2).mean().sqrt())
    diff = float((y0 - y_ref).abs().max()) / rms if rms > 0 else 0.0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fwd()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del w_in_t, w_out_t, subs, outs
    torch.cuda.empty_cache()
    return {"forward_ms": ms, "max_rel_diff_vs_dense_mode": diff}


def torch_dense_backward_ms(runner, dy, steps: int) -> float:
    """The dense all-experts layer's backward through torch autograd (hipBLASLt
    bf16 GEMMs over the concatenated experts, gates recomputed from z): the
    comparison for blockffn_backward on the same batch."""
    import torch
    t = runner.dl.tensors(0)
    E, d, de = runner.cfg.n_experts, runner.cfg.d, runner.cfg.d_expert
    w_in_t = t["w_in"].reshape(E * de, d).t().contiguous().requires_grad_(True)   # [d][E d_e]
    w_out = t["w_out"].permute(0, 2, 1).reshape(E * de, d).contiguous().requires_grad_(True)
    w_r = t["w_router"].detach().clone().float().requires_grad_(True)
    b = t["b_router"].detach().clone().requires_grad_(True)
    x = runner.xd.detach().clone().requires_grad_(True)
    dyb = dy.to(torch.bfloat16)
    eps = runner.layer.rms_eps

    def step():
        z = x.float() @ w_r.t() + b
        a = torch.relu(z)
        g = a / torch.sqrt((a * a).mean(dim=1, keepdim=True) + eps)
        u = torch.matmul(x, w_in_t)
        h = (torch.nn.functional.silu(u.float()) * g.repeat_interleave(de, dim=1)).to(torch.bfloat16)
        y = torch.matmul(h, w_out)
        y.backward(dyb)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def backward_measure(runner, steps: int, warmup: int, dense_steps: int) -> dict:
    """Times blockffn_backward on the workload's batch (one layer), with the
    library's stage events, and reports algorithmic matrix flops."""
    import numpy as np
    import torch
    B, cfg = runner.B, runner.cfg
    T, d, E, de = cfg.n_tokens, cfg.d, cfg.n_experts, cfg.d_expert
    _, _, z = B.blockffn_route(runner.dl, runner.xd, cfg.chunk_len, n_layers=1, want_preact=True)
    dy = torch.from_numpy(np.random.default_rng(cfg.seed + 100).standard_normal((T, d)).astype(np.float32)).cuda()
    ws = B.alloc_backward_workspace(runner.dl, T)
    out = B.blockffn_backward(runner.dl, runner.xd, z, dy, workspace=ws)
    for _ in range(warmup):
        B.blockffn_backward(runner.dl, runner.xd, z, dy, workspace=ws, dx=out["dx"],
                            grads={k: v for k, v in out.items() if k != "dx"})
    torch.cuda.synchronize()
    names = ("plan", "pair", "weights", "dx_rows", "combine")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
    for row in ev:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    handles = [(ctypes.c_void_p * len(row))(*[e.cuda_event for e in row]) for row in ev]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(steps):
        runner.lib.blockffn_set_stage_events(ctypes.cast(handles[k], ctypes.c_void_p), len(names) + 1)
        B.blockffn_backward(runner.dl, runner.xd, z, dy, workspace=ws, dx=out["dx"],
                            grads={k2: v for k2, v in out.items() if k2 != "dx"})
        runner.lib.blockffn_set_stage_events(None, 0)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    stage = {n: round(sum(ev[k][j].elapsed_time(ev[k][j + 1]) for k in range(steps)) / steps, 5)
             for j, n in enumerate(names)}
    P = int((z > 0).sum().item())
    flops = 10 * P * d * de + 2 * T * E * d   # U, Q, dW_in, dW_out, dx rows; dW_r
    res = {"ms": round(ms, 5), "stage_ms": stage, "pairs": P, "algorithmic_flops": flops,
           "tflops": round(flops / ms / 1e9, 1), "frac_of_bf16_mfma_peak": round(flops / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4)}
    # the CLS-aware objectives (alpha 8, both weights 1) and a backward that takes their dz
    losses, dzx = B.blockffn_cls_losses(E, z, cfg.chunk_len, 8.0)
    grads = {k2: v for k2, v in out.items() if k2 != "dx"}

    def timed_ms(fn, n):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    res["cls_losses_ms"] = round(timed_ms(lambda: B.blockffn_cls_losses(E, z, cfg.chunk_len, 8.0, losses=losses,
                                                                        dz=dzx), steps), 5)
    res["ms_with_cls_gradient"] = round(timed_ms(lambda: B.blockffn_backward(
        runner.dl, runner.xd, z, dy, workspace=ws, dx=out["dx"], grads=grads, dz_extra=dzx), steps), 5)
    if dense_steps > 0:
        dms = torch_dense_backward_ms(runner, dy, dense_steps)
        res["torch_dense_autograd_ms"] = round(dms, 4)
        res["speedup_vs_dense_autograd"] = round(dms / ms, 3)
    return res


def measure_ceilings(gemm: bool) -> dict:
    """Measured ceilings the achieved figures are also set against: the HBM
    streaming-read probe (blockffn_read_probe over 8 GiB, best over grid
    sizes) and, for matrix-core workloads, a large bf16 GEMM through
    torch.matmul (hipBLASLt)."""
    import torch
    from activation_sparse_moe_amd import binding as B
    n = 8 << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    best, best_blocks = 0.0, 0
    for blocks in (0, 2048, 4096, 8192, 16384):
        B.blockffn_read_probe(buf, sink, blocks)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            B.blockffn_read_probe(buf, sink, blocks)
        e1.record()
        torch.cuda.synchronize()
        gbs = n / (e0.elapsed_time(e1) / 3 * 1e-3) / 1e9
        if gbs > best:
            best, best_blocks = gbs, blocks
    del buf
    out = {"hbm_read_gbs": round(best, 1), "hbm_read_probe": f"blockffn_read_probe, 8 GiB, {best_blocks or 'resident'} blocks"}
    if gemm:
        m = 8192
        a = torch.randn((m, m), device="cuda").to(torch.bfloat16)
        b = torch.randn((m, m), device="cuda").to(torch.bfloat16)
        torch.matmul(a, b)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            torch.matmul(a, b)
        e1.record()
        torch.cuda.synchronize()
        out["bf16_gemm_tflops"] = round(2 * m ** 3 / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e12, 1)
        out["bf16_gemm"] = f"torch.matmul (hipBLASLt) {m} x {m} x {m} bf16"
        del a, b
    torch.cuda.empty_cache()
    return out


def latency_measure(runner, units: int, mode: str) -> dict:
    """Latency mode: `units` units run one after another, each unit through
    its own layer copy, the chain captured in one HIP graph and replayed;
    per-unit latency = replay time / units.  Two chains: one
    blockffn_layer_forward call per unit (router, union, forward and
    statistics in one call), and the four separate calls per unit."""
    import torch
    B, cfg = runner.B, runner.cfg
    L, E = cfg.chunk_len, cfg.n_experts
    C = cfg.n_tokens // L
    units = min(units, C)
    views = [runner.dl.single_copy(u % max(1, cfg.replicas)) for u in range(units)]
    ws = B.alloc_workspace(views[0], L, L, mode)
    step_ws = torch.empty(max(B.blockffn_layer_forward_workspace_size(views[0], L, L), 256), dtype=torch.uint8,
                          device="cuda")

    def separate():
        for u in range(units):
            t0, t1 = u * L, (u + 1) * L
            x, g, m = runner.xd[t0:t1], runner.gates[t0:t1], runner.masks[t0:t1]
            cnt, lst, um = runner.count[u:u + 1], runner.lst[u:u + 1], runner.umask[u:u + 1]
            B.blockffn_route(views[u], x, L, gates=g, token_masks=m)
            B.blockffn_chunk_union(E, m, L, chunk_masks=um, active_count=cnt, active_list=lst)
            B.blockffn_forward(views[u], x, L, g, cnt, lst, mode=mode, workspace=ws, y=runner.y[t0:t1])
            B.blockffn_sparsity_stats(E, m, L, stats_dev=runner.stats)

    outs = []
    for u in range(units):
        t0, t1 = u * L, (u + 1) * L
        outs.append({"gates": runner.gates[t0:t1], "token_masks": runner.masks[t0:t1], "preact": None,
                     "chunk_masks": runner.umask[u:u + 1], "active_count": runner.count[u:u + 1],
                     "active_list": runner.lst[u:u + 1], "stats": runner.stats, "workspace": step_ws,
                     "y": runner.y[t0:t1]})

    def one_call():
        for u in range(units):
            B.blockffn_layer_forward(views[u], runner.xd[u * L:(u + 1) * L], L, out=outs[u])

    def per_unit_us(chain):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            chain()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            chain()
        graph.replay()
        torch.cuda.synchronize()
        reps = 5
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        del graph
        return e0.elapsed_time(e1) / reps / units * 1e3

    us_sep = per_unit_us(separate)
    us_one = per_unit_us(one_call)
    # the four-kernel step adds its counters and router partials to the split forward's workspace
    fused = B.blockffn_layer_forward_workspace_size(views[0], L, L) != B.blockffn_workspace_size(views[0], L, L)
    return {"us_per_unit": round(us_one, 2), "us_per_unit_separate_calls": round(us_sep, 2),
            "units_chained": units, "tokens_per_unit": L,
            "kernels_per_unit": 3 if fused else None,
            "kind": "units one after another, each through its own layer copy, one HIP graph per chain; "
                    "us_per_unit: one blockffn_layer_forward call per unit; separate: route, union, forward "
                    f"({mode}), stats"}


def copy_calibration():
    """A plain device copy of 1 GiB: its FETCH_SIZE / WRITE_SIZE counters
    scale the expert kernels' counters to bytes."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    torch.cuda.empty_cache()


def fff_byte_model(cfg) -> dict:
    """Algorithmic HBM bytes of one FFF forward over the batch: every visited
    node's two rows, each token's x, and its fp32 output row."""
    per_token_nodes = cfg.n_trees * (cfg.depth + 1) * cfg.node_bytes
    io = cfg.d * cfg.elt_bytes + 4 * cfg.d
    return {"per_token": per_token_nodes + io, "node_bytes_per_token": per_token_nodes,
            "step": cfg.tokens * (per_token_nodes + io),
            "dense_per_token": cfg.n_trees * cfg.nodes * cfg.node_bytes + io}


def fff_cpu_baseline(cfg, layer, x_host, target_s: float):
    """The FFF oracle as it stands, on the host cores, on a bounded sample of tokens."""
    import oracle

    def run(n):
        t = time.perf_counter()
        oracle.fff_forward(x_host[:n], layer.w_node, layer.b_node, layer.w_out, want_paths=False)
        return time.perf_counter() - t

    cores = oracle.num_threads()
    n = min(64, cfg.tokens)
    dt = run(n)
    if dt * cores < target_s and n < cfg.tokens:
        n = int(min(cfg.tokens, max(n + 1, n * target_s / max(dt * cores, 1e-3))))
        dt = run(n)
    reps = 1
    while dt * cores < target_s:  # the whole workload is short: repeat it
        dt += run(n)
        reps += 1
    return {"value": round(reps * n / dt, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of {cfg.tokens} tokens of this workload, layer copy 0, x{reps}: the tree walk and "
                      f"output sum, fp64 C oracle, {dt:.1f} s on {cores} threads ({dt * cores:.0f} CPU-s)"}


def torch_dense_fff_ms(dl, xd, n: int, reps: int) -> float:
    """The dense feed-forward block the tree layer replaces (every node of
    every tree, GELU, output projection), for n tokens each through its own
    layer copy, as two batched vendor GEMMs (torch.bmm -> hipBLASLt)."""
    import torch
    rows = dl.rows
    w_node = dl.rows_view("w_node", 0, n)                                    # [n][rows][d], row stride node_stride
    w_out = dl.rows_view("w_out", 0, n)
    t0 = dl.tensors(0)
    b = t0["b_node"].reshape(-1).as_strided((n, rows, 1), (dl.stride // 4, 1, 1)) if t0["b_node"] is not None \
        else None
    x = xd[:n].unsqueeze(2).contiguous()                                      # [n][d][1]

    def fwd():
        c = torch.bmm(w_node, x).float()                                      # [n][rows][1]
        if b is not None:
            c = c + b
        a = torch.nn.functional.gelu(c).to(xd.dtype).reshape(n, 1, rows)
        return torch.bmm(a, w_out)                                            # [n][1][d]

    fwd()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fwd()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def fff_latency(dl, xd, units: int) -> dict:
    """Latency mode: single tokens one after another, each through its own
    layer copy, the chain captured in one HIP graph (per-token latency =
    replay time / units); beside it the dense block for one token as two
    torch.bmm calls, chained the same way."""
    import torch
    from activation_sparse_moe_amd import binding as B
    views = [dl.single_copy(u) for u in range(units)]
    ws = B.alloc_fff_workspace(views[0], 1)
    y = torch.empty((units, dl.d), dtype=torch.float32, device="cuda")
    rows = dl.rows
    wn = [v.rows_view("w_node") for v in views]
    wo = [v.rows_view("w_out") for v in views]
    bias = [v.tensors(0)["b_node"] for v in views]
    xs = [xd[u:u + 1].unsqueeze(2).contiguous() for u in range(units)]

    def sparse_chain():
        for u in range(units):
            B.blockffn_fff_forward(views[u], xd[u:u + 1], y=y[u:u + 1], workspace=ws)

    def dense_chain():
        for u in range(units):
            c = torch.bmm(wn[u], xs[u]).float()
            if bias[u] is not None:
                c = c + bias[u].reshape(1, rows, 1)
            a = torch.nn.functional.gelu(c).to(xd.dtype).reshape(1, 1, rows)
            torch.bmm(a, wo[u])

    out = {}
    for name, chain in (("us_per_token", sparse_chain), ("dense_torch_bmm_us_per_token", dense_chain)):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            chain()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            chain()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        out[name] = round(e0.elapsed_time(e1) / 3 / units * 1e3, 2)
    out["speedup_vs_dense"] = round(out["dense_torch_bmm_us_per_token"] / out["us_per_token"], 2)
    out.update({"tokens_chained": units, "blocks_per_token": _fff_split(views[0], 1),
                "kind": "tokens one after another, each through its own layer copy, one HIP graph per chain"})
    return out


def _fff_split(layer, n_tokens: int) -> int:
    """Blocks per token the library uses (workspace bytes / (T d 4), at least 1)."""
    from activation_sparse_moe_amd import binding as B
    nb = B.blockffn_fff_workspace_size(layer, n_tokens, 0)
    return max(1, nb // (n_tokens * layer.d * 4))


def fff_main(args, cfg) -> int:
    import torch
    from activation_sparse_moe_amd import binding as B
    from activation_sparse_moe_amd._capi import BF16, F32
    from workload import make_fff_workload

    mode = args.mode or "sparse"
    if mode not in ("sparse", "dense"):
        print(f"FFF workloads take --mode sparse or dense, not {mode!r}", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
    layer, x = make_fff_workload(cfg)
    dl = B.DeviceFffLayer.from_workload(layer, replicas=cfg.replicas)
    xd = B.tokens_to_device(x, F32 if cfg.dtype == "f32" else BF16)
    T = cfg.tokens
    y = torch.empty((T, cfg.d), dtype=torch.float32, device="cuda")
    ws = B.alloc_fff_workspace(dl, T, args.fff_split)
    fwd = lambda: B.blockffn_fff_forward(dl, xd, mode=mode, y=y, split=args.fff_split, workspace=ws)  # noqa: E731

    # eager launches, each bracketed by events on the launch stream: the
    # kernel's average duration for the roofline
    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start.record()
    for a, b in ev:
        a.record()
        fwd()
        b.record()
    t_end.record()
    torch.cuda.synchronize()
    kernel_ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    eager_ms = t_start.elapsed_time(t_end) / args.steps
    ms = eager_ms
    if not args.eager:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fwd()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            fwd()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps

    bm = fff_byte_model(cfg)
    step_bytes = bm["step"] if mode == "sparse" else T * bm["dense_per_token"]
    achieved = step_bytes / (kernel_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "kernel": f"fff_walk ({mode})", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": profiled_traffic("fff_walk", cfg.name) if mode == "sparse" else None,
                "algorithmic_bytes_per_launch": step_bytes, "avg_launch_ms": round(kernel_ms, 5),
                "launches_per_step": 1}

    dense = None
    if args.dense_steps > 0 and mode == "sparse":
        n = min(256, T, cfg.replicas)
        yd = torch.empty((n, cfg.d), dtype=torch.float32, device="cuda")
        B.blockffn_fff_forward(dl, xd[:n], mode="dense", y=yd)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.dense_steps):
            B.blockffn_fff_forward(dl, xd[:n], mode="dense", y=yd)
        e1.record()
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / args.dense_steps
        tms = torch_dense_fff_ms(dl, xd, n, args.dense_steps)
        dense_tps, torch_tps = n / (dms * 1e-3), n / (tms * 1e-3)
        dense = {"kind": "every node of every tree (the dense block of width P N) on the first "
                         f"{n} tokens, each through its own layer copy",
                 "same_kernel_tokens_per_s": round(dense_tps, 1),
                 "same_kernel_gbs": round(n * bm["dense_per_token"] / (dms * 1e-3) / 1e9, 1),
                 "torch_bmm_tokens_per_s": round(torch_tps, 1),
                 "speedup_vs_same_kernel": round(T / (ms * 1e-3) / dense_tps, 2),
                 "speedup_vs_torch_bmm": round(T / (ms * 1e-3) / torch_tps, 2),
                 "ideal_byte_ratio": round(bm["dense_per_token"] / bm["per_token"], 2)}

    latency = None
    if args.latency_units > 0 and mode == "sparse":
        latency = fff_latency(dl, xd, min(args.latency_units, T, cfg.replicas))
    ceilings = None
    if not args.no_ceilings:
        del dl
        torch.cuda.empty_cache()
        ceilings = measure_ceilings(gemm=False)
        roofline["frac_of_measured_ceiling"] = round(roofline["achieved"] / ceilings["hbm_read_gbs"], 4)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = fff_cpu_baseline(cfg, layer, x, args.cpu_seconds)
    step_gbs = step_bytes / (ms * 1e-3) / 1e9
    out = {
        "metric": FFF_METRIC, "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0, 1/d) node rows and N(0, I) tokens)",
        "config": {"workload": cfg.name, "d": cfg.d, "n_trees": cfg.n_trees, "depth": cfg.depth,
                   "nodes_per_tree": cfg.nodes, "tokens": T, "layer_copies": cfg.replicas, "mode": mode,
                   "activation": "gelu_nodes"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "visited_node_gbs": round(step_gbs, 1),
        "visited_node_frac_of_peak": round(step_gbs / HBM_PEAK_GBS, 4),
        "sparsity": {"nodes_visited_per_token": cfg.n_trees * (cfg.depth + 1),
                     "fraction_idle": round(1 - (cfg.depth + 1) / cfg.nodes, 4)},
        "dense": dense,
        "latency": latency,
        "ceilings": ceilings,
        "timing": {"steps": "eager launches" if args.eager else "HIP graph replay of the forward",
                   "eager_ms_per_step": round(eager_ms, 5), "kernel_ms": round(kernel_ms, 5)},
        "source_digest": source_digest(),
        "build_digest": _build_digest(),
    }
    print(json.dumps(out), flush=True)
    return 0


def main(argv=None) -> int:
    args = parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    from workload import FFF_CONFIGS, get_config

    if args.workload in FFF_CONFIGS:
        return fff_main(args, FFF_CONFIGS[args.workload])
    cfg = get_config(args.workload)
    mode = args.mode or cfg.mode
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
    runner = StepRunner(cfg, mode, args.router, args.top_k)
    # eager steps, instrumented: per-kernel times for the roofline
    _, avg = runner.timed(mode, args.steps, args.warmup)
    eager_ms = runner.eager_ms(mode, args.steps, args.warmup)
    # the timed steps: each whole step (every sub-batch) replayed from a HIP
    # graph, so host launch overhead is not in the figure (--eager: eager)
    ms = eager_ms if args.eager else runner.graph_ms(mode, args.steps, args.warmup)
    # the forward alone (planning and expert kernels of every sub-batch), replayed from a graph: the
    # figure the dense comparisons divide by
    avg["forward"] = runner.graph_ms(mode, args.steps, args.warmup, forward_only=True)
    from activation_sparse_moe_amd import binding as B
    st = B.stats_dict(runner.stats)
    bytes_per, U, active_weight, step_alg = runner.byte_model()
    T = cfg.n_tokens
    value = T / (ms / 1e3)

    dense = None
    grouped = mode == "grouped"
    if args.dense_steps > 0 and grouped:
        dfwd = torch_dense_reference_ms(runner, args.dense_steps)
        dense = {"kind": "torch.matmul (hipBLASLt) dense GEMMs over all experts", "forward_ms": round(dfwd, 4),
                 "speedup_forward": round(dfwd / avg["forward"], 3) if "forward" in avg else None}
    elif args.dense_steps > 0:
        dms = runner.eager_ms("dense", args.dense_steps, 1) if args.eager else runner.graph_ms("dense", args.dense_steps, 1)
        davg = {"forward": runner.graph_ms("dense", args.dense_steps, 1, forward_only=True)}
        dense = {"kind": "same kernels, every expert (BLOCKFFN_MODE_DENSE)", "ms_per_step": round(dms, 4),
                 "speedup_step": round(dms / ms, 3)}
        if "forward" in davg and "forward" in avg:
            dense.update({"forward_ms": round(davg["forward"], 4),
                          "speedup_forward": round(davg["forward"] / avg["forward"], 3)})
        if cfg.dtype == "bf16":
            vend = torch_dense_chunks_reference(runner, args.dense_steps)
            sparse_fwd = avg.get("forward", sum(avg[k] for k in ("up", "down") if k in avg))
            dense["vendor"] = {
                "kind": "torch.bmm (hipBLASLt) per sub-batch over each unit's layer copy, concatenated experts",
                "forward_ms": round(vend["forward_ms"], 4),
                "speedup_forward": round(vend["forward_ms"] / sparse_fwd, 3),
                "max_rel_diff_vs_dense_mode": round(vend["max_rel_diff_vs_dense_mode"], 5)}

    dom = "up" if avg["up"] >= avg["down"] else "down"
    kernel_name = {"up": "expert_up", "down": "expert_down"}[dom]
    if grouped:
        fm = runner.flop_model()
        fl = fm[f"{dom}_flops"]
        achieved = fl / (avg[dom] * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": f"grouped_{dom} ({mode})", "achieved": round(achieved, 1),
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                    "traffic": profiled_traffic(f"grouped_{dom}", cfg.name),
                    "algorithmic_flops_per_launch": fl, "avg_launch_ms": round(avg[dom], 5), "launches_per_step": 1}
    else:
        achieved = bytes_per[dom] / (avg[dom] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": f"{kernel_name} ({mode})", "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": profiled_traffic(kernel_name, cfg.name),
                    "algorithmic_bytes_per_launch": bytes_per[dom] // runner.n_sub,
                    "avg_launch_ms": round(avg[dom] / runner.n_sub, 5), "launches_per_step": runner.n_sub}


    backward = None
    if args.backward:
        backward = backward_measure(runner, args.steps, args.warmup, args.dense_steps)

    latency = None
    if args.latency_units > 0 and not grouped:
        latency = latency_measure(runner, args.latency_units, mode)
    ceilings = None
    if not args.no_ceilings:
        ceilings = measure_ceilings(gemm=grouped)
        if grouped and "bf16_gemm_tflops" in ceilings:
            roofline["frac_of_measured_ceiling"] = round(roofline["achieved"] / ceilings["bf16_gemm_tflops"], 4)
        elif not grouped:
            roofline["frac_of_measured_ceiling"] = round(roofline["achieved"] / ceilings["hbm_read_gbs"], 4)

    cpu = None
    if not args.no_cpu_baseline and args.router == "blockffn":
        cpu = cpu_baseline(cfg, runner.layer, runner.x_host, args.cpu_seconds)

    if grouped:
        # each expert's weights are read once for the whole batch
        fm = runner.flop_model()
        step_alg = fm["layer_bytes"] + fm["x_bytes"] + fm["y_bytes"]
    step_gbs = step_alg / (ms * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic (seeded generator shaped to the pages' sparsity)",
        "config": {"workload": cfg.name, "d": cfg.d, "n_experts": cfg.n_experts, "d_expert": cfg.d_expert,
                   "chunk_len": cfg.chunk_len, "chunks": T // cfg.chunk_len, "tokens": T,
                   "layer_copies": cfg.replicas, "mode": mode,
                   "router": args.router if args.router != "topk_softmax" else f"topk_softmax(k={args.top_k})"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "active_weight_gbs": round(step_gbs, 1),
        "active_weight_frac_of_peak": round(step_gbs / HBM_PEAK_GBS, 4),
        "kernel_ms": {k: round(v, 5) for k, v in avg.items()},
        "kernel_gbs": ({k: round(bytes_per[k] / (avg[k] * 1e-3) / 1e9, 1) for k in bytes_per if k in avg}
                       if not grouped else None),
        "grouped": (dict(runner.flop_model(), up_tflops=round(runner.flop_model()["up_flops"] / avg["up"] / 1e9, 1),
                         down_tflops=round(runner.flop_model()["down_flops"] / avg["down"] / 1e9, 1))
                    if grouped else None),
        "dense": dense,
        "timing": {"steps": "eager launches" if args.eager else "HIP graph replay of each whole step",
                   "eager_ms_per_step": round(eager_ms, 5),
                   "kernel_ms": "eager steps with HIP events around each launch; forward: the forward calls alone "
                                "(planning and expert kernels, every sub-batch) replayed from a HIP graph"},
        "backward": backward,
        "latency": latency,
        "ceilings": ceilings,
        "sparsity": {"tls": round(st["tls"], 4), "cls": round(st["cls"], 4), "mean_union": round(U / (T // cfg.chunk_len), 2),
                     "reuse": round(st["reuse"], 4)},
        "source_digest": source_digest(),
        "build_digest": _build_digest(),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
