"""Workload shapes for the BlockFFN layer forward.

The pages (the BlockFFN write-up on lsdiaocha.cn, §3 and §5, and the arXiv
2507.08771 abstract) report trained layers with token-level sparsity above 80%
and 8-token chunk-level sparsity above 70%, verified by speculative decoding
with chunks of up to 32 candidate tokens (write-up §4).  No trained weights or
benchmark data are available, so every workload below is synthetic, shaped to
land on those sparsity levels:

* ``bias_k`` sets each expert's router bias to ``-bias_k`` times the standard
  deviation of its pre-activation, so a token activates an expert with
  probability ``1 - Phi(bias_k)``.
* ``alpha`` mixes a per-chunk base vector into every token of the chunk, which
  is what makes consecutive tokens share experts (chunk-level sparsity).

``units`` counts independent pieces of work: tokens when ``chunk_len == 1``,
chunks otherwise.
"""
from __future__ import annotations

from dataclasses import dataclass
from statistics import NormalDist

_PHI_INV = NormalDist().inv_cdf


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    d: int            # hidden size
    n_experts: int    # E
    d_expert: int     # d_e, hidden width of one expert MLP
    dtype: str        # "f32" or "bf16": weights and tokens
    chunk_len: int    # L
    units: int        # chunks (or tokens when L == 1)
    bias_k: float     # router bias = -bias_k * std(pre-activation)
    alpha: float      # chunk-base mixing weight (0 = independent tokens)
    seed: int
    mode: str = "auto"  # forward mode the workload exercises
    # Distinct device copies of the layer used when the workload is timed:
    # chunk c streams copy c % replicas, so no two chunks of one launch read
    # the same weight bytes (a chunk passing through a deep stack of distinct
    # layers).  1 for the batched workload, which runs every chunk through one
    # layer on purpose.
    replicas: int = 1

    @property
    def n_tokens(self) -> int:
        return self.units * self.chunk_len

    @property
    def expert_bytes(self) -> int:
        """Bytes of one expert's two matrices (W_in and W_out)."""
        return 2 * self.d * self.d_expert * (4 if self.dtype == "f32" else 2)

    @property
    def router_bytes(self) -> int:
        return self.d * self.n_experts * (4 if self.dtype == "f32" else 2)

    @property
    def layer_bytes(self) -> int:
        return self.router_bytes + self.n_experts * self.expert_bytes + 2 * 4 * self.n_experts


# Router bias for about 12 of 64 experts active per token (81.25% TLS).
_K_12_OF_64 = _PHI_INV(1.0 - 12.0 / 64.0)
# Router bias for 15% of experts active per token (85% TLS).
_K_15PCT = _PHI_INV(0.85)

CONFIGS: dict[str, WorkloadConfig] = {
    c.name: c
    for c in [
        # Tiny fp32 layer, the case the oracle and brute force finish in seconds.
        WorkloadConfig("tiny_f32_L4", d=64, n_experts=8, d_expert=16, dtype="f32",
                       chunk_len=4, units=16, bias_k=0.8, alpha=0.7, seed=1),
        # Single-token decode: 4096 independent tokens, bandwidth-bound GEMV.
        WorkloadConfig("decode_L1_d2048_E64", d=2048, n_experts=64, d_expert=128,
                       dtype="bf16", chunk_len=1, units=4096, bias_k=_K_12_OF_64,
                       alpha=0.0, seed=2, replicas=512),
        # Speculative-verify chunk of 8 tokens, 512 chunks (about 19 of 64 experts per chunk).
        WorkloadConfig("chunk8_d2048_E64", d=2048, n_experts=64, d_expert=128,
                       dtype="bf16", chunk_len=8, units=512, bias_k=_K_12_OF_64,
                       alpha=0.8, seed=3, replicas=512),
        # Larger layer, chunks of 8 and of 32 tokens, 256 chunks each.
        WorkloadConfig("large_L8_d4096_E128", d=4096, n_experts=128, d_expert=128,
                       dtype="bf16", chunk_len=8, units=256, bias_k=_K_15PCT,
                       alpha=0.647, seed=4, replicas=256),
        WorkloadConfig("large_L32_d4096_E128", d=4096, n_experts=128, d_expert=128,
                       dtype="bf16", chunk_len=32, units=256, bias_k=_K_15PCT,
                       alpha=0.647, seed=4, replicas=256),
        # Prefill-like batch: 4096 tokens as 512 chunks of 8 through one layer,
        # token-expert pairs grouped by expert.
        WorkloadConfig("batched_L8_d4096_E128", d=4096, n_experts=128, d_expert=128,
                       dtype="bf16", chunk_len=8, units=512, bias_k=_K_15PCT,
                       alpha=0.647, seed=5, mode="grouped"),
    ]
}


def get_config(name: str) -> WorkloadConfig:
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}") from None
