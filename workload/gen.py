"""Seeded generator of BlockFFN layers and token streams.

One fixed definition, so that every consumer sees the same bits for a seed:

* Random source: ``numpy.random.default_rng(seed)`` (PCG64).  Draw order:
  router, expert input matrices, expert output matrices, chunk bases, token
  noise; every draw is float32 standard normal.
* Weights are N(0, 1/fan_in): the router ``W_r`` and every ``W_in`` have
  fan-in ``d``, every ``W_out`` has fan-in ``d_e``.  For bf16 workloads each
  float32 draw is rounded to bfloat16 (round to nearest, ties to even) and kept
  as its 16-bit pattern.
* Router bias ``b_i = -k * ||W_r[i]||_2``, computed on the stored (rounded)
  weights: ``||W_r[i]||_2`` is the standard deviation of expert ``i``'s
  pre-activation for a unit-variance token, so ``k`` sets how often the expert
  fires.  RMSNorm scale: none (unit), epsilon 1e-6.
* Tokens: ``x_t = (a * base_c + (1 - a) * n_t) / sqrt(a^2 + (1 - a)^2)`` with
  ``base_c`` shared by the chunk and ``n_t`` per token, both N(0, I).  Every
  coordinate has unit variance and two tokens of one chunk have Pearson
  correlation ``a^2 / (a^2 + (1 - a)^2)``.

Storage layout (row-major, the nn.Linear [out][in] convention, so each
expert's rows are contiguous): ``w_router[E][d]``, ``w_in[E][d_e][d]``,
``w_out[E][d][d_e]``, ``x[T][d]``.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import WorkloadConfig


def bf16_round_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Layer:
    dtype: str                 # "f32" (arrays are float32) or "bf16" (arrays are uint16 bit patterns)
    w_router: np.ndarray       # [E][d]
    b_router: np.ndarray       # [E] float32
    rms_scale: Optional[np.ndarray]  # [E] float32, or None for unit scale
    w_in: np.ndarray           # [E][d_e][d]
    w_out: np.ndarray          # [E][d][d_e]
    rms_eps: float = 1e-6

    @property
    def d(self) -> int:
        return self.w_router.shape[1]

    @property
    def n_experts(self) -> int:
        return self.w_router.shape[0]

    @property
    def d_expert(self) -> int:
        return self.w_in.shape[1]


@dataclass
class Tokens:
    x: np.ndarray              # [T][d], float32 or uint16 bf16 bits
    chunk_len: int


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":
        return bf16_round_bits(a)
    raise ValueError(f"unknown dtype {dtype!r}")


def _as_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    return a if dtype == "f32" else bf16_bits_to_f32(a)


def make_layer(d: int, n_experts: int, d_expert: int, dtype: str, bias_k: float,
               rng: np.random.Generator) -> Layer:
    w_r = rng.standard_normal((n_experts, d), dtype=np.float32) * np.float32(1.0 / np.sqrt(d))
    w_r = _store(w_r, dtype)
    w_in = rng.standard_normal((n_experts, d_expert, d), dtype=np.float32)
    w_in *= np.float32(1.0 / np.sqrt(d))
    w_in = _store(w_in, dtype)
    w_out = rng.standard_normal((n_experts, d, d_expert), dtype=np.float32)
    w_out *= np.float32(1.0 / np.sqrt(d_expert))
    w_out = _store(w_out, dtype)
    norms = np.sqrt((_as_f32(w_r, dtype).astype(np.float64) ** 2).sum(axis=1))
    b = (-bias_k * norms).astype(np.float32)
    return Layer(dtype=dtype, w_router=w_r, b_router=b, rms_scale=None, w_in=w_in, w_out=w_out)


def make_tokens(d: int, n_chunks: int, chunk_len: int, alpha: float, dtype: str,
                rng: np.random.Generator) -> Tokens:
    base = rng.standard_normal((n_chunks, d), dtype=np.float32)
    noise = rng.standard_normal((n_chunks * chunk_len, d), dtype=np.float32)
    a = np.float32(alpha)
    scale = np.float32(1.0 / np.sqrt(alpha * alpha + (1.0 - alpha) ** 2))
    x = (a * np.repeat(base, chunk_len, axis=0) + (np.float32(1.0) - a) * noise) * scale
    return Tokens(x=_store(x, dtype), chunk_len=chunk_len)


def make_workload(cfg: WorkloadConfig, units: Optional[int] = None) -> tuple[Layer, Tokens]:
    """Layer and token stream for a workload; ``units`` overrides the chunk count."""
    rng = np.random.default_rng(cfg.seed)
    layer = make_layer(cfg.d, cfg.n_experts, cfg.d_expert, cfg.dtype, cfg.bias_k, rng)
    n = cfg.units if units is None else units
    tokens = make_tokens(cfg.d, n, cfg.chunk_len, cfg.alpha, cfg.dtype, rng)
    return layer, tokens
