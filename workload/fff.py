"""Seeded synthetic workloads for the FFF tree layer (P parallel perfect binary
trees of depth D with hard routing; "Dynamic sparsity in tree-structured
feed-forward layers at scale", write-up on gist.science, §2 and §4).

Like the rest of this package it draws weights and tokens and holds none of
the layer's arithmetic.

Shapes.  The write-up evaluates OPT-1.3B with depth-6 trees (about 94% of the
block idle per token) and quotes a layer-level speed-up over the dense
feed-forward block.  OPT-1.3B has model width 2048 and a feed-forward width of
8192; 64 trees of depth 6 hold 64 x 127 = 8128 nodes, the closest tree layer
of that width, so the timed workload is d = 2048, P = 64, D = 6 in bf16.  No
trained weights or text are available: the weights and tokens are synthetic.

Definition (one fixed draw order for a seed, numpy default_rng / PCG64,
float32 standard normal draws):

* ``w_node[P][N][d]`` ~ N(0, 1/d): fan-in d, so a unit-variance token gives
  pre-activations of unit variance and each turn is a fair coin.
* ``b_node[P][N]`` ~ U(-1/sqrt(d), 1/sqrt(d)), the default bias of a linear
  layer with fan-in d.
* ``w_out[P][N][d]`` ~ N(0, 1/(P (D + 1))): each token sums P (D + 1) node
  rows, so the output has a variance of the order of one.
* tokens ``x[T][d]`` ~ N(0, I), independent (one token per unit, as in
  decoding).
* bf16 workloads round every float32 draw to bfloat16 (nearest, ties to even)
  and keep the 16-bit patterns; the bias stays float32.

Storage: node-major rows, ``w_node[p][n]`` and ``w_out[p][n]`` contiguous, in
heap order within a tree (root 0, children of n at 2n + 1 and 2n + 2).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .gen import _store


@dataclass(frozen=True)
class FffConfig:
    name: str
    d: int            # model width
    n_trees: int      # P
    depth: int        # D: levels 0..D, 2^(D+1) - 1 nodes per tree
    dtype: str        # "f32" or "bf16"
    tokens: int       # tokens per step (one unit each)
    seed: int
    # Distinct device copies of the layer when timed: token t reads copy
    # t % replicas, so no two tokens resident at once share node rows (a
    # token passing through a stack of distinct layers).
    replicas: int = 1

    @property
    def nodes(self) -> int:
        return (1 << (self.depth + 1)) - 1

    @property
    def elt_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def node_bytes(self) -> int:
        """Bytes of one node's input and output rows."""
        return 2 * self.d * self.elt_bytes

    @property
    def layer_bytes(self) -> int:
        return self.n_trees * self.nodes * (self.node_bytes + 4)


FFF_CONFIGS: dict[str, FffConfig] = {
    c.name: c
    for c in [
        # Small fp32 layer for the oracle and the parity tests.
        FffConfig("fff_tiny_f32", d=256, n_trees=5, depth=3, dtype="f32", tokens=48, seed=11),
        # OPT-1.3B-sized tree layer, 4096 independent tokens, each through its
        # own layer copy (1024 copies of 66.6 MB).
        FffConfig("fff_D6_P64_d2048", d=2048, n_trees=64, depth=6, dtype="bf16", tokens=4096, seed=12,
                  replicas=1024),
    ]
}


@dataclass
class FffLayer:
    dtype: str
    w_node: np.ndarray           # [P][N][d] float32 or uint16 bf16 bits
    b_node: Optional[np.ndarray]  # [P][N] float32
    w_out: np.ndarray            # [P][N][d]

    @property
    def d(self) -> int:
        return self.w_node.shape[2]

    @property
    def n_trees(self) -> int:
        return self.w_node.shape[0]

    @property
    def depth(self) -> int:
        return int(self.w_node.shape[1] + 1).bit_length() - 2


def make_fff_layer(d: int, n_trees: int, depth: int, dtype: str, rng: np.random.Generator,
                   bias: bool = True) -> FffLayer:
    n = (1 << (depth + 1)) - 1
    w_node = rng.standard_normal((n_trees, n, d), dtype=np.float32) * np.float32(1.0 / np.sqrt(d))
    lim = 1.0 / np.sqrt(d)
    b = rng.uniform(-lim, lim, size=(n_trees, n)).astype(np.float32)
    w_out = rng.standard_normal((n_trees, n, d), dtype=np.float32)
    w_out *= np.float32(1.0 / np.sqrt(n_trees * (depth + 1)))
    return FffLayer(dtype=dtype, w_node=_store(w_node, dtype), b_node=b if bias else None,
                    w_out=_store(w_out, dtype))


def make_fff_tokens(d: int, n_tokens: int, dtype: str, rng: np.random.Generator) -> np.ndarray:
    return _store(rng.standard_normal((n_tokens, d), dtype=np.float32), dtype)


def make_fff_workload(cfg: FffConfig, tokens: Optional[int] = None) -> tuple[FffLayer, np.ndarray]:
    rng = np.random.default_rng(cfg.seed)
    layer = make_fff_layer(cfg.d, cfg.n_trees, cfg.depth, cfg.dtype, rng)
    x = make_fff_tokens(cfg.d, cfg.tokens if tokens is None else tokens, cfg.dtype, rng)
    return layer, x


def get_fff_config(name: str) -> FffConfig:
    try:
        return FFF_CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown FFF workload {name!r}; known: {sorted(FFF_CONFIGS)}") from None
