"""GPU parity of the baseline routers (blockffn_route_with) against the oracle,
and the rest of the path (union, forward) run on their gates.

Bars: pre-activations as for the BlockFFN router; masks bit-exact except
tokens whose decision sits within 1e-3 of its threshold in the oracle's fp64
z (for top-k: the gap between the k-th and (k+1)-th largest z; for the
ReLU-sum router: some |z_i| < 1e-3), which are counted and left out; gates
within 1e-4 (bf16) / 1e-5 (fp32) x RMS of the oracle's; y within 2e-2 (bf16)
/ 1e-5 (fp32) x RMS.
"""
import numpy as np
import pytest

from gpu_parity_util import check_baseline_router, say
from workload import make_layer, make_tokens

pytestmark = pytest.mark.gpu

# name: (d, E, d_e, dtype, L, chunks, bias_k, alpha, seed)
SHAPES = {
    "bf16_d512_E64_L8": (512, 64, 128, "bf16", 8, 10, 0.9, 0.8, 701),    # MFMA router
    "bf16_d640_E70_L3": (640, 70, 128, "bf16", 3, 11, 0.9, 0.6, 702),    # VALU router, two mask words
    "f32_d128_E24_L4": (128, 24, 32, "f32", 4, 6, 0.5, 0.7, 703),        # fp32
}
ROUTERS = [("topk_softmax", 1), ("topk_softmax", 2), ("topk_softmax", 8), ("relu_sum", 0)]


@pytest.mark.parametrize("router,k", ROUTERS, ids=[f"{r}{k}" for r, k in ROUTERS])
@pytest.mark.parametrize("shape", sorted(SHAPES))
def test_router_matches_oracle(shape, router, k):
    d, E, de, dt, L, C, bias_k, a, seed = SHAPES[shape]
    rng = np.random.default_rng(seed)
    layer = make_layer(d, E, de, dt, bias_k, rng)
    x = make_tokens(d, C, L, a, dt, rng).x
    say(f"[gpu] router {router}{k} {shape} T={x.shape[0]}")
    check_baseline_router(layer, x, L, router, k, shape)
