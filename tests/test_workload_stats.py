"""The synthetic workloads land on the sparsity the pages report.

The BlockFFN abstract (arXiv 2507.08771) and write-up §3 report over 80%
token-level sparsity (TLS) and about 70% 8-token chunk-level sparsity (CLS).
For the generator, expert i's normalised pre-activation on token t of chunk c
is sqrt(rho) U_c + sqrt(1 - rho) V_t with U, V independent standard normals,
so the closed forms are

    TLS   = Phi(k)
    CLS_L = integral phi(u) Phi((k - sqrt(rho) u) / sqrt(1 - rho))^L du

(the chance that none of the L tokens fires).  The realised statistics, from
the oracle's router and stats on the full workload, must land within two
percentage points.
"""
import numpy as np
import pytest
from scipy.special import ndtr

import oracle
from workload import CONFIGS, make_workload


def _closed_form(k, alpha, L):
    rho = alpha * alpha / (alpha * alpha + (1.0 - alpha) ** 2)
    tls = float(ndtr(k))
    if rho == 0.0:
        return tls, tls ** L
    u = np.linspace(-12.0, 12.0, 48001)
    phi = np.exp(-0.5 * u * u) / np.sqrt(2.0 * np.pi)
    inner = ndtr((k - np.sqrt(rho) * u) / np.sqrt(1.0 - rho)) ** L
    return tls, float(np.trapezoid(phi * inner, u))


@pytest.mark.parametrize("name", ["decode_L1_d2048_E64", "chunk8_d2048_E64", "large_L8_d4096_E128",
                                  "large_L32_d4096_E128", "batched_L8_d4096_E128"])
def test_generator_sparsity_matches_closed_form(name):
    cfg = CONFIGS[name]
    layer, tok = make_workload(cfg)
    z, g, m = oracle.route(tok.x, layer.w_router, layer.b_router, None, layer.rms_eps)
    st = oracle.stats(m, cfg.n_experts, cfg.chunk_len)
    tls, cls = _closed_form(cfg.bias_k, cfg.alpha, cfg.chunk_len)
    print(f"{name}: TLS {st['tls']:.4f} (closed form {tls:.4f}), CLS_{cfg.chunk_len} "
          f"{st['cls']:.4f} (closed form {cls:.4f}), reuse {st['reuse']:.3f}")
    assert abs(st["tls"] - tls) < 0.02
    assert abs(st["cls"] - cls) < 0.02
    # the pages' setting: TLS above 80%
    assert st["tls"] > 0.79


def test_chunk8_workload_hits_the_pages_setting():
    # 8-token CLS about 70% (abstract: "70% 8-token CLS"), about 19 of 64 experts per chunk.
    _, cls = _closed_form(CONFIGS["chunk8_d2048_E64"].bias_k, 0.8, 8)
    assert 0.68 < cls < 0.73
    assert 64 * (1 - cls) == pytest.approx(18.6, abs=0.5)


def test_generator_is_deterministic_and_layout():
    cfg = CONFIGS["tiny_f32_L4"]
    l1, t1 = make_workload(cfg)
    l2, t2 = make_workload(cfg)
    np.testing.assert_array_equal(t1.x, t2.x)
    np.testing.assert_array_equal(l1.w_in, l2.w_in)
    assert l1.w_router.shape == (8, 64) and l1.w_in.shape == (8, 16, 64) and l1.w_out.shape == (8, 64, 16)
    assert t1.x.shape == (64, 64) and t1.x.dtype == np.float32
    # bias = -k * std of the pre-activation
    np.testing.assert_allclose(l1.b_router, -0.8 * np.linalg.norm(l1.w_router.astype(np.float64), axis=1),
                               rtol=1e-6)
