"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (on the CPU,
in a temporary directory), builds it, and runs the pin suite against it; the
suite must fail.  The mistakes are the ones a reader of the pages could make:
a non-strict ReLU threshold, a wrong RMS denominator, epsilon outside the
root, a different activation, a transposed matrix, a dropped gate, AND
instead of OR for the union, a chunk boundary off by one, a wrong bf16
widening, a wrong reuse denominator, a flipped bias sign; and in the backward
a dropped or sign-flipped RMSNorm term, a wrong Swish derivative, a dropped
gate, gradients taken through inactive pairs, a wrong scale gradient, a dropped router term of
dx, a missing gate in dW_out; and in the baseline routers a tie broken the
other way, an unshifted softmax sum, a missing ReMoE normalisation; and in
the CLS-aware objectives an unshifted locality target, the complement of the
chunk probability, a chunk gradient that includes the token itself, and an
extra router gradient applied to active pairs only; and in the FFF tree layer
a turn taken at c >= 0, swapped children, one level too few, the tanh
approximation of GELU, a dropped node bias, GELU kept at the nodes in the
post variant, a dense evaluation that skips the leaves, and the output taken
from the input row.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_DIR = os.path.join(ROOT, "oracle")
SOURCES = ("blockffn_oracle.c", "fff_oracle.c")

MUTANTS = {
    "relu_not_strict": ("if (acc > 0.0) m[i / 64]", "if (acc >= 0.0) m[i / 64]"),
    "rms_denominator": ("ms /= (double)E;", "ms /= (double)(E + 1);"),
    "eps_outside_root": ("sqrt(ms + eps)", "(sqrt(ms) + eps)"),
    "relu_instead_of_swish": ("h[j] = u / (1.0 + exp(-u));", "h[j] = u > 0.0 ? u : 0.0;"),
    "w_out_transposed": ("widen(w_out, w_out_off + (int64_t)k * de + j, dtype)",
                         "widen(w_out, w_out_off + (int64_t)j * d + k, dtype)"),
    "gate_dropped": ("if (!mask_bit(mask + t * W, i)) continue;\n        expert_eval(d, de, dtype, x, t * d, w_in, (int64_t)i * de * d, w_out, (int64_t)i * d * de, h, e);\n        for (int k = 0; k < d; ++k) yt[k] += g[t * E + i] * e[k];",
                     "if (!mask_bit(mask + t * W, i)) continue;\n        expert_eval(d, de, dtype, x, t * d, w_in, (int64_t)i * de * d, w_out, (int64_t)i * d * de, h, e);\n        for (int k = 0; k < d; ++k) yt[k] += e[k];"),
    "union_and": ("for (int64_t t = c * L; t < (c + 1) * L; ++t) u |= mask[t * W + w];",
                  "for (int64_t t = c * L; t < (c + 1) * L; ++t) u &= mask[t * W + w];"),
    "chunk_boundary": ("for (int64_t t = c * L; t < (c + 1) * L; ++t) u |= mask[t * W + w];",
                       "for (int64_t t = c * L + 1; t < (c + 1) * L; ++t) u |= mask[t * W + w];"),
    "bf16_widening": ("[idx]) << 16;", "[idx]) << 15;"),
    "reuse_denominator": ("out->reuse_den += count_bits(mask + (t - 1) * W, E);",
                          "out->reuse_den += count_bits(mask + t * W, E);"),
    "bias_sign": ("if (b_router) acc += (double)b_router[i];", "if (b_router) acc -= (double)b_router[i];"),
    # the backward
    "bwd_rms_term_dropped": ("const double da = dg[t * E + i] * s * r + dms * 2.0 * a / (double)E;",
                             "const double da = dg[t * E + i] * s * r;"),
    "bwd_rms_denominator": ("const double r = 1.0 / sqrt(ms / (double)E + eps);",
                            "const double r = 1.0 / sqrt(ms / (double)(E + 1) + eps);"),
    "bwd_rms_term_sign": ("const double dms = -0.5 * dr * r * r * r;", "const double dms = 0.5 * dr * r * r * r;"),
    "bwd_swish_derivative": ("du[j] = g * qj * sig * (1.0 + u * (1.0 - sig));", "du[j] = g * qj * sig;"),
    "bwd_gate_dropped": ("du[j] = g * qj * sig * (1.0 + u * (1.0 - sig));",
                         "du[j] = qj * sig * (1.0 + u * (1.0 - sig));"),
    # (dropping the ReLU mask on dz alone is an equivalent change: inactive
    # pairs have a = 0 and are never visited, so their dg and da are 0; the
    # mistake that matters is visiting them)
    "bwd_inactive_pairs_visited": ("if (mask_bit(m + t * W, i) && ok) {", "if (ok) {"),
    "bwd_scale_grad_uses_gate": ("dsc[t * E + i] = dgi * a * r;", "dsc[t * E + i] = dgi * g[t * E + i];"),
    "bwd_router_dx_dropped": ("for (int i = 0; i < E; ++i) acc += dz[t * E + i] * widen(w_router,",
                              "for (int i = 0; i < E; ++i) acc += 0.0 * dz[t * E + i] * widen(w_router,"),
    "bwd_w_out_grad_gate_dropped": ("go[(int64_t)k * de + j] += gti * (double)dy[t * d + k] * h[j];",
                                    "go[(int64_t)k * de + j] += (double)dy[t * d + k] * h[j];"),
    # the baseline routers
    "topk_tie_to_higher_index": ("if (!taken[i] && (best < 0 || z[i] > z[best])) best = i;",
                                 "if (!taken[i] && (best < 0 || z[i] >= z[best])) best = i;"),
    "topk_softmax_unshifted_sum": ("for (int i = 0; i < E; ++i) sum += exp(z[i] - zmax);",
                                   "for (int i = 0; i < E; ++i) sum += exp(z[i]);"),
    "relu_sum_unnormalised": ("g[i] = z[i] / sum;", "g[i] = z[i];"),
    # the CLS-aware objectives
    "cls_locality_target_not_shifted": ("const double y = z[(t + 1) * E + i] > 0.0 ? 1.0 : 0.0;\n      al +=",
                                        "const double y = z[t * E + i] > 0.0 ? 1.0 : 0.0;\n      al +="),
    "cls_chunk_loss_complement": ("cs += 1.0 - q;", "cs += q;"),
    "cls_chunk_grad_includes_self": ("if (u != t) others *= 1.0", "others *= 1.0"),
    "bwd_extra_gradient_only_active": ("dz[t * E + i] = (z[t * E + i] > 0.0 ? da : 0.0) + (dz_extra ? dz_extra[t * E + i] : 0.0);",
                                       "dz[t * E + i] = z[t * E + i] > 0.0 ? da + (dz_extra ? dz_extra[t * E + i] : 0.0) : 0.0;"),
}
PIN_FILES = ("test_oracle_pins.py", "test_oracle_backward_pins.py", "test_oracle_router_pins.py",
             "test_oracle_cls_pins.py")

# mistakes in the FFF tree layer (fff_oracle.c), caught by its own pins
FFF_MUTANTS = {
    "fff_turn_not_strict": ("n = 2 * n + 1 + (c > 0.0 ? 1 : 0);", "n = 2 * n + 1 + (c >= 0.0 ? 1 : 0);"),
    "fff_children_swapped": ("n = 2 * n + 1 + (c > 0.0 ? 1 : 0);", "n = 2 * n + 1 + (c > 0.0 ? 0 : 1);"),
    "fff_one_level_short": ("const int64_t V = dense ? N : (int64_t)D + 1;", "const int64_t V = dense ? N : (int64_t)D;"),
    "fff_gelu_tanh": ("return 0.5 * c * (1.0 + erf(c / sqrt(2.0)));",
                      "return 0.5 * c * (1.0 + tanh(0.7978845608028654 * (c + 0.044715 * c * c * c)));"),
    "fff_bias_dropped": ("if (b_node) c += (double)b_node[row];", ""),
    "fff_post_gelu_at_nodes": ("const double a = post ? c : fff_gelu(c);", "const double a = fff_gelu(c);"),
    "fff_dense_skips_leaves": ("const int64_t V = dense ? N : (int64_t)D + 1;",
                               "const int64_t V = dense ? (N - 1) / 2 : (int64_t)D + 1;"),
    "fff_output_from_input_row": ("yt[k] += a * fff_widen(w_out, row * d + k, dtype);",
                                  "yt[k] += a * fff_widen(w_node, row * d + k, dtype);"),
}
FFF_PIN_FILES = ("test_oracle_fff_pins.py",)


def _run_mutant(name, target, old, new, pin_files):
    path = os.path.join(ORACLE_DIR, target)
    src = open(path).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    with tempfile.TemporaryDirectory() as tmp:
        files = []
        for f in SOURCES:
            c = os.path.join(tmp, f)
            text = open(os.path.join(ORACLE_DIR, f)).read()
            open(c, "w").write(src.replace(old, new) if f == target else text)
            files.append(c)
        so = os.path.join(tmp, "libmutant.so")
        subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
                        "-o", so, *files, "-lm"], check=True)
        env = dict(os.environ, BLOCKFFN_ORACLE_LIB=so)
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            *[os.path.join(ROOT, "tests", f) for f in pin_files]],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
        assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    old, new = MUTANTS[name]
    _run_mutant(name, "blockffn_oracle.c", old, new, PIN_FILES)


@pytest.mark.parametrize("name", sorted(FFF_MUTANTS))
def test_fff_pins_catch_planted_mistake(name):
    old, new = FFF_MUTANTS[name]
    _run_mutant(name, "fff_oracle.c", old, new, FFF_PIN_FILES)
