"""The pins must be able to fail: plant plausible mistakes in a copy of the
oracle's C source (on the CPU, in a temporary directory), build the mutant, and
check that at least one pin (tests/test_oracle_pins.py, test_oracle_backward.py,
test_oracle_forced.py) rejects it."""
import os
import subprocess

import pytest

import oracle as oracle_pkg
from tests import test_oracle_backward as bpins
from tests import test_oracle_forced as fpins
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle_pkg.__file__), "oracle.c")

MUTANTS = {
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "swap_w1_w3": ("h[f] = silu(a) * b;", "h[f] = silu(b) * a;"),
    "tie_to_higher_index": ("if (best < 0 || l[i] > l[best]) best = i;",
                            "if (best < 0 || l[i] >= l[best]) best = i;"),
    "softmax_sign": ("g[j] = exp(l[sel[j]] - m);", "g[j] = exp(m - l[sel[j]]);"),
    "router_transposed": ("s += u[k] * (double)Wg[k * n + i];",
                          "s += u[k] * (double)Wg[i * d + k];"),
    "down_transposed": ("const float* w2 = W2 + c * d_ff;\n        for (int64_t f = 0; f < d_ff; ++f) s += (double)w2[f] * h[f];",
                        "for (int64_t f = 0; f < d_ff; ++f) s += (double)W2[f * d + c] * h[f];"),
    "gate_dropped": ("y[c] += g[j] * o[c];", "y[c] += o[c];"),
    "expert_stride": ("W1 + e * d_ff * d, W3 + e * d_ff * d", "W1 + e * d_ff, W3 + e * d_ff"),
    "rms_mean": ("ss / (double)d + eps", "ss + eps"),
    "rms_eps_outside_sqrt": ("const double inv = 1.0 / sqrt(ss / (double)d + eps);",
                             "const double inv = 1.0 / (sqrt(ss / (double)d) + eps);"),
    "rms_eps_dropped": ("const double inv = 1.0 / sqrt(ss / (double)d + eps);",
                        "const double inv = 1.0 / sqrt(ss / (double)d);"),
    "residual_dropped": ("yr[k] += (double)xt[k];", "yr[k] += 0.0;"),
    "softmax_before_topk": (
        "    masked_softmax(l, sel, K, g);\n    for (int64_t c = 0; c < d; ++c) y[c] = 0.0;",
        "    {\n        double m0 = l[0], z0 = 0.0;\n"
        "        for (int32_t i = 1; i < n; ++i) if (l[i] > m0) m0 = l[i];\n"
        "        for (int32_t i = 0; i < n; ++i) z0 += exp(l[i] - m0);\n"
        "        for (int32_t j = 0; j < K; ++j) g[j] = exp(l[sel[j]] - m0) / z0;\n"
        "    }\n    for (int64_t c = 0; c < d; ++c) y[c] = 0.0;"),
    "second_slot_gate": ("for (int32_t j = 0; j < K; ++j) g[j] /= z;",
                         "for (int32_t j = 0; j < K; ++j) g[j] /= (j ? z : 1.0);"),
    # the caller's expert set ignored (TopK's own choice used instead), at
    # every forced-routing site
    "forced_ignored": ("if (forced) {", "if (forced && 0) {"),
    # the caller's set taken, but sorted back into logit order
    "forced_reordered": ("for (int32_t j = 0; j < K; ++j) sel[j] = forced[j];",
                         "for (int32_t j = 0; j < K; ++j) sel[j] = forced[j];\n"
                         "        for (int32_t j = 1; j < K; ++j)\n"
                         "            for (int32_t q = j; q > 0 && l[sel[q]] > l[sel[q - 1]]; --q) {\n"
                         "                int32_t tmp = sel[q]; sel[q] = sel[q - 1]; sel[q - 1] = tmp;\n"
                         "            }"),
}

PIN_TESTS = [
    lambda o: pins.test_dense_mixture_when_K_equals_n(o),
    lambda o: pins.test_single_expert_is_swiglu_ffn(o),
    lambda o: pins.test_silu_branch_closed_form(o),
    lambda o: pins.test_gates_nonnegative_normalised_ordered(o),
    lambda o: pins.test_two_way_softmax_is_logistic(o),
    lambda o: pins.test_logits_match_library_matmul(o),
    lambda o: pins.test_bruteforce_selection_and_output(o, 8, 2),
    lambda o: pins.test_sparse_equals_dense_with_zero_gates(o),
    lambda o: pins.test_zero_token(o),
    lambda o: pins.test_duplicate_router_columns_tie_to_lower_index(o),
    lambda o: pins.test_block_layer_is_residual_over_rmsnorm(o),
    lambda o: fpins.test_forced_forward_takes_the_given_set(None),
    lambda o: fpins.test_forced_forward_takes_the_given_set(1e-5),
    lambda o: fpins.test_forced_rows_subset_and_three_slots(),
]


# Mistakes in the backward pass, each to be rejected by a backward pin.
BACKWARD_MUTANTS = {
    "bwd_silu_derivative": ("da[f] = dh[f] * b[f] * (s + a[f] * s * (1.0 - s));",
                            "da[f] = dh[f] * b[f] * s;"),
    "bwd_up_branch": ("db[f] = dh[f] * a[f] * s;", "db[f] = dh[f] * s;"),
    "bwd_softmax_uncentred": ("sg->dl[sel[j]] = g[j] * (dg[j] - gdg);",
                              "sg->dl[sel[j]] = g[j] * dg[j];"),
    "bwd_gate_dropped": ("dO[c] = g[j] * (double)dy[c];", "dO[c] = (double)dy[c];"),
    "bwd_router_dx_dropped": ("        dx[k] += s;\n    }\n}", "        dx[k] += 0.0 * s;\n    }\n}"),
    "bwd_w1_w3_swapped": ("if (dW1) dW1[(e * d_ff + f) * d + k] = s1;",
                          "if (dW1) dW1[(e * d_ff + f) * d + k] = s3;"),
}

# Mistakes in the per-entry weight gradients (oracle_backward_entries).
BACKWARD_MUTANTS.update({
    "entries_silu_derivative": ("dh * b * (sg + a * sg * (1.0 - sg))", "dh * b * sg"),
    "entries_gate_dropped": ("s += g * (double)dyt[ri[q]] * (silu(a) * b);",
                             "s += (double)dyt[ri[q]] * (silu(a) * b);"),
    "entries_w2_transposed": ("r += (double)w2[c * d_ff + f] * (double)dyt[c];",
                              "r += (double)w2[f * d + c] * (double)dyt[c];"),
})

# Mistakes in the stack layer's backward (oracle_block_backward).
BACKWARD_MUTANTS.update({
    "block_projection_dropped": ("sc * (du[r * d + k] - u[k] * c / (double)d)",
                                 "sc * du[r * d + k]"),
    "block_residual_dropped": ("dx[r * d + k] = (double)dy[t * d + k] + sc",
                               "dx[r * d + k] = 0.0 * (double)dy[t * d + k] + sc"),
    "block_scale_missing": ("sc * (du[r * d + k] - u[k] * c / (double)d)",
                            "(du[r * d + k] - u[k] * c / (double)d)"),
    "block_eps_outside_sqrt": ("const double sc = 1.0 / sqrt(ss / (double)d + eps);",
                               "const double sc = 1.0 / (sqrt(ss / (double)d) + eps);"),
})

# The forced-routing sites of the backward (token_backward) and of the entry
# path (entries_impl), one at a time: (old, new, which occurrence).
BACKWARD_MUTANTS.update({
    "bwd_forced_ignored": ("if (forced) {", "if (forced && 0) {", 1),
    "entries_forced_ignored": ("if (forced) {", "if (forced && 0) {", 2),
})

BACKWARD_PINS = [
    lambda o: bpins.test_block_backward_matches_finite_differences(),
    lambda o: bpins.test_block_backward_dense_mixture_autograd(),
    lambda o: bpins.test_block_backward_scale_invariance(),
    lambda o: bpins.test_block_backward_entries_match_full_block_backward(),
    lambda o: bpins.test_backward_entries_match_dense_autograd(),
    lambda o: bpins.test_backward_entries_match_full_backward(),
    lambda o: bpins.test_backward_matches_finite_differences(),
    lambda o: bpins.test_single_expert_backward_is_swiglu_autograd(),
    lambda o: bpins.test_dense_mixture_backward_when_K_equals_n(),
    lambda o: bpins.test_router_gradient_rows_sum_to_zero(),
    lambda o: fpins.test_forced_backward_matches_autograd(None),
    lambda o: fpins.test_forced_backward_matches_autograd(1e-5),
    lambda o: fpins.test_forced_backward_entries_match_autograd(None),
    lambda o: fpins.test_forced_backward_entries_match_autograd(1e-5),
]


def _mutate(src, old, new, nth=None):
    """src with old replaced by new: every occurrence, or only the nth
    (0-based) when nth is given."""
    assert src.count(old) >= 1, f"mutation site not found: {old!r}"
    if nth is None:
        return src.replace(old, new)
    parts = src.split(old)
    assert len(parts) > nth + 1, f"occurrence {nth} of {old!r} not found"
    return old.join(parts[:nth + 1]) + new + old.join(parts[nth + 1:])


def _build_mutant(site, tmp_path, monkeypatch):
    """Compile the oracle with one planted mistake; site = (old, new) or
    (old, new, nth)."""
    mutated = _mutate(open(SRC).read(), *site)
    c_path = tmp_path / "mutant.c"
    so_path = tmp_path / "libmutant.so"
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-o",
                    str(so_path), str(c_path), "-lm"], check=True)
    monkeypatch.setattr(oracle_pkg, "_LIB_PATH", str(so_path))
    monkeypatch.setattr(oracle_pkg, "_lib", None)


@pytest.mark.parametrize("name", sorted(BACKWARD_MUTANTS))
def test_backward_mutant_is_caught(name, tmp_path, monkeypatch):
    _build_mutant(BACKWARD_MUTANTS[name], tmp_path, monkeypatch)
    caught = 0
    for pin in BACKWARD_PINS:
        try:
            pin(oracle_pkg)
        except (AssertionError, ValueError, IndexError):
            caught += 1
    monkeypatch.setattr(oracle_pkg, "_lib", None)
    assert caught > 0, f"no backward pin rejects the mutant {name}"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path, monkeypatch):
    _build_mutant(MUTANTS[name], tmp_path, monkeypatch)
    caught = 0
    for pin in PIN_TESTS:
        try:
            pin(oracle_pkg)
        except (AssertionError, ValueError, IndexError):
            caught += 1
    monkeypatch.setattr(oracle_pkg, "_lib", None)
    assert caught > 0, f"no pin rejects the mutant {name}"
