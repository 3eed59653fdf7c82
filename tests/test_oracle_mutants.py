"""Planted mistakes in the oracle must be caught by its pins.

Each case compiles a copy of ``oracle/oracle.c`` with one plausible mistake (a
dropped term, a wrong constant or sign, a missing shard offset, a missing bias,
a skipped partial, swapped gate and up operands, swapped GeLU forms, a wrong
attention scale, mask, head group or query position, a wrong GeLU derivative
or gradient operand) and runs every pin of ``test_oracle.py``,
``test_oracle_attention.py`` and ``test_oracle_backward.py`` against it; at
least one pin has to fail.  Everything runs on the CPU.
"""
import os
import subprocess

import pytest

import oracle
from tests import test_oracle as pins
from tests import test_oracle_attention as attn_pins
from tests import test_oracle_backward as bwd_pins

MUTANTS = {
    "gelu_no_cubic": ("0.044715 * x * x * x", "0.0 * x"),
    "gelu_wrong_scale": ("sqrt(2.0 / acos(-1.0))", "sqrt(acos(-1.0) / 2.0)"),
    "gelu_wrong_sign": ("(1.0 + tanh(", "(1.0 - tanh("),
    "gelu_mistyped_coeff": ("0.044715", "0.04715"),
    "up_missing_shard_offset": ("W1 + h * F + o;", "W1 + h * F;"),
    "up_dropped_first_term": ("for (int64_t h = 0; h < H; ++h) {", "for (int64_t h = 1; h < H; ++h) {"),
    "up_bias_dropped": ("acc[c] + b1[o + c]", "acc[c]"),
    "up_bias_wrong_offset": ("acc[c] + b1[o + c]", "acc[c] + b1[c]"),
    "down_missing_shard_offset": ("W2 + (o + c) * H", "W2 + c * H"),
    "down_wrong_sign": ("z[n] += y * w[n];", "z[n] -= y * w[n];"),
    "reduce_skips_last": ("for (int32_t j = 0; j < T; ++j)", "for (int32_t j = 0; j + 1 < T; ++j)"),
    "reduce_residual_sign": ("residual[m * H + n] + s", "residual[m * H + n] - s"),
    "rms_no_eps": ("ss / (double)H + eps", "ss / (double)H"),
    "rms_wrong_mean": ("ss / (double)H + eps", "ss / (double)(H + 1) + eps"),
    "erf_wrong_scale": ("erf(x / sqrt(2.0))", "erf(x * sqrt(2.0))"),
    "erf_wrong_sign": ("(1.0 + erf(", "(1.0 - erf("),
    "act_forms_swapped": ("act == ORC_ACT_GELU_ERF ? gelu_erf(x) : gelu_tanh(x)",
                          "act == ORC_ACT_GELU_ERF ? gelu_tanh(x) : gelu_erf(x)"),
    "gated_gate_up_swapped": ("act_apply(act, gate) * up", "act_apply(act, up) * gate"),
    "gated_up_bias_dropped": ("u[c] + bu[o + c]", "u[c]"),
    "gated_up_missing_shard_offset": ("Wu + h * F + o;", "Wu + h * F;"),
    "gated_gate_reads_up": ("const double *wg = Wg + h * F + o;", "const double *wg = Wu + h * F + o;"),
    "linear_applies_gelu": ("if (act == ORC_ACT_NONE) return x;", "if (act == ORC_ACT_NONE) return gelu_tanh(x);"),
    "attn_no_scale": ("w[t] = dot * scale;", "w[t] = dot;"),
    "attn_scale_one_over_d": ("1.0 / sqrt((double)d)", "1.0 / (double)d"),
    "attn_mask_hides_own_position": ("causal ? p + 1 : len", "causal ? (p > 0 ? p : 1) : len"),
    "attn_mask_shows_next_position": ("causal ? p + 1 : len", "causal ? (p + 1 < len ? p + 2 : len) : len"),
    "attn_gqa_wrong_group": ("const int32_t g = h / G;", "const int32_t g = h % nkv;"),
    "attn_no_max_subtraction": ("w[t] = exp(w[t] - mx);", "w[t] = exp(w[t]);"),
    "attn_not_normalised": ("c[e] /= den;", "c[e] /= 1.0;"),
    "attn_value_of_other_key": ("V + ((b * Lk + t) * nkv + g) * d", "V + ((b * Lk + (nkeys - 1 - t)) * nkv + g) * d"),
    "attn_queries_from_sequence_start": ("const int64_t p = len - Sq + s;", "const int64_t p = s;"),
    "attn_key_head_offset_dropped": ("K + ((b * Lk + t) * nkv + g) * d", "K + ((b * Lk + t) * nkv) * d"),
    "bwd_tanh_grad_drops_second_term": ("return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * c * (1.0 + 3.0 * 0.044715 * x * x);",
                                        "return 0.5 * (1.0 + t);"),
    "bwd_tanh_grad_cubic_coefficient": ("(1.0 + 3.0 * 0.044715 * x * x)", "(1.0 + 0.044715 * x * x)"),
    "bwd_erf_grad_no_density_term": ("return Phi + x * phi;", "return Phi;"),
    "bwd_dy_missing_shard_offset": ("dy += dZ[m * H + h] * W2[(o + c) * H + h];", "dy += dZ[m * H + h] * W2[c * H + h];"),
    "bwd_dx_missing_shard_offset": ("s += dU[m * Fs + c] * W1[h * F + o + c];", "s += dU[m * Fs + c] * W1[h * F + c];"),
    "bwd_dw1_uses_activation": ("s += X[m * H + h] * dU[m * Fs + c];", "s += X[m * H + h] * Y[m * Fs + c];"),
    "bwd_db1_before_activation_grad": ("s += dU[m * Fs + c];", "s += dU[m * Fs + c] / act_grad(act, U[m * Fs + c]);"),
    "bwd_dw2_uses_preactivation": ("s += Y[m * Fs + c] * dZ[m * H + h];", "s += U[m * Fs + c] * dZ[m * H + h];"),
}


def _all_pins():
    calls = []
    for mod in (pins, attn_pins, bwd_pins):
        for name in dir(mod):
            f = getattr(mod, name)
            if not name.startswith("test_") or not callable(f):
                continue
            if name == "test_shard_sum_equals_unsharded":
                calls += [(name + "[T=%d]" % T, (lambda f=f, T=T: f(T))) for T in (1, 2, 4, 8)]
            elif name == "test_attn_head_shards_are_the_unsharded_heads":
                calls += [(name + "[T=%d]" % T, (lambda f=f, T=T: f(T))) for T in (2, 4)]
            elif name in ("test_backward_shards_reassemble_the_unsharded_gradients",
                          "test_gelu_grad_is_the_derivative_of_gelu", "test_gelu_grad_odd_part_identity",
                          "test_backward_matches_finite_differences"):
                params = (2, 4) if name.startswith("test_backward_shards") else (oracle.ACT_GELU_TANH,
                                                                                  oracle.ACT_GELU_ERF)
                calls += [(name + "[%d]" % a, (lambda f=f, a=a: f(a))) for a in params]
            elif name in ("test_oracle_rejects_bad_arguments", "test_attn_rejects_bad_arguments",
                          "test_backward_rejects_bad_arguments"):
                continue
            else:
                calls.append((name, f))
    return calls


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistake_is_caught(mutant, tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    old, new = MUTANTS[mutant]
    assert src.count(old) >= 1, "mutation target vanished from oracle.c: %r" % old
    path = tmp_path / "oracle_mut.c"
    path.write_text(src.replace(old, new))
    lib = str(tmp_path / ("lib%s.so" % mutant))
    subprocess.check_call(["gcc", *oracle.CFLAGS, str(path), "-o", lib, "-lm"])
    caught = None
    with oracle._swapped(lib):
        for name, f in _all_pins():
            try:
                f()
            except AssertionError:
                caught = name   # one rejecting pin is enough
                break
    assert caught, "no pin rejects the planted mistake %s" % mutant
