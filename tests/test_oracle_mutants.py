"""Planted mistakes in the oracle must be caught by its pins.

Each case compiles a copy of ``oracle/oracle.c`` with one plausible mistake (a
dropped term, a wrong constant or sign, a missing shard offset, a missing bias,
a skipped partial, swapped gate and up operands, swapped GeLU forms) and runs
every pin of ``test_oracle.py`` against it; at
least one pin has to fail.  Everything runs on the CPU.
"""
import os
import subprocess

import pytest

import oracle
from tests import test_oracle as pins

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
}


def _all_pins():
    calls = []
    for name in dir(pins):
        f = getattr(pins, name)
        if not name.startswith("test_") or not callable(f):
            continue
        if name == "test_shard_sum_equals_unsharded":
            calls += [(name + "[T=%d]" % T, (lambda f=f, T=T: f(T))) for T in (1, 2, 4, 8)]
        elif name == "test_oracle_rejects_bad_arguments":
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
    caught = []
    with oracle._swapped(lib):
        for name, f in _all_pins():
            try:
                f()
            except AssertionError:
                caught.append(name)
    assert caught, "no pin rejects the planted mistake %s" % mutant
