"""Plant plausible slips in a copy of the oracle and check the pins catch them.

Each mutant is a one-line edit of oracle.c (wrong scale direction, wrong
Qmax, truncation instead of rounding, eps outside the square root, dropped
1/K, a transposed operand, a sign slip, a shuffled tile layout, ...).  It is
compiled with gcc into a temporary library, swapped in for the real one, and
the pin tests are run against it: at least one must fail.  CPU only.
"""
import inspect
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_gate as gate_pins
from tests import test_oracle_glu as glu_pins
from tests import test_oracle_mlgru as mlgru_pins
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "epilogue_multiplies_by_s": ("((double)acc[m * N + n] / (double)s[m])",
                                 "((double)acc[m * N + n] * (double)s[m])"),
    "qmax_128": ("127.0f / gamma", "128.0f / gamma"),
    "truncate_instead_of_round": ("float q = rintf(v);", "float q = truncf(v);"),
    "eps_outside_sqrt": ("1.0f / sqrtf(ms + eps)", "1.0f / (sqrtf(ms) + eps)"),
    "mean_square_without_1_over_K": ("(float)(sumsq / (double)K)", "(float)(sumsq)"),
    "sum_abs_instead_of_squares": ("sumsq += (double)row[k] * (double)row[k];",
                                   "sumsq += fabs((double)row[k]);"),
    "gain_without_norm": ("float t = row[k] * r;", "float t = row[k];"),
    "signed_max_not_absmax": ("float a = fabsf(row[k]);", "float a = row[k];"),
    "weight_multiplied_by_scale": ("rintf(w / beta)", "rintf(w * beta)"),
    "weight_mean_over_rows_only": ("(double)(N * K))", "(double)(N))"),
    "weight_sum_without_abs": ("sum += fabs((double)W[i]);", "sum += (double)W[i];"),
    "no_ternary_clamp": ("if (q > 1.0f) q = 1.0f;", ""),
    "contraction_reads_untransposed": ("B[k * N + n] = Wq[n * K + k];",
                                       "B[k * N + n] = Wq[k * N + n];"),
    "matmul_sign_slip": ("acc += A[i * k + p] * B[p * n + j];",
                         "acc -= A[i * k + p] * B[p * n + j];"),
    "tile_words_h_s_swapped": ("4 * (2 * h + j % 2)", "4 * (2 * (j % 2) + h)"),
    "tile_bits_e_order_swapped": ("8 * (e % 4) + 2 * (e / 4)", "8 * (e / 4) + 2 * (e % 4)"),
    "silu_sign_slip": ("return a / (1.0 + exp(-a));", "return a / (1.0 + exp(a));"),
    "silu_missing_factor": ("return a / (1.0 + exp(-a));", "return 1.0 / (1.0 + exp(-a));"),
    "glu_gates_the_wrong_half": ("oracle_silu(y[m * 2 * F + j]) * y[m * 2 * F + F + j]",
                                 "y[m * 2 * F + j] * oracle_silu(y[m * 2 * F + F + j])"),
    "glu_rows_halves_swapped": ("(half == 0 ? 0 : F) + 16 * t + c", "(half == 0 ? F : 0) + 16 * t + c"),
    "glu_rows_tile_of_32": ("(half == 0 ? 0 : F) + 16 * t + c", "(half == 0 ? 0 : F) + 32 * t + c"),
    "gate_normalizes_g": ("sumsq += (double)orow[k] * (double)orow[k];",
                          "sumsq += (double)grow[k] * (double)grow[k];"),
    "gate_sigmoid_not_swish": ("(double)w[k] * oracle_silu((double)grow[k]);",
                               "(double)w[k] / (1.0 + exp(-(double)grow[k]));"),
    "gate_eps_outside_sqrt": ("1.0 / sqrt(sumsq / (double)K + eps);",
                              "1.0 / (sqrt(sumsq / (double)K) + eps);"),
    "gate_without_1_over_K": ("1.0 / sqrt(sumsq / (double)K + eps);", "1.0 / sqrt(sumsq + eps);"),
    "gate_drops_gain": ("((double)orow[k] * r) * (double)w[k] * oracle_silu",
                        "((double)orow[k] * r) * oracle_silu"),
    "gate_unnormalized": ("((double)orow[k] * r) * (double)w[k]", "((double)orow[k]) * (double)w[k]"),
    "scan_gate_on_the_input": ("state = a * state + (1.0 - a) * (double)i[e];",
                               "state = (1.0 - a) * state + a * (double)i[e];"),
    "scan_sigmoid_sign_slip": ("1.0 / (1.0 + exp(-(double)f[e]))", "1.0 / (1.0 + exp((double)f[e]))"),
    "scan_gate_without_sigmoid": ("1.0 / (1.0 + exp(-(double)f[e]))", "(double)f[e]"),
    "scan_i_and_f_swapped": ("state = a * state + (1.0 - a) * (double)i[e];",
                             "state = a * state + (1.0 - a) * (double)f[e];"),
    "scan_stores_before_update": ("                state = a * state + (1.0 - a) * (double)i[e];\n"
                                  "                h[e] = state;",
                                  "                h[e] = state;\n"
                                  "                state = a * state + (1.0 - a) * (double)i[e];"),
    "scan_ignores_h0": ("double state = h0 ? h0[b * D + d] : 0.0;", "double state = 0.0;"),
    "scan_time_major_layout": ("const int64_t e = (b * T + t) * D + d;",
                               "const int64_t e = (t * B + b) * D + d;"),
}


def _pin_tests():
    return [f for mod in (pins, glu_pins, gate_pins, mlgru_pins)
            for name, f in inspect.getmembers(mod, inspect.isfunction)
            if name.startswith("test_") and not hasattr(f, "pytestmark")]


def _run_pins(mod):
    failures = []
    for f in _pin_tests():
        try:
            f(mod)
        except (AssertionError, ValueError, OverflowError, RuntimeError, IndexError) as e:
            failures.append((f.__name__, type(e).__name__))
    return failures


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path, orc):
    old, new = MUTANTS[name]
    src = open(SRC, encoding="utf-8").read()
    assert src.count(old) == 1, f"mutation anchor not unique for {name}"
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new), encoding="utf-8")
    hdr = os.path.join(os.path.dirname(SRC), "oracle.h")
    (tmp_path / "oracle.h").write_text(open(hdr, encoding="utf-8").read(),
                                       encoding="utf-8")
    so = tmp_path / "liboracle_mut.so"
    subprocess.check_call(["gcc", *oracle.CFLAGS, str(mutated), "-o", str(so), "-lm"])
    saved = oracle._lib
    oracle._lib = oracle.load(str(so))
    try:
        failures = _run_pins(oracle)
    finally:
        oracle._lib = saved
    assert failures, f"mutant {name} survived every pin"


def test_unmutated_oracle_passes_every_pin(orc):
    assert _run_pins(orc) == []
