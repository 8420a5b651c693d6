"""Mistakes planted in a copy of the oracle source must each fail a pin.

The real oracle passes every pin (``test_oracle.py``). Here each plausible
mistake -- a wrong mean denominator, epsilon outside the root, a flipped or
dropped correction term, r^2 for r^3, a missing factor in dW, a wrong weight
or input index, a wrong bf16 or fp16 decode, ties rounded away from zero, a
wrong format width or overflow bound, an unrounded residual sum, a missing
residual gradient, a row skipped in the dW sum -- is planted by text
substitution in a temporary copy of ``rmsnorm_oracle.c``, compiled with gcc,
and run against the same pins. No mutant may pass them all.
"""

import os

import pytest

import oracle
import oracle_pins

MUTANTS = {
    "denominator_N_plus_1": ("double ms = s / (double)N;", "double ms = s / (double)(N + 1);"),
    "eps_outside_root": ("return 1.0 / sqrt(ms + eps);", "return 1.0 / (sqrt(ms) + eps);"),
    "eps_dropped": ("return 1.0 / sqrt(ms + eps);", "return 1.0 / sqrt(ms);"),
    "dx_correction_sign": ("ri * V - in_elem(x, res, dtype, i * N + j) * ri3 * S / (double)N",
                           "ri * V + in_elem(x, res, dtype, i * N + j) * ri3 * S / (double)N"),
    "dx_correction_dropped": ("ri * V - in_elem(x, res, dtype, i * N + j) * ri3 * S / (double)N", "ri * V"),
    "dx_r_squared": ("double ri3 = ri * ri * ri;", "double ri3 = ri * ri;"),
    "dx_correction_no_N": ("ri3 * S / (double)N;", "ri3 * S;"),
    "S_without_weight": ("S += V * in_elem(x, res, dtype, i * N + j);",
                         "S += elem(dy, dtype, i * N + j) * in_elem(x, res, dtype, i * N + j);"),
    "dw_without_r": ("in_elem(x, res, dtype, i * N + j) * ri;\n    }", "in_elem(x, res, dtype, i * N + j);\n    }"),
    "dw_skips_first_row": ("for (int64_t i = 0; i < M; ++i) {", "for (int64_t i = 1; i < M; ++i) {"),
    "y_weight_index": ("* ri * elem(w, wdtype, j);", "* ri * elem(w, wdtype, (i + j) % N);"),
    "y_input_transposed": ("double v = in_elem(x, res, dtype, i * N + j);\n            if (h && res)",
                           "double v = in_elem(x, res, dtype, (j * M + i) % (M * N));\n            if (h && res)"),
    "bf16_decode_shift": ("<< 16;", "<< 15;"),
    "y_missing_weight": ("* ri * elem(w, wdtype, j);", "* ri;"),
    "half_exponent_bias": ("e - 25); /* (1 + f/1024)", "e - 24); /* (1 + f/1024)"),
    "half_subnormal_scale": ("ldexp((double)f, -24);", "ldexp((double)f, -25);"),
    "round_ties_away": ("nearbyint(ldexp(v, -q))", "round(ldexp(v, -q))"),
    "round_bf16_bits": ("round_format(v, 8, -126, 127)", "round_format(v, 9, -126, 127)"),
    "round_f16_overflow": ("round_format(v, 11, -14, 15)", "round_format(v, 11, -14, 16)"),
    "residual_not_rounded": ("return round_storage(elem(x, dtype, idx) + elem(res, dtype, idx), dtype);",
                             "return elem(x, dtype, idx) + elem(res, dtype, idx);"),
    "residual_dh_not_added": ("dx[k * N + j] = dh ? g + elem(dh, dtype, i * N + j) : g;", "dx[k * N + j] = g;"),
    "residual_ignored_in_dw": ("* in_elem(x, res, dtype, i * N + j) * ri;", "* elem(x, dtype, i * N + j) * ri;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique in the oracle source"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.build(str(mutated), str(tmp_path / f"lib_{name}.so"), extra_flags=("-Wno-error",))
    orc = oracle.Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
