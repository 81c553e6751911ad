"""Planted mistakes in the oracle (on the CPU) must each fail at least one pin.

Each mutant is a copy of oracle/qmv_oracle.c with one plausible mistake -- a
dropped term, a wrong sign, a wrong index, a transposed operand, a wrong field
order, a wrong conversion -- compiled into a temporary library.  The test
passes when every mutant is rejected by the pins of tests/pins.py.
"""
import os

import pytest

import pins
from oracle import oracle

MUTANTS = {
    "bias_sign": ("acc += s * D + b * S;", "acc += s * D - b * S;"),
    "bias_dropped": ("acc += s * D + b * S;", "acc += s * D;"),
    "scale_bias_swapped": ("double s = elem(scales,", "double s = elem(biases,"),
    "sum_x_weighted": ("S += xv;", "S += q * xv;"),
    "field_order_reversed": ("return (w >> (bits * j))", "return (w >> (bits * (pf - 1 - j)))"),
    "field_mask_wide": ("& ((1u << bits) - 1u);", "& ((1u << (bits + 1)) - 1u);"),
    "group_param_shifted": ("double s = elem(scales, (size_t)n * G + g, sb_dt);",
                            "double s = elem(scales, (size_t)n * G + (g + 1) % G, sb_dt);"),
    "x_row_ignored": ("elem(x, (size_t)m * (size_t)K + (size_t)k, x_dt)", "elem(x, (size_t)k, x_dt)"),
    "group_short": ("for (int k = g * gs; k < (g + 1) * gs; ++k)", "for (int k = g * gs; k < (g + 1) * gs - 1; ++k)"),
    "f16_exponent_bias": ("e - 25", "e - 24"),
    "f16_subnormal_flushed": ("v = ldexp((double)f, -24);", "v = 0.0;"),
    "bf16_ties_away": ("(lower == 0x8000u && (upper & 1u))", "(lower == 0x8000u)"),
    "row_stride_wrong": ("(size_t)n * (size_t)(K * bits / 32)", "(size_t)n * (size_t)(K * bits / 32 - 1)"),
    # term magnitude of the a-priori error bound
    "mag_bias_dropped": ("acc += (span * s + b) * A;", "acc += (span * s) * A;"),
    "mag_span_short": ("ldexp(1.0, bits + 2);", "ldexp(1.0, bits + 1);"),
    "mag_x_signed": ("A += fabs(elem(x, (size_t)m * (size_t)K + (size_t)k, x_dt));\n                double s",
                     "A += elem(x, (size_t)m * (size_t)K + (size_t)k, x_dt);\n                double s"),
    "mag_bias_signed": ("double b = fabs(elem(biases,", "double b = (elem(biases,"),
    # output rounding
    "round_f32_truncates": ("float f = (float)y[i];", "float f = (float)y[i]; { uint32_t t; memcpy(&t, &f, 4); "
                            "if (fabs((double)f) > fabs(y[i])) { t -= 1u; memcpy(&f, &t, 4); } }"),
    # mxfp4 mode
    "mx_mag_six": ("* 6.0 * A;", "* 4.0 * A;"),
    "e2m1_exponent_bias": ("ldexp(1.0 + 0.5 * m, e - 1)", "ldexp(1.0 + 0.5 * m, e)"),
    "e2m1_subnormal": ("(e == 0) ? 0.5 * m :", "(e == 0) ? 1.0 * m :"),
    "e2m1_sign_ignored": ("ldexp(1.0 + 0.5 * m, e - 1);\n    return sign ? -v : v;",
                          "ldexp(1.0 + 0.5 * m, e - 1);\n    return v;"),
    "e8m0_bias": ("(int)(E & 0xffu) - 127", "(int)(E & 0xffu) - 126"),
    "mx_block_scale_shifted": ("scales[(size_t)n * B + b]", "scales[(size_t)n * B + (b + 1) % B]"),
    "mx_block_short": ("for (int k = b * 32; k < (b + 1) * 32; ++k)", "for (int k = b * 32; k < (b + 1) * 32 - 1; ++k)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    with open(oracle.SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old}"
    mutated = src.replace(old, new)
    cpath = os.path.join(tmp_path, f"orc_{name}.c")
    with open(cpath, "w") as f:
        f.write(mutated)
    lib = oracle.compile_source(cpath, os.path.join(tmp_path, f"liborc_{name}.so"))
    orc = oracle.Oracle(lib)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
