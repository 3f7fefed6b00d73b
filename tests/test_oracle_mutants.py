"""Plant mistakes in copies of the oracle source and check that a pin catches each.

Every mutant is a plausible slip (a dropped term, a wrong sign or index, a
swapped operand or field); each is compiled on the CPU into a temporary
library and run through the pins.  A mutant that no pin catches fails here.
"""
import os

import pytest

import oracle
import pins

MUTANTS = {
    "dropped_bias": ("+ value_at(b, sb_dt, (size_t)n * G + g);\n            acc += value_at(x, x_dt",
                     ";\n            acc += value_at(x, x_dt"),
    "nibble_order_reversed": ("return (unsigned)((window >> sh) & ((1u << bits) - 1u));",
                              "return (unsigned)((window >> (32 - bits - sh)) & ((1u << bits) - 1u));"),
    "straddling_field_truncated": ("if (sh + bits > 32) window |= (uint64_t)row[wi + 1] << 32;", ""),
    "wrong_group_index": ("long g = k / gs;", "long g = (k + 1) / gs; if (g >= G) g = G - 1;"),
    "x_index_transposed": ("acc += value_at(x, x_dt, (size_t)m * K + k) * wk;",
                           "acc += value_at(x, x_dt, (size_t)k * M + m) * wk;"),
    "scale_bias_swapped": ("double wk = value_at(s, sb_dt, (size_t)n * G + g) * (double)code_at(row, k, bits)\n                      + value_at(b, sb_dt, (size_t)n * G + g);",
                           "double wk = value_at(b, sb_dt, (size_t)n * G + g) * (double)code_at(row, k, bits)\n                      + value_at(s, sb_dt, (size_t)n * G + g);"),
    "split_end_inclusive": ("for (long k = (long)g0 * gs; k < (long)g1 * gs; ++k) {",
                            "for (long k = (long)g0 * gs; k < (long)(g1 < G ? g1 + 1 : g1) * gs; ++k) {"),
    "hoisted_sum_x_per_row": ("        for (int g = 0; g < G; ++g) {\n            double qx = 0.0, xs = 0.0;",
                              "        double xs = 0.0;\n        for (int g = 0; g < G; ++g) {\n            double qx = 0.0;"),
    "i8_no_sign_extension": ("return v >= 128 ? (int)v - 256 : (int)v;", "return (int)v;"),
    "i8_block_scale_shifted": ("acc += (double)wd[(long)n * nb + b] * (double)dot;",
                               "acc += (double)wd[(long)n * nb + (b + 1) % nb] * (double)dot;"),
    "q8_no_sign_extension": ("int q = byte >= 128 ? (int)byte - 256 : (int)byte;", "int q = (int)byte;"),
    "q8_scale_high_half": ("double d = dec_f16((uint16_t)(blk[0] & 0xFFFFu));",
                           "double d = dec_f16((uint16_t)(blk[0] >> 16));"),
    "q4k_min_sub_block": ("m1 = dmin * q4k_field(sw, 2 * g, 1);", "m1 = dmin * q4k_field(sw, 2 * g + 1, 1);"),
    "q4k_nibbles_swapped": ("acc += (d1 * (double)(qb & 15u) - m1)", "acc += (d1 * (double)(qb >> 4) - m1)"),
    "q4k_min_sign": ("acc += (d2 * (double)(qb >> 4) - m2)", "acc += (d2 * (double)(qb >> 4) + m2)"),
    "q4k_high_scale_bits": ("| ((byte_of(scale_words, j - 4) >> 6) << 4);", "| ((byte_of(scale_words, j - 4) >> 4) << 4);"),
    "f16_exponent_off_by_one": ("v = ldexp((double)(1024 + f), e - 25);", "v = ldexp((double)(1024 + f), e - 24);"),
    "round_ties_away": ("double r = nearbyint(v / ulp) * ulp;", "double r = round(v / ulp) * ulp;"),
    "bf16_decode_low_half": ("uint32_t u = (uint32_t)h << 16;", "uint32_t u = ((uint32_t)h << 16) | 0x8000u;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique or missing"
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(old, new))
    lib = oracle.build(str(mutant_src), str(tmp_path / f"libmut_{name}.so"))
    failed = pins.failing_pins(oracle.Oracle(lib))
    assert failed, f"no pin catches mutant {name}"
