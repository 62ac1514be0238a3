"""Planted mistakes: each test copies the oracle's C source, plants one
plausible mistake (a wrong rounding, scale, index, sign, operand, order or a
dropped term), builds the copy with gcc and checks that at least one pin of
``tests/pins.py`` fails on it.  The real oracle is never modified.  No GPU."""
import os

import pytest

import oracle
import pins
import pins_e4m3
import pins_int4

MUTANTS = {
    "round_half_away": ("float r = nearbyintf(t); /* default rounding mode", "float r = roundf(t); /* default rounding mode"),
    "scale_over_128": ("float s = absmax / 127.0f;", "float s = absmax / 128.0f;"),
    "scale_by_reciprocal": ("float s = absmax / 127.0f;", "float s = absmax * (1.0f / 127.0f);"),
    "quotient_by_reciprocal": ("float t = v[i] / s;\n        float r = nearbyintf(t); /* default",
                               "float t = v[i] * (1.0f / s);\n        float r = nearbyintf(t); /* default"),
    "clamp_to_minus_128": ("if (r < -127.0f)\n            r = -127.0f;",
                           "if (r < -128.0f)\n            r = -128.0f;"),
    "no_clamp": ("if (r > 127.0f)\n            r = 127.0f;\n        if (r < -127.0f)\n            r = -127.0f;\n",
                 ""),
    "zero_rule_on_absmax": ("if (s == 0.0f) {\n            q[i] = 0;", "if (absmax == 0.0f) {\n            q[i] = 0;"),
    "absmax_without_abs": ("float m = fabsf(v[i]);\n        if (m > absmax)\n            absmax = m;\n    }\n    float s = absmax / 127.0f;",
                           "float m = v[i];\n        if (m > absmax)\n            absmax = m;\n    }\n    float s = absmax / 127.0f;"),
    "reduce_drops_last_rank": ("for (size_t r = 1; r < nranks; r++)\n            for (size_t i = 0; i < len; i++)\n                acc[i] = acc[i] + dequant_value(",
                               "for (size_t r = 1; r + 1 < nranks; r++)\n            for (size_t i = 0; i < len; i++)\n                acc[i] = acc[i] + dequant_value("),
    "reduce_rank_order": ("acc[i] = acc[i] + dequant_value(codes[r][start + i], scales[r][b]);",
                          "acc[i] = acc[i] + dequant_value(codes[nranks - r][start + i], scales[nranks - r][b]);"),
    "reduce_fma": ("acc[i] = acc[i] + dequant_value(codes[r][start + i], scales[r][b]);",
                   "acc[i] = fmaf((float)codes[r][start + i], scales[r][b], acc[i]);"),
    "dequant_scale_index": ("out[i] = dequant_value(codes[i], scales[i / block]);",
                            "out[i] = dequant_value(codes[i], scales[(i / block) & ~(size_t)1]);"),
    "ring_subtracts_local": ("dequant_value(codes_in[start + i], scales_in[b]) +\n", "dequant_value(codes_in[start + i], scales_in[b]) -\n"),
    "ring_first_scale": ("acc[i] = dequant_value(codes_in[start + i], scales_in[b]) +",
                         "acc[i] = dequant_value(codes_in[start + i], scales_in[0]) +"),
    "ring_local_as_bf16": ("scales_in[b]) +\n                     load_element(local, dtype, start + i);\n        if (!all_finite(acc, len)) {\n            free(acc);\n            return ORACLE_NONFINITE;\n        }\n        quantize_one_block(acc",
                           "scales_in[b]) +\n                     load_element(local, ORACLE_BF16, start + i);\n        if (!all_finite(acc, len)) {\n            free(acc);\n            return ORACLE_NONFINITE;\n        }\n        quantize_one_block(acc"),
    "bf16_ties_away": ("if (rest > 0x8000u || (rest == 0x8000u && (upper & 1u)))", "if (rest >= 0x8000u)"),
    "bf16_truncates": ("upper += 1u;", "upper += 0u;"),
    "unquantized_drops_rank": ("for (size_t r = 1; r < nranks; r++)\n            acc = acc + load_element(x[r], dtype, i);",
                               "for (size_t r = 2; r < nranks; r++)\n            acc = acc + load_element(x[r], dtype, i);"),
    "unquantized_reverse_order": ("float acc = load_element(x[0], dtype, i);\n        for (size_t r = 1; r < nranks; r++)\n            acc = acc + load_element(x[r], dtype, i);",
                                  "float acc = load_element(x[nranks - 1], dtype, i);\n        for (size_t r = 1; r < nranks; r++)\n            acc = acc + load_element(x[nranks - 1 - r], dtype, i);"),
    # FP8 E4M3 codes
    "e4m3_scale_over_240": ("float s = absmax / E4M3_MAX;", "float s = absmax / 240.0f;"),
    "e4m3_ties_up": ("(above == below && (c & 1u))", "(above == below)"),
    "e4m3_truncates": ("if (above < below || (above == below && (c & 1u)))\n            c++;",
                       "if (above < below && 0)\n            c++;"),
    "e4m3_bias_8": ("ldexpf((float)(8 + m), e - 10)", "ldexpf((float)(8 + m), e - 11)"),
    "e4m3_subnormal_step": ("ldexpf((float)m, -9)", "ldexpf((float)m, -10)"),
    "e4m3_unsigned_zero": ("uint8_t sign = signbit(t) ? 0x80 : 0x00;", "uint8_t sign = t < 0.0f ? 0x80 : 0x00;"),
    "e4m3_clamp_240": ("if (t > E4M3_MAX)\n            t = E4M3_MAX;", "if (t > 240.0f)\n            t = 240.0f;"),
    "e4m3_zero_code_negative": ("q[i] = 0x00;\n            continue;", "q[i] = 0x80;\n            continue;"),
    "e4m3_reduce_order": ("acc[i] = acc[i] + dequant_value_e4m3(codes[r][start + i], scales[r][b]);",
                          "acc[i] = acc[i] + dequant_value_e4m3(codes[nranks - r][start + i], scales[nranks - r][b]);"),
    "e4m3_reduce_fma": ("acc[i] = acc[i] + dequant_value_e4m3(codes[r][start + i], scales[r][b]);",
                        "acc[i] = fmaf(e4m3_value(codes[r][start + i]), scales[r][b], acc[i]);"),
    "e4m3_ring_subtracts": ("acc[i] = dequant_value_e4m3(codes_in[start + i], scales_in[b]) +",
                            "acc[i] = dequant_value_e4m3(codes_in[start + i], scales_in[b]) -"),
    "e4m3_dequant_bf16_truncates": ("dequant_value_e4m3(codes[i], scales[i / block]);\n        if (out_dtype == ORACLE_BF16)\n            ((uint16_t*)out)[i] = float_to_bf16_bits(y);",
                                    "dequant_value_e4m3(codes[i], scales[i / block]);\n        if (out_dtype == ORACLE_BF16)\n            { uint32_t u_; memcpy(&u_, &y, 4); ((uint16_t*)out)[i] = (uint16_t)(u_ >> 16); }"),
    # 4-bit codes
    "int4_scale_over_8": ("float s = absmax / 7.0f;", "float s = absmax / 8.0f;"),
    "int4_ties_away": ("float r = nearbyintf(t); /* to nearest, ties to even */",
                       "float r = roundf(t); /* to nearest, ties to even */"),
    "int4_clamp_8": ("if (r < -7.0f)\n            r = -7.0f;", "if (r < -8.0f)\n            r = -8.0f;"),
    "int4_nibbles_swapped": ("unsigned shift = 4 * (unsigned)(i % 2);", "unsigned shift = 4 * (unsigned)(1 - i % 2);"),
    "int4_sign_extension": ("return v >= 8 ? (int)v - 16 : (int)v;", "return v >= 8 ? (int)v - 15 : (int)v;"),
    "int4_reduce_order": ("acc[i] = acc[i] + dequant_value_int4(codes[r], start + i, scales[r][b]);",
                          "acc[i] = acc[i] + dequant_value_int4(codes[nranks - r], start + i, scales[nranks - r][b]);"),
    "int4_ring_subtracts": ("dequant_value_int4(codes_in, start + i, scales_in[b]) + load_element",
                            "dequant_value_int4(codes_in, start + i, scales_in[b]) - load_element"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique in the oracle source"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib = oracle.build(str(path), str(tmp_path / f"lib{name}.so"))
    mutant = oracle.Oracle(lib)
    caught = None
    for pin in pins.ALL_PINS + pins_e4m3.ALL_PINS + pins_int4.ALL_PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError) as e:
            caught = (pin.__name__, str(e)[:120])
            break
    assert caught is not None, f"no pin catches the planted mistake {name}"
    print(f"{name}: caught by {caught[0]} ({caught[1]})")
    os.remove(lib)
