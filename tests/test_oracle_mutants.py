"""Plant mistakes in copies of the oracle (on the CPU) and check the pins catch them.

Each mutant is oracle.c with one textual change, compiled into a temporary
directory.  A mutant that no pin rejects means the pins are too weak."""
import os
import shutil

import pytest

import oracle
import oracle_pins

MUTANTS = {
    "order_map_other_reading": ("static const int AWQ_ORDER[8] = {0, 2, 4, 6, 1, 3, 5, 7};",
                                "static const int AWQ_ORDER[8] = {0, 4, 1, 5, 2, 6, 3, 7};"),
    "zero_point_dropped": ("w[col * t->K + k] = (double)(q - z) * s;",
                           "w[col * t->K + k] = (double)(q) * s;"),
    "zero_point_sign": ("w[col * t->K + k] = (double)(q - z) * s;",
                        "w[col * t->K + k] = (double)(z - q) * s;"),
    "group_index": ("int64_t g = k / t->G;", "int64_t g = (k / t->G) / 2;"),
    "scale_column_index": ("t->scales[g * t->N + 8 * j + col]", "t->scales[g * t->N + 8 * j + i]"),
    "matmul_dropped_term": ("for (int64_t k = 0; k < t->K; k++) acc += xr[k] * wc[k];",
                            "for (int64_t k = 1; k < t->K; k++) acc += xr[k] * wc[k];"),
    "k8_order": ("static const int K8_ORDER[8] = {0, 4, 1, 5, 2, 6, 3, 7};",
                 "static const int K8_ORDER[8] = {0, 1, 2, 3, 4, 5, 6, 7};"),
    "int4_offset_binary": ("static int sext4(unsigned v) { return (int)(v ^ 8u) - 8; }",
                           "static int sext4(unsigned v) { return (int)v - 8; }"),
    "round_half_away": ("float r = rintf(xf / s);", "float r = roundf(xf / s);"),
    "s1_not_rounded": ("float s = (float)round_act((double)q32, dtype);", "float s = q32;"),
    "s1_fp16_for_bf16": ("return dtype == 1 ? orc_bf16_to_f64(orc_f64_to_bf16(v)) : orc_f16_to_f64(orc_f64_to_f16(v));",
                         "return orc_f16_to_f64(orc_f64_to_f16(v));"),
    "bf16_ties_away": ("double r = nearbyint(ldexp(a, 7 - E));", "double r = floor(ldexp(a, 7 - E) + 0.5);"),
    "bf16_subnormal_quantum": ("double r = nearbyint(ldexp(a, 133));", "double r = nearbyint(ldexp(a, 134));"),
    "w4a8_scale_dtype_ignored": ("double s2 = decode_act(t->s2[n], t->dtype);", "double s2 = decode_act(t->s2[n], 0);"),
    "quant_input_dtype_ignored": ("double v = fabs(decode_act(row[k], dtype));", "double v = fabs(decode_act(row[k], 0));"),
    "clamp_low_bound": ("if (r < -128.0f) r = -128.0f;", "if (r < -127.0f) r = -127.0f;"),
    "group_scale_dropped": ("w8[k] = q * mult;", "w8[k] = q;"),
    "w4a8_s1_dropped": ("(double)acc * (double)t->s1[m] * s2;", "(double)acc * s2;"),
    "f16_subnormal_exponent": ("v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    "f16_ties_away": ("double r = nearbyint(ldexp(a, 10 - E));",
                      "double r = floor(ldexp(a, 10 - E) + 0.5);"),
    "pack_no_clamp": ("if (v > 15) {\n                    v = 15;", "if (v > 15) {\n                    v = v & 15;"),
    "w4a16_act_dtype_ignored": ("for (int64_t i = 0; i < M * K; i++) xd[i] = decode_act(x[i], dtype);",
                                "for (int64_t i = 0; i < M * K; i++) xd[i] = decode_act(x[i], 0);"),
    "w4a16_scale_dtype_ignored": ("double s = decode_act(t->scales[g * t->N + 8 * j + col], t->dtype);",
                                  "double s = decode_act(t->scales[g * t->N + 8 * j + col], 0);"),
    "e4m3_bias": ("v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */",
                  "v = ldexp((double)(8 + m), e - 11); /* (1 + m/8) * 2^(e-7) */"),
    "e4m3_subnormal_quantum": ("v = ldexp((double)m, -9); /* subnormal: m * 2^-9 */",
                               "v = ldexp((double)m, -10); /* subnormal: m * 2^-9 */"),
    "e4m3_no_saturation": ("if (a > 448.0) a = 448.0;", "if (a > 480.0) a = 480.0;"),
    "e4m3_ties_away": ("double r = nearbyint(ldexp(a, 3 - E));", "double r = floor(ldexp(a, 3 - E) + 0.5);"),
    "fp8_divisor_127": ("float quot = (float)amax / 448.0f;", "float quot = (float)amax / 127.0f;"),
    "fp8_s1_not_rounded": ("float s = (float)round_act((double)quot, dtype);", "float s = quot;"),
    "fp8_input_dtype_ignored": ("double mag = fabs(decode_act(row[k], dtype));", "double mag = fabs(decode_act(row[k], 0));"),
    "fp8_asum_magnitudes": ("sum += orc_e4m3_to_f64(c);", "sum += fabs(orc_e4m3_to_f64(c));"),
    "fp8_gemm_s1_dropped": ("if (y) y[m * N + n] = sacc * (double)s1[m] * s2n;", "if (y) y[m * N + n] = sacc * s2n;"),
    "fp8_gemm_k8_order": ("for (int i = 0; i < 8; i++) q[8 * kb + K8_ORDER[i]] = sext4((w >> (4 * i)) & 0xF);",
                          "for (int i = 0; i < 8; i++) q[8 * kb + i] = sext4((w >> (4 * i)) & 0xF);"),
    "v2_order_reversed": ("int q = (int)(((uint32_t)qweight[k * wc + n / 8] >> (4 * (n % 8))) & 0xF);",
                          "int q = (int)(((uint32_t)qweight[k * wc + n / 8] >> (4 * (7 - n % 8))) & 0xF);"),
    "v2_zero_nibble": ("(int)(((uint32_t)qzeros[n * zw + g / 8] >> (4 * (g % 8))) & 0xF)",
                       "(int)(((uint32_t)qzeros[n * zw + g / 8] >> (4 * (g % 4))) & 0xF)"),
    "v2_pack_order": ("word |= (uint32_t)v << (4 * i);", "word |= (uint32_t)v << (4 * (7 - i));"),
    "bf16_shift": ("uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mpath = tmp_path / "oracle_mutant.c"
    mpath.write_text(src.replace(old, new))
    lib = oracle.compile_oracle(str(mpath), str(tmp_path / "libmut.so"))
    mut = oracle.Oracle(lib)
    caught = None
    for pin in oracle_pins.ALL_PINS:  # cheap pins first; the first catch is enough
        try:
            pin(mut)
        except (AssertionError, ValueError):
            caught = pin.__name__
            break
    assert caught, f"no pin catches mutant {name}"
