"""The pins must be strong enough to catch plausible mistakes in the oracle.

Each case below plants one mistake in a copy of the oracle's C source (on the
CPU, in a temporary directory), builds that copy with gcc and runs the pins on
it.  The copy must fail at least one pin.  Mistakes are chosen so that every
access stays in bounds.
"""
import pytest

import oracle
import oracle_pins

MUTANTS = {
    # activation quantizer
    "qb_128": ("#define OR_QB 127.0f", "#define OR_QB 128.0f"),
    "act_round_half_away": ("float r = nearbyintf(q);", "float r = roundf(q);"),
    "act_reciprocal_multiply": ("float q = scaled / e;", "float q = scaled * (1.0f / e);"),
    "act_divide_before_multiply": ("float scaled = row[k] * OR_QB;   /* x * 127.0 */\n"
                                   "            float q = scaled / e;",
                                   "float scaled = row[k] / e;\n"
                                   "            float q = scaled * OR_QB;"),
    "act_no_abs": ("float a = fabsf(row[k]);", "float a = row[k];"),
    "act_no_floor": ("float e = amax < OR_SCALE_FLOOR ? OR_SCALE_FLOOR : amax;",
                     "float e = amax;"),
    # weight quantizer
    "gamma_divides_by_rows": ("const uint64_t D = (uint64_t)N * (uint64_t)K;",
                              "const uint64_t D = (uint64_t)N;"),
    "gamma_exponent_off_by_one": ("int t = e ? (int)e - 1 : 0;", "int t = e ? (int)e : 0;"),
    "gamma_unit_off_by_one": ("float g = big_ratio_to_f32(&S, -149, D);", "float g = big_ratio_to_f32(&S, -148, D);"),
    "gamma_divides_by_one_less": ("float g = big_ratio_to_f32(&S, -149, D);",
                                  "float g = big_ratio_to_f32(&S, -149, D > 1 ? D - 1 : 1);"),
    "gamma_no_floor": ("if (g < OR_SCALE_FLOOR) g = OR_SCALE_FLOOR;", ""),
    "ternary_round_half_away": ("float r = nearbyintf(t);", "float r = roundf(t);"),
    "ternary_no_clip": ("if (r > 1.0f) r = 1.0f;", ""),
    "ternary_reciprocal": ("float t = W[i] / gamma;", "float t = W[i] * (1.0f / gamma);"),
    # packing
    "pack_field_order_reversed": ("byte |= (uint8_t)(code << (2 * j));",
                                  "byte |= (uint8_t)(code << (6 - 2 * j));"),
    "pack_codes_swapped": ("if (Wt[n * K + k] == 1) code = 2;\n"
                           "                else if (Wt[n * K + k] == 0) code = 1;\n"
                           "                else if (Wt[n * K + k] == -1) code = 0;",
                           "if (Wt[n * K + k] == 1) code = 0;\n"
                           "                else if (Wt[n * K + k] == 0) code = 1;\n"
                           "                else if (Wt[n * K + k] == -1) code = 2;"),
    "pack_pad_code_zero": ("if (k >= K) code = 1;", "if (k >= K) code = 0;"),
    # contraction
    "contract_sign_swapped": ("int64_t acc = plus - minus;", "int64_t acc = minus - plus;"),
    "contract_drops_minus": ("else if (wr[k] == -1) minus += xr[k];",
                             "else if (wr[k] == -1) minus += 0;"),
    "contract_short_loop": ("for (int64_t k = 0; k < j->K; ++k) {\n                if (wr[k]",
                            "for (int64_t k = 0; k + 1 < j->K; ++k) {\n                if (wr[k]"),
    "contract_transposed_store": ("j->y[m * j->N + n] = (int32_t)acc;",
                                  "j->y[n * j->M + m] = (int32_t)acc;"),
    # absmedian gamma
    "absmedian_lower_median": ("const uint32_t lo = mag[(D - 1) / 2], hi = mag[D / 2];",
                               "const uint32_t lo = mag[(D - 1) / 2], hi = mag[(D - 1) / 2];"),
    "absmedian_upper_median": ("const uint32_t lo = mag[(D - 1) / 2], hi = mag[D / 2];",
                               "const uint32_t lo = mag[D / 2], hi = mag[D / 2];"),
    "absmedian_index_off_by_one": ("const uint32_t lo = mag[(D - 1) / 2], hi = mag[D / 2];",
                                   "const uint32_t lo = mag[D / 2], hi = mag[D / 2 < D - 1 ? D / 2 + 1 : D / 2];"),
    "absmedian_no_floor": ("    if (!(g >= OR_SCALE_FLOOR)) g = OR_SCALE_FLOOR;", ""),
    "absmedian_sum_not_mean": ("float g = big_ratio_to_f32(&S, -149, 2);", "float g = big_ratio_to_f32(&S, -149, 1);"),
    # base-3 packing
    "pack3_digit_order_reversed": ("int v = 0, place = 1;\n            for (int j = 0; j < 5; ++j, place *= 3) {",
                                   "int v = 0, place = 81;\n            for (int j = 0; j < 5; ++j, place /= 3) {"),
    "pack3_pad_digit_zero": ("if (k >= K) digit = 1;                    /* pad: zero weight */",
                             "if (k >= K) digit = 0;                    /* pad: zero weight */"),
    "pack3_codes_swapped": ("else if (Wt[n * K + k] == 1) digit = 2;", "else if (Wt[n * K + k] == 1) digit = 0;"),
    "unpack3_accepts_243": ("if (v >= 243) return -4;", "if (v >= 244) return -4;"),
    "pack3_row_bytes": ("int64_t oracle_packed3_row_bytes(int64_t K) { return (K + 4) / 5; }",
                        "int64_t oracle_packed3_row_bytes(int64_t K) { return K / 5 + 1; }"),
    # RMSNorm
    "rms_mean_over_k_minus_1": ("const float ms = big_ratio_to_f32(&S, -298, (uint64_t)K);",
                                "const float ms = big_ratio_to_f32(&S, -298, (uint64_t)(K > 1 ? K - 1 : 1));"),
    "rms_abs_not_square": ("uint64_t sq = sig * sig;", "uint64_t sq = sig;"),
    "rms_no_eps": ("const float t = ms + OR_RMS_EPS;", "const float t = ms;"),
    "rms_eps_1e5": ("#define OR_RMS_EPS 1e-6f", "#define OR_RMS_EPS 1e-5f"),
    "rms_no_sqrt": ("const float s = sqrtf(t);", "const float s = t;"),
    "rms_divide_by_s": ("xn[m * K + k] = row[k] * norm;", "xn[m * K + k] = row[k] / s;"),
    "rms_float_running_sum": ("const float ms = big_ratio_to_f32(&S, -298, (uint64_t)K);",
                              "float fs = 0.0f;\n"
                              "        for (int64_t q = 0; q < K; ++q) fs += row[q] * row[q];\n"
                              "        const float ms = fs / (float)K;"),
    "ratio_truncates": ("if (rb && (sticky || (sig & 1u))) ++sig;             /* round half to even */", ""),
    "ratio_no_sticky": ("sticky = rem != 0 || big_any_below(S, pos);", "sticky = 0;"),
    "ratio_25_bit_significand": ("p_lsb = a - 23 > -149 ? a - 23 : -149;",
                                 "p_lsb = a - 24 > -149 ? a - 24 : -149;"),
    "ratio_flush_subnormal": ("if (a <= -151) return 0.0f;", "if (a <= -127) return 0.0f;"),
    # dequant
    "dequant_drops_gamma": ("float eg = eta[m] * gamma;", "float eg = eta[m];"),
    "dequant_divides_by_128": ("float s = eg / OR_QB;", "float s = eg / 128.0f;"),
    "dequant_reciprocal_association": ("float s = eg / OR_QB;        /* ... / 127.0 */",
                                       "float s = eta[m] * (gamma / OR_QB);"),
    "dequant_eta_over_127_first": ("float s = eg / OR_QB;        /* ... / 127.0 */",
                                   "float s = (eta[m] / OR_QB) * gamma;"),
}


def _pins_fail(O) -> list:
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(O)
        except (AssertionError, oracle.OracleError) as e:  # noqa: F841
            failed.append(pin.__name__)
            break
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = oracle.source_text()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    O = oracle.compile_variant(src.replace(old, new), str(tmp_path / f"liboracle_{name}.so"))
    assert _pins_fail(O), f"no pin caught the planted mistake {name}"
