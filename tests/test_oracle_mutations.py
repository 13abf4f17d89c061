"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (on the CPU; the real oracle is not
touched), compiles it, and runs the pins from test_oracle_e4m3 / _quant / _gemm / _dequant / _moe / _fp4 /
_per_channel / _e5m6 / _swiglu
against it until one fails.  At least one pin must fail for every planted mistake.
"""
import os

import pytest

import oracle
import test_oracle_dequant as td
import test_oracle_e4m3 as te
import test_oracle_e5m6 as t56
import test_oracle_fp4 as tf
import test_oracle_gemm as tg
import test_oracle_moe as tm
import test_oracle_per_channel as tp
import test_oracle_swiglu as ts
import test_oracle_quant as tq

SRC = open(os.path.join(os.path.dirname(oracle.__file__), "fp8q_oracle.c")).read()

MUTATIONS = {
    "scale_divisor_447": ("amax / 448.0f", "amax / 447.0f"),
    "ties_away_from_zero": ("(a == half && (c & 1u))", "(a == half)"),
    "ties_down": ("(a == half && (c & 1u))", "(a == half && 0)"),
    "midpoint_inclusive": ("if (a > half ||", "if (a >= half ||"),
    "sign_dropped": ("return (uint8_t)(sign | c);", "return (uint8_t)c;"),
    "subnormal_exponent": ("ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    "normal_bias_8": ("(int)e - 7)", "(int)e - 8)"),
    "bf16_widen_shift": ("(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    "act_scale_layout_row_major": ("s[kb * M + m] = scale;", "s[m * KB + kb] = scale;"),
    "gemm_act_scale_wrong_index": ("(double)sa[kb * M + m]", "(double)sa[m]"),
    "gemm_weight_scale_dropped": ("* (double)sw_rowblock[kb];", ";"),
    "gemm_weight_transposed": ("qw + n * K, sw + (n / GROUP) * KB", "qw + n, sw + (n / GROUP) * KB"),
    "gemm_bound_signed": ("b += fabs(a_deq) * fabs(w_deq);", "b += a_deq * w_deq;"),
    "weight_amax_one_row": ("const uint16_t *row = w + (nb * GROUP + i) * K + kb * GROUP;",
                            "const uint16_t *row = w + (nb * GROUP) * K + kb * GROUP;"),
    "weight_scale_layout": ("s[nb * KB + kb] = scale;", "s[kb * NB + nb] = scale;"),
    "grouped_expert_off_by_one": ("const uint8_t *w_e = qw + e * N * K;",
                                  "const uint8_t *w_e = qw + (e > 0 ? e - 1 : 0) * N * K;"),
    "zero_group_sign_lost": ("return signbit(x) ? 0x80u : 0x00u; /* all-zero group */", "return 0x00u;"),
    "dequant_truncates_to_bf16": ("if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))", "if (0)"),
    "dequant_bf16_ties_away": ("if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))", "if (lower >= 0x8000u)"),
    "dequant_scale_ignores_k_block": ("(double)s[(n / GROUP) * KB + k / GROUP]", "(double)s[(n / GROUP) * KB]"),
    "route_ties_to_higher_index": ("(best < 0 || v[e] > v[best])", "(best < 0 || v[e] >= v[best])"),
    "route_segments_descending": ("for (int64_t t = 0; t < T; t++) /* ascending tokens",
                                  "for (int64_t t = T - 1; t >= 0; t--) /* ascending tokens"),
    "route_no_padding": ("end += (count[e] + pad - 1) / pad * pad;", "end += count[e];"),
    "route_signed_zero_ordered": ("(best < 0 || v[e] > v[best])",
                                  "(best < 0 || v[e] > v[best] || (v[e] == v[best] && signbit(v[best]) && !signbit(v[e])))"),
    "gather_scale_row_major": ("sa[kb * rows + r] = t >= 0", "sa[r * KB + kb] = t >= 0"),
    "gather_empty_row_copies_token_0": ("qa[r * K + k] = t >= 0 ? q[t * K + k] : 0;", "qa[r * K + k] = q[(t >= 0 ? t : 0) * K + k];"),
    "fp4_ties_not_to_even": ("(dc == db && (c & 1u) == 0)", "(dc == db)"),
    "fp4_divisor_4": ("float scale = amax / 6.0f;", "float scale = amax / 4.0f;"),
    "fp4_nibbles_swapped": ("(uint8_t)(lo | (hi << 4))", "(uint8_t)(hi | (lo << 4))"),
    "fp4_table_entry": ("{0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}", "{0.0, 0.5, 1.0, 1.5, 2.0, 2.5, 4.0, 6.0}"),
    "fp4_no_saturation": ("    if (a >= 6.0) return (uint8_t)(sign | 7u);", ""),
    "per_channel_amax_first_group": ("        for (int64_t k = 0; k < K; k++) {\n            float v = bf16_to_f32(row[k]);\n            if (!isfinite(v)) bad = 1;\n            if (fabsf(v) > amax) amax = fabsf(v);",
                                     "        for (int64_t k = 0; k < K && k < 128; k++) {\n            float v = bf16_to_f32(row[k]);\n            if (!isfinite(v)) bad = 1;\n            if (fabsf(v) > amax) amax = fabsf(v);"),
    "per_channel_signed_amax": ("            if (fabsf(v) > amax) amax = fabsf(v);\n        }\n        float scale = amax / 448.0f;\n        s[n] = scale;",
                                "            if (v > amax) amax = v;\n        }\n        float scale = amax / 448.0f;\n        s[n] = scale;"),
    "e5m6_bias_14": ("return ldexp(64.0 + (double)m, (int)e - 15 - 6);", "return ldexp(64.0 + (double)m, (int)e - 14 - 6);"),
    "e5m6_no_subnormals": ("if (e == 0) return ldexp((double)m, -20);", "if (0) return ldexp((double)m, -20);"),
    "e5m6_ties_away": ("(du == dl && (up & 1u) == 0)", "(du == dl)"),
    "e5m6_divisor_fp16_max": ("float scale = amax / 65024.0f;", "float scale = amax / 65504.0f;"),
    "e5m6_pair_order_swapped": ("out[j / 2 * 3 + 1] = (uint8_t)((c[0] >> 8) | ((c[1] & 0xFu) << 4));",
                                "out[j / 2 * 3 + 1] = (uint8_t)((c[1] >> 8) | ((c[0] & 0xFu) << 4));"),
    "act_amax_skips_last_element": ("for (int j = 0; j < GROUP; j++) {\n                float v = bf16_to_f32(g[j]);\n                if (!isfinite(v)) bad = 1;\n                float av = fabsf(v);",
                                    "for (int j = 0; j < GROUP - 1; j++) {\n                float v = bf16_to_f32(g[j]);\n                if (!isfinite(v)) bad = 1;\n                float av = fabsf(v);"),
    "fp4_weight_amax_one_row": ("const uint16_t *row = w + (nb * GROUP + i) * K + kb * GROUP;\n                for (int j = 0; j < GROUP; j++) {\n                    float v = bf16_to_f32(row[j]);\n                    if (!isfinite(v)) bad = 1;\n                    if (fabsf(v) > amax) amax = fabsf(v);\n                }\n            }\n            float scale = amax / 6.0f;",
                                "const uint16_t *row = w + (nb * GROUP) * K + kb * GROUP;\n                for (int j = 0; j < GROUP; j++) {\n                    float v = bf16_to_f32(row[j]);\n                    if (!isfinite(v)) bad = 1;\n                    if (fabsf(v) > amax) amax = fabsf(v);\n                }\n            }\n            float scale = amax / 6.0f;"),
    "e5m6_no_saturation": ("    if (a >= e5m6_magnitude(E5M6_MAX_CODE)) return (uint16_t)(sign | E5M6_MAX_CODE);\n", ""),
    "e5m6_third_byte_shift": ("out[j / 2 * 3 + 2] = (uint8_t)(c[1] >> 4);", "out[j / 2 * 3 + 2] = (uint8_t)(c[1] >> 8);"),
    "swiglu_sigmoid_sign": ("double v = p / (1.0 + exp(-xv));", "double v = p / (1.0 + exp(xv));"),
    "swiglu_fp32_intermediate": ("double v = p / (1.0 + exp(-xv));", "double v = (double)(float)(p / (1.0 + exp(-xv)));"),
    "swiglu_tiny_gate_side_flipped": ("xv > 0 ? 1 : -1", "xv > 0 ? -1 : 1"),
    "swiglu_large_gate_tie_to_even": ("r = bf16_round_double(p, -1, 0.0, &nt2, &pmid);", "r = bf16_round_double(p, 0, 0.0, &nt2, &pmid);"),
    "swiglu_subnormal_spacing_dropped": ("    if (ex < -126) ex = -126; /* bf16 subnormals share the spacing 2^-133 */", ""),
}


def pins():
    out = [
        (te.test_decode_closed_form_points, {}),
        (te.test_decode_matches_torch_and_is_monotone, {}),
        (te.test_roundtrip_all_finite_codes, {}),
        (te.test_encoder_vs_brute_force_all_bf16_quotients, {"amax": 3.5}),
        (te.test_encoder_signed_zero_and_underflow, {}),
        (tq.test_amax_element_encodes_to_448, {}),
        (tq.test_negation_flips_sign_bits_only, {}),
        (tq.test_dequant_error_bound, {}),
        (tq.test_weight_blocks_use_their_own_scale, {}),
        (tg.test_hand_worked_gemm, {}),
        (tg.test_lossless_case_equals_float64_matmul, {"M": 37, "N": 256, "K": 384}),
        (tg.test_exact_rational_brute_force, {"M": 2, "K": 256}),
        (tg.test_grouped_lossless_and_padding, {}),
        (td.test_every_code_times_sampled_scales_is_rounded_exactly, {}),
        (td.test_unit_code_returns_the_scale_and_powers_of_two_are_exact, {}),
        (td.test_double_rounding_follows_the_fp32_route, {}),
        (td.test_each_block_uses_its_own_scale, {}),
    ]
    out += [
        (tm.test_hand_worked_routing, {}),
        (tm.test_topk_satisfies_the_pairwise_definition, {"T": 25, "E": 64, "k": 8, "heavy": True}),
        (tm.test_k1_is_argmax_and_k_equal_E_is_a_stable_sort, {}),
        (tm.test_layout_invariants, {"T": 300, "E": 64, "k": 8, "extra": 200}),
        (tm.test_gather_hand_case, {}),
        (tm.test_gather_matches_numpy_indexing, {}),
        (tm.test_gather_commutes_with_the_row_quantizer, {}),
    ]
    out += [
        (tf.test_decode_table, {}),
        (tf.test_encoder_against_exact_nearest_search, {}),
        (tf.test_round_trip_of_every_code, {}),
        (tf.test_hand_worked_activation_group, {}),
        (tf.test_amax_encodes_to_six_and_negation_flips_sign_bits, {}),
        (tf.test_error_bound_and_weight_blocks, {}),
        (tp.test_hand_worked_row, {}),
        (tp.test_matches_rowwise_numpy, {}),
        (tp.test_equals_one_group_per_row_when_k_is_128, {}),
        (t56.test_decode_equals_half_precision_with_four_zero_bits, {}),
        (t56.test_hand_worked_group_and_byte_layout, {}),
        (t56.test_encoder_on_every_half_precision_value, {}),
        (t56.test_encoder_against_exact_search_on_midpoints, {}),
        (t56.test_amax_encodes_to_the_largest_code_and_negation_flips_sign_bits, {}),
        (t56.test_error_bound_and_scales, {}),
    ]
    for case in tq.load_golden()["act_groups"]:
        out.append((tq.test_hand_worked_activation_groups, {"case": case}))
    for case in tq.load_golden()["weight_blocks"]:
        out.append((tq.test_hand_worked_weight_block, {"case": case}))
    out += [   # last: the slower ones run only for mistakes that no earlier pin catches
        (ts.test_closed_forms, {}),
        (ts.test_double_evaluation_decides_every_value, {"y_exp": None, "x_max": 126}),
        (ts.test_matches_numpy_float64_away_from_midpoints, {}),
        (ts.test_matches_decimal_on_a_sample, {}),
    ]
    return out


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTATIONS[name]
    assert SRC.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = tmp_path / f"mut_{name}.c"
    src.write_text(SRC.replace(old, new))
    lib = oracle.load(oracle.build(str(src), str(tmp_path / f"mut_{name}.so")))
    caught = None
    for fn, kw in pins():
        try:
            fn(lib, **kw)
        except (AssertionError, ValueError, IndexError):
            caught = fn.__name__
            break
    assert caught, f"no pin catches the planted mistake {name}"
