"""The oracle's pins catch plausible slips.

Each case below plants one plausible mistake in a scratch copy of the
oracle's C source (a swapped lane map, another summation or fold order, a
reciprocal instead of a true division, round half away from zero, another
grouping of the rescale, ...), compiles that copy on the CPU, points the
oracle module at it, and checks that at least one of the named pins in
tests/test_oracle_pins.py now fails.  The correct oracle passes all of them
(test_oracle_pins.py itself), so every slip listed here is one the pins
would reveal.  Nothing here touches a GPU.
"""
import os
import subprocess

import pytest

import oracle
from oracle import build as obuild

import test_oracle_attention as attn_pins
import test_oracle_backward as backward_pins
import test_oracle_pins as pins
import test_oracle_sampler as sampler_pins

SRC = obuild.SRC

FOLD = ("    for (int h = 128; h >= 1; h /= 2)\n"
        "        for (int t = 0; t < h; ++t)\n"
        "            p[t] = p[t] + p[t + h];\n")
ADJ = ("    for (int w = 256; w > 1; w /= 2)\n"
       "        for (int t = 0; t < w / 2; ++t)\n"
       "            p[t] = p[2 * t] + p[2 * t + 1];\n")

# name -> (list of (old, new) substitutions, pins expected to catch it)
MUTANTS = {
    # --- the absmean order ("the bytes": beta = mean|W| + eps) --------------
    "absmean_lane_map_t_plus_256j": (
        [("1024 * (int64_t)i + 4 * t + j;", "1024 * (int64_t)i + t + 256 * j;")],
        ["test_absmean_stated_order_fixtures"]),
    "absmean_lane_value_sequential": (
        [("        float lo = acc[0] + acc[1];\n        float hi = acc[2] + acc[3];\n"
          "        p[t] = lo + hi;",
          "        p[t] = ((acc[0] + acc[1]) + acc[2]) + acc[3];")],
        ["test_absmean_stated_order_fixtures"]),
    "absmean_lane_value_pairs_0_2": (
        [("float lo = acc[0] + acc[1];", "float lo = acc[0] + acc[2];"),
         ("float hi = acc[2] + acc[3];", "float hi = acc[1] + acc[3];")],
        ["test_absmean_stated_order_fixtures"]),
    "absmean_steps_reversed": (
        [("        for (int i = 0; i < 8; ++i)\n            for (int j = 0; j < 4; ++j) {",
          "        for (int i = 7; i >= 0; --i)\n            for (int j = 0; j < 4; ++j) {")],
        ["test_absmean_stated_order_fixtures"]),
    "absmean_chunk_fold_adjacent_pairs": (
        [(FOLD + "    return p[0];\n}\n\n/* Stage 2", ADJ + "    return p[0];\n}\n\n/* Stage 2")],
        ["test_absmean_stated_order_fixtures"]),
    "absmean_stage2_contiguous_lanes": (
        [("        for (int64_t c = t; c < nchunks; c += 256)\n            acc = acc + S[c];",
          "        int64_t q = (nchunks + 255) / 256;\n"
          "        for (int64_t c = t * q; c < (t + 1) * q && c < nchunks; ++c)\n"
          "            acc = acc + S[c];")],
        ["test_absmean_stated_order_fixtures"]),
    "absmean_stage2_sequential": (
        [("    float T = combine_chunks(S, nchunks);",
          "    float T = 0.0f;\n    for (int64_t c = 0; c < nchunks; ++c)\n        T = T + S[c];")],
        ["test_absmean_stated_order_fixtures"]),
    "absmean_eps_before_mean": (
        [("    float mean = T / (float)(N * K);\n    float beta = mean + eps;",
          "    float beta = (T + eps) / (float)(N * K);")],
        ["test_absmean_closed_forms", "test_absmean_stated_order_fixtures"]),
    # --- the RMSNorm order ("attention, as graph ops") ----------------------
    "row_slot_k_mod_256": (
        [("int t = (int)((k / 4) % 256);", "int t = (int)(k % 256);")],
        ["test_row_sum_squares_stated_order_fixtures"]),
    "row_sum_sequential": (
        [("    return p[0];\n}\n\n/* RMSNorm(x)",
          "    float T = 0.0f;\n    for (int64_t k = 0; k < K; ++k)\n        T = T + x[k] * x[k];\n"
          "    return T;\n}\n\n/* RMSNorm(x)")],
        ["test_row_sum_squares_stated_order_fixtures"]),
    "row_fold_adjacent_pairs": (
        [(FOLD + "    return p[0];\n}\n\n/* RMSNorm(x)", ADJ + "    return p[0];\n}\n\n/* RMSNorm(x)")],
        ["test_row_sum_squares_stated_order_fixtures"]),
    "rmsnorm_eps_outside_sqrt": (
        [("float r = sqrtf(ms + eps_n);", "float r = sqrtf(ms) + eps_n;")],
        ["test_row_sum_squares_stated_order_fixtures", "test_rmsnorm_exact_given_sum"]),
    "rmsnorm_reciprocal_of_r": (
        [("float v = x[k] / r;", "float v = x[k] * (1.0f / r);")],
        ["test_rmsnorm_exact_given_sum"]),
    "rmsnorm_gain_first": (
        [("xn[k] = g ? v * g[k] : v;", "xn[k] = g ? (x[k] * g[k]) / r : v;")],
        ["test_rmsnorm_exact_given_sum"]),
    # --- activation quantization ("the bytes") ------------------------------
    "act_scale_times_reciprocal_127": (
        [("float a_over = a / 127.0f;", "float a_over = a * (1.0f / 127.0f);")],
        ["test_act_scale_divides_by_127"]),
    "act_reciprocal_of_s": (
        [("float q = x[k] / s;", "float q = x[k] * (1.0f / s);")],
        ["test_act_quant_true_division_cases"]),
    "act_round_half_away": (
        [("        float q = x[k] / s;\n        float r = rintf(q);",
          "        float q = x[k] / s;\n        float r = roundf(q);")],
        ["test_act_quant_golden_ties", "test_act_quant_true_division_cases"]),
    # (A clip at -128 instead of -127 is not listed: s >= max|x|/127 keeps
    # every |x/s| below 127.5, so the clip never engages for finite inputs
    # and such a build computes the same bits.)
    # --- ternary quantization ("the bytes") ---------------------------------
    "tern_reciprocal_of_beta": (
        [("float q = W[r * ldw + k] / beta;", "float q = W[r * ldw + k] * (1.0f / beta);")],
        ["test_ternary_true_division_cases"]),
    "tern_round_half_away": (
        [("            float t = rintf(q);", "            float t = roundf(q);")],
        ["test_ternary_golden_ties", "test_ternary_true_division_cases"]),
    # --- the rescale ("autograd on a byte-graph") ---------------------------
    "epilogue_acc_times_s_first": (
        [("float v = (float)acc[m * ldacc + n] * scale;",
          "float v = ((float)acc[m * ldacc + n] * s[m]) * beta;")],
        ["test_epilogue_grouping_cases"]),
    "epilogue_acc_times_beta_first": (
        [("float v = (float)acc[m * ldacc + n] * scale;",
          "float v = ((float)acc[m * ldacc + n] * beta) * s[m];")],
        ["test_epilogue_grouping_cases"]),
    "epilogue_bias_fused_multiply_add": (
        [("            float v = (float)acc[m * ldacc + n] * scale;\n"
          "            if (b)\n                v = v + b[n];",
          "            float v = (float)acc[m * ldacc + n] * scale;\n"
          "            if (b)\n                v = fmaf((float)acc[m * ldacc + n], scale, b[n]);")],
        ["test_epilogue_bias_cases"]),
    "epilogue_bias_before_rescale": (
        [("            float v = (float)acc[m * ldacc + n] * scale;\n"
          "            if (b)\n                v = v + b[n];",
          "            float v = (float)acc[m * ldacc + n] * scale;\n"
          "            if (b)\n                v = ((float)acc[m * ldacc + n] + b[n]) * scale;")],
        ["test_epilogue_bias_cases"]),
    # --- causal attention over the K/V cache ("attention, as graph ops") ----
    "attention_no_root_dh_scale": (
        [("                sc[j] = dot / root;", "                sc[j] = dot;")],
        ["test_attention_two_keys_closed_form_with_root_dh_scale"]),
    "attention_scale_by_dh": (
        [("    double root = sqrt((double)dh);", "    double root = (double)dh;")],
        ["test_attention_two_keys_closed_form_with_root_dh_scale"]),
    "attention_mask_drops_own_position": (
        [("            int64_t n = pos0 + m + 1; /* keys 0 .. pos0 + m */",
          "            int64_t n = pos0 + m; /* keys 0 .. pos0 + m */")],
        ["test_attention_single_key_returns_its_value", "test_attention_is_causal"]),
    "attention_mask_sees_next_position": (
        [("            int64_t n = pos0 + m + 1; /* keys 0 .. pos0 + m */",
          "            int64_t n = pos0 + m + 2; /* keys 0 .. pos0 + m */")],
        ["test_attention_single_key_returns_its_value", "test_attention_is_causal"]),
    "attention_value_columns_of_head_0": (
        [("                    o += sc[j] * (double)vc[j * ldv + h * dh + d];",
          "                    o += sc[j] * (double)vc[j * ldv + d];")],
        ["test_attention_heads_are_independent"]),
    "attention_unnormalized": (
        [("                out[m * ldo + h * dh + d] = (float)(o / sum);",
          "                out[m * ldo + h * dh + d] = (float)o;")],
        ["test_attention_equal_keys_average_the_values"]),
    # --- top-k sampling ("a 1-bit llm, from scratch") ----------------------
    "sampler_ties_to_higher_index": (
        [("    return (x->i > y->i) - (x->i < y->i);", "    return (x->i < y->i) - (x->i > y->i);")],
        ["test_k1_is_argmax", "test_ranking_matches_a_stable_sort"]),
    "sampler_temperature_multiplied": (
        [("            run += exp(((double)e[r].v - (double)e[0].v) / (double)temp);",
          "            run += exp(((double)e[r].v - (double)e[0].v) * (double)temp);")],
        ["test_two_kept_logits_with_temperature"]),
    "sampler_smallest_first": (
        [("    if (x->v > y->v)\n        return -1;\n    if (x->v < y->v)\n        return 1;",
          "    if (x->v < y->v)\n        return -1;\n    if (x->v > y->v)\n        return 1;")],
        ["test_k1_is_argmax"]),
    "sampler_cdf_from_the_bottom_rank": (
        [("            run += exp(((double)e[r].v - (double)e[0].v) / (double)temp);",
          "            run += exp(((double)e[k - 1 - r].v - (double)e[0].v) / (double)temp);")],
        ["test_sampling_frequencies_follow_the_softmax", "test_two_kept_logits_with_temperature"]),
    # --- the straight-through backward ("autograd on a byte-graph") ---------
    "backward_dx_drops_last_output": (
        [("            for (int64_t n = 0; n < N; ++n) {\n                double gv = g[m * ldg + n];\n"
          "                for (int64_t k = 0; k < K; ++k)\n"
          "                    row[k] += gv * (double)W[n * ldw + k];",
          "            for (int64_t n = 0; n + 1 < N; ++n) {\n                double gv = g[m * ldg + n];\n"
          "                for (int64_t k = 0; k < K; ++k)\n"
          "                    row[k] += gv * (double)W[n * ldw + k];")],
        ["test_finite_differences_of_the_unquantized_layer", "test_one_hot_upstream_gradient"]),
    "backward_dW_first_input_row_only": (
        [("                    row[k] += gv * (double)x[m * ldx + k];",
          "                    row[k] += gv * (double)x[k];")],
        ["test_finite_differences_of_the_unquantized_layer", "test_one_hot_upstream_gradient"]),
    "backward_dx_sign": (
        [("                    row[k] += gv * (double)W[n * ldw + k];",
          "                    row[k] -= gv * (double)W[n * ldw + k];")],
        ["test_finite_differences_of_the_unquantized_layer"]),
    "backward_db_skips_first_row": (
        [("            for (int64_t m = 0; m < M; ++m)\n                s += (double)g[m * ldg + n];",
          "            for (int64_t m = 1; m < M; ++m)\n                s += (double)g[m * ldg + n];")],
        ["test_finite_differences_of_the_unquantized_layer", "test_one_hot_upstream_gradient"]),
    # --- five trits per byte (README "A whole ternary GPT") -----------------
    "pack_digits_reversed": (
        [("                int pow3 = 1;\n                for (int j = 0; j < 5; ++j) {",
          "                int pow3 = 81;\n                for (int j = 0; j < 5; ++j) {"),
         ("                    code += t * pow3;\n                    pow3 *= 3;",
          "                    code += t * pow3;\n                    pow3 /= 3;")],
        ["test_pack_golden_codes"]),
    "pack_pad_byte_zero": (
        [("            int code = 121;\n            if (g < groups) {",
          "            int code = g < groups ? 121 : 0;\n            if (g < groups) {")],
        ["test_pack_tail_padding_and_bad_entries"]),
    # --- the integer matmul -------------------------------------------------
    "matmul_drops_last_k": (
        [("            for (int64_t k = 0; k < K; ++k)\n"
          "                sum += (int64_t)xq[m * ldx + k] * (int64_t)wq[n * ldw + k];",
          "            for (int64_t k = 0; k + 1 < K; ++k)\n"
          "                sum += (int64_t)xq[m * ldx + k] * (int64_t)wq[n * ldw + k];")],
        ["test_matmul_brute_force_tiny", "test_matmul_special_cases"]),
}


def _pin(name):
    for mod in (pins, attn_pins, sampler_pins, backward_pins):
        if hasattr(mod, name):
            return getattr(mod, name)
    raise AttributeError(name)


def _compile(text, out):
    src = out + ".c"
    with open(src, "w") as f:
        f.write(text)
    cmd = ["gcc", *obuild.CFLAGS, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True)
    return out


def _mutate(text, subs):
    for old, new in subs:
        assert text.count(old) == 1, "substitution target not unique or missing: %r" % old[:60]
        text = text.replace(old, new)
    return text


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    subs, catchers = MUTANTS[name]
    with open(SRC) as f:
        text = f.read()
    lib = _compile(_mutate(text, subs), str(tmp_path / ("libugref_%s.so" % name)))
    failed = []
    with oracle.use_library(lib):
        for pin in catchers:
            try:
                _pin(pin)()
            except AssertionError:
                failed.append(pin)
    assert failed, "no pin caught the planted slip %s" % name


def test_unmutated_copy_passes_the_same_pins(tmp_path):
    """Control: the same compile-and-swap route with no substitution passes
    every pin the mutants are checked against."""
    with open(SRC) as f:
        text = f.read()
    lib = _compile(text, str(tmp_path / "libugref_copy.so"))
    used = sorted({p for _, cs in MUTANTS.values() for p in cs})
    with oracle.use_library(lib):
        for pin in used:
            _pin(pin)()
