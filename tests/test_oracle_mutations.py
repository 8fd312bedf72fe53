"""The pins reject an oracle with a planted mistake.

Each case copies ep_oracle.c, applies one plausible slip (a wrong index, an
inclusive instead of exclusive scan, a dropped term, truncation instead of
round-to-nearest-even, ...), builds it with gcc into a temporary library and
runs the pin tests against that build.  At least one pin must fail.  This
runs on the CPU only.
"""
import json
import os
import subprocess

import numpy as np
import pytest

import oracle
import test_oracle_fp8 as fp8pins
import test_oracle_hier as hierpins
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "ep_oracle.c")

MUTATIONS = {
    "rank_of_expert_modulo": ("valid_expert(e, E) && e / L == r", "valid_expert(e, E) && e % R == r"),
    "inclusive_offset_scan": (
        "expert_offset[e] = (int32_t)run;\n            run += align_up(expert_count[e], A);",
        "run += align_up(expert_count[e], A);\n            expert_offset[e] = (int32_t)run;"),
    "alignment_dropped": ("run += align_up(expert_count[e], A);", "run += expert_count[e];"),
    "cursor_not_advanced": ("cursor[e] += 1;", ""),
    "slice_base_from_local": ("(int64_t)(e / L) * S + off", "(int64_t)(e % L) * S + off"),
    "capacity_off_by_one": ("off < S ?", "off <= S ?"),
    "weights_reversed": ("(double)topk_weights[t * K + j]", "(double)topk_weights[t * K + (K - 1 - j)]"),
    "round_by_truncation": ("rint(ldexp(a, -qexp))", "floor(ldexp(a, -qexp))"),
    "one_bit_too_many": ("int qexp = e - 8;", "int qexp = e - 9;"),
    "src_index_is_topk_pos": (
        "memcpy(recv_x + s * H, x + t * H, (size_t)H * sizeof(uint16_t));\n            if (recv_src_token) recv_src_token[s] = (int32_t)t;",
        "memcpy(recv_x + s * H, x + t * H, (size_t)H * sizeof(uint16_t));\n            if (recv_src_token) recv_src_token[s] = (int32_t)j;"),
    "group_range_shifted": ("for (int32_t r = g * ranks_per_group; r < (g + 1) * ranks_per_group; ++r)",
                            "for (int32_t r = g; r < g + ranks_per_group; ++r)"),
    "empty_id_counted_bad": ("if (e == -1) continue;", ""),
    "row_sum_uses_aligned": ("rows += expert_count[e];", "rows += align_up(expert_count[e], A);"),
    "e4m3_ties_away": ("((lo & 1) == 0 ? lo : hi)", "hi"),
    "fp8_scale_constant": ("const float inv = amax > 0.0f ? 448.0f / amax : 0.0f;",
                           "const float inv = amax > 0.0f ? 240.0f / amax : 0.0f;"),
    "fp8_scale_inverted": ("sf[t * nb + b] = amax / 448.0f;", "sf[t * nb + b] = 448.0f / amax;"),
    "group_slot_off_by_one": ("group_slot[t * G + g] = pos < SG ? (int32_t)(g * SG + pos) : -1;",
                              "group_slot[t * G + g] = pos < SG ? (int32_t)(g * SG + pos + 1) : -1;"),
    "slot_group_modulo": ("return (int32_t)((s / S) / (R / G));", "return (int32_t)((s / S) % G);"),
    "partial_folded_in_double": (
        "float acc = 0.0f;\n                for (int32_t j = 0; j < K; ++j) {",
        "double acc = 0.0;\n                for (int32_t j = 0; j < K; ++j) {"
        "\n#define fmaf(a, b, c) fma((double)(a), (double)(b), (c))"),
    "partial_topk_order_reversed": (
        "for (int32_t j = 0; j < K; ++j) {\n                    int64_t s = token_slot[t * K + j];\n"
        "                    if (s < 0 || s >= num_rows || slot_group(s, S, R, G) != g) continue;",
        "for (int32_t j = K - 1; j >= 0; --j) {\n                    int64_t s = token_slot[t * K + j];\n"
        "                    if (s < 0 || s >= num_rows || slot_group(s, S, R, G) != g) continue;"),
    "group_sum_in_float": (
        "double acc = 0.0;\n            for (int32_t g = 0; g < G; ++g) {",
        "float acc = 0.0f;\n            for (int32_t g = 0; g < G; ++g) {"),
    "partials_summed_unrounded": (
        "acc += (double)bf16_to_float(group_buf[gs * H + h]);",
        "{ float pa = 0.0f; for (int32_t j = 0; j < K; ++j) { int64_t s = token_slot[t * K + j]; "
        "if (s < 0 || s >= num_rows || slot_group(s, S, R, G) != g) continue; "
        "pa = fmaf(topk_weights ? topk_weights[t * K + j] : 1.0f, bf16_to_float(y[s * H + h]), pa); } "
        "acc += (double)pa; }"),
    "fp8_scale_strides_swapped": ("recv_sf[s * sf_token_stride + b * sf_hidden_stride]",
                                  "recv_sf[s * sf_hidden_stride + b * sf_token_stride]"),
}


def _pin_suite():
    pins.test_golden_handworked_layout()
    pins.test_golden_handworked_combine()
    pins.test_golden_rounding_ties()
    for seed in range(30):
        pins.test_layout_matches_brute_force(seed)
    pins.test_negative_bad_id_flags_error()
    pins.test_workload_layout_invariants("tiny")
    pins.test_workload_layout_invariants("large16k")
    pins.test_layout_invariants_with_alignment()
    pins.test_dispatch_rows_are_copies("tiny")
    pins.test_unit_weight_combine_is_x_times_k("tiny")
    pins.test_one_hot_combine_returns_x()
    pins.test_weighted_combine_matches_numpy_gather("tiny")
    pins.test_bf16_rounding_matches_torch_on_floats()
    fp8pins.test_e4m3_rounding_matches_torch()
    fp8pins.test_quantize_matches_restatement("tiny")
    fp8pins.test_quantize_zero_block_and_extremes()
    hierpins.test_group_slots("prefill4k", 2)
    hierpins.test_two_level_dispatch_equals_flat("tiny")
    hierpins.test_two_level_combine_one_hot_returns_x()
    for c in json.load(open(hierpins.GOLDEN))["cases"]:
        hierpins.test_golden_handworked_two_level_combine(c["name"])
    # token-major scales: a planted stride mistake then stays inside the buffer
    fp8pins.test_dispatch_fp8_moves_codes_and_scales(False)


def test_unmutated_build_passes(tmp_path):
    lib = tmp_path / "lib_clean.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", str(lib), SRC, "-lm"])
    with oracle.use_library(oracle.open_library(str(lib))):
        _pin_suite()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    before, after = MUTATIONS[name]
    text = open(SRC).read()
    assert text.count(before) == 1, f"mutation anchor for {name} not unique"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(before, after))
    lib = tmp_path / f"lib_{name}.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", str(lib), str(src), "-lm"])
    with oracle.use_library(oracle.open_library(str(lib))):
        with pytest.raises(AssertionError):
            np.seterr(all="ignore")
            _pin_suite()
