"""Planted mistakes: each mutant is a copy of oracle.c with one plausible error (a dropped
term, a wrong sign, a wrong index, a transposed operand...).  Built on the CPU into a
temporary directory and run against the pins, every mutant must fail at least one pin.
This shows the pins constrain every function of the oracle, not just that it agrees with
itself."""
import os
import shutil
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "causal_drops_diagonal": ("int n = causal ? i + 1 : N;", "int n = causal ? i : N;"),
    "online_skips_rescale": ("for (int c = 0; c < dv; ++c) acc[c] *= corr;",
                             "for (int c = 0; c < dv; ++c) acc[c] *= 1.0;"),
    "lse_wrong_sign": ("*lse = m + log(l);", "*lse = m - log(l);"),
    "gqa_wrong_head_map": ("int kvh = h / group;\n                const uint16_t* kbase",
                           "int kvh = h % Hkv;\n                const uint16_t* kbase"),
    "k_and_v_swapped": ("kr[j] = kbase + (int64_t)j * d;\n                    vr[j] = vbase",
                        "kr[j] = vbase + (int64_t)j * d;\n                    vr[j] = kbase"),
    "scale_dropped": ("        s[j] = scale * acc;\n    }", "        s[j] = acc;\n    }"),
    "merge_weight_inverted": ("double w = exp(lse_s[s] - M);", "double w = exp(M - lse_s[s]);"),
    "decode_wrong_slot": ("int slot = tok % page_size;", "int slot = (tok + 1) % page_size;"),
    "fp16_wrong_bias": ("expo - 25);", "expo - 24);"),
    "online_l_not_rescaled": ("l = l * corr + rowsum;", "l = l + rowsum;"),
    "softmax_not_normalised": ("s[j] = s[j] / l;   /* P_ij */", "s[j] = s[j];"),
    "cascade_prefix_other_head": ("int64_t off = ((int64_t)kvh * prefix_len + tok) * d;",
                                  "int64_t off = ((int64_t)((kvh + 1) % Hkv) * prefix_len + tok) * d;"),
    "cascade_drops_prefix": ("for (int tok = 0; tok < prefix_len; ++tok, ++n) {",
                             "for (int tok = 0; tok < 0; ++tok, ++n) {"),
    "cascade_own_tokens_wrong_slot": ("int in_page = tok % page_size;", "int in_page = (tok + 3) % page_size;"),
    "paged_prefill_top_left_mask": ("int last = kv_len - q_len + i;", "int last = i;"),
    "paged_prefill_row_not_rebased": ("int i = tok - cu_seqlens_q[r];", "int i = tok;"),
    "paged_prefill_wrong_kv_slot": ("int in_page = key % page_size;",
                                    "int in_page = (key + 1) % page_size;"),
    "window_one_key_too_many": ("int lo = window > 0 && i - window + 1 > 0 ? i - window + 1 : 0;",
                                "int lo = window > 0 && i - window > 0 ? i - window : 0;"),
    "softcap_without_inner_division": ("if (softcap > 0.0) s[j] = softcap * tanh(s[j] / softcap);",
                                       "if (softcap > 0.0) s[j] = softcap * tanh(s[j]);"),
    "softcap_before_scale": ("s[j] = scale * acc;\n                if (softcap > 0.0) s[j] = softcap * tanh(s[j] / softcap);",
                             "s[j] = acc;\n                if (softcap > 0.0) s[j] = softcap * tanh(s[j] / softcap);\n                s[j] *= scale;"),
}

PINS = [
    lambda: pins.test_widen16_matches_numpy_for_every_pattern(pins.FP16),
    pins.test_single_visible_key_returns_v_bits_exactly,
    pins.test_three_scores_two_tiles_zwjcode_section04,
    pins.test_rechunk_lse_and_weights_llm_internals_10_3_2,
    pins.test_element_stream_cs349d_exercise1,
    pins.test_split_merge_max_refresh_handbook_exercise1,
    lambda: pins.test_attention_matches_torch_sdpa_float64(2, 4, 2, 37, 16, True, pins.BF16),
    lambda: pins.test_attention_matches_torch_sdpa_float64(1, 3, 1, 50, 8, True, pins.FP16),
    pins.test_scale_is_applied_to_scores_not_values,
    lambda: pins.test_tiled_online_equals_library_softmax(257, 16),
    lambda: pins.test_merge_is_order_free(8),
    pins.test_bsr_example_paged_equals_contiguous_exactly,
    pins.test_decode_matches_torch_sdpa_and_is_page_order_free,
    pins.test_cascade_matches_torch_sdpa_over_prefix_then_own_tokens,
    lambda: pins.test_paged_prefill_matches_torch_sdpa_bottom_right(True),
    lambda: pins.test_sliding_window_matches_torch_sdpa_with_its_own_mask(5, pins.BF16),
    pins.test_softcap_tends_to_plain_attention_as_the_cap_grows,
    pins.test_softcap_bounds_the_weight_ratio_and_follows_the_scale,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                    str(mut), "-o", str(lib), "-lm"], check=True)
    failed = []
    oracle.use_library(str(lib))
    try:
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError):
                failed.append(pin)
    finally:
        oracle.use_library(None)
    assert failed, f"mutant {name} passed every pin"
