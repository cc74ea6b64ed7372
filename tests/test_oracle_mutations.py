"""Mutation check of the oracle's pins, entirely on the CPU.

Each case compiles a copy of oracle.c with one plausible mistake planted
(a dropped term, a wrong sign or index, an off-by-one window, a transposed
head mapping) and runs the pins of test_oracle_pins against it.  At least
one pin must fail for every planted mistake; the real oracle passes them all.
"""
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "oracle.c")
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

MUTATIONS = {
    "window_holds_w_plus_1_keys": ("dist % dilation == 0 && dist / dilation < window",
                                   "dist % dilation == 0 && dist / dilation <= window"),
    "stride_relative_to_query": ("stride > 0 && j <= i && j % stride == 0", "stride > 0 && j <= i && (i - j) % stride == 0"),
    "stride_ignores_causality": ("stride > 0 && j <= i && j % stride == 0", "stride > 0 && j % stride == 0"),
    "dilation_ignored": ("dist >= 0 && dist % dilation == 0 && dist / dilation < window",
                         "dist >= 0 && dist < window"),
    "dilation_span_not_stretched": ("dist >= 0 && dist % dilation == 0 && dist / dilation < window",
                                    "dist >= 0 && dist % dilation == 0 && dist < window"),
    "global_columns_dropped": ("(j < n_global || i < n_global)", "(i < n_global)"),
    "global_ignores_causality": ("n_global > 0 && j <= i && (", "n_global > 0 && ("),
    "tile_band_not_stretched_by_dilation": ("band += (j <= i && i - j <= span);",
                                            "band += (j <= i && i - j < window);"),
    "prefix_keys_miss_globals": ("prefix_keys[qt] += (j < n_global || (stride > 0 && j % stride == 0));",
                                 "prefix_keys[qt] += (stride > 0 && j % stride == 0);"),
    "gqa_interleaved_heads": ("h = bh % Hq, b = bh / Hq, g = h / G;\n        for (int64_t j = 0; j < N; ++j)\n            mrow[j] = (uint8_t)orc_allowed(i, j, N, window, stride, dilation, n_global);\n        const float *qi",
                              "h = bh % Hq, b = bh / Hq, g = h % Hkv;\n        for (int64_t j = 0; j < N; ++j)\n            mrow[j] = (uint8_t)orc_allowed(i, j, N, window, stride, dilation, n_global);\n        const float *qi"),
    "scale_dropped": ("s[j] = scale * acc;", "s[j] = acc;"),
    "no_max_subtraction": ("s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
    "value_transposed": ("out[c] += w * (double)V[j * v_stride + c];", "out[c] += w * (double)V[c * v_stride + j];"),
    "tiled_no_rescale_of_sum": ("        l *= alpha;\n", "\n"),
    "diff_sign_flipped": ("double w = w1[j] - lambda * w2[j];", "double w = w1[j] + lambda * w2[j];"),
    "decode_slot_off_by_one": ("int64_t slot = p % window;", "int64_t slot = (p + 1) % window;"),
    "decode_window_one_short": ("int64_t first = L - window > 0 ? L - window : 0;", "int64_t first = L - window + 1 > 0 ? L - window + 1 : 0;"),
    "tile_kind_full_never": ("else if (c == (i1 - i0) * (j1 - j0))", "else if (c == (i1 - i0) * (j1 - j0) + 1)"),
    "nsa_branch_dropped": ("return n / l + k * l + w;", "return n / l + k * l;"),
    "lse_without_max": ("return l > 0.0 ? m + log(l) : -INFINITY;", "return l > 0.0 ? log(l) : -INFINITY;"),
    "kv_cache_keys_only": ("return 2 * per_tensor;   /* K and V */", "return per_tensor;"),
    "kv_cache_layers_dropped": ("const int64_t per_tensor = n * n_layers * n_heads_kv * d_head * dtype_bytes;",
                                "const int64_t per_tensor = n * n_heads_kv * d_head * dtype_bytes;"),
}


def all_pins():
    """(name, callable) for every pin, with fixed parameters."""
    out = [
        ("masks_8x8", lambda: pins.test_masks_match_hand_drawn_8x8(GOLDEN)),
        ("counts_8x8", pins.test_8x8_counts),
        ("band_closed", lambda: pins.test_band_count_closed_form(33)),
        ("local_stride_closed", pins.test_local_stride_closed_form),
        ("tile_hand", lambda: pins.test_tile_list_hand_worked(GOLDEN)),
        ("tile_blocks", lambda: pins.test_tile_list_against_block_sums(64, 16, 7, 16, 8, 1, 0)),
        ("tile_blocks_full", lambda: pins.test_tile_list_against_block_sums(50, 50, 0, 16, 16, 1, 0)),
        ("tile_blocks_dil_global", lambda: pins.test_tile_list_against_block_sums(70, 5, 4, 16, 8, 2, 11)),
        ("tile_blocks_dilated", lambda: pins.test_tile_list_against_block_sums(90, 6, 5, 8, 8, 8, 0)),
        ("tile_blocks_global_rows", lambda: pins.test_tile_list_against_block_sums(90, 7, 9, 8, 8, 1, 20)),
        ("dilated_counts", pins.test_dilated_row_counts_closed_form),
        ("dilated_residues", lambda: pins.test_dilated_window_is_plain_window_on_residue_classes(30, 4, 3)),
        ("global_gather", lambda: pins.test_global_tokens_by_key_gather(30, 5, 9, 0)),
        ("global_counts", pins.test_global_count_closed_form),
        ("global_vs_sinks", lambda: pins.test_global_prefill_row_is_sink_decode(40, 8, 4)),
        ("attn_sdpa", lambda: pins.test_attention_matches_sdpa_with_pinned_mask(2, 4, 2, 33, 16, 8, 5, 4)),
        ("causal_sdpa", lambda: pins.test_window_ge_n_reduces_to_causal_sdpa(17, 17)),
        ("peaky", pins.test_peaky_scores_need_max_subtraction),
        ("w1", pins.test_window_one_returns_own_value),
        ("tiled", lambda: pins.test_tiled_softmax_equals_direct(30, 7)),
        ("diff", pins.test_diff_matches_two_sdpa_maps),
        ("decode", lambda: pins.test_decode_is_last_row_of_window_attention(30, 8)),
        ("decode_partial_ring", lambda: pins.test_decode_is_last_row_of_window_attention(5, 8)),
        ("sinks", lambda: pins.test_decode_with_sinks(40, 8, 4)),
        ("nsa", pins.test_nsa_key_count_printed_value),
        ("kv_worked", pins.test_kv_cache_bytes_worked_example),
        ("kv_rolling", pins.test_kv_cache_bytes_rolling_window_and_sinks),
    ]
    return out


def failing_pins():
    bad = []
    for name, fn in all_pins():
        try:
            fn()
        except AssertionError:
            bad.append(name)
    return bad


def test_real_oracle_passes_every_pin():
    assert failing_pins() == []


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistake_is_caught(mutation, tmp_path):
    old, new = MUTATIONS[mutation]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor must match exactly once"
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", str(mutated), "-o", str(lib), "-lm"],
                   check=True)
    with oracle.using_library(str(lib)):
        bad = failing_pins()
    assert bad, f"no pin catches {mutation}"
