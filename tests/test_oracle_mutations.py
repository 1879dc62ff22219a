"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a private copy of the oracle source (string
substitution on the C text), compiles it with gcc into a temporary directory,
swaps it in for the real oracle and runs a group of pins from
test_oracle_pins.py.  At least one pin must fail for every planted mistake.
Nothing here touches the committed oracle or any GPU code.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
import test_oracle_pins as pins
import test_accept_oracle as accept_pins
import test_tree_oracle as tree_pins
import test_neighbour_oracle as nb_pins
import workloads

wl_theta = workloads.ROPE_THETA

SRC = os.path.join(os.path.dirname(oracle.__file__), "ddtv_oracle.c")
SRC_TREE = os.path.join(os.path.dirname(oracle.__file__), "ddtv_tree_oracle.c")
SRC_ACCEPT = os.path.join(os.path.dirname(oracle.__file__), "ddtv_accept_oracle.c")
SRC_NEIGHBOUR = os.path.join(os.path.dirname(oracle.__file__), "ddtv_neighbour_oracle.c")

# (id, original text, mutated text)
MUTATIONS = [
    ("drop_rope_term", "rope += (double)qr[t] *", "rope += 0.0 * (double)qr[t] *"),
    ("rope_sign", "return scale * (nope + rope);", "return scale * (nope - rope);"),
    ("no_scale", "return scale * (nope + rope);", "return (nope + rope);"),
    ("transposed_value_index",
     "out[d] += s[j] * kv_value(ckv, kv_dtype, row * D_LAT + d);",
     "out[d] += s[j] * kv_value(ckv, kv_dtype, row * D_LAT + (d ^ 1));"),
    ("value_from_next_row",
     "out[d] += s[j] * kv_value(ckv, kv_dtype, row * D_LAT + d);",
     "out[d] += s[j] * kv_value(ckv, kv_dtype, (row > 0 ? row - 1 : row) * D_LAT + d);"),
    ("kv_offset_ignores_tree_rows", "off += (int64_t)prefix[i] + Q;", "off += (int64_t)prefix[i];"),
    ("prefix_off_by_one", "if (j < P) return 1;", "if (j <= P) return 1;"),
    ("walk_skips_root", "cur = par[cur];\n", "cur = par[cur];\n                if (cur == 0) break;\n"),
    ("walk_skips_self", "row[cur / 32] |= 1u << (cur % 32);",
     "if (cur != i) row[cur / 32] |= 1u << (cur % 32);"),
    ("bits_msb_first", "row[cur / 32] |= 1u << (cur % 32);", "row[cur / 32] |= 1u << (31 - cur % 32);"),
    ("lse_drops_max", "*lse = m + log(l);", "*lse = log(l);"),
    ("no_normalise", "for (int d = 0; d < D_LAT; ++d) out[d] /= l;", ""),
    ("merge_ignores_rescale", "L += w * l[s];", "L += l[s];"),
    ("head_index_swapped", "int h = (int)(r % H);\n        int q = (int)((r / H) % Q);",
     "int q = (int)(r % Q);\n        int h = (int)((r / Q) % H);"),
    ("bf16_misread", "uint32_t u = ((uint32_t)h) << 16;", "uint32_t u = ((uint32_t)h) << 15;"),
    ("accept_root_with_parent", "if (i == 0) return par[0] == -1;", "if (i == 0) return 1;"),
    ("fp8_bias_off_by_one", "else v = ldexp(1.0 + m / 8.0, e - 7);", "else v = ldexp(1.0 + m / 8.0, e - 8);"),
    ("fp8_subnormal_scale", "if (e == 0) v = ldexp((double)m, -9);", "if (e == 0) v = ldexp((double)m, -10);"),
    ("fp8_read_as_bf16", "if (kv_dtype == 2) return ddtvref_fp8_value(((const uint8_t *)base)[idx]);", ""),
]

PINS = [
    pins.test_closed_form_latent_scores,
    pins.test_closed_form_rope_scores_value_excludes_rope,
    pins.test_bf16_widening_exact,
    lambda: pins.test_chain_equals_causal(0),
    lambda: pins.test_chain_equals_causal(1),
    pins.test_single_query_equals_dense,
    pins.test_single_bit_mask_exact,
    lambda: pins.test_small_configs_match_torch("c2"),
    lambda: pins.test_bruteforce_masks(5),
    lambda: pins.test_lse_merge_identity(0),
    pins.test_invalid_trees_reported,
    pins.test_scale_zero_is_mean,
    pins.test_fp8_decode_every_code,
    pins.test_fp8_cache_matches_torch,
]


# Mistakes planted in the best-first tree builder's oracle.
TREE_MUTATIONS = [
    ("child_reads_wrong_depth", "float s = c.score + logp[c.depth * K + k];",
     "float s = c.score + logp[(c.depth > 0 ? c.depth - 1 : 0) * K + k];"),
    ("worst_first", "if (a->score != b->score) return a->score > b->score;",
     "if (a->score != b->score) return a->score < b->score;"),
    ("ties_later_parent_first", "if (a->parent != b->parent) return a->parent < b->parent;",
     "if (a->parent != b->parent) return a->parent > b->parent;"),
    ("ties_worse_rank_first", "return a->rank < b->rank;", "return a->rank > b->rank;"),
    ("choices_skip_last", "for (int k = 0; k < K; ++k) {\n                float s",
     "for (int k = 0; k < K - 1; ++k) {\n                float s"),
    ("depth_cap_one_short", "if (c.depth < D) {", "if (c.depth < D - 1) {"),
    ("child_parented_to_grandparent", "Cand ch = {s, i, c.depth + 1, rank_of[c.depth * K + k], k};",
     "Cand ch = {s, c.parent < 0 ? i : c.parent, c.depth + 1, rank_of[c.depth * K + k], k};"),
    ("rank_is_position", "Cand ch = {s, i, c.depth + 1, rank_of[c.depth * K + k], k};",
     "Cand ch = {s, i, c.depth + 1, k, k};"),
    ("ranking_ascending", "if (a->v != b->v) return a->v > b->v ? -1 : 1;",
     "if (a->v != b->v) return a->v < b->v ? -1 : 1;"),
    ("equal_values_later_index_first", "return a->k < b->k ? -1 : (a->k > b->k ? 1 : 0);",
     "return a->k > b->k ? -1 : (a->k < b->k ? 1 : 0);"),
    ("token_by_rank", "tokens[(c.depth - 1) * K + c.choice]", "tokens[(c.depth - 1) * K + c.rank]"),
]

# Mistakes planted in the tree-accept / compaction oracle.
ACCEPT_MUTATIONS = [
    ("argmax_last_on_ties", "if (row[v] > row[best]) best = v;", "if (row[v] >= row[best]) best = v;"),
    ("walk_uses_child_prediction", "if (parent[c] == cur && token[c] == pred[cur]) {",
     "if (parent[c] == cur && token[c] == pred[c]) {"),
    ("last_matching_child", "                next = c;\n                break;", "                next = c;"),
    ("bonus_from_root", "out_tokens[k] = pred[cur];", "out_tokens[k] = pred[0];"),
    ("no_bonus", "out_tokens[k] = pred[cur];", ""),
    ("compaction_off_by_one", "memcpy(dst + (int64_t)(prefix + j) * row_bytes", "memcpy(dst + (int64_t)(prefix + j - 1) * row_bytes"),
    ("compaction_moves_root", "for (int32_t j = 1; j <= k; ++j)", "for (int32_t j = 0; j < k; ++j)"),
]

ACCEPT_PINS = [
    lambda: accept_pins.test_walk_equals_matching_edge_set(1, 6, 32),
    lambda: accept_pins.test_walk_equals_matching_edge_set(2, 4, 128),
    accept_pins.test_special_cases,
    lambda: accept_pins.test_compaction_equals_fancy_indexing(np.float32),
]

# Mistakes planted in the oracle of the steps around the attention.
NEIGHBOUR_MUTATIONS = [
    ("rope_interleaved_pairs", "double x0 = (double)x[i], x1 = (double)x[i + N_HALF];",
     "double x0 = (double)x[2 * i], x1 = (double)x[2 * i + 1];"),
    ("rope_sign", "y[i] = x0 * c - x1 * s;", "y[i] = x0 * c + x1 * s;"),
    ("rope_frequency_exponent", "-(double)(2 * i) / (double)N_ROPE", "-(double)(i) / (double)N_ROPE"),
    ("rope_reads_nope_part", "const float *pe = nope + d_nope;", "const float *pe = nope;"),
    ("absorb_head_and_row_swapped", "w_kc[(h * d_nope + k) * N_LAT + c]", "w_kc[(k * H + h) * N_LAT + c]"),
    ("absorb_drops_last_term", "for (int k = 0; k < d_nope; ++k)", "for (int k = 0; k < d_nope - 1; ++k)"),
    ("value_wrong_head", "const float *w = w_vc + (h * d_v + n) * N_LAT;",
     "const float *w = w_vc + (((h + 1) % H) * d_v + n) * N_LAT;"),
    ("value_column_shift", "acc += (double)x[c] * (double)w[c];", "acc += (double)x[c] * (double)w[c ^ 1];"),
    ("position_ignores_prefix", "pos[(int64_t)b * Q + i] = prefix[b] + d;", "pos[(int64_t)b * Q + i] = d;"),
    ("position_counts_root", "int32_t d = 0;", "int32_t d = 1;"),
    ("append_key_unrotated", "ddtvref_rope_neox(k_pe + node * N_ROPE, pos[node], theta, k_rope + r * N_ROPE);",
     "ddtvref_rope_neox(k_pe + node * N_ROPE, 0, theta, k_rope + r * N_ROPE);"),
    ("append_row_ignores_prefix", "int64_t r = off + prefix[b] + i;", "int64_t r = off + i;"),
]

NEIGHBOUR_PINS = [
    lambda: nb_pins.test_rope_is_complex_rotation(wl_theta),
    nb_pins.test_rope_unit_vectors_closed_form,
    nb_pins.test_rope_identity_norms_and_relative_positions,
    nb_pins.test_absorb_equals_unabsorbed_key_and_rope_part,
    nb_pins.test_absorb_one_hot_picks_weight_rows,
    nb_pins.test_value_projection_matmul_and_one_hot,
    nb_pins.test_tree_positions,
    nb_pins.test_append_kv_rows,
    lambda: nb_pins.test_chain_equals_unabsorbed_attention(128, 128),
]

TREE_PINS = [
    lambda: tree_pins.test_bruteforce_top_scores(3, 3, 20),
    lambda: tree_pins.test_bruteforce_top_scores(5, 3, 60),
    lambda: tree_pins.test_bruteforce_top_scores_unsorted(3, 3, 20),
    lambda: tree_pins.test_shuffled_choices_change_nothing(0),
    tree_pins.test_equal_values_rank_by_index,
    tree_pins.test_positive_log_prob_worked_example,
    tree_pins.test_tree_invariants,
    tree_pins.test_k1_is_a_chain_and_d1_is_a_star,
    tree_pins.test_ties_go_to_the_earlier_parent_then_rank,
]


def _run_mutation(tmp_path, target, mid, old, new, pins_to_run):
    """Compile the oracle with one planted mistake in `target`; return the pins that fail."""
    src = open(target).read()
    assert src.count(old) >= 1, f"mutation anchor for {mid} not found"
    mutated = src.replace(old, new, 1)
    c = tmp_path / ("mut_" + os.path.basename(target))
    so = tmp_path / "libmut.so"
    c.write_text(mutated)
    sources = [str(c) if f == target else f for f in (SRC, SRC_TREE, SRC_ACCEPT, SRC_NEIGHBOUR)]
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", str(so), *sources, "-lm"])
    lib = oracle.configure(ctypes.CDLL(str(so)))
    saved = oracle._lib
    oracle._lib = lib
    failed = []
    try:
        for pin in pins_to_run:
            try:
                pin()
            except (AssertionError, ValueError):
                failed.append(getattr(pin, "__name__", "lambda"))
    finally:
        oracle._lib = saved
    return failed


@pytest.mark.parametrize("mid,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(tmp_path, mid, old, new):
    failed = _run_mutation(tmp_path, SRC, mid, old, new, PINS)
    assert failed, f"no pin caught mutation {mid}"


@pytest.mark.parametrize("mid,old,new", TREE_MUTATIONS, ids=[m[0] for m in TREE_MUTATIONS])
def test_tree_pins_catch_mutation(tmp_path, mid, old, new):
    failed = _run_mutation(tmp_path, SRC_TREE, mid, old, new, TREE_PINS)
    assert failed, f"no pin caught mutation {mid}"



@pytest.mark.parametrize("mid,old,new", ACCEPT_MUTATIONS, ids=[m[0] for m in ACCEPT_MUTATIONS])
def test_accept_pins_catch_mutation(tmp_path, mid, old, new):
    failed = _run_mutation(tmp_path, SRC_ACCEPT, mid, old, new, ACCEPT_PINS)
    assert failed, f"no pin caught mutation {mid}"


@pytest.mark.parametrize("mid,old,new", NEIGHBOUR_MUTATIONS, ids=[m[0] for m in NEIGHBOUR_MUTATIONS])
def test_neighbour_pins_catch_mutation(tmp_path, mid, old, new):
    failed = _run_mutation(tmp_path, SRC_NEIGHBOUR, mid, old, new, NEIGHBOUR_PINS)
    assert failed, f"no pin caught mutation {mid}"
