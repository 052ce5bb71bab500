"""The oracle's pins catch plausible mistakes in it.

Each case plants one mistake in one oracle function, on the CPU: the
function's source with one expression changed (a dropped term, a wrong sign,
bound or index, swapped operands, a wrong stream), compiled in the oracle
module's namespace and patched over the original for the duration of the test.
The pins of that function's area then run, and at least one of them must fail.
A planted mistake that every pin lets through would be a gap in the pins.
The original source must hold the changed expression exactly once, so an edit
of the oracle that moves it fails here loudly instead of passing silently.
"""
import inspect
import textwrap

import pytest

import oracle
import oracle.s3r_oracle as om
from tests import test_oracle_acceptance as tacc
from tests import test_oracle_attention as ta
from tests import test_oracle_kv_commit as tk
from tests import test_oracle_philox as tp
from tests import test_oracle_round_select as tr
from tests import test_oracle_sample as ts
from tests import test_oracle_select as tsel


def _mutant(name, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(om, name)))
    assert src.count(old) == 1, (name, old)
    ns = dict(vars(om))
    exec(compile(src.replace(old, new), f"<{name} with a planted mistake>", "exec"), ns)
    return ns[name]


# Pins per area, cheapest first; each is a call of a pin test with its arguments.
PHILOX = [lambda c=c, k=k: tp.test_philox_matches_numpy(c, k)
          for c, k in [((2, 2, 3, 4), (5, 7)), ((0, 0, 0, 0), (0, 0))]] + [
    tp.test_philox_random_coordinates_match_numpy, tp.test_uniform_is_top53_bits_of_word0,
    tp.test_uniforms_are_uniform]
SELECT = [tsel.test_bounds_are_min_max_and_bound_every_logit,
          tsel.test_one_token_page_score_is_the_exact_logit,
          tsel.test_ties_keep_lowest_indices] + [
    lambda b=b: tsel.test_selection_equals_lexsort_ranking(b) for b in (16, 48, 80, 160)] + [
    tsel.test_heavy_pages_always_selected, tsel.test_selection_is_invariant_to_pool_permutation]
ROUND = [lambda a=a: tr.test_forced_pages_hand_worked(*a) for a in [
    (33, 1, 8, [2]), (33, 6, 8, [2]), (32, 2, 8, [1, 2]), (16, 16, 8, [0, 1]), (48, 16, 8, [2, 3]),
    (1, 4, 8, [0]), (0, 3, 8, [0]), (0, 1, 8, []), (32, 2, 2, [1])]] + [
    lambda a=a: tr.test_kept_set_is_forced_plus_best_candidates(*a) for a in [
        (0, (200, 75, 16), 64, 2), (1, (511, 129, 300), 96, 6), (2, (1000, 47), 128, 16),
        (3, (257, 64, 33), 32, 3)]] + [
    tr.test_gamma_one_with_a_top_tail_page_equals_page_select,
    tr.test_full_budget_keeps_every_page_and_the_future_tail]
ATTENTION = [ta.test_value_layout_is_transposed_per_page, ta.test_closed_forms,
             lambda: ta.test_dense_verify_matches_torch_sdpa("f32"),
             ta.test_dense_verify_equals_sequential_streaming_decodes,
             ta.test_sparse_with_all_pages_equals_dense_decode,
             ta.test_sparse_matches_sdpa_on_gathered_pages]
COMMIT = [lambda a=a: tk.test_rows_land_and_bounds_follow(*a) for a in [
    ((40, 17, 64), 6, (5, 0, 2)), ((15, 16, 200), 3, (2, 2, 2)), ((33, 1, 90), 1, (0, 0, 0))]] + [
    tk.test_rolled_back_rows_do_not_move_bounds, tk.test_one_row_at_a_time_equals_all_at_once,
    tk.test_rows_past_the_table_are_dropped, tk.test_pure_rollback_shrinks_the_tail_page,
    tk.test_rows_in_an_unallocated_page_are_dropped,
    tk.test_rollback_across_a_page_boundary_rebounds_the_new_tail_page]
SAMPLE = [ts.test_icdf_edges, ts.test_output_format] + [
    lambda a=a: ts.test_exact_enumeration_vocab8(*a) for a in [(0, 2, 1.0), (2, 2, 0.7), (1, 3, 1.0)]] + [
    ts.test_q_equals_p_accepts_everything, ts.test_monte_carlo_chi_square_vocab1024,
    ts.test_accepted_length_law]
DIRECT = [tacc.test_acceptance_q_equals_p_is_one, tacc.test_acceptance_disjoint_supports_is_zero] + [
    lambda a=a: tacc.test_acceptance_two_tokens_closed_form(*a) for a in [(1.5, -0.5, 1.0), (3.0, 2.0, 0.5)]] + [
    lambda a=a: tacc.test_acceptance_is_one_minus_total_variation(*a) for a in [(2, 1.0), (3, 0.7)]] + [
    lambda a=a: tacc.test_acceptance_equals_enumerated_accept_probability(*a) for a in [(5, 1.0), (6, 0.7)]] + [
    lambda s=s: tacc.test_draws_follow_the_definition_on_stream_2(s) for s in (0, 3)] + [
    tacc.test_one_position_at_a_time_equals_all_at_once]

# (case, function, expression in the oracle, planted replacement, pins)
MUTANTS = [
    # Philox4x64-10 and the uniforms
    ("philox_nine_rounds", "philox4x64_10", "range(10)", "range(9)", PHILOX),
    ("philox_one_multiplier", "philox4x64_10", "PHILOX_M1 * x2", "PHILOX_M0 * x2", PHILOX),
    ("philox_no_second_key_bump", "philox4x64_10", "k1 = (k1 + PHILOX_W1) & _MASK64", "k1 = k1", PHILOX),
    ("philox_high_words_swapped", "philox4x64_10", "hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1",
     "hi0 ^ x1 ^ k0, lo1, hi1 ^ x3 ^ k1", PHILOX),
    ("uniform_52_bits", "uniform", "(w0 >> 11) * (2.0 ** -53)", "(w0 >> 12) * (2.0 ** -52)", PHILOX),
    ("uniform_seed_in_the_counter", "uniform", "((offset, b, slot, stream), (seed, 0))",
     "((seed, b, slot, stream), (offset, 0))", PHILOX),
    ("uniform_word_1", "uniform", "(seed, 0))[0]", "(seed, 0))[1]", PHILOX),
    # page bounds, scores and selection
    ("bounds_whole_page", "page_bounds", "range(j * P, min((j + 1) * P, L))", "range(j * P, (j + 1) * P)",
     SELECT),
    ("bounds_min_is_max", "page_bounds", "out[phys, h, 0] = rows.min(axis=0)",
     "out[phys, h, 0] = rows.max(axis=0)", SELECT),
    ("bounds_skip_first_token", "page_bounds", "range(j * P, min((j + 1) * P, L))",
     "range(j * P + 1, min((j + 1) * P, L))", SELECT),
    ("scores_min_term_dropped", "page_scores", "np.maximum(q[b, g] * kmin, q[b, g] * kmax)",
     "q[b, g] * kmax", SELECT),
    ("scores_lower_bound", "page_scores", "np.maximum(q[b, g] * kmin", "np.minimum(q[b, g] * kmin", SELECT),
    ("scores_sum_over_group", "page_scores", "best = max(best, s)",
     "best = s if best == -math.inf else best + s", SELECT),
    ("scores_no_scale", "page_scores", "s = scale * float(", "s = float(", SELECT),
    ("scores_wrong_group", "page_scores", "range(h * G, (h + 1) * G)", "range(h, h + G)", SELECT),
    ("select_ties_high_index", "page_select", "key=lambda j: (-sc[j], j)", "key=lambda j: (-sc[j], -j)",
     SELECT),
    ("select_lowest_scores", "page_select", "key=lambda j: (-sc[j], j)", "key=lambda j: (sc[j], j)",
     SELECT),
    ("select_rank_order", "page_select", "selected[b, h, :] = sorted(order[:k])",
     "selected[b, h, :] = order[:k]", SELECT),
    ("select_count_is_k", "page_select", "num_selected[b] = min(k, n)", "num_selected[b] = k", SELECT),
    # once-per-round selection
    ("forced_one_position_more", "round_forced_pages", "0), seq_len + gamma - 2", "0), seq_len + gamma - 1",
     ROUND),
    ("forced_current_position_left_out", "round_forced_pages", "lo, hi = max(seq_len - 1, 0)",
     "lo, hi = max(seq_len, 0)", ROUND),
    ("forced_not_clipped_to_table", "round_forced_pages", "if p // P < max_pages", "if True", ROUND),
    ("round_forced_also_candidates", "page_select_round", "if j not in forced]", "]", ROUND),
    ("round_candidates_ranked_ascending", "page_select_round", "key=lambda j: (-sc[j], j)",
     "key=lambda j: (sc[j], j)", ROUND),
    # attention
    ("attend_no_scale", "attend", "logits = scale * (Kt @ qv)", "logits = Kt @ qv", ATTENTION),
    ("attend_unnormalised", "attend", "(w / w.sum()) @ Vt", "w @ Vt", ATTENTION),
    ("value_row_untransposed", "value_row", "h, :, t % P]", "h, t % P, :]", ATTENTION),
    ("verify_query_misses_itself", "dense_verify_attn", "L - nq + i + 1", "L - nq + i", ATTENTION),
    ("verify_sees_one_more", "dense_verify_attn", "L - nq + i + 1", "L - nq + i + 2", ATTENTION),
    ("verify_gqa_modulo", "dense_verify_attn", "h = g // G", "h = g % hkv", ATTENTION),
    ("draft_tail_not_masked", "sparse_draft_attn", "range(j * P, min((j + 1) * P, L))",
     "range(j * P, (j + 1) * P)", ATTENTION),
    ("draft_gqa_modulo", "sparse_draft_attn", "h = g // G", "h = g % hkv", ATTENTION),
    # KV commit
    ("commit_rollback_floor_ignored", "kv_commit", "lo = min(f, max(L - 1, 0)) // P", "lo = f // P", COMMIT),
    ("commit_bounds_not_refreshed", "kv_commit", "Bd[page_table[b, j]] = fresh[page_table[b, j]]",
     "Bd[page_table[b, j]] = Bd[page_table[b, j]]", COMMIT),
    ("commit_key_one_slot_late", "kv_commit", "K[phys, :, pos % P, :]", "K[phys, :, (pos + 1) % P, :]",
     COMMIT),
    ("commit_value_one_slot_late", "kv_commit", "V[phys, :, :, pos % P]", "V[phys, :, :, (pos + 1) % P]",
     COMMIT),
    ("commit_rollback_ignored", "kv_commit", "fresh = page_bounds(K, page_table, seq_lens)",
     "fresh = page_bounds(K, page_table, np.asarray(first_pos) + count)", COMMIT),
    ("commit_unallocated_written", "kv_commit", " or page_table[b, pos // P] < 0:", ":", COMMIT),
    # speculative sampling
    ("accept_ratio_inverted", "spec_sample", "ratio = p[x] / q[x]", "ratio = q[x] / p[x]", SAMPLE),
    ("residual_sign_flipped", "spec_sample", "np.maximum(0.0, p - q)", "np.maximum(0.0, q - p)", SAMPLE),
    ("residual_is_target", "spec_sample", "w = np.maximum(0.0, p - q)", "w = p", SAMPLE),
    ("bonus_from_last_draft_row", "spec_sample", "softmax(target_logits[b, gamma], temperature)",
     "softmax(target_logits[b, gamma - 1], temperature)", SAMPLE),
    ("draft_law_without_temperature", "spec_sample", "softmax(draft_logits[b, i], temperature)",
     "softmax(draft_logits[b, i], 1.0)", SAMPLE),
    ("draw_on_the_accept_stream", "spec_sample", "icdf(w, uniform_fn(b, i, 1))",
     "icdf(w, uniform_fn(b, i, 0))", SAMPLE),
    ("no_stop_after_rejection", "spec_sample", "rejected = True\n            break", "rejected = True",
     SAMPLE),
    ("softmax_ignores_temperature", "softmax", "np.float64) / temperature", "np.float64)", SAMPLE),
    ("icdf_non_strict", "icdf", "c > target", "c >= target", SAMPLE),
    # direct sparse sampling: the drafter's draws and the acceptance rate
    ("alpha_max_not_min", "acceptance_rate", "np.minimum(p, q)", "np.maximum(p, q)", DIRECT),
    ("alpha_next_target_row", "acceptance_rate", "target_logits[b, i], temperature",
     "target_logits[b, i + 1], temperature", DIRECT),
    ("alpha_without_temperature", "acceptance_rate", "softmax(draft_logits[b, i], temperature)",
     "softmax(draft_logits[b, i], 1.0)", DIRECT),
    ("alpha_unnormalised_min", "acceptance_rate", "np.minimum(p, q).sum()", "np.minimum(p, q).max()", DIRECT),
    ("draws_on_the_residual_stream", "draw_tokens", "uniform(seed, offset, b, first_slot + r, 2)",
     "uniform(seed, offset, b, first_slot + r, 1)", DIRECT),
    ("draws_ignore_first_slot", "draw_tokens", "uniform(seed, offset, b, first_slot + r, 2)",
     "uniform(seed, offset, b, r, 2)", DIRECT),
    ("draws_without_temperature", "draw_tokens", "softmax(logits[b, r], temperature)",
     "softmax(logits[b, r], 1.0)", DIRECT),
]


@pytest.mark.parametrize("case,fn,old,new,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(case, fn, old, new, pins, monkeypatch):
    mutant = _mutant(fn, old, new)
    monkeypatch.setattr(om, fn, mutant)
    monkeypatch.setattr(oracle, fn, mutant)
    for pin in pins:
        try:
            pin()
        except Exception:  # an assertion, or an error the mistake provokes
            return
    pytest.fail(f"no pin caught the planted mistake {case!r} in {fn}")


def test_unplanted_oracle_passes_every_pin():
    for pins in (PHILOX, SELECT, ROUND, ATTENTION, COMMIT, SAMPLE, DIRECT):
        for pin in pins:
            pin()
