"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of oracle.c (a flipped comparison, a
wrong row or uniform index, a transposed ratio, a dropped temperature, a
wrong search direction ...), compiles the copy with gcc, and runs the pins
of the affected function against it.  At least one pin must fail for every
planted mistake; the shipped oracle passes them all.  Mistakes are planted
only in the CPU oracle and only in temporary copies.
"""
import os

import pytest

import oracle
import test_oracle_greedy as G
import test_oracle_rejection as R
import test_oracle_suffix as SX
import test_oracle_tree_ngram as TN
from conftest import golden

TAU = golden("tau_values.json")["cases"]

GREEDY_PINS = [G.test_worked_example, G.test_all_accepted_plus_one,
               G.test_argmax_matches_numpy_with_ties, G.test_draft_len_and_flags,
               lambda o: G.test_greedy_identity_planted_proposer(o, 0.9),
               lambda o: G.test_tau_closed_form(o, TAU[0])]
REJECTION_PINS = [R.test_worked_example_sampling_form, R.test_flags_and_draft_len,
                  R.test_one_hot_target_is_greedy,
                  R.test_probabilities_match_scipy_softmax_with_temperature,
                  lambda o: R.test_output_distribution_chisquare_v8(o, 1),
                  lambda o: R.test_output_distribution_chisquare_v8(o, 3),
                  R.test_identical_draft_accepts_everything, R.test_one_hot_draft_accepts_with_p]
TIE_PINS = ([lambda o, d=d: R.test_accept_tie_flag_band(o, d)
             for d in (-3e-7, 3e-7, -9e-7, 9e-7, -1.1e-6, 1.1e-6, -3e-6, 3e-6)] +
            [R.test_accept_tie_counts_only_decisions_taken] +
            [lambda o, e=e, f=f: R.test_sample_tie_flag_band_bonus(o, e[0], e[1], f)
             for e in ((0.5, 0), (0.75, 1), (0.875, 2)) for f in (-1.5, -0.8, 0.8, 1.5)] +
            [lambda o, f=f: R.test_sample_tie_flag_band_residual(o, f)
             for f in (-1.25, -0.85, 0.85, 1.25)] +
            [R.test_sample_tie_at_the_top_of_the_distribution,
             R.test_flagged_fraction_at_the_rejection_workload_size])
TREE_PINS = [TN.test_tree_single_node, TN.test_tree_equal_depth_tie_lowest_id,
             TN.test_chain_tree_is_greedy,
             TN.test_random_trees_brute_force]
NGRAM_PINS = [TN.test_ngram_overlap_short_and_ragged, TN.test_ngram_planted_copy,
              TN.test_ngram_exhaustive_ternary]
SUFFIX_PINS = [SX.test_worked_example, SX.test_history_tree_and_separators,
               SX.test_better_text_wins_and_context_wins_ties,
               SX.test_periodic_context_continues_the_period,
               SX.test_one_occurrence_reduces_to_ngram_lookup,
               lambda o: SX.test_exhaustive_ternary_against_brute_force(o, 1, 3, 3, 0.0, 256)]

MUTANTS = [
    ("argmax keeps the last maximum", "if (x > bv) {", "if (x >= bv) {", GREEDY_PINS),
    ("greedy compares with the next row",
     "draft[(size_t)b * K + n] == t[n])", "draft[(size_t)b * K + n] == t[n + 1])", GREEDY_PINS),
    ("bonus from the previous row", "e = t[n];", "e = t[n > 0 ? n - 1 : 0];", GREEDY_PINS),
    ("temperature dropped from the normaliser",
     "Z += exp(orc_widen(row, dtype, v) / T - M);", "Z += exp(orc_widen(row, dtype, v) - M);",
     REJECTION_PINS),
    ("ratio transposed", "ratio = qi > 0.0 ? pi / qi : INFINITY;",
     "ratio = pi > 0.0 ? qi / pi : INFINITY;", REJECTION_PINS),
    ("accept test reversed", "if (ui < ratio)", "if (ui > ratio)", REJECTION_PINS),
    ("residual sign flipped", "double d = P[v] - Q[v];", "double d = Q[v] - P[v];",
     REJECTION_PINS),
    ("residual not clipped at zero", "r[v] = d > 0.0 ? d : 0.0;", "r[v] = d;", REJECTION_PINS),
    ("final sample uses the first uniform", "double thr = (double)ub[K] * S;",
     "double thr = (double)ub[0] * S;", REJECTION_PINS),
    ("no stop at the first rejection", "stopped = 1;", "stopped = 0;", REJECTION_PINS),
    ("every accept test flagged", "if (valid && fabs(ui - ratio) < accept_band)", "if (valid)",
     TIE_PINS),
    ("accept band ten times wider", "fabs(ui - ratio) < accept_band", "fabs(ui - ratio) < 10.0 * accept_band",
     TIE_PINS),
    ("accept ties flagged at invalid ids", "if (valid && fabs(ui - ratio) < accept_band)",
     "if (fabs(ui - ratio) < accept_band)", TIE_PINS),
    ("accept ties never flagged", "atie = 1;", "atie = 0;", TIE_PINS),
    ("sample band a million times wider", "double band = sample_band_scale * sqrt(sq);",
     "double band = 1e6 * sample_band_scale * sqrt(sq);", TIE_PINS),
    ("sample band without the square root", "double band = sample_band_scale * sqrt(sq);",
     "double band = sample_band_scale * sq;", TIE_PINS),
    ("sample band ignores the draft row",
     "        if (n < len)\n            for (int32_t v = 0; v < V; ++v)\n                sq += Q[v] * Q[v];\n",
     "", TIE_PINS),
    ("every draw flagged", "} else if (thr - lo < band || hi - thr < band) {", "} else if (1) {",
     TIE_PINS),
    ("sample band on one side only", "thr - lo < band || hi - thr < band", "hi - thr < band",
     TIE_PINS),
    ("sample ties never flagged", "} else if (thr - lo < band || hi - thr < band) {",
     "} else if (0) {", TIE_PINS),
    ("tree checks the node's own row", "acc[j] = acc[p] && tok[j] == t[p];",
     "acc[j] = acc[p] && tok[j] == t[j];", TREE_PINS),
    ("tree ignores the parent's acceptance", "acc[j] = acc[p] && tok[j] == t[p];",
     "acc[j] = tok[j] == t[p];", TREE_PINS),
    ("tree ties go to the largest id", "if (acc[j] && depth[j] > bestd) {",
     "if (acc[j] && depth[j] >= bestd) {", TREE_PINS),
    ("n-gram takes the earliest occurrence", "for (int64_t s = L - n - 1; s >= 0; --s) {",
     "for (int64_t s = 0; s <= L - n - 1; ++s) {", NGRAM_PINS),
    ("n-gram tries the shortest length first",
     "for (int32_t n = n_max; n >= n_min && got_n == 0; --n) {",
     "for (int32_t n = n_min; n <= n_max && got_n == 0; ++n) {", NGRAM_PINS),
    ("n-gram copies from the match start", "pr[k] = c[got_s + got_n + k];",
     "pr[k] = c[got_s + k];", NGRAM_PINS),
    ("n-gram lets the suffix match itself", "for (int64_t s = L - n - 1; s >= 0; --s) {",
     "for (int64_t s = L - n; s >= 0; --s) {", NGRAM_PINS),
    ("given probabilities are not normalised", "p[v] = orc_widen(row, dtype, v) / Z;",
     "p[v] = orc_widen(row, dtype, v);",
     [R.test_probability_input_equals_logit_input, lambda o: R.test_probability_input_chisquare_v8(o, 1)]),
    ("suffix counts the oldest occurrences",
     "for (int64_t e = len_t - 2; e >= 0 && n < occ_cap; --e)",
     "for (int64_t e = 0; e <= len_t - 2 && n < occ_cap; ++e)", SUFFIX_PINS),
    ("suffix ties go to the larger id", "(cnt == cnt_best && t < tok)",
     "(cnt == cnt_best && t > tok)", SUFFIX_PINS),
    ("suffix path does not narrow the occurrences",
     "alive[i] = alive[i] && occ[i] + j < len_t && text[occ[i] + j] == tok;",
     "alive[i] = alive[i] && occ[i] + j < len_t;", SUFFIX_PINS),
    ("suffix ignores document separators", "        if (text[e + 1] < 0)\n            continue;",
     "", SUFFIX_PINS),
    ("suffix prefers the history on equal scores", "sc * (int64_t)nh >= sh * (int64_t)nc",
     "sc * (int64_t)nh > sh * (int64_t)nc", SUFFIX_PINS),
    ("suffix score counts tokens, not probabilities", "sum += cnt_best;", "sum += n;",
     SUFFIX_PINS),
    ("suffix takes the shortest pattern", "if (m > best)", "if (m > 0 && (best == 0 || m < best))",
     SUFFIX_PINS),
]


@pytest.mark.parametrize("name,old,new,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new, pins):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    assert src.count(old) == 1, "mutation anchor must be unique: %r" % old
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(old, new))
    so = oracle.compile_source(str(mut), str(tmp_path / "liboracle_mut.so"))
    m = oracle.Oracle(so)
    failed = []
    for pin in pins:
        try:
            pin(m)
        except AssertionError:
            failed.append(getattr(pin, "__name__", "pin"))
            break
    assert failed, "no pin caught the planted mistake: %s" % name
