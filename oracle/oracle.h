/*
 * oracle.h -- plain, slow, obviously-correct CPU oracle for the speculative
 * decoding hot path: greedy, rejection-sampling and tree verification, and
 * n-gram prompt-lookup proposal.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this code; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no source with the GPU path.
 *
 * Sources (the pages this follows; section names as the pages give them):
 *  [Arctic]   "Fastest Speculative Decoding in vLLM with Arctic Inference and
 *             Arctic Training" (Snowflake; Chinese repost) -- sections
 *             "what is speculative decoding" (proposer / scorer / verifier),
 *             "a simple example" (the 16 -> 13, 578, 7301 -> 21747 step),
 *             "inference pipeline optimisation" (greedy verification).
 *  [Handbook] LLM Inference Handbook, chapter "speculative decoding" --
 *             sections "how it works" (longest agreeing prefix + the
 *             (h+1)-th token from the target), "key metrics" (tau formula),
 *             "Medusa" (candidate tree, longest accepted prefix),
 *             "N-gram" (four-step prompt lookup).
 *  [vLLM-03]  "vLLM features 03: speculative decoding" (ttlab) -- sections
 *             "1. principle" (stop at the first wrong token, replace it by
 *             the target's token; rejection sampling keeps the target
 *             distribution), "2. draft methods" (prompt_lookup_min/max),
 *             "3-1. re-measure" (no match -> no draft).
 *  The rejection rule itself (accept x with probability min(1, p(x)/q(x)),
 *  else sample from the normalised positive part of p - q) is the
 *  Leviathan et al. / Chen et al. rule that [vLLM-03] cites; the pages never
 *  print it as a formula, so it is written here from those papers' statement.
 *
 * Arithmetic: every floating-point step is fp64 from exactly widened inputs
 * (bf16 -> fp32 by a 16-bit shift, then fp32 -> fp64).  Plain scalar loops,
 * no blocking, no threads, no reordering beyond what each definition states.
 *
 * Layouts are row-major.  All pointers are host pointers.
 */
#ifndef SV_ORACLE_H
#define SV_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* input element types */
#define ORC_F32 0
#define ORC_BF16 1
#define ORC_PROBS 2    /* rejection sampling only: fp32 rows of probabilities */

/* per-sequence data-error flag bits (same meaning as the library's) */
#define ORC_FLAG_DRAFT_OOR 1u    /* a draft / node token id outside [0, V) */
#define ORC_FLAG_BAD_LEN 2u      /* draft_len outside [0, K] (clamped) or context length outside [0, stride] */
#define ORC_FLAG_BAD_PARENT 4u   /* tree parent[j] outside [0, j) for j >= 1, or parent[0] != -1 */

/* Widen element i of a row to fp64, exactly. */
double orc_widen(const void *row, int dtype, int64_t i);

/* Smallest index holding the row maximum (numpy / torch argmax convention). */
int32_t orc_argmax(const void *row, int dtype, int64_t V);

/*
 * Greedy verification.  logits [B][K+1][row_stride] (first V used),
 * draft [B][K], draft_len [B] or NULL (= K).
 * Outputs: accepted [B], emitted [B][K+1] (-1 padded),
 * argmax_out [B][K+1] or NULL (rows past draft_len are not needed and
 * are reported as -1), flags [B] or NULL.
 */
void orc_verify_greedy(const void *logits, int dtype, int64_t row_stride,
                       const int32_t *draft, const int32_t *draft_len,
                       int32_t B, int32_t K, int32_t V,
                       int32_t *accepted, int32_t *emitted,
                       int32_t *argmax_out, uint32_t *flags);

/*
 * Rejection-sampling verification.
 * target [B][K+1][row_stride], draftl [B][K][row_stride], draft [B][K],
 * draft_len [B] or NULL, u [B][K+1] in [0,1): u[b][i] drives accept test i,
 * u[b][K] drives the one final sample.  T > 0 is applied to both models.
 * dtype ORC_PROBS: the rows hold probabilities (fp32, non-negative, each
 * row with a positive sum); a row's distribution is the row over its sum,
 * and T is not used.
 * Outputs: accepted [B], emitted [B][K+1] (-1 padded),
 *   p_draft / q_draft [B][K] (p_i(x_i), q_i(x_i) for i < draft_len and a
 *   valid id, else 0) or NULL,
 *   accept_tie [B] or NULL: 1 when some accept test that was evaluated had
 *     |u - p/q| < accept_band,
 *   sample_tie [B] or NULL: 1 when u*S lies within
 *     sample_band_scale * sqrt(sum_v p_v^2 + sum_v q_v^2) (probability mass;
 *     the q term only when a residual is sampled) of either end of the
 *     chosen token's CDF interval, or when no CDF entry exceeds u*S,
 *   flags [B] or NULL.
 */
void orc_verify_rejection(const void *target, const void *draftl, int dtype,
                          int64_t row_stride, const int32_t *draft,
                          const int32_t *draft_len, const float *u, double T,
                          int32_t B, int32_t K, int32_t V,
                          double accept_band, double sample_band_scale,
                          int32_t *accepted, int32_t *emitted,
                          double *p_draft, double *q_draft,
                          uint8_t *accept_tie, uint8_t *sample_tie,
                          uint32_t *flags);

/*
 * The final sample's cumulative distribution for one row pair: r = max(0,
 * p - q) when draft_row is given (p when that sums to 0), r = p when it is
 * NULL; cdf[v] = sum_{w <= v} r_w over V entries; returns S = sum_v r_v.
 * The rows are single rows of dtype (ORC_PROBS: probabilities).
 */
double orc_sample_cdf(const void *target_row, const void *draft_row, int dtype, int32_t V,
                      double T, double *cdf);

/*
 * Tree verification.  logits [B][N][row_stride]: row j scores the children
 * of node j.  parent [B][N] (parent[b][0] = -1, parent[b][j] in [0, j)),
 * token [B][N] (root token ignored).
 * Outputs: accepted [B] = depth of the chosen node, path [B][N] (node ids
 * root excluded, -1 padded), emitted [B][N] (path tokens then the bonus;
 * depth <= N-1 so N slots always suffice; -1 padded), argmax_out [B][N] or NULL, flags [B] or NULL.
 */
void orc_verify_tree(const void *logits, int dtype, int64_t row_stride,
                     const int32_t *parent, const int32_t *token,
                     int32_t B, int32_t N, int32_t V,
                     int32_t *accepted, int32_t *path, int32_t *emitted,
                     int32_t *argmax_out, uint32_t *flags);

/*
 * N-gram prompt lookup.  tokens [B][ctx_stride], lengths [B].
 * Outputs: proposal [B][K] (-1 padded), proposal_len [B],
 * match_n [B] (0 when no match) and match_pos [B] (start of the matched
 * earlier occurrence, -1 when none) or NULL, flags [B] or NULL.
 */
void orc_ngram_propose(const int32_t *tokens, int64_t ctx_stride,
                       const int32_t *lengths, int32_t B,
                       int32_t n_min, int32_t n_max, int32_t K,
                       int32_t *proposal, int32_t *proposal_len,
                       int32_t *match_n, int32_t *match_pos, uint32_t *flags);

/*
 * Suffix-decoding proposal ([Arctic] "suffix decoding": the recent tokens
 * are matched against suffix trees of the current prompt and of earlier
 * outputs, and candidate tokens are ranked by how often they followed).
 * tokens [B][ctx_stride] with lengths [B] (the current contexts);
 * history [H] (earlier outputs, one shared text; negative entries separate
 * documents and never match or continue); occ_cap = how many of the most
 * recent occurrences of the matched pattern are counted.
 * Outputs: proposal [B][K] (-1 padded), proposal_len [B], score [B] (the
 * expected number of accepted tokens, sum of the path's probabilities),
 * match_len [B] (the matched pattern's length, 0 when none), source [B]
 * (0 context, 1 history, -1 none) or NULL, flags [B] or NULL.
 */
void orc_suffix_propose(const int32_t *tokens, int64_t ctx_stride,
                        const int32_t *lengths, int32_t B,
                        const int32_t *history, int64_t H,
                        int32_t m_min, int32_t m_max, int32_t K, double min_prob,
                        int32_t occ_cap,
                        int32_t *proposal, int32_t *proposal_len, double *score,
                        int32_t *match_len, int32_t *source, uint32_t *flags);

#ifdef __cplusplus
}
#endif

#endif /* SV_ORACLE_H */
