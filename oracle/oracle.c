/*
 * oracle.c -- plain CPU oracle for the speculative-decoding hot path.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * CPU-baseline leg of the benchmark, never by the product library.  It shares
 * no code, header, table or helper with the GPU path.
 *
 * Every function below is the plain definition of what the method computes,
 * written as scalar loops in fp64.  Page references name the page and its
 * section (see oracle.h for the page list).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* bf16 is the top half of an IEEE binary32; widening is a 16-bit shift. */
double orc_widen(const void *row, int dtype, int64_t i)
{
    if (dtype == ORC_F32 || dtype == ORC_PROBS)
        return (double)((const float *)row)[i];
    uint32_t bits = ((uint32_t)((const uint16_t *)row)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static const void *row_ptr(const void *base, int dtype, int64_t row, int64_t row_stride)
{
    size_t esize = dtype == ORC_BF16 ? 2 : 4;
    return (const char *)base + (size_t)row * (size_t)row_stride * esize;
}

/* argmax with the lowest index on ties: scan left to right, replace only on
 * a strictly larger value. */
int32_t orc_argmax(const void *row, int dtype, int64_t V)
{
    int32_t best = 0;
    double bv = orc_widen(row, dtype, 0);
    for (int64_t v = 1; v < V; ++v) {
        double x = orc_widen(row, dtype, v);
        if (x > bv) {
            bv = x;
            best = (int32_t)v;
        }
    }
    return best;
}

static int32_t clamp_len(int32_t len, int32_t K, uint32_t *fl)
{
    if (len < 0) {
        *fl |= ORC_FLAG_BAD_LEN;
        return 0;
    }
    if (len > K) {
        *fl |= ORC_FLAG_BAD_LEN;
        return K;
    }
    return len;
}

/*
 * Greedy verification ([Arctic] "inference pipeline optimisation": only
 * tokens that agree with greedy decoding are accepted; [Handbook] "how it
 * works": accept the longest agreeing prefix h, the target supplies token
 * h+1; [vLLM-03] "1. principle": stop at the first wrong draft, put the
 * target's own token there).
 *   t_i = argmax row i;  n = first i < len with draft_i != t_i (else len);
 *   emitted = draft_0 .. draft_{n-1}, t_n.
 */
void orc_verify_greedy(const void *logits, int dtype, int64_t row_stride,
                       const int32_t *draft, const int32_t *draft_len,
                       int32_t B, int32_t K, int32_t V,
                       int32_t *accepted, int32_t *emitted,
                       int32_t *argmax_out, uint32_t *flags)
{
    int32_t *t = (int32_t *)malloc(sizeof(int32_t) * (size_t)(K + 1));
    for (int32_t b = 0; b < B; ++b) {
        uint32_t fl = 0;
        int32_t len = draft_len ? clamp_len(draft_len[b], K, &fl) : K;
        for (int32_t i = 0; i <= K; ++i) {
            if (i <= len)
                t[i] = orc_argmax(row_ptr(logits, dtype, (int64_t)b * (K + 1) + i, row_stride), dtype, V);
            else
                t[i] = -1; /* row not needed: position past the draft */
            if (argmax_out)
                argmax_out[(size_t)b * (K + 1) + i] = t[i];
        }
        for (int32_t i = 0; i < len; ++i) {
            int32_t x = draft[(size_t)b * K + i];
            if (x < 0 || x >= V)
                fl |= ORC_FLAG_DRAFT_OOR;
        }
        int32_t n = 0;
        while (n < len && draft[(size_t)b * K + n] == t[n])
            ++n;
        for (int32_t i = 0; i <= K; ++i) {
            int32_t e = -1;
            if (i < n)
                e = draft[(size_t)b * K + i];
            else if (i == n)
                e = t[n];
            emitted[(size_t)b * (K + 1) + i] = e;
        }
        accepted[b] = n;
        if (flags)
            flags[b] = fl;
    }
    free(t);
}

/* Softmax of one row at temperature T, in fp64:
 *   z_v = l_v / T,  M = max_v z_v,  p_v = exp(z_v - M) / sum_w exp(z_w - M). */
static void softmax_row(const void *row, int dtype, int32_t V, double T, double *p)
{
    if (dtype == ORC_PROBS) {          /* given probabilities: normalise the row */
        double Z = 0.0;
        for (int32_t v = 0; v < V; ++v)
            Z += orc_widen(row, dtype, v);
        for (int32_t v = 0; v < V; ++v)
            p[v] = orc_widen(row, dtype, v) / Z;
        return;
    }
    double M = -INFINITY;
    for (int32_t v = 0; v < V; ++v) {
        double z = orc_widen(row, dtype, v) / T;
        if (z > M)
            M = z;
    }
    double Z = 0.0;
    for (int32_t v = 0; v < V; ++v)
        Z += exp(orc_widen(row, dtype, v) / T - M);
    for (int32_t v = 0; v < V; ++v)
        p[v] = exp(orc_widen(row, dtype, v) / T - M) / Z;
}

/* The distribution of the final sample: after a rejection (Q given) the
 * residual r = max(0, p - q), or p itself when that has no mass; with no
 * draft row (every draft accepted) r = p.  Returns S = sum_v r_v. */
static double final_distribution(const double *P, const double *Q, int32_t V, double *r)
{
    double S = 0.0;
    if (Q) {
        for (int32_t v = 0; v < V; ++v) {
            double d = P[v] - Q[v];
            r[v] = d > 0.0 ? d : 0.0;
            S += r[v];
        }
    }
    if (!Q || S == 0.0) {
        S = 0.0;
        for (int32_t v = 0; v < V; ++v) {
            r[v] = P[v];
            S += r[v];
        }
    }
    return S;
}

/*
 * Rejection-sampling verification (Leviathan et al.; Chen et al.; cited by
 * [vLLM-03] "1. principle" for keeping the target distribution at T > 0;
 * [Arctic] "what is speculative decoding" names rejection sampling as the
 * usual verifier).  Per sequence:
 *   for i < len: accept draft x_i iff u_i < p_i(x_i) / q_i(x_i)
 *                (q = 0 -> ratio +inf; an id outside [0, V) is rejected);
 *                stop at the first rejection, n = number accepted.
 *   final token: n < len -> r = max(0, p_n - q_n) (if sum r == 0, r = p_n);
 *                n = len -> r = p_n (the target's own next token).
 *   y = smallest j with C_j = sum_{v<=j} r_v > u_K * S, S = sum_v r_v;
 *       if no such j (rounding), the largest j with r_j > 0.
 *   emitted = x_0 .. x_{n-1}, y.
 * u_i < ratio is the same event as u_i < min(1, ratio) for u_i in [0, 1).
 */
void orc_verify_rejection(const void *target, const void *draftl, int dtype,
                          int64_t row_stride, const int32_t *draft,
                          const int32_t *draft_len, const float *u, double T,
                          int32_t B, int32_t K, int32_t V,
                          double accept_band, double sample_band_scale,
                          int32_t *accepted, int32_t *emitted,
                          double *p_draft, double *q_draft,
                          uint8_t *accept_tie, uint8_t *sample_tie,
                          uint32_t *flags)
{
    double *P = (double *)malloc(sizeof(double) * (size_t)V);
    double *Q = (double *)malloc(sizeof(double) * (size_t)V);
    double *r = (double *)malloc(sizeof(double) * (size_t)V);
    for (int32_t b = 0; b < B; ++b) {
        uint32_t fl = 0;
        int32_t len = draft_len ? clamp_len(draft_len[b], K, &fl) : K;
        const float *ub = u + (size_t)b * (K + 1);
        int32_t n = 0;
        int stopped = 0;
        uint8_t atie = 0, stie = 0;
        for (int32_t i = 0; i < K; ++i) {
            double pi = 0.0, qi = 0.0;
            int32_t x = draft[(size_t)b * K + i];
            int valid = x >= 0 && x < V;
            if (i < len) {
                if (!valid)
                    fl |= ORC_FLAG_DRAFT_OOR;
                if (valid) {
                    softmax_row(row_ptr(target, dtype, (int64_t)b * (K + 1) + i, row_stride), dtype, V, T, P);
                    softmax_row(row_ptr(draftl, dtype, (int64_t)b * K + i, row_stride), dtype, V, T, Q);
                    pi = P[x];
                    qi = Q[x];
                }
                if (!stopped) {
                    double ratio = 0.0;
                    if (valid)
                        ratio = qi > 0.0 ? pi / qi : INFINITY;
                    double ui = (double)ub[i];
                    if (valid && fabs(ui - ratio) < accept_band)
                        atie = 1;
                    if (ui < ratio)
                        ++n;
                    else
                        stopped = 1;
                }
            }
            if (p_draft)
                p_draft[(size_t)b * K + i] = pi;
            if (q_draft)
                q_draft[(size_t)b * K + i] = qi;
        }

        /* the final token: residual after a rejection, else the bonus */
        softmax_row(row_ptr(target, dtype, (int64_t)b * (K + 1) + n, row_stride), dtype, V, T, P);
        if (n < len)
            softmax_row(row_ptr(draftl, dtype, (int64_t)b * K + n, row_stride), dtype, V, T, Q);
        double S = final_distribution(P, n < len ? Q : NULL, V, r);
        /* tie band for this draw, in probability mass: band_scale times
         * sqrt(sum p^2 + sum q^2) over the rows the final sample reads */
        double sq = 0.0;
        for (int32_t v = 0; v < V; ++v)
            sq += P[v] * P[v];
        if (n < len)
            for (int32_t v = 0; v < V; ++v)
                sq += Q[v] * Q[v];
        double band = sample_band_scale * sqrt(sq);
        double thr = (double)ub[K] * S;
        double C = 0.0, lo = 0.0, hi = 0.0;
        int32_t y = -1;
        for (int32_t v = 0; v < V; ++v) {
            double prev = C;
            C += r[v];
            if (C > thr) {
                y = v;
                lo = prev;
                hi = C;
                break;
            }
        }
        if (y < 0) {
            for (int32_t v = V - 1; v >= 0; --v)
                if (r[v] > 0.0) {
                    y = v;
                    break;
                }
            stie = 1;
        } else if (thr - lo < band || hi - thr < band) {
            stie = 1;
        }

        for (int32_t i = 0; i <= K; ++i) {
            int32_t e = -1;
            if (i < n)
                e = draft[(size_t)b * K + i];
            else if (i == n)
                e = y;
            emitted[(size_t)b * (K + 1) + i] = e;
        }
        accepted[b] = n;
        if (accept_tie)
            accept_tie[b] = atie;
        if (sample_tie)
            sample_tie[b] = stie;
        if (flags)
            flags[b] = fl;
    }
    free(P);
    free(Q);
    free(r);
}

/* The final sample's cumulative distribution for one row pair (the
 * definition orc_verify_rejection draws from): cdf[v] = C_v = the sum of
 * r_w over w <= v in token order; returns S = C_{V-1}.  draft_row NULL:
 * r = p (the bonus). */
double orc_sample_cdf(const void *target_row, const void *draft_row, int dtype, int32_t V,
                      double T, double *cdf)
{
    double *P = (double *)malloc(sizeof(double) * (size_t)V);
    double *Q = (double *)malloc(sizeof(double) * (size_t)V);
    softmax_row(target_row, dtype, V, T, P);
    if (draft_row)
        softmax_row(draft_row, dtype, V, T, Q);
    double S = final_distribution(P, draft_row ? Q : NULL, V, cdf);
    double C = 0.0;
    for (int32_t v = 0; v < V; ++v) {
        C += cdf[v];
        cdf[v] = C;
    }
    free(P);
    free(Q);
    return S;
}

/*
 * Tree verification ([Handbook] "Medusa": the heads' candidates form a tree
 * scored in one pass; the longest accepted candidate prefix is kept).
 *   t_j = argmax row j (row j predicts the children of node j);
 *   node 0 (root) is accepted; node j >= 1 is accepted iff its parent is
 *   accepted and token_j == t_parent;
 *   the chosen node j* is the deepest accepted node (smallest id on ties);
 *   emitted = the tokens on the root -> j* path (root excluded), then t_{j*}.
 */
void orc_verify_tree(const void *logits, int dtype, int64_t row_stride,
                     const int32_t *parent, const int32_t *token,
                     int32_t B, int32_t N, int32_t V,
                     int32_t *accepted, int32_t *path, int32_t *emitted,
                     int32_t *argmax_out, uint32_t *flags)
{
    int32_t *t = (int32_t *)malloc(sizeof(int32_t) * (size_t)N);
    int32_t *depth = (int32_t *)malloc(sizeof(int32_t) * (size_t)N);
    uint8_t *acc = (uint8_t *)malloc((size_t)N);
    for (int32_t b = 0; b < B; ++b) {
        uint32_t fl = 0;
        const int32_t *par = parent + (size_t)b * N;
        const int32_t *tok = token + (size_t)b * N;
        for (int32_t j = 0; j < N; ++j) {
            t[j] = orc_argmax(row_ptr(logits, dtype, (int64_t)b * N + j, row_stride), dtype, V);
            if (argmax_out)
                argmax_out[(size_t)b * N + j] = t[j];
        }
        if (par[0] != -1)
            fl |= ORC_FLAG_BAD_PARENT;
        acc[0] = 1;
        depth[0] = 0;
        for (int32_t j = 1; j < N; ++j) {
            int32_t p = par[j];
            if (tok[j] < 0 || tok[j] >= V)
                fl |= ORC_FLAG_DRAFT_OOR;
            if (p < 0 || p >= j) {
                fl |= ORC_FLAG_BAD_PARENT;
                acc[j] = 0;
                depth[j] = 0;
                continue;
            }
            acc[j] = acc[p] && tok[j] == t[p];
            depth[j] = depth[p] + 1;
        }
        int32_t best = 0, bestd = 0;
        for (int32_t j = 1; j < N; ++j)
            if (acc[j] && depth[j] > bestd) {
                bestd = depth[j];
                best = j;
            }
        int32_t *pb = path + (size_t)b * N;
        int32_t *eb = emitted + (size_t)b * N;
        for (int32_t j = 0; j < N; ++j) {
            pb[j] = -1;
            eb[j] = -1;
        }
        int32_t cur = best;
        for (int32_t d = bestd - 1; d >= 0; --d) {
            pb[d] = cur;
            eb[d] = tok[cur];
            cur = par[cur];
        }
        eb[bestd] = t[best];
        accepted[b] = bestd;
        if (flags)
            flags[b] = fl;
    }
    free(t);
    free(depth);
    free(acc);
}

/*
 * N-gram prompt lookup ([Handbook] "N-gram": take a suffix of the current
 * sequence, search the earlier text for it, copy what followed;
 * [vLLM-03] "2. draft methods": lookup lengths prompt_lookup_max down to
 * prompt_lookup_min; "3-1. re-measure": no match, no draft).
 *   for n = n_max .. n_min:  for s = L-n-1 .. 0 (most recent first):
 *     if c[s .. s+n) == c[L-n .. L): copy c[s+n .. s+n+m), m = min(K, L-s-n).
 */
void orc_ngram_propose(const int32_t *tokens, int64_t ctx_stride,
                       const int32_t *lengths, int32_t B,
                       int32_t n_min, int32_t n_max, int32_t K,
                       int32_t *proposal, int32_t *proposal_len,
                       int32_t *match_n, int32_t *match_pos, uint32_t *flags)
{
    for (int32_t b = 0; b < B; ++b) {
        uint32_t fl = 0;
        const int32_t *c = tokens + (size_t)b * (size_t)ctx_stride;
        int64_t L = lengths[b];
        if (L < 0 || L > ctx_stride) {
            fl |= ORC_FLAG_BAD_LEN;
            L = 0;
        }
        int32_t *pr = proposal + (size_t)b * K;
        for (int32_t k = 0; k < K; ++k)
            pr[k] = -1;
        int32_t got_n = 0, got_s = -1, m = 0;
        for (int32_t n = n_max; n >= n_min && got_n == 0; --n) {
            for (int64_t s = L - n - 1; s >= 0; --s) {
                int32_t j = 0;
                while (j < n && c[s + j] == c[L - n + j])
                    ++j;
                if (j == n) {
                    got_n = n;
                    got_s = (int32_t)s;
                    break;
                }
            }
        }
        if (got_n > 0) {
            int64_t avail = L - got_s - got_n;
            m = (int32_t)(avail < K ? avail : K);
            for (int32_t k = 0; k < m; ++k)
                pr[k] = c[got_s + got_n + k];
        }
        proposal_len[b] = m;
        if (match_n)
            match_n[b] = got_n;
        if (match_pos)
            match_pos[b] = got_s;
        if (flags)
            flags[b] = fl;
    }
}

/* ------------------------------------------------------------------ suffix
 * [Arctic] "suffix decoding": suffix trees over the current prompt and over
 * earlier outputs are searched with the most recently generated tokens, and
 * each candidate token is ranked by its frequency (an empirical
 * probability); the candidate sequence is as long as it stays likely.  A
 * suffix tree answers "where does this pattern occur, and what followed
 * it"; the oracle answers the same questions directly from the texts.
 */

/* Length of the common suffix of text[..e] and the context c[..L-1], at
 * most m_max; a context token below 0 never matches. */
static int32_t suffix_match(const int32_t *text, int64_t e, const int32_t *c, int64_t L,
                            int32_t m_max)
{
    int32_t m = 0;
    while (m < m_max && e - m >= 0 && L - 1 - m >= 0 && c[L - 1 - m] >= 0 &&
           text[e - m] == c[L - 1 - m])
        ++m;
    return m;
}

/* One text.  An occurrence is an end position e whose next token exists and
 * is a token (text[e + 1] >= 0).  The pattern is the longest context suffix
 * (m_min <= length <= m_max) with an occurrence; the occ_cap most recent
 * occurrences are counted.  Depth by depth, the next candidate is the token
 * that follows the current path most often among them (lowest id on equal
 * counts); its probability is that count over the number of occurrences,
 * and the path stops before a token whose probability is below min_prob, or
 * when nothing follows.  Returns the path length; *n_occ, *count_sum (the
 * sum of the counts) and *m_star describe the match. */
static int32_t suffix_one(const int32_t *text, int64_t len_t, const int32_t *c, int64_t L,
                          int32_t m_min, int32_t m_max, int32_t K, double min_prob,
                          int32_t occ_cap, int64_t *occ, unsigned char *alive,
                          int32_t *path, int32_t *n_occ, int64_t *count_sum, int32_t *m_star)
{
    int32_t best = 0;
    for (int64_t e = len_t - 2; e >= 0; --e) {
        if (text[e + 1] < 0)
            continue;
        const int32_t m = suffix_match(text, e, c, L, m_max);
        if (m > best)
            best = m;
    }
    *n_occ = 0;
    *count_sum = 0;
    *m_star = 0;
    if (best < m_min || best == 0)
        return 0;
    int32_t n = 0;
    for (int64_t e = len_t - 2; e >= 0 && n < occ_cap; --e)
        if (text[e + 1] >= 0 && suffix_match(text, e, c, L, m_max) == best)
            occ[n++] = e;
    for (int32_t i = 0; i < n; ++i)
        alive[i] = 1;
    int32_t len = 0;
    int64_t sum = 0;
    for (int32_t j = 1; j <= K; ++j) {
        int32_t tok = -1;
        int64_t cnt_best = 0;
        for (int32_t i = 0; i < n; ++i) {
            if (!alive[i] || occ[i] + j >= len_t || text[occ[i] + j] < 0)
                continue;
            const int32_t t = text[occ[i] + j];
            int64_t cnt = 0;
            for (int32_t k = 0; k < n; ++k)
                if (alive[k] && occ[k] + j < len_t && text[occ[k] + j] == t)
                    ++cnt;
            if (cnt > cnt_best || (cnt == cnt_best && t < tok)) {
                cnt_best = cnt;
                tok = t;
            }
        }
        if (cnt_best == 0 || (double)cnt_best < min_prob * (double)n)
            break;
        path[len++] = tok;
        sum += cnt_best;
        for (int32_t i = 0; i < n; ++i)
            alive[i] = alive[i] && occ[i] + j < len_t && text[occ[i] + j] == tok;
    }
    *n_occ = n;
    *count_sum = sum;
    *m_star = best;
    return len;
}

void orc_suffix_propose(const int32_t *tokens, int64_t ctx_stride,
                        const int32_t *lengths, int32_t B,
                        const int32_t *history, int64_t H,
                        int32_t m_min, int32_t m_max, int32_t K, double min_prob,
                        int32_t occ_cap,
                        int32_t *proposal, int32_t *proposal_len, double *score,
                        int32_t *match_len, int32_t *source, uint32_t *flags)
{
    int64_t *occ = (int64_t *)malloc(sizeof(int64_t) * (size_t)(occ_cap > 0 ? occ_cap : 1));
    unsigned char *alive = (unsigned char *)malloc((size_t)(occ_cap > 0 ? occ_cap : 1));
    int32_t *path_c = (int32_t *)malloc(sizeof(int32_t) * (size_t)(K > 0 ? K : 1));
    int32_t *path_h = (int32_t *)malloc(sizeof(int32_t) * (size_t)(K > 0 ? K : 1));
    for (int32_t b = 0; b < B; ++b) {
        uint32_t fl = 0;
        const int32_t *c = tokens + (size_t)b * (size_t)ctx_stride;
        int64_t L = lengths[b];
        if (L < 0 || L > ctx_stride) {
            fl |= ORC_FLAG_BAD_LEN;
            L = 0;
        }
        int32_t nc, nh, mc, mh;
        int64_t sc, sh;
        const int32_t lc = suffix_one(c, L, c, L, m_min, m_max, K, min_prob, occ_cap, occ, alive,
                                      path_c, &nc, &sc, &mc);
        int32_t lh = 0;
        nh = 0;
        sh = 0;
        mh = 0;
        if (history && H > 0)
            lh = suffix_one(history, H, c, L, m_min, m_max, K, min_prob, occ_cap, occ, alive,
                            path_h, &nh, &sh, &mh);
        /* the higher expected number of accepted tokens, sc/nc against
         * sh/nh (exact in integers); the context wins ties */
        int which = -1;
        if (lc > 0 && (lh == 0 || sc * (int64_t)nh >= sh * (int64_t)nc))
            which = 0;
        else if (lh > 0)
            which = 1;
        int32_t *pr = proposal + (size_t)b * K;
        for (int32_t k = 0; k < K; ++k)
            pr[k] = -1;
        int32_t len = 0;
        double sco = 0.0;
        int32_t ml = 0;
        if (which == 0) {
            len = lc;
            for (int32_t k = 0; k < lc; ++k)
                pr[k] = path_c[k];
            sco = (double)sc / (double)nc;
            ml = mc;
        } else if (which == 1) {
            len = lh;
            for (int32_t k = 0; k < lh; ++k)
                pr[k] = path_h[k];
            sco = (double)sh / (double)nh;
            ml = mh;
        }
        proposal_len[b] = len;
        score[b] = sco;
        match_len[b] = ml;
        if (source)
            source[b] = which;
        if (flags)
            flags[b] = fl;
    }
    free(occ);
    free(alive);
    free(path_c);
    free(path_h);
}
