/*
 * specverify.h -- C ABI of libspecverify, the data-parallel hot path of
 * speculative decoding on AMD Instinct MI355X (gfx950):
 *
 *   sv_verify_greedy     greedy verification of K drafts per sequence
 *   sv_verify_rejection  rejection-sampling verification (target p, draft q)
 *   sv_verify_rejection_probs  the same on given probabilities
 *   sv_verify_rejection_noalloc  the same on the library's own device array
 *   sv_verify_tree       greedy verification of a candidate tree
 *   sv_ngram_propose     n-gram prompt-lookup drafting
 *   sv_suffix_propose    suffix-decoding drafting (context + shared history)
 *   sv_argmax_shard, sv_verify_*_partials, sv_rejection_shard_*
 *                        the verifiers on vocabulary-sharded logits
 *   sv_adaptive_*        adaptive speculation length (host side)
 *
 * Pages this follows (section names as the pages give them):
 *  [Arctic]   "Fastest Speculative Decoding in vLLM with Arctic Inference and
 *             Arctic Training" (Snowflake; Chinese repost): proposer / scorer
 *             / verifier split ("what is speculative decoding"), the worked
 *             step ("a simple example"), greedy verification by a custom
 *             kernel ("inference pipeline optimisation").
 *  [Handbook] LLM Inference Handbook, "speculative decoding": the
 *             draft-verify loop ("how it works"), candidate trees ("Medusa"),
 *             prompt lookup ("N-gram").
 *  [vLLM-03]  "vLLM features 03: speculative decoding" (ttlab): stop at the
 *             first wrong draft and substitute the target's token; rejection
 *             sampling at T > 0 ("1. principle"); prompt_lookup_min/max
 *             ("2. draft methods"); no match means no draft ("3-1").
 * The rejection rule is Leviathan et al. / Chen et al., which [vLLM-03]
 * cites: accept draft x with probability min(1, p(x)/q(x)); after a
 * rejection sample from max(0, p - q) normalised.
 *
 * Conventions for every call
 *  - All array arguments are DEVICE pointers (hipMalloc'd or equivalent),
 *    row-major, owned by the caller, which must keep them alive until the
 *    work enqueued on `stream` has completed.  The library allocates and
 *    frees nothing inside these calls.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every call only enqueues kernels and returns; outputs are valid after
 *    the stream reaches that point.  No call synchronises, and no kernel
 *    waits on another workgroup: each call is a short chain of kernels whose
 *    boundaries order its phases.
 *  - Logits are fp32 (SV_F32) or bf16 (SV_BF16, raw IEEE bf16 bits) with
 *    `row_stride` elements between consecutive rows (row_stride >= V); the
 *    base pointer must be aligned to the element size.
 *  - Scalars and pointers are validated on the host BEFORE anything is
 *    enqueued; on error the call returns a non-zero status, writes nothing
 *    and sv_last_error_message() explains.  Malformed DATA found on the
 *    device has a defined result and sets a bit in flags[b] (flags may be
 *    NULL): see SV_FLAG_*.
 *  - Workspaces are device scratch for per-row partial results; size one
 *    with the matching sv_*_workspace_bytes() (16-byte aligned).  They need
 *    no initialisation and their contents are undefined after a call,
 *    except where a call documents a part of them.
 *    Calls that share a workspace must be ordered on one stream; calls
 *    running concurrently need their own.
 *  - argmax ties resolve to the LOWEST token id (the numpy / torch rule);
 *    -0.0 and +0.0 compare equal.  -inf entries are allowed (a masked
 *    vocabulary); NaN and +inf are not.
 *  - The device must be gfx950 (else SV_ERR_UNSUPPORTED).
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_ABI_VERSION 1

/* status codes */
#define SV_OK 0
#define SV_ERR_INVALID_ARG 1   /* a scalar or a required pointer is invalid */
#define SV_ERR_UNSUPPORTED 2   /* not a gfx950 device, or a size above a documented limit */
#define SV_ERR_WORKSPACE 3     /* workspace missing, too small or misaligned */
#define SV_ERR_HIP 4           /* a HIP runtime call or launch failed */

/* logit element types */
#define SV_F32 0
#define SV_BF16 1

/* per-sequence data flags (flags[b], written by every call that takes flags) */
#define SV_FLAG_DRAFT_OOR 1u   /* a draft or tree-node token id outside [0, V):
                                  it never matches / is rejected */
#define SV_FLAG_BAD_LEN 2u     /* draft_len outside [0, K] (clamped to it), or an
                                  n-gram context length outside [0, ctx_stride]
                                  (treated as empty) */
#define SV_FLAG_BAD_PARENT 4u  /* tree parent[j] outside [0, j) for j >= 1 (node
                                  never accepted), or parent[0] != -1 (ignored) */

/* size limits (SV_ERR_UNSUPPORTED beyond them) */
#define SV_MAX_V (1 << 30)          /* vocabulary */
#define SV_MAX_TREE_NODES 1024      /* N of sv_verify_tree */
#define SV_MAX_NGRAM 31             /* n_max of sv_ngram_propose */
#define SV_MAX_CONTEXT (1 << 26)    /* n-gram context length / ctx_stride */
#define SV_SUFFIX_MAX_MATCH 32      /* m_max of sv_suffix_propose */
#define SV_SUFFIX_MAX_K 32          /* K of sv_suffix_propose */
#define SV_SUFFIX_OCC 256           /* occurrences counted per text */
#define SV_MAX_PROPOSAL 4096        /* K of sv_ngram_propose */
#define SV_MAX_DRAFTS 4096          /* K of the verifiers */

int sv_abi_version(void);
const char *sv_status_string(int status);
/* Detail of the last non-OK status returned on the calling thread. */
const char *sv_last_error_message(void);

/*
 * Launch tuning of the row-streaming kernels (process-wide; a value <= 0
 * restores the default).  Rows are cut into segments so that a call
 * launches about SV_TUNE_TARGET_WORKGROUPS workgroups (default 2048: eight
 * per compute unit) without segments shorter than SV_TUNE_MIN_SEGMENT_BYTES
 * (default 32768).  The rejection statistics kernel works per wave: about
 * 4 * SV_TUNE_TARGET_WORKGROUPS pieces, at most 16 per row, none shorter
 * than a quarter of SV_TUNE_MIN_SEGMENT_BYTES.
 * Thread safety: the setting is atomic, and every call (including the
 * sv_*_workspace_bytes queries) reads it once and plans from that copy, so
 * one call never mixes two settings.  Workspace needs follow the setting: a
 * workspace sized before a change may be too small after it, and the call
 * then returns SV_ERR_WORKSPACE (it never writes past workspace_bytes).
 * Results do not depend on the setting except within the rounding band of a
 * rejection-sampling tie (sums are associated by piece).
 */
#define SV_TUNE_TARGET_WORKGROUPS 1
#define SV_TUNE_MIN_SEGMENT_BYTES 2
int sv_set_tuning(int32_t key, int64_t value);

/*
 * sv_verify_greedy -- [Arctic] "inference pipeline optimisation" (accept
 * only drafts equal to the greedy choice), [Handbook] "how it works"
 * (longest agreeing prefix h, the target supplies token h+1), [vLLM-03]
 * "1. principle".  Per sequence b:
 *   t_i = argmax_v logits[b][i][v]            for i = 0 .. len
 *   n   = first i < len with draft[b][i] != t_i (else len)
 *   accepted[b] = n;  emitted[b] = draft[b][0..n) ++ [t_n], -1 padded
 * where len = draft_len[b] clamped to [0, K] (K when draft_len is NULL).
 *
 *   logits     [B][K+1][row_stride]  row i scores the token after draft i-1
 *   draft      [B][K] int32
 *   draft_len  [B] int32 or NULL
 *   accepted   [B] int32               (out)
 *   emitted    [B][K+1] int32          (out)
 *   argmax_out [B][K+1] int32 or NULL  (out; rows past len are not read
 *                                       and report -1)
 *   flags      [B] uint32 or NULL      (out)
 *   stats      int64[3 + K] or NULL    (accumulated, never reset:
 *              [0] accepted total, [1] drafted total, [2] emitted total,
 *              [3 + i] sequences whose draft i was accepted)
 * Limits: 1 <= B, 0 <= K <= SV_MAX_DRAFTS, 1 <= V <= SV_MAX_V.
 */
size_t sv_greedy_workspace_bytes(int32_t B, int32_t K, int32_t V);
int sv_verify_greedy(const void *logits, int32_t dtype, int64_t row_stride,
                     const int32_t *draft, const int32_t *draft_len,
                     int32_t B, int32_t K, int32_t V,
                     int32_t *accepted, int32_t *emitted, int32_t *argmax_out,
                     uint32_t *flags, int64_t *stats,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * sv_verify_rejection -- Leviathan / Chen rejection sampling ([vLLM-03]
 * "1. principle"; [Arctic] "what is speculative decoding").  Per sequence:
 *   p_i = softmax(target[b][i] / T), q_i = softmax(draft_logits[b][i] / T)
 *   for i < len: accept x_i = draft[b][i] iff u[b][i] < p_i(x_i) / q_i(x_i)
 *                (q_i(x_i) = 0 accepts; an id outside [0, V) is rejected);
 *                stop at the first rejection; n = number accepted
 *   final token y: n < len -> inverse-CDF sample, in increasing token id,
 *                  of r = max(0, p_n - q_n) with u[b][K] (r = p_n if it sums
 *                  to 0); n = len -> the same over r = p_n (the bonus).
 *   accepted[b] = n;  emitted[b] = x_0 .. x_{n-1}, y, -1 padded.
 *
 *   target_logits [B][K+1][row_stride], draft_logits [B][K][row_stride]
 *                 (same dtype and row_stride)
 *   draft      [B][K] int32, draft_len [B] int32 or NULL
 *   uniforms   [B][K+1] fp32 in [0, 1): K accept tests, then the final sample
 *   temperature  finite, > 0
 *   accepted [B], emitted [B][K+1] int32 (out)
 *   p_draft, q_draft [B][K] fp32 or NULL (out: p_i(x_i), q_i(x_i) for
 *              i < len with a valid id, else 0)
 *   flags, stats as for sv_verify_greedy.
 * Arithmetic: e^(l/T) per element in fp32 -- for bf16 logits the hardware
 * exp2 of the exact product l * c1 (c1 = log2(e)/T rounded to 16
 * significant bits) times (1 + l * k2), the first-order correction for the
 * rest of the constant; for fp32 logits a Cody-Waite exp (within 1.25 ulp)
 * -- summed in fp32 over the 8 (bf16) or 4 (fp32) elements of one 16-byte
 * vector and in fp64 across vectors; normalisers, p/q ratios, the residual,
 * the masses and the CDF in fp64; p_i(x_i) and q_i(x_i) with an fp64 exp
 * of the logit at the draft token.  The final sample's per-element
 * probabilities use the exp their normaliser was summed with.  Decisions
 * agree with an fp64 evaluation except within a rounding band of a tie: an
 * accept test with |u - p/q| < 1e-6, a final sample whose u*S lies within
 * SV_SAMPLE_BAND_SCALE * sqrt(sum p^2 + sum q^2) probability mass of an
 * end of the chosen token's CDF interval (q only after a rejection).  A
 * -inf logit has probability 0; every row needs at least one finite logit.
 * Workspace: sized by sv_rejection_workspace_bytes.  Once the call has
 * completed, the workspace begins with B * ceil(V / SV_SAMPLE_BLOCK)
 * sv_sample_mass records: for sequence b, record k holds the masses of r =
 * max(0, p_n - q_n) (0 after a full acceptance) and of p_n over tokens
 * [k * SV_SAMPLE_BLOCK, (k + 1) * SV_SAMPLE_BLOCK) of the row pair n the
 * final sample was drawn from -- the CDF the sample inverted, for callers
 * that audit the sampling.  The rest of the workspace is undefined.
 * Limits: 1 <= B, 0 <= K <= SV_MAX_DRAFTS, 1 <= V <= SV_MAX_V.
 */
#define SV_SAMPLE_BLOCK 1024             /* tokens per final-sample mass record */
#define SV_SAMPLE_BAND_SCALE 7.152557373046875e-07  /* 6 * 2^-23: final-sample tie band */

size_t sv_rejection_workspace_bytes(int32_t B, int32_t K, int32_t V);
int sv_verify_rejection(const void *target_logits, const void *draft_logits,
                        int32_t dtype, int64_t row_stride,
                        const int32_t *draft, const int32_t *draft_len,
                        const float *uniforms, float temperature,
                        int32_t B, int32_t K, int32_t V,
                        int32_t *accepted, int32_t *emitted,
                        float *p_draft, float *q_draft,
                        uint32_t *flags, int64_t *stats,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * sv_verify_rejection_probs -- sv_verify_rejection on given probabilities
 * (the interface takes the models' logits or their probabilities): the
 * rows are fp32, non-negative, each needed row with a positive finite sum;
 * a row's distribution is the row divided by its sum (rows need not be
 * normalised) and no temperature applies.  The same steps, layout,
 * outputs, workspace (sv_rejection_workspace_bytes) and limits as
 * sv_verify_rejection with dtype SV_F32; p_draft and q_draft report the
 * normalised values at the drafted ids.  (Greedy and tree verification
 * take probabilities as they are: the argmax is the same.)
 */
int sv_verify_rejection_probs(const float *target_probs, const float *draft_probs,
                              int64_t row_stride,
                              const int32_t *draft, const int32_t *draft_len,
                              const float *uniforms,
                              int32_t B, int32_t K, int32_t V,
                              int32_t *accepted, int32_t *emitted,
                              float *p_draft, float *q_draft,
                              uint32_t *flags, int64_t *stats,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * sv_verify_rejection_noalloc -- for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops or harnesses that
 * forbid hipMalloc): sv_verify_rejection with the same arguments, results
 * and limits, without a workspace argument.  Its workspace is a device
 * array of SV_NOALLOC_WORKSPACE_BYTES that the library holds on each GPU it
 * runs on (loaded with the library's code, kept until the process ends);
 * the call allocates and frees nothing.  A call whose workspace need
 * (sv_rejection_workspace_bytes) exceeds the array returns
 * SV_ERR_UNSUPPORTED before anything is enqueued.  Every call on one GPU
 * uses that GPU's one array, which keeps the last call's contents (its
 * final-sample masses, as sv_verify_rejection leaves in its workspace):
 * calls that can overlap on one GPU -- on different streams, or from other
 * host threads -- race and must be serialised by the caller.  Nothing in
 * the array needs clearing between calls: a call writes every byte it reads.
 */
#define SV_NOALLOC_WORKSPACE_BYTES (8u << 20)

int sv_verify_rejection_noalloc(const void *target_logits, const void *draft_logits,
                                int32_t dtype, int64_t row_stride,
                                const int32_t *draft, const int32_t *draft_len,
                                const float *uniforms, float temperature,
                                int32_t B, int32_t K, int32_t V,
                                int32_t *accepted, int32_t *emitted,
                                float *p_draft, float *q_draft,
                                uint32_t *flags, int64_t *stats, void *stream);

/*
 * sv_verify_tree -- [Handbook] "Medusa": candidate continuations form a
 * tree scored in one pass; the longest accepted candidate prefix is kept.
 *   t_j = argmax logits[b][j] (row j scores the children of node j);
 *   node 0 (root) is accepted; node j >= 1 is accepted iff its parent is
 *   accepted and token[b][j] == t_parent;
 *   j* = the deepest accepted node, lowest id on ties;
 *   accepted[b] = depth(j*); path[b] = node ids root -> j* (root excluded);
 *   emitted[b] = token[path] ++ [t_{j*}]; both -1 padded.
 *
 *   logits [B][N][row_stride]; parent, token [B][N] int32 (parent[b][0] = -1,
 *   parent[b][j] in [0, j); the root token is ignored)
 *   accepted [B], path [B][N], emitted [B][N] int32 (out)
 *   argmax_out [B][N] int32 or NULL (out), flags [B] or NULL (out)
 * Limits: 1 <= B, 1 <= N <= SV_MAX_TREE_NODES, 1 <= V <= SV_MAX_V.
 */
size_t sv_tree_workspace_bytes(int32_t B, int32_t N, int32_t V);
int sv_verify_tree(const void *logits, int32_t dtype, int64_t row_stride,
                   const int32_t *parent, const int32_t *token,
                   int32_t B, int32_t N, int32_t V,
                   int32_t *accepted, int32_t *path, int32_t *emitted,
                   int32_t *argmax_out, uint32_t *flags,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * Vocabulary-sharded verification (logits split by vocabulary range, as a
 * tensor-parallel output layer leaves them).  Greedy and tree verification
 * need only each row's maximum and its lowest id, and those merge across
 * shards in the same total order (larger value, then lower id), so each
 * shard reduces its columns to one partial per row and the verification
 * runs on the partials.  On one device this is a split of the streaming
 * pass; across devices the partials (8 bytes per row and shard) are what an
 * all-gather would exchange.
 *
 * sv_argmax_shard -- per-row partial of one shard:
 *   out[r].value = max_v logits[r][v], out[r].index = v_offset + the lowest
 *   v holding it, over v in [0, V) of the shard; a row with no value above
 *   -inf gives {-inf, SV_NO_INDEX}.
 *   logits [rows][row_stride] (the shard's columns; row_stride >= V)
 *   v_offset  the shard's first global token id (0 <= v_offset,
 *             v_offset + V <= SV_MAX_V)
 *   out [rows] sv_argmax_partial (out; 8-byte aligned)
 *   workspace as sized by sv_argmax_shard_workspace_bytes.
 *
 * sv_verify_greedy_partials / sv_verify_tree_partials -- sv_verify_greedy /
 * sv_verify_tree on shard partials: partials [P][rows] with rows = B*(K+1)
 * (greedy) or B*N (tree), shard p's row r at partials[p * rows + r]; V is
 * the full vocabulary (draft ids outside [0, V) never match).  The results
 * equal those of the unsharded call on the concatenated logits.  No
 * workspace.  Limits: 1 <= P <= SV_MAX_SHARDS, and those of the unsharded
 * calls.
 */
typedef struct {
    float value;
    int32_t index;
} sv_argmax_partial;

#define SV_NO_INDEX 0x7fffffff      /* index of a partial whose row is all -inf */
#define SV_MAX_SHARDS 4096          /* P of the *_partials calls */

size_t sv_argmax_shard_workspace_bytes(int32_t rows, int32_t V);
int sv_argmax_shard(const void *logits, int32_t dtype, int64_t row_stride,
                    int32_t rows, int32_t V, int32_t v_offset,
                    sv_argmax_partial *out,
                    void *workspace, size_t workspace_bytes, void *stream);
int sv_verify_greedy_partials(const sv_argmax_partial *partials, int32_t P,
                              const int32_t *draft, const int32_t *draft_len,
                              int32_t B, int32_t K, int32_t V,
                              int32_t *accepted, int32_t *emitted, int32_t *argmax_out,
                              uint32_t *flags, int64_t *stats, void *stream);
int sv_verify_tree_partials(const sv_argmax_partial *partials, int32_t P,
                            const int32_t *parent, const int32_t *token,
                            int32_t B, int32_t N, int32_t V,
                            int32_t *accepted, int32_t *path, int32_t *emitted,
                            int32_t *argmax_out, uint32_t *flags, void *stream);

/*
 * Vocabulary-sharded rejection sampling: sv_verify_rejection split into
 * four steps with three small exchanges between them ([Arctic] "inference
 * pipeline optimisation" reduces sharded logits per shard before gathering;
 * here the per-shard reductions are softmax statistics and sample masses).
 * Shard s holds the columns [v_offset_s, v_offset_s + V_s) of every target
 * and draft row; the shards must cover [0, V) once.
 *
 * 1. sv_rejection_shard_stats (per shard): for every row of the sequence's
 *    K+1 target and K draft rows (row order: target rows 0..K, then draft
 *    rows 0..K-1; out[b * (2K+1) + r]): z = sum over the shard's columns of
 *    exp((l - m) / T) against the reference m (a row with nothing above
 *    -inf, or a row past draft_len that the call skips, gives z = 0,
 *    m = -inf), and lx = the row's logit at its draft token x_i (target
 *    row i < K and draft row i) when x_i lies in the shard, else NaN.
 *    Arguments as for sv_verify_rejection, with V the shard's width; out
 *    [B][2K+1] sv_softmax_partial (8-byte aligned); workspace as sized by
 *    sv_rejection_shard_workspace_bytes(B, K, V).
 * 2. sv_verify_rejection_partials (once, on every shard's partials):
 *    partials [P][B][2K+1], shard p's row r at partials[p * B*(2K+1) + r];
 *    V the full vocabulary.  Merges each row's shards, then runs the accept
 *    test exactly as sv_verify_rejection: writes accepted, p_draft,
 *    q_draft, flags and stats as it does, and state[b] for the steps below.
 * 3. sv_rejection_shard_mass (per shard): out[b] = the shard's sum of
 *    r = max(0, p_n - q_n) (the residual; 0 when every draft was accepted)
 *    and of p_n, over its columns of row pair n = state[b].n.
 * 4. sv_rejection_shard_sample (per shard, the same workspace as its step
 *    3, unchanged since): masses [P][B] of every shard (shard p's at
 *    masses[p * B + b]).  S = the sum over shards in shard order of the
 *    residual masses (of p_n when every draft was accepted or the residual
 *    sums to 0); the shard where the running sum first exceeds u[b][K] * S
 *    (else the last shard with mass) owns the sample.  Only the owner's
 *    call writes emitted[b] (as sv_verify_rejection would), so after the
 *    calls of all P shards every sequence is written once.
 * Decisions and samples agree with sv_verify_rejection on the concatenated
 * logits except within the rounding band of a tie (sums are associated by
 * shard).  Limits: 1 <= P <= SV_MAX_REJECT_SHARDS, 0 <= v_offset,
 * v_offset + V <= SV_MAX_V, and those of sv_verify_rejection.
 */
typedef struct {
    double z;          /* sum of exp((l - m) / T) over the shard's columns */
    float m;           /* reference of z */
    float lx;          /* logit at the row's draft token, or NaN */
} sv_softmax_partial;

typedef struct {
    double zt, zd;     /* normalisers of target row n and draft row n */
    float mt, md;      /* their references: p_n(v) = exp((l - mt) / T) / zt */
    int32_t n;         /* accepted drafts */
    int32_t len;       /* draft length used (n < len: residual sample) */
} sv_rejection_state;

typedef struct {
    double r;          /* sum of max(0, p_n - q_n) */
    double p;          /* sum of p_n */
} sv_sample_mass;

#define SV_MAX_REJECT_SHARDS 16

size_t sv_rejection_shard_workspace_bytes(int32_t B, int32_t K, int32_t V);
int sv_rejection_shard_stats(const void *target_logits, const void *draft_logits,
                             int32_t dtype, int64_t row_stride,
                             const int32_t *draft, const int32_t *draft_len, float temperature,
                             int32_t B, int32_t K, int32_t V, int32_t v_offset,
                             sv_softmax_partial *out,
                             void *workspace, size_t workspace_bytes, void *stream);
int sv_verify_rejection_partials(const sv_softmax_partial *partials, int32_t P,
                                 const int32_t *draft, const int32_t *draft_len,
                                 const float *uniforms, float temperature,
                                 int32_t B, int32_t K, int32_t V,
                                 int32_t *accepted, float *p_draft, float *q_draft,
                                 uint32_t *flags, int64_t *stats,
                                 sv_rejection_state *state, void *stream);
int sv_rejection_shard_mass(const void *target_logits, const void *draft_logits,
                            int32_t dtype, int64_t row_stride,
                            const sv_rejection_state *state, float temperature,
                            int32_t B, int32_t K, int32_t V,
                            sv_sample_mass *out,
                            void *workspace, size_t workspace_bytes, void *stream);
int sv_rejection_shard_sample(const void *target_logits, const void *draft_logits,
                              int32_t dtype, int64_t row_stride,
                              const int32_t *draft, const float *uniforms,
                              const sv_rejection_state *state,
                              const sv_sample_mass *masses, int32_t P, int32_t shard,
                              float temperature, int32_t B, int32_t K, int32_t V, int32_t v_offset,
                              int32_t *emitted,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * sv_read_probe -- a measurement helper, not a step of the method: one
 * streaming read of buf[0 .. bytes) with the verifiers' 16-byte loads, the
 * reference their HBM rates are compared with.  buf: device memory,
 * 16-byte aligned, bytes a positive multiple of 16; out: one device uint32
 * (written only in a case that practically never occurs).  Enqueues one
 * kernel on stream.
 */
int sv_read_probe(const void *buf, size_t bytes, uint32_t *out, void *stream);

/*
 * Adaptive speculation length -- [Handbook] "adaptive" (the mechanism it
 * describes for SGLang): after each verification round, the mean number of
 * accepted draft tokens per sequence updates an exponential moving average,
 * ema <- (1 - beta) * ema + beta * accepted_mean, and the next round's
 * speculation length K is chosen from fixed tiers (the pages' default is
 * 1, 3, 7): the smallest tier of at least 2 * ema, else the largest.  Only
 * K changes, never the verification, so the output is unchanged.  Host code:
 * the state is a caller-owned host struct; nothing touches the GPU.  The
 * round's accepted_mean is, e.g., the growth of a verifier's stats[0]
 * divided by the number of sequences.
 *
 * sv_adaptive_init: tiers strictly increasing in [1, SV_MAX_DRAFTS],
 *   1 <= ntiers <= SV_MAX_TIERS, 0 < beta <= 1, ema0 finite and >= 0;
 *   sets state->k to the first round's length.
 * sv_adaptive_update: accepted_mean finite and >= 0; sets state->ema and
 *   state->k (the next round's length).
 * Both return SV_OK or SV_ERR_INVALID_ARG (state unchanged).
 */
#define SV_MAX_TIERS 16

typedef struct {
    double ema;                      /* moving average of accepted drafts per sequence */
    double beta;                     /* smoothing factor */
    int32_t ntiers;
    int32_t tiers[SV_MAX_TIERS];
    int32_t k;                       /* speculation length for the next round */
} sv_adaptive;

int sv_adaptive_init(sv_adaptive *state, const int32_t *tiers, int32_t ntiers, double beta,
                     double ema0);
int sv_adaptive_update(sv_adaptive *state, double accepted_mean);

/*
 * sv_suffix_propose -- [Arctic] "suffix decoding": the most recent tokens
 * are looked up in suffix trees of the current prompt and of earlier
 * outputs, candidate tokens are ranked by how often they followed (an
 * empirical probability), and the candidate sequence grows while it stays
 * likely.  Per sequence b, for each text T (its context c = tokens[b][0..L),
 * L = lengths[b]; and the shared history[0..H)):
 *   an occurrence is an end position e with a token after it (T[e+1] >= 0;
 *   negative entries separate history documents and never match);
 *   m(e) = the common suffix length of T[..e] and c, at most m_max;
 *   the pattern length m* = the largest m(e) (a text with m* < m_min has
 *   no candidates); the SV_SUFFIX_OCC most recent occurrences with
 *   m(e) = m* (n of them) are counted;
 *   step j = 1..K: among the occurrences that continue with the path so
 *   far, the most frequent next token x_j (lowest id on equal counts),
 *   count_j of them; the path stops before a step with count_j <
 *   min_prob * n (in fp64) or with nothing following;
 *   score = sum of count_j / n (the expected number of accepted tokens).
 * The text with the larger score gives the proposal (the context on equal
 * scores; compared exactly); no text with a path: proposal_len 0.
 *
 *   tokens [B][ctx_stride] int32, lengths [B] int32 (outside
 *   [0, ctx_stride]: flagged SV_FLAG_BAD_LEN, treated as 0)
 *   history [H] int32 or NULL (H = 0)
 *   proposal [B][K] (-1 padded), proposal_len [B] (out)
 *   score [B] double, match_len [B] (m* of the chosen text, 0 if none),
 *   source [B] (0 context, 1 history, -1 none), flags [B]: each NULL or out
 *   workspace as sized by sv_suffix_workspace_bytes(B, ctx_stride, H).
 * Limits: 1 <= B, 1 <= m_min <= m_max <= SV_SUFFIX_MAX_MATCH,
 *         0 <= K <= SV_SUFFIX_MAX_K, 0 <= min_prob <= 1,
 *         1 <= ctx_stride <= SV_MAX_CONTEXT, 0 <= H <= SV_MAX_CONTEXT.
 */
size_t sv_suffix_workspace_bytes(int32_t B, int64_t ctx_stride, int64_t H);
int sv_suffix_propose(const int32_t *tokens, int64_t ctx_stride, const int32_t *lengths, int32_t B,
                      const int32_t *history, int64_t H,
                      int32_t m_min, int32_t m_max, int32_t K, double min_prob,
                      int32_t *proposal, int32_t *proposal_len, double *score,
                      int32_t *match_len, int32_t *source, uint32_t *flags,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * sv_ngram_propose -- [Handbook] "N-gram" (take a suffix, find an earlier
 * occurrence, copy what followed), [vLLM-03] "2. draft methods"
 * (prompt_lookup_max down to prompt_lookup_min) and "3-1" (no match, no
 * draft).  Per context b of length L = lengths[b]:
 *   for n = n_max down to n_min: the most recent start s <= L-n-1 with
 *   c[s .. s+n) == c[L-n .. L); the first n with a match wins;
 *   proposal = c[s+n .. s+n+m), m = min(K, L-s-n);
 *   no match: proposal_len 0, match_n 0, match_pos -1.
 *
 *   tokens [B][ctx_stride] int32, lengths [B] int32
 *   proposal [B][K] int32 (out, -1 padded), proposal_len [B] int32 (out)
 *   match_n, match_pos [B] int32 or NULL (out), flags [B] or NULL (out)
 * Limits: 1 <= B, 1 <= n_min <= n_max <= SV_MAX_NGRAM,
 *         0 <= K <= SV_MAX_PROPOSAL, 1 <= ctx_stride <= SV_MAX_CONTEXT.
 * Needs no workspace.
 */
int sv_ngram_propose(const int32_t *tokens, int64_t ctx_stride,
                     const int32_t *lengths, int32_t B,
                     int32_t n_min, int32_t n_max, int32_t K,
                     int32_t *proposal, int32_t *proposal_len,
                     int32_t *match_n, int32_t *match_pos,
                     uint32_t *flags, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
