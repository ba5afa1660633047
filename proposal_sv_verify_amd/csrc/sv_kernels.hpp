// sv_kernels.hpp -- launch parameters and launchers of the libspecverify
// kernels (internal; the public interface is include/specverify.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "specverify.h"

namespace sv {

// Elements of one final-sample chunk in rejection sampling (16 per thread of
// a 256-thread workgroup); each wave's quarter of a chunk (a sub-chunk of
// 1024 elements, SV_SAMPLE_BLOCK) publishes its own masses.
constexpr int kRejChunk = 4096;
constexpr int kRejSub = 1024;

// Most segments a rejection-sampling row is cut into (the merge of a row's
// segment partials loads them all at once).
constexpr int kMaxSegs = 16;

// Per-(row, segment) argmax partial.
struct ArgPartial {
    float v;
    int i;
};

// Per-(row, segment) softmax partial: z = sum exp((l - m) / T) over the
// segment against the reference m (at least the segment's largest logit's
// neighbourhood; see the statistics kernel).  lx: the logit at the row's
// draft token when a vocabulary-shard call captures it and the token lies in
// the segment, else NaN.  Same layout as the public sv_softmax_partial.
struct SoftPartial {
    double z;
    float m;
    float lx;
};

// Per-chunk masses of the final sample.
struct ChunkMass {
    double r;   // sum of max(0, p - q) over the chunk
    double p;   // sum of p over the chunk
};

// Per-sequence state handed from the accept scan to the final-sample
// kernels (same layout as the public sv_rejection_state).
struct SeqState {
    double zt, zd;   // normalisers of target row n and draft row n
    float mt, md;    // their references
    int n;           // accepted drafts
    int len;         // the sequence's draft length (n < len: residual sample)
};

// Greedy and tree verification: a streaming argmax per (row, segment), then
// one small per-sequence kernel.
struct ArgVerifyParams {
    const void *logits;
    int64_t row_stride;
    int32_t B, V;
    int32_t rows_per_seq;   // K+1 (greedy) or N (tree)
    int32_t segs, seg_len;  // each row is cut into segs segments of seg_len elements
    // greedy
    const int32_t *draft;
    const int32_t *draft_len;
    int32_t K;
    int64_t *stats;
    // tree
    const int32_t *parent;
    const int32_t *token;
    int32_t *path;
    // outputs
    int32_t *accepted;
    int32_t *emitted;
    int32_t *argmax_out;    // [B * rows_per_seq] or null
    uint32_t *flags;
    // workspace: the partial of (row, segment s) is partial[row * part_row_step
    // + s * part_seg_step]; segments of one row are merged in the total order
    const ArgPartial *partial_in;
    ArgPartial *partial;    // written by the row kernel: [rows * segs]
    int64_t part_row_step, part_seg_step;
    // per-row partials of a vocabulary shard
    int32_t v_offset;
    ArgPartial *shard_out;  // [rows]
};

hipError_t launch_greedy(const ArgVerifyParams &p, int dtype, hipStream_t s);
hipError_t launch_tree(const ArgVerifyParams &p, int dtype, hipStream_t s);
// the per-sequence kernels alone, on partials the caller supplies
hipError_t launch_greedy_scan(const ArgVerifyParams &p, hipStream_t s);
hipError_t launch_tree_scan(const ArgVerifyParams &p, hipStream_t s);
// per-row (max, argmax + v_offset) of a vocabulary shard into shard_out
hipError_t launch_argmax_shard(const ArgVerifyParams &p, int dtype, hipStream_t s);

// Rejection sampling.  Rows per sequence: K+1 target rows then K draft rows.
struct RejectParams {
    const void *target;
    const void *draftl;
    int64_t row_stride;
    int32_t B, K, V;
    int32_t segs, seg_len;
    int32_t nchunks;          // ceil(V / kRejChunk)
    int32_t nsub;             // ceil(V / kRejSub): sub-chunk masses per sequence
    int32_t vec_ok;           // both logit tensors 16-byte aligned, rows a whole
                              // number of 16-byte vectors and V a multiple of
                              // the elements per vector
    float inv_t;
    double inv_t_d;
    // log2(e) / T = split_c1 + split_c2 with split_c1 rounded to 16
    // significant bits, so that a bf16 logit (8 significant bits) times
    // split_c1 is exact in fp32; split_k2 = split_c2 * ln 2 in fp32.
    // split_ok: split_c1 lies far from fp32's range ends.
    float split_c1;
    float split_k2;
    int32_t split_ok;
    // the rows are fp32 probabilities (a row's distribution is the row over
    // its sum; no temperature) instead of logits
    int32_t probs;
    // vocabulary shards: V above is the shard's width and the logit pointers
    // address its columns; v_offset is its first global id.  capture_x: the
    // statistics kernel records each row's logit at its draft token.
    int32_t v_offset;
    int32_t capture_x;
    // accept scan: segment s of row r at partial[r * part_row_step + s *
    // part_seg_step]; v_full bounds valid draft ids (the full vocabulary)
    int64_t part_row_step, part_seg_step;
    int32_t v_full;
    // owner-shard sampling: masses[s * B + b] of shard s, shard_index = this one
    const ChunkMass *shard_mass;
    int32_t shard_count, shard_index;
    ChunkMass *mass_out;      // [B] the shard's totals
    // draft, draftl and draft_len always point at valid memory, so kernels can
    // load from them unconditionally: with K == 0 draft and draftl stand in
    // for nothing (any int array, the target logits), and without lengths
    // (has_len == 0) draft_len is any int array of B entries, ignored.
    const int32_t *draft;
    const int32_t *draft_len;
    int32_t has_len;
    const float *u;
    int32_t *accepted;
    int32_t *emitted;
    float *p_draft;
    float *q_draft;
    uint32_t *flags;
    int64_t *stats;
    // workspace
    SoftPartial *partial;     // [B*(2K+1)*segs]
    SeqState *seq;            // [B]
    ChunkMass *cmass;         // [B][nsub] masses per sub-chunk
};

hipError_t launch_rejection(const RejectParams &p, int dtype, hipStream_t s);
// vocabulary-shard pieces: statistics (then a per-row merge when rows are
// cut into segments), the accept scan on per-shard partials, the shard's
// final-sample masses, and the owner shard's sample
hipError_t launch_rejection_shard_stats(const RejectParams &p, int dtype, SoftPartial *out, hipStream_t s);
hipError_t launch_rejection_decide(const RejectParams &p, hipStream_t s);
hipError_t launch_rejection_shard_mass(const RejectParams &p, int dtype, hipStream_t s);
hipError_t launch_rejection_shard_sample(const RejectParams &p, int dtype, hipStream_t s);

struct NgramParams {
    const int32_t *tokens;
    int64_t ctx_stride;
    const int32_t *lengths;
    int32_t B, n_min, n_max, K;
    int32_t *proposal;
    int32_t *proposal_len;
    int32_t *match_n;
    int32_t *match_pos;
    uint32_t *flags;
    int32_t vec_ok;           // tokens base 16-byte aligned and ctx_stride % 4 == 0
};

hipError_t launch_ngram(const NgramParams &p, hipStream_t s);

// Suffix decoding.  A scan item is one wave over one chunk of candidate end
// positions of one text (the sequence's context, or the shared history) for
// one sequence; it leaves the chunk's longest match and that match's most
// recent occurrences.
constexpr int kSfxChunk = 4 * 256;      // candidate ends per scan item

struct SuffixScanRec {
    int best;                    // longest match in the chunk (0: none)
    int cnt;                     // occurrences recorded (at most SV_SUFFIX_OCC)
    int occ[SV_SUFFIX_OCC];      // their end positions, most recent first
};

struct SuffixParams {
    const int32_t *tokens;
    int64_t ctx_stride;
    const int32_t *lengths;
    int32_t B;
    const int32_t *history;   // a valid stand-in (tokens) when H == 0
    int64_t H;
    int32_t m_min, m_max, K;
    double min_prob;
    int32_t *proposal;        // [B][K], a stand-in when K == 0
    int32_t *proposal_len;
    double *score;
    int32_t *match_len;
    int32_t *source;
    uint32_t *flags;
    SuffixScanRec *rec;       // [B][nch_ctx + nch_hist]
    int32_t nch_ctx, nch_hist;
    int32_t vec_ok;           // 16-byte loads: aligned rows and history, ctx_stride % 4 == 0
};

hipError_t launch_suffix(const SuffixParams &p, hipStream_t s);

// a plain streaming read of `bytes` over about `wgs` workgroups
hipError_t launch_read_probe(const void *buf, int64_t bytes, uint32_t *out, int wgs, hipStream_t s);

} // namespace sv
