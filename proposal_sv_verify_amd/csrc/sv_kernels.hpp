// sv_kernels.hpp -- launch parameters and launchers of the libspecverify
// kernels (internal; the public interface is include/specverify.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

// Elements of one final-sample chunk in rejection sampling (16 per thread of
// a 256-thread workgroup).
constexpr int kRejChunk = 4096;

// Per-(row, segment) argmax partial.
struct ArgPartial {
    float v;
    int i;
};

// Per-(row, segment) softmax partial: Z relative to the segment's raw max M.
struct SoftPartial {
    double z;
    float m;
    int pad;
};

// Per-chunk residual masses of the final sample.
struct ChunkMass {
    double r;   // sum of max(0, p - q) over the chunk
    double p;   // sum of p over the chunk
};

// Greedy and tree verification: one argmax per row, then a per-sequence
// scan by the last workgroup that finishes a row of the sequence.
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
    int32_t *amax;          // [B * rows_per_seq]: argmax_out or workspace
    int32_t amax_scratch;   // amax lives in the workspace (cleared after use)
    uint32_t *flags;
    // workspace
    ArgPartial *partial;    // [rows * segs] (segs > 1)
    unsigned *row_ctr;      // [rows] (segs > 1)
    unsigned *seq_ctr;      // [B]
};

hipError_t launch_greedy(const ArgVerifyParams &p, int dtype, hipStream_t s);
hipError_t launch_tree(const ArgVerifyParams &p, int dtype, hipStream_t s);

// Rejection sampling.  Rows per sequence: K+1 target rows then K draft rows.
struct RejectParams {
    const void *target;
    const void *draftl;
    int64_t row_stride;
    int32_t B, K, V;
    int32_t segs, seg_len;
    int32_t nchunks;          // ceil(V / kRejChunk)
    float inv_t;
    double inv_t_d;
    const int32_t *draft;
    const int32_t *draft_len;
    const float *u;
    int32_t *accepted;
    int32_t *emitted;
    float *p_draft;
    float *q_draft;
    uint32_t *flags;
    int64_t *stats;
    // workspace
    SoftPartial *partial;     // [B*(2K+1)*segs] (segs > 1)
    SoftPartial *rstat;       // [B*(2K+1)] row max and normaliser
    unsigned *row_ctr;        // [B*(2K+1)] (segs > 1)
    unsigned *seq_ctr;        // [B]
    int32_t *seq_n;           // [B] accepted count for the final-sample kernel
    ChunkMass *cmass;         // [B*nchunks]
    unsigned *chunk_ctr;      // [B]
};

hipError_t launch_rejection(const RejectParams &p, int dtype, hipStream_t s);

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

} // namespace sv
