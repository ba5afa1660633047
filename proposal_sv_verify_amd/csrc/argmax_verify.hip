// argmax_verify.hip -- greedy and tree verification on gfx950.
//
// One workgroup per (row, segment) streams its slice of the logits with
// 16-byte loads and reduces a (value, index) argmax with the total order
// "larger value, then lower token id".  When a row is cut into several
// segments, the last segment to finish (arrival counter) merges them.  The
// last row of a sequence to finish runs the per-sequence step:
//
//  greedy  ([Arctic] "inference pipeline optimisation"; [Handbook] "how it
//          works"; [vLLM-03] "1. principle"): accept the longest prefix of
//          drafts equal to the row argmaxes, then emit the argmax of the
//          first disagreeing (or last) row;
//  tree    ([Handbook] "Medusa"): accept node j when its parent is accepted
//          and its token equals the parent row's argmax; keep the deepest
//          accepted node (lowest id on ties), emit the path and the argmax
//          of the chosen node.
//
// No kernel waits on another workgroup: arrival counters only elect the
// workgroup that finishes a row or a sequence.  That workgroup resets the
// counter and clears every workspace slot it consumed, so the workspace is
// all-zero again when the kernel ends, whatever call used it before.

#include "sv_device.hpp"
#include "sv_kernels.hpp"

namespace sv {
namespace {

enum { kGreedy = 0, kTree = 1 };

// Sequential tree scan of one sequence, run by thread 0 of the finishing
// workgroup.  Shared arrays hold the row argmaxes, the chosen path and the
// per-node depth / acceptance.
__device__ void tree_finalize(const ArgVerifyParams &p, int b, int *s_t, int *s_depth,
                              unsigned char *s_acc, int *s_path, int &s_best, int &s_bestd)
{
    const int N = p.rows_per_seq;
    const int *par = p.parent + static_cast<int64_t>(b) * N;
    const int *tok = p.token + static_cast<int64_t>(b) * N;
    for (int j = threadIdx.x; j < N; j += kThreads) {
        s_t[j] = p.amax[static_cast<int64_t>(b) * N + j];
        if (p.amax_scratch)                  // the workspace is left all-zero
            p.amax[static_cast<int64_t>(b) * N + j] = 0;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned fl = 0;
        if (par[0] != -1)
            fl |= SV_FLAG_BAD_PARENT;
        s_acc[0] = 1;
        s_depth[0] = 0;
        int best = 0, bestd = 0;
        for (int j = 1; j < N; ++j) {
            const int pj = par[j];
            const int tj = tok[j];
            if (tj < 0 || tj >= p.V)
                fl |= SV_FLAG_DRAFT_OOR;
            if (pj < 0 || pj >= j) {
                fl |= SV_FLAG_BAD_PARENT;
                s_acc[j] = 0;
                s_depth[j] = 0;
                continue;
            }
            const unsigned char a = s_acc[pj] && tj == s_t[pj];
            const int d = s_depth[pj] + 1;
            s_acc[j] = a;
            s_depth[j] = d;
            if (a && d > bestd) {
                bestd = d;
                best = j;
            }
        }
        int cur = best;
        for (int d = bestd - 1; d >= 0; --d) {
            s_path[d] = cur;
            cur = par[cur];
        }
        s_best = best;
        s_bestd = bestd;
        p.accepted[b] = bestd;
        if (p.flags)
            p.flags[b] = fl;
    }
    __syncthreads();
    const int best = s_best, bestd = s_bestd;
    for (int j = threadIdx.x; j < N; j += kThreads) {
        const int64_t o = static_cast<int64_t>(b) * N + j;
        p.path[o] = j < bestd ? s_path[j] : -1;
        p.emitted[o] = j < bestd ? tok[s_path[j]] : (j == bestd ? s_t[best] : -1);
    }
}

// Greedy prefix scan of one sequence, run by thread 0 of the finishing
// workgroup.
__device__ void greedy_finalize(const ArgVerifyParams &p, int b)
{
    const int K = p.K;
    unsigned fl = 0;
    const int len = p.draft_len ? clamp_len(p.draft_len[b], K, fl) : K;
    const int *d = p.draft + static_cast<int64_t>(b) * K;
    const int *t = p.amax + static_cast<int64_t>(b) * (K + 1);
    int n = 0;
    bool agree = true;
    for (int i = 0; i < len; ++i) {
        const int x = d[i];
        if (x < 0 || x >= p.V)
            fl |= SV_FLAG_DRAFT_OOR;
        if (agree && x == t[i])
            ++n;
        else
            agree = false;
    }
    int *e = p.emitted + static_cast<int64_t>(b) * (K + 1);
    for (int i = 0; i <= K; ++i)
        e[i] = i < n ? d[i] : (i == n ? t[n] : -1);
    if (p.amax_scratch)                      // the workspace is left all-zero
        for (int i = 0; i <= K; ++i)
            p.amax[static_cast<int64_t>(b) * (K + 1) + i] = 0;
    p.accepted[b] = n;
    if (p.flags)
        p.flags[b] = fl;
    if (p.stats) {
        stats_add(p.stats + 0, n);
        stats_add(p.stats + 1, len);
        stats_add(p.stats + 2, n + 1);
        for (int i = 0; i < n; ++i)
            stats_add(p.stats + 3 + i, 1);
    }
}

template <typename E, int MODE>
__global__ __launch_bounds__(kThreads) void k_argmax_verify(const ArgVerifyParams p)
{
    const int wg = blockIdx.x;
    const int row = wg / p.segs;
    const int seg = wg - row * p.segs;
    const int b = row / p.rows_per_seq;
    const int i = row - b * p.rows_per_seq;

    // greedy rows past the draft length are not needed
    bool needed = true;
    if (MODE == kGreedy && p.draft_len != nullptr) {
        unsigned unused = 0;
        needed = i <= clamp_len(p.draft_len[b], p.K, unused);
    }

    float bv = -__builtin_inff();
    int bi = kIdxNone;
    if (needed) {
        const E *rp = static_cast<const E *>(p.logits) + static_cast<int64_t>(row) * p.row_stride;
        const int lo = seg * p.seg_len;
        const int hi = min(p.V, lo + p.seg_len);
        for_each_in_segment<E, 4>(
            rp, lo, hi,
            [&](const float(&f)[Elem<E>::kPerVec], int base) { arg_visit_vec(bv, bi, f, base); },
            [&](float x, int idx) {
                if (x > bv) {
                    bv = x;
                    bi = idx;
                }
            });
    }
    block_argmax(bv, bi);

    __shared__ int s_last_row, s_last_seq;
    if (p.segs > 1) {
        if (threadIdx.x == 0) {
            p.partial[static_cast<int64_t>(row) * p.segs + seg] = ArgPartial{bv, bi};
            s_last_row = arrive(p.row_ctr + row) == static_cast<unsigned>(p.segs - 1);
        }
        __syncthreads();
        if (!s_last_row)
            return;
        if (threadIdx.x == 0) {
            reset_counter(p.row_ctr + row);
            bv = -__builtin_inff();
            bi = kIdxNone;
            ArgPartial *pp = p.partial + static_cast<int64_t>(row) * p.segs;
            for (int s = 0; s < p.segs; ++s) {
                const ArgPartial q = pp[s];
                arg_combine(bv, bi, q.v, q.i);
                pp[s] = ArgPartial{0.0f, 0};    // the workspace is left all-zero
            }
        }
    }
    if (threadIdx.x == 0) {
        // all elements equal to -inf (or NaN) leave the sentinel: id 0 is then
        // the lowest id holding the maximum
        p.amax[row] = needed ? (bi == kIdxNone ? 0 : bi) : -1;
        s_last_seq = arrive(p.seq_ctr + b) == static_cast<unsigned>(p.rows_per_seq - 1);
    }
    __syncthreads();
    if (!s_last_seq)
        return;
    acquire_agent();
    if (threadIdx.x == 0)
        reset_counter(p.seq_ctr + b);

    if constexpr (MODE == kGreedy) {
        if (threadIdx.x == 0)
            greedy_finalize(p, b);
    } else {
        __shared__ int s_t[SV_MAX_TREE_NODES];
        __shared__ int s_depth[SV_MAX_TREE_NODES];
        __shared__ int s_path[SV_MAX_TREE_NODES];
        __shared__ unsigned char s_acc[SV_MAX_TREE_NODES];
        __shared__ int s_best, s_bestd;
        tree_finalize(p, b, s_t, s_depth, s_acc, s_path, s_best, s_bestd);
    }
}

template <int MODE>
hipError_t launch_argmax(const ArgVerifyParams &p, int dtype, hipStream_t s)
{
    const int64_t grid = static_cast<int64_t>(p.B) * p.rows_per_seq * p.segs;
    if (dtype == SV_BF16)
        hipLaunchKernelGGL((k_argmax_verify<uint16_t, MODE>), dim3(static_cast<unsigned>(grid)),
                           dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((k_argmax_verify<float, MODE>), dim3(static_cast<unsigned>(grid)),
                           dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

} // namespace

hipError_t launch_greedy(const ArgVerifyParams &p, int dtype, hipStream_t s)
{
    return launch_argmax<kGreedy>(p, dtype, s);
}

hipError_t launch_tree(const ArgVerifyParams &p, int dtype, hipStream_t s)
{
    return launch_argmax<kTree>(p, dtype, s);
}

} // namespace sv
