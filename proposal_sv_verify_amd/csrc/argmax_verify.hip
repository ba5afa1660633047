// argmax_verify.hip -- greedy and tree verification on gfx950.
//
// Kernel 1 streams the logits: one workgroup per (row, segment) reads its
// slice with 16-byte non-temporal loads and reduces a (value, index) argmax
// with the total order "larger value, then lower token id", writing one
// partial per segment.  Kernel 2 works per sequence: it merges the segment
// partials of each row and runs
//
//  greedy  ([Arctic] "inference pipeline optimisation"; [Handbook] "how it
//          works"; [vLLM-03] "1. principle"): one wave per sequence, one
//          lane per draft position; a ballot of the positions whose draft
//          differs from the row argmax gives the first disagreement n, and
//          the wave writes drafts 0..n-1 plus the argmax of row n;
//  tree    ([Handbook] "Medusa"): node j is accepted when its parent is
//          accepted and its token equals the parent row's argmax (pointer
//          jumping gives every node's path acceptance and depth in log N
//          rounds); the deepest accepted node (lowest id on ties) gives the
//          path and the bonus token.
//
// The kernel boundary orders the two phases: no workgroup ever waits for, or
// fences against, another one.

#include "sv_device.hpp"
#include "sv_kernels.hpp"

namespace sv {
namespace {

template <typename E>
__global__ __launch_bounds__(kThreads) void k_row_argmax(const ArgVerifyParams p)
{
    const int wg = blockIdx.x;
    const int row = wg / p.segs;
    const int seg = wg - row * p.segs;
    // greedy rows past the draft length are never read
    bool needed = true;
    if (p.draft_len != nullptr) {
        const int b = row / p.rows_per_seq;
        unsigned unused = 0;
        needed = row - b * p.rows_per_seq <= clamp_len(p.draft_len[b], p.K, unused);
    }
    float bv = -__builtin_inff();
    int bi = kIdxNone;
    if (needed) {
        const E *rp = static_cast<const E *>(p.logits) + static_cast<int64_t>(row) * p.row_stride;
        const int lo = seg * p.seg_len;
        const int hi = min(p.V, lo + p.seg_len);
        stream_segment<E, 6, kThreads>(
            rp, lo, hi, threadIdx.x,
            [&](const float(&f)[Elem<E>::kPerVec], int base) { arg_visit_vec(bv, bi, f, base); },
            [&](float x, int idx) {
                if (x > bv) {
                    bv = x;
                    bi = idx;
                }
            });
    }
    block_argmax(bv, bi);
    if (threadIdx.x == 0) {
        if (p.shard_out != nullptr && p.segs == 1)   // a shard's row in one segment: final already
            p.shard_out[row] = ArgPartial{bv, bi == kIdxNone ? kIdxNone : bi + p.v_offset};
        else
            p.partial[static_cast<int64_t>(row) * p.segs + seg] = ArgPartial{bv, bi};
    }
}

// Row argmax from its segment partials.  A row whose elements all compare
// false against -inf keeps the sentinel; id 0 is then the lowest id holding
// the maximum.
__device__ __forceinline__ int merged_argmax(const ArgVerifyParams &p, int64_t row, const ArgPartial &q0)
{
    const ArgPartial *pp = p.partial_in + row * p.part_row_step;
    float bv = -__builtin_inff();
    int bi = kIdxNone;
    arg_combine(bv, bi, q0.v, q0.i);
    for (int s = 1; s < p.segs; ++s) {
        const ArgPartial q = pp[s * p.part_seg_step];
        arg_combine(bv, bi, q.v, q.i);
    }
    return bi == kIdxNone ? 0 : bi;
}

// A shard's per-row partial: its segments merged, the index moved to the
// global vocabulary (a row with nothing above -inf keeps "none").
__global__ __launch_bounds__(kThreads) void k_shard_rows(const ArgVerifyParams p)
{
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (row >= static_cast<int64_t>(p.B) * p.rows_per_seq)
        return;
    const ArgPartial *pp = p.partial + row * p.segs;
    float bv = -__builtin_inff();
    int bi = kIdxNone;
    for (int s = 0; s < p.segs; ++s)
        arg_combine(bv, bi, pp[s].v, pp[s].i);
    p.shard_out[row] = ArgPartial{bv, bi == kIdxNone ? kIdxNone : bi + p.v_offset};
}

// One wave per sequence, one lane per position (in blocks of 64 positions).
__global__ __launch_bounds__(kThreads) void k_greedy_scan(const ArgVerifyParams p)
{
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (b >= p.B)
        return;
    const int K = p.K;
    unsigned fl = 0;
    const int len = p.draft_len ? clamp_len(p.draft_len[b], K, fl) : K;
    const int *d = p.draft + static_cast<int64_t>(b) * K;
    int *e = p.emitted + static_cast<int64_t>(b) * (K + 1);
    int n = -1;          // wave-uniform once known
    bool oor = false;
    for (int base = 0; base <= K; base += 64) {
        const int i = base + lane;
        // both loads first (indices clamped onto existing entries), so that
        // they travel in one round: the row's first partial and the draft
        const int64_t row = static_cast<int64_t>(b) * (K + 1) + min(i, K);
        const ArgPartial q0 = p.partial_in[row * p.part_row_step];
        const int xr = K > 0 ? d[max(0, min(i, K - 1))] : 0;
        int t = -1;
        if (i <= len)
            t = merged_argmax(p, row, q0);
        if (p.argmax_out && i <= K)
            p.argmax_out[static_cast<int64_t>(b) * (K + 1) + i] = t;
        const int x = i < len ? xr : 0;
        if (i < len && (x < 0 || x >= p.V))
            oor = true;
        const unsigned long long mism = __ballot(i < len && x != t);
        int here = -1;
        if (n < 0) {
            if (mism)
                here = base + __builtin_ctzll(mism);
            else if (len < base + 64)
                here = len;          // every draft agreed: the bonus row is len
        }
        if (i <= K) {
            int v;
            if (n >= 0)
                v = -1;              // decided in an earlier block
            else if (here < 0)
                v = x;               // no disagreement up to the end of this block
            else
                v = i < here ? x : (i == here ? t : -1);
            e[i] = v;
        }
        if (n < 0)
            n = here;
    }
    if (__ballot(oor))
        fl |= SV_FLAG_DRAFT_OOR;
    if (lane == 0) {
        p.accepted[b] = n;
        if (p.flags)
            p.flags[b] = fl;
        if (p.stats) {
            stats_add(p.stats + 0, n);
            stats_add(p.stats + 1, len);
            stats_add(p.stats + 2, n + 1);
        }
    }
    if (p.stats)
        for (int i = lane; i < n; i += 64)
            stats_add(p.stats + 3 + i, 1);
}

// One workgroup per tree, all in LDS.  Acceptance and depth are prefix
// quantities along the path to the root, computed for every node at once by
// pointer jumping: node j starts with its parent as "up", ok(j) = its own
// edge test, dep(j) = 1; each round folds in the values at up(j) and jumps
// up to up(up(j)), so after ceil(log2 N) rounds ok(j) is the acceptance of
// the whole path and dep(j) its depth.  The chosen node is the maximum of
// (depth, -id) over accepted nodes; one thread then walks its path.
__global__ __launch_bounds__(kThreads) void k_tree_scan(const ArgVerifyParams p)
{
    constexpr int kPer = (SV_MAX_TREE_NODES + kThreads - 1) / kThreads;
    __shared__ int s_t[SV_MAX_TREE_NODES];
    __shared__ int s_par[SV_MAX_TREE_NODES];
    __shared__ int s_tok[SV_MAX_TREE_NODES];
    __shared__ int s_up[SV_MAX_TREE_NODES];
    __shared__ int s_dep[SV_MAX_TREE_NODES];
    __shared__ unsigned char s_ok[SV_MAX_TREE_NODES];
    __shared__ int s_path[SV_MAX_TREE_NODES];
    __shared__ unsigned s_fl;
    const int b = blockIdx.x;
    const int N = p.rows_per_seq;
    if (threadIdx.x == 0)
        s_fl = 0;
    for (int j = threadIdx.x; j < N; j += kThreads) {
        const int64_t o = static_cast<int64_t>(b) * N + j;
        // the three loads first, so that they travel in one round
        const ArgPartial q0 = p.partial_in[o * p.part_row_step];
        const int par = p.parent[o];
        const int tok = p.token[o];
        __builtin_amdgcn_sched_barrier(0);
        const int t = merged_argmax(p, o, q0);
        s_t[j] = t;
        s_par[j] = par;
        s_tok[j] = tok;
        if (p.argmax_out)
            p.argmax_out[o] = t;
    }
    __syncthreads();
    unsigned fl = 0;
    for (int j = threadIdx.x; j < N; j += kThreads) {
        const int pj = s_par[j];
        int up = 0, dep = 0;
        unsigned char ok = 1;
        if (j == 0) {
            if (pj != -1)
                fl |= SV_FLAG_BAD_PARENT;
        } else {
            const int tj = s_tok[j];
            if (tj < 0 || tj >= p.V)
                fl |= SV_FLAG_DRAFT_OOR;
            if (pj < 0 || pj >= j) {
                fl |= SV_FLAG_BAD_PARENT;
                ok = 0;                       // never accepted; depth unused
            } else {
                up = pj;
                dep = 1;
                ok = tj == s_t[pj];
            }
        }
        s_up[j] = up;
        s_dep[j] = dep;
        s_ok[j] = ok;
    }
    if (fl)
        atomicOr(&s_fl, fl);
    __syncthreads();
    for (int span = 1; span < N; span <<= 1) {
        int nup[kPer], ndep[kPer];
        unsigned char nok[kPer];
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int j = threadIdx.x + q * kThreads;
            if (j < N) {
                const int u = s_up[j];
                nup[q] = s_up[u];
                ndep[q] = s_dep[j] + s_dep[u];
                nok[q] = s_ok[j] & s_ok[u];
            }
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int j = threadIdx.x + q * kThreads;
            if (j < N) {
                s_up[j] = nup[q];
                s_dep[j] = ndep[q];
                s_ok[j] = nok[q];
            }
        }
        __syncthreads();
    }
    // chosen node: deepest accepted, lowest id on ties (the root always qualifies)
    int key = 0;
    for (int j = threadIdx.x; j < N; j += kThreads)
        if (s_ok[j])
            key = max(key, s_dep[j] * 2 * SV_MAX_TREE_NODES + (2 * SV_MAX_TREE_NODES - 1 - j));
    key = block_max_int(key);
    const int bestd = key / (2 * SV_MAX_TREE_NODES);
    const int best = 2 * SV_MAX_TREE_NODES - 1 - (key - bestd * 2 * SV_MAX_TREE_NODES);
    if (threadIdx.x == 0) {
        int cur = best;
        for (int dd = bestd - 1; dd >= 0; --dd) {
            s_path[dd] = cur;
            cur = s_par[cur];
        }
        p.accepted[b] = bestd;
        if (p.flags)
            p.flags[b] = s_fl;
    }
    __syncthreads();
    for (int j = threadIdx.x; j < N; j += kThreads) {
        const int64_t o = static_cast<int64_t>(b) * N + j;
        p.path[o] = j < bestd ? s_path[j] : -1;
        p.emitted[o] = j < bestd ? s_tok[s_path[j]] : (j == bestd ? s_t[best] : -1);
    }
}

hipError_t launch_rows(const ArgVerifyParams &p, int dtype, hipStream_t s)
{
    const int64_t grid = static_cast<int64_t>(p.B) * p.rows_per_seq * p.segs;
    if (dtype == SV_BF16)
        hipLaunchKernelGGL(k_row_argmax<uint16_t>, dim3(static_cast<unsigned>(grid)), dim3(kThreads),
                           0, s, p);
    else
        hipLaunchKernelGGL(k_row_argmax<float>, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                           s, p);
    return hipGetLastError();
}

} // namespace

hipError_t launch_greedy_scan(const ArgVerifyParams &p, hipStream_t s)
{
    hipLaunchKernelGGL(k_greedy_scan, dim3(static_cast<unsigned>((p.B + kWaves - 1) / kWaves)),
                       dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_tree_scan(const ArgVerifyParams &p, hipStream_t s)
{
    hipLaunchKernelGGL(k_tree_scan, dim3(static_cast<unsigned>(p.B)), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_greedy(const ArgVerifyParams &p, int dtype, hipStream_t s)
{
    hipError_t e = launch_rows(p, dtype, s);
    if (e != hipSuccess)
        return e;
    ArgVerifyParams q = p;
    q.partial_in = p.partial;
    q.part_row_step = p.segs;
    q.part_seg_step = 1;
    return launch_greedy_scan(q, s);
}

hipError_t launch_tree(const ArgVerifyParams &p, int dtype, hipStream_t s)
{
    ArgVerifyParams q = p;
    q.draft_len = nullptr;          // every node row is needed
    hipError_t e = launch_rows(q, dtype, s);
    if (e != hipSuccess)
        return e;
    q.partial_in = p.partial;
    q.part_row_step = p.segs;
    q.part_seg_step = 1;
    return launch_tree_scan(q, s);
}

hipError_t launch_argmax_shard(const ArgVerifyParams &p, int dtype, hipStream_t s)
{
    ArgVerifyParams q = p;
    q.draft_len = nullptr;          // every row is needed
    hipError_t e = launch_rows(q, dtype, s);
    if (e != hipSuccess || p.segs == 1)
        return e;                   // one segment per row: the row kernel wrote shard_out
    const int64_t rows = static_cast<int64_t>(p.B) * p.rows_per_seq;
    hipLaunchKernelGGL(k_shard_rows, dim3(static_cast<unsigned>((rows + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, s, q);
    return hipGetLastError();
}

} // namespace sv
