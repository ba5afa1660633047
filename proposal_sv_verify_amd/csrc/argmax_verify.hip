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
//          accepted and its token equals the parent row's argmax; the
//          deepest accepted node (lowest id on ties) gives the path and the
//          bonus token.
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
    if (threadIdx.x == 0)
        p.partial[static_cast<int64_t>(row) * p.segs + seg] = ArgPartial{bv, bi};
}

// Row argmax from its segment partials.  A row whose elements all compare
// false against -inf keeps the sentinel; id 0 is then the lowest id holding
// the maximum.
__device__ __forceinline__ int merged_argmax(const ArgVerifyParams &p, int64_t row)
{
    const ArgPartial *pp = p.partial + row * p.segs;
    float bv = -__builtin_inff();
    int bi = kIdxNone;
    for (int s = 0; s < p.segs; ++s) {
        const ArgPartial q = pp[s];
        arg_combine(bv, bi, q.v, q.i);
    }
    return bi == kIdxNone ? 0 : bi;
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
        int t = -1;
        if (i <= len)
            t = merged_argmax(p, static_cast<int64_t>(b) * (K + 1) + i);
        if (p.argmax_out && i <= K)
            p.argmax_out[static_cast<int64_t>(b) * (K + 1) + i] = t;
        const int x = i < len ? d[i] : 0;
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

// One workgroup per tree; thread 0 walks the nodes in id order (parents
// precede children), the workgroup writes the outputs.
__global__ __launch_bounds__(kThreads) void k_tree_scan(const ArgVerifyParams p)
{
    __shared__ int s_t[SV_MAX_TREE_NODES];
    __shared__ int s_depth[SV_MAX_TREE_NODES];
    __shared__ int s_path[SV_MAX_TREE_NODES];
    __shared__ unsigned char s_acc[SV_MAX_TREE_NODES];
    __shared__ int s_best, s_bestd;
    const int b = blockIdx.x;
    const int N = p.rows_per_seq;
    const int *par = p.parent + static_cast<int64_t>(b) * N;
    const int *tok = p.token + static_cast<int64_t>(b) * N;
    for (int j = threadIdx.x; j < N; j += kThreads) {
        const int t = merged_argmax(p, static_cast<int64_t>(b) * N + j);
        s_t[j] = t;
        if (p.argmax_out)
            p.argmax_out[static_cast<int64_t>(b) * N + j] = t;
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
            const int dj = s_depth[pj] + 1;
            s_acc[j] = a;
            s_depth[j] = dj;
            if (a && dj > bestd) {
                bestd = dj;
                best = j;
            }
        }
        int cur = best;
        for (int dd = bestd - 1; dd >= 0; --dd) {
            s_path[dd] = cur;
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

hipError_t launch_greedy(const ArgVerifyParams &p, int dtype, hipStream_t s)
{
    hipError_t e = launch_rows(p, dtype, s);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(k_greedy_scan, dim3(static_cast<unsigned>((p.B + kWaves - 1) / kWaves)),
                       dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_tree(const ArgVerifyParams &p, int dtype, hipStream_t s)
{
    ArgVerifyParams q = p;
    q.draft_len = nullptr;          // every node row is needed
    hipError_t e = launch_rows(q, dtype, s);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(k_tree_scan, dim3(static_cast<unsigned>(p.B)), dim3(kThreads), 0, s, q);
    return hipGetLastError();
}

} // namespace sv
