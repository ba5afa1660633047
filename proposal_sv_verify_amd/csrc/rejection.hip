// rejection.hip -- rejection-sampling verification on gfx950 (Leviathan et
// al. / Chen et al., the rule [vLLM-03] "1. principle" cites for keeping the
// target distribution at T > 0).
//
// Kernel 1 (row statistics).  One workgroup per (row, segment) over the
// K+1 target rows and K draft rows of every sequence streams the logits
// once with 16-byte loads and keeps, per thread, an online (max, sum of exp)
// pair: the max is taken per 8-element vector, the exp is fp32 (expf)
// relative to the running max, sums are fp64, and a new max rescales the
// fp64 sum with an fp64 exp.  Each segment writes (max, sum).
//
// Kernel 2 (accept scan + final-sample masses).  One workgroup per
// (sequence, chunk).  Wave 0 merges the segment statistics of the rows it
// needs, computes p_i(x_i) and q_i(x_i) with fp64 exp, tests u_i < p/q in
// fp64 and finds the first rejection n.  The final token is drawn from one
// row pair: r = max(0, p_n - q_n) after a rejection (p_n when that sums to
// zero), or p_n when every draft was accepted.  Each workgroup forms r
// over its chunk of the row pair (fp32 exp, fp64 after) and writes the
// chunk's masses.
//
// Kernel 3 (selection).  One workgroup per sequence finds the chunk where
// the running mass first exceeds u_K * S and scans it in token order for
// the token whose cumulative mass first exceeds it.
//
// Kernel boundaries order the phases; no workgroup waits for another.

#include "sv_device.hpp"
#include "sv_kernels.hpp"

namespace sv {
namespace {

constexpr int kChunkPerThread = kRejChunk / kThreads;   // contiguous elements per thread in kernel 2
static_assert(kChunkPerThread * kThreads == kRejChunk, "chunk must split evenly over the threads");

__device__ __forceinline__ float block_max(float x)
{
    __shared__ float s_m[kWaves];
    x = wave_max(x);
    if ((threadIdx.x & 63) == 0)
        s_m[threadIdx.x >> 6] = x;
    __syncthreads();
    float m = s_m[0];
    for (int k = 1; k < kWaves; ++k)
        m = fmaxf(m, s_m[k]);
    __syncthreads();
    return m;
}

__device__ __forceinline__ double block_sum(double x)
{
    __shared__ double s_s[kWaves];
    x = wave_sum(x);
    if ((threadIdx.x & 63) == 0)
        s_s[threadIdx.x >> 6] = x;
    __syncthreads();
    double s = 0.0;
    for (int k = 0; k < kWaves; ++k)
        s += s_s[k];
    __syncthreads();
    return s;
}

// sum_k z_k * exp((m_k - M) / T) over partials (m_k, z_k) with M = max m_k;
// partials with z_k == 0 saw no element.
__device__ __forceinline__ double rescale(double z, float m, float M, double inv_t_d)
{
    return z != 0.0 ? z * exp((static_cast<double>(m) - static_cast<double>(M)) * inv_t_d) : 0.0;
}

template <typename E>
__global__ __launch_bounds__(kThreads) void k_rej_stats(const RejectParams p)
{
    const int K = p.K;
    const int rows_per_seq = 2 * K + 1;
    const int wg = blockIdx.x;
    const int row = wg / p.segs;
    const int seg = wg - row * p.segs;
    const int b = row / rows_per_seq;
    const int r = row - b * rows_per_seq;
    unsigned unused = 0;
    const int len = p.draft_len ? clamp_len(p.draft_len[b], K, unused) : K;
    const bool is_target = r <= K;
    const int i = is_target ? r : r - (K + 1);
    const bool needed = is_target ? i <= len : i < len;

    float m = -__builtin_inff();
    double z = 0.0;
    if (needed) {
        const E *rp = is_target
                          ? static_cast<const E *>(p.target) + (static_cast<int64_t>(b) * (K + 1) + i) * p.row_stride
                          : static_cast<const E *>(p.draftl) + (static_cast<int64_t>(b) * K + i) * p.row_stride;
        const int lo = seg * p.seg_len;
        const int hi = min(p.V, lo + p.seg_len);
        const float inv_t = p.inv_t;
        const double inv_t_d = p.inv_t_d;
        for_each_in_segment<E, 4>(
            rp, lo, hi,
            [&](const float(&f)[Elem<E>::kPerVec], int) {
                constexpr int PV = Elem<E>::kPerVec;
                float vm = f[0];
#pragma unroll
                for (int j = 1; j < PV; ++j)
                    vm = fmaxf(vm, f[j]);
                if (vm > m) {
                    z = rescale(z, m, vm, inv_t_d);
                    m = vm;
                }
                float s = 0.0f;
#pragma unroll
                for (int j = 0; j < PV; ++j)
                    s += expf((f[j] - m) * inv_t);
                z += static_cast<double>(s);
            },
            [&](float x, int) {
                if (x > m) {
                    z = rescale(z, m, x, inv_t_d);
                    m = x;
                }
                z += static_cast<double>(expf((x - m) * inv_t));
            });
    }
    const float M = block_max(m);
    const double Z = block_sum(rescale(z, m, M, p.inv_t_d));
    if (threadIdx.x == 0)
        p.partial[static_cast<int64_t>(row) * p.segs + seg] = SoftPartial{Z, M, 0};
}

// Row maximum and normaliser from the segment partials (same order and
// arithmetic wherever it is called, so every caller gets identical values).
__device__ __forceinline__ void merged_stats(const RejectParams &p, int64_t row, float &M, double &Z)
{
    const SoftPartial *pp = p.partial + row * p.segs;
    M = -__builtin_inff();
    for (int s = 0; s < p.segs; ++s)
        M = fmaxf(M, pp[s].m);
    Z = 0.0;
    for (int s = 0; s < p.segs; ++s)
        Z += rescale(pp[s].z, pp[s].m, M, p.inv_t_d);
}

// This thread's elements [v0, v0 + cnt) of final-sample chunk cc.
__device__ __forceinline__ void chunk_span(const RejectParams &p, int cc, int &v0, int &cnt)
{
    v0 = cc * kRejChunk + threadIdx.x * kChunkPerThread;
    const int end = min(p.V, (cc + 1) * kRejChunk);
    cnt = max(0, min(kChunkPerThread, end - v0));
}

// Per-element masses of one thread's contiguous elements [v0, v0 + cnt):
// p_v = exp((l_v - M) / T) / Z (fp32 exp, fp64 after) and, after a
// rejection, r_v = max(0, p_v - q_v).
template <typename E>
struct ChunkRows {
    const E *pt;
    const E *pd;        // null when sampling the bonus
    float mt, md;
    double izt, izd;
    float inv_t;

    __device__ __forceinline__ void load(const E *row, int v0, int cnt, float (&f)[kChunkPerThread]) const
    {
        constexpr int PV = Elem<E>::kPerVec;
        const E *src = row + v0;
        if (cnt == kChunkPerThread && (reinterpret_cast<uintptr_t>(src) & 15u) == 0) {
            const u32x4 *vp = reinterpret_cast<const u32x4 *>(src);
#pragma unroll
            for (int q = 0; q < kChunkPerThread / PV; ++q) {
                float g[PV];
                Elem<E>::unpack(vp[q], g);
#pragma unroll
                for (int j = 0; j < PV; ++j)
                    f[q * PV + j] = g[j];
            }
        } else {
#pragma unroll
            for (int j = 0; j < kChunkPerThread; ++j)
                f[j] = j < cnt ? Elem<E>::one(src, j) : 0.0f;
        }
    }

    // p and r for every element; entries j >= cnt are zero
    __device__ __forceinline__ void values(int v0, int cnt, double (&pv)[kChunkPerThread],
                                           double (&rv)[kChunkPerThread]) const
    {
        float ft[kChunkPerThread];
        load(pt, v0, cnt, ft);
        float fd[kChunkPerThread];
        if (pd)
            load(pd, v0, cnt, fd);
#pragma unroll
        for (int j = 0; j < kChunkPerThread; ++j) {
            pv[j] = 0.0;
            rv[j] = 0.0;
            if (j < cnt) {
                const double a = static_cast<double>(expf((ft[j] - mt) * inv_t)) * izt;
                pv[j] = a;
                if (pd) {
                    const double d = a - static_cast<double>(expf((fd[j] - md) * inv_t)) * izd;
                    rv[j] = d > 0.0 ? d : 0.0;
                }
            }
        }
    }
};

// Kernel 2: one workgroup per (sequence, chunk).  Wave 0 runs the accept
// scan of its sequence (cheap, so every chunk redoes it rather than waiting
// for a separate launch): one lane per draft position computes p_k(x_k) and
// q_k(x_k) in fp64 from the merged row statistics, a ballot of the
// rejections gives the first one, n.  The workgroup then forms the final
// sample's masses over its chunk of row pair n.  Chunk 0 also writes the
// per-sequence outputs of the accept scan.
template <typename E>
__global__ __launch_bounds__(kThreads) void k_rej_chunks(const RejectParams p)
{
    const int K = p.K;
    const int rows_per_seq = 2 * K + 1;
    const int b = blockIdx.x / p.nchunks;
    const int c = blockIdx.x - b * p.nchunks;
    unsigned fl = 0;
    const int len = p.draft_len ? clamp_len(p.draft_len[b], K, fl) : K;
    const int64_t row0 = static_cast<int64_t>(b) * rows_per_seq;
    __shared__ SeqState s_seq;

    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int n = -1;
        bool oor = false;
        for (int base = 0; base < K; base += 64) {
            const int k = base + lane;
            double pk = 0.0, qk = 0.0;
            bool rejected = false;
            if (k < len) {
                const int x = p.draft[static_cast<int64_t>(b) * K + k];
                const bool valid = x >= 0 && x < p.V;
                oor |= !valid;
                double ratio = 0.0;
                if (valid) {
                    float Mt, Md;
                    double Zt, Zd;
                    merged_stats(p, row0 + k, Mt, Zt);
                    merged_stats(p, row0 + K + 1 + k, Md, Zd);
                    const E *tr = static_cast<const E *>(p.target) + (static_cast<int64_t>(b) * (K + 1) + k) * p.row_stride;
                    const E *dr = static_cast<const E *>(p.draftl) + (static_cast<int64_t>(b) * K + k) * p.row_stride;
                    pk = exp((static_cast<double>(Elem<E>::one(tr, x)) - static_cast<double>(Mt)) * p.inv_t_d) / Zt;
                    qk = exp((static_cast<double>(Elem<E>::one(dr, x)) - static_cast<double>(Md)) * p.inv_t_d) / Zd;
                    ratio = qk > 0.0 ? pk / qk : __builtin_inf();
                }
                const double uk = static_cast<double>(p.u[static_cast<int64_t>(b) * (K + 1) + k]);
                rejected = !(uk < ratio);
            }
            if (c == 0 && k < K) {
                if (p.p_draft)
                    p.p_draft[static_cast<int64_t>(b) * K + k] = static_cast<float>(pk);
                if (p.q_draft)
                    p.q_draft[static_cast<int64_t>(b) * K + k] = static_cast<float>(qk);
            }
            const unsigned long long rej = __ballot(rejected);
            if (n < 0 && rej)
                n = base + __builtin_ctzll(rej);
        }
        if (n < 0)
            n = len;
        if (__ballot(oor))
            fl |= SV_FLAG_DRAFT_OOR;
        if (lane == 0) {
            SeqState st{};
            st.n = n;
            merged_stats(p, row0 + n, st.mt, st.zt);
            if (n < len)
                merged_stats(p, row0 + K + 1 + n, st.md, st.zd);
            s_seq = st;
            if (c == 0) {
                p.seq[b] = st;
                p.accepted[b] = n;
                if (p.flags)
                    p.flags[b] = fl;
                if (p.stats) {
                    stats_add(p.stats + 0, n);
                    stats_add(p.stats + 1, len);
                    stats_add(p.stats + 2, n + 1);
                }
            }
        }
        if (c == 0 && p.stats)
            for (int k = lane; k < n; k += 64)
                stats_add(p.stats + 3 + k, 1);
    }
    __syncthreads();

    const SeqState st = s_seq;
    const int n = st.n;
    ChunkRows<E> cr;
    cr.pt = static_cast<const E *>(p.target) + (static_cast<int64_t>(b) * (K + 1) + n) * p.row_stride;
    cr.mt = st.mt;
    cr.izt = 1.0 / st.zt;
    cr.inv_t = p.inv_t;
    cr.pd = nullptr;
    cr.md = 0.0f;
    cr.izd = 0.0;
    if (n < len) {
        cr.pd = static_cast<const E *>(p.draftl) + (static_cast<int64_t>(b) * K + n) * p.row_stride;
        cr.md = st.md;
        cr.izd = 1.0 / st.zd;
    }
    int v0, cnt;
    chunk_span(p, c, v0, cnt);
    double pv[kChunkPerThread], rv[kChunkPerThread];
    cr.values(v0, cnt, pv, rv);
    double ps = 0.0, rsum = 0.0;
#pragma unroll
    for (int j = 0; j < kChunkPerThread; ++j) {
        ps += pv[j];
        rsum += rv[j];
    }
    const double Ptot = block_sum(ps);
    const double Rtot = block_sum(rsum);
    if (threadIdx.x == 0)
        p.cmass[static_cast<int64_t>(b) * p.nchunks + c] = ChunkMass{Rtot, Ptot};
}

// Kernel 3: one workgroup per sequence draws the final token y: the chunk
// where the running mass first exceeds u_K * S, then the token inside it,
// scanning in token order; writes the emitted tokens.
template <typename E>
__global__ __launch_bounds__(kThreads) void k_rej_select(const RejectParams p)
{
    const int K = p.K;
    const int b = blockIdx.x;
    unsigned unused = 0;
    const int len = p.draft_len ? clamp_len(p.draft_len[b], K, unused) : K;
    const SeqState st = p.seq[b];
    const int n = st.n;
    const bool residual = n < len;

    __shared__ int s_cs, s_use_p, s_first, s_lastpos;
    __shared__ double s_before, s_thr;
    if (threadIdx.x == 0) {
        const ChunkMass *cm = p.cmass + static_cast<int64_t>(b) * p.nchunks;
        double SR = 0.0, SP = 0.0;
        for (int k = 0; k < p.nchunks; ++k) {
            SR += cm[k].r;
            SP += cm[k].p;
        }
        const int use_p = !residual || SR == 0.0;
        const double S = use_p ? SP : SR;
        const double thr = static_cast<double>(p.u[static_cast<int64_t>(b) * (K + 1) + K]) * S;
        int cs = -1, lastpos = 0;
        double before = 0.0, run = 0.0, before_last = 0.0;
        for (int k = 0; k < p.nchunks; ++k) {
            const double X = use_p ? cm[k].p : cm[k].r;
            if (X > 0.0) {
                lastpos = k;
                before_last = run;
            }
            if (cs < 0 && run + X > thr) {
                cs = k;
                before = run;
            }
            run += X;
        }
        if (cs < 0) {           // rounding left u*S at or past the total
            cs = lastpos;
            before = before_last;
        }
        s_cs = cs;
        s_use_p = use_p;
        s_before = before;
        s_thr = thr;
        s_first = kIdxNone;
        s_lastpos = -1;
    }
    __syncthreads();

    ChunkRows<E> cr;
    cr.pt = static_cast<const E *>(p.target) + (static_cast<int64_t>(b) * (K + 1) + n) * p.row_stride;
    cr.mt = st.mt;
    cr.izt = 1.0 / st.zt;
    cr.inv_t = p.inv_t;
    cr.pd = nullptr;
    cr.md = 0.0f;
    cr.izd = 0.0;
    if (residual) {
        cr.pd = static_cast<const E *>(p.draftl) + (static_cast<int64_t>(b) * K + n) * p.row_stride;
        cr.md = st.md;
        cr.izd = 1.0 / st.zd;
    }
    const bool use_p = s_use_p != 0;
    int v0, cnt;
    chunk_span(p, s_cs, v0, cnt);
    double pv[kChunkPerThread], rv[kChunkPerThread];
    cr.values(v0, cnt, pv, rv);
    double own = 0.0;
#pragma unroll
    for (int j = 0; j < kChunkPerThread; ++j)
        own += use_p ? pv[j] : rv[j];
    double tot;
    const double incl = block_inclusive_scan(own, tot);
    double cum = s_before + (incl - own);
    const double thr = s_thr;
    int first = kIdxNone, lastpos = -1;
#pragma unroll
    for (int j = 0; j < kChunkPerThread; ++j) {
        const double x = use_p ? pv[j] : rv[j];
        cum += x;
        if (j < cnt && x > 0.0) {
            lastpos = v0 + j;
            if (first == kIdxNone && cum > thr)
                first = v0 + j;
        }
    }
    if (first != kIdxNone)
        atomicMin(&s_first, first);
    if (lastpos >= 0)
        atomicMax(&s_lastpos, lastpos);
    __syncthreads();
    if (threadIdx.x == 0) {
        const int y = s_first != kIdxNone ? s_first : s_lastpos;
        int *e = p.emitted + static_cast<int64_t>(b) * (K + 1);
        const int *d = p.draft + static_cast<int64_t>(b) * K;
        for (int k = 0; k <= K; ++k)
            e[k] = k < n ? d[k] : (k == n ? y : -1);
    }
}

template <typename E>
hipError_t launch_typed(const RejectParams &p, hipStream_t s)
{
    const int64_t g1 = static_cast<int64_t>(p.B) * (2 * p.K + 1) * p.segs;
    hipLaunchKernelGGL(k_rej_stats<E>, dim3(static_cast<unsigned>(g1)), dim3(kThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t g2 = static_cast<int64_t>(p.B) * p.nchunks;
    hipLaunchKernelGGL(k_rej_chunks<E>, dim3(static_cast<unsigned>(g2)), dim3(kThreads), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    hipLaunchKernelGGL(k_rej_select<E>, dim3(static_cast<unsigned>(p.B)), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

} // namespace

hipError_t launch_rejection(const RejectParams &p, int dtype, hipStream_t s)
{
    return dtype == SV_BF16 ? launch_typed<uint16_t>(p, s) : launch_typed<float>(p, s);
}

} // namespace sv
