// rejection.hip -- rejection-sampling verification on gfx950 (Leviathan et
// al. / Chen et al., the rule [vLLM-03] "1. principle" cites for keeping the
// target distribution at T > 0).
//
// Kernel 1 (row statistics + accept scan).  One workgroup per (row,
// segment) over the K+1 target rows and K draft rows of every sequence
// streams the logits once with 16-byte loads and keeps, per thread, an
// online (max, sum of exp) pair: the max is taken per 8-element vector, the
// exp is fp32 (expf) relative to the running max, sums are fp64, and a new
// max rescales the fp64 sum with an fp64 exp.  Segments merge through an
// arrival counter; the last row of a sequence runs the accept scan:
// p_i(x_i) and q_i(x_i) with fp64 exp from the row max and normaliser, the
// test u_i < p/q in fp64, and the first rejection n.
//
// Kernel 2 (final sample).  The final token is drawn from one row pair per
// sequence: r = max(0, p_n - q_n) after a rejection (p_n when that sums to
// zero), or p_n when every draft was accepted.  B x C workgroups each take a
// chunk of the row pair, form r per element (fp32 exp, fp64 after), and
// publish the chunk's mass; the last chunk of a sequence finds the chunk
// where the running mass first exceeds u_K * S and scans it in token order
// for the token whose cumulative mass first exceeds it.
//
// Arrival counters only elect the workgroup that finishes a row, a sequence
// or a sequence's chunks; it resets the counter and clears the workspace
// slots it consumed, so the workspace is all-zero again after the call.

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
    unsigned len_flag = 0;
    const int len = p.draft_len ? clamp_len(p.draft_len[b], K, len_flag) : K;
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
    double Z = block_sum(rescale(z, m, M, p.inv_t_d));
    float Mr = M;

    __shared__ int s_last_row, s_last_seq;
    if (p.segs > 1) {
        if (threadIdx.x == 0) {
            p.partial[static_cast<int64_t>(row) * p.segs + seg] = SoftPartial{Z, M, 0};
            s_last_row = arrive(p.row_ctr + row) == static_cast<unsigned>(p.segs - 1);
        }
        __syncthreads();
        if (!s_last_row)
            return;
        if (threadIdx.x == 0) {
            reset_counter(p.row_ctr + row);
            SoftPartial *pp = p.partial + static_cast<int64_t>(row) * p.segs;
            Mr = -__builtin_inff();
            for (int s = 0; s < p.segs; ++s)
                Mr = fmaxf(Mr, pp[s].m);
            Z = 0.0;
            for (int s = 0; s < p.segs; ++s) {
                Z += rescale(pp[s].z, pp[s].m, Mr, p.inv_t_d);
                pp[s] = SoftPartial{0.0, 0.0f, 0};   // the workspace is left all-zero
            }
        }
    }
    if (threadIdx.x == 0) {
        p.rstat[row] = SoftPartial{Z, Mr, 0};
        s_last_seq = arrive(p.seq_ctr + b) == static_cast<unsigned>(rows_per_seq - 1);
    }
    __syncthreads();
    if (!s_last_seq)
        return;

    // ---- accept scan of sequence b (this workgroup finished its last row)
    acquire_agent();
    __shared__ int s_first_reject;
    __shared__ unsigned s_flags;
    if (threadIdx.x == 0) {
        reset_counter(p.seq_ctr + b);
        s_first_reject = len;
        s_flags = len_flag;
    }
    __syncthreads();
    const SoftPartial *rs = p.rstat + static_cast<int64_t>(b) * rows_per_seq;
    for (int k = threadIdx.x; k < K; k += kThreads) {
        const int x = p.draft[static_cast<int64_t>(b) * K + k];
        const bool valid = x >= 0 && x < p.V;
        double pk = 0.0, qk = 0.0;
        if (k < len && valid) {
            const E *tr = static_cast<const E *>(p.target) + (static_cast<int64_t>(b) * (K + 1) + k) * p.row_stride;
            const E *dr = static_cast<const E *>(p.draftl) + (static_cast<int64_t>(b) * K + k) * p.row_stride;
            const SoftPartial st = rs[k], sd = rs[K + 1 + k];
            pk = exp((static_cast<double>(Elem<E>::one(tr, x)) - static_cast<double>(st.m)) * p.inv_t_d) / st.z;
            qk = exp((static_cast<double>(Elem<E>::one(dr, x)) - static_cast<double>(sd.m)) * p.inv_t_d) / sd.z;
        }
        if (p.p_draft)
            p.p_draft[static_cast<int64_t>(b) * K + k] = static_cast<float>(pk);
        if (p.q_draft)
            p.q_draft[static_cast<int64_t>(b) * K + k] = static_cast<float>(qk);
        if (k < len) {
            if (!valid)
                atomicOr(&s_flags, SV_FLAG_DRAFT_OOR);
            const double ratio = !valid ? 0.0 : (qk > 0.0 ? pk / qk : __builtin_inf());
            const double uk = static_cast<double>(p.u[static_cast<int64_t>(b) * (K + 1) + k]);
            if (!(uk < ratio))
                atomicMin(&s_first_reject, k);
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const int n = s_first_reject;
        p.accepted[b] = n;
        p.seq_n[b] = n;
        if (p.flags)
            p.flags[b] = s_flags;
        if (p.stats) {
            stats_add(p.stats + 0, n);
            stats_add(p.stats + 1, len);
            stats_add(p.stats + 2, n + 1);
            for (int k = 0; k < n; ++k)
                stats_add(p.stats + 3 + k, 1);
        }
    }
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

template <typename E>
__global__ __launch_bounds__(kThreads) void k_rej_final(const RejectParams p)
{
    const int K = p.K;
    const int rows_per_seq = 2 * K + 1;
    const int b = blockIdx.x / p.nchunks;
    const int c = blockIdx.x - b * p.nchunks;
    unsigned unused = 0;
    const int len = p.draft_len ? clamp_len(p.draft_len[b], K, unused) : K;
    const int n = p.seq_n[b];
    const bool residual = n < len;

    ChunkRows<E> cr;
    const SoftPartial st = p.rstat[static_cast<int64_t>(b) * rows_per_seq + n];
    cr.pt = static_cast<const E *>(p.target) + (static_cast<int64_t>(b) * (K + 1) + n) * p.row_stride;
    cr.mt = st.m;
    cr.izt = 1.0 / st.z;
    cr.inv_t = p.inv_t;
    cr.pd = nullptr;
    cr.md = 0.0f;
    cr.izd = 0.0;
    if (residual) {
        const SoftPartial sd = p.rstat[static_cast<int64_t>(b) * rows_per_seq + K + 1 + n];
        cr.pd = static_cast<const E *>(p.draftl) + (static_cast<int64_t>(b) * K + n) * p.row_stride;
        cr.md = sd.m;
        cr.izd = 1.0 / sd.z;
    }

    // this thread's elements of chunk cc
    auto span = [&](int cc, int &v0, int &cnt) {
        v0 = cc * kRejChunk + threadIdx.x * kChunkPerThread;
        const int end = min(p.V, (cc + 1) * kRejChunk);
        cnt = max(0, min(kChunkPerThread, end - v0));
    };

    int v0, cnt;
    span(c, v0, cnt);
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

    __shared__ int s_last;
    if (threadIdx.x == 0) {
        p.cmass[static_cast<int64_t>(b) * p.nchunks + c] = ChunkMass{Rtot, Ptot};
        s_last = arrive(p.chunk_ctr + b) == static_cast<unsigned>(p.nchunks - 1);
    }
    __syncthreads();
    if (!s_last)
        return;

    // ---- this workgroup finished the last chunk of sequence b: draw y
    acquire_agent();
    __shared__ int s_cs, s_use_p, s_first, s_lastpos;
    __shared__ double s_before, s_thr;
    if (threadIdx.x == 0) {
        reset_counter(p.chunk_ctr + b);
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
        // every slot of this sequence has been consumed: clear it, so the
        // workspace is all-zero when the call ends
        for (int k = 0; k < p.nchunks; ++k)
            p.cmass[static_cast<int64_t>(b) * p.nchunks + k] = ChunkMass{0.0, 0.0};
        for (int k = 0; k < rows_per_seq; ++k)
            p.rstat[static_cast<int64_t>(b) * rows_per_seq + k] = SoftPartial{0.0, 0.0f, 0};
        p.seq_n[b] = 0;
        s_cs = cs;
        s_use_p = use_p;
        s_before = before;
        s_thr = thr;
        s_first = kIdxNone;
        s_lastpos = -1;
    }
    __syncthreads();
    const int cs = s_cs;
    const bool use_p = s_use_p != 0;
    span(cs, v0, cnt);
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
    hipLaunchKernelGGL(k_rej_final<E>, dim3(static_cast<unsigned>(g2)), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

} // namespace

hipError_t launch_rejection(const RejectParams &p, int dtype, hipStream_t s)
{
    return dtype == SV_BF16 ? launch_typed<uint16_t>(p, s) : launch_typed<float>(p, s);
}

} // namespace sv
