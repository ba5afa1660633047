// ngram.hip -- n-gram prompt-lookup proposal on gfx950 ([Handbook] "N-gram":
// take a suffix, find its most recent earlier occurrence, copy what
// followed; [vLLM-03] "2. draft methods": lookup lengths n_max down to
// n_min; "3-1": no match, no draft).
//
// For a candidate end position e (e <= L-2) let m(e) be the number of
// consecutive matches c[e-j] == c[L-1-j], j = 0, 1, ..., capped at n_max and
// at the start of the context.  The method's answer is the largest n with
// some m(e) >= n (n >= n_min), and for that n the largest such e -- i.e. the
// maximum of the key (min(m(e), n_max) << 26) | e over all e with
// m(e) >= n_min.  One workgroup per context scans 1024-position tiles from
// the end of the context backwards: the tile goes to LDS with the 32
// positions below it (the halo, which the prefetched next tile supplies),
// every thread scores four consecutive candidates against the suffix held
// in LDS, a workgroup max combines the keys, and the scan stops as soon as
// a full-length (n_max) match is known, since nothing further back can beat
// it.

#include "sv_device.hpp"
#include "sv_kernels.hpp"

namespace sv {
namespace {

constexpr int kTile = 4 * kThreads;   // candidate end positions per tile
constexpr int kHalo = 32;             // positions kept below a tile (>= SV_MAX_NGRAM)
constexpr int kEndBits = 26;          // key = (match length << 26) | end position
static_assert(SV_MAX_NGRAM < kHalo + 1, "halo must cover the longest lookup");
static_assert((1 << kEndBits) >= SV_MAX_CONTEXT, "end positions must fit the key");

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Four tokens at positions pos .. pos+3 (pos % 4 == 0); positions >= L read 0.
__device__ __forceinline__ i32x4 load4(const int32_t *c, int pos, int L, bool vec_ok)
{
    if (vec_ok && pos + 3 < L)
        return __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(c + pos));
    i32x4 r = {0, 0, 0, 0};
    if (pos < L)
        r.x = c[pos];
    if (pos + 1 < L)
        r.y = c[pos + 1];
    if (pos + 2 < L)
        r.z = c[pos + 2];
    if (pos + 3 < L)
        r.w = c[pos + 3];
    return r;
}

__global__ __launch_bounds__(kThreads) void k_ngram(const NgramParams p)
{
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int32_t *c = p.tokens + static_cast<int64_t>(b) * p.ctx_stride;
    const bool vec_ok = p.vec_ok != 0;
    unsigned fl = 0;
    int L = p.lengths[b];
    if (L < 0 || static_cast<int64_t>(L) > p.ctx_stride) {
        fl |= SV_FLAG_BAD_LEN;
        L = 0;
    }
    const int nmax = p.n_max, nmin = p.n_min;

    __shared__ int s_suf[kHalo];                 // s_suf[j] = c[L-1-j]
    __shared__ int s_buf[kHalo + kTile];         // positions [lo - kHalo, lo + kTile)
    if (tid < nmax && tid < L)
        s_suf[tid] = c[L - 1 - tid];

    int best = 0;                                // best key so far; 0 = no match
    const int e_hi = L - 2;                      // most recent candidate end
    const int e_lo = nmin - 1;                   // earliest end holding n_min tokens
    if (e_hi >= e_lo) {
        const int t_top = e_hi / kTile, t_bot = e_lo / kTile;
        i32x4 cur = load4(c, t_top * kTile + 4 * tid, L, vec_ok);
        i32x4 nxt = {0, 0, 0, 0};
        if (t_top > 0)
            nxt = load4(c, (t_top - 1) * kTile + 4 * tid, L, vec_ok);
        for (int t = t_top; t >= t_bot; --t) {
            const int lo = t * kTile;
            s_buf[kHalo + 4 * tid + 0] = cur.x;
            s_buf[kHalo + 4 * tid + 1] = cur.y;
            s_buf[kHalo + 4 * tid + 2] = cur.z;
            s_buf[kHalo + 4 * tid + 3] = cur.w;
            if (t > 0 && tid >= kThreads - kHalo / 4) {   // the halo: top of tile t-1
                const int h = 4 * (tid - (kThreads - kHalo / 4));
                s_buf[h + 0] = nxt.x;
                s_buf[h + 1] = nxt.y;
                s_buf[h + 2] = nxt.z;
                s_buf[h + 3] = nxt.w;
            }
            __syncthreads();
            cur = nxt;
            if (t - 2 >= 0 && t - 1 >= t_bot)    // prefetch tile t-2 (halo or scan)
                nxt = load4(c, (t - 2) * kTile + 4 * tid, L, vec_ok);

            int key = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int e = lo + 4 * tid + k;
                if (e < e_lo || e > e_hi)
                    continue;
                int m = 0;
                while (m < nmax && e - m >= 0 && s_buf[kHalo + (e - lo) - m] == s_suf[m])
                    ++m;
                if (m >= nmin)
                    key = max(key, (m << kEndBits) | e);
            }
            key = block_max_int(key);
            if ((key >> kEndBits) > (best >> kEndBits))
                best = key;                      // longer match; ties keep the later end
            if ((best >> kEndBits) == nmax)
                break;                           // uniform: every thread holds `best`
        }
    }

    const int n = best >> kEndBits;
    const int e = best & ((1 << kEndBits) - 1);
    const int m = n > 0 ? min(p.K, L - 1 - e) : 0;
    for (int k = tid; k < p.K; k += kThreads)
        p.proposal[static_cast<int64_t>(b) * p.K + k] = k < m ? c[e + 1 + k] : -1;
    if (tid == 0) {
        p.proposal_len[b] = m;
        if (p.match_n)
            p.match_n[b] = n;
        if (p.match_pos)
            p.match_pos[b] = n > 0 ? e - n + 1 : -1;
        if (p.flags)
            p.flags[b] = fl;
    }
}

} // namespace

hipError_t launch_ngram(const NgramParams &p, hipStream_t s)
{
    hipLaunchKernelGGL(k_ngram, dim3(static_cast<unsigned>(p.B)), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

} // namespace sv
