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
// m(e) >= n_min.
//
// kW waves work on one context (kW = 1 for many contexts, so that each
// wave's in-flight reads are few at its early exit; kW = 4 or 16 for fewer,
// so that a context is scanned that many tiles at a time: with 16 waves a
// 8192-token context is in flight in one round).  Wave `sub` scores the
// 256-position tiles t_top - sub, t_top - sub - kW, ... from the end of the
// context backwards; each tile comes with the 32 positions below it (the
// longest comparison's reach), through a ring of kDepth loads per lane, so
// kDepth - 1 tiles are in flight while one is scored.  A lane holds four
// consecutive candidate ends and tests their last token against the
// suffix's last token in registers; only the rare hits compare further,
// from the tile staged in the wave's LDS.  A wave stops once a full-length
// (n_max) match is known at or above its next tile, since nothing further
// back can beat it; the keys' maximum is the answer.

#include "sv_device.hpp"
#include "sv_kernels.hpp"

namespace sv {
namespace {

constexpr int kTile = 4 * 64;         // candidate end positions per tile (one wave, 4 per lane)
constexpr int kHalo = 32;             // positions staged below a tile (> the longest comparison)
constexpr int kDepth = 2;             // tiles per lane in the load ring (measured best: deeper
                                      // rings fetch more past each early exit)
constexpr int kEndBits = 26;          // key = (match length << 26) | end position
static_assert(SV_MAX_NGRAM < kHalo + 1, "the halo must cover the longest comparison");
static_assert((1 << kEndBits) >= SV_MAX_CONTEXT, "end positions must fit the key");

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Four tokens at positions pos .. pos+3 of a context row of `stride` ints
// (pos % 4 == 0), loaded unconditionally: positions outside the row are
// clamped into it, and the caller never uses them.  kVec: the row is
// 16-byte aligned and stride % 4 == 0.  kKeep: a load whose lines are read
// again soon allocates in the caches (the halo under a tile is the top of
// the tile the wave reads next); tiles stream past them.
template <bool kVec, bool kKeep = false>
__device__ __forceinline__ i32x4 load4(const int32_t *c, int pos, int stride)
{
    if constexpr (kVec && kKeep) {
        return *reinterpret_cast<const i32x4 *>(c + max(0, min(pos, stride - 4)));
    } else if constexpr (kVec) {
        return __builtin_nontemporal_load(
            reinterpret_cast<const i32x4 *>(c + max(0, min(pos, stride - 4))));
    } else {
        const int last = stride - 1;
        i32x4 r;
        r.x = c[max(0, min(pos, last))];
        r.y = c[max(0, min(pos + 1, last))];
        r.z = c[max(0, min(pos + 2, last))];
        r.w = c[max(0, min(pos + 3, last))];
        return r;
    }
}

template <bool kVec, int kW, int kWG>
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(8))) void k_ngram(const NgramParams p)
{
    constexpr int kWv = kWG / 64;                 // waves per workgroup
    static_assert(kWv % kW == 0, "whole contexts per workgroup");
    __shared__ int s_buf[kWv][kHalo + kTile];     // a wave's tile, halo below it
    __shared__ int s_suf[kWv][64];                // s_suf[j] = c[L-1-j] for j < n_max
    __shared__ int s_full[kWv / kW];              // highest tile with a full-length match
    __shared__ int s_key[kWv];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int sub = w % kW;
    const int slot = w / kW;
    const int b = blockIdx.x * (kWv / kW) + slot;
    const bool live = b < p.B;                    // uniform over the context's waves
    const int stride = static_cast<int>(p.ctx_stride);
    const int32_t *c = p.tokens + static_cast<int64_t>(live ? b : 0) * p.ctx_stride;
    int *buf = s_buf[w];
    int *sfx = s_suf[w];
    unsigned fl = 0;
    int L = live ? p.lengths[b] : 0;
    if (L < 0 || L > stride) {
        fl |= SV_FLAG_BAD_LEN;
        L = 0;
    }
    const int nmax = p.n_max, nmin = p.n_min;
    if (kW > 1) {
        if (threadIdx.x < kWv / kW)
            s_full[threadIdx.x] = -1;
        __syncthreads();
    }

    int best = 0;                                 // this lane's best key; 0 = no match
    const int e_hi = L - 2;                       // most recent candidate end
    const int e_lo = nmin - 1;                    // earliest end holding n_min tokens
    if (live && e_hi >= e_lo) {
        const int t_top = e_hi / kTile, t_bot = e_lo / kTile;
        // the suffix loads go first, so waiting for them drains nothing else
        const int suf = c[max(0, L - 1 - min(lane, nmax - 1))];
        const int s0 = c[L - 1];
        __builtin_amdgcn_sched_barrier(0);
        // ring slot u holds the i-th tile of this wave, i = u + kDepth * r;
        // lanes 0..7 also fetch the halo (the 32 positions below the tile)
        auto tile_of = [&](int i) { return t_top - sub - kW * i; };
        auto fetch = [&](int i, i32x4 &v, i32x4 &h) {
            const int t = max(tile_of(i), t_bot);
            v = load4<kVec>(c, t * kTile + 4 * lane, stride);
            h = load4<kVec, true>(c, t * kTile - kHalo + 4 * (lane & 7), stride);
        };
        i32x4 q[kDepth], hq[kDepth];
#pragma unroll
        for (int u = 0; u < kDepth; ++u)
            fetch(u, q[u], hq[u]);
        sfx[lane] = suf;                          // entries past n_max - 1 are not read
        // Every ring load is issued whether or not its step still scores a
        // tile (the scan ends only at the end of a round): with the same loads
        // on every path, the compiler's wait counts stay exact.  Past the
        // bottom they re-read the last tile.
        bool stop = false;
        for (int r = 0;; r += kDepth) {
#pragma unroll
            for (int u = 0; u < kDepth; ++u) {
                const int i = r + u;
                const int t = tile_of(i);
                int full = -1;
                if (kW > 1)
                    full = s_full[slot];
                const bool active = !stop && t >= t_bot && full < t;   // uniform over the wave
                const i32x4 v = q[u];
                if (active) {
                    buf[kHalo + 4 * lane + 0] = v.x;
                    buf[kHalo + 4 * lane + 1] = v.y;
                    buf[kHalo + 4 * lane + 2] = v.z;
                    buf[kHalo + 4 * lane + 3] = v.w;
                    if (lane < 8) {
                        const i32x4 h = hq[u];
                        buf[4 * lane + 0] = h.x;
                        buf[4 * lane + 1] = h.y;
                        buf[4 * lane + 2] = h.z;
                        buf[4 * lane + 3] = h.w;
                    }
                }
                fetch(active ? i + kDepth : i, q[u], hq[u]);
                if (active) {
                    const int lo = t * kTile;
                    const int tok[4] = {v.x, v.y, v.z, v.w};
                    unsigned hit = 0;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const int e = lo + 4 * lane + k;
                        if (tok[k] == s0 && e >= e_lo && e <= e_hi)
                            hit |= 1u << k;
                    }
                    if (__ballot(hit != 0)) {
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            if (hit & (1u << k)) {
                                const int e = lo + 4 * lane + k;
                                int m = 1;
                                while (m < nmax && e - m >= 0 &&
                                       buf[kHalo + 4 * lane + k - m] == sfx[m])
                                    ++m;
                                if (m >= nmin)
                                    best = max(best, (m << kEndBits) | e);
                            }
                        }
                    }
                    if (__ballot((best >> kEndBits) == nmax)) {
                        stop = true;
                        if (kW > 1 && lane == 0)
                            atomicMax(&s_full[slot], t);
                    }
                } else {
                    stop = true;
                }
            }
            if (stop)
                break;
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            best = max(best, __shfl_xor(best, off, 64));
    }
    if (kW > 1) {
        if (lane == 0)
            s_key[w] = best;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kW; ++k)
            best = max(best, s_key[slot * kW + k]);
        if (sub != 0 || !live)
            return;
    } else if (!live) {
        return;
    }

    const int n = best >> kEndBits;
    const int e = best & ((1 << kEndBits) - 1);
    const int m = n > 0 ? min(p.K, L - 1 - e) : 0;
    for (int k = lane; k < p.K; k += 64)
        p.proposal[static_cast<int64_t>(b) * p.K + k] = k < m ? c[e + 1 + k] : -1;
    if (lane == 0) {
        p.proposal_len[b] = m;
        if (p.match_n)
            p.match_n[b] = n;
        if (p.match_pos)
            p.match_pos[b] = n > 0 ? e - n + 1 : -1;
        if (p.flags)
            p.flags[b] = fl;
    }
}

template <bool kVec, int kW, int kWG>
hipError_t launch_w(const NgramParams &p, hipStream_t s)
{
    constexpr int kPerWg = kWG / 64 / kW;
    hipLaunchKernelGGL((k_ngram<kVec, kW, kWG>), dim3(static_cast<unsigned>((p.B + kPerWg - 1) / kPerWg)),
                       dim3(kWG), 0, s, p);
    return hipGetLastError();
}

} // namespace

hipError_t launch_ngram(const NgramParams &p, hipStream_t s)
{
    // one wave per context once the contexts alone fill the chip's wave slots
    // (256 CUs x 32) twice; four waves per context below that, and sixteen
    // (one 1024-thread workgroup) for a batch of at most 512 contexts
    const bool many = p.B >= 2 * 256 * 32, few = p.B <= 512;
    if (p.vec_ok)
        return many ? launch_w<true, 1, kThreads>(p, s)
                    : (few ? launch_w<true, 16, 1024>(p, s) : launch_w<true, 4, kThreads>(p, s));
    return many ? launch_w<false, 1, kThreads>(p, s)
                : (few ? launch_w<false, 16, 1024>(p, s) : launch_w<false, 4, kThreads>(p, s));
}

} // namespace sv
