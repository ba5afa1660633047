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
// A scan: wave by wave, 256-position tiles are read from the end of the
// context backwards, each with the 32 positions below it (the longest
// comparison's reach), through a ring of kDepth loads per lane, so kDepth - 1
// tiles are in flight while one is scored.  A lane holds four consecutive
// candidate ends and tests their last token against the suffix's last token
// in registers; only the rare hits compare further, from the tile staged in
// the wave's LDS.  Once a full-length (n_max) match is known at some tile,
// no tile below it can beat it, so those are skipped; the keys' maximum is
// the answer.
//
// Two kernels share that scan:
// - k_ngram, for up to 16383 contexts: kW waves per context (16, one
//   1024-thread workgroup, for at most 512 contexts, so that a context is
//   in flight 16 tiles at a time; else 4), wave `sub` taking the tiles
//   t_top - sub, t_top - sub - kW, ...
// - k_ngram_groups, for 16384 contexts and more: one round of 1024-thread
//   workgroups (two per CU), each owning 32 contexts.  A context's tiles
//   are cut into groups of 16 and the workgroup's 16 waves take groups
//   from an LDS counter, breadth first (every context's top group, then
//   every second group, ...).  Within a group a tile is scored one step
//   after it is staged: the next tile down, staged meanwhile, supplies its
//   halo, so only the group's bottom tile needs a halo load of its own.  Measured on 16384 contexts of 8192 tokens,
//   one wave per context left half the chip's wave slots idle in the
//   second half of the call: a workgroup's slots are only refilled once
//   all of its contexts have ended, and a context scanned to the start
//   takes 32 tiles in series.  With groups every slot stays busy until
//   the workgroups start to finish.

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

constexpr int kGroupWaves = 16;            // waves per workgroup of k_ngram_groups
constexpr int kGroupCtx = 32;              // contexts per workgroup
constexpr int kGroupTiles = 16;            // tiles per group

template <bool kVec>
__global__ __launch_bounds__(kGroupWaves * 64) __attribute__((amdgpu_waves_per_eu(8))) void k_ngram_groups(const NgramParams p)
{
    __shared__ int s_buf[kGroupWaves][2][kHalo + kTile];   // two tiles per wave, each with its halo
    __shared__ int s_suf[kGroupCtx][64];          // s_suf[j][i] = c[L-1-i] for i < n_max
    __shared__ int s_len[kGroupCtx];              // length (0 if invalid), -1 past the batch
    __shared__ int s_full[kGroupCtx];             // highest tile known to hold a full-length match
    __shared__ int s_key[kGroupCtx];              // maximum of the groups' keys
    __shared__ unsigned s_next;                   // 64 x the next group to take
    __shared__ int s_tiles;                       // most candidate tiles of any context here
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int stride = static_cast<int>(p.ctx_stride);
    const int nmax = p.n_max, nmin = p.n_min;
    const int b0 = blockIdx.x * kGroupCtx;
    for (int idx = threadIdx.x; idx < kGroupCtx * 64; idx += kGroupWaves * 64) {
        const int j = idx >> 6, i = idx & 63;
        const int b = b0 + j;
        int L = b < p.B ? p.lengths[b] : -1;
        if (b < p.B && (L < 0 || L > stride))
            L = 0;                                // flagged with the outputs
        const int32_t *c = p.tokens + static_cast<int64_t>(b < p.B ? b : 0) * p.ctx_stride;
        s_suf[j][i] = L > 0 ? c[max(0, L - 1 - min(i, nmax - 1))] : 0;
        if (i == 0) {
            s_len[j] = L;
            s_full[j] = -1;
            s_key[j] = 0;
        }
    }
    if (threadIdx.x == 0) {
        s_next = 0;
        s_tiles = 0;
    }
    __syncthreads();
    if (threadIdx.x < kGroupCtx) {                // the groups come from the contexts' lengths,
        const int L = s_len[threadIdx.x];         // not the row stride
        if (L - 2 >= nmin - 1)
            atomicMax(&s_tiles, (L - 2) / kTile - (nmin - 1) / kTile + 1);
    }
    __syncthreads();

    const int groups = (s_tiles + kGroupTiles - 1) / kGroupTiles;
    const int units = groups * kGroupCtx;
    int *buf0 = s_buf[w][0];
    int *buf1 = s_buf[w][1];
    for (;;) {
        // every lane adds 1, so the wave's 64 returns are 64u .. 64u + 63
        // and u is the same in every lane, with no hand-off between lanes;
        // reading it (and the LDS words below) as wave-uniform values lets
        // the group's control flow run on scalar branches
        const int u = __builtin_amdgcn_readfirstlane(static_cast<int>(atomicAdd(&s_next, 1u) >> 6));
        if (u >= units)
            break;
        const int j = u % kGroupCtx, g = u / kGroupCtx;
        const int L = __builtin_amdgcn_readfirstlane(s_len[j]);
        const int e_hi = L - 2, e_lo = nmin - 1;
        if (L < 0 || e_hi < e_lo)
            continue;
        const int t_top = e_hi / kTile, t_bot = e_lo / kTile;
        const int g_top = t_top - g * kGroupTiles;          // this group: tiles g_top down to g_low
        const int g_low = max(t_bot, g_top - kGroupTiles + 1);
        if (g_top < t_bot || __builtin_amdgcn_readfirstlane(s_full[j]) >= g_top)
            continue;
        const int32_t *c = p.tokens + static_cast<int64_t>(b0 + j) * p.ctx_stride;
        const int *sfx = s_suf[j];
        const int s0 = sfx[0];
        const int n = g_top - g_low + 1;                    // tiles in the group
        // step s of the ring: tile g_top - s for s < n; past the bottom tile,
        // the 32 positions under it (its halo; lanes 0..7 hold them)
        auto fetch = [&](int st) {
            const int pos = st < n ? (g_top - st) * kTile + 4 * lane : g_low * kTile - kHalo + 4 * (lane & 7);
            return load4<kVec>(c, pos, stride);
        };
        i32x4 q0 = fetch(0), q1 = fetch(1), pv = q0;
        int best = 0;
        bool stop = false;
        // Step k stages tile k (its top 32 positions also become the halo of
        // tile k - 1, staged one step earlier) and then scores tile k - 1,
        // whose halo is now complete; after the last tile, step n stages the
        // bottom tile's halo from the extra load and scores it.
        auto step = [&](int k, i32x4 &qs, int *bs, int *bo) {
            const i32x4 v = qs;
            if (!stop) {
                if (k < n) {
                    bs[kHalo + 4 * lane + 0] = v.x;
                    bs[kHalo + 4 * lane + 1] = v.y;
                    bs[kHalo + 4 * lane + 2] = v.z;
                    bs[kHalo + 4 * lane + 3] = v.w;
                    if (k >= 1 && lane >= 56) {
                        bo[4 * (lane - 56) + 0] = v.x;
                        bo[4 * (lane - 56) + 1] = v.y;
                        bo[4 * (lane - 56) + 2] = v.z;
                        bo[4 * (lane - 56) + 3] = v.w;
                    }
                } else if (lane < 8) {
                    bo[4 * lane + 0] = v.x;
                    bo[4 * lane + 1] = v.y;
                    bo[4 * lane + 2] = v.z;
                    bo[4 * lane + 3] = v.w;
                }
            }
            qs = fetch(min(k + 2, n));
            if (!stop && k >= 1) {
                const int t = g_top - (k - 1);
                if (__builtin_amdgcn_readfirstlane(s_full[j]) >= t) {
                    stop = true;
                } else {
                    const int lo = t * kTile;
                    unsigned hit = static_cast<unsigned>(pv.x == s0) | (static_cast<unsigned>(pv.y == s0) << 1) |
                                   (static_cast<unsigned>(pv.z == s0) << 2) | (static_cast<unsigned>(pv.w == s0) << 3);
                    if (lo < e_lo || lo + kTile - 1 > e_hi) {     // a tile at either end of the range
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk) {
                            const int e = lo + 4 * lane + kk;
                            if (e < e_lo || e > e_hi)
                                hit &= ~(1u << kk);
                        }
                    }
                    if (__ballot(hit != 0)) {
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk) {
                            if (hit & (1u << kk)) {
                                const int e = lo + 4 * lane + kk;
                                int m = 1;
                                while (m < nmax && e - m >= 0 &&
                                       bo[kHalo + 4 * lane + kk - m] == sfx[m])
                                    ++m;
                                if (m >= nmin)
                                    best = max(best, (m << kEndBits) | e);
                            }
                        }
                    }
                    if (__ballot((best >> kEndBits) == nmax)) {
                        stop = true;
                        if (lane == 0)
                            atomicMax(&s_full[j], t);
                    }
                }
            }
            pv = v;
            if (k >= n)
                stop = true;
        };
        for (int k = 0;; k += 2) {
            step(k, q0, buf0, buf1);
            step(k + 1, q1, buf1, buf0);
            if (stop)
                break;
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            best = max(best, __shfl_xor(best, off, 64));
        if (lane == 0 && best > 0)
            atomicMax(&s_key[j], best);
    }
    __syncthreads();

    for (int j = w; j < kGroupCtx; j += kGroupWaves) {
        const int b = b0 + j;
        if (b >= p.B)
            break;
        const int32_t *c = p.tokens + static_cast<int64_t>(b) * p.ctx_stride;
        const int Lr = p.lengths[b];
        const unsigned fl = (Lr < 0 || Lr > stride) ? SV_FLAG_BAD_LEN : 0u;
        const int L = s_len[j];
        const int best = s_key[j];
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
    // 16384 contexts (32 per workgroup, two workgroups per CU) fill the chip
    // in one round; below that, sixteen waves per context (one 1024-thread
    // workgroup) for at most 512 contexts, four otherwise
    if (p.B >= 2 * 256 * kGroupCtx) {
        const dim3 grid(static_cast<unsigned>((p.B + kGroupCtx - 1) / kGroupCtx));
        if (p.vec_ok)
            hipLaunchKernelGGL((k_ngram_groups<true>), grid, dim3(kGroupWaves * 64), 0, s, p);
        else
            hipLaunchKernelGGL((k_ngram_groups<false>), grid, dim3(kGroupWaves * 64), 0, s, p);
        return hipGetLastError();
    }
    const bool few = p.B <= 512;
    if (p.vec_ok)
        return few ? launch_w<true, 16, 1024>(p, s) : launch_w<true, 4, kThreads>(p, s);
    return few ? launch_w<false, 16, 1024>(p, s) : launch_w<false, 4, kThreads>(p, s);
}

} // namespace sv
