// suffix.hip -- suffix-decoding proposal on gfx950 ([Arctic] "suffix
// decoding": the most recent tokens are looked up in suffix trees of the
// current prompt and of earlier outputs, candidate tokens are ranked by how
// often they followed, and the candidate sequence grows while it stays
// likely).
//
// A suffix tree answers two questions: where does the context's recent
// suffix occur, and what followed those occurrences.  On the GPU both are
// answered by scanning the texts, which is bandwidth work with no pointer
// chasing:
//
// Kernel 1 (scan).  One wave per (sequence, text, chunk of 1024 candidate
// end positions); the texts are the sequence's context and the shared
// history.  A candidate end e needs a token after it (text[e+1] >= 0); its
// match length m(e) is the common suffix of text[..e] and the context, at
// most m_max.  The wave walks its chunk downwards in 256-position tiles (4
// per lane, staged in the wave's LDS with the 32 positions below), testing
// each candidate's last token against the context's last token in
// registers first.  It keeps the chunk's longest match (at least m_min) and
// that match's most recent SV_SUFFIX_OCC occurrences, and stops once it
// holds that many full-length (m_max) ones.
//
// Kernel 2 (path).  One wave per sequence and text (two per workgroup, no
// workgroup barriers until the pick): the longest match over the chunks, its most recent SV_SUFFIX_OCC occurrences gathered from
// the chunks in descending order, their continuations loaded in one round,
// then depth by depth the most frequent next token among the occurrences
// still on the path (lowest id on equal counts), kept while its count is at
// least min_prob times the number of occurrences.  The text whose path has
// the larger expected number of accepted tokens (sum of the counts over the
// number of occurrences, compared exactly in integers) gives the proposal;
// the context wins ties.

#include "sv_device.hpp"
#include "sv_kernels.hpp"

namespace sv {
namespace {

constexpr int kTile = 256;            // candidate ends per wave tile, 4 per lane
constexpr int kHalo = 32;             // positions staged below a tile
constexpr int kOcc = SV_SUFFIX_OCC;
static_assert(SV_SUFFIX_MAX_MATCH <= kHalo, "the halo must cover the longest pattern");
static_assert(kOcc == kThreads, "one occurrence per thread in the path kernel");

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Tokens pos .. pos+3 of a text of `lim` allocated entries, loaded
// unconditionally with positions clamped into the text (the caller drops
// what lies outside).  kVec: the text is 16-byte aligned, pos % 4 == 0 and
// lim >= 4.
template <bool kVec>
__device__ __forceinline__ i32x4 load4(const int32_t *t, int64_t pos, int64_t lim)
{
    if constexpr (kVec) {
        const int64_t q = pos < 0 ? 0 : (pos > lim - 4 ? lim - 4 : pos);
        return __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(t + q));
    } else {
        const int64_t last = lim - 1;
        i32x4 r;
        r.x = t[max<int64_t>(0, min<int64_t>(pos, last))];
        r.y = t[max<int64_t>(0, min<int64_t>(pos + 1, last))];
        r.z = t[max<int64_t>(0, min<int64_t>(pos + 2, last))];
        r.w = t[max<int64_t>(0, min<int64_t>(pos + 3, last))];
        return r;
    }
}

struct Text {
    const int32_t *t;
    int64_t len;      // tokens that belong to the text
    int64_t lim;      // entries that may be read (the context row's stride)
};

__device__ __forceinline__ int seq_len(const SuffixParams &p, int b, unsigned &fl)
{
    const int L = p.lengths[b];
    if (L < 0 || L > p.ctx_stride) {
        fl |= SV_FLAG_BAD_LEN;
        return 0;
    }
    return L;
}

// Reads of a context are clamped into the whole row with 16-byte loads
// (rows of ctx_stride entries, a multiple of 4) and into its L tokens
// otherwise.
template <bool kVec>
__device__ __forceinline__ Text text_of(const SuffixParams &p, int b, int L, bool hist)
{
    if (hist)
        return Text{p.history, p.H, p.H > 0 ? p.H : 1};
    return Text{p.tokens + static_cast<int64_t>(b) * p.ctx_stride, L, kVec ? p.ctx_stride : max(L, 1)};
}

// Scores one chunk for one pattern, in one wave.  buf holds the chunk staged
// in LDS: buf[0..32) the 32 positions below it, buf[32..32+1024) the chunk
// (first end lo), buf[32+1024] the token above it; sfx is the pattern
// (s0 = sfx[0] >= 0).  Lane l takes the ends lo + 256 q + 4 l + k (q, k <
// 4).  Leaves the chunk's longest match (at least m_min; 0 if none) in best
// and its most recent occurrences, highest end first, in occ (cnt <= kOcc).
__device__ __forceinline__ void score_chunk(const int *buf, const int *sfx, int s0, int64_t lo,
                                            int64_t e_lo, int64_t e_hi, int m_min, int m_max,
                                            int &best, int &cnt, int *occ)
{
    const int lane = threadIdx.x & 63;
    int mk[4][4];
    int lbest = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int o = kHalo + kTile * q + 4 * lane + k;    // LDS index of end e
            const int64_t e = lo + (o - kHalo);
            int m = 0;
            if (buf[o] == s0 && e >= e_lo && e <= e_hi && buf[o + 1] >= 0) {
                // one step, then (for the rare long matches) four steps per
                // round: eight independent LDS reads, one wait (reads past
                // m_max are clamped into the buffer and unused)
                m = 1;
                if (m < m_max && e - 1 >= 0 && sfx[1] >= 0 && buf[o - 1] == sfx[1]) {
                    m = 2;
                    for (;;) {
                        int t[4], pt[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            t[j] = buf[max(o - m - j, 0)];
                            pt[j] = sfx[min(m + j, kHalo - 1)];
                        }
                        int adv = 0;
                        bool run = true;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            run = run && m + j < m_max && e - m - j >= 0 && pt[j] >= 0 && t[j] == pt[j];
                            adv += run ? 1 : 0;
                        }
                        m += adv;
                        if (adv < 4)
                            break;
                    }
                }
                if (m < m_min)
                    m = 0;
            }
            mk[q][k] = m;
            lbest = max(lbest, m);
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        lbest = max(lbest, __shfl_xor(lbest, off, 64));
    best = lbest;
    cnt = 0;
    if (best == 0)
        return;
    // offsets in descending end order: tiles q from the top, then lanes from
    // the top, then a lane's own ends from the top
    const unsigned long long higher = lane == 63 ? 0ull : (~0ull << (lane + 1));
    int base = 0;
#pragma unroll
    for (int q = 3; q >= 0; --q) {
        int above = 0, total = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const unsigned long long bal = __ballot(mk[q][k] == best);
            above += __popcll(bal & higher);
            total += __popcll(bal);
        }
        int within = 0;
#pragma unroll
        for (int k = 3; k >= 0; --k) {
            if (mk[q][k] == best) {
                const int slot = base + above + within;
                if (slot < kOcc)
                    occ[slot] = static_cast<int>(lo + kTile * q + 4 * lane + k);
                ++within;
            }
        }
        base += total;
    }
    cnt = min(kOcc, base);
}

__device__ __forceinline__ void write_rec(SuffixScanRec *r, int best, int cnt, const int *occ)
{
    const int lane = threadIdx.x & 63;
    for (int k = lane; k < cnt; k += 64)
        r->occ[k] = occ[k];
    if (lane == 0) {
        r->best = best;
        r->cnt = cnt;
    }
}

// The pattern of sequence b into sfx (one wave): the context read
// backwards from its last token, -1 past its start, past m_max or at a
// negative token.
__device__ __forceinline__ void load_pattern(const SuffixParams &p, int b, int *sfx)
{
    const int lane = threadIdx.x & 63;
    const int L_raw = p.lengths[b];
    const int L = (L_raw < 0 || L_raw > p.ctx_stride) ? 0 : L_raw;
    const int cj = p.tokens[static_cast<int64_t>(b) * p.ctx_stride + max(0, L - 1 - min(lane, kHalo - 1))];
    if (lane < kHalo)
        sfx[lane] = (lane < p.m_max && lane < L && cj >= 0) ? cj : -1;
}

constexpr int kChunkLds = kHalo + kSfxChunk + 4;    // a staged chunk: halo, chunk, the token above
constexpr int kHistSeqs = 16;                        // sequences per history workgroup

// Context chunks: one wave per (sequence, chunk); the wave stages its chunk
// in its own LDS region.
template <bool kVec>
__device__ void scan_context(const SuffixParams &p, int64_t item, int *buf, int *sfx, int *occ)
{
    const int lane = threadIdx.x & 63;
    const int b = static_cast<int>(item / p.nch_ctx);
    const int chunk = static_cast<int>(item - static_cast<int64_t>(b) * p.nch_ctx);
    const int32_t *text = p.tokens + static_cast<int64_t>(b) * p.ctx_stride;
    const int64_t lim = p.ctx_stride;
    const int64_t lo = static_cast<int64_t>(chunk) * kSfxChunk;
    // the chunk (loaded over the whole row: it does not wait for the
    // length), the halo and the token above, then the pattern
    i32x4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        v[q] = load4<kVec>(text, lo + kTile * q + 4 * lane, lim);
    const i32x4 h = load4<kVec>(text, lo - kHalo + 4 * (lane & 7), lim);
    const int a = text[min<int64_t>(lo + kSfxChunk, lim - 1)];
    load_pattern(p, b, sfx);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        buf[kHalo + kTile * q + 4 * lane + 0] = v[q].x;
        buf[kHalo + kTile * q + 4 * lane + 1] = v[q].y;
        buf[kHalo + kTile * q + 4 * lane + 2] = v[q].z;
        buf[kHalo + kTile * q + 4 * lane + 3] = v[q].w;
    }
    if (lane < 8) {
        buf[4 * lane + 0] = h.x;
        buf[4 * lane + 1] = h.y;
        buf[4 * lane + 2] = h.z;
        buf[4 * lane + 3] = h.w;
    }
    if (lane == 0)
        buf[kHalo + kSfxChunk] = a;
    const int L_raw = p.lengths[b];
    const int L = (L_raw < 0 || L_raw > p.ctx_stride) ? 0 : L_raw;
    const int64_t e_hi = min<int64_t>(lo + kSfxChunk - 1, static_cast<int64_t>(L) - 2);
    const int64_t e_lo = max<int64_t>(lo, p.m_min - 1);
    const int s0 = sfx[0];
    int best = 0, cnt = 0;
    if (s0 >= 0 && e_hi >= e_lo)
        score_chunk(buf, sfx, s0, lo, e_lo, e_hi, p.m_min, p.m_max, best, cnt, occ);
    write_rec(p.rec + static_cast<int64_t>(b) * (p.nch_ctx + p.nch_hist) + chunk, best, cnt, occ);
}

// History chunks: one workgroup per (chunk, group of kHistSeqs sequences).
// The chunk is staged in LDS once; each wave scores it against its share
// of the group's patterns.
template <bool kVec>
__device__ void scan_history(const SuffixParams &p, int hb, int *text_lds, int (*sfx)[kHalo],
                             int *occ)
{
    const int t = threadIdx.x;
    const int w = t >> 6;
    const int chunk = hb % p.nch_hist;
    const int group = hb / p.nch_hist;
    const int64_t lo = static_cast<int64_t>(chunk) * kSfxChunk;
    const int64_t lim = p.H;
    const i32x4 v = load4<kVec>(p.history, lo + 4 * t, lim);
    const i32x4 h = load4<kVec>(p.history, lo - kHalo + 4 * (t & 7), lim);
    const int a = p.history[min<int64_t>(lo + kSfxChunk, lim - 1)];
    // the group's patterns: wave w loads sequences w, w + 4, ...
#pragma unroll
    for (int k = 0; k < kHistSeqs / kWaves; ++k) {
        const int g = w + kWaves * k;
        load_pattern(p, min(group * kHistSeqs + g, p.B - 1), sfx[g]);
    }
    text_lds[kHalo + 4 * t + 0] = v.x;
    text_lds[kHalo + 4 * t + 1] = v.y;
    text_lds[kHalo + 4 * t + 2] = v.z;
    text_lds[kHalo + 4 * t + 3] = v.w;
    if (t < 8) {
        text_lds[4 * t + 0] = h.x;
        text_lds[4 * t + 1] = h.y;
        text_lds[4 * t + 2] = h.z;
        text_lds[4 * t + 3] = h.w;
    }
    if (t == 0)
        text_lds[kHalo + kSfxChunk] = a;
    __syncthreads();
    const int64_t e_hi = min<int64_t>(lo + kSfxChunk - 1, p.H - 2);
    const int64_t e_lo = max<int64_t>(lo, p.m_min - 1);
#pragma unroll 1
    for (int k = 0; k < kHistSeqs / kWaves; ++k) {
        const int g = w + kWaves * k;
        const int b = group * kHistSeqs + g;
        if (b >= p.B)
            break;                                  // uniform over the wave
        const int s0 = sfx[g][0];
        int best = 0, cnt = 0;
        if (s0 >= 0 && e_hi >= e_lo)
            score_chunk(text_lds, sfx[g], s0, lo, e_lo, e_hi, p.m_min, p.m_max, best, cnt, occ);
        write_rec(p.rec + static_cast<int64_t>(b) * (p.nch_ctx + p.nch_hist) + p.nch_ctx + chunk, best,
                  cnt, occ);
    }
}

// Kernel 1: the first workgroups take context chunks (four per workgroup,
// one per wave), the rest history chunks.
template <bool kVec>
__global__ __launch_bounds__(kThreads) void k_suffix_scan(const SuffixParams p, int ctx_wgs)
{
    __shared__ int s_text[kWaves * kChunkLds];      // four context chunks, or one history chunk
    __shared__ int s_sfx[kHistSeqs][kHalo];
    __shared__ int s_occ[kWaves][kOcc];
    const int w = threadIdx.x >> 6;
    if (static_cast<int>(blockIdx.x) < ctx_wgs) {
        const int64_t item = static_cast<int64_t>(blockIdx.x) * kWaves + w;
        if (item >= static_cast<int64_t>(p.B) * p.nch_ctx)
            return;                                    // the whole wave; no barriers on this side
        scan_context<kVec>(p, item, s_text + w * kChunkLds, s_sfx[w], s_occ[w]);
    } else {
        scan_history<kVec>(p, static_cast<int>(blockIdx.x) - ctx_wgs, s_text, s_sfx, s_occ[w]);
    }
}

// Wave-wide reductions (every lane gets the result).
__device__ __forceinline__ int wave_sum_int(int x)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        x += __shfl_xor(x, off, 64);
    return x;
}

__device__ __forceinline__ int wave_min_int(int x)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        x = min(x, __shfl_xor(x, off, 64));
    return x;
}

__device__ __forceinline__ int wave_max_int(int x)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        x = max(x, __shfl_xor(x, off, 64));
    return x;
}

__device__ __forceinline__ long long wave_max_i64(long long x)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        x = max(x, static_cast<long long>(__shfl_xor(x, off, 64)));
    return x;
}

constexpr int kPer = kOcc / 64;       // occurrences per lane in the path wave
constexpr int kSortMin = 64;          // above this many continuing occurrences a step sorts them
constexpr int kHdr = 8;               // chunk headers per lane per gather round
constexpr int kRound = 64 * kHdr;     // chunks per gather round

// Per-wave LDS of the path kernel.
struct PathLds {
    int occ[kOcc];                    // end positions, most recent first
    int tok[kOcc];                    // this depth's continuing tokens, packed
    int end[kRound];                  // gather: inclusive end of each chunk's slots
    int cont[SV_SUFFIX_MAX_K][kOcc];  // continuation tokens [depth][occurrence]
    int path[SV_SUFFIX_MAX_K];
    long long S;
    int n, mstar, len;
};

__device__ __forceinline__ int wave_inclusive_int(int x)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off)
            x += y;
    }
    return x;
}

// The most frequent token among a wave's kOcc slots (kPer per lane; values
// below 0 are empty), the lowest token on equal counts, as the key
// (count << 32) | (0x7fffffff - token), 0 when every slot is empty: a
// bitonic sort of the slots in element order 4 * lane + q (partners kPer or
// more apart are in other lanes), then each run of equal values is measured
// from its first element, found by a max-scan of the run heads.
__device__ long long wave_mode(const int (&tok)[kPer])
{
    const int lane = threadIdx.x & 63;
    int v[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q)
        v[q] = tok[q] >= 0 ? tok[q] : -1;
#pragma unroll
    for (int k = 2; k <= kPer * 64; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            int o[kPer];
#pragma unroll
            for (int q = 0; q < kPer; ++q)
                o[q] = j >= kPer ? __shfl_xor(v[q], j / kPer, 64) : v[q ^ (j % kPer)];
#pragma unroll
            for (int q = 0; q < kPer; ++q) {
                const int i = kPer * lane + q;
                const bool up = (i & k) == 0, low = (i & j) == 0;
                v[q] = up == low ? min(v[q], o[q]) : max(v[q], o[q]);
            }
        }
    }
    // runs: start[q] = the index of the first element of element q's run
    const int prev = __shfl_up(v[kPer - 1], 1, 64);
    const int next = __shfl_down(v[0], 1, 64);
    int start[kPer];
    int s = -1;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int pv = q == 0 ? prev : v[q - 1];
        if ((lane == 0 && q == 0) || v[q] != pv)
            s = kPer * lane + q;
        start[q] = s;
    }
    int scan = s;                                 // inclusive max-scan of the lanes' last heads
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(scan, off, 64);
        if (lane >= off)
            scan = max(scan, y);
    }
    const int before = __shfl_up(scan, 1, 64);    // the last head in earlier lanes
    long long key = 0;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int i = kPer * lane + q;
        const int st = start[q] >= 0 ? start[q] : before;
        const int nv = q + 1 < kPer ? v[q + 1] : next;
        const bool end = (lane == 63 && q == kPer - 1) || v[q] != nv;
        if (end && v[q] >= 0)
            key = max(key, (static_cast<long long>(i - st + 1) << 32) | (0x7fffffffll - v[q]));
    }
    return wave_max_i64(key);
}

// The path of one text, computed by one wave (all control flow is uniform
// over the wave).  Occurrence i lives in lane i % 64, slot i / 64.
__device__ void text_path(const SuffixParams &p, int b, bool hist, PathLds &W)
{
    const int lane = threadIdx.x & 63;
    unsigned unused = 0;
    const int L = seq_len(p, b, unused);
    const Text tx = text_of<false>(p, b, L, hist);
    const int nct = hist ? p.nch_hist : p.nch_ctx;
    const SuffixScanRec *recs = p.rec + static_cast<int64_t>(b) * (p.nch_ctx + p.nch_hist) +
                                (hist ? p.nch_ctx : 0);
    // chunks in rounds of kRound, from the top: position j of a round is
    // chunk top - j, held by lane j % 64 in slot j / 64; every header of a
    // round is loaded at once
    auto headers = [&](int top, int (&hb)[kHdr], int (&hc)[kHdr]) {
#pragma unroll
        for (int r = 0; r < kHdr; ++r) {
            const int cc = top - (64 * r + lane);
            const SuffixScanRec *rr = recs + max(cc, 0);
            hb[r] = rr->best;
            hc[r] = rr->cnt;
            if (cc < 0)
                hb[r] = hc[r] = 0;
        }
    };
    int mb = 0;
    for (int top = nct - 1; top >= 0; top -= kRound) {
        int hb[kHdr], hc[kHdr];
        headers(top, hb, hc);
#pragma unroll
        for (int r = 0; r < kHdr; ++r)
            mb = max(mb, hb[r]);
    }
    const int mstar = wave_max_int(mb);
    int n = 0;
    if (mstar > 0 && p.K > 0) {
        // the most recent kOcc occurrences, round by round
        for (int top = nct - 1; top >= 0 && n < kOcc; top -= kRound) {
            int hb[kHdr], hc[kHdr];
            headers(top, hb, hc);
            int carry = 0;
#pragma unroll
            for (int r = 0; r < kHdr; ++r) {
                const int take = hb[r] == mstar ? hc[r] : 0;
                const int incl = wave_inclusive_int(take) + carry;
                W.end[64 * r + lane] = incl;
                carry = __shfl(incl, 63, 64);
            }
            const int need = min(carry, kOcc - n);
            int e[kPer];
#pragma unroll
            for (int q = 0; q < kPer; ++q) {
                const int slot = lane + 64 * q;
                e[q] = 0;
                if (slot < need) {
                    int j = 0;                    // positions whose slots end at or before slot
                    for (int step = kRound / 2; step > 0; step >>= 1)
                        if (W.end[j + step - 1] <= slot)
                            j += step;
                    const int before = j > 0 ? W.end[j - 1] : 0;
                    e[q] = recs[top - j].occ[slot - before];
                }
            }
#pragma unroll
            for (int q = 0; q < kPer; ++q)
                if (lane + 64 * q < need)
                    W.occ[n + lane + 64 * q] = e[q];
            n += need;
        }
        // continuations: every occurrence's next K tokens, one round of loads
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int i = lane + 64 * q;
            const int64_t e0 = i < n ? W.occ[i] : 0;
            int cont[SV_SUFFIX_MAX_K];
#pragma unroll
            for (int j = 0; j < SV_SUFFIX_MAX_K; ++j)
                cont[j] = tx.t[min<int64_t>(e0 + 1 + j, tx.lim - 1)];
#pragma unroll
            for (int j = 0; j < SV_SUFFIX_MAX_K; ++j)
                W.cont[j][i] = (i < n && e0 + 1 + j < tx.len) ? cont[j] : -1;
        }
    }
    long long sum = 0;
    int len = 0;
    if (n > 0) {
        const double need_n = p.min_prob * static_cast<double>(n);
        bool alive[kPer];
#pragma unroll
        for (int q = 0; q < kPer; ++q)
            alive[q] = lane + 64 * q < n;
        for (int j = 0; j < p.K; ++j) {
            int tok[kPer];
            unsigned long long val[kPer];
            int nv = 0;
#pragma unroll
            for (int q = 0; q < kPer; ++q) {
                const int cj = W.cont[j][lane + 64 * q];
                tok[q] = (alive[q] && cj >= 0) ? cj : -1;
                val[q] = __ballot(tok[q] >= 0);
                nv += __popcll(val[q]);
            }
            if (nv == 0)
                break;
            // the first continuing occurrence's token, and whether all agree
            int x0 = 0;
#pragma unroll
            for (int q = kPer - 1; q >= 0; --q)
                if (val[q])
                    x0 = __builtin_amdgcn_readlane(tok[q], __builtin_ctzll(val[q]));
            unsigned long long differ = 0;
#pragma unroll
            for (int q = 0; q < kPer; ++q)
                differ |= __ballot(tok[q] >= 0 && tok[q] != x0);
            int count, x;
            if (!differ) {                         // every continuing occurrence agrees
                count = nv;
                x = x0;
            } else if (nv > kSortMin) {
                const long long key = wave_mode(tok);
                count = static_cast<int>(key >> 32);
                x = static_cast<int>(0x7fffffffll - (key & 0xffffffffll));
            } else {
                // the continuing occurrences' tokens packed into W.tok[0, nv)
                // (their order does not matter), so that one pass over them
                // counts all of a lane's tokens; occurrences off the path do
                // not take part, and the path narrows them step by step
                int base = 0;
#pragma unroll
                for (int q = 0; q < kPer; ++q) {
                    const int below = __builtin_amdgcn_mbcnt_hi(static_cast<unsigned>(val[q] >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(val[q]), 0));
                    if (tok[q] >= 0)
                        W.tok[base + below] = tok[q];
                    base += __popcll(val[q]);
                }
                int mc[kPer] = {};
                for (int k = 0; k < nv; ++k) {           // one pass counts all of a lane's tokens
                    const int y = W.tok[k];
#pragma unroll
                    for (int q = 0; q < kPer; ++q)
                        mc[q] += y == tok[q] ? 1 : 0;
                }
                long long key = 0;
#pragma unroll
                for (int q = 0; q < kPer; ++q)
                    if (tok[q] >= 0)
                        key = max(key, (static_cast<long long>(mc[q]) << 32) | (0x7fffffffll - tok[q]));
                key = wave_max_i64(key);
                count = static_cast<int>(key >> 32);
                x = static_cast<int>(0x7fffffffll - (key & 0xffffffffll));
            }
            if (static_cast<double>(count) < need_n)
                break;
            if (lane == 0)
                W.path[len] = x;
            ++len;
            sum += count;
#pragma unroll
            for (int q = 0; q < kPer; ++q)
                alive[q] = alive[q] && tok[q] == x;
        }
    }
    if (lane == 0) {
        W.S = sum;
        W.n = n;
        W.mstar = mstar;
        W.len = len;
    }
}

// One workgroup of two waves per sequence: wave 0 the context, wave 1 the
// history; then wave 0 picks the better path and writes the outputs.
__global__ __launch_bounds__(128) void k_suffix_path(const SuffixParams p)
{
    __shared__ PathLds s_w[2];
    const int b = blockIdx.x;
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    if (w == 0 || p.H > 0) {
        text_path(p, b, w == 1, s_w[w]);
    } else if (lane == 0) {
        s_w[1].S = 0;
        s_w[1].n = 0;
        s_w[1].mstar = 0;
        s_w[1].len = 0;
    }
    __syncthreads();
    if (w != 0)
        return;
    const PathLds &C = s_w[0], &Hh = s_w[1];
    int which = -1;
    if (C.len > 0 && (Hh.len == 0 || C.S * Hh.n >= Hh.S * C.n))
        which = 0;
    else if (Hh.len > 0)
        which = 1;
    const PathLds &R = s_w[max(which, 0)];
    const int m = which >= 0 ? R.len : 0;
    for (int k = lane; k < p.K; k += 64)
        p.proposal[static_cast<int64_t>(b) * p.K + k] = k < m ? R.path[k] : -1;
    if (lane == 0) {
        unsigned fl = 0;
        seq_len(p, b, fl);
        p.proposal_len[b] = m;
        if (p.score)
            p.score[b] = which >= 0 ? static_cast<double>(R.S) / static_cast<double>(R.n) : 0.0;
        if (p.match_len)
            p.match_len[b] = which >= 0 ? R.mstar : 0;
        if (p.source)
            p.source[b] = which;
        if (p.flags)
            p.flags[b] = fl;
    }
}

} // namespace

hipError_t launch_suffix(const SuffixParams &p, hipStream_t s)
{
    const int64_t ctx_wgs = (static_cast<int64_t>(p.B) * p.nch_ctx + kWaves - 1) / kWaves;
    const int64_t hist_wgs = static_cast<int64_t>(p.nch_hist) * ((p.B + kHistSeqs - 1) / kHistSeqs);
    const dim3 g1(static_cast<unsigned>(ctx_wgs + hist_wgs));
    if (p.vec_ok)
        hipLaunchKernelGGL(k_suffix_scan<true>, g1, dim3(kThreads), 0, s, p, static_cast<int>(ctx_wgs));
    else
        hipLaunchKernelGGL(k_suffix_scan<false>, g1, dim3(kThreads), 0, s, p, static_cast<int>(ctx_wgs));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(k_suffix_path, dim3(static_cast<unsigned>(p.B)), dim3(128), 0, s, p);
    return hipGetLastError();
}

} // namespace sv
