// rejection.hip -- rejection-sampling verification on gfx950 (Leviathan et
// al. / Chen et al., the rule [vLLM-03] "1. principle" cites for keeping the
// target distribution at T > 0).
//
// Kernel 1 (row statistics).  One wave per (row, piece) over the K+1
// target rows and K draft rows of every sequence streams the logits once
// with 16-byte loads (the pieces are sized so that every wave of the launch
// is resident at once).  Each lane sums exp(l / T) against the fixed
// reference 0: fp32 sums of the 8 terms of a 16-byte vector, fp64 across
// vectors.  For bf16 logits the hardware exp2 takes the exact product of l
// and log2(e)/T rounded to 16 bits, and the rounding is corrected to first
// order through a second fp32 sum, of the terms weighted by l; fp32 logits
// use the compensated exp (about one ulp either way).  The rare vectors
// whose fp32 sum leaves a wide range (logits above about 44 T, -inf
// entries, rows far below 0) go through a careful path with its own
// reference and fp64 rescales.  The wave combines its lanes onto their
// largest reference and writes (reference, sum), with the logit at the
// row's draft token when the piece holds it.
//
// Kernel 2 (accept decision and final-sample masses).  One workgroup per
// (sequence, 4096-element chunk).  Wave 0 merges the statistics of the
// sequence's rows and takes the accept decision: per draft position p_k(x_k)
// and q_k(x_k) with an fp64 exp, the test u_k < p/q in fp64, a ballot of the
// rejections for the first one, n (the workgroup of chunk 0 also writes the
// per-sequence outputs).  The final token is drawn from one row pair: r =
// max(0, p_n - q_n) after a rejection (p_n when that sums to zero), or p_n
// when every draft was accepted.  Every wave then forms p and r per element
// of its 1024-element sub-chunk of that pair (the statistics kernel's exp,
// fp64 after it) and publishes the sub-chunk's masses.
//
// Kernel 3 (selection).  One workgroup per sequence prefix-sums the
// sub-chunk masses to find the sub-chunk where the running mass first
// exceeds u_K * S, then scans that sub-chunk in token order for the token
// whose cumulative mass first exceeds it, and writes the emitted tokens.
//
// Kernel boundaries order the phases; no workgroup waits for another.

#include "sv_device.hpp"
#include "sv_kernels.hpp"

namespace sv {
namespace {

constexpr int kSubPerChunk = kRejChunk / kRejSub;                 // 4: one per wave
constexpr int kChunkPerThread = kRejChunk / kThreads;             // 16 elements
constexpr int kSubPerThread = kRejSub / kThreads;                 // 4 elements
static_assert(kChunkPerThread * kThreads == kRejChunk, "chunk must split evenly over the threads");
static_assert(kSubPerChunk == kWaves, "one sub-chunk per wave");
static_assert(kSubPerThread * kThreads == kRejSub, "sub-chunk must split evenly over the threads");

// A lane's fast path sums e^(l/T) against the fixed reference 0 -- no
// subtraction per element -- in fp32 per vector of 8 and fp64 across
// vectors.  A vector whose fp32 sum leaves [kTiny, kBig] (a term above
// about e^44, NaN from a -inf logit, or every term below about e^-41 while
// nothing larger has been seen) goes through the careful path, which keeps
// a second sum against the lane's own reference.
constexpr float kBig = 18446744073709551616.0f;   // 2^64
constexpr float kTiny = 8.67361737988403547e-19f; // 2^-60

// z * exp((m - M) / T) in fp64: moves a sum z taken against the reference m
// onto the reference M (z == 0: nothing was summed).  Out of line: it runs
// rarely, and inlined it would hold the fp64 exp's constants in registers
// across the streaming loop.
__device__ __attribute__((noinline)) double rescale_slow(double z, float m, float M, double inv_t_d)
{
    return z * exp((static_cast<double>(m) - static_cast<double>(M)) * inv_t_d);
}

__device__ __forceinline__ double rescale(double z, float m, float M, double inv_t_d)
{
    return z != 0.0 ? rescale_slow(z, m, M, inv_t_d) : 0.0;
}

// A lane's two running sums: z0 = sum of e^(l/T) (reference 0) and zc =
// sum of e^((l - rc)/T) over the vectors the careful path could not add to
// z0 (rc = -inf while there are none).
struct LaneSums {
    double z0 = 0.0;
    double zc = 0.0;
    float rc = -__builtin_inff();
};

// How the fast path forms e^(l/T).
enum ExpMode : int {
    kExpUnitT = 0,    // compensated exp of l (T == 1)
    kExpScaled = 1,   // compensated exp of l * (1/T)
    kExpSplit = 2,    // bf16 only: split constant, first-order correction summed apart
    kProbs = 3,       // the values are probabilities: summed as they are
};

// e^(f / T) of one value by the fast path's arithmetic, -inf giving 0.
// kExpSplit: f is clamped to a finite value whose exp2 underflows, so the
// first-order correction stays finite.
template <int kMode>
__device__ __forceinline__ float one_term(float f, float inv_t, float c1, float k2)
{
    if constexpr (kMode == kExpSplit) {
        const float fc = fmaxf(f, -3.0e38f);
        const float e = __builtin_amdgcn_exp2f(fc * c1);
        return __builtin_fmaf(e, k2 * fc, e);
    } else {
        return exp_cz(kMode == kExpUnitT ? f : f * inv_t);
    }
}

// The careful path for n values whose fast fp32 sum `s` is out of range.
template <int kMode, int n>
__device__ __forceinline__ void careful_add(const float (&f)[n], float s, LaneSums &ls, float inv_t,
                                            double inv_t_d, float c1, float k2)
{
    constexpr bool kUnitT = kMode == kExpUnitT;
    // -inf values made the sum NaN: the same sum, by the same arithmetic,
    // with -inf read as 0
    if (!(s == s)) {
        s = 0.0f;
#pragma unroll
        for (int j = 0; j < n; ++j)
            s += one_term<kMode>(f[j], inv_t, c1, k2);
    }
    // in range, or too small to matter next to what z0 already holds
    if ((s >= kTiny || (s >= 0.0f && ls.z0 >= 1.0)) && s <= kBig) {
        ls.z0 += static_cast<double>(s);
        return;
    }
    float vm = f[0];
#pragma unroll
    for (int j = 1; j < n; ++j)
        vm = fmaxf(vm, f[j]);
    if (vm == -__builtin_inff())
        return;
    float t = 0.0f;
#pragma unroll
    for (int j = 0; j < n; ++j)
        t += exp_cz(kUnitT ? f[j] - vm : (f[j] - vm) * inv_t);
    if (vm > ls.rc) {
        ls.zc = rescale(ls.zc, ls.rc, vm, inv_t_d) + static_cast<double>(t);
        ls.rc = vm;
    } else {
        ls.zc += rescale(static_cast<double>(t), vm, ls.rc, inv_t_d);
    }
}

// Sum of e^(f_j / T) over a vector, in fp32.  kExpSplit: with log2(e)/T =
// c1 + c2, c1 of 16 significant bits, y = f c1 is exact for bf16 f, and
// e^(f/T) = 2^y 2^(f c2) = 2^y (1 + f c2 ln 2 + ...), so the vector's sum is
// s1 + k2 s2 with s1 = sum of 2^y, s2 = sum of 2^y f and k2 = c2 ln 2.  The
// dropped terms are below (|y| 2^-16 ln 2)^2 / 2 relative: under 2.3e-7
// for the |y| <= 64 that an in-range sum allows, about 1e-9 at |y| <= 10.
template <int kMode, int n>
__device__ __forceinline__ float vec_exp_sum(const float (&f)[n], float inv_t, float c1, float k2)
{
    if constexpr (kMode == kProbs) {
        float s = f[0];
#pragma unroll
        for (int j = 1; j < n; ++j)
            s += f[j];
        return s;
    } else if constexpr (kMode == kExpSplit) {
        float e = __builtin_amdgcn_exp2f(f[0] * c1);
        float s1 = e, s2 = e * f[0];
#pragma unroll
        for (int j = 1; j < n; ++j) {
            e = __builtin_amdgcn_exp2f(f[j] * c1);
            s1 += e;
            s2 = __builtin_fmaf(e, f[j], s2);
        }
        return __builtin_fmaf(k2, s2, s1);
    } else {
        float s = exp_c(kMode == kExpUnitT ? f[0] : f[0] * inv_t);
#pragma unroll
        for (int j = 1; j < n; ++j)
            s += exp_c(kMode == kExpUnitT ? f[j] : f[j] * inv_t);
        return s;
    }
}

// One wave per work item (row, piece); a workgroup carries four items.
// The partial's reference is at most about e^44 below every element of the
// piece (fast-path vectors sum to at most 2^64 against 0; careful vectors
// are taken against their own maximum) and, when the piece has terms of
// non-negligible size against 0, at least 0.
template <typename E, int kMode>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8))) void k_rej_stats(const RejectParams p)
{
    const int lane = threadIdx.x & 63;
    const int K = p.K;
    const int rows_per_seq = 2 * K + 1;
    const int64_t item = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
    if (item >= static_cast<int64_t>(p.B) * rows_per_seq * p.segs)
        return;
    const int64_t row = item / p.segs;
    const int seg = static_cast<int>(item - row * p.segs);
    const int b = static_cast<int>(row / rows_per_seq);
    const int r = static_cast<int>(row - static_cast<int64_t>(b) * rows_per_seq);
    unsigned unused = 0;
    const int len = p.has_len ? clamp_len(p.draft_len[b], K, unused) : K;
    const bool is_target = r <= K;
    const int i = is_target ? r : r - (K + 1);
    const bool needed = is_target ? i <= len : i < len;
    // the row's draft token (target row K has none), loaded ahead of the
    // stream and used after it when the logit at the token is captured
    const int x = p.draft[static_cast<int64_t>(b) * K + max(0, min(i, K - 1))];
    const int lo = seg * p.seg_len;
    const int hi = min(p.V, lo + p.seg_len);
    float lx = __builtin_nanf("");

    LaneSums ls;
    if (needed) {
        const E *rp = is_target
                          ? static_cast<const E *>(p.target) + (static_cast<int64_t>(b) * (K + 1) + i) * p.row_stride
                          : static_cast<const E *>(p.draftl) + (static_cast<int64_t>(b) * K + i) * p.row_stride;
        const float inv_t = p.inv_t;
        const double inv_t_d = p.inv_t_d;
        const float c1 = p.split_c1, k2 = p.split_k2;
        stream_segment<E, 4, 64, true>(
            rp, lo, hi, lane,
            [&](const float(&f)[Elem<E>::kPerVec], int) {
                const float s = vec_exp_sum<kMode>(f, inv_t, c1, k2);
                if (kMode == kProbs || (s >= kTiny && s <= kBig))
                    ls.z0 += static_cast<double>(s);
                else
                    careful_add<kMode>(f, s, ls, inv_t, inv_t_d, c1, k2);
            },
            [&](float x, int) {
                const float f1[1] = {x};
                const float s = vec_exp_sum<kMode>(f1, inv_t, c1, k2);
                if (kMode == kProbs || (s >= kTiny && s <= kBig)) {
                    ls.z0 += static_cast<double>(s);
                } else {
                    careful_add<kMode>(f1, s, ls, inv_t, inv_t_d, c1, k2);
                }
            });
        const int xl = x - p.v_offset;
        if (p.capture_x && i < K && xl >= lo && xl < hi)
            lx = Elem<E>::one(rp, xl);
    }
    // the lane's sums onto its reference R, then the wave's onto their
    // largest R.  With terms summed against 0, R = max(0, rc): those terms
    // put the lane's maximum within about e^42 of 0.  Without any (a lane
    // whose values all lie far below 0), R = rc, so that the sampling
    // kernels' fp32 exp against the row's reference stays clear of
    // underflow.
    const float R = ls.z0 != 0.0 ? fmaxf(0.0f, ls.rc) : ls.rc;
    const double zl = (R == 0.0f ? ls.z0 : rescale(ls.z0, 0.0f, R, p.inv_t_d)) +
                      (ls.rc == R ? ls.zc : rescale(ls.zc, ls.rc, R, p.inv_t_d));
    const float M = wave_max(R);
    const double zz = wave_sum(R == M ? zl : rescale(zl, R, M, p.inv_t_d));
    if (lane == 0)
        p.partial[item] = SoftPartial{zz, M, lx};
}

// Per-row merge of a shard's segment partials (one thread per row): the
// segments move onto the largest reference and add up in segment order; lx
// comes from the one segment that captured it.
__global__ __launch_bounds__(kThreads) void k_rej_shard_rows(const RejectParams p, SoftPartial *out)
{
    const int64_t rows = static_cast<int64_t>(p.B) * (2 * p.K + 1);
    const int64_t r = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (r >= rows)
        return;
    const int segs = p.segs;
    SoftPartial q[kMaxSegs];
#pragma unroll
    for (int s = 0; s < kMaxSegs; ++s)
        q[s] = p.partial[r * segs + min(s, segs - 1)];
    float M = -__builtin_inff();
    float lx = __builtin_nanf("");
#pragma unroll
    for (int s = 0; s < kMaxSegs; ++s) {
        if (s < segs) {
            M = fmaxf(M, q[s].m);
            if (q[s].lx == q[s].lx)
                lx = q[s].lx;
        }
    }
    double z = 0.0;
#pragma unroll
    for (int s = 0; s < kMaxSegs; ++s)
        if (s < segs)
            z += q[s].m == M ? q[s].z : rescale(q[s].z, q[s].m, M, p.inv_t_d);
    out[r] = SoftPartial{z, M, lx};
}

// The small kernels below issue every load of a phase before using any of
// them (addresses are clamped in bounds instead of guarded by branches, the
// values outside the wanted range are dropped after loading): a load consumed
// inside a branch or loop is waited for on the spot, and each such wait costs
// a full memory round trip.

// A lane's value in every lane (uniform source lane `l`).
__device__ __forceinline__ double read_lane(double x, int l)
{
    const unsigned long long u = static_cast<unsigned long long>(__double_as_longlong(x));
    const unsigned lo = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(u & 0xffffffffu), l));
    const unsigned hi = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(u >> 32), l));
    return __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo));
}

__device__ __forceinline__ float read_lane(float x, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// The accept decision of one sequence (step a4, and the choice of the row
// pair step a5 draws from), taken by one wave over blocks of 8 draft
// positions.  Four lanes hold each row of a block: lane h * 16 + j, j < 8,
// target row base + j, and lane h * 16 + 8 + j draft row base + j, where
// quarter h takes the row's partials (pieces of the row, or its vocabulary
// shards) s = h, h + 4, ...  Each quarter moves its partials onto their
// largest reference and the quarters combine in fp64.  The draft row's
// statistics then move to its position's lane, and the lanes of positions
// below the draft length test u < p/q in fp64 (p and q from the logits at
// the draft token, which the statistics kernel captured, with an fp64 exp).
// A ballot of the rejections gives the first one, n; after a block with no
// rejection that holds the draft length, n is the length (the bonus row).
// With `publish` the wave writes the call's per-sequence outputs for every
// position and the sequence state; without, it stops at the block holding
// n.  The state comes back in every lane.
constexpr int kDecBlock = 8;
constexpr int kDecSplit = 4;                      // lanes per row
constexpr int kDecPer = kMaxSegs / kDecSplit;     // partials per lane, at most
static_assert(2 * kDecBlock * kDecSplit == 64, "one wave holds a block's rows");

__device__ __forceinline__ SeqState wave_decide(const RejectParams &p, int b, bool publish)
{
    const int lane = threadIdx.x & 63;
    const int K = p.K;
    const int segs = p.segs;
    const int64_t row0 = static_cast<int64_t>(b) * (2 * K + 1);
    const int h = lane >> 4;                  // which quarter of the row's partials
    const int slot = lane & 15;               // the lane's row in the block
    const bool tgt = slot < kDecBlock;
    const int j = slot & (kDecBlock - 1);
    unsigned fl = 0;
    const int len = p.has_len ? clamp_len(p.draft_len[b], K, fl) : K;
    SeqState st{};
    int n = -1;
    bool oor = false;
    for (int base = 0; base <= K; base += kDecBlock) {
        const int i = base + j;
        const bool has_row = tgt ? i <= K : i < K;
        const bool use = has_row && (tgt ? i <= len : i < len);
        // the row within the sequence, clamped onto an existing one
        const int ri = min(tgt ? min(i, K) : K + 1 + max(0, min(i, K - 1)), 2 * K);
        const int x = p.draft[static_cast<int64_t>(b) * K + max(0, min(i, K - 1))];
        const float u = p.u[static_cast<int64_t>(b) * (K + 1) + min(i, K)];
        SoftPartial q[kDecPer];
#pragma unroll
        for (int k = 0; k < kDecPer; ++k)
            q[k] = p.partial[(row0 + ri) * p.part_row_step +
                             min(h + kDecSplit * k, segs - 1) * p.part_seg_step];
        float M = -__builtin_inff();
        float lx = __builtin_nanf("");
#pragma unroll
        for (int k = 0; k < kDecPer; ++k) {
            if (h + kDecSplit * k < segs) {
                M = fmaxf(M, q[k].m);
                if (q[k].lx == q[k].lx)
                    lx = q[k].lx;
            }
        }
#pragma unroll
        for (int off = 16; off < 64; off <<= 1) {
            M = fmaxf(M, __shfl_xor(M, off, 64));
            const float o = __shfl_xor(lx, off, 64);
            if (!(lx == lx))
                lx = o;
        }
        double Z = 0.0;
#pragma unroll
        for (int k = 0; k < kDecPer; ++k)
            if (h + kDecSplit * k < segs)
                Z += q[k].m == M ? q[k].z : rescale(q[k].z, q[k].m, M, p.inv_t_d);
        Z += __shfl_xor(Z, 16, 64);
        Z += __shfl_xor(Z, 32, 64);
        if (!use) {
            M = -__builtin_inff();
            Z = 0.0;
            lx = __builtin_nanf("");
        }
        const double Zd = __shfl(Z, lane + kDecBlock, 64);     // lanes of target rows: their draft row
        const float Md = __shfl(M, lane + kDecBlock, 64);
        const float lxd = __shfl(lx, lane + kDecBlock, 64);
        const bool test = lane < kDecBlock && i < len;      // one lane per position
        const bool valid = K > 0 && x >= 0 && x < p.v_full;
        double pk = 0.0, qk = 0.0;
        bool rejected = false;
        if (test) {
            double ratio = 0.0;
            if (valid) {
                if (p.probs) {                 // given probabilities: value over the row's sum
                    pk = static_cast<double>(lx) / Z;
                    qk = static_cast<double>(lxd) / Zd;
                } else {
                    pk = exp((static_cast<double>(lx) - static_cast<double>(M)) * p.inv_t_d) / Z;
                    qk = exp((static_cast<double>(lxd) - static_cast<double>(Md)) * p.inv_t_d) / Zd;
                }
                ratio = qk > 0.0 ? pk / qk : __builtin_inf();
            }
            rejected = !(static_cast<double>(u) < ratio);
            oor = oor || !valid;
        }
        if (publish && lane < kDecBlock && i < K) {
            if (p.p_draft)
                p.p_draft[static_cast<int64_t>(b) * K + i] = static_cast<float>(pk);
            if (p.q_draft)
                p.q_draft[static_cast<int64_t>(b) * K + i] = static_cast<float>(qk);
        }
        const unsigned long long rej = __ballot(rejected);
        if (n < 0) {
            int here = -1;
            if (rej)
                here = base + __builtin_ctzll(rej);
            else if (len < base + kDecBlock)
                here = len;
            if (here >= 0) {
                const int l = here - base;
                n = here;
                st.n = here;
                st.len = len;
                st.zt = read_lane(Z, l);
                st.mt = read_lane(M, l);
                if (here < len) {
                    st.zd = read_lane(Zd, l);
                    st.md = read_lane(Md, l);
                }
            }
        }
        if (n >= 0 && !publish)
            break;
    }
    if (publish) {
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
            p.seq[b] = st;
        }
        if (p.stats)
            for (int k = lane; k < n; k += 64)
                stats_add(p.stats + 3 + k, 1);
    }
    return st;
}

// The accept decision alone (the vocabulary-shard call, on every shard's
// partials): one wave per sequence, four sequences per workgroup.
__global__ __launch_bounds__(kThreads) void k_rej_scan(const RejectParams p)
{
    const int b = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (b < p.B)
        wave_decide(p, b, true);
}

// kN consecutive elements [v0, v0 + kN) of a row, loaded before use.  kVec:
// the row is a whole number of aligned 16-byte vectors, so each vector of
// the slice lies wholly inside the row or wholly past it, and one past it
// loads the row's last vector instead.  Otherwise elements are loaded one by
// one with the index clamped to V - 1.  Values past the row are garbage for
// the caller to drop.
template <typename E, int kN, bool kVec>
struct Slice {
    static constexpr int PV = Elem<E>::kPerVec;
    static constexpr int NV = kVec ? kN / PV : 1;
    static constexpr int NE = kVec ? 1 : kN;
    static_assert(!kVec || kN % PV == 0, "vector slices hold whole vectors");
    u32x4 v[NV];
    E e[NE];

    __device__ __forceinline__ void fetch(const E *row, int v0, int V)
    {
        if constexpr (kVec) {
            const u32x4 *vp = reinterpret_cast<const u32x4 *>(row);
            const int last = V / PV - 1;
#pragma unroll
            for (int q = 0; q < NV; ++q)
                v[q] = vp[min(v0 / PV + q, last)];
        } else {
#pragma unroll
            for (int j = 0; j < NE; ++j)
                e[j] = row[min(v0 + j, V - 1)];
        }
    }

    __device__ __forceinline__ void widen(float (&f)[kN]) const
    {
        if constexpr (kVec) {
#pragma unroll
            for (int q = 0; q < NV; ++q) {
                float g[PV];
                Elem<E>::unpack(v[q], g);
#pragma unroll
                for (int j = 0; j < PV; ++j)
                    f[q * PV + j] = g[j];
            }
        } else {
#pragma unroll
            for (int j = 0; j < NE; ++j)
                f[j] = Elem<E>::widen(e[j]);
        }
    }
};

// The rows of the final sample and the per-element masses over a thread's
// kN contiguous elements [v0, v0 + cnt).  Each element's e^((l - m)/T) is
// formed the way the statistics kernel formed the normaliser it is divided
// by: for bf16 logits summed with the split constant against the reference
// 0, the hardware exp2 of the exact product l c1 with the first-order
// correction (1 + l k2); otherwise the compensated exp.  The normalised
// values then carry the exp's rounding only as independent per-element
// errors, whatever its bias, and the residual max(0, p - q) is not skewed by
// one row's normaliser against the other's.
//
// The per-element work is fp32 on the unnormalised terms: p_j Z_t = e_j and
// r_j Z_t = max(0, e_j - kappa d_j) with kappa = Z_t / Z_d carried as two
// fp32 parts (hi + lo, folded in by two FMAs, so the draft row is scaled to
// about 2^-48 and not to fp32's 2^-24, which would shift r coherently).
// Sums of terms are scaled by 1 / Z_t in fp64.
template <typename E>
struct SampleRows {
    const E *pt;
    const E *pd;        // the target row again when sampling the bonus
    bool residual;      // a draft row is present: r is formed
    bool probs;         // the rows are probabilities: the terms are the values
    bool split;         // split-constant exp (bf16, both references 0)
    float mt, md;
    double izt;         // 1 / Z_t
    float kap_hi, kap_lo;
    float inv_t, c1, k2;
    int V;

    __device__ __forceinline__ SampleRows(const RejectParams &p, int b, int len, const SeqState &st)
    {
        const int K = p.K, n = st.n;
        pt = static_cast<const E *>(p.target) + (static_cast<int64_t>(b) * (K + 1) + n) * p.row_stride;
        mt = st.mt;
        izt = 1.0 / st.zt;
        inv_t = p.inv_t;
        c1 = p.split_c1;
        k2 = p.split_k2;
        V = p.V;
        probs = p.probs != 0;
        residual = n < len;
        pd = pt;
        md = 0.0f;
        kap_hi = kap_lo = 0.0f;
        if (residual) {
            pd = static_cast<const E *>(p.draftl) + (static_cast<int64_t>(b) * K + n) * p.row_stride;
            md = st.md;
            const double kap = st.zt / st.zd;
            kap_hi = static_cast<float>(kap);
            kap_lo = static_cast<float>(kap - static_cast<double>(kap_hi));
        }
        split = sizeof(E) == 2 && p.split_ok && !probs && mt == 0.0f && md == 0.0f;
    }

    // e^((l - m) / T) (the value itself for probabilities), -inf giving 0
    // (split: l clamped to a finite value whose exp2 underflows, so the
    // correction term stays finite)
    __device__ __forceinline__ float term(float l, float m) const
    {
        if (probs)
            return l;
        if (split) {
            const float lc = fmaxf(l, -3.0e38f);
            const float e = __builtin_amdgcn_exp2f(lc * c1);
            return __builtin_fmaf(e, k2 * lc, e);
        }
        return exp_cz((l - m) * inv_t);
    }

    // visit(j, a_j, r_j) for j < cnt in order, with a_j = p_j Z_t and, after
    // a rejection, r_j = max(0, p_j - q_j) Z_t (else 0), in fp32.  Both rows
    // are loaded before either is used.
    template <int kN, bool kVec, typename F>
    __device__ __forceinline__ void visit(int v0, int cnt, F &&f) const
    {
        Slice<E, kN, kVec> st, sd;
        st.fetch(pt, v0, V);
        if (residual)
            sd.fetch(pd, v0, V);
        float ft[kN], fd[kN];
        st.widen(ft);
        if (residual)
            sd.widen(fd);
#pragma unroll
        for (int j = 0; j < kN; ++j) {
            if (j < cnt) {
                const float a = term(ft[j], mt);
                float r = 0.0f;
                if (residual) {
                    const float d = term(fd[j], md);
                    // kappa d - a with the product exact in each FMA
                    const float x = __builtin_fmaf(d, kap_lo, __builtin_fmaf(d, kap_hi, -a));
                    r = fmaxf(-x, 0.0f);
                }
                f(j, a, r);
            }
        }
    }
};

// The final-sample masses of one chunk of row pair n (step a5): p and
// r = max(0, p - q) per element, one mass pair per 1024-element sub-chunk
// (one per wave; a sub-chunk past the row's last is not written).  A
// thread's 16 terms add in fp32, the wave's 64 partial sums in fp64.
template <typename E, bool kVec>
__device__ __forceinline__ void chunk_masses(const RejectParams &p, int b, int c, const SeqState &st)
{
    const SampleRows<E> sr(p, b, st.len, st);
    const int v0 = c * kRejChunk + threadIdx.x * kChunkPerThread;
    const int cnt = max(0, min(kChunkPerThread, p.V - v0));
    float ps = 0.0f, rs = 0.0f;
    sr.template visit<kChunkPerThread, kVec>(v0, cnt, [&](int, float a, float r) {
        ps += a;
        rs += r;
    });
    const double pm = wave_sum(static_cast<double>(ps) * sr.izt);
    const double rm = wave_sum(static_cast<double>(rs) * sr.izt);
    const int sub = c * kSubPerChunk + (threadIdx.x >> 6);
    if ((threadIdx.x & 63) == 0 && sub < p.nsub)
        p.cmass[static_cast<int64_t>(b) * p.nsub + sub] = ChunkMass{rm, pm};
}

// Kernel 2: the final-sample masses, one workgroup per (sequence, 4096-element
// chunk).  kDecide (the whole call): wave 0 first takes the sequence's
// accept decision from the row statistics (the workgroup of chunk 0 also
// publishes it), then every wave forms the masses of its sub-chunk of row
// pair n.  Otherwise (a vocabulary shard's masses) the decision comes from
// the sequence state.
template <typename E, bool kVec, bool kDecide>
__device__ __forceinline__ void final_masses(const RejectParams &p)
{
    const int b = blockIdx.x / p.nchunks;
    const int c = blockIdx.x - b * p.nchunks;
    SeqState st;
    if constexpr (kDecide) {
        __shared__ SeqState s_st;
        if (threadIdx.x < 64) {
            const SeqState d = wave_decide(p, b, c == 0);
            if (threadIdx.x == 0)
                s_st = d;
        }
        __syncthreads();
        st = s_st;
    } else {
        st = p.seq[b];
    }
    chunk_masses<E, kVec>(p, b, c, st);
}

// 16-byte loads: every wave of the launch fits on the chip at once.
template <typename E, bool kDecide>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8))) void k_rej_final(const RejectParams p)
{
    final_masses<E, true, kDecide>(p);
}

// Element loads (rows not made of aligned 16-byte vectors).
template <typename E, bool kDecide>
__global__ __launch_bounds__(kThreads) void k_rej_final_scalar(const RejectParams p)
{
    final_masses<E, false, kDecide>(p);
}

// A vocabulary shard's final-sample totals: the sum of its sub-chunk masses
// per sequence, in sub-chunk order (one workgroup per sequence).
__global__ __launch_bounds__(kThreads) void k_rej_shard_total(const RejectParams p)
{
    const int b = blockIdx.x;
    const int nsub = p.nsub;
    const ChunkMass *cm = p.cmass + static_cast<int64_t>(b) * nsub;
    double r = 0.0, q = 0.0;
    for (int k = threadIdx.x; k < nsub; k += kThreads) {
        const ChunkMass m = cm[k];
        r += m.r;
        q += m.p;
    }
    double R, P;
    block_inclusive_scan(r, R);
    block_inclusive_scan(q, P);
    if (threadIdx.x == 0)
        p.mass_out[b] = ChunkMass{R, P};
}

// Kernel 3: one workgroup per sequence, two memory rounds.  Round 1 loads
// everything that does not depend on the chosen sub-chunk: the sequence
// state, u_K, the sequence's sub-chunk masses (kept in registers, and staged
// in LDS when they fit) and the drafts it re-emits.  Round 2 loads the one
// sub-chunk where the running mass crosses u_K * S.
//
// kShardIn (vocabulary shards): S and the mass before this shard come from
// every shard's totals, summed in shard order; the shard where the running
// mass crosses u_K * S (else the last one with mass) owns the sample, and
// only its call goes on to write the sequence's emitted tokens.
constexpr int kSelStage = 2048;                   // sub-chunk masses staged in LDS (V up to 2M)
constexpr int kSelPer = kSelStage / kThreads;     // masses per thread held in registers

template <typename E, bool kShardIn>
__global__ __launch_bounds__(kThreads) void k_rej_select(const RejectParams p)
{
    __shared__ ChunkMass s_cm[kSelStage];
    __shared__ double s_before;
    const int K = p.K;
    const int b = blockIdx.x;
    const int t = threadIdx.x;
    const SeqState st = p.seq[b];
    ChunkMass sh[kMaxSegs];                       // every shard's totals (shard input)
    if (kShardIn) {
#pragma unroll
        for (int s = 0; s < kMaxSegs; ++s)
            sh[s] = p.shard_mass[static_cast<int64_t>(min(s, p.shard_count - 1)) * p.B + b];
    }
    const float ufin = p.u[static_cast<int64_t>(b) * (K + 1) + K];
    const int nsub = p.nsub;
    const ChunkMass *cm = p.cmass + static_cast<int64_t>(b) * nsub;
    const bool staged = nsub <= kSelStage;
    const int per = (nsub + kThreads - 1) / kThreads;      // sub-chunks per thread
    const int k0 = min(nsub, t * per);
    const int k1 = min(nsub, k0 + per);
    ChunkMass mine[kSelPer];
    if (staged) {
#pragma unroll
        for (int j = 0; j < kSelPer; ++j)
            mine[j] = cm[min(k0 + j, nsub - 1)];
    }
    const int *d = p.draft + static_cast<int64_t>(b) * K;
    const int d_own = d[max(0, min(t, K - 1))];
    double myr = 0.0, myp = 0.0;
    if (staged) {
#pragma unroll
        for (int j = 0; j < kSelPer; ++j) {
            if (k0 + j < k1) {
                s_cm[k0 + j] = mine[j];
                myr += mine[j].r;
                myp += mine[j].p;
            }
        }
    } else {
        for (int k = k0; k < k1; ++k) {
            const ChunkMass q = cm[k];
            myr += q.r;
            myp += q.p;
        }
    }
    const int len = st.len;
    const int n = st.n;
    const bool residual = n < len;
    // (the barriers inside the scans also publish s_cm)
    double SR, SP;
    const double inclr = block_inclusive_scan(myr, SR);
    const double inclp = block_inclusive_scan(myp, SP);
    bool use_p = !residual || SR == 0.0;
    double S = use_p ? SP : SR;
    double base = 0.0;                            // mass before this shard
    if (kShardIn) {
        double tr = 0.0, tp = 0.0;
#pragma unroll
        for (int s = 0; s < kMaxSegs; ++s) {
            if (s < p.shard_count) {
                tr += sh[s].r;
                tp += sh[s].p;
            }
        }
        use_p = !residual || tr == 0.0;
        S = use_p ? tp : tr;
        const double u_s = static_cast<double>(ufin) * S;
        int owner = -1, last = 0;
        double run = 0.0, before = 0.0, before_last = 0.0;
#pragma unroll
        for (int s = 0; s < kMaxSegs; ++s) {
            if (s < p.shard_count) {
                const double X = use_p ? sh[s].p : sh[s].r;
                if (X > 0.0) {
                    last = s;
                    before_last = run;
                }
                if (owner < 0 && run + X > u_s) {
                    owner = s;
                    before = run;
                }
                run += X;
            }
        }
        if (owner < 0) {                          // rounding left u*S at or past the total
            owner = last;
            before = before_last;
        }
        if (owner != p.shard_index)
            return;                               // uniform over the workgroup
        base = before;
    }
    const double thr = static_cast<double>(ufin) * S;
    int first_cs, last_c;
    auto mass = [&](int k) {
        const ChunkMass q = staged ? s_cm[k] : cm[k];
        return use_p ? q.p : q.r;
    };
    {
        double run = base + (use_p ? inclp - myp : inclr - myr);
        int cs = kIdxNone, lastc = -1;
        for (int k = k0; k < k1; ++k) {
            const double X = mass(k);
            if (X > 0.0)
                lastc = k;
            if (cs == kIdxNone && run + X > thr)
                cs = k;
            run += X;
        }
        block_first_last(cs != kIdxNone, cs, lastc >= 0, lastc, first_cs, last_c);
    }
    // rounding can leave u*S at or past the total: take the last sub-chunk with mass
    const int cs = first_cs != kIdxNone ? first_cs : max(last_c, 0);
    if (cs >= k0 && cs < k1) {                    // the owner knows the mass before cs
        double run = base + (use_p ? inclp - myp : inclr - myr);
        for (int k = k0; k < cs; ++k)             // only when a thread owns several
            run += mass(k);
        s_before = run;
    }
    __syncthreads();

    const SampleRows<E> sr(p, b, len, st);
    const int v0 = cs * kRejSub + t * kSubPerThread;
    const int cnt = max(0, min(kSubPerThread, p.V - v0));
    double xs[kSubPerThread];
    double own = 0.0;
    sr.template visit<kSubPerThread, false>(v0, cnt, [&](int j, float a, float r) {
        xs[j] = static_cast<double>(use_p ? a : r) * sr.izt;
        own += xs[j];
    });
    double tot;
    const double incl = block_inclusive_scan(own, tot);
    double cum = s_before + (incl - own);
    int first = kIdxNone, lastpos = -1;
#pragma unroll
    for (int j = 0; j < kSubPerThread; ++j) {
        if (j < cnt) {
            const double x = xs[j];
            cum += x;
            if (x > 0.0) {
                lastpos = v0 + j;
                if (first == kIdxNone && cum > thr)
                    first = v0 + j;
            }
        }
    }
    int yf, yl;
    block_first_last(first != kIdxNone, first, lastpos >= 0, lastpos, yf, yl);
    const int y = p.v_offset + (yf != kIdxNone ? yf : yl);
    int *e = p.emitted + static_cast<int64_t>(b) * (K + 1);
    for (int k = t; k <= K; k += kThreads)
        e[k] = k < n ? (k == t ? d_own : d[k]) : (k == n ? y : -1);
}

template <typename E>
hipError_t launch_typed(const RejectParams &p, hipStream_t s)
{
    const int64_t items = static_cast<int64_t>(p.B) * (2 * p.K + 1) * p.segs;
    const dim3 g1(static_cast<unsigned>((items + kWaves - 1) / kWaves));
    if (sizeof(E) == 4 && p.probs)
        hipLaunchKernelGGL((k_rej_stats<E, kProbs>), g1, dim3(kThreads), 0, s, p);
    else if (sizeof(E) == 2 && p.split_ok)
        hipLaunchKernelGGL((k_rej_stats<E, kExpSplit>), g1, dim3(kThreads), 0, s, p);
    else if (p.inv_t == 1.0f)
        hipLaunchKernelGGL((k_rej_stats<E, kExpUnitT>), g1, dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((k_rej_stats<E, kExpScaled>), g1, dim3(kThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const dim3 g2(static_cast<unsigned>(static_cast<int64_t>(p.B) * p.nchunks));
    if (p.vec_ok)
        hipLaunchKernelGGL((k_rej_final<E, true>), g2, dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((k_rej_final_scalar<E, true>), g2, dim3(kThreads), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    hipLaunchKernelGGL((k_rej_select<E, false>), dim3(static_cast<unsigned>(p.B)), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

template <typename E>
hipError_t launch_shard_stats_typed(const RejectParams &p, SoftPartial *out, hipStream_t s)
{
    const int64_t rows = static_cast<int64_t>(p.B) * (2 * p.K + 1);
    const int64_t items = rows * p.segs;
    const dim3 g1(static_cast<unsigned>((items + kWaves - 1) / kWaves));
    RejectParams q = p;
    if (p.segs == 1)
        q.partial = out;                          // one segment per row: already merged
    if (sizeof(E) == 2 && p.split_ok)
        hipLaunchKernelGGL((k_rej_stats<E, kExpSplit>), g1, dim3(kThreads), 0, s, q);
    else if (p.inv_t == 1.0f)
        hipLaunchKernelGGL((k_rej_stats<E, kExpUnitT>), g1, dim3(kThreads), 0, s, q);
    else
        hipLaunchKernelGGL((k_rej_stats<E, kExpScaled>), g1, dim3(kThreads), 0, s, q);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.segs == 1)
        return e;
    hipLaunchKernelGGL(k_rej_shard_rows, dim3(static_cast<unsigned>((rows + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, s, p, out);
    return hipGetLastError();
}

template <typename E>
hipError_t launch_shard_mass_typed(const RejectParams &p, hipStream_t s)
{
    const dim3 g3(static_cast<unsigned>(static_cast<int64_t>(p.B) * p.nchunks));
    if (p.vec_ok)
        hipLaunchKernelGGL((k_rej_final<E, false>), g3, dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((k_rej_final_scalar<E, false>), g3, dim3(kThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(k_rej_shard_total, dim3(static_cast<unsigned>(p.B)), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

} // namespace

hipError_t launch_rejection(const RejectParams &p, int dtype, hipStream_t s)
{
    return dtype == SV_BF16 ? launch_typed<uint16_t>(p, s) : launch_typed<float>(p, s);
}

hipError_t launch_rejection_shard_stats(const RejectParams &p, int dtype, SoftPartial *out, hipStream_t s)
{
    return dtype == SV_BF16 ? launch_shard_stats_typed<uint16_t>(p, out, s)
                            : launch_shard_stats_typed<float>(p, out, s);
}

hipError_t launch_rejection_decide(const RejectParams &p, hipStream_t s)
{
    hipLaunchKernelGGL(k_rej_scan, dim3(static_cast<unsigned>((p.B + kWaves - 1) / kWaves)), dim3(kThreads), 0,
                       s, p);
    return hipGetLastError();
}

hipError_t launch_rejection_shard_mass(const RejectParams &p, int dtype, hipStream_t s)
{
    return dtype == SV_BF16 ? launch_shard_mass_typed<uint16_t>(p, s) : launch_shard_mass_typed<float>(p, s);
}

hipError_t launch_rejection_shard_sample(const RejectParams &p, int dtype, hipStream_t s)
{
    if (dtype == SV_BF16)
        hipLaunchKernelGGL((k_rej_select<uint16_t, true>), dim3(static_cast<unsigned>(p.B)), dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((k_rej_select<float, true>), dim3(static_cast<unsigned>(p.B)), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

} // namespace sv
