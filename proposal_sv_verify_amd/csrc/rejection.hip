// rejection.hip -- rejection-sampling verification on gfx950 (Leviathan et
// al. / Chen et al., the rule [vLLM-03] "1. principle" cites for keeping the
// target distribution at T > 0).
//
// Kernel 1 (row statistics).  One wave per (row, piece) over the K+1
// target rows and K draft rows of every sequence streams the logits once
// with 16-byte loads (the pieces are sized so that every wave of the launch
// is resident at once).  Each lane sums exp(l / T) against the fixed
// reference 0 (fp32 sums of 8 terms, fp64 across them).  For bf16 logits
// the hardware exp2 takes the exact product of l and log2(e)/T rounded to
// 16 bits, and the rounding is corrected to first order through a second
// sum, of the terms weighted by l; fp32 logits use the compensated exp
// (about one ulp either way).  The rare vectors whose fp32 sum leaves a
// wide range (logits above about 44 T, -inf entries, rows far below 0) go
// through a careful path with its own reference and fp64 rescales.  The
// wave combines its lanes onto their largest reference and writes
// (reference, sum).
//
// Kernel 2 (accept scan).  One workgroup per sequence: merge the segment
// statistics of each row in LDS, with the logits at the draft tokens that
// the statistics kernel captured, then one lane per draft position computes
// p_k(x_k) and q_k(x_k) with fp64 exp and the test u_k < p/q in fp64; a
// ballot of the rejections gives the first one, n.  The lane at position n
// publishes the statistics of row pair n.  (Running this inside kernel 3's
// workgroups instead was measured slower, 18.5-19.7 us against 5 + 9.6 us:
// every chunk then waits out the whole decision before loading its data.)
//
// Kernel 3 (final-sample masses).  The final token is drawn from one row
// pair: r = max(0, p_n - q_n) after a rejection (p_n when that sums to
// zero), or p_n when every draft was accepted.  One workgroup per (sequence,
// 4096-element chunk) forms p and r per element (fp32 exp, fp64 after);
// each wave publishes the masses of its 1024-element sub-chunk.
//
// Kernel 4 (selection).  One workgroup per sequence prefix-sums the
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

// The careful path for n values whose fast fp32 sum `s` is out of range.
template <bool kUnitT, int n>
__device__ __forceinline__ void careful_add(const float (&f)[n], float s, LaneSums &ls, float inv_t,
                                            double inv_t_d)
{
    // -inf values made the sum NaN: the same sum with -inf read as 0
    if (!(s == s)) {
        s = 0.0f;
#pragma unroll
        for (int j = 0; j < n; ++j)
            s += exp_cz(kUnitT ? f[j] : f[j] * inv_t);
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

// How the fast path forms e^(l/T).
enum ExpMode : int {
    kExpUnitT = 0,    // compensated exp of l (T == 1)
    kExpScaled = 1,   // compensated exp of l * (1/T)
    kExpSplit = 2,    // bf16 only: split constant, first-order correction summed apart
    kProbs = 3,       // the values are probabilities: summed as they are
};

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
    constexpr bool kUnitT = kMode == kExpUnitT;
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
                    careful_add<kUnitT>(f, s, ls, inv_t, inv_t_d);
            },
            [&](float x, int) {
                const float f1[1] = {x};
                const float s = vec_exp_sum<kMode>(f1, inv_t, c1, k2);
                if (kMode == kProbs || (s >= kTiny && s <= kBig)) {
                    ls.z0 += static_cast<double>(s);
                } else {
                    careful_add<kUnitT>(f1, s, ls, inv_t, inv_t_d);
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

// The accept decision of one sequence (steps a4 and the choice of row pair
// for a5), run by a whole workgroup: draft positions in blocks of 64.  A
// block needs the statistics of its target rows and draft rows: their
// segment partials are staged in LDS, each row's maximum is found, every
// partial is moved onto it (the fp64 rescales run in parallel, one thread per
// partial) and the row sums are formed; then wave 0 runs the accept test with
// one lane per position.  In LDS, target row base + i sits at slot i and
// draft row base + i at slot D0 + i, D0 = min(64, K + 1): for K < 64 the rows
// are packed (2K + 1 of them).  With `publish` the workgroup also writes the
// call's per-sequence outputs and the sequence state; every thread gets the
// state back.  The logits at the draft tokens come with the partials (the
// statistics kernel captures them); the "segments" are a row's pieces, or
// its vocabulary shards.
constexpr int kScanRows = 128;                                 // LDS row slots, at most
constexpr int kScanPer = kScanRows * kMaxSegs / kThreads;      // partials per thread, at most

__host__ __device__ constexpr int scan_rows(int K) { return (K + 1 < 64 ? K + 1 : 64) + (K < 64 ? K : 64); }

__host__ __device__ constexpr size_t scan_lds_bytes(int K, int segs)
{
    return static_cast<size_t>(scan_rows(K)) * (segs * 16 + 16) + sizeof(SeqState);
}

struct ScanLds {
    double *z;      // [rows * segs]
    double *Z;      // [rows]
    float *m;       // [rows * segs]
    float *M;       // [rows]
    float *lxs;     // [rows * segs] captured logits at the draft tokens (shard input)
    float *lx;      // [rows]
    SeqState *seq;

    __device__ ScanLds(char *base, int K, int segs)
    {
        const int rows = scan_rows(K);
        z = reinterpret_cast<double *>(base);
        Z = z + static_cast<size_t>(rows) * segs;
        seq = reinterpret_cast<SeqState *>(Z + rows);
        m = reinterpret_cast<float *>(seq + 1);
        M = m + static_cast<size_t>(rows) * segs;
        lxs = M + rows;
        lx = lxs + static_cast<size_t>(rows) * segs;
    }
};

__device__ __forceinline__ SeqState decide(const RejectParams &p, int b, bool publish, const ScanLds &S,
                                           int &len_out)
{
    const int t = threadIdx.x;
    const int lane = t & 63;
    const bool lead = t < 64;                 // wave 0 runs the per-position test
    const int K = p.K;
    const int segs = p.segs;
    const int D0 = K + 1 < 64 ? K + 1 : 64;
    const int64_t row0 = static_cast<int64_t>(b) * (2 * K + 1);
    int n = -1;                               // known to wave 0
    bool oor = false;
    unsigned fl = 0;
    int len = K;
    for (int base = 0; base <= K; base += 64) {
        const int nt = min(64, K + 1 - base);            // target rows of this block
        const int nd = max(0, min(64, K - base));        // draft rows of this block
        const int cnt = (nt + nd) * segs;
        const int k = base + lane;
        const int kc = max(0, min(k, K - 1));
        // the draft token first, so its logits can follow it (every wave
        // loads them; wave 0 uses them)
        const int x = p.draft[static_cast<int64_t>(b) * K + kc];
        // every thread: its partials of the block's rows
        SoftPartial q[kScanPer];
#pragma unroll
        for (int j = 0; j < kScanPer; ++j) {
            const int ci = min(t + j * kThreads, cnt - 1);
            const int rc = ci / segs;
            const int s = ci - rc * segs;
            const int ri = rc < nt ? base + rc : K + 1 + base + (rc - nt);   // row within the sequence
            q[j] = p.partial[(row0 + ri) * p.part_row_step + s * p.part_seg_step];
        }
        const bool valid = K > 0 && x >= 0 && x < p.v_full;
        const int xc = valid ? x : 0;
        (void)xc;
        const int len_raw = p.draft_len[b];
        len = p.has_len ? clamp_len(len_raw, K, fl) : K;
#pragma unroll
        for (int j = 0; j < kScanPer; ++j) {
            const int ci = t + j * kThreads;
            if (ci < cnt) {
                const int rc = ci / segs;
                const int s = ci - rc * segs;
                const bool tgt = rc < nt;
                const int kk = base + (tgt ? rc : rc - nt);
                const bool use = tgt ? kk <= len : kk < len;
                const int slot = (tgt ? rc : D0 + rc - nt) * segs + s;
                S.m[slot] = use ? q[j].m : -__builtin_inff();
                S.z[slot] = use ? q[j].z : 0.0;
                S.lxs[slot] = use ? q[j].lx : __builtin_nanf("");
            }
        }
        __syncthreads();
        const int srow = t < nt ? t : (t >= D0 && t < D0 + nd ? t : -1);   // an LDS row slot, or none
        if (srow >= 0) {
            float M = -__builtin_inff();
            float l = __builtin_nanf("");
            for (int s = 0; s < segs; ++s) {
                M = fmaxf(M, S.m[srow * segs + s]);
                const float c = S.lxs[srow * segs + s];
                if (c == c)
                    l = c;
            }
            S.M[srow] = M;
            S.lx[srow] = l;
        }
        __syncthreads();
        for (int ci = t; ci < cnt; ci += kThreads) {
            const int rc = ci / segs;
            const int s = ci - rc * segs;
            const int slot_row = rc < nt ? rc : D0 + rc - nt;
            const int slot = slot_row * segs + s;
            const float m = S.m[slot];
            const float M = S.M[slot_row];
            if (m != M)
                S.z[slot] = rescale(S.z[slot], m, M, p.inv_t_d);
        }
        __syncthreads();
        if (srow >= 0) {
            double Z = 0.0;
            for (int s = 0; s < segs; ++s)
                Z += S.z[srow * segs + s];
            S.Z[srow] = Z;
        }
        __syncthreads();
        if (lead) {
            oor |= k < len && !valid;
            const bool has_t = lane < nt, has_d = lane < nd;
            const double zt = has_t ? S.Z[lane] : 0.0, zd = has_d ? S.Z[D0 + lane] : 0.0;
            const float mt = has_t ? S.M[lane] : 0.0f, md = has_d ? S.M[D0 + lane] : 0.0f;
            const float lt = has_t ? S.lx[lane] : 0.0f;
            const float ld = has_d ? S.lx[D0 + lane] : 0.0f;
            double pk = 0.0, qk = 0.0;
            bool rejected = false;
            if (k < len) {
                double ratio = 0.0;
                if (valid) {
                    if (p.probs) {              // given probabilities: value over the row's sum
                        pk = static_cast<double>(lt) / zt;
                        qk = static_cast<double>(ld) / zd;
                    } else {
                        pk = exp((static_cast<double>(lt) - static_cast<double>(mt)) * p.inv_t_d) / zt;
                        qk = exp((static_cast<double>(ld) - static_cast<double>(md)) * p.inv_t_d) / zd;
                    }
                    ratio = qk > 0.0 ? pk / qk : __builtin_inf();
                }
                rejected = !(static_cast<double>(p.u[static_cast<int64_t>(b) * (K + 1) + k]) < ratio);
            }
            if (publish && k < K) {
                if (p.p_draft)
                    p.p_draft[static_cast<int64_t>(b) * K + k] = static_cast<float>(pk);
                if (p.q_draft)
                    p.q_draft[static_cast<int64_t>(b) * K + k] = static_cast<float>(qk);
            }
            const unsigned long long rej = __ballot(rejected);
            int here = -1;
            if (n < 0) {
                if (rej)
                    here = base + __builtin_ctzll(rej);
                else if (len < base + 64)
                    here = len;               // every draft accepted: the bonus row
            }
            if (here >= 0 && k == here) {
                SeqState sq{};
                sq.n = here;
                sq.len = len;
                sq.zt = zt;
                sq.mt = mt;
                if (here < len) {
                    sq.zd = zd;
                    sq.md = md;
                }
                *S.seq = sq;
                if (publish)
                    p.seq[b] = sq;
            }
            if (n < 0)
                n = here;
        }
        __syncthreads();                      // LDS is restaged by the next block
    }
    if (publish && lead) {
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
            for (int k = lane; k < n; k += 64)
                stats_add(p.stats + 3 + k, 1);
    }
    len_out = len;
    return *S.seq;                            // written before the last barrier
}

// Kernel 2: the accept decision, one workgroup per sequence.
__global__ __launch_bounds__(kThreads) void k_rej_scan(const RejectParams p)
{
    extern __shared__ __align__(16) char s_dyn[];
    const ScanLds S(s_dyn, p.K, p.segs);
    int len;
    decide(p, blockIdx.x, true, S, len);
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
// kN contiguous elements [v0, v0 + cnt).
template <typename E>
struct SampleRows {
    const E *pt;
    const E *pd;        // the target row again when sampling the bonus
    bool residual;      // a draft row is present: r is formed
    bool probs;         // the rows are probabilities: p_j = value / Z
    float mt, md;
    double izt, izd;
    float inv_t;
    int V;

    __device__ __forceinline__ SampleRows(const RejectParams &p, int b, int len, const SeqState &st)
    {
        const int K = p.K, n = st.n;
        pt = static_cast<const E *>(p.target) + (static_cast<int64_t>(b) * (K + 1) + n) * p.row_stride;
        mt = st.mt;
        izt = 1.0 / st.zt;
        inv_t = p.inv_t;
        V = p.V;
        probs = p.probs != 0;
        residual = n < len;
        pd = pt;
        md = 0.0f;
        izd = 0.0;
        if (residual) {
            pd = static_cast<const E *>(p.draftl) + (static_cast<int64_t>(b) * K + n) * p.row_stride;
            md = st.md;
            izd = 1.0 / st.zd;
        }
    }

    // visit(j, p_j, r_j) for j < cnt in order: p_j = exp((l - M) / T) / Z
    // (fp32 exp, fp64 after), or value / Z for probabilities; after a rejection r_j = max(0, p_j - q_j),
    // with no draft row r_j = 0.  Both rows are loaded before either is used.
    template <int kN, bool kVec, typename F>
    __device__ __forceinline__ void visit(int v0, int cnt, F &&f) const
    {
        Slice<E, kN, kVec> st, sd;
        st.fetch(pt, v0, V);
        sd.fetch(pd, v0, V);
        float ft[kN], fd[kN];
        st.widen(ft);
        sd.widen(fd);
#pragma unroll
        for (int j = 0; j < kN; ++j) {
            if (j < cnt) {
                const double a = probs ? static_cast<double>(ft[j]) * izt
                                       : static_cast<double>(exp_cz((ft[j] - mt) * inv_t)) * izt;
                double r = 0.0;
                if (residual) {
                    const double b = probs ? static_cast<double>(fd[j]) * izd
                                           : static_cast<double>(exp_cz((fd[j] - md) * inv_t)) * izd;
                    const double d = a - b;
                    r = d > 0.0 ? d : 0.0;
                }
                f(j, a, r);
            }
        }
    }
};

// The final-sample masses of one chunk of row pair n (step a5): p and
// r = max(0, p - q) per element, one mass pair per 1024-element sub-chunk.
template <typename E, bool kVec>
__device__ __forceinline__ void chunk_masses(const RejectParams &p, int b, int c, int len, const SeqState &st)
{
    const SampleRows<E> sr(p, b, len, st);
    const int v0 = c * kRejChunk + threadIdx.x * kChunkPerThread;
    const int cnt = max(0, min(kChunkPerThread, p.V - v0));
    double ps = 0.0, rs = 0.0;
    sr.template visit<kChunkPerThread, kVec>(v0, cnt, [&](int, double a, double r) {
        ps += a;
        rs += r;
    });
    ps = wave_sum(ps);
    rs = wave_sum(rs);
    if ((threadIdx.x & 63) == 0)
        p.cmass[(static_cast<int64_t>(b) * p.nchunks + c) * kSubPerChunk + (threadIdx.x >> 6)] =
            ChunkMass{rs, ps};
}

// Kernel 3: final-sample masses, one workgroup per (sequence, chunk), on
// the sequence state of the accept decision: two memory rounds (the state,
// then both rows' slices).
template <typename E, bool kVec>
__global__ __launch_bounds__(kThreads) void k_rej_chunks(const RejectParams p)
{
    const int b = blockIdx.x / p.nchunks;
    const int c = blockIdx.x - b * p.nchunks;
    const SeqState st = p.seq[b];
    chunk_masses<E, kVec>(p, b, c, st.len, st);
}

// A vocabulary shard's final-sample totals: the sum of its sub-chunk masses
// per sequence, in sub-chunk order (one workgroup per sequence).
__global__ __launch_bounds__(kThreads) void k_rej_shard_total(const RejectParams p)
{
    const int b = blockIdx.x;
    const int nsub = p.nchunks * kSubPerChunk;
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

// Kernel 4: one workgroup per sequence, two memory rounds.  Round 1 loads
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
    const int nsub = p.nchunks * kSubPerChunk;
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
    sr.template visit<kSubPerThread, false>(v0, cnt, [&](int j, double a, double r) {
        xs[j] = use_p ? a : r;
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
    const size_t lds = scan_lds_bytes(p.K, p.segs);
    hipLaunchKernelGGL(k_rej_scan, dim3(static_cast<unsigned>(p.B)), dim3(kThreads), lds, s, p);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    const dim3 g3(static_cast<unsigned>(static_cast<int64_t>(p.B) * p.nchunks));
    if (p.vec_ok)
        hipLaunchKernelGGL((k_rej_chunks<E, true>), g3, dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((k_rej_chunks<E, false>), g3, dim3(kThreads), 0, s, p);
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
        hipLaunchKernelGGL((k_rej_chunks<E, true>), g3, dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((k_rej_chunks<E, false>), g3, dim3(kThreads), 0, s, p);
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
    const size_t lds = scan_lds_bytes(p.K, p.segs);
    hipLaunchKernelGGL(k_rej_scan, dim3(static_cast<unsigned>(p.B)), dim3(kThreads), lds, s, p);
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
