// sv_device.hpp -- device helpers shared by the libspecverify kernels
// (gfx950, wave64).  Streaming loops over logit rows with 16-byte loads,
// (value, index) argmax combines with a total order, wave and workgroup
// reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specverify.h"

namespace sv {

constexpr int kThreads = 256;          // workgroup size of every kernel (4 waves)
constexpr int kWaves = kThreads / 64;
constexpr int kIdxNone = 0x7fffffff;   // "no element seen" index sentinel

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- elements

template <typename E> struct Elem;
template <> struct Elem<uint16_t> {   // bf16 bit patterns
    static constexpr int kPerVec = 8;
    __device__ static __forceinline__ float widen(uint16_t x) { return __uint_as_float(static_cast<unsigned>(x) << 16); }
    __device__ static __forceinline__ float one(const uint16_t *p, int64_t i) { return widen(p[i]); }
    __device__ static __forceinline__ void unpack(u32x4 q, float (&f)[8])
    {
        f[0] = __uint_as_float(q.x << 16);
        f[1] = __uint_as_float(q.x & 0xffff0000u);
        f[2] = __uint_as_float(q.y << 16);
        f[3] = __uint_as_float(q.y & 0xffff0000u);
        f[4] = __uint_as_float(q.z << 16);
        f[5] = __uint_as_float(q.z & 0xffff0000u);
        f[6] = __uint_as_float(q.w << 16);
        f[7] = __uint_as_float(q.w & 0xffff0000u);
    }
};
template <> struct Elem<float> {
    static constexpr int kPerVec = 4;
    __device__ static __forceinline__ float widen(float x) { return x; }
    __device__ static __forceinline__ float one(const float *p, int64_t i) { return p[i]; }
    __device__ static __forceinline__ void unpack(u32x4 q, float (&f)[4])
    {
        f[0] = __uint_as_float(q.x);
        f[1] = __uint_as_float(q.y);
        f[2] = __uint_as_float(q.z);
        f[3] = __uint_as_float(q.w);
    }
};

__device__ __forceinline__ u32x4 load16(const u32x4 *p)
{
    return __builtin_nontemporal_load(p);
}

// A 16-byte load with the default cache policy, for data read again soon.
__device__ __forceinline__ u32x4 load16_keep(const u32x4 *p)
{
    return *p;
}

// Visit elements [lo, hi) of one row with kSpan cooperating threads (a
// workgroup, or one wave); t is this thread's index among them.  Each thread
// sees its elements in increasing index order: one unaligned head element,
// then 16-byte vectors t, t + kSpan, ..., then one tail element; fvec(float
// (&)[kPerVec], first_index) and fone(float, index) receive them.  The
// vectors stream through a rolling pipeline: a ring of kDepth registers
// loaded in order, each slot processed and then refilled with the vector
// kDepth ahead, so kDepth - 1 loads stay in flight while a vector is
// processed and the thread only ever waits for its oldest load.  Loads past the last vector are
// clamped onto it (every load is issued unconditionally, which keeps the
// compiler's wait counts exact) and their data is dropped.
template <typename E, int kDepth, int kSpan, bool kKeep = false, typename FV, typename F1>
__device__ __forceinline__ void stream_segment(const E *row, int lo, int hi, int t, FV &&fvec, F1 &&fone)
{
    auto ld = [](const u32x4 *p) { return kKeep ? load16_keep(p) : load16(p); };
    constexpr int PV = Elem<E>::kPerVec;
    const uintptr_t addr = reinterpret_cast<uintptr_t>(row + lo);
    int head = static_cast<int>(((16u - (addr & 15u)) & 15u) / sizeof(E));
    if (head > hi - lo)
        head = hi - lo;
    if (t < head)
        fone(Elem<E>::one(row, lo + t), lo + t);
    const int a = lo + head;
    const int nvec = (hi - a) / PV;
    const u32x4 *vp = reinterpret_cast<const u32x4 *>(row + a);
    if (t < nvec) {
        const int last = nvec - 1;
        u32x4 q[kDepth];
#pragma unroll
        for (int u = 0; u < kDepth; ++u)
            q[u] = ld(vp + min(t + u * kSpan, last));
        for (int v = t; v < nvec; v += kDepth * kSpan) {
#pragma unroll
            for (int u = 0; u < kDepth; ++u) {
                const int vi = v + u * kSpan;
                if (vi < nvec) {
                    float f[PV];
                    Elem<E>::unpack(q[u], f);
                    fvec(f, a + vi * PV);
                }
                q[u] = ld(vp + min(vi + kDepth * kSpan, last));
            }
        }
    }
    const int t0 = a + nvec * PV;
    if (t < hi - t0)
        fone(Elem<E>::one(row, t0 + t), t0 + t);
}

// ---------------------------------------------------------------- argmax

// Total order used at every level: larger value first, then smaller index.
// -0.0 == +0.0 under float comparison, so they tie and the index decides.
__device__ __forceinline__ void arg_combine(float &bv, int &bi, float ov, int oi)
{
    if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
    }
}

template <int PV>
__device__ __forceinline__ void arg_visit_vec(float &bv, int &bi, const float (&f)[PV], int base)
{
    float m = f[0];
#pragma unroll
    for (int j = 1; j < PV; ++j)
        m = fmaxf(m, f[j]);
    if (m > bv) {
        int j = PV - 1;
#pragma unroll
        for (int k = PV - 2; k >= 0; --k)
            if (f[k] == m)
                j = k;
        bv = m;
        bi = base + j;
    }
}

// Workgroup argmax; the result is valid in thread 0.
__device__ __forceinline__ void block_argmax(float &bv, int &bi)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int oi = __shfl_xor(bi, off, 64);
        arg_combine(bv, bi, ov, oi);
    }
    __shared__ float s_v[kWaves];
    __shared__ int s_i[kWaves];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) {
        s_v[w] = bv;
        s_i[w] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int k = 1; k < kWaves; ++k)
            arg_combine(bv, bi, s_v[k], s_i[k]);
    }
    __syncthreads();
}

// ---------------------------------------------------------------- exp

// e^d in fp32 for d below about 80 (Cody-Waite reduction around the
// hardware exp2): y = d * log2(e) rounded, t = d - y * ln 2 formed with two
// FMAs (ln 2 split into its fp32 value and the remainder), e^d = 2^y * e^t
// with e^t = 1 + t since |t| < 2^-23 |d|.  Measured on gfx950 against fp64:
// at most 1.25 ulp, 0.33 ulp on average, over d in [-100, 0].  Finite
// arguments below about -87 give subnormals or 0; d = -inf gives NaN.
__device__ __forceinline__ float exp_c(float d)
{
    const float kLog2e = 1.44269504088896340736f;
    const float kLn2Hi = 0.693147182464599609375f;      // fp32(ln 2)
    const float kLn2Lo = -1.9046542999481136e-09f;      // ln 2 - kLn2Hi
    const float y = d * kLog2e;
    float t = __builtin_fmaf(-y, kLn2Hi, d);
    t = __builtin_fmaf(-y, kLn2Lo, t);
    const float e = __builtin_amdgcn_exp2f(y);
    return __builtin_fmaf(e, t, e);
}

// e^d for any d up to about 80, -inf included (gives 0): the argument is
// clamped to -256 first, where the result has underflowed to 0 anyway.
// exp_c itself would form -inf + inf = NaN in its correction term.
__device__ __forceinline__ float exp_cz(float d) { return exp_c(fmaxf(d, -256.0f)); }

// ---------------------------------------------------------------- reductions

__device__ __forceinline__ double wave_sum(double x)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        x += __shfl_xor(x, off, 64);
    return x;
}

__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        x = fmaxf(x, __shfl_xor(x, off, 64));
    return x;
}

// Inclusive prefix sum over the workgroup in thread order; `total` receives
// the workgroup sum (identical in every thread).  The association order is
// fixed by the code, so equal inputs always give bit-identical outputs.
__device__ __forceinline__ double block_inclusive_scan(double x, double &total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double y = __shfl_up(x, off, 64);
        if (lane >= off)
            x += y;
    }
    __shared__ double s_w[kWaves];
    if (lane == 63)
        s_w[w] = x;
    __syncthreads();
    double before = 0.0;
    for (int k = 0; k < w; ++k)
        before += s_w[k];
    double tot = 0.0;
    for (int k = 0; k < kWaves; ++k)
        tot += s_w[k];
    __syncthreads();
    total = tot;
    return before + x;
}

// Largest int over the workgroup, in every thread (two barriers).
__device__ __forceinline__ int block_max_int(int x)
{
    __shared__ int s_k[kWaves];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        x = max(x, __shfl_xor(x, off, 64));
    if ((threadIdx.x & 63) == 0)
        s_k[threadIdx.x >> 6] = x;
    __syncthreads();
    int m = s_k[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k)
        m = max(m, s_k[k]);
    __syncthreads();
    return m;
}

// First and last hits over the workgroup, for values that increase with the
// thread index: `first` receives vf of the lowest thread with has_f (kIdxNone
// if none), `last` vl of the highest thread with has_l (-1 if none).  One
// ballot per wave and one LDS slot per wave, no atomics; every thread gets
// the results.  Two barriers, so consecutive calls do not race on the slots.
__device__ __forceinline__ void block_first_last(bool has_f, int vf, bool has_l, int vl, int &first, int &last)
{
    __shared__ int s_f[kWaves], s_l[kWaves];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const unsigned long long bf = __ballot(has_f), bl = __ballot(has_l);
    if (lane == 0) {
        s_f[w] = bf ? __builtin_amdgcn_readlane(vf, __builtin_ctzll(bf)) : kIdxNone;
        s_l[w] = bl ? __builtin_amdgcn_readlane(vl, 63 - __builtin_clzll(bl)) : -1;
    }
    __syncthreads();
    first = kIdxNone;
    last = -1;
#pragma unroll
    for (int k = kWaves - 1; k >= 0; --k)
        if (s_f[k] != kIdxNone)
            first = s_f[k];
#pragma unroll
    for (int k = 0; k < kWaves; ++k)
        if (s_l[k] >= 0)
            last = s_l[k];
    __syncthreads();
}

// ---------------------------------------------------------------- misc

// Accumulate into a caller's statistics counter (relaxed device-scope
// atomic; the host reads the counters after the stream completes).
__device__ __forceinline__ void stats_add(int64_t *p, int64_t v)
{
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int clamp_len(int len, int K, unsigned &fl)
{
    if (len < 0) {
        fl |= SV_FLAG_BAD_LEN;
        return 0;
    }
    if (len > K) {
        fl |= SV_FLAG_BAD_LEN;
        return K;
    }
    return len;
}

} // namespace sv
