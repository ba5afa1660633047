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
    __device__ static __forceinline__ float one(const uint16_t *p, int64_t i)
    {
        return __uint_as_float(static_cast<unsigned>(p[i]) << 16);
    }
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

// Visit elements [lo, hi) of one row with the whole workgroup.  Each thread
// sees its elements in increasing index order: one unaligned head element,
// then 16-byte vectors (kUnroll independent loads in flight), then one tail
// element.  fvec(float (&)[kPerVec], first_index) and fone(float, index).
template <typename E, int kUnroll, typename FV, typename F1>
__device__ __forceinline__ void for_each_in_segment(const E *row, int lo, int hi, FV &&fvec,
                                                    F1 &&fone)
{
    constexpr int PV = Elem<E>::kPerVec;
    const int tid = threadIdx.x;
    const uintptr_t addr = reinterpret_cast<uintptr_t>(row + lo);
    int head = static_cast<int>(((16u - (addr & 15u)) & 15u) / sizeof(E));
    if (head > hi - lo)
        head = hi - lo;
    if (tid < head)
        fone(Elem<E>::one(row, lo + tid), lo + tid);
    const int a = lo + head;
    const int nvec = (hi - a) / PV;
    const u32x4 *vp = reinterpret_cast<const u32x4 *>(row + a);
    int v = tid;
    for (; v + (kUnroll - 1) * kThreads < nvec; v += kUnroll * kThreads) {
        u32x4 q[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            q[u] = load16(vp + v + u * kThreads);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float f[PV];
            Elem<E>::unpack(q[u], f);
            fvec(f, a + (v + u * kThreads) * PV);
        }
    }
    for (; v < nvec; v += kThreads) {
        float f[PV];
        Elem<E>::unpack(load16(vp + v), f);
        fvec(f, a + v * PV);
    }
    const int t0 = a + nvec * PV;
    if (tid < hi - t0)
        fone(Elem<E>::one(row, t0 + tid), t0 + tid);
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
