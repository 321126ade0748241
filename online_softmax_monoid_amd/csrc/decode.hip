// decode.hip -- split-KV decode attention on gfx950: a bandwidth-bound split
// kernel and a small combine kernel, both the online-softmax monoid.
//
// Split kernel (a7): one workgroup per (stream b, kv-head, group of GH query
// heads, split s). The split covers keys [floor(s*len/S), floor((s+1)*len/S))
// of the stream's cache. LPK = d/8 lanes share one key row (16 bytes each), so
// a 256-thread workgroup reads 256/LPK whole key rows per load instruction;
// each row of K and V is read from HBM exactly once and serves all GH query
// heads (the paper's decode kernel shares one set of probabilities across the
// GQA heads, §7.4 / appendix). Every lane group runs the monoid over its own
// keys, U keys per step with one rescale per step; the lane groups' states
// are then folded through LDS, and the unnormalised partial state
// (m, l, acc[d]) goes to the workspace.
//
// Combine kernel (a8): one wave per (b, query head) folds the S partial states
// with the monoid combine (rescale to the largest max, add) and finishes
// O = acc / l and LSE = m + ln l; a stream with no key gets O = +0, LSE = -inf.
// Splitting is valid because the combine is associative (§2.5 "Schedules":
// split on any associative monoid).
//
// Scores are kept in log2 units (q is pre-multiplied by scale*log2(e)) so
// every exponential is one v_exp_f32. Decode keeps the probabilities in f32.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "launch.h"

namespace miattn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
    bf16x2 p;
    p[0] = (__bf16)lo;
    p[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, p);
}

// Sum over the LPK lanes of a key group (aligned groups of LPK lanes).
template <int LPK>
__device__ __forceinline__ float group_sum(float x)
{
#pragma unroll
    for (int off = 1; off < LPK; off <<= 1)
        x += __shfl_xor(x, off, 64);
    return x;
}

template <int D, int GH, int U>
struct DecCfg {
    static constexpr int NT = 256;
    static constexpr int LPK = D / 8;        // lanes per key row
    static constexpr int NKG = NT / LPK;     // key groups per workgroup
    static constexpr int STEP = NKG * U;     // keys per loop step
};

template <int D, int GH, int U>
__global__ void __launch_bounds__(256)
decode_split_kernel(DecodeArgs a)
{
    using C = DecCfg<D, GH, U>;
    __shared__ float s_m[C::NKG][GH];
    __shared__ float s_l[C::NKG][GH];
    __shared__ __attribute__((aligned(16))) float s_acc[C::NKG][GH][D];

    const int tid = threadIdx.x;
    const int kgrp = tid / C::LPK;
    const int dl = tid % C::LPK;  // this lane's 8 dims: [8*dl, 8*dl + 8)

    const int G = a.Hq / a.Hkv;
    const int hchunks = G / GH;
    int id = blockIdx.x;
    const int split = id % a.splits;
    id /= a.splits;
    const int hc = id % hchunks;
    id /= hchunks;
    const int kvh = id % a.Hkv;
    const int b = id / a.Hkv;
    const int h0 = kvh * G + hc * GH;

    int len = a.lens[b];
    len = len < 0 ? 0 : (len > a.S_cap ? a.S_cap : len);
    const int k_lo = (int)(((int64_t)split * len) / a.splits);
    const int k_hi = (int)(((int64_t)(split + 1) * len) / a.splits);

    const float c = a.scale * kLog2e;
    float q[GH][8];
#pragma unroll
    for (int h = 0; h < GH; ++h) {
        const uint4 w = *(const uint4 *)(a.q + ((int64_t)b * a.Hq + h0 + h) * D + 8 * dl);
        q[h][0] = bf16_lo(w.x) * c; q[h][1] = bf16_hi(w.x) * c;
        q[h][2] = bf16_lo(w.y) * c; q[h][3] = bf16_hi(w.y) * c;
        q[h][4] = bf16_lo(w.z) * c; q[h][5] = bf16_hi(w.z) * c;
        q[h][6] = bf16_lo(w.w) * c; q[h][7] = bf16_hi(w.w) * c;
    }

    float m[GH], l[GH], acc[GH][8];
#pragma unroll
    for (int h = 0; h < GH; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[h][i] = 0.f;
    }

    const int64_t row0 = ((int64_t)b * a.Hkv + kvh) * a.S_cap;
    const uint16_t *Kp = a.k + row0 * D + 8 * dl;
    const uint16_t *Vp = a.v + row0 * D + 8 * dl;

    for (int kb = k_lo; kb < k_hi; kb += C::STEP) {
        uint4 kr[U], vr[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int key = kb + u * C::NKG + kgrp;
            ok[u] = key < k_hi;
            kr[u] = ok[u] ? *(const uint4 *)(Kp + (int64_t)key * D) : make_uint4(0, 0, 0, 0);
            vr[u] = ok[u] ? *(const uint4 *)(Vp + (int64_t)key * D) : make_uint4(0, 0, 0, 0);
        }
        float s[U][GH];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float k0 = bf16_lo(kr[u].x), k1 = bf16_hi(kr[u].x);
            const float k2 = bf16_lo(kr[u].y), k3 = bf16_hi(kr[u].y);
            const float k4 = bf16_lo(kr[u].z), k5 = bf16_hi(kr[u].z);
            const float k6 = bf16_lo(kr[u].w), k7 = bf16_hi(kr[u].w);
#pragma unroll
            for (int h = 0; h < GH; ++h) {
                float t = q[h][0] * k0;
                t = __builtin_fmaf(q[h][1], k1, t);
                t = __builtin_fmaf(q[h][2], k2, t);
                t = __builtin_fmaf(q[h][3], k3, t);
                t = __builtin_fmaf(q[h][4], k4, t);
                t = __builtin_fmaf(q[h][5], k5, t);
                t = __builtin_fmaf(q[h][6], k6, t);
                t = __builtin_fmaf(q[h][7], k7, t);
                s[u][h] = group_sum<C::LPK>(t);
            }
        }
#pragma unroll
        for (int h = 0; h < GH; ++h) {
            float mx = -INFINITY;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                s[u][h] = ok[u] ? s[u][h] : -INFINITY;
                mx = fmaxf(mx, s[u][h]);
            }
            const float m_new = fmaxf(m[h], mx);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m[h] - m_use);
            l[h] *= alpha;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[h][i] *= alpha;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float p = __builtin_amdgcn_exp2f(s[u][h] - m_use);
                l[h] += p;
                acc[h][0] = __builtin_fmaf(p, bf16_lo(vr[u].x), acc[h][0]);
                acc[h][1] = __builtin_fmaf(p, bf16_hi(vr[u].x), acc[h][1]);
                acc[h][2] = __builtin_fmaf(p, bf16_lo(vr[u].y), acc[h][2]);
                acc[h][3] = __builtin_fmaf(p, bf16_hi(vr[u].y), acc[h][3]);
                acc[h][4] = __builtin_fmaf(p, bf16_lo(vr[u].z), acc[h][4]);
                acc[h][5] = __builtin_fmaf(p, bf16_hi(vr[u].z), acc[h][5]);
                acc[h][6] = __builtin_fmaf(p, bf16_lo(vr[u].w), acc[h][6]);
                acc[h][7] = __builtin_fmaf(p, bf16_hi(vr[u].w), acc[h][7]);
            }
            m[h] = m_new;
        }
    }

    // fold the key groups' states through LDS
    if (dl == 0) {
#pragma unroll
        for (int h = 0; h < GH; ++h) {
            s_m[kgrp][h] = m[h];
            s_l[kgrp][h] = l[h];
        }
    }
#pragma unroll
    for (int h = 0; h < GH; ++h) {
        *(float4 *)&s_acc[kgrp][h][8 * dl] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
        *(float4 *)&s_acc[kgrp][h][8 * dl + 4] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
    }
    __syncthreads();

    const int64_t part0 = ((int64_t)b * a.Hq + h0) * a.splits + split;
    for (int e = tid; e < GH * D; e += C::NT) {
        const int h = e / D, dd = e % D;
        float M = -INFINITY;
        for (int kg = 0; kg < C::NKG; ++kg)
            M = fmaxf(M, s_m[kg][h]);
        float L = 0.f, A = 0.f;
        if (M != -INFINITY) {
            for (int kg = 0; kg < C::NKG; ++kg) {
                const float mk = s_m[kg][h];
                const float w = (mk == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mk - M);
                L = __builtin_fmaf(w, s_l[kg][h], L);
                A = __builtin_fmaf(w, s_acc[kg][h][dd], A);
            }
        }
        const int64_t p = part0 + (int64_t)h * a.splits;
        a.part_acc[p * D + dd] = A;
        if (dd == 0) {
            a.part_ml[2 * p] = M;
            a.part_ml[2 * p + 1] = L;
        }
    }
}

// One 64-lane wave per (b, query head); lane handles d/64 output dims.
template <int D>
__global__ void __launch_bounds__(64)
decode_combine_kernel(DecodeArgs a)
{
    constexpr int PER = D / 64;
    const int lane = threadIdx.x;
    const int64_t bh = blockIdx.x;
    const int S = a.splits;
    const float *ml = a.part_ml + bh * S * 2;
    const float *pa = a.part_acc + bh * S * D;

    float M = -INFINITY;
    for (int s = 0; s < S; ++s)
        M = fmaxf(M, ml[2 * s]);
    float L = 0.f;
    float o[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i)
        o[i] = 0.f;
    if (M != -INFINITY) {
        for (int s = 0; s < S; ++s) {
            const float ms = ml[2 * s];
            const float w = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - M);
            L = __builtin_fmaf(w, ml[2 * s + 1], L);
#pragma unroll
            for (int i = 0; i < PER; ++i)
                o[i] = __builtin_fmaf(w, pa[(int64_t)s * D + PER * lane + i], o[i]);
        }
    }
    const bool empty = !(L > 0.f);
    const float inv = empty ? 0.f : 1.f / L;
    uint16_t *orow = a.o + bh * D + PER * lane;
    if constexpr (PER == 1) {
        *orow = empty ? (uint16_t)0 : (uint16_t)(pack_bf16x2(o[0] * inv, 0.f) & 0xffffu);
    } else {
#pragma unroll
        for (int i = 0; i < PER; i += 2)
            *(uint32_t *)(orow + i) = empty ? 0u : pack_bf16x2(o[i] * inv, o[i + 1] * inv);
    }
    if (lane == 0)
        a.lse[bh] = empty ? -INFINITY : (M + __log2f(L)) * kLn2;
}

template <int D, int GH>
hipError_t launch_split(const DecodeArgs &a, hipStream_t stream)
{
    const int G = a.Hq / a.Hkv;
    const long long grid = (long long)a.B * a.Hkv * (G / GH) * a.splits;
    if (grid > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_split_kernel<D, GH, 4>), dim3((unsigned)grid), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs &a, hipStream_t stream)
{
    const int G = a.Hq / a.Hkv;
    hipError_t e;
    if (G % 4 == 0)
        e = launch_split<D, 4>(a, stream);
    else if (G % 2 == 0)
        e = launch_split<D, 2>(a, stream);
    else
        e = launch_split<D, 1>(a, stream);
    if (e != hipSuccess)
        return e;
    const long long grid = (long long)a.B * a.Hq;
    if (grid > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)grid), dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, int d, hipStream_t stream)
{
    switch (d) {
    case 64:
        return launch_d<64>(a, stream);
    case 128:
        return launch_d<128>(a, stream);
    case 256:
        return launch_d<256>(a, stream);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace miattn
