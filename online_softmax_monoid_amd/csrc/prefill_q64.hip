// prefill_q64.hip -- fused attention forward on gfx950, head dimension 128,
// 64 query rows per wave.
//
// Same operation and online-softmax monoid as prefill.hip. The schedule is
// shaped by the gfx950 LDS read bandwidth (about 150-200 bytes per ns per
// CU): with 32 query rows per wave every 16-byte K or V fragment read from LDS
// feeds one 32x32x16 MFMA, and the fragment traffic alone takes longer than
// the MFMAs. Here each wave owns two 32-row query blocks (64 rows), so every
// fragment feeds two MFMAs, halving LDS bytes per flop. The register file
// then holds one wave per SIMD (four waves, 256 query rows per workgroup),
// and each wave hides its own latencies by software pipelining:
//
//   stage A of tile j: S_{j+1} = K_{j+1} Q^T (16 MFMAs)  interleaved with
//       the second key chunk of tile j's probabilities (exp2, bf16 rounding,
//       row sums) and the transposing LDS reads of V_j's fragments;
//   stage B of tile j: O^T += V_j^T P_j (16 MFMAs)  interleaved with mask,
//       row max and lazy reference update of tile j+1, the first key chunk of
//       its probabilities, and the LDS reads of K_{j+2}'s fragments.
//
// K and V tiles of 32 keys go global -> LDS with range-checked buffer DMA
// (rows past Sk arrive as zeros) into four-deep rings, each buffer its own LDS
// array; one workgroup barrier per tile orders the rings. K rows carry a
// 16-byte-chunk XOR swizzle by row, V rows the swizzle that keeps the
// transposing reads free of bank conflicts (both as in prefill_pp.hip).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "launch.h"

namespace miattn {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kXcds = 8;
constexpr float kLog2e = 1.4426950408889634f;

template <int N>
struct IntC {
    static constexpr int value = N;
};

union Frag8 {
    bf16x8 v;
    uint4 u;
    uint32_t w[4];
};

__device__ __forceinline__ float halves_max(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float halves_sum(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2 p;
    p[0] = (__bf16)lo;
    p[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// keeps a value's computation before this point (see prefill_pp.hip)
__device__ __forceinline__ void pin(float &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(uint32_t &x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ int xcd_remap(int id, int n)
{
    const int per = n / kXcds;
    if (id < per * kXcds)
        return (id % kXcds) * per + id / kXcds;
    return id;
}

// V rows: 16-byte chunk c of row r sits at chunk c ^ vswz(r)
__device__ __forceinline__ int vswz(int r)
{
    return (0xEA40 >> (4 * (r & 3))) & 15;  // 0, 4, 10, 14 for r % 4 = 0..3
}

template <bool CAUSAL>
__global__ void __launch_bounds__(256, 1)
fwd_q64_kernel(FwdArgs a, int n_qtiles, int n_tiles)
{
    constexpr int D = 128;
    constexpr int QB = 2;             // 32-row query blocks per wave
    constexpr int BN = 32;            // keys per tile
    constexpr int BM = 4 * 32 * QB;   // query rows per workgroup
    constexpr int KCH = D / 8;        // 16-byte chunks per row
    constexpr int TILE_CH = BN * KCH; // 512 chunks = 8 KB = 8 DMA instructions

    __shared__ __attribute__((aligned(16))) uint4 sK0[TILE_CH];
    __shared__ __attribute__((aligned(16))) uint4 sK1[TILE_CH];
    __shared__ __attribute__((aligned(16))) uint4 sK2[TILE_CH];
    __shared__ __attribute__((aligned(16))) uint4 sK3[TILE_CH];
    __shared__ __attribute__((aligned(16))) uint4 sV0[TILE_CH];
    __shared__ __attribute__((aligned(16))) uint4 sV1[TILE_CH];
    __shared__ __attribute__((aligned(16))) uint4 sV2[TILE_CH];
    __shared__ __attribute__((aligned(16))) uint4 sV3[TILE_CH];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int g = lane >> 5;

    // ---- work decomposition (same order as prefill.hip) ---------------------
    const int G = a.Hq / a.Hkv;
    const int t = xcd_remap((int)blockIdx.x, n_tiles);
    const int per_unit = G * n_qtiles;
    const int unit = t / per_unit;
    const int rem = t - unit * per_unit;
    const int rank = rem / G;
    const int gq = rem - rank * G;
    const int qtile = CAUSAL ? (n_qtiles - 1 - rank) : rank;
    const int b = unit / a.Hkv;
    const int kvh = unit - b * a.Hkv;
    const int hq = kvh * G + gq;

    const int Sq = a.Sq, Sk = a.Sk;
    const int diag = Sk - Sq;
    const int64_t qrow0 = ((int64_t)b * a.Hq + hq) * Sq;
    const int64_t krow0 = ((int64_t)b * a.Hkv + kvh) * Sk;

    const int q_wg = qtile * BM;
    const int q_wg_last = min(q_wg + BM, Sq) - 1;
    const int q0 = q_wg + wave * 32 * QB;  // first row of this wave
    const bool wave_live = q0 < Sq;

    int kv_end = Sk;
    int wave_end = wave_live ? Sk : 0;
    if (CAUSAL) {
        kv_end = min(Sk, max(0, q_wg_last + diag + 1));
        if (wave_live)
            wave_end = min(Sk, max(0, min(q0 + 32 * QB - 1, Sq - 1) + diag + 1));
    }
    const int nblk = (kv_end + BN - 1) / BN;   // tiles the workgroup walks
    const int nwb = (wave_end + BN - 1) / BN;  // tiles this wave computes

    // ---- Q fragments (B operands of S^T = K Q^T) ------------------------------
    bf16x8 qf[QB][D / 16];
    {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + qrow0 * D, (uint32_t)Sq * D * 2);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const uint32_t off = (uint32_t)(q0 + 32 * qb + l32) * D * 2 + 16 * g;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                Frag8 f;
                f.u = buf_load16(rq, off + 32 * kk);  // rows >= Sq read as 0
                qf[qb][kk] = f.v;
            }
        }
    }

    // ---- global -> LDS copies: each wave issues 2 of a tile's 8 instructions --
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + krow0 * D, (uint32_t)Sk * D * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + krow0 * D, (uint32_t)Sk * D * 2);
    auto dma_k = [&](uint4 *buf, int tile) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int i = 2 * wave + h;
            const int r = 4 * i + (lane >> 4);
            const int c = (lane & 15) ^ (r & 15);
            const uint32_t off = ((uint32_t)(tile * BN + r) * D + 8 * c) * 2;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)(buf + 64 * i), 16, (int)off,
                                                     0, 0, 0);
        }
    };
    auto dma_v = [&](uint4 *buf, int tile) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int i = 2 * wave + h;
            const int r = 4 * i + (lane >> 4);
            const int c = (lane & 15) ^ vswz(r);
            const uint32_t off = ((uint32_t)(tile * BN + r) * D + 8 * c) * 2;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(buf + 64 * i), 16, (int)off,
                                                     0, 0, 0);
        }
    };

    // ---- fragments from LDS ---------------------------------------------------
    Frag8 kf[D / 16];   // K rows l32 of the tile, per 16-dim step
    bf16x8 vf[4][2];    // V^T rows 32 db + l32, per (d-block, 16-key chunk)
    auto read_k = [&](const uint4 *buf) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            kf[kk].u = buf[l32 * KCH + ((2 * kk + g) ^ (l32 & 15))];
    };
    // transposing reads: lane L = 16 G + 4 jr + q addresses row
    // 16 kc + 8 hh + 4 (G / 2) + jr at column 32 db + 16 (G % 2) + 4 q
    auto read_v = [&](const uint4 *buf) __attribute__((always_inline)) {
        const int G4 = lane >> 4, i = lane & 15;
        const int jr = i >> 2, q = i & 3;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                i16x4 half[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int row = 16 * kc + 8 * hh + 4 * (G4 >> 1) + jr;
                    const int c = 4 * db + 2 * (G4 & 1) + (q >> 1);
                    const char *p = (const char *)buf + row * (D * 2) + 16 * (c ^ vswz(row)) +
                                    8 * (q & 1);
                    half[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)(const_cast<char *>(p)));
                }
                const i16x8 both = __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7);
                vf[db][kc] = __builtin_bit_cast(bf16x8, both);
            }
    };

    // ---- monoid state per query block -----------------------------------------
    constexpr float kLazy = 8.f;
    const float c = a.scale * kLog2e;
    const float thr = kLazy / c;
    float m_ref[QB], mc[QB], alpha_acc[QB], l_half[QB];
    f32x16 acc[QB][D / 32];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_ref[qb] = -INFINITY;
        mc[qb] = 0.f;
        alpha_acc[qb] = 1.f;
        l_half[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[qb][db][r] = 0.f;
    }

    using Sc = f32x16[QB];
    using Pc = Frag8[QB];
    auto qk = [&](Sc &s) __attribute__((always_inline)) {
        // Q fragments stay in AGPRs, read there directly by the MFMAs (else
        // the allocator parks them in AGPRs and copies them back every tile)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
                asm volatile("" : "+a"(qf[qb][kk]));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                s[qb][r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk].v, qf[qb][kk], s[qb], 0, 0, 0);
    };
    // probabilities of key chunk h (scores s[8h .. 8h+7]) -> bf16 fragments
    auto probs = [&](const Sc &s, int h, Pc &p) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float rs = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][8 * h + 2 * w], c, -mc[qb]));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][8 * h + 2 * w + 1], c, -mc[qb]));
                p[qb].w[w] = pack_bf16x2(p0, p1);
                rs += p0 + p1;
            }
            l_half[qb] += rs;
        }
    };
    // last key of tile j this row may see; -1 when the wave computes nothing
    // for tile j (all of its probabilities are then exactly 0)
    auto mask_lim = [&](int j, int qb) __attribute__((always_inline)) {
        const int my_q = q0 + 32 * qb + l32;
        const int lim = CAUSAL ? min(Sk - 1, my_q + diag) : Sk - 1;
        return j < nwb ? lim : -1;
    };
    // mask (MASK), row max and lazy update of the reference for tile j
    auto row_stats = [&](Sc &s, int j, auto MASKc) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            if (decltype(MASKc)::value) {
                const int j0 = j * BN;
                const int lim = mask_lim(j, qb);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = j0 + 8 * (r >> 2) + 4 * g + (r & 3);
                    s[qb][r] = (key <= lim) ? s[qb][r] : -INFINITY;
                }
            }
            float mx = s[qb][0];
#pragma unroll
            for (int r = 1; r < 16; ++r)
                mx = fmaxf(mx, s[qb][r]);
            mx = halves_max(mx);
            const bool move = __any(mx > m_ref[qb] + thr);
            const float m_new = move ? fmaxf(m_ref[qb], mx) : m_ref[qb];
            const float alpha =
                (m_new == m_ref[qb]) ? 1.f : __builtin_amdgcn_exp2f((m_ref[qb] - m_new) * c);
            l_half[qb] *= alpha;
            alpha_acc[qb] *= alpha;
            m_ref[qb] = m_new;
            mc[qb] = (m_new == -INFINITY) ? 0.f : m_new * c;
        }
    };
    auto pv = [&](const Pc &p0, const Pc &p1) __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db][0], p0[qb].v, acc[qb][db], 0, 0, 0);
                acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db][1], p1[qb].v, acc[qb][db], 0, 0, 0);
            }
    };
    auto apply_alpha = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            if (__any(alpha_acc[qb] != 1.f)) {
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acc[qb][db][r] *= alpha_acc[qb];
            }
            alpha_acc[qb] = 1.f;
        }
    };
    auto pin_p = [&](Pc &p) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int w = 0; w < 4; ++w)
                pin(p[qb].w[w]);
    };
    auto pin_stats = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            pin(l_half[qb]);
            pin(m_ref[qb]);
            pin(mc[qb]);
            pin(alpha_acc[qb]);
        }
    };

    // ---- prologue ---------------------------------------------------------------
    // Copies of K tiles 0-3 and V tiles 0-2, drained; every wave computes S_0,
    // its statistics and P_0's first key chunk, then reads K tile 1.
    dma_k(sK0, 0);
    dma_k(sK1, 1);
    dma_k(sK2, 2);
    dma_k(sK3, 3);
    dma_v(sV0, 0);
    dma_v(sV1, 1);
    dma_v(sV2, 2);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q and the copies
    __syncthreads();
    Sc sA, sB;            // scores of tiles j (even) and j+1
    Pc pA, pA2, pB, pB2;  // probabilities: key chunks 0 and 1 of each tile
    read_k(sK0);
    qk(sA);
    row_stats(sA, 0, IntC<1>{});
    probs(sA, 0, pA);
    read_k(sK1);
    __syncthreads();      // everyone has read K tile 0 before K tile 4 replaces it

    // ---- one tile step ------------------------------------------------------------
    // Tile m's K lives in buffer m % 4, its V likewise. Step j: copies of K tile
    // j+4 (into tile j's K buffer, last read in step j-2) and V tile j+3 (into
    // tile j-1's V buffer, last read in step j-1); stage A; stage B; wait until
    // the copies the next step reads (K tile j+3, V tile j+1) are complete --
    // the six newer copy instructions of this wave may still fly; barrier.
    auto step = [&](auto PI, auto MASKc, int j, Sc &sc, Sc &sn, Pc &pc0, Pc &pc1, Pc &pn0)
        __attribute__((always_inline)) {
        constexpr int P = decltype(PI)::value;  // j % 4
        uint4 *const kb[4] = {sK0, sK1, sK2, sK3};
        uint4 *const vb[4] = {sV0, sV1, sV2, sV3};
        dma_k(kb[P], j + 4);
        dma_v(vb[(P + 3) & 3], j + 3);
        // stage A
        apply_alpha();
        qk(sn);
        read_v(vb[P]);
        probs(sc, 1, pc1);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
        }
        pin_p(pc1);
        pin_stats();
        // stage B
        pv(pc0, pc1);
        read_k(kb[(P + 2) & 3]);
        row_stats(sn, j + 1, MASKc);
        probs(sn, 0, pn0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            if (i < 8)
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
            __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // VALU
        }
        pin_p(pn0);
        pin_stats();
        __builtin_amdgcn_s_waitcnt(0x0F76);  // vmcnt(6)
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    // Leading steps of this wave that need no mask (a multiple of 4): tile j+1
    // fully visible to every row of the wave and within its range.
    int n_fast;
    {
        int first_masked = Sk / BN;  // ragged key tail
        if (CAUSAL)
            first_masked = min(first_masked, max(0, (q0 + diag + 1) / BN));
        n_fast = min(nwb, first_masked) - 1;
        n_fast = max(0, n_fast) & ~3;
        n_fast = __builtin_amdgcn_readfirstlane(n_fast);
    }

    int j = 0;
    for (; j < n_fast; j += 4) {
        step(IntC<0>{}, IntC<0>{}, j, sA, sB, pA, pA2, pB);
        step(IntC<1>{}, IntC<0>{}, j + 1, sB, sA, pB, pB2, pA);
        step(IntC<2>{}, IntC<0>{}, j + 2, sA, sB, pA, pA2, pB);
        step(IntC<3>{}, IntC<0>{}, j + 3, sB, sA, pB, pB2, pA);
    }
    for (; j + 3 < nblk; j += 4) {
        step(IntC<0>{}, IntC<1>{}, j, sA, sB, pA, pA2, pB);
        step(IntC<1>{}, IntC<1>{}, j + 1, sB, sA, pB, pB2, pA);
        step(IntC<2>{}, IntC<1>{}, j + 2, sA, sB, pA, pA2, pB);
        step(IntC<3>{}, IntC<1>{}, j + 3, sB, sA, pB, pB2, pA);
    }
    if (j < nblk)
        step(IntC<0>{}, IntC<1>{}, j, sA, sB, pA, pA2, pB);
    if (j + 1 < nblk)
        step(IntC<1>{}, IntC<1>{}, j + 1, sB, sA, pB, pB2, pA);
    if (j + 2 < nblk)
        step(IntC<2>{}, IntC<1>{}, j + 2, sA, sB, pA, pA2, pB);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // no copy may still target LDS
    apply_alpha();

    // ---- epilogue ------------------------------------------------------------------
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int my_q = q0 + 32 * qb + l32;
        const float l_tot = halves_sum(l_half[qb]);
        if (my_q < Sq) {
            const bool empty = !(l_tot > 0.f);
            const float inv = empty ? 0.f : 1.f / l_tot;
            uint16_t *orow = a.o + (qrow0 + my_q) * D + 4 * g;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int rho = 0; rho < 4; ++rho) {
                    uint2 w;
                    if (empty) {
                        w = make_uint2(0, 0);
                    } else {
                        w.x = pack_bf16x2(acc[qb][db][4 * rho] * inv, acc[qb][db][4 * rho + 1] * inv);
                        w.y = pack_bf16x2(acc[qb][db][4 * rho + 2] * inv, acc[qb][db][4 * rho + 3] * inv);
                    }
                    *(uint2 *)(orow + 32 * db + 8 * rho) = w;
                }
            if (g == 0)
                a.lse[qrow0 + my_q] = empty ? -INFINITY : m_ref[qb] * a.scale + logf(l_tot);
        }
    }
}

}  // namespace

hipError_t launch_fwd_q64(const FwdArgs &a, bool causal, hipStream_t stream)
{
    constexpr int BM = 256;
    const int n_qtiles = (a.Sq + BM - 1) / BM;
    const long long n_tiles = (long long)a.B * a.Hq * n_qtiles;
    if (n_tiles > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;
    if (causal)
        hipLaunchKernelGGL(fwd_q64_kernel<true>, dim3((unsigned)n_tiles), dim3(256), 0, stream, a,
                           n_qtiles, (int)n_tiles);
    else
        hipLaunchKernelGGL(fwd_q64_kernel<false>, dim3((unsigned)n_tiles), dim3(256), 0, stream,
                           a, n_qtiles, (int)n_tiles);
    return hipGetLastError();
}

}  // namespace miattn
