// prefill_pingpong.hip -- fused attention forward on gfx950 for head
// dimension 128: eight waves of 32 query rows, two per SIMD, that take turns
// on the matrix core.
//
// Same operation and online-softmax monoid as prefill.hip; same tile shapes,
// LDS layouts and DMA scheme as prefill_q64.hip. What differs is the schedule.
// At head dimension 128 the softmax of a 32 x 32 score tile (one exp, one
// FMA, one add, half a pack and about two thirds of a max per score) needs
// about as many VALU cycles as the tile's 16 MFMAs keep the matrix core
// busy, so the two only reach full rate when they overlap almost perfectly.
// Inside one wave that overlap is limited by the softmax's dependent chains.
// Here the two waves sharing a SIMD split the roles instead:
//
//   MFMA phase (step j):  copies of K_{j+4} and V_{j+3}; bf16 packing of tile
//                         j's exponentials and their f32 row sum, placed
//                         between PV of tile j (8 MFMAs) and QK of tile j+1
//                         (8 MFMAs, the first four alternating with the last
//                         four PV); every MFMA operand is in registers
//   VALU phase (step j):  LDS reads of the V_{j+1} fragments; mask, row
//                         maximum, lazy reference update and exp2 of S_{j+1}
//                         (in place of the scores); LDS reads of the K_{j+2}
//                         fragments
//
// Every phase ends at a workgroup barrier. Waves 0-3 start with their first
// MFMA phase while waves 4-7 wait one barrier, so from then on one wave of
// each SIMD runs MFMAs while the other runs its softmax, and they swap at
// each barrier (a workgroup's waves are placed on the SIMDs round-robin, so
// waves w and w+4 share one). The MFMA-phase wave raises its issue priority
// so that its next MFMA goes out as soon as the matrix core frees up.
//
// K / V ring (four tiles each). With barrier slots numbered from the first
// MFMA phase, waves 0-3 run MFMA(j) in slot 2j+2 and VALU(j) in slot 2j+3,
// waves 4-7 one slot later. K tile t is read in VALU(t-2) and V tile t in
// VALU(t-1), last in slots 2t and 2t+2, and a wave consumes what it reads in
// its next phase. A wave issues the copies of K_{j+4} and V_{j+3} in its
// MFMA(j) (slot 2j+2 or 2j+3), after the tiles they replace (K_j, V_{j-1})
// were last read in slot 2j and consumed in slot 2j+1, and waits for them by
// the end of slot 2j+6 (waves 0-3: end of MFMA(j+2), with the four newer
// copies still in flight; waves 4-7: end of VALU(j+1), with the two newer
// ones in flight), before any wave reads them in slot 2j+7.
//
// Causal masking: a wave walks the workgroup's tiles but skips the MFMAs
// and the softmax of tiles it cannot see, which leaves the SIMD to its
// partner; tiles it sees partly are masked by a select before the maximum.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "launch.h"
#include "lds_copy.h"
#include "tile_order.h"

namespace miattn {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;

union Frag8 {
    bf16x8 v;
    uint4 u;
    uint32_t w[4];
};

template <int N>
struct IntC {
    static constexpr int value = N;
};

__device__ __forceinline__ float fmax_ieee(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float uniform_f(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

__device__ __forceinline__ float halves_max(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmax_ieee(__uint_as_float(r[0]), __uint_as_float(r[1]));
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

__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

#ifndef MIATTN_PP_PRIO
#define MIATTN_PP_PRIO 1
#endif

template <bool CAUSAL>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_pingpong_kernel(FwdArgs a, int n_qtiles)
{
    constexpr int D = 128;
    constexpr int NWV = 8;
    constexpr int BN = 32;             // keys per tile
    constexpr int BM = NWV * 32;       // query rows per workgroup
    constexpr int KKN = D / 16;        // 16-dim steps of QK = copy instructions per tile
    constexpr int DBN = D / 32;        // 32-dim blocks of the output
    constexpr int TILE_CH = BN * D / 8;  // 16-byte chunks per tile
    static_assert(KKN == NWV, "one copy instruction per wave per tile");

    // One array per ring slot, addressed with compile-time slot numbers: the
    // compiler then sees that an LDS read and an in-flight copy into another
    // slot cannot alias, and does not drain the copies before every read.
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
    const TileOrder to = tile_order((int)blockIdx.x, a.B * a.Hkv, G, n_qtiles, CAUSAL);
    const int unit = to.unit, gq = to.gq, qtile = to.qtile;
    const int b = unit / a.Hkv;
    const int kvh = unit - b * a.Hkv;
    const int hq = kvh * G + gq;

    const int Sq = a.Sq, Sk = a.Sk;
    const int diag = Sk - Sq;
    const int64_t qrow0 = ((int64_t)b * a.Hq + hq) * Sq;
    const int64_t krow0 = ((int64_t)b * a.Hkv + kvh) * Sk;

    const int q_wg = qtile * BM;
    const int q_wg_last = min(q_wg + BM, Sq) - 1;
    const int q0 = q_wg + wave * 32;  // first row of this wave
    const bool wave_live = q0 < Sq;

    int kv_end = Sk;
    int wave_end = wave_live ? Sk : 0;
    if (CAUSAL) {
        kv_end = min(Sk, max(0, q_wg_last + diag + 1));
        if (wave_live)
            wave_end = min(Sk, max(0, min(q0 + 31, Sq - 1) + diag + 1));
    }
    const int nblk = (kv_end + BN - 1) / BN;   // tiles the workgroup walks
    const int nwb = (wave_end + BN - 1) / BN;  // tiles this wave computes
    // first tile of this wave that needs a mask (ragged key tail or diagonal)
    int first_masked = Sk / BN;
    if (CAUSAL)
        first_masked = min(first_masked, max(0, (q0 + diag + 1) / BN));
    first_masked = __builtin_amdgcn_readfirstlane(first_masked);

    // ---- Q fragments (B operands of S^T = K Q^T) ------------------------------
    bf16x8 qf[KKN];
    {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + qrow0 * D, (uint32_t)Sq * D * 2);
        const uint32_t off = (uint32_t)(q0 + l32) * D * 2 + 16 * g;
#pragma unroll
        for (int kk = 0; kk < KKN; ++kk) {
            Frag8 f;
            f.u = buf_load16(rq, off + 32 * kk);  // rows >= Sq read as 0
            qf[kk] = f.v;
        }
    }

    // ---- global -> LDS copies (layouts as in prefill_q64.hip) -------------------
    // K block kk (1 KB) holds lane L's A fragment for dims 16kk + 8(L/32) .. +7
    // of key L%32, at byte 16L. V block r = (2 db + kc) * 2 + hh (512 B) holds,
    // at byte 8L for L = 16G + 4jj + q, the four values V[16kc + 8hh + 4(G/2)
    // + jj][32db + 16(G%2) + 4q .. +3]; a transposing 8-byte read gives lane L
    // the values of dim 32db + L%32 at four consecutive keys. Wave w copies
    // block w of each tile.
    uint32_t koff, voff;
    {
        const int i = wave;
        koff = (uint32_t)(l32 * D + 16 * i + 8 * g) * 2;
        const int db = i >> 1, kc = i & 1, tt = l32;
        const int G4 = tt >> 3, jj = (tt >> 1) & 3, qh = tt & 1;
        const int key = 16 * kc + 8 * g + 4 * (G4 >> 1) + jj;
        const int dim = 32 * db + 16 * (G4 & 1) + 8 * qh;
        voff = (uint32_t)(key * D + dim) * 2;
    }
    const uint16_t *const kbase = a.k + krow0 * D;
    const uint16_t *const vbase = a.v + krow0 * D;
    // keys at or past kv_end (at most Sk; no row of the workgroup sees them)
    // arrive as zeros, and tiles past the range cost no memory traffic
    auto tile_desc = [&](const uint16_t *base, int tile) __attribute__((always_inline)) {
        const int keys = min(max(kv_end - tile * BN, 0), BN);
        return make_desc(base + (int64_t)tile * (BN * D), (uint32_t)keys * (D * 2));
    };
    auto dma_k = [&](uint4 *buf, int tile) __attribute__((always_inline)) {
        copy_to_lds(tile_desc(kbase, tile), koff, lds_addr(buf + 64 * wave));
    };
    auto dma_v = [&](uint4 *buf, int tile) __attribute__((always_inline)) {
        copy_to_lds(tile_desc(vbase, tile), voff, lds_addr(buf + 64 * wave));
    };

    // ---- fragments from LDS -------------------------------------------------------
    Frag8 kf[KKN];      // A fragments of the K tile the next QK uses
    bf16x8 vf[DBN][2];  // A fragments of V^T: [d-block][16-key chunk]
    auto read_k = [&](const uint4 *buf) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < KKN; ++kk)
            kf[kk].u = buf[64 * kk + lane];
    };
    auto read_v = [&](const uint4 *buf) __attribute__((always_inline)) {
        const char *base = (const char *)buf + 8 * lane;
#pragma unroll
        for (int db = 0; db < DBN; ++db)
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4 *)(const_cast<char *>(base + ((2 * db + kc) * 2 + 0) * 512)));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4 *)(const_cast<char *>(base + ((2 * db + kc) * 2 + 1) * 512)));
                const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                vf[db][kc] = __builtin_bit_cast(bf16x8, both);
            }
    };

    // ---- monoid state ---------------------------------------------------------------
    constexpr float kLazy = 8.f;  // the reference moves only past 2^8
    const float c = uniform_f(a.scale * kLog2e);
    const float thr = uniform_f(kLazy / c);
    float m_ref = -INFINITY, nmc = 0.f, m_thr = -INFINITY, l_half = 0.f;  // nmc = -m_ref * c
    f32x16 acc[DBN];
#pragma unroll
    for (int db = 0; db < DBN; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[db][r] = 0.f;
    // Scores of the tile in flight (key 8(r/4) + 4g + r%4, query l32); the
    // VALU phase replaces them by their exponentials exp2(s c - m_ref c),
    // which the next MFMA phase packs before its QK MFMAs write new scores.
    f32x16 s;
    Frag8 p[2];  // the bf16 probabilities, one B fragment per 16-key chunk
#pragma unroll
    for (int r = 0; r < 16; ++r)
        s[r] = 0.f;

    // MFMA phase of step j: copies of K_{j+4} and V_{j+3}; bf16 packing of
    // tile j's exponentials, PV of tile j with the f32 row sum between the
    // MFMAs, then QK of tile j+1 (its K fragments, read last in the VALU
    // phase, get the PV MFMAs' time to arrive). PV MFMAs on one accumulator
    // are four apart; the last four QK are back to back.
    auto mfma_phase = [&](int j, uint4 *kdst, uint4 *vdst) __attribute__((always_inline)) {
#if MIATTN_PP_PRIO
        __builtin_amdgcn_s_setprio(1);
#endif
        dma_k(kdst, j + 4);
        dma_v(vdst, j + 3);
        fence();
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                p[h].w[i] = pack_bf16x2(s[8 * h + 2 * i], s[8 * h + 2 * i + 1]);
        l_half += (((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]))) +
                  (((s[8] + s[9]) + (s[10] + s[11])) + ((s[12] + s[13]) + (s[14] + s[15])));
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i][0], p[0].v, acc[i], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i].v, qf[i], i == 0 ? f32x16{} : s, 0, 0, 0);
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i][1], p[1].v, acc[i], 0, 0, 0);
        }
#pragma unroll
        for (int i = 4; i < 8; ++i)
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i].v, qf[i], s, 0, 0, 0);
        // interleave: each MFMA followed by up to two of the pack / sum VALU ops
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
        }
        fence();
    };

    // softmax of tile t's scores up to the exponentials (monoid update of the
    // row state; packing and row sum follow in the next MFMA phase)
    auto softmax = [&](int t, bool masked) __attribute__((always_inline)) {
        if (masked) {
            const int my_q = q0 + l32;
            const int lim = CAUSAL ? min(Sk - 1, my_q + diag) : Sk - 1;
            const int rel = lim - t * BN - 4 * g;  // key r visible iff offset(r) <= rel
#pragma unroll
            for (int r = 0; r < 16; ++r)
                s[r] = (8 * (r >> 2) + (r & 3) <= rel) ? s[r] : -INFINITY;
        }
        float m0 = fmax_ieee(fmax_ieee(s[0], s[1]), s[2]);
        float m1 = fmax_ieee(fmax_ieee(s[8], s[9]), s[10]);
        m0 = fmax_ieee(fmax_ieee(m0, s[3]), s[4]);
        m1 = fmax_ieee(fmax_ieee(m1, s[11]), s[12]);
        m0 = fmax_ieee(fmax_ieee(m0, s[5]), s[6]);
        m1 = fmax_ieee(fmax_ieee(m1, s[13]), s[14]);
        m0 = fmax_ieee(fmax_ieee(m0, s[7]), m1);
        const float mx = halves_max(fmax_ieee(m0, s[15]));
        if (__any(mx > m_thr)) {  // lazy reference update, rare after the first tiles
            const float m_new = fmax_ieee(m_ref, mx);
            const float alpha = (m_new == m_ref) ? 1.f : __builtin_amdgcn_exp2f((m_ref - m_new) * c);
            l_half *= alpha;
            if (__any(alpha != 1.f)) {
#pragma unroll
                for (int db = 0; db < DBN; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acc[db][r] *= alpha;
            }
            m_ref = m_new;
            nmc = (m_new == -INFINITY) ? 0.f : -(m_new * c);
            m_thr = m_new + thr;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
            s[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, nmc));
    };

    // VALU phase of step j: LDS reads of the V_{j+1} fragments, softmax of
    // S_{j+1} up to its exponentials, LDS reads of the K_{j+2} fragments
    auto valu_phase = [&](int j, bool live, bool masked, bool rd_k, const uint4 *ksrc, const uint4 *vsrc)
        __attribute__((always_inline)) {
#if MIATTN_PP_PRIO
        __builtin_amdgcn_s_setprio(0);
#endif
        if (live) {
            read_v(vsrc);
            softmax(j + 1, masked);
        }
        fence();
        if (rd_k)
            read_k(ksrc);
        fence();
    };

    // ---- prologue ------------------------------------------------------------------
    dma_k(sK0, 0);
    dma_k(sK1, 1);
    dma_k(sK2, 2);
    dma_k(sK3, 3);
    dma_v(sV0, 0);
    dma_v(sV1, 1);
    dma_v(sV2, 2);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q and the copies
    __syncthreads();
    read_k(sK0);

    // A live step j < nwb computes QK of tile j+1 even when the wave cannot
    // see that tile (j = nwb-1): the tile then lies past the wave's last key,
    // so the mask hides all of it and its softmax is skipped anyway. A dead
    // step only issues the wave's share of the copies.
    const int grp = wave >> 2;  // waves w and w+4 share a SIMD
    auto run = [&](auto GRP) __attribute__((always_inline)) {
        constexpr int GR = decltype(GRP)::value;
        auto end_mfma = [&]() __attribute__((always_inline)) {
            if (GR == 0)
                __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4): copies of MFMA(j-2) done
            __builtin_amdgcn_s_barrier();
            fence();
        };
        auto end_valu = [&]() __attribute__((always_inline)) {
            if (GR == 1)
                __builtin_amdgcn_s_waitcnt(0x0F72);  // vmcnt(2): copies of MFMA(j-1) done
            __builtin_amdgcn_s_barrier();
            fence();
        };
        if (GR == 1)
            __builtin_amdgcn_s_barrier();  // one phase behind waves 0-3
        // step -1: S_0 only
        if (nwb > 0) {
#if MIATTN_PP_PRIO
            __builtin_amdgcn_s_setprio(1);
#endif
#pragma unroll
            for (int i = 0; i < 8; ++i)
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i].v, qf[i], i == 0 ? f32x16{} : s, 0, 0, 0);
        }
        end_mfma();
        if (nblk > 0) {
            valu_phase(-1, nwb > 0, 0 >= first_masked, 1 < nblk && 0 < nwb, sK1, sV0);
            end_valu();
        }
        // step j (slot P = j % 4 of both rings): copies of K_{j+4} into K slot
        // P and of V_{j+3} into V slot P+3; K_{j+2} from K slot P+2 and
        // V_{j+1} from V slot P+1
        auto step = [&](auto PI, int j) __attribute__((always_inline)) {
            constexpr int P = decltype(PI)::value;
            uint4 *const kb[4] = {sK0, sK1, sK2, sK3};
            uint4 *const vb[4] = {sV0, sV1, sV2, sV3};
            if (j < nwb) {
                mfma_phase(j, kb[P], vb[(P + 3) & 3]);
            } else {
                dma_k(kb[P], j + 4);
                dma_v(vb[(P + 3) & 3], j + 3);
            }
            end_mfma();
            if (j + 1 < nblk) {
                valu_phase(j, j + 1 < nwb, j + 1 >= first_masked, j + 2 < nblk && j + 1 < nwb, kb[(P + 2) & 3],
                           vb[(P + 1) & 3]);
                end_valu();
            }
        };
        int j = 0;
        for (; j + 3 < nblk; j += 4) {
            step(IntC<0>{}, j);
            step(IntC<1>{}, j + 1);
            step(IntC<2>{}, j + 2);
            step(IntC<3>{}, j + 3);
        }
        if (j < nblk)
            step(IntC<0>{}, j);
        if (j + 1 < nblk)
            step(IntC<1>{}, j + 1);
        if (j + 2 < nblk)
            step(IntC<2>{}, j + 2);
        if (GR == 0)
            __builtin_amdgcn_s_barrier();  // matches the first barrier of waves 4-7
    };
    if (grp == 0)
        run(IntC<0>{});
    else
        run(IntC<1>{});
    __builtin_amdgcn_s_waitcnt(0x0F70);  // no copy may still target LDS
#if MIATTN_PP_PRIO
    __builtin_amdgcn_s_setprio(0);
#endif

    // ---- epilogue ------------------------------------------------------------------
    const int my_q = q0 + l32;
    const float l_tot = halves_sum(l_half);
    if (my_q < Sq) {
        const bool empty = !(l_tot > 0.f);
        const float inv = empty ? 0.f : 1.f / l_tot;
        uint16_t *orow = a.o + (qrow0 + my_q) * D + 4 * g;
#pragma unroll
        for (int db = 0; db < DBN; ++db)
#pragma unroll
            for (int rho = 0; rho < 4; ++rho) {
                uint2 w;
                if (empty) {
                    w = make_uint2(0, 0);
                } else {
                    w.x = pack_bf16x2(acc[db][4 * rho] * inv, acc[db][4 * rho + 1] * inv);
                    w.y = pack_bf16x2(acc[db][4 * rho + 2] * inv, acc[db][4 * rho + 3] * inv);
                }
                *(uint2 *)(orow + 32 * db + 8 * rho) = w;
            }
        if (g == 0)
            a.lse[qrow0 + my_q] = empty ? -INFINITY : m_ref * a.scale + logf(l_tot);
    }
}

template <bool CAUSAL>
hipError_t launch_pp(const FwdArgs &a, hipStream_t stream)
{
    constexpr int BM = 256;
    const int n_qtiles = (a.Sq + BM - 1) / BM;
    const long long n_tiles = (long long)a.B * a.Hq * n_qtiles;
    if (n_tiles > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fwd_pingpong_kernel<CAUSAL>), dim3((unsigned)n_tiles), dim3(512), 0, stream, a,
                       n_qtiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_pingpong(const FwdArgs &a, bool causal, hipStream_t stream)
{
    return causal ? launch_pp<true>(a, stream) : launch_pp<false>(a, stream);
}

}  // namespace miattn
