// prefill_q64.hip -- fused attention forward on gfx950, head dimensions 128
// and 256, software-pipelined.
//
// Same operation and online-softmax monoid as prefill.hip. The design answers
// two gfx950 limits measured on the simpler kernel:
//
//  * LDS read bandwidth (about 150-200 bytes/ns per CU): every 16-byte K or V
//    fragment a wave reads from LDS feeds one 32x32x16 MFMA per 32-row query
//    block the wave owns. The kernel is written for QB = 1 or 2 blocks per
//    wave (32 or 64 query rows).
//  * VALU issue: the softmax costs about four VALU instructions and one
//    v_exp_f32 per score, roughly what the score's MFMA share takes on the
//    matrix unit. A wave can issue independent VALU work while its own MFMA
//    runs, so the softmax of one tile is spread between the MFMAs of another.
//
// Shapes in use: head dimension 128 runs eight waves of 32 query rows (two
// waves per SIMD, 256 rows per workgroup), which measured a few per cent
// faster than four waves of 64 rows: the second wave on the SIMD fills the
// issue slots the first leaves idle while it waits on a dependent VALU chain.
// Head dimension 256 runs four waves of 32 rows, one per SIMD: the f32
// accumulator alone takes 128 registers. Each wave runs a two-stage software
// pipeline per 32-key tile j, laid out in groups of four MFMAs with the VALU
// and LDS work placed between them:
//
//   stage A: S_{j+1} = K_{j+1} Q^T                   | exp/pack/row-sum of the
//            second 16 keys of tile j; row max of S_{j+1} for query block 0;
//            transposing LDS reads of V_j
//   stage B: O^T += V_j^T P_j                         | row max of S_{j+1} for
//            the last query block; exp/pack/row-sum of the first 16 keys of
//            tile j+1; LDS reads of K_{j+2}
//
// K and V tiles of 32 keys go global -> LDS by range-checked buffer DMA (keys
// past the workgroup's last visible key arrive as zeros) into four-deep rings, one barrier per tile. Both
// are stored fragment-major: each LDS read instruction of a wave reads one
// contiguous 1 KB (K, ds_read_b128) or 512 B (V, ds_read_b64_tr_b16) block,
// which is free of bank conflicts and needs no address arithmetic.
//
// The running maximum moves lazily: probabilities stay at most 2^8 above the
// reference and the accumulator is rescaled only on the rare tiles that move
// it. With two query blocks per wave the reference moves when a tile's row
// maximum exceeds it by more than 8 in log2 units. With one block the check
// uses the tile's row sums, which the softmax computes anyway: a lane whose
// 16 probabilities sum to at most 2^8 has none above 2^8, and only a tile
// that fails (or a wave with a row that has seen no key yet) takes the exact
// maximum and recomputes its probabilities.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "launch.h"
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

template <int N>
struct IntC {
    static constexpr int value = N;
};

union Frag8 {
    bf16x8 v;
    uint4 u;
    uint32_t w[4];
};

// IEEE maximum (NaN-propagating): on gfx950 it maps to v_maximum3_f32 and,
// unlike fmaxf, needs no quieting of its operands first
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

__device__ __forceinline__ void slot_end() { __builtin_amdgcn_sched_barrier(0); }

// Keep a value's computation inside its slot: an input pinned here cannot be
// consumed earlier, an output pinned here cannot be computed later (the
// compiler would otherwise sink work towards its uses across slots).
__device__ __forceinline__ void pin(float &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(uint32_t &x) { asm volatile("" : "+v"(x)); }

template <bool CAUSAL, int NWV, int D, int QB, int WPE>
__global__ void __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
fwd_q64_kernel(FwdArgs a, int n_qtiles)
{
    // D = 128 runs QB = 2 query blocks (64 rows) per wave, D = 256 one block
    // (32 rows): either way a tile step is 16 QK and 16 PV MFMAs per wave
    constexpr int BN = 32;             // keys per tile
    constexpr int BM = NWV * 32 * QB;  // query rows per workgroup
    constexpr int KKN = D / 16;        // 16-dim steps of QK = K fragments = copy instructions per tile
    constexpr int DBN = D / 32;        // 32-dim blocks of the output
    constexpr int DPW = KKN / NWV;     // copy instructions per wave per tile, each of K and V
    constexpr int NG = QB * KKN / 4;   // groups of four MFMAs per stage
    constexpr int NPV = QB * DBN;      // PV MFMAs per 16-key chunk
    static_assert((NG == 2 || NG == 4) && NWV * DPW == KKN && 3 * DPW < 16, "tile step shape");
    constexpr int TILE_CH = BN * D / 8;     // 16-byte chunks per tile

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
    bf16x8 qf[QB][KKN];
    {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + qrow0 * D, (uint32_t)Sq * D * 2);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const uint32_t off = (uint32_t)(q0 + 32 * qb + l32) * D * 2 + 16 * g;
#pragma unroll
            for (int kk = 0; kk < KKN; ++kk) {
                Frag8 f;
                f.u = buf_load16(rq, off + 32 * kk);  // rows >= Sq read as 0
                qf[qb][kk] = f.v;
            }
        }
    }

    // ---- global -> LDS copies ---------------------------------------------------
    // A tile takes D/16 DMA instructions (1 KB each) for K and as many for V;
    // wave w issues instructions DPW w .. DPW w + DPW - 1 of each. Every copy gets a buffer
    // resource covering just its tile, so keys at or past Sk read as zero.
    //
    // K layout: block kk (1 KB) holds lane L's A fragment for dims
    // 16kk + 8(L/32) .. +7 of key L%32, at byte 16L.
    // V layout: block r = (2 db + kc) * 2 + hh (512 B) holds, at byte 8L for
    // L = 16G + 4jj + q, the four values V[16kc + 8hh + 4(G/2) + jj]
    // [32db + 16(G%2) + 4q .. +3]; a transposing 8-byte read of the block
    // gives lane L the values of dim 32db + L%32 at four consecutive keys.
    uint32_t koff[DPW], voff[DPW];
#pragma unroll
    for (int h = 0; h < DPW; ++h) {
        const int i = DPW * wave + h;
        koff[h] = (uint32_t)(l32 * D + 16 * i + 8 * g) * 2;
        const int db = i >> 1, kc = i & 1, tt = l32;
        const int G4 = tt >> 3, jj = (tt >> 1) & 3, qh = tt & 1;
        const int key = 16 * kc + 8 * g + 4 * (G4 >> 1) + jj;
        const int dim = 32 * db + 16 * (G4 & 1) + 8 * qh;
        voff[h] = (uint32_t)(key * D + dim) * 2;
    }
    const uint16_t *const kbase = a.k + krow0 * D;
    const uint16_t *const vbase = a.v + krow0 * D;
    // keys at or past kv_end (at most Sk; no row of the workgroup sees them)
    // arrive as zeros, and the prefetches past the range cost no memory traffic
    auto tile_rsrc = [&](const uint16_t *base, int tile) __attribute__((always_inline)) {
        const int keys = __builtin_amdgcn_readfirstlane(min(max(kv_end - tile * BN, 0), BN));
        return make_rsrc(base + (int64_t)tile * (BN * D), (uint32_t)keys * (D * 2));
    };
    auto dma_k = [&](uint4 *buf, int tile) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t r = tile_rsrc(kbase, tile);
#pragma unroll
        for (int h = 0; h < DPW; ++h)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(buf + 64 * (DPW * wave + h)), 16,
                                                     (int)koff[h], 0, 0, 0);
    };
    auto dma_v = [&](uint4 *buf, int tile) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t r = tile_rsrc(vbase, tile);
#pragma unroll
        for (int h = 0; h < DPW; ++h)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(buf + 64 * (DPW * wave + h)), 16,
                                                     (int)voff[h], 0, 0, 0);
    };

    // ---- fragments from LDS -------------------------------------------------------
    Frag8 kf[KKN];      // A fragments of the K tile the next QK uses
    bf16x8 vf[DBN][2];  // A fragments of V^T: [d-block][16-key chunk]
    auto read_k = [&](const uint4 *buf, int kk) __attribute__((always_inline)) {
        kf[kk].u = buf[64 * kk + lane];
    };
    auto read_v = [&](const uint4 *buf, int db, int kc) __attribute__((always_inline)) {
        const char *base = (const char *)buf + 8 * lane;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(const_cast<char *>(base + ((2 * db + kc) * 2 + 0) * 512)));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(const_cast<char *>(base + ((2 * db + kc) * 2 + 1) * 512)));
        const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        vf[db][kc] = __builtin_bit_cast(bf16x8, both);
    };

    // ---- monoid state per query block -------------------------------------------
    constexpr float kLazy = 8.f;
    // wave-uniform constants held in scalar registers (the VALU computes them,
    // so without the readfirstlane each would occupy a vector register)
    const float c = uniform_f(a.scale * kLog2e);
    const float thr = uniform_f(kLazy / c);
    float m_ref[QB], nmc[QB], m_thr[QB], alpha_acc[QB], l_half[QB];  // nmc = -m_ref * c
    // One query block per wave: the row sum of the tile whose probabilities
    // are being built, added to l_half once the tile passes its check
    float tsum = 0.f;
    f32x16 acc[QB][D / 32];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_ref[qb] = -INFINITY;
        nmc[qb] = 0.f;
        m_thr[qb] = -INFINITY;
        alpha_acc[qb] = 1.f;
        l_half[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[qb][db][r] = 0.f;
    }

    using Sc = f32x16[QB];
    using Pc = Frag8[QB][2];  // [query block][16-key chunk]
    auto qk_mfma = [&](Sc &s, int qb, int kk) __attribute__((always_inline)) {
        // At one wave per SIMD (512 registers, more than the 256 VGPRs) Q
        // stays in AGPRs and is read there by the MFMA, else the allocator
        // parks it in AGPRs and copies it back every tile. At two waves per
        // SIMD the whole working set fits in 256 VGPRs, and any AGPR use
        // would split the budget into 128 + 128.
        if constexpr (WPE == 1)
            asm volatile("" : "+a"(qf[qb][kk]));
        if (kk == 0) {
            const f32x16 zero = {};
            s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk].v, qf[qb][kk], zero, 0, 0, 0);
        } else {
            s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk].v, qf[qb][kk], s[qb], 0, 0, 0);
        }
    };
    auto pv_mfma = [&](const Pc &p, int qb, int db, int kc) __attribute__((always_inline)) {
        acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db][kc], p[qb][kc].v, acc[qb][db],
                                                              0, 0, 0);
    };

    // Softmax work, in pieces placed between the MFMAs. Scores of a query
    // block: s[qb][r], key 8(r/4) + 4g + r%4 of the tile; chunk h = keys
    // 16h .. 16h+15 = r in [8h, 8h+8). Every piece pins     // its outputs at the end of its group of MFMAs (else the compiler sinks
    // them towards their uses); inside the group its independent chains
    // overlap one another.
    //
    // probabilities of scores r = 8h + 4quad .. +3 -> two packed bf16 pairs
    auto probs_quad = [&](const Sc &s, Pc &p, int qb, int h, int quad)
        __attribute__((always_inline)) {
        float e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][8 * h + 4 * quad + i], c, nmc[qb]));
        p[qb][h].w[2 * quad] = pack_bf16x2(e[0], e[1]);
        p[qb][h].w[2 * quad + 1] = pack_bf16x2(e[2], e[3]);
        if constexpr (QB == 1) {
            tsum += (e[0] + e[1]) + (e[2] + e[3]);
            pin(tsum);
        } else {
            l_half[qb] += (e[0] + e[1]) + (e[2] + e[3]);
            pin(l_half[qb]);
        }
        pin(p[qb][h].w[2 * quad]);
        pin(p[qb][h].w[2 * quad + 1]);
    };
    // row maximum in three parts (scores 0-7, scores 8-15, both halves of the
    // wave); a masked tile first selects hidden keys to -inf
    float mxa[QB], mxb[QB];
    auto row_max = [&](Sc &s, int qb, int part, int j, bool masked) __attribute__((always_inline)) {
        if (part < 2) {
            if (masked) {
                const int my_q = q0 + 32 * qb + l32;
                const int lim = j < nwb ? (CAUSAL ? min(Sk - 1, my_q + diag) : Sk - 1) : -1;
                const int rel = lim - j * BN - 4 * g;  // key r visible iff offset(r) <= rel
#pragma unroll
                for (int r = 8 * part; r < 8 * part + 8; ++r)
                    s[qb][r] = (8 * (r >> 2) + (r & 3) <= rel) ? s[qb][r] : -INFINITY;
            }
            const int r0 = 8 * part;
            float m = fmax_ieee(fmax_ieee(s[qb][r0], s[qb][r0 + 1]), s[qb][r0 + 2]);
            m = fmax_ieee(fmax_ieee(m, s[qb][r0 + 3]), s[qb][r0 + 4]);
            m = fmax_ieee(fmax_ieee(m, s[qb][r0 + 5]), s[qb][r0 + 6]);
            m = fmax_ieee(m, s[qb][r0 + 7]);
            pin(m);
            (part == 0 ? mxa[qb] : mxb[qb]) = m;
        } else {
            mxa[qb] = halves_max(fmax_ieee(mxa[qb], mxb[qb]));
            pin(mxa[qb]);
        }
    };
    // lazy reference update of a query block, taken only when some row of
    // the wave exceeds its reference by more than the threshold
    auto move_ref = [&](int qb) __attribute__((always_inline)) {
        if (__any(mxa[qb] > m_thr[qb])) {
            const float m_new = fmax_ieee(m_ref[qb], mxa[qb]);
            const float alpha =
                (m_new == m_ref[qb]) ? 1.f : __builtin_amdgcn_exp2f((m_ref[qb] - m_new) * c);
            l_half[qb] *= alpha;
            alpha_acc[qb] *= alpha;
            m_ref[qb] = m_new;
            nmc[qb] = (m_new == -INFINITY) ? 0.f : -(m_new * c);
            m_thr[qb] = m_new + thr;
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
                alpha_acc[qb] = 1.f;
            }
        }
    };

    // hide the keys of tile j a row of query block qb cannot see (select to -inf)
    auto mask_tile = [&](Sc &s, int qb, int j) __attribute__((always_inline)) {
        const int my_q = q0 + 32 * qb + l32;
        const int lim = j < nwb ? (CAUSAL ? min(Sk - 1, my_q + diag) : Sk - 1) : -1;
        const int rel = lim - j * BN - 4 * g;  // key r visible iff offset(r) <= rel
#pragma unroll
        for (int r = 0; r < 16; ++r)
            s[qb][r] = (8 * (r >> 2) + (r & 3) <= rel) ? s[qb][r] : -INFINITY;
    };
    // One query block per wave: the lazy reference is checked by the tile's
    // row sums instead of its row maximum. A lane's 16 probabilities are all
    // at most 2^8 when their sum is, which is the bound the reference keeps;
    // otherwise (or while some row has not seen a key) the tile takes this
    // slow path: exact maximum, reference update, rescale, probabilities
    // again. The scores are already masked.
    bool ref_unset = true;  // some row of the wave still has m_ref = -inf
    auto slow_tile = [&](Sc &s, Pc &p) __attribute__((always_inline)) {
        row_max(s, 0, 0, 0, false);
        row_max(s, 0, 1, 0, false);
        row_max(s, 0, 2, 0, false);
        move_ref(0);
        apply_alpha();
        tsum = 0.f;
        probs_quad(s, p, 0, 0, 0);
        probs_quad(s, p, 0, 0, 1);
        probs_quad(s, p, 0, 1, 0);
        probs_quad(s, p, 0, 1, 1);
        ref_unset = __any(m_ref[0] == -INFINITY);
    };
    auto check_tile = [&](Sc &s, Pc &p) __attribute__((always_inline)) {
        if (ref_unset || __any(tsum > 256.f))
            slow_tile(s, p);
        l_half[0] += tsum;
        tsum = 0.f;
    };

    // ---- prologue -------------------------------------------------------------------
    // Copies of K tiles 0-3 and V tiles 0-2, drained. Then S_0, its statistics
    // and the first chunk of P_0 without overlap, and K tile 1 into registers.
    dma_k(sK0, 0);
    dma_k(sK1, 1);
    dma_k(sK2, 2);
    dma_k(sK3, 3);
    dma_v(sV0, 0);
    dma_v(sV1, 1);
    dma_v(sV2, 2);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q and the copies
    __syncthreads();
    Sc sA, sB;      // scores of the even / odd tile in flight
    Pc pA, pB;      // probabilities of the even / odd tile
#pragma unroll
    for (int kk = 0; kk < KKN; ++kk)
        read_k(sK0, kk);
#pragma unroll
    for (int kk = 0; kk < KKN; ++kk)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
            qk_mfma(sA, qb, kk);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        row_max(sA, qb, 0, 0, true);
        row_max(sA, qb, 1, 0, true);
        row_max(sA, qb, 2, 0, true);
        move_ref(qb);
        probs_quad(sA, pA, qb, 0, 0);
        probs_quad(sA, pA, qb, 0, 1);
    }
    apply_alpha();  // the first reference moves consume their rescale here
    if constexpr (QB == 1)
        ref_unset = __any(m_ref[0] == -INFINITY);
#pragma unroll
    for (int kk = 0; kk < KKN; ++kk)
        read_k(sK1, kk);
    __syncthreads();  // every wave has read K tile 0 before K tile 4 replaces it

    // ---- one tile step ------------------------------------------------------------------
    // Tile m's K and V live in buffer m % 4. Step j: copies of K tile j+4 (into
    // tile j's K buffer, last read in step j-2) and V tile j+3 (into tile j-1's
    // V buffer, last read in step j-1); stage A; stage B; wait until the copies
    // the next step reads (V tile j+1, K tile j+3) are complete -- the 3 DPW
    // newer copy instructions of this wave may still fly -- and barrier.
    auto step = [&](auto PI, auto MASKc, int j, Sc &sc, Sc &sn, Pc &pc, Pc &pn)
        __attribute__((always_inline)) {
        constexpr int P = decltype(PI)::value;  // j % 4
        constexpr bool MASK = decltype(MASKc)::value;
        uint4 *const kb[4] = {sK0, sK1, sK2, sK3};
        uint4 *const vb[4] = {sV0, sV1, sV2, sV3};
        dma_k(kb[P], j + 4);
        dma_v(vb[(P + 3) & 3], j + 3);
        if constexpr (QB == 2)
            apply_alpha();
        slot_end();

        // Stage A, NG groups of four MFMAs (QK of tile j+1; with two query
        // blocks, block 0 then block 1). Groups 0-1 read V_j; the groups
        // compute chunk 1 of tile j's probabilities and, with two query
        // blocks, in groups 2-3 the row maximum of block 0 of tile j+1 (its
        // MFMAs finished in group 1).
        constexpr int NRV = 2 * DBN;  // read_v calls per tile (two reads each)
#pragma unroll
        for (int grp = 0; grp < NG; ++grp) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int sl = 4 * grp + i;
                qk_mfma(sn, sl / KKN, sl % KKN);
                if (grp < 2)
#pragma unroll
                    for (int c = sl * NRV / 8; c < (sl + 1) * NRV / 8; ++c)
                        read_v(vb[P], c >> 1, c & 1);
            }
            if (grp < 2 * QB)
                probs_quad(sc, pc, grp >> 1, 1, grp & 1);
            if constexpr (QB == 2) {
                if (grp == 2)
                    row_max(sn, 0, 0, j + 1, MASK);
                if (grp == 3) {
                    row_max(sn, 0, 1, j + 1, MASK);
                    row_max(sn, 0, 2, j + 1, MASK);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                if (grp < 2)
                    __builtin_amdgcn_sched_group_barrier(0x100, NRV / 4, 0);  // LDS reads
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
            }
            slot_end();
        }
        if constexpr (QB == 2) {
            move_ref(0);
            slot_end();
        } else {
            check_tile(sc, pc);  // tile j's probabilities are complete
            slot_end();
        }

        // Stage B, NG groups of four MFMAs (PV of tile j). Each group reads
        // D/64 K_{j+2} fragments. With two query blocks, groups 0-1 compute
        // chunk 0 of tile j+1 for block 0 and the row maximum of block 1,
        // groups 2-3 chunk 0 for block 1 after its reference update; with one,
        // group 0 takes the row maximum and groups 1-2 chunk 0.
        constexpr int KPG = KKN / NG;  // K reads per group
#pragma unroll
        for (int grp = 0; grp < NG; ++grp) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int sl = 4 * grp + i;
                const int idx = sl % NPV;
                pv_mfma(pc, idx % QB, idx / QB, sl / NPV);
                if (i < KPG)
                    read_k(kb[(P + 2) & 3], KPG * grp + i);
            }
            if constexpr (QB == 2) {
                probs_quad(sn, pn, grp >> 1, 0, grp & 1);
                if (grp == 0)
                    row_max(sn, 1, 0, j + 1, MASK);
                if (grp == 1) {
                    row_max(sn, 1, 1, j + 1, MASK);
                    row_max(sn, 1, 2, j + 1, MASK);
                }
            } else {
                if (MASK && grp == 0)
                    mask_tile(sn, 0, j + 1);
                if (NG == 2 && grp == 1) {
                    probs_quad(sn, pn, 0, 0, 0);
                    probs_quad(sn, pn, 0, 0, 1);
                }
                if (NG == 4 && (grp == 1 || grp == 2))
                    probs_quad(sn, pn, 0, 0, grp - 1);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                if (i < KPG)
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
            }
            slot_end();
            if (QB == 2 && grp == 1) {
                move_ref(QB - 1);
                slot_end();
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0F70 | (3 * DPW));  // vmcnt(3 DPW)
        __builtin_amdgcn_s_barrier();
        slot_end();
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
        step(IntC<0>{}, IntC<0>{}, j, sA, sB, pA, pB);
        step(IntC<1>{}, IntC<0>{}, j + 1, sB, sA, pB, pA);
        step(IntC<2>{}, IntC<0>{}, j + 2, sA, sB, pA, pB);
        step(IntC<3>{}, IntC<0>{}, j + 3, sB, sA, pB, pA);
    }
    // Masked steps. From tile nwb on the wave sees no key of the tiles it
    // would touch (PV of tile j, QK of tile j+1): it only issues its share of
    // the copies and keeps the barrier, leaving its SIMD to the other wave.
    // (Step nwb-1 still runs: its PV is live, and the tile nwb it scores is
    // all masked and never checked.)
    auto mstep = [&](auto PI, int j, Sc &sc, Sc &sn, Pc &pc, Pc &pn) __attribute__((always_inline)) {
        constexpr int P = decltype(PI)::value;
        if (j < nwb) {
            step(PI, IntC<1>{}, j, sc, sn, pc, pn);
        } else {
            uint4 *const kb[4] = {sK0, sK1, sK2, sK3};
            uint4 *const vb[4] = {sV0, sV1, sV2, sV3};
            dma_k(kb[P], j + 4);
            dma_v(vb[(P + 3) & 3], j + 3);
            __builtin_amdgcn_s_waitcnt(0x0F70 | (3 * DPW));  // vmcnt(3 DPW)
            __builtin_amdgcn_s_barrier();
            slot_end();
        }
    };
    for (; j + 3 < nblk; j += 4) {
        mstep(IntC<0>{}, j, sA, sB, pA, pB);
        mstep(IntC<1>{}, j + 1, sB, sA, pB, pA);
        mstep(IntC<2>{}, j + 2, sA, sB, pA, pB);
        mstep(IntC<3>{}, j + 3, sB, sA, pB, pA);
    }
    if (j < nblk)
        mstep(IntC<0>{}, j, sA, sB, pA, pB);
    if (j + 1 < nblk)
        mstep(IntC<1>{}, j + 1, sB, sA, pB, pA);
    if (j + 2 < nblk)
        mstep(IntC<2>{}, j + 2, sA, sB, pA, pB);
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

// Build switches for measuring other shapes: the number of waves per
// workgroup at each head dimension, and 64 (QB=2, one wave per SIMD) or 32
// (QB=1, two waves per SIMD) query rows per wave at head dimension 128.
#ifndef MIATTN_Q64_D128_QB
#define MIATTN_Q64_D128_QB 1
#endif
#ifndef MIATTN_Q64_D128_WAVES
#define MIATTN_Q64_D128_WAVES 8
#endif
#ifndef MIATTN_Q64_D256_WAVES
#define MIATTN_Q64_D256_WAVES 4
#endif
#ifndef MIATTN_Q64_D128_WPE  // waves per SIMD the d = 128 kernel is compiled for
#define MIATTN_Q64_D128_WPE (2 * MIATTN_Q64_D128_WAVES / 8)
#endif

template <int D, int QB, int NWV, int WPE>
hipError_t launch_q64(const FwdArgs &a, bool causal, hipStream_t stream)
{
    constexpr int BM = NWV * 32 * QB;
    const int n_qtiles = (a.Sq + BM - 1) / BM;
    const long long n_tiles = (long long)a.B * a.Hq * n_qtiles;
    if (n_tiles > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;
    if (causal)
        hipLaunchKernelGGL((fwd_q64_kernel<true, NWV, D, QB, WPE>), dim3((unsigned)n_tiles), dim3(64 * NWV),
                           0, stream, a, n_qtiles);
    else
        hipLaunchKernelGGL((fwd_q64_kernel<false, NWV, D, QB, WPE>), dim3((unsigned)n_tiles), dim3(64 * NWV),
                           0, stream, a, n_qtiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_q64(const FwdArgs &a, int d, bool causal, hipStream_t stream)
{
    switch (d) {
    case 128:
#if MIATTN_Q64_D128_QB == 1
        return launch_q64<128, 1, MIATTN_Q64_D128_WAVES, MIATTN_Q64_D128_WPE>(a, causal, stream);
#else
        return launch_q64<128, 2, MIATTN_Q64_D128_WAVES, MIATTN_Q64_D128_WAVES / 4>(a, causal, stream);
#endif
    case 256:
        return launch_q64<256, 1, MIATTN_Q64_D256_WAVES, MIATTN_Q64_D256_WAVES / 4>(a, causal, stream);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace miattn
