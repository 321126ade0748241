// prefill_pp.hip -- fused attention forward on gfx950 with two alternating
// wave groups ("ping-pong") for head dimension 128.
//
// Same operation and the same online-softmax monoid as prefill.hip; only the
// schedule differs. A workgroup has 8 waves in two groups of four; the waves
// of a SIMD come one from each group. Each wave owns 32 query rows (BM = 256
// rows per workgroup) and the keys stream in tiles of 32. Per tile every
// group runs four phases separated by workgroup barriers, and group 1 runs
// one phase behind group 0, so on every SIMD one wave issues MFMAs while the
// other issues its LDS and global traffic:
//
//   C1(j): S_{j+1} = K_{j+1} Q^T (8 MFMAs)  with  second half of tile j's
//          probabilities (exp2, bf16 rounding, row sums) on the VALU
//   L1(j): V_j fragments from LDS (transposing reads); group 0 also issues
//          the K tile j+3 global->LDS copy
//   C2(j): O^T += V_j^T P_j (8 MFMAs)  with  mask, row max and lazy
//          reference update of tile j+1 and the first half of its
//          probabilities
//   L2(j): K_{j+2} fragments from LDS; group 0 also issues the V tile j+2
//          global->LDS copy
//
// K and V tiles go from global memory straight to LDS with range-checked
// buffer loads (rows past Sk arrive as zeros), each pipeline buffer in its
// own LDS array so the compiler's wait analysis sees that the copy in flight
// does not alias the tile being read. K rows are stored with a 16-byte chunk
// XOR swizzle by row; V rows are stored row-major with a swizzle chosen so the
// transposing reads (ds_read_b64_tr_b16) that build the V^T MFMA operand are
// free of bank conflicts. The probability accumulator layout and the key
// permutation between the two contractions are those of prefill.hip.

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

// The lane id as a value the compiler cannot hoist: address arithmetic for
// the LDS fragment reads and copies is recomputed where it is used (in the
// memory phases, where the VALU is otherwise idle) instead of being kept live
// across the whole loop in registers.
__device__ __forceinline__ int opaque_lane()
{
    int l = (int)(threadIdx.x & 63);
    asm volatile("" : "+v"(l));
    return l;
}

// Empty asm that claims to read and rewrite a register: the value must be
// computed before this point and cannot be sunk past it. Used to keep each
// phase's results inside that phase.
__device__ __forceinline__ void pin(float &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(uint32_t &x) { asm volatile("" : "+v"(x)); }

// V rows: 16-byte chunk c of row r sits at chunk c ^ vswz(r). With this
// pattern the four rows x four 8-byte column blocks addressed by one 16-lane
// group of a transposing read land in distinct banks (32 or 64 banks).
__device__ __forceinline__ int vswz(int r)
{
    return (0xEA40 >> (4 * (r & 3))) & 15;  // 0, 4, 10, 14 for r % 4 = 0..3
}

template <bool CAUSAL>
__global__ void __launch_bounds__(512)
fwd_pp_kernel(FwdArgs a, int n_qtiles)
{
    constexpr int D = 128;
    constexpr int BN = 32;            // keys per tile
    constexpr int BM = 256;           // query rows per workgroup (8 waves x 32)
    constexpr int KCH = D / 8;        // 16-byte chunks per row
    constexpr int TILE_CH = BN * KCH; // 16-byte chunks per tile (512 = 8 KB)
    static_assert(TILE_CH == 512, "one tile = 8 DMA instructions of 1 KB");

    // four K and four V tile buffers (tile m in buffer m % 4), each its own
    // array so a copy in flight never aliases the buffer being read
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
    const int grp = wave >> 2;        // 0: waves 0-3, 1: waves 4-7
    const int wig = wave & 3;         // wave within its group
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
    const int q0 = q_wg + wave * 32;
    const int my_q = q0 + l32;
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

    // ---- Q fragment (B operand of S^T = K Q^T) --------------------------------
    bf16x8 qf[D / 16];
    {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + qrow0 * D, (uint32_t)Sq * D * 2);
        const uint32_t off = (uint32_t)my_q * D * 2 + 16 * g;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            Frag8 f;
            f.u = buf_load16(rq, off + 32 * kk);
            qf[kk] = f.v;
        }
    }

    // ---- global -> LDS copies (group 0 issues them) ---------------------------
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + krow0 * D, (uint32_t)Sk * D * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + krow0 * D, (uint32_t)Sk * D * 2);
    // This lane's part of a 1 KB DMA instruction i (4 rows of a tile): physical
    // chunk p = 64 i + lane holds logical chunk (p % 16) ^ swizzle(row).
    auto dma_k = [&](uint4 *buf, int tile) __attribute__((always_inline)) {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int i = 2 * wig + h;
            const int r = 4 * i + (lane >> 4);
            const int c = (lane & 15) ^ (r & 15);
            const uint32_t off = ((uint32_t)(tile * BN + r) * D + 8 * c) * 2;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)(buf + 64 * i), 16, (int)off,
                                                     0, 0, 0);
        }
    };
    auto dma_v = [&](uint4 *buf, int tile) __attribute__((always_inline)) {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int i = 2 * wig + h;
            const int r = 4 * i + (lane >> 4);
            const int c = (lane & 15) ^ vswz(r);
            const uint32_t off = ((uint32_t)(tile * BN + r) * D + 8 * c) * 2;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(buf + 64 * i), 16, (int)off,
                                                     0, 0, 0);
        }
    };

    // ---- fragments from LDS ---------------------------------------------------
    Frag8 kf[D / 16];   // K rows l32 of the tile: A operand of S^T, per 16-dim step
    bf16x8 vf[4][2];    // V^T rows 32 db + l32: A operand of O^T, per (d-block, key chunk)
    auto read_k = [&](const uint4 *buf) __attribute__((always_inline)) {
        const int ln = threadIdx.x & 63;
        const int row = ln & 31, gg = ln >> 5;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            kf[kk].u = buf[row * KCH + ((2 * kk + gg) ^ (row & 15))];
    };
    // transposing read: lane L = 16 G + 4 j + q addresses row 16 kc + 4 (G/2) + j
    // (+8 for the second half) at column 32 db + 16 (G%2) + 4 q; the result gives
    // every lane four keys of its own column.
    auto read_v = [&](const uint4 *buf) __attribute__((always_inline)) {
        const int ln = threadIdx.x & 63;
        const int G4 = ln >> 4, i = ln & 15;
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

    // ---- monoid state ---------------------------------------------------------
    constexpr float kLazy = 8.f;
    const float c = a.scale * kLog2e;
    const float thr = kLazy / c;
    float m_ref = -INFINITY;
    float mc = 0.f;          // m_ref * c, or 0 while m_ref = -inf
    float alpha_acc = 1.f;   // pending rescale of acc
    float l_half = 0.f;   // running sum of P over this lane half's keys (f32)
    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[db][r] = 0.f;


    auto qk = [&](f32x16 &s) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            s[r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk].v, qf[kk], s, 0, 0, 0);
    };
    // probabilities of key chunk h (scores s[8h .. 8h+7]) -> bf16 fragment
    auto probs = [&](const f32x16 &s, int h, Frag8 &p) __attribute__((always_inline)) {
        float rs = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * h + 2 * w], c, -mc));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * h + 2 * w + 1], c, -mc));
            const uint32_t pk = pack_bf16x2(p0, p1);
            p.w[w] = pk;
            rs += p0 + p1;
        }
        l_half += rs;
    };
    auto pin_frag = [&](Frag8 &p) __attribute__((always_inline)) {
#pragma unroll
        for (int w = 0; w < 4; ++w)
            pin(p.w[w]);
    };
    auto pin_stats = [&]() __attribute__((always_inline)) {
        pin(l_half);
        pin(m_ref);
        pin(mc);
        pin(alpha_acc);
    };
    // mask (keys above `lim` -> -inf; lim = -1 masks the whole tile), row
    // max and lazy update of the reference, for tile j
    auto row_stats = [&](f32x16 &s, int j, auto MASKc, int lim) __attribute__((always_inline)) {
        if (decltype(MASKc)::value) {
            const int j0 = j * BN;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = j0 + 8 * (r >> 2) + 4 * g + (r & 3);
                s[r] = (key <= lim) ? s[r] : -INFINITY;
            }
        }
        float mx = s[0];
#pragma unroll
        for (int r = 1; r < 16; ++r)
            mx = fmaxf(mx, s[r]);
        mx = halves_max(mx);
        const bool move = __any(mx > m_ref + thr);
        const float m_new = move ? fmaxf(m_ref, mx) : m_ref;
        const float alpha = (m_new == m_ref) ? 1.f : __builtin_amdgcn_exp2f((m_ref - m_new) * c);
        l_half *= alpha;
        alpha_acc *= alpha;
        m_ref = m_new;
        mc = (m_ref == -INFINITY) ? 0.f : m_ref * c;
    };
    auto pv = [&](const Frag8 &p0, const Frag8 &p1) __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db][0], p0.v, acc[db], 0, 0, 0);
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db][1], p1.v, acc[db], 0, 0, 0);
        }
    };
    auto apply_alpha = [&]() __attribute__((always_inline)) {
        if (__any(alpha_acc != 1.f)) {
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[db][r] *= alpha_acc;
        }
        alpha_acc = 1.f;
    };
    // last key of tile j this lane may see; -1 when the wave computes nothing
    // for tile j (all of its probabilities are then exactly 0)
    auto mask_lim = [&](int j) __attribute__((always_inline)) {
        const int lim = CAUSAL ? min(Sk - 1, my_q + diag) : Sk - 1;
        return j < nwb ? lim : -1;
    };

    // Interleave MFMAs with VALU work inside a compute phase: one MFMA, then
    // NV VALU instructions, eight times.
    auto interleave = [&](auto NVc) __attribute__((always_inline)) {
        constexpr int NV = decltype(NVc)::value;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);  // VALU
        }
    };
    auto barrier = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    // group 0 issues one K and one V tile copy (2 instructions each) per
    // step; a copy is first read 14 phases after it is issued, by which time
    // six newer copies (12 instructions) may still be in flight
    auto wait_dma = [&]() __attribute__((always_inline)) {
        if (grp == 0)
            __builtin_amdgcn_s_waitcnt(0x0F7C);  // vmcnt(12)
    };

    // ---- prologue ---------------------------------------------------------------
    // Copies of K and V tiles 0-3 (group 0), drained; every wave computes S_0,
    // its statistics and P_0's first key chunk; then K tile 4 goes into the
    // buffer of K tile 0 and every wave reads K tile 1.
    if (grp == 0) {
        dma_k(sK0, 0);
        dma_k(sK1, 1);
        dma_k(sK2, 2);
        dma_k(sK3, 3);
        dma_v(sV0, 0);
        dma_v(sV1, 1);
        dma_v(sV2, 2);
        dma_v(sV3, 3);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q and the copies
    __syncthreads();
    f32x16 sA, sB;           // scores of tiles j (even) and j+1
    Frag8 pA, pA2, pB, pB2;  // bf16 probabilities: key chunks 0 and 1 of each tile
    {
        read_k(sK0);
        qk(sA);
        row_stats(sA, 0, IntC<1>{}, mask_lim(0));
        probs(sA, 0, pA);
    }
    __syncthreads();
    if (grp == 0)
        dma_k(sK0, 4);
    read_k(sK1);
    // K tile 4 must be complete before the loop: its first wait there sees
    // only five newer copies, which vmcnt(12) would not cover
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();

    // ---- phases -------------------------------------------------------------------
    // K tile m lives in LDS buffer m % 2, V tile m likewise. In step j the
    // scores of tile j are `sc`, those of tile j+1 go to `sn`; P_j's key chunk
    // 0 (pc0) was made in the previous C2, chunk 1 (pc1) is made in C1.
    // One tile step with static buffer parity (j % 2): C1 | L1 | C2 | L2, a
    // barrier after each phase. Both groups run this same code; group 1 is
    // one phase behind because it passes one extra barrier before the loop
    // (and group 0 one after it), so every phase of group 0 runs beside the
    // complementary phase of group 1. FAST steps are those where this wave
    // computes everything and tile j+1 needs no mask (all but a wave's last
    // two or three tiles); they have no branches, so the MFMAs and the VALU
    // work of a compute phase share one scheduling region.
    auto step = [&](auto PI, auto MASKc, int j, f32x16 &sc, f32x16 &sn, Frag8 &pc0,
                    Frag8 &pc1, Frag8 &pn0) __attribute__((always_inline)) {
        constexpr int P = decltype(PI)::value;  // j % 4
        uint4 *const kb[4] = {sK0, sK1, sK2, sK3};
        uint4 *const vb[4] = {sV0, sV1, sV2, sV3};
        uint4 *k1 = kb[(P + 1) & 3];  // K tile j+1; K tile j+5 is copied here
        uint4 *k2 = kb[(P + 2) & 3];  // K tile j+2
        uint4 *v0 = vb[P];            // V tile j; V tile j+4 is copied here
        // C1: S_{j+1} = K_{j+1} Q^T  ||  P_j key chunk 1
        apply_alpha();
        qk(sn);
        probs(sc, 1, pc1);
        interleave(IntC<4>{});
        pin_frag(pc1);
        pin_stats();
        wait_dma();
        barrier();
        // L1: V_j fragments; copy of K tile j+5
        read_v(v0);
        if (grp == 0)
            dma_k(k1, j + 5);
        barrier();
        // C2: O^T += V_j^T P_j  ||  statistics of tile j+1, P_{j+1} key chunk 0
        pv(pc0, pc1);
        row_stats(sn, j + 1, MASKc, mask_lim(j + 1));
        probs(sn, 0, pn0);
        interleave(IntC<7>{});
        pin_frag(pn0);
        pin_stats();
        wait_dma();
        barrier();
        // L2: K_{j+2} fragments; copy of V tile j+4
        read_k(k2);
        if (grp == 0)
            dma_v(v0, j + 4);
        barrier();
    };

    // Leading steps of this wave that need no mask (a multiple of 4): tile
    // j+1 is fully visible and within the wave's range. Masks are needed from
    // some tile on (causal diagonal, ragged key tail) and for every tile past
    // the wave's range.
    int n_fast;
    {
        int first_masked = Sk / BN;  // ragged key tail
        if (CAUSAL)
            first_masked = min(first_masked, max(0, (q0 + diag + 1) / BN));
        n_fast = min(nwb, first_masked) - 1;
        n_fast = max(0, n_fast) & ~3;
        n_fast = __builtin_amdgcn_readfirstlane(n_fast);
    }

    if (grp == 1)
        barrier();
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
    if (grp == 0)
        barrier();
    __builtin_amdgcn_s_waitcnt(0x0F70);  // no copy may still target LDS
    apply_alpha();

    // ---- epilogue ------------------------------------------------------------------
    const float l_tot = halves_sum(l_half);
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
                    w.x = pack_bf16x2(acc[db][4 * rho] * inv, acc[db][4 * rho + 1] * inv);
                    w.y = pack_bf16x2(acc[db][4 * rho + 2] * inv, acc[db][4 * rho + 3] * inv);
                }
                *(uint2 *)(orow + 32 * db + 8 * rho) = w;
            }
        if (g == 0)
            a.lse[qrow0 + my_q] = empty ? -INFINITY : m_ref * a.scale + logf(l_tot);
    }
}

}  // namespace

hipError_t launch_fwd_pp(const FwdArgs &a, bool causal, hipStream_t stream)
{
    constexpr int BM = 256;
    const int n_qtiles = (a.Sq + BM - 1) / BM;
    const long long n_tiles = (long long)a.B * a.Hq * n_qtiles;
    if (n_tiles > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;
    if (causal)
        hipLaunchKernelGGL(fwd_pp_kernel<true>, dim3((unsigned)n_tiles), dim3(512), 0, stream, a,
                           n_qtiles);
    else
        hipLaunchKernelGGL(fwd_pp_kernel<false>, dim3((unsigned)n_tiles), dim3(512), 0, stream, a,
                           n_qtiles);
    return hipGetLastError();
}

}  // namespace miattn
