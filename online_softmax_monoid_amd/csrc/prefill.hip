// prefill.hip -- fused attention forward on gfx950 MFMA.
//
// One workgroup owns BM = 32*NW query rows of one (batch, query head) and
// streams the keys of that head's kv-head in tiles of BN keys. Per tile:
//
//   (a2) stage the K tile into LDS (row-major, 16-byte chunks XOR-swizzled)
//        and the V tile transposed (V^T, key order permuted to match the
//        score accumulator), double-buffered so the next tile's global loads
//        are in flight while this tile computes;
//   (a2) S^T = K Q^T with v_mfma_f32_32x32x16_bf16: each lane owns one query
//        column and 16 key rows of every 32x32 score block;
//   (a3) scale and mask by select (masked key -> -inf, the identity of max);
//   (a4) the online-softmax monoid update (tang paper, §2.2): reference max
//        (moved lazily, see below), probabilities exp2(s*c - m*c) with
//        c = scale*log2(e), rounded to bf16 for the value contraction, and
//        their f32 row sum (plain adds: the packed bf16 dot instruction
//        shares the matrix pipe on gfx950 and would stall the MFMAs);
//   (a5) O^T += V^T P^T with the same MFMA, P used straight from registers as
//        the B operand. The score accumulator holds keys
//        {4g..4g+3, 8+4g..8+4g+3} of each 16-key chunk in lane half g; V^T is
//        stored with exactly that key order, so no data moves between the two
//        contractions (legal because the sum over keys is commutative and
//        associative -- the paper's §5 "Lowering" makes the same move with
//        permuted keys on another ISA);
//   (a6) epilogue on the reducing lanes (§2.3): O = acc / l, LSE = m*scale +
//        ln l; rows with no visible key get O = +0 and LSE = -inf.
//
// The score matrix never leaves registers. Workgroups take their tiles in
// the order of tile_order.h: each XCD owns a set of (batch, kv-head) units,
// whose K and V then stay in its L2, and walks them heaviest causal tile
// first; the query heads of one GQA group sharing a kv-head are adjacent.
//
// Head dimension 64 uses this kernel; head dimensions 128 and 256 the
// software-pipelined persistent kernel of prefill_q64.hip.

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

constexpr float kLog2e = 1.4426950408889634f;

union Frag8 {
    bf16x8 v;
    uint4 u;
    uint32_t w[4];
};

// Combine a per-lane value with the one in lane l ^ 32 (the other half of the
// wave). v_permlane32_swap exchanges the two halves; its two results hold the
// values of lanes l % 32 and l % 32 + 32 (in some order), so a symmetric
// combine of the pair gives both lanes bit-identical results.
__device__ __forceinline__ float halves_max(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                              false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float halves_sum(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                              false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);  // IEEE add commutes
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2 p;
    p[0] = (__bf16)lo;
    p[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, p);
}

// Raw buffer resource over [base, base + bytes): loads past the end return 0,
// which is how ragged tails and rows beyond Sq/Sk are read without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// Physical tile index -> logical tile index. Consecutive logical tiles land on
// one XCD: physical id x runs on XCD x % 8.
template <int D, int BN, int NW>
struct Cfg {
    static constexpr int NT = NW * 64;
    static constexpr int BM = NW * 32;
    static constexpr int KCH = D / 8;                      // 16-byte chunks per K row
    static constexpr int SWZ = (KCH < 16 ? KCH : 16) - 1;  // XOR mask on the chunk index
    static constexpr int VTS = BN + 8;                     // V^T row stride (elements)
    static constexpr int K_TILE = BN * D;
    static constexpr int VT_TILE = D * VTS;
    static constexpr int KPT = BN * KCH / NT;              // K chunks per thread
    static constexpr int VUNITS = (BN / 4) * (D / 8);      // 4-key x 8-dim units
    static constexpr int VPT = (VUNITS + NT - 1) / NT;
    static_assert(BN % 32 == 0, "BN must be a multiple of 32");
    static_assert((BN * KCH) % NT == 0, "K tile must split evenly over threads");
};

// Score modifiers: none, soft cap, ALiBi
enum { kModNone = 0, kModSoftcap = 1, kModAlibi = 2 };

template <int D, int BN, int NW, bool CAUSAL, int MOD>
__global__ void __launch_bounds__(NW * 64)
fwd_kernel(FwdArgs a, int n_qtiles)
{
    using C = Cfg<D, BN, NW>;
    __shared__ __attribute__((aligned(16))) uint16_t sK[2][C::K_TILE];
    __shared__ __attribute__((aligned(16))) uint16_t sVT[2][C::VT_TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int l32 = lane & 31;
    const int g = lane >> 5;

    // ---- work decomposition ---------------------------------------------
    const int G = a.Hq / a.Hkv;
    const TileOrder to = tile_order((int)blockIdx.x, a.B * a.Hkv, G, n_qtiles, CAUSAL);
    const int unit = to.unit, gq = to.gq, qtile = to.qtile;
    const int b = unit / a.Hkv;
    const int kvh = unit - b * a.Hkv;
    const int hq = kvh * G + gq;

    const int Sq = a.Sq, Sk = a.Sk;
    const int diag = Sk - Sq;  // key j is visible to query i iff j <= i + diag
    const int64_t qrow0 = ((int64_t)b * a.Hq + hq) * Sq;
    const int q_wg = qtile * C::BM;
    const int q_wg_last = min(q_wg + C::BM, Sq) - 1;
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
    // Sliding window: the workgroup's keys start at the tile holding its first
    // row's first visible key; tiles below it are hidden from every row and
    // are never loaded. Tile indices below count from there (key kofs).
    const bool windowed = a.window >= 0;
    const int kofs = windowed ? min(kv_end, max(0, q_wg + diag - a.window)) / BN * BN : 0;
    const int64_t krow0 = ((int64_t)b * a.Hkv + kvh) * Sk + kofs;
    const uint16_t *__restrict__ Kp = a.k + krow0 * D;
    const uint16_t *__restrict__ Vp = a.v + krow0 * D;
    const int nblk = (kv_end - kofs + BN - 1) / BN;

    // ---- Q fragment: B operand of S^T = K Q^T (a1) ------------------------
    bf16x8 qf[D / 16];
    {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + qrow0 * D, (uint32_t)Sq * D * 2);
        const uint32_t off = (uint32_t)my_q * D * 2 + 16 * g;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            Frag8 f;
            f.u = buf_load16(rq, off + 32 * kk);  // rows >= Sq read as 0
            qf[kk] = f.v;
        }
    }

    // ---- staging (a2) -----------------------------------------------------
    // K and V tiles travel together through registers into double buffers:
    // while tile j computes from LDS, the global loads of tile j+1 are in
    // flight in registers and land in the buffers freed by tile j-1.
    uint4 kreg[C::KPT];
    uint4 vreg[C::VPT][4];

    // keys at or beyond Sk read as 0 (buffer range check)
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kp, (uint32_t)(Sk - kofs) * D * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vp, (uint32_t)(Sk - kofs) * D * 2);
    auto load_k = [&](int blk) {
        const uint32_t base = (uint32_t)blk * BN * D * 2;
#pragma unroll
        for (int u = 0; u < C::KPT; ++u) {
            const int ci = tid + C::NT * u;  // 16-byte chunk ci of the tile, row-major
            kreg[u] = buf_load16(rk, base + 16 * ci);
        }
    };
    auto load_v = [&](int blk) {
        const uint32_t base = (uint32_t)blk * BN * D * 2;
#pragma unroll
        for (int w = 0; w < C::VPT; ++w) {
            const int un = tid + C::NT * w;
            const int kg = un % (BN / 4), dc = un / (BN / 4);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                vreg[w][i] = (C::VUNITS % C::NT == 0 || un < C::VUNITS)
                    ? buf_load16(rv, base + (uint32_t)(4 * kg + i) * D * 2 + 16 * dc)
                    : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_k = [&](int buf) {
#pragma unroll
        for (int u = 0; u < C::KPT; ++u) {
            const int ci = tid + C::NT * u;
            const int key = ci / C::KCH, c = ci % C::KCH;
            *(uint4 *)(&sK[buf][key * D + 8 * (c ^ (key & C::SWZ))]) = kreg[u];
        }
    };
    auto store_v = [&](int buf) {
#pragma unroll
        for (int w = 0; w < C::VPT; ++w) {
            const int un = tid + C::NT * w;
            if (un < C::VUNITS) {
                const int kg = un % (BN / 4), dc = un / (BN / 4);
                const int gam = kg & 3;
                const int col = 16 * (kg >> 2) + 8 * (gam & 1) + 4 * (gam >> 1);
                const uint32_t *r0 = (const uint32_t *)&vreg[w][0];
                const uint32_t *r1 = (const uint32_t *)&vreg[w][1];
                const uint32_t *r2 = (const uint32_t *)&vreg[w][2];
                const uint32_t *r3 = (const uint32_t *)&vreg[w][3];
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const int wd = jj >> 1;
                    uint32_t lo, hi;
                    if (jj & 1) {
                        lo = (r0[wd] >> 16) | (r1[wd] & 0xffff0000u);
                        hi = (r2[wd] >> 16) | (r3[wd] & 0xffff0000u);
                    } else {
                        lo = (r0[wd] & 0xffffu) | (r1[wd] << 16);
                        hi = (r2[wd] & 0xffffu) | (r3[wd] << 16);
                    }
                    *(uint2 *)(&sVT[buf][(8 * dc + jj) * C::VTS + col]) = make_uint2(lo, hi);
                }
            }
        }
    };

    // S^T = K Q^T for the tile in K buffer `buf` (a2)
    auto scores = [&](int buf, f32x16 (&s)[BN / 32]) {
#pragma unroll
        for (int bb = 0; bb < BN / 32; ++bb) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                s[bb][r] = 0.f;
            const int key = 32 * bb + l32;
            const uint16_t *krow = &sK[buf][key * D];
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                Frag8 f;
                f.u = *(const uint4 *)(krow + 8 * ((2 * kk + g) ^ (key & C::SWZ)));
                s[bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.v, qf[kk], s[bb], 0, 0, 0);
            }
        }
    };

    // ---- running monoid state of this lane's query row (a4) ---------------
    // m_ref is a reference maximum: probabilities are exp2((s - m_ref) * c).
    // It moves (and the state is rescaled) only when a tile's maximum exceeds
    // it by more than kLazy in log2 units, so p stays below 2^kLazy; O = acc/l
    // and LSE = m_ref*scale + ln(l) are the same for any reference.
    constexpr float kLazy = 8.f;
    const float c = a.scale * kLog2e;
    const float thr = kLazy / c;  // in raw score units
    float m_ref = -INFINITY;
    float l_half = 0.f;   // running sum of P over this lane half's keys (f32)
    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[db][r] = 0.f;

    // mask (a3), monoid update (a4) and value contraction (a5) of tile blk
    // Score modifiers on the raw scores (q.k before the scale), applied before
    // the mask: the soft cap keeps (cap / scale) tanh(s scale / cap), with
    // tanh(x) = 1 - 2 / (exp(2x) + 1); ALiBi subtracts (slope / scale) times
    // the distance |i + Sk - Sq - key|.
    const float sc_in = MOD == kModSoftcap ? 2.f * a.scale / a.softcap * kLog2e : 0.f;
    const float sc_out = MOD == kModSoftcap ? a.softcap / a.scale : 0.f;
    const float slope = MOD == kModAlibi ? a.alibi[hq] / a.scale : 0.f;
    auto softmax_pv = [&](int blk, f32x16 (&s)[BN / 32]) {
        const int j0 = kofs + blk * BN;  // first key of the tile
        if constexpr (MOD == kModSoftcap) {
#pragma unroll
            for (int bb = 0; bb < BN / 32; ++bb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float e = __builtin_amdgcn_exp2f(s[bb][r] * sc_in);
                    s[bb][r] = sc_out * __builtin_fmaf(-2.f, __builtin_amdgcn_rcpf(e + 1.f), 1.f);
                }
        } else if constexpr (MOD == kModAlibi) {
#pragma unroll
            for (int bb = 0; bb < BN / 32; ++bb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = j0 + 32 * bb + 8 * (r >> 2) + 4 * g + (r & 3);
                    s[bb][r] = __builtin_fmaf(-slope, (float)abs(my_q + diag - key), s[bb][r]);
                }
        }
        const bool full = (j0 + BN <= Sk) && (!CAUSAL || j0 + BN - 1 <= q0 + diag) &&
                          (!windowed || j0 >= q0 + 31 + diag - a.window);
        if (!full) {
            const int lim = CAUSAL ? min(Sk - 1, my_q + diag) : Sk - 1;
            const int low = windowed ? my_q + diag - a.window : 0;  // first visible key
#pragma unroll
            for (int bb = 0; bb < BN / 32; ++bb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = j0 + 32 * bb + 8 * (r >> 2) + 4 * g + (r & 3);
                    s[bb][r] = (key <= lim && key >= low) ? s[bb][r] : -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int bb = 0; bb < BN / 32; ++bb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                mx = fmaxf(mx, s[bb][r]);
        mx = halves_max(mx);
        if (__any(mx > m_ref + thr)) {  // rare after the first tile
            const float m_new = fmaxf(m_ref, mx);
            // 0 when the row sees its first key; 1 when its maximum does not
            // move, also for a row that has seen no key yet (-inf - -inf is
            // NaN) while another row of the wave moves
            const float alpha =
                (m_new == m_ref) ? 1.f : __builtin_amdgcn_exp2f((m_ref - m_new) * c);
            l_half *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[db][r] *= alpha;
            m_ref = m_new;
        }
        const float mc = (m_ref == -INFINITY) ? 0.f : m_ref * c;

        Frag8 pf[BN / 16];
        float rs = 0.f;
#pragma unroll
        for (int bb = 0; bb < BN / 32; ++bb)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[bb][8 * h + 2 * w], c, -mc));
                    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[bb][8 * h + 2 * w + 1], c, -mc));
                    const uint32_t pk = pack_bf16x2(p0, p1);
                    pf[2 * bb + h].w[w] = pk;
                    rs += p0 + p1;
                }
        l_half += rs;

        // O^T += V^T P^T (a5)
        const int vb = blk & 1;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const uint16_t *vrow = &sVT[vb][(32 * db + l32) * C::VTS + 8 * g];
#pragma unroll
            for (int kc = 0; kc < BN / 16; ++kc) {
                Frag8 f;
                f.u = *(const uint4 *)(vrow + 16 * kc);
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.v, pf[kc].v, acc[db], 0, 0, 0);
            }
        }
    };

    // Blocks this wave computes (the workgroup iterates over nblk for the
    // barriers; fully masked tiles of a wave are skipped).
    const int nwb = (max(0, wave_end - kofs) + BN - 1) / BN;

    // ---- prologue: K and V tile 0 -----------------------------------------
    // Staged on every path (an empty key range reads zeros), then all global
    // loads are drained, so none issued before the loop is still in flight in
    // it: the prefetch issued inside the loop is waited on only where its
    // registers are consumed.
    load_k(0);
    load_v(0);
    store_k(0);
    store_v(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();

    // one step: the loads of tile j+1 go out, tile j's scores, softmax and PV
    // run from LDS, then tile j+1 is stored into the other buffers and the
    // workgroup syncs
    f32x16 s[BN / 32];
    for (int j = 0; j < nblk; ++j) {
        if (j + 1 < nblk) {
            load_k(j + 1);
            load_v(j + 1);
        }
        if (j < nwb) {
            scores(j & 1, s);
            softmax_pv(j, s);
        }
        if (j + 1 < nblk) {
            store_k((j + 1) & 1);
            store_v((j + 1) & 1);
        }
        __syncthreads();
    }

    // ---- epilogue (a6) ----------------------------------------------------
    const float l_tot = halves_sum(l_half);
    if (my_q < Sq) {
        // a row that saw a key has l >= 1 relative to its reference; l = 0
        // exactly means no key, and a NaN sum propagates
        const bool empty = l_tot == 0.f;
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

template <int D, int BN, int NW, bool CAUSAL, int MOD>
hipError_t launch_mod(const FwdArgs &a, hipStream_t stream)
{
    constexpr int BM = NW * 32;
    const int n_qtiles = (a.Sq + BM - 1) / BM;
    const long long n_tiles = (long long)a.B * a.Hq * n_qtiles;
    if (n_tiles > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fwd_kernel<D, BN, NW, CAUSAL, MOD>), dim3((unsigned)n_tiles), dim3(NW * 64),
                       0, stream, a, n_qtiles);
    return hipGetLastError();
}

template <int D, int BN, int NW, bool CAUSAL>
hipError_t launch(const FwdArgs &a, hipStream_t stream)
{
    if (a.softcap > 0.f)
        return launch_mod<D, BN, NW, CAUSAL, kModSoftcap>(a, stream);
    if (a.alibi != nullptr)
        return launch_mod<D, BN, NW, CAUSAL, kModAlibi>(a, stream);
    return launch_mod<D, BN, NW, CAUSAL, kModNone>(a, stream);
}

}  // namespace

// Tile configuration per head dimension: <BN keys per tile, NW waves,
// K staged one tile ahead of V>.
hipError_t launch_fwd(const FwdArgs &a, int d, bool causal, hipStream_t stream)
{
    if (a.cu_q != nullptr)  // packed variable-length batches: the persistent kernel only
        return d == 64 ? hipErrorNotSupported : launch_fwd_q64(a, d, causal, stream);
    switch (d) {
    case 64:  // 64-key tiles, four waves of 32 query rows
        return causal ? launch<64, 64, 4, true>(a, stream)
                      : launch<64, 64, 4, false>(a, stream);
    case 128:
    case 256:
        return launch_fwd_q64(a, d, causal, stream);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace miattn
