// prefill_kernel.h -- fused attention forward on gfx950 (head dimensions 64,
// 128 and 256), software-pipelined, on a persistent grid. The kernel template
// and its launcher; prefill_d64.hip, prefill_d128.hip and prefill_d256.hip
// instantiate one head dimension each.
//
// For every (batch, query head, query row) it computes the softmax-weighted
// sum of the visible value rows and the log-sum-exp of the scaled scores, as
// one pass over the keys under the online-softmax monoid (the tang paper,
// muni.works/research/tang, §2.2 "Comprehensions and monoids" and §2.3
// "Rewrites": running max, sum rescaled to it, accumulator rescaled to it).
// S^T = K Q^T runs on v_mfma_f32_32x32x16_bf16, so each lane owns one query
// column and 16 keys of every 32x32 score block; masked keys are selected to
// -inf (the identity of max); probabilities are rounded to bf16 in registers
// and feed O^T += V^T P^T directly, V^T read in the accumulator's permuted
// key order (the sum over keys is associative and commutative); the epilogue
// O = acc / l, LSE = m scale + ln l runs on the lanes that hold the row
// (§2.3: epilogues on the reducing thread), and a row with no visible key
// gets (+0, -inf).
//
// The design answers two gfx950 limits measured on a simpler kernel:
//
//  * LDS read bandwidth (about 150-200 bytes/ns per CU): every 16-byte K or V
//    fragment a wave reads from LDS feeds one 32x32x16 MFMA for the 32 query
//    rows the wave owns.
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
// accumulator alone takes 128 registers. Head dimension 64 runs four waves of
// 32 rows and two workgroups per CU (a tile step is then one group of four
// MFMAs per stage). Each wave runs a two-stage software pipeline per 32-key
// tile j, laid out in groups of four MFMAs with the VALU and LDS work placed
// between them:
//
//   stage A: S_{j+1} = K_{j+1} Q^T                   | exp/pack/row-sum of the
//            second 16 keys of tile j; row max of S_{j+1} for query block 0;
//            transposing LDS reads of V_j
//   stage B: O^T += V_j^T P_j                         | row max of S_{j+1} for
//            the last query block; exp/pack/row-sum of the first 16 keys of
//            tile j+1; LDS reads of K_{j+2}
//
// K and V tiles of 32 keys go global -> LDS by range-checked buffer DMA (keys
// past the item's last visible key arrive as zeros) into rings of four tiles,
// one barrier per tile. Both are stored fragment-major:
// each LDS read instruction
// of a wave reads one contiguous 1 KB (K, ds_read_b128) or 512 B (V,
// ds_read_b64_tr_b16) block, which is free of bank conflicts.
//
// The grid is persistent: one workgroup per resident slot walks a fixed list
// of work items (query tile of one query head). The copy stream does not stop
// at an item's end: the last steps of an item already copy the next item's
// first K and V tiles, so the next item starts without waiting for HBM.
//
// Variants, each a template argument so that the plain kernel carries none of
// their work: a sliding window (WIN: items start at the first tile any of
// their rows sees, tiles below are never copied), a score modifier (MOD: soft
// cap or ALiBi, applied to a tile's scores right after its QK MFMAs), and
// packed variable-length batches (VARLEN: each item takes its sequence's
// lengths, and the walk skips items past a sequence's end).
//
// The running maximum moves lazily: probabilities stay at most 2^8 above the
// reference and the accumulator is rescaled only on the rare tiles that move
// it. The check uses the tile's row sums, which the softmax computes anyway:
// a lane whose
// 16 probabilities sum to at most 2^8 has none above 2^8, and only a tile
// that fails (or a wave with a row that has seen no key yet) takes the exact
// maximum and recomputes its probabilities.

#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "launch.h"
#include "lds_copy.h"
#include "resident.h"
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


// Workgroup barrier that no memory access of the source crosses: the copies
// into LDS are invisible to the compiler, so it must not move an LDS read
// above the barrier that publishes the copied data.
__device__ __forceinline__ void barrier()
{
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Keep a value's computation inside its slot: an input pinned here cannot be
// consumed earlier, an output pinned here cannot be computed later (the
// compiler would otherwise sink work towards its uses across slots).
__device__ __forceinline__ void pin(float &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(uint32_t &x) { asm volatile("" : "+v"(x)); }

// One work item: the BM query rows of one (batch, query head) and the keys
// they see
struct Item {
    int64_t qrow0, krow0;  // first row of the query head / the item's first key row
    int q_wg, kv_end, nblk;
    int kofs;  // key of the item's tile 0 (nonzero only with a sliding window)
    float slope;  // ALiBi slope of the query head over the scale (raw score units)
    int sq, sk;   // query rows and keys of the item's sequence
    bool live;    // the item has query rows (a packed batch has items past its sequences' ends)
};

// Score modifiers: none, soft cap, ALiBi, or the soft cap and then ALiBi
enum { kModNone = 0, kModSoftcap = 1, kModAlibi = 2, kModBoth = 3 };

template <bool CAUSAL, int NWV, int D, int WPE, bool WIN, int MOD, bool VARLEN>
__global__ void __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
fwd_q64_kernel(FwdArgs a, int n_qtiles, int n_items)
{
    // one block of 32 query rows per wave (the state arrays below keep a
    // query-block index of extent QB = 1)
    constexpr int QB = 1;
    constexpr int BN = 32;             // keys per tile
    constexpr int BM = NWV * 32 * QB;  // query rows per work item
    constexpr int KKN = D / 16;        // 16-dim steps of QK = K fragments = copy instructions per tile
    constexpr int DBN = D / 32;        // 32-dim blocks of the output
    constexpr int DPW = KKN / NWV;     // copy instructions per wave per tile, each of K and V
    constexpr int NG = QB * KKN / 4;   // groups of four MFMAs per stage
    constexpr int NPV = QB * DBN;      // PV MFMAs per 16-key chunk
    // K and V rings of RING tiles: K tile j+RING and V tile j+RING-1 are copied
    // in step j (8 KB per tile at head dimension 128, 16 KB at 256: 64 or
    // 128 KB of the 160 KB of LDS)
    constexpr int RING = 4;
    // ROWCOPY (head dimensions 128 and 256): copy i of a tile takes RPB whole
    // rows of 2D bytes, keys i, i + NBLK, .., into a 1 KB block; the blocks lie
    // KPB (K) or VPB (V) bytes apart. Otherwise (64) fragment-major (see the
    // copies below). A fragment-major copy (32 keys x 32 bytes) touches four
    // times the cache lines of a copy of whole rows and kept the L1 busy.
    constexpr bool ROWCOPY = D == 128 || D == 256;
    constexpr int RPB = 512 / D;      // rows per 1 KB block (ROWCOPY)
    constexpr int NBLK = 32 / RPB;    // blocks per tile (ROWCOPY)
    constexpr int CPT = DPW;  // copy instructions per wave per tile, each of K and V
    // A step's copies go one after each group of four MFMAs (the K copies
    // after the last CPT groups of stage A, the V copies after the first CPT of
    // stage B) instead of all at the step's start, where every wave's copies
    // queued at once in the CU's address unit (12 to 27 ns per 1 KB copy, by
    // shape) and held the waves at issue: 2.9% at head dimension 256, 3.5% at
    // 128, 1-2% at 64, outputs bit-identical. (The masked steps still issue
    // theirs at once.)
    constexpr bool SPREAD = true;
    constexpr int INFLIGHT = CPT + 2 * CPT * (RING - 3);  // copies newer than K tile j+3 at step j's end
    static_assert((RING & (RING - 1)) == 0 && RING >= 4, "ring of 2^n >= 4 tiles");
    static_assert((NG == 1 || NG == 2 || NG == 4) && NWV * DPW == KKN && INFLIGHT < 64,
                  "tile step shape");
    static_assert(!ROWCOPY || (BN == 32 && NBLK == KKN), "row copies: 32-key tiles, one block per copy");
    static_assert(!SPREAD || CPT <= NG, "at most one copy of K and one of V per group");
    constexpr int TILE_CH = BN * D / 8;  // 16-byte chunks per tile
    constexpr int KPB = D == 256 ? 1040 : 1056, VPB = 1088;  // block strides of ROWCOPY (bytes)
    constexpr uint32_t KTILE_B = ROWCOPY ? NBLK * KPB : TILE_CH * 16;
    constexpr uint32_t VTILE_B = ROWCOPY ? NBLK * VPB : TILE_CH * 16;

    __shared__ __attribute__((aligned(16))) uint4 sK_[RING * KTILE_B / 16];  // K ring
    __shared__ __attribute__((aligned(16))) uint4 sV_[RING * VTILE_B / 16];  // V ring
    uint4 *const sK = sK_;  // the lambdas below may not name __shared__ variables
    uint4 *const sV = sV_;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int g = lane >> 5;

    // query rows and keys of the current item's sequence (all items share them
    // unless the batch is packed with variable lengths)
    int Sq = a.Sq, Sk = a.Sk;
    int diag = Sk - Sq;
    // WIN: sliding window (a separate instantiation, so that the kernel
    // without one carries none of its work); query i sees keys from i + wlo on
    int wlo = WIN ? diag - a.window : 0;
    const int G = a.Hq / a.Hkv;

    // ---- schedule --------------------------------------------------------------------
    // Workgroup w runs on XCD w % 8 and takes, round after round, items
    // xcd + 8 li: li = r GX + s in even rounds, r GX + GX-1-s in odd ones (s =
    // w / 8, GX = workgroups per XCD). The items of an XCD are the ones the
    // tile order puts there, and the alternating direction pairs heavy
    // causal tiles with light ones.
    const int xcd = (int)blockIdx.x & 7, wslot = (int)blockIdx.x >> 3, GX = (int)gridDim.x >> 3;
    auto item_id = [&](int r) __attribute__((always_inline)) {
        const int li = r * GX + ((r & 1) ? GX - 1 - wslot : wslot);
        return xcd + 8 * li;
    };
    // Fewer (batch, kv-head) units than XCDs, dividing them (e.g. two): each
    // unit gets 8 / units XCDs, each XCD an equal share of the unit's query
    // heads, heaviest query tile first. The workgroups of an XCD then read one
    // unit's K and V, in step, instead of every unit's.
    const int n_units = a.B * a.Hkv;
    const int xpu = n_units < 8 && 8 % n_units == 0 ? 8 / n_units : 0;  // XCDs per unit
    const bool by_xcd = xpu > 0 && G % xpu == 0;
    // A packed batch of at most 64 sequences walks a compacted list instead:
    // every wave holds sequence b's ranges in lane b, ranks the sequences by
    // query tiles then keys (longest first), and numbers the live items rank
    // by rank (rank r: each sequence's r-th heaviest query tile), the
    // sequences of a rank in that order and their query heads together. No
    // item of the list is past a sequence's end, and the heavy tiles come
    // first.
    const bool compact = VARLEN && a.B <= 64;
    const int xpu_v = a.Hkv < 8 && 8 % a.Hkv == 0 ? 8 / a.Hkv : 0;  // XCDs per kv-head
    const bool heads_by_xcd =
        compact && a.Hq % 8 == 0 && (a.Hkv % 8 == 0 || (xpu_v > 0 && G % xpu_v == 0));
    int v_qlo = 0, v_sq = 0, v_klo = 0, v_sk = 0, v_nq = 0, v_pos = 0;  // lane b: sequence b
    int n_live = n_items;
    if constexpr (VARLEN) {
        if (compact) {
            if (lane < a.B) {
                v_qlo = min(max(a.cu_q[lane], 0), a.total_q);
                const int q_hi = min(max(a.cu_q[lane + 1], v_qlo), a.total_q);
                v_klo = min(max(a.cu_k[lane], 0), a.total_k);
                const int k_hi = min(max(a.cu_k[lane + 1], v_klo), a.total_k);
                v_sq = min(q_hi - v_qlo, a.Sq);
                v_sk = min(k_hi - v_klo, a.Sk);
                v_nq = (v_sq + BM - 1) / BM;
            }
            int pos = 0, live = 0;
            for (int o = 0; o < a.B; ++o) {
                const int nqo = __builtin_amdgcn_readlane(v_nq, o);
                const int sko = __builtin_amdgcn_readlane(v_sk, o);
                pos += (nqo > v_nq) || (nqo == v_nq && (sko > v_sk || (sko == v_sk && o < lane)));
                live += nqo;
            }
            v_pos = pos;
            n_live = min(n_items, live * a.Hq);
        }
    }
    int rank_r = 0, rank_c0 = 0;  // the walk's current rank and its first list index
    auto rank_size = [&](int r) __attribute__((always_inline)) {
        return a.Hq * (int)__builtin_popcountll(__ballot(lane < a.B && v_nq > r));
    };
    auto describe = [&](int id) __attribute__((always_inline)) {
        TileOrder to;
        int b_c = 0;
        if (compact) {
            // ids only grow along a workgroup's walk
            for (int n = rank_size(rank_r); id >= rank_c0 + n; n = rank_size(rank_r)) {
                rank_c0 += n;
                ++rank_r;
            }
            const int idx = id - rank_c0, k = idx / a.Hq, pq = idx - k * a.Hq;
            // A (sequence, rank) block of Hq items starts at a multiple of Hq,
            // so with Hq % 8 == 0 item pq runs on XCD pq % 8. The G query heads
            // of a kv-head then go to one XCD (or, with fewer than 8 kv-heads,
            // to an equal share of XCDs), where they read its K and V through
            // one L2 instead of one L2 each.
            int hq_c = pq;
            if (heads_by_xcd) {
                const int x = pq & 7, t = pq >> 3;
                hq_c = a.Hkv % 8 == 0 ? (x + 8 * (t / G)) * G + t % G
                                      : (x / xpu_v) * G + (x % xpu_v) * (G / xpu_v) + t;
            }
            const unsigned long long hit = __ballot(lane < a.B && v_pos == k);
            b_c = hit ? (int)__builtin_ctzll(hit) : 0;  // exactly one lane matches
            to.unit = b_c * a.Hkv + hq_c / G;
            to.gq = hq_c % G;
            to.qtile = __builtin_amdgcn_readlane(v_nq, b_c) - 1 - rank_r;
        } else if (by_xcd) {
            const int gsub = G / xpu, x = id & 7, pos = id >> 3;
            const int rank = pos / gsub;
            to.unit = x / xpu;
            to.gq = (x % xpu) * gsub + (pos - rank * gsub);
            to.qtile = CAUSAL ? n_qtiles - 1 - rank : rank;
        } else {
            to = tile_order_grouped(id, n_units, G, n_qtiles, CAUSAL, GX);
        }
        const int b = to.unit / a.Hkv;
        const int kvh = to.unit - b * a.Hkv;
        const int hq = kvh * G + to.gq;
        Item it;
        int64_t kbase;
        if (compact) {
            it.sq = __builtin_amdgcn_readlane(v_sq, b_c);
            it.sk = __builtin_amdgcn_readlane(v_sk, b_c);
            it.qrow0 = (int64_t)hq * a.total_q + __builtin_amdgcn_readlane(v_qlo, b_c);
            kbase = (int64_t)kvh * a.total_k + __builtin_amdgcn_readlane(v_klo, b_c);
        } else if constexpr (VARLEN) {
            // sequence b of a packed batch; offsets clamped into the tensors
            // (at most the longest length), so no access leaves them
            const int q_lo = min(max(a.cu_q[b], 0), a.total_q);
            const int q_hi = min(max(a.cu_q[b + 1], q_lo), a.total_q);
            const int k_lo = min(max(a.cu_k[b], 0), a.total_k);
            const int k_hi = min(max(a.cu_k[b + 1], k_lo), a.total_k);
            it.sq = min(q_hi - q_lo, a.Sq);
            it.sk = min(k_hi - k_lo, a.Sk);
            it.qrow0 = (int64_t)hq * a.total_q + q_lo;
            kbase = (int64_t)kvh * a.total_k + k_lo;
        } else {
            it.sq = a.Sq;
            it.sk = a.Sk;
            it.qrow0 = ((int64_t)b * a.Hq + hq) * a.Sq;
            kbase = ((int64_t)b * a.Hkv + kvh) * a.Sk;
        }
        const int dg = it.sk - it.sq;
        it.slope = (MOD & kModAlibi) ? a.alibi[hq] / a.scale : 0.f;
        it.q_wg = to.qtile * BM;
        it.live = it.q_wg < it.sq;
        const int q_wg_last = min(it.q_wg + BM, it.sq) - 1;
        const int kv_end = CAUSAL ? min(it.sk, max(0, q_wg_last + dg + 1)) : it.sk;
        // With a sliding window the item's keys start at the tile holding its
        // first row's first visible key; tiles below it are hidden from every
        // row and never copied. Tile indices and key counts of the item count
        // from that tile's first key.
        it.kofs = WIN ? min(kv_end, max(0, it.q_wg + dg - a.window)) / BN * BN : 0;
        it.krow0 = kbase + it.kofs;
        it.kv_end = kv_end - it.kofs;
        it.nblk = (it.kv_end + BN - 1) / BN;
        return it;
    };

    // ---- global -> LDS copies ---------------------------------------------------
    // A tile takes D/16 copy instructions (1 KB each) for K and as many for V;
    // wave w issues instructions DPW w .. DPW w + DPW - 1 of each. Every copy's
    // descriptor covers just its tile up to the item's last visible key, so
    // keys past it read as zero and copies past the range move no data.
    //
    // K layout: block kk (1 KB) holds lane L's A fragment for dims
    // 16kk + 8(L/32) .. +7 of key L%32, at byte 16L.
    // V layout: block r = (2 db + kc) * 2 + hh (512 B) holds, at byte 8L for
    // L = 16G + 4jj + q, the four values V[16kc + 8hh + 4(G/2) + jj]
    // [32db + 16(G%2) + 4q .. +3]; a transposing 8-byte read of the block
    // gives lane L the values of dim 32db + L%32 at four consecutive keys.
    //
    // ROWCOPY layout: key r at byte (r % NBLK) * PB + (r / NBLK) * 2D of the
    // tile (PB = KPB or VPB); wave w issues copies CPT w .. CPT w + CPT - 1,
    // lane L of copy i taking 16 bytes of key i + NBLK (L / (D/8)). At 128 the
    // K rows of odd r / NBLK hold their 16-byte chunks in pairs swapped (chunk
    // c at c ^ 1). Strides and swap keep both kinds of read free of bank
    // conflicts under the way LDS serves them (16-byte reads in passes of 16
    // lanes: l % 16 < 8 of one 16-lane row with l % 16 >= 8 of its neighbour;
    // transposing 8-byte reads in passes of 32 lanes): each pass of a K
    // fragment read reaches 16 different 16-byte bank groups, and the
    // transposing V reads of a key quad start 64 bytes apart.
    const auto kswap = [](int quarter) { return D == 128 ? (quarter & 1) : 0; };
    uint32_t koff[CPT], voff[CPT];
#pragma unroll
    for (int h = 0; h < CPT; ++h) {
        if constexpr (ROWCOPY) {
            constexpr int CPR = D / 8;  // 16-byte chunks per row
            const int quarter = lane / CPR, chunk = lane % CPR;
            const int key = CPT * wave + h + NBLK * quarter;
            koff[h] = (uint32_t)(key * 2 * D + 16 * (chunk ^ kswap(quarter)));
            voff[h] = (uint32_t)(key * 2 * D + 16 * chunk);
        } else {
            const int i = DPW * wave + h;
            koff[h] = (uint32_t)(l32 * D + 16 * i + 8 * g) * 2;
            const int db = i >> 1, kc = i & 1, tt = l32;
            const int G4 = tt >> 3, jj = (tt >> 1) & 3, qh = tt & 1;
            const int key = 16 * kc + 8 * g + 4 * (G4 >> 1) + jj;
            const int dim = 32 * db + 16 * (G4 & 1) + 8 * qh;
            voff[h] = (uint32_t)(key * D + dim) * 2;
        }
    }
    // LDS byte addresses (M0 values) of this wave's share of ring slot 0, and
    // the distance between its consecutive copies
    const uint32_t m0k = lds_addr(sK) + (ROWCOPY ? KPB * CPT * wave : 1024 * DPW * wave);
    const uint32_t m0v = lds_addr(sV) + (ROWCOPY ? VPB * CPT * wave : 1024 * DPW * wave);
    constexpr uint32_t KSTEP = ROWCOPY ? KPB : 1024, VSTEP = ROWCOPY ? VPB : 1024;
    // copy of the BN keys from src on, of which `keys` exist (none if keys <=
    // 0), into ring slot s. The descriptor ends at the last key that exists:
    // keys past it read as zero, and a copy of no key moves no data.
    auto dma_k = [&](int s, const uint16_t *src, int keys) __attribute__((always_inline)) {
        const u32x4 d = make_desc(src, (uint32_t)max(keys, 0) * (D * 2));
        const uint32_t m0 = m0k + (uint32_t)(s & (RING - 1)) * KTILE_B;
#pragma unroll
        for (int h = 0; h < CPT; ++h)
            copy_to_lds(d, koff[h], m0 + KSTEP * h);
    };
    auto dma_v = [&](int s, const uint16_t *src, int keys) __attribute__((always_inline)) {
        const u32x4 d = make_desc(src, (uint32_t)max(keys, 0) * (D * 2));
        const uint32_t m0 = m0v + (uint32_t)(s & (RING - 1)) * VTILE_B;
#pragma unroll
        for (int h = 0; h < CPT; ++h)
            copy_to_lds(d, voff[h], m0 + VSTEP * h);
    };
    // ---- fragments from LDS -------------------------------------------------------
    Frag8 kf[KKN];      // A fragments of the K tile the next QK uses
    bf16x8 vf[DBN][2];  // A fragments of V^T: [d-block][16-key chunk]
    // Reads take a lane's LDS byte address in the slot (K: slot + 16 lane, V:
    // slot + 8 lane), computed once per step ahead of everything else so that
    // the reads can start with the step's first MFMA.
    // (ROWCOPY: K lane l reads key l%32 at dims 16kk + 8(l/32), 32 bytes per
    // kk further; V lane 16m + 4e + c supplies key 16kc + 8hh + 4(m/2) + e at
    // dims 32db + 16(m%2) + 4c .. +3 to the transposing read of its group)
    auto read_k = [&](uint32_t addr, int kk) __attribute__((always_inline)) {
        typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
        kf[kk].u = __builtin_bit_cast(uint4, *(lds_u32x4 *)(uintptr_t)(addr + (ROWCOPY ? 32 : 1024) * kk));
    };
    auto vimm = [](int db, int kc, int hh) {
        if constexpr (ROWCOPY)
            return D == 256 ? (uint32_t)(8 * hh * VPB + 512 * kc + 64 * db)
                            : (uint32_t)(512 * kc + 256 * hh + 64 * db);
        return (uint32_t)(((2 * db + kc) * 2 + hh) * 512);
    };
    auto read_v = [&](uint32_t addr, int db, int kc) __attribute__((always_inline)) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(uintptr_t)(addr + vimm(db, kc, 0)));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(uintptr_t)(addr + vimm(db, kc, 1)));
        const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        vf[db][kc] = __builtin_bit_cast(bf16x8, both);
    };
    const uint32_t lds_k = lds_addr(sK), lds_v = lds_addr(sV);
    const uint32_t klane =
        ROWCOPY ? (uint32_t)((l32 % NBLK) * KPB + 2 * D * (l32 / NBLK) + 16 * (g ^ kswap(l32 / NBLK)))
                : (uint32_t)(16 * lane);
    const uint32_t vlane =
        ROWCOPY ? (uint32_t)((4 * (lane >> 5) + ((lane & 15) >> 2)) * VPB + 32 * ((lane >> 4) & 1) +
                             16 * ((lane & 3) >> 1) + 8 * (lane & 1))
                : (uint32_t)(8 * lane);
    auto kread_addr = [&](int s) __attribute__((always_inline)) {
        return lds_k + (uint32_t)(s & (RING - 1)) * KTILE_B + klane;
    };
    auto vread_addr = [&](int s) __attribute__((always_inline)) {
        return lds_v + (uint32_t)(s & (RING - 1)) * VTILE_B + vlane;
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
    bool ref_unset = true;  // some row of the wave still has m_ref = -inf
    f32x16 acc[QB][D / 32];
    auto reset_state = [&]() __attribute__((always_inline)) {
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
        tsum = 0.f;
        ref_unset = true;
    };

    // ---- the current and the next item (the lambdas below read these) ---------------
    int ph = 0;                      // ring slot of the current item's tile 0
    int nblk = 0, nwb = 0, q0 = 0, kv_end = 0, kofs = 0;
    float slope = 0.f;
    int64_t qrow0 = 0, krow0 = 0;
    bool has_next = false;
    int kv_end_n = 0, q_wg_n = 0;  // kv_end_n = 0 without a next item
    int64_t qrow0_n = 0;
    // The copy stream: the next K / V copy's source and the keys that exist
    // from it on, and the next item's tile 0
    const uint16_t *kp = a.k, *vp = a.v, *kn = a.k, *vn = a.v;
    int krem = 0, vrem = 0;

    // ---- Q fragments (B operands of S^T = K Q^T) ------------------------------
    bf16x8 qf[QB][KKN];
    // Q rows of an item (query head rows from qrow0_, the wave's first row q0w)
    // straight from global memory into the fragments; rows >= Sq read as 0
    auto load_q = [&](int64_t qrow0_, int q0w, int sq_) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + qrow0_ * D, (uint32_t)sq_ * D * 2);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const uint32_t off = (uint32_t)(q0w + 32 * qb + l32) * D * 2 + 16 * g;
#pragma unroll
            for (int kk = 0; kk < KKN; ++kk) {
                Frag8 f;
                f.u = buf_load16(rq, off + 32 * kk);
                qf[qb][kk] = f.v;
            }
        }
    };

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
    // 16h .. 16h+15 = r in [8h, 8h+8). Every piece pins
    // its outputs at the end of its group of MFMAs (else the compiler sinks
    // them towards their uses); inside the group its independent chains
    // overlap one another.
    //
    // probabilities of scores r = 8h + 4quad .. +3 -> two packed bf16 pairs;
    // init: the tile's first quad, whose sum starts tsum (an add to the zero
    // it was reset to would cost one VALU instruction per tile: x + 0 is not
    // x for x = -0, so the compiler keeps it)
    auto probs_quad = [&](const Sc &s, Pc &p, int qb, int h, int quad, bool init = false)
        __attribute__((always_inline)) {
        float e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][8 * h + 4 * quad + i], c, nmc[qb]));
        p[qb][h].w[2 * quad] = pack_bf16x2(e[0], e[1]);
        p[qb][h].w[2 * quad + 1] = pack_bf16x2(e[2], e[3]);
        const float q4 = (e[0] + e[1]) + (e[2] + e[3]);
        tsum = init ? q4 : tsum + q4;
        pin(tsum);
        pin(p[qb][h].w[2 * quad]);
        pin(p[qb][h].w[2 * quad + 1]);
    };
    // Score modifiers on the raw scores of tile j (the kernel's scores are
    // q.k before the scale): the soft cap keeps (cap / scale) tanh(s scale /
    // cap), tanh(x) = 1 - 2 / (exp(2x) + 1); ALiBi subtracts (slope / scale)
    // times the distance |i + Sk - Sq - key|; with both, the cap comes first.
    // Applied before the mask.
    const float sc_in = (MOD & kModSoftcap) ? 2.f * a.scale / a.softcap * kLog2e : 0.f;
    const float sc_out = (MOD & kModSoftcap) ? a.softcap / a.scale : 0.f;
    auto modify_tile = [&](Sc &s, int j) __attribute__((always_inline)) {
        if constexpr ((MOD & kModSoftcap) != 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = __builtin_amdgcn_exp2f(s[0][r] * sc_in);
                s[0][r] = sc_out * __builtin_fmaf(-2.f, __builtin_amdgcn_rcpf(e + 1.f), 1.f);
            }
        }
        if constexpr ((MOD & kModAlibi) != 0) {
            // distance to key offset 0, in f32 (exact below 2^24): per score one
            // subtraction of a constant and one FMA whose operand modifier
            // takes the absolute value
            const float d0 = (float)(q0 + l32 + diag - kofs - j * BN - 4 * g);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float dist = d0 - (float)(8 * (r >> 2) + (r & 3));
                s[0][r] = __builtin_fmaf(-slope, __builtin_fabsf(dist), s[0][r]);
            }
        }
    };
    // The keys of tile j that row q0 + 32 qb + l32 sees: score r (key
    // 8(r/4) + 4g + r%4 of the tile) is visible iff rlo <= 8(r/4) + r%4 <= rel.
    // Past the wave's last tile it sees none.
    auto visible_offsets = [&](int qb, int j, int &rel, int &rlo) __attribute__((always_inline)) {
        const int my_q = q0 + 32 * qb + l32;
        const int lim = j < nwb ? (CAUSAL ? min(Sk - 1, my_q + diag) : Sk - 1) - kofs : -1;
        const int base = j * BN + 4 * g;
        rel = lim - base;
        rlo = WIN ? my_q + wlo - kofs - base : -BN;
    };
    // row maximum in three parts (scores 0-7, scores 8-15, both halves of the
    // wave); a masked tile first selects hidden keys to -inf
    float mxa[QB], mxb[QB];
    auto row_max = [&](Sc &s, int qb, int part, int j, bool masked) __attribute__((always_inline)) {
        if (part < 2) {
            if (masked) {
                int rel, rlo;
                visible_offsets(qb, j, rel, rlo);
#pragma unroll
                for (int r = 8 * part; r < 8 * part + 8; ++r) {
                    const int o = 8 * (r >> 2) + (r & 3);
                    s[qb][r] = (o <= rel && (!WIN || o >= rlo)) ? s[qb][r] : -INFINITY;
                }
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
        int rel, rlo;
        visible_offsets(qb, j, rel, rlo);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int o = 8 * (r >> 2) + (r & 3);
            s[qb][r] = (o <= rel && (!WIN || o >= rlo)) ? s[qb][r] : -INFINITY;
        }
    };
    // One query block per wave: the lazy reference is checked by the tile's
    // row sums instead of its row maximum. A lane's 16 probabilities are all
    // at most 2^8 when their sum is, which is the bound the reference keeps;
    // otherwise (or while some row has not seen a key) the tile takes this
    // slow path: exact maximum, reference update, rescale, probabilities
    // again. The scores are already masked.
    auto slow_tile = [&](Sc &s, Pc &p) __attribute__((always_inline)) {
        row_max(s, 0, 0, 0, false);
        row_max(s, 0, 1, 0, false);
        row_max(s, 0, 2, 0, false);
        move_ref(0);
        apply_alpha();
        probs_quad(s, p, 0, 0, 0, true);
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

    // ---- prologue of an item ------------------------------------------------------
    // The first K tiles (0 .. RING-1) and V tiles (0 .. RING-2) are normally
    // copied during the previous item's last steps; the first item, and one
    // that follows an item of fewer than RING tiles, copies what is missing
    // here and drains. Then S_0, its statistics and the first chunk of P_0
    // without overlap, and K tile 1 into registers.
    Sc sA, sB;  // scores of the even / odd tile in flight
    Pc pA, pB;  // probabilities of the even / odd tile
    // Head dimension 256 loads the next item's Q rows into registers during
    // the current item's epilogue, 128 loads them here (each the faster of the
    // two as measured).
    constexpr bool QPREF = (D == 256);
    auto prologue = [&](int kmiss, int vmiss) __attribute__((always_inline)) {
        if constexpr (!QPREF)
            load_q(qrow0, q0, Sq);
        if (!QPREF || kmiss > 0 || vmiss > 0) {
            for (int t = 0; t < kmiss; ++t)
                dma_k(ph + t, a.k + (krow0 + t * BN) * D, kv_end - t * BN);
            for (int t = 0; t < vmiss; ++t)
                dma_v(ph + t, a.v + (krow0 + t * BN) * D, kv_end - t * BN);
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the copies (and Q)
        }
        barrier();
#pragma unroll
        for (int kk = 0; kk < KKN; ++kk)
            read_k(kread_addr(ph), kk);
#pragma unroll
        for (int kk = 0; kk < KKN; ++kk)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                qk_mfma(sA, qb, kk);
        modify_tile(sA, 0);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            row_max(sA, qb, 0, 0, true);
            row_max(sA, qb, 1, 0, true);
            row_max(sA, qb, 2, 0, true);
            move_ref(qb);
            probs_quad(sA, pA, qb, 0, 0, qb == 0);
            probs_quad(sA, pA, qb, 0, 1);
        }
        apply_alpha();  // the first reference moves consume their rescale here
        ref_unset = __any(m_ref[0] == -INFINITY);
#pragma unroll
        for (int kk = 0; kk < KKN; ++kk)
            read_k(kread_addr(ph + 1), kk);
        // every wave has read K tile 0 before step 0 copies K tile RING into its slot
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        barrier();
    };

    // Copies of step j of an item: K of stream position j+RING and V of
    // j+RING-1, which are the item's own tiles, the next item's first tiles (K
    // 0 .. RING-1, V 0 .. RING-2), or nothing.
    // (SPREAD: descriptors and LDS addresses only; the step issues copy h of K
    // after its stage-A group h and copy h of V after its stage-B group h)
    u32x4 cdk, cdv;
    uint32_t cmk = 0, cmv = 0;
    auto step_copies = [&](int j, auto SPREADc) __attribute__((always_inline)) {
        if constexpr (decltype(SPREADc)::value) {
            cdk = make_desc(kp, (uint32_t)max(krem, 0) * (D * 2));
            cdv = make_desc(vp, (uint32_t)max(vrem, 0) * (D * 2));
            cmk = m0k + (uint32_t)((ph + j) & (RING - 1)) * KTILE_B;
            cmv = m0v + (uint32_t)((ph + j + RING - 1) & (RING - 1)) * VTILE_B;
        } else {
            dma_k(ph + j, kp, krem);
            dma_v(ph + j + RING - 1, vp, vrem);
        }
        // after the item's last tile, the next item's first ones
        if (j + RING + 1 == nblk) {
            kp = kn;
            krem = kv_end_n;
        } else {
            kp += BN * D;
            krem -= BN;
        }
        if (j + RING == nblk) {
            vp = vn;
            vrem = kv_end_n;
        } else {
            vp += BN * D;
            vrem -= BN;
        }
    };
    // wait until the copies the next step reads (V tile j+1, K tile j+3) are
    // complete -- the INFLIGHT newer copy instructions of this wave may still
    // fly -- and barrier
    auto step_end = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(INFLIGHT));
        barrier();
    };

    // ---- one tile step ------------------------------------------------------------------
    // Tile t of the copy stream lives in ring slot t % RING; the current
    // item's tile j is stream position ph + j. Step j: copies of stream
    // positions j+RING (K, into tile j's slot, last read in step j-2) and
    // j+RING-1 (V, into tile j-1's slot, last read in step j-1); stage A;
    // stage B; wait; barrier.
    auto step = [&](auto MASKc, int j, Sc &sc, Sc &sn, Pc &pc, Pc &pn) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(MASKc)::value;
        uint32_t kread = kread_addr(ph + j + 2);  // K tile j+2
        uint32_t vread = vread_addr(ph + j);      // V tile j
        pin(kread);
        pin(vread);
        step_copies(j, IntC<SPREAD>{});
        slot_end();

        // Stage A, NG groups of four MFMAs (QK of tile j+1). The first (at
        // most two) groups read V_j and compute chunk 1 of tile j's
        // probabilities.
        constexpr int NRV = 2 * DBN;          // read_v calls per tile (two reads each)
        constexpr int VSL = NG >= 2 ? 8 : 4;  // MFMA slots that carry them
#pragma unroll
        for (int grp = 0; grp < NG; ++grp) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int sl = 4 * grp + i;
                qk_mfma(sn, sl / KKN, sl % KKN);
                if (sl < VSL)
#pragma unroll
                    for (int c = sl * NRV / VSL; c < (sl + 1) * NRV / VSL; ++c)
                        read_v(vread, c >> 1, c & 1);
            }
            if (NG == 1) {
                probs_quad(sc, pc, 0, 1, 0);
                probs_quad(sc, pc, 0, 1, 1);
            } else if (grp < 2) {
                probs_quad(sc, pc, 0, 1, grp);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                if (grp < 2)
                    __builtin_amdgcn_sched_group_barrier(0x100, 2 * NRV / VSL, 0);  // LDS reads
                __builtin_amdgcn_sched_group_barrier(0x002, NG == 1 ? 8 : 4, 0);  // VALU
            }
            slot_end();
            if constexpr (SPREAD) {
                if (grp >= NG - CPT) {
                    copy_to_lds(cdk, koff[grp - (NG - CPT)], cmk + KSTEP * (grp - (NG - CPT)));
                    slot_end();
                }
            }
        }
        check_tile(sc, pc);  // tile j's probabilities are complete
        slot_end();

        // Stage B, NG groups of four MFMAs (PV of tile j). Each group reads
        // KKN/NG K_{j+2} fragments. Group 0 applies the score modifier and the
        // mask to tile j+1, the next groups compute its chunk 0.
        constexpr int KPG = KKN / NG;  // K reads per group
#pragma unroll
        for (int grp = 0; grp < NG; ++grp) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int sl = 4 * grp + i;
                const int idx = sl % NPV;
                pv_mfma(pc, 0, idx, sl / NPV);
                if (i < KPG)
                    read_k(kread, KPG * grp + i);
            }
            if (MOD != kModNone && grp == 0)
                modify_tile(sn, j + 1);
            if (MASK && grp == 0)
                mask_tile(sn, 0, j + 1);
            if (NG == 1) {
                probs_quad(sn, pn, 0, 0, 0, true);
                probs_quad(sn, pn, 0, 0, 1);
            }
            if (NG == 2 && grp == 1) {
                probs_quad(sn, pn, 0, 0, 0, true);
                probs_quad(sn, pn, 0, 0, 1);
            }
            if (NG == 4 && (grp == 1 || grp == 2))
                probs_quad(sn, pn, 0, 0, grp - 1, grp == 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                if (i < KPG)
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
                __builtin_amdgcn_sched_group_barrier(0x002, NG == 1 ? 8 : 4, 0);  // VALU
            }
            slot_end();
            if constexpr (SPREAD) {
                if (grp < CPT) {
                    copy_to_lds(cdv, voff[grp], cmv + VSTEP * grp);
                    slot_end();
                }
            }
        }
        step_end();
    };

    // Masked steps. From tile nwb on the wave sees no key of the tiles it
    // would touch (PV of tile j, QK of tile j+1): it only issues its share of
    // the copies and keeps the barrier, leaving its SIMD to the other wave.
    // (Step nwb-1 still runs: its PV is live, and the tile nwb it scores is
    // all masked and never checked.)
    auto mstep = [&](int j, Sc &sc, Sc &sn, Pc &pc, Pc &pn) __attribute__((always_inline)) {
        if (j < nwb) {
            step(IntC<1>{}, j, sc, sn, pc, pn);
        } else {
            step_copies(j, IntC<0>{});
            step_end();
        }
    };

    // ---- epilogue of an item ------------------------------------------------------
    // O = acc / l in bf16 and LSE. Lanes l and l+32 hold the same row, dims
    // 4(l/32) .. +3 of every 8: they swap half of their packed values so that
    // each stores 16 contiguous bytes (half the store instructions).
    auto epilogue = [&]() __attribute__((always_inline)) {
        apply_alpha();
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int my_q = q0 + 32 * qb + l32;
            const float l_tot = halves_sum(l_half[qb]);
            // l = 0 exactly only for a row that saw no key (otherwise l >= 1
            // relative to the reference); a NaN sum propagates
            const bool empty = l_tot == 0.f;
            const float inv = empty ? 0.f : __builtin_amdgcn_rcpf(l_tot);
            uint16_t *orow = a.o + (qrow0 + min(my_q, Sq - 1)) * D + 8 * g;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const f32x16 &x = acc[qb][db];
                    const int r0 = 8 * pr, r1 = 8 * pr + 4;  // rho 2pr and 2pr+1
                    const uint32_t a0 = empty ? 0u : pack_bf16x2(x[r0] * inv, x[r0 + 1] * inv);
                    const uint32_t a1 = empty ? 0u : pack_bf16x2(x[r0 + 2] * inv, x[r0 + 3] * inv);
                    const uint32_t b0 = empty ? 0u : pack_bf16x2(x[r1] * inv, x[r1 + 1] * inv);
                    const uint32_t b1 = empty ? 0u : pack_bf16x2(x[r1 + 2] * inv, x[r1 + 3] * inv);
                    // lane g = 0 keeps rho 2pr and receives the partner's; g = 1 keeps 2pr+1
                    const uint32_t s0 = g == 0 ? b0 : a0, s1 = g == 0 ? b1 : a1;
                    const auto t0 = __builtin_amdgcn_permlane32_swap(s0, s0, false, false);
                    const auto t1 = __builtin_amdgcn_permlane32_swap(s1, s1, false, false);
                    const uint32_t p0 = g == 0 ? t0[1] : t0[0], p1 = g == 0 ? t1[1] : t1[0];
                    const uint4 w = g == 0 ? make_uint4(a0, a1, p0, p1) : make_uint4(p0, p1, b0, b1);
                    if (my_q < Sq)
                        *(uint4 *)(orow + 32 * db + 16 * pr) = w;
                }
            if (g == 0 && my_q < Sq)
                a.lse[qrow0 + my_q] = empty ? -INFINITY : m_ref[qb] * a.scale + logf(l_tot);
        }
    };

    // ---- the items of this workgroup ----------------------------------------------
    int kmiss = RING, vmiss = RING - 1;  // first tiles of the current item not yet copied
    // the walk's next item from round r on (a packed batch skips items past
    // its sequences' ends)
    auto next_item = [&](int &r, Item &it) __attribute__((always_inline)) {
        int id_ = item_id(r);
        if (id_ < n_live)
            it = describe(id_);
        if constexpr (VARLEN) {
            while (id_ < n_live && !it.live) {
                id_ = item_id(++r);
                if (id_ < n_live)
                    it = describe(id_);
            }
        }
        return id_;
    };
    int r = 0;
    Item nx{};
    int id = next_item(r, nx);
    if constexpr (QPREF)
        load_q(nx.qrow0, nx.q_wg + wave * 32 * QB, nx.sq);
    int sq_n = 0;
    while (id < n_live) {
        const Item cur = nx;
        int r_n = r + 1;
        const int id_n = next_item(r_n, nx);
        has_next = id_n < n_live;
        kv_end_n = 0;
        if (has_next) {
            sq_n = nx.sq;
            qrow0_n = nx.qrow0;
            kv_end_n = nx.kv_end;
            q_wg_n = nx.q_wg;
            kn = a.k + nx.krow0 * D;
            vn = a.v + nx.krow0 * D;
        }
        if constexpr (VARLEN) {
            Sq = cur.sq;
            Sk = cur.sk;
            diag = Sk - Sq;
            if constexpr (WIN)
                wlo = diag - a.window;
        }
        qrow0 = cur.qrow0;
        krow0 = cur.krow0;
        kv_end = cur.kv_end;
        nblk = cur.nblk;
        kofs = WIN ? cur.kofs : 0;
        slope = cur.slope;
        q0 = cur.q_wg + wave * 32 * QB;  // first row of this wave
        const bool wave_live = q0 < Sq;
        int wave_end = wave_live ? Sk : 0;
        if (CAUSAL && wave_live)
            wave_end = min(Sk, max(0, min(q0 + 32 * QB - 1, Sq - 1) + diag + 1));
        nwb = (max(0, wave_end - kofs) + BN - 1) / BN;  // tiles this wave computes
        // the copy stream of step 0: K tile RING and V tile RING-1, of this item or
        // (when it is shorter) of the next
        if (nblk > RING) {
            kp = a.k + (krow0 + RING * BN) * D;
            krem = kv_end - RING * BN;
        } else {
            kp = kn + (RING - nblk) * BN * D;
            krem = kv_end_n - (RING - nblk) * BN;
        }
        if (nblk > RING - 1) {
            vp = a.v + (krow0 + (RING - 1) * BN) * D;
            vrem = kv_end - (RING - 1) * BN;
        } else {
            vp = vn + (RING - 1 - nblk) * BN * D;
            vrem = kv_end_n - (RING - 1 - nblk) * BN;
        }

        reset_state();
        prologue(kmiss, vmiss);

        // Leading steps of this wave that need no mask (an even number): tile
        // j+1 fully visible to every row of the wave and within its range.
        int n_fast, n_lead = 0;
        {
            int first_masked = (Sk - kofs) / BN;  // ragged key tail
            if (CAUSAL)
                first_masked = min(first_masked, max(0, q0 + diag + 1 - kofs) / BN);
            n_fast = min(nwb, first_masked) - 1;
            n_fast = max(0, n_fast) & ~1;
            n_fast = __builtin_amdgcn_readfirstlane(n_fast);
            if constexpr (WIN) {
                // leading steps whose tile j+1 starts below the window of the
                // wave's last row (an even number, at most n_fast)
                const int qmax = min(q0 + 32 * QB - 1, Sq - 1);
                const int first_full = (max(0, qmax + wlo - kofs) + BN - 1) / BN;
                n_lead = min(n_fast, (max(0, first_full - 1) + 1) & ~1);
                n_lead = __builtin_amdgcn_readfirstlane(n_lead);
            }
        }
        int j = 0;
        for (; j < n_lead; j += 2) {  // sliding window: masked leading steps
            mstep(j, sA, sB, pA, pB);
            mstep(j + 1, sB, sA, pB, pA);
        }
        if constexpr (D == 256) {  // four steps per iteration (measured faster at 256, not at 128)
            for (; j + 3 < n_fast; j += 4) {
                step(IntC<0>{}, j, sA, sB, pA, pB);
                step(IntC<0>{}, j + 1, sB, sA, pB, pA);
                step(IntC<0>{}, j + 2, sA, sB, pA, pB);
                step(IntC<0>{}, j + 3, sB, sA, pB, pA);
            }
        }
        for (; j < n_fast; j += 2) {
            step(IntC<0>{}, j, sA, sB, pA, pB);
            step(IntC<0>{}, j + 1, sB, sA, pB, pA);
        }
        for (; j + 1 < nblk; j += 2) {
            mstep(j, sA, sB, pA, pB);
            mstep(j + 1, sB, sA, pB, pA);
        }
        if (j < nblk)
            mstep(j, sA, sB, pA, pB);
        // the last QK has used Q: the next item's rows load during the epilogue
        if (QPREF && has_next)
            load_q(qrow0_n, q_wg_n + wave * 32 * QB, sq_n);
        epilogue();

        kmiss = max(0, RING - nblk);
        vmiss = max(0, RING - 1 - nblk);
        ph = (ph + nblk) & (RING - 1);
        id = id_n;
        r = r_n;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // no copy may still target LDS
}

// One workgroup per resident slot (a multiple of 8, so that each XCD holds the
// same number), each walking its share of the n_items work items.
template <bool CAUSAL, int D, int NWV, int WPE, bool WIN, int MOD, bool VARLEN = false>
hipError_t launch_q64_t(const FwdArgs &a, int n_qtiles, int n_items, hipStream_t stream)
{
    constexpr auto kernel = fwd_q64_kernel<CAUSAL, NWV, D, WPE, WIN, MOD, VARLEN>;
    const int resident = resident_workgroups<kernel>(64 * NWV);
    if (resident < 8)
        return hipErrorInvalidConfiguration;
    const long long want = ((long long)n_items + 7) / 8 * 8;
    const int grid = (int)std::min<long long>(want, resident / 8 * 8);
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(64 * NWV), 0, stream, a, n_qtiles, n_items);
    return hipGetLastError();
}

template <int D, int NWV, int WPE, int MOD, bool VARLEN>
hipError_t dispatch_win(const FwdArgs &a, bool causal, int n_qtiles, int n, hipStream_t stream)
{
    if (a.window >= 0)
        return causal ? launch_q64_t<true, D, NWV, WPE, true, MOD, VARLEN>(a, n_qtiles, n, stream)
                      : launch_q64_t<false, D, NWV, WPE, true, MOD, VARLEN>(a, n_qtiles, n, stream);
    return causal ? launch_q64_t<true, D, NWV, WPE, false, MOD, VARLEN>(a, n_qtiles, n, stream)
                  : launch_q64_t<false, D, NWV, WPE, false, MOD, VARLEN>(a, n_qtiles, n, stream);
}

template <int D, int NWV, int WPE, bool VARLEN>
hipError_t dispatch_mod(const FwdArgs &a, bool causal, int n_qtiles, int n, hipStream_t stream)
{
    if (a.softcap > 0.f && a.alibi != nullptr)
        return dispatch_win<D, NWV, WPE, kModBoth, VARLEN>(a, causal, n_qtiles, n, stream);
    if (a.softcap > 0.f)
        return dispatch_win<D, NWV, WPE, kModSoftcap, VARLEN>(a, causal, n_qtiles, n, stream);
    if (a.alibi != nullptr)
        return dispatch_win<D, NWV, WPE, kModAlibi, VARLEN>(a, causal, n_qtiles, n, stream);
    return dispatch_win<D, NWV, WPE, kModNone, VARLEN>(a, causal, n_qtiles, n, stream);
}

// NWV waves of 32 query rows per workgroup, WPE waves per SIMD
template <int D, int NWV, int WPE>
hipError_t launch_q64(const FwdArgs &a, bool causal, hipStream_t stream)
{
    constexpr int BM = NWV * 32;
    const int n_qtiles = (a.Sq + BM - 1) / BM;
    const long long n_items = (long long)a.B * a.Hq * n_qtiles;
    // item ids, and 8 GX per round past the last one, stay within int
    if (n_items > 0x7fff0000LL)
        return hipErrorInvalidConfiguration;
    if (n_items == 0)
        return hipSuccess;
    const int n = (int)n_items;
    if (a.cu_q != nullptr)  // packed variable-length batch
        return dispatch_mod<D, NWV, WPE, true>(a, causal, n_qtiles, n, stream);
    return dispatch_mod<D, NWV, WPE, false>(a, causal, n_qtiles, n, stream);
}

}  // namespace
}  // namespace miattn
