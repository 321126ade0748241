// backward.hip -- attention backward on gfx950: gradients dQ, dK, dV of the
// prefill forward from the saved log-sum-exp (the flash backward; the tang
// paper derives it as a comprehension, §3 "Gradients are comprehensions"):
//
//   P_ij  = exp(scale q_i.k_j - LSE_i)   (0 where the forward masks)
//   D_i   = dO_i . O_i
//   dS_ij = P_ij (dO_i.v_j - D_i)
//   dV_j  = sum_i P_ij dO_i      dK_j = scale sum_i dS_ij q_i
//   dQ_i  = scale sum_j dS_ij k_j
//
// Two kernels, no atomics. First a workgroup per block of query rows
// accumulates dQ over the key tiles; its waves, which hold their rows' dO
// anyway, also compute each row's D_i and write it (with LSE_i log2 e) to the
// caller's workspace. Then a workgroup per 128-key block accumulates dK and
// dV over the query heads of its kv-head and their query tiles, reading those
// row statistics. Every product is a v_mfma_f32_32x32x16_bf16 with f32 accumulation.
// As in the forward, a score accumulator holds, in lane l, one column (l % 32)
// and the 16 rows 8(r/4) + 4(l/32) + r%4 of its registers r; its registers
// packed to bf16 are then directly the A operand of the next product over
// those rows, with the other operand read in the same permuted row order.
// The streamed operand tiles go through LDS, copied once per workgroup; the
// ones that need a transpose (Q and dO for dK/dV, K for dQ) are also stored in
// the forward's V layout and read by transposing reads. A wave's fixed rows
// are read from global memory by buffer loads, so rows past the ends read as
// zeros.

#include <hip/hip_runtime.h>
#include <float.h>
#include <math.h>
#include <stdint.h>

#include "launch.h"
#include "lds_copy.h"
#include "resident.h"
#include "tile_order.h"

namespace miattn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

union Frag8 {
    bf16x8 v;
    uint4 u;
    uint32_t w[4];
    uint16_t h[8];
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
    bf16x2 p;
    p[0] = (__bf16)lo;
    p[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ uint16_t to_bf16(float x) { return (uint16_t)(pack_bf16x2(x, 0.f) & 0xffffu); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// 16 bytes of row `row`, dims 16 kk + 8 g .. +7 (a fragment of the 32 x 16
// A operand, or of the 16 x 32 B operand read by rows)
template <int D>
__device__ __forceinline__ bf16x8 frag(__amdgpu_buffer_rsrc_t r, int row, int kk, int g)
{
    Frag8 f;
    f.u = buf_load16(r, (uint32_t)(row * D + 16 * kk + 8 * g) * 2);
    return f.v;
}

// registers 8c .. 8c+7 of an accumulator as the bf16 A operand over rows
// 16c + 4g + 0..3 and 16c + 8 + 4g + 0..3
__device__ __forceinline__ bf16x8 pack_chunk(const f32x16 &x, int c)
{
    Frag8 f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        f.w[i] = pack_bf16x2(x[8 * c + 2 * i], x[8 * c + 2 * i + 1]);
    return f.v;
}

// ---- workgroups of waves sharing a copy ring -------------------------------------
// The operand tiles that every wave of a workgroup reads go global -> LDS by
// buffer DMA (inline assembly, explicit waits) into a ring of RING stages, one
// barrier per step: stage t is copied RING - 1 steps ahead, into the slot that
// stage t - 1 used, which every wave has left once it passes step t's barrier.
// Past the walk's end the copies cover no bytes (descriptors of length 0), so
// every step issues the same number of copies and the waits stay fixed.
// A tile read both ways is stored twice:
//   fragment-major, block kk (1 KB): lane L's 16 bytes of row L%32, dims
//     16kk + 8(L/32) .. +7 -- the operand of a product over the head dimension;
//   transposing, the forward's V layout -- the operand of a product over the
//     tile's rows: 512-byte blocks b = (2 db + c) 2 + hh, and in block b at
//     byte 8L, for L = 16 G + 4 jj + q, the four values of row
//     16c + 8hh + 4(G/2) + jj at dims 32 db + 16 (G%2) + 4q .. +3 (64 bytes
//     per dimension).
// Copy instruction i of a tile moves 1 KB, 16 bytes per lane from the offsets
// below (rows past the descriptor's end read as zero).
__device__ __forceinline__ uint32_t off_frag(int D, int i, int l32, int g)
{
    return (uint32_t)(l32 * D + 16 * i + 8 * g) * 2;
}
__device__ __forceinline__ uint32_t off_tr(int D, int i, int l32, int g)
{
    const int db = i >> 1, kc = i & 1;
    const int G4 = l32 >> 3, jj = (l32 >> 1) & 3, qh = l32 & 1;
    const int row = 16 * kc + 8 * g + 4 * (G4 >> 1) + jj;
    const int dim = 32 * db + 16 * (G4 & 1) + 8 * qh;
    return (uint32_t)(row * D + dim) * 2;
}

typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;

// 16 bytes at LDS byte address addr
__device__ __forceinline__ u32x4 lds16(uint32_t addr) { return *(lds_u32x4 *)(uintptr_t)addr; }

// B operand over the permuted rows of pack_chunk, from a transposing tile: a
// transposing 8-byte read of each block gives lane l dim 32 db + l%32 at rows
// 16c + 8hh + 4(l/32) .. +3. addr = the tile's first LDS byte + 8 lane.
__device__ __forceinline__ bf16x8 lds_tr(uint32_t addr, int db, int c)
{
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const uint32_t p = addr + ((2 * db + c) * 2) * 512;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(uintptr_t)p);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(uintptr_t)(p + 512));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Row-major tiles (head dimension 256): a 32-row tile as its rows of
// 2D bytes, the 16-byte chunk c of row r at chunk c ^ rm_swz(r) of the row.
// One copy of the tile serves both reads, and a copy instruction reads whole
// rows (1 KB = 1024 / 2D rows): 16 L1 accesses per KB where a fragment-shaped
// copy takes 64, and 2.3 times the copy rate (measured). The key keeps both
// reads free of bank conflicts under the way LDS serves them (measured with a
// probe kernel and the bank-conflict counter): a 16-byte read goes in four
// passes of 16 lanes (lanes l % 16 < 8 of one 16-lane row with lanes
// l % 16 >= 8 of another, the two rows' indices differing in bit 0), a
// transposing 8-byte read in two passes of 32 lanes. Every pass of every read
// below (checked at head dimensions 128 and 256) then reaches 16 different
// 16-byte bank groups (a transposing read: four rows 4m + jj, whose keys differ in bits
// 2-3, times four consecutive chunks).
__device__ __forceinline__ int rm_swz(int r) { return 4 * (r & 3) | ((r >> 2) & 1) | 2 * ((r >> 4) & 1); }

// copy instruction i of a row-major tile: the offset of lane l's 16 bytes in
// the tile's rows in global memory (row 1024 i / 2D + l / (D/8)); the copy puts
// them at byte 1024 i + 16 l of the LDS tile, slot l % (D/8) of that row
__device__ __forceinline__ uint32_t off_rm(int D, int i, int lane)
{
    const int cpr = D / 8, row = (64 / cpr) * i + lane / cpr, c = lane % cpr;
    return (uint32_t)(row * 2 * D + 16 * (c ^ rm_swz(row)));
}

// a lane's fragment-read offsets in a row-major tile: row l % 32, chunk
// 2 k8 + l / 32 (k8 < 8; 16-dim step kk = k8 + 8 h adds 256 h bytes)
__device__ __forceinline__ uint32_t rm_frag_off(int D, int k8, int lane)
{
    const int r = lane & 31, g = lane >> 5;
    return (uint32_t)(r * 2 * D + 16 * ((2 * k8 + g) ^ rm_swz(r)));
}

// a lane's transposing-read offsets in a row-major tile, for 16-row chunk ch and
// 32-dim block db % 4 (db / 4 adds 256 bytes): lane L = 16 G + 4 jj + q reads
// dims 32 db + 16 (G % 2) + 4 q .. +3 of row 16 ch + 4 (G / 2) + jj, which is
// chunk 4 db + 2 (G % 2) + q / 2 of the row; the rows + 8 (hh = 1) are 16 D
// bytes further
__device__ __forceinline__ uint32_t rm_tr_off(int D, int ch, int db4, int lane)
{
    const int G = lane >> 4, jj = (lane >> 2) & 3, q = lane & 3;
    const int R = 16 * ch + 4 * (G >> 1) + jj;
    return (uint32_t)(R * 2 * D + 64 * (db4 ^ jj) + 16 * ((2 * (G & 1) + (q >> 1)) ^ ((G >> 1) + 2 * ch)) +
                      8 * (q & 1));
}

// the B operand of lds_tr from a row-major tile; p = tile + the lane's offset
__device__ __forceinline__ bf16x8 lds_tr_rm(uint32_t p, int D)
{
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(uintptr_t)p);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(uintptr_t)(p + 16 * D));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Both-ways tiles (head dimension 128): one copy of a 32-row tile serves the
// fragment reads and the transposing reads. Block i (FT_PB bytes apart) holds
// the rows i, i + 8, i + 16, i + 24 whole (256 bytes each), the 16-byte chunk c
// of row r at chunk c ^ ft_swz(r) of its row. A copy instruction reads four
// whole rows (8 cache lines per KB, against 32 for a fragment-shaped copy),
// and under the way LDS serves reads (as above) every pass of both kinds of
// read reaches all banks once, with each read's step (16-dim step kk, 16-row
// chunk, 32-dim block) in the instruction's offset field.
constexpr int FT_PB = 1088;
__device__ __forceinline__ int ft_swz(int r) { return 2 * ((r & 7) >> 2) + ((r >> 3) & 1); }

// copy instruction i of a both-ways tile: lane l's 16 bytes in global memory
// (row i + 8 (l / 16), the chunk stored at slot l % 16)
__device__ __forceinline__ uint32_t off_ft(int i, int lane)
{
    const int r = i + 8 * (lane >> 4), p = lane & 15;
    return (uint32_t)(r * 256 + 16 * (p ^ ft_swz(r)));
}

// a lane's fragment-read offset in a both-ways tile for even (odd = 0) or odd
// 16-dim steps kk; the read of step kk is at this offset + 32 kk (row l % 32,
// chunk 2 kk + l / 32)
__device__ __forceinline__ uint32_t ft_frag_off(int lane, int odd)
{
    const int r = lane & 31, g = lane >> 5, sw = ft_swz(r);
    const int flip = 32 * (sw >> 1);  // chunk bit 1 swapped: kk ^ 1
    return (uint32_t)((r & 7) * FT_PB + 256 * (r >> 3) + 16 * (g ^ (sw & 1)) + (odd ? -flip : flip));
}

// a lane's transposing-read offset in a both-ways tile for row half hh: lane
// L = 16 m + 4 e + c supplies row 16 ch + 8 hh + 4 (m / 2) + e at dims
// 32 db + 16 (m % 2) + 4 c .. +3, at this offset + 512 ch + 64 db
__device__ __forceinline__ uint32_t ft_tr_off(int lane, int hh)
{
    const int m = lane >> 4, e = (lane >> 2) & 3, c = lane & 3, a2 = m >> 1;
    const int r = 8 * hh + 4 * a2 + e;  // the row's place in its 16-row chunk
    return (uint32_t)((r & 7) * FT_PB + 256 * hh + 16 * ((2 * (m & 1) + (c >> 1)) ^ ft_swz(r)) +
                      8 * (c & 1));
}

// a tile's LDS byte address plus a lane's offset, opaque to the compiler:
// the reads from it then carry their constant steps in the instruction's
// offset field (otherwise the compiler keeps offset + step per read in a
// register, hoisted out of the loop, and adds the tile address before every
// read)
__device__ __forceinline__ uint32_t lane_addr(uint32_t tile, uint32_t off)
{
    uint32_t a = tile + off;
    asm volatile("" : "+v"(a));
    return a;
}

// the B operand of lds_tr from a both-ways tile: p0, p1 = the tile's address
// plus the lane's offsets of ft_tr_off (lane_addr)
__device__ __forceinline__ bf16x8 lds_tr_ft(uint32_t p0, uint32_t p1, int db, int ch)
{
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const uint32_t step = 512 * ch + 64 * db;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(uintptr_t)(p0 + step));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(uintptr_t)(p1 + step));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Workgroup barrier that no memory access of the source crosses: the copies
// into LDS are invisible to the compiler, so it must not move an LDS read
// above the barrier that publishes the copied data.
__device__ __forceinline__ void ring_barrier()
{
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Wait for the fragments a wave loaded for itself and pin them there: the
// compiler counts only its own loads, and with a use inside the loop it would
// put the wait there, where it also drains every copy in flight.
// AGPR: pin them in AGPRs instead (the MFMAs read their A/B operands there),
// leaving the VGPRs to the softmax work.
template <bool AGPR = false, int N>
__device__ __forceinline__ void settle(bf16x8 (&f)[N])
{
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
#pragma unroll
    for (int i = 0; i < N; ++i) {
        u32x4 w = __builtin_bit_cast(u32x4, f[i]);
        if constexpr (AGPR)
            asm volatile("" : "+a"(w));
        else
            asm volatile("" : "+v"(w));
        f[i] = __builtin_bit_cast(bf16x8, w);
    }
}

// ---- dK, dV: one workgroup of four waves per (b, kv-head, 128-key block) -------------
// Wave w holds keys j0 + 32w + l32 (K and V rows: the B operands of S = Q K^T
// and dP = dO V^T, in registers). The workgroup walks the query tiles that see
// any of its keys, over the kv-head's query heads, as one sequence of steps;
// per step the ring holds the tile's Q and dO in the layouts its products read
// and, per wave, its rows' (D_i, LSE_i log2 e) pairs from the workspace. S and
// dP put the key in the lane and 16 query rows in the registers; P and dS
// packed by registers are the A operands of dV += P^T dO and dK += dS^T Q over
// those rows, with dO and Q read transposed.
// PART 0 makes both gradients. At head dimension 256 the dK and dV
// accumulators of all dimensions do not fit a wave's registers beside its K and
// V rows, so two launches share the work: PART 1 makes dV (S and P only: no V
// rows, no dP, Q fragment-major and dO transposing), PART 2 makes dK (S, dP and
// dS: Q both ways and dO fragment-major).
template <int D, bool CAUSAL, int PART>
__global__ void __launch_bounds__(256) bwd_dkdv_ring_kernel(BwdArgs a, int nkb, int gx)
{
    constexpr bool DODV = PART != 2, DODK = PART != 1;  // DODK: dP, dS and V rows too
    // row-major tiles at 256; at 64 and 128 fragment-major and transposing
    // copies (at 128 the row-major reads' per-lane addresses cost more issue
    // time than the cheaper copies save: 1.226 against 1.177 ms)
    constexpr bool RM = D == 256;
    constexpr bool FT = D == 128;  // both-ways tiles
    constexpr bool ONE = RM || FT;  // one copy of Q and of dO serves both reads
    constexpr int KK = D / 16, DB = D / 32, NW = 4;
    constexpr int CPF = KK / NW, CPT = KK / NW;  // copies per tile and wave
    constexpr int TILE_F = FT ? 8 * FT_PB : D * 64;  // one 32-row tile
    constexpr int TILE_T = D * 64;
    constexpr uint32_t BLK = FT ? FT_PB : 1024;  // distance of a tile's copy blocks
    // stage: Q, dO (row-major or both-ways), or Q frag, [Q tr], [dO frag], [dO tr]
    constexpr int OFF_QT = ONE ? 0 : TILE_F;
    constexpr int OFF_OF = ONE ? TILE_F : OFF_QT + (DODK ? TILE_T : 0);
    constexpr int OFF_OT = ONE ? TILE_F : OFF_OF + (DODK ? TILE_F : 0);
    constexpr int STAGE_B = ONE ? 2 * TILE_F : OFF_OT + (DODV ? TILE_T : 0);
    constexpr int RING = STAGE_B > 32768 ? 3 : 4;
    constexpr int NCOPY = (ONE ? 2 * CPF : CPF + (DODK ? CPT + CPF : 0) + (DODV ? CPT : 0)) + 1;  // per stage and wave
    __shared__ __attribute__((aligned(1024))) uint4 sRing[RING * STAGE_B / 16];
    __shared__ __attribute__((aligned(16))) float sStat[RING * NW * 64];

    const int lane = threadIdx.x & 63, l32 = lane & 31, g = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const TileOrder to = tile_order_grouped(blockIdx.x, a.B * a.Hkv, 1, nkb, false, gx);
    const int kvh = to.unit % a.Hkv, b = to.unit / a.Hkv;
    const int Sq = a.Sq, Sk = a.Sk, diag = Sk - Sq, G = a.Hq / a.Hkv;
    const int j0 = 128 * to.qtile, jw0 = j0 + 32 * wave, my_key = jw0 + l32;
    const int64_t krow0 = ((int64_t)b * a.Hkv + kvh) * Sk;
    const float c = a.scale * kLog2e;

    // this wave's keys, loaded before the first copy is issued
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + krow0 * D, (uint32_t)Sk * D * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + krow0 * D, (uint32_t)Sk * D * 2);
    bf16x8 kf[KK], vf[DODK ? KK : 1];  // key my_key, dims 16kk + 8g
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        kf[kk] = frag<D>(rk, my_key, kk, g);
        if constexpr (DODK)
            vf[kk] = frag<D>(rv, my_key, kk, g);
    }
    settle<true>(kf);
    if constexpr (DODK)
        settle<true>(vf);
    f32x16 dk[DODK ? DB : 1], dv[DODV ? DB : 1];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if constexpr (DODK)
                dk[db][r] = 0.f;
            if constexpr (DODV)
                dv[db][r] = 0.f;
        }

    // query tiles that see any key of the block: rows i >= j0 - diag
    const int i_first = CAUSAL ? max(0, j0 - diag) : 0;
    const int qt0 = i_first / 32, nqt = (Sq + 31) / 32;
    const int per_head = max(0, nqt - qt0), n_steps = G * per_head;

    uint32_t foff[CPF], toff[CPT];
#pragma unroll
    for (int h = 0; h < CPF; ++h)
        foff[h] = RM ? off_rm(D, CPF * wave + h, lane)
                     : FT ? off_ft(CPF * wave + h, lane) : off_frag(D, CPF * wave + h, l32, g);
#pragma unroll
    for (int h = 0; h < CPT; ++h)
        toff[h] = ONE ? 0u : off_tr(D, CPT * wave + h, l32, g);
    // row-major read offsets: fragments by 16-dim step % 8, transposing reads by
    // (16-row chunk, 32-dim block % 4)
    uint32_t fro[8], tro[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        fro[i] = RM ? rm_frag_off(D, i, lane) : 0u;
        tro[i] = RM ? rm_tr_off(D, i >> 2, i & 3, lane) : 0u;
    }
    // both-ways read offsets: fragments by kk % 2, transposing reads by row half
    const uint32_t fto[2] = {FT ? ft_frag_off(lane, 0) : 0u, FT ? ft_frag_off(lane, 1) : 0u};
    const uint32_t tto[2] = {FT ? ft_tr_off(lane, 0) : 0u, FT ? ft_tr_off(lane, 1) : 0u};
    const uint32_t ring0 = lds_addr(sRing), stat0 = lds_addr(sStat);
    // stage t's copies; past the walk's end they cover no bytes (the index
    // math is clamped and the lengths selected, so that no branch splits the
    // step)
    // A stage's copies in four parts, issued at four points of a step (its
    // start, before the next S/dP products, before the dV/dK products, between
    // their two 16-row chunks) rather than at once, where every wave's copies
    // would queue together in the CU's address unit. The descriptors of stage
    // t come first.
    u32x4 cq, cd, cw;
    uint32_t cslot = 0;
    auto prep = [&](int t) __attribute__((always_inline)) {
        const int tc = min(t, max(n_steps - 1, 0));
        const int hq = kvh * G + (per_head > 0 ? tc / per_head : 0);
        const int i0 = 32 * (qt0 + (per_head > 0 ? tc % per_head : 0));
        const int64_t r0 = ((int64_t)b * a.Hq + hq) * Sq + min(i0, Sq);
        const bool live = t < n_steps;
        const uint32_t nq = live ? (uint32_t)(Sq - i0) * (D * 2) : 0u;
        const uint32_t nw = live ? (uint32_t)(Sq - i0) * 8 : 0u;
        cq = make_desc(a.q + r0 * D, nq);
        cd = make_desc(a.dout + r0 * D, nq);
        cw = make_desc(a.dsum + 2 * r0, nw);
        cslot = (uint32_t)(t % RING);
    };
    // part p of NP of the prepared stage's copies (copy e goes in part e NP / NCOPY)
    auto issue = [&](int p, int np) __attribute__((always_inline)) {
        const uint32_t base = ring0 + cslot * STAGE_B;
        const uint32_t fb = base + BLK * CPF * wave, tb = base + 1024 * CPT * wave;
        int e = 0;
        auto one = [&](auto &&f) __attribute__((always_inline)) {
            if (e * np / NCOPY == p)
                f();
            ++e;
        };
#pragma unroll
        for (int h = 0; h < CPF; ++h) {
            one([&] { copy_to_lds(cq, foff[h], fb + BLK * h); });
            if constexpr (DODK || ONE)
                one([&] { copy_to_lds(cd, foff[h], fb + OFF_OF + BLK * h); });
        }
        if constexpr (!ONE) {
#pragma unroll
            for (int h = 0; h < CPT; ++h) {
                if constexpr (DODK)
                    one([&] { copy_to_lds(cq, toff[h], tb + OFF_QT + 1024 * h); });
                if constexpr (DODV)
                    one([&] { copy_to_lds(cd, toff[h], tb + OFF_OT + 1024 * h); });
            }
        }
        one([&] { copy_to_lds_b32(cw, 4 * lane, stat0 + (cslot * NW + wave) * 256); });
    };
    // S (and dP) of stage t (16 query rows per lane, key my_key)
    auto qk = [&](int t, f32x16 &s, f32x16 &dp) __attribute__((always_inline)) {
        const uint32_t sb = ring0 + (uint32_t)(t % RING) * STAGE_B + (ONE ? 0 : 16 * lane);
        const uint32_t fa0 = FT ? lane_addr(sb, fto[0]) : 0u, fa1 = FT ? lane_addr(sb, fto[1]) : 0u;
        uint32_t fra[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            fra[i] = RM ? lane_addr(sb, fro[i]) : 0u;
        // fragment kk of the tile at byte o
        auto fr = [&](uint32_t o, int kk) __attribute__((always_inline)) {
            return __builtin_bit_cast(bf16x8, RM ? lds16(fra[kk & 7] + o + 256 * (kk >> 3))
                                              : FT ? lds16((kk & 1 ? fa1 : fa0) + o + 32 * kk)
                                                   : lds16(sb + o + 1024 * kk));
        };
#pragma unroll
        for (int r = 0; r < 16; ++r)
            s[r] = dp[r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr(0, kk), kf[kk], s, 0, 0, 0);
            if constexpr (DODK)
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr(OFF_OF, kk), vf[kk], dp, 0, 0, 0);
        }
    };
    // One step: the softmax (gradient) of step t (its S and dP in registers)
    // alongside S and dP of step t+1, then dV and dK of step t. full: no
    // (row, key) pair of the step is hidden (not diagonal, not a ragged end).
    auto step = [&](int t, bool full, f32x16 &s, f32x16 &dp) __attribute__((always_inline)) {
        const int i0 = 32 * (qt0 + t % per_head);
        // lane: key my_key; register r: row i0 + 8(r/4) + 4g + r%4. Hidden
        // pairs get the score -inf, so that their probability is exactly 0.
        if (!full) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = i0 + 8 * (r >> 2) + 4 * g + (r & 3);
                const bool vis = my_key < Sk && i < Sq && (!CAUSAL || my_key <= i + diag);
                s[r] = vis ? s[r] : -INFINITY;
            }
        }
        // row r's (D, L) pair sits at byte 8 (8(r/4) + 4g + r%4) of the wave's
        // statistics
        const uint32_t st = stat0 + ((uint32_t)(t % RING) * NW + wave) * 256 + 32 * g;
        f32x16 p, ds;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const u32x4 w0 = lds16(st + 64 * r4), w1 = lds16(st + 64 * r4 + 16);
            const float Dr[4] = {__uint_as_float(w0.x), __uint_as_float(w0.z),
                                 __uint_as_float(w1.x), __uint_as_float(w1.z)};
            const float Lr[4] = {__uint_as_float(w0.y), __uint_as_float(w0.w),
                                 __uint_as_float(w1.y), __uint_as_float(w1.w)};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = 4 * r4 + u;
                p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -Lr[u]));
                if constexpr (DODK)
                    ds[r] = p[r] * (dp[r] - Dr[u]);
            }
        }
        bf16x8 pa0, pa1, sa0, sa1;
        if constexpr (DODV) {
            pa0 = pack_chunk(p, 0);
            pa1 = pack_chunk(p, 1);
        }
        if constexpr (DODK) {
            sa0 = pack_chunk(ds, 0);
            sa1 = pack_chunk(ds, 1);
        }
        issue(1, 4);
        qk(t + 1, s, dp);
        const uint32_t sb = ring0 + (uint32_t)(t % RING) * STAGE_B + (ONE ? 0 : 8 * lane);
        const uint32_t ta0 = FT ? lane_addr(sb, tto[0]) : 0u, ta1 = FT ? lane_addr(sb, tto[1]) : 0u;
        uint32_t tra[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            tra[i] = RM ? lane_addr(sb, tro[i]) : 0u;
        // block (ch, db) of the transposing operand in the tile at byte o
        auto tr = [&](uint32_t o, int db, int ch) __attribute__((always_inline)) {
            return RM   ? lds_tr_rm(tra[4 * ch + (db & 3)] + o + 256 * (db >> 2), D)
                   : FT ? lds_tr_ft(ta0 + o, ta1 + o, db, ch)
                        : lds_tr(sb + o, db, ch);
        };
        issue(2, 4);
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                if constexpr (DODV)
                    dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ch ? pa1 : pa0, tr(OFF_OT, db, ch), dv[db],
                                                                     0, 0, 0);
                if constexpr (DODK)
                    dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ch ? sa1 : sa0, tr(OFF_QT, db, ch), dk[db],
                                                                     0, 0, 0);
            }
            if (ch == 0)
                issue(3, 4);
        }
    };

    // stage t is waited for at the top of step t - 1 (its S and dP are made
    // there), copied at the top of step t + 1 - RING into the slot of stage
    // t - RING
#pragma unroll
    for (int t = 0; t < RING - 1; ++t) {
        prep(t);
        issue(0, 1);
    }
    f32x16 s, dp;
    if (n_steps > 0) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((RING - 2) * NCOPY));
        ring_barrier();
        qk(0, s, dp);
    }
    for (int t = 0; t < n_steps; ++t) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((RING - 3) * NCOPY));  // this wave's copies of stage t+1
        ring_barrier();                                              // and every other wave's
        prep(t + RING - 1);
        issue(0, 4);
        const int i0 = 32 * (qt0 + t % per_head);
        const bool full = (!CAUSAL || i0 + diag >= jw0 + 31) && jw0 + 31 < Sk && i0 + 31 < Sq;
        step(t, full, s, dp);
    }
    // no copy may land in LDS after the workgroup has ended
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    // lane: dim 32 db + l32; register r: key jw0 + 8(r/4) + 4g + r%4
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int j = jw0 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (j < Sk) {
                if constexpr (DODK)
                    a.dk[(krow0 + j) * D + 32 * db + l32] = to_bf16(dk[db][r] * a.scale);
                if constexpr (DODV)
                    a.dv[(krow0 + j) * D + 32 * db + l32] = to_bf16(dv[db][r]);
            }
        }
}

// ---- dQ: one workgroup of NW waves per (b, query head, 32 NW-row block) ------------
// Wave w holds rows ib0 + 32w + l32 (Q and dO rows: the B operands of
// S^T = K Q^T and dP^T = V dO^T, in registers, with the rows' D_i and
// LSE_i log2 e). The workgroup walks the key tiles that any of its rows sees;
// per step the ring holds the tile's K and V fragment-major and K transposing
// (at head dimension 256: K and V row-major).
// S^T and dP^T put the query row in the lane and 16 keys in the registers; dS
// packed by registers is the A operand of dQ += dS K over those keys.
template <int D, bool CAUSAL, int NW>
__global__ void __launch_bounds__(64 * NW) bwd_dq_ring_kernel(BwdArgs a, int nrb, int gx)
{
    constexpr int KK = D / 16, DB = D / 32;
    constexpr bool RM = D == 256;          // row-major tiles (K read both ways)
    constexpr bool FT = D == 128;          // both-ways tiles (K read both ways)
    constexpr int NT = RM || FT ? 2 : 3;   // tiles per stage: K, V or K frag, V frag, K tr
    static_assert((NT * KK) % NW == 0, "copies must split evenly over the waves");
    constexpr int NCOPY = NT * KK / NW;    // copies per stage and wave
    constexpr int TILE_B = FT ? 8 * FT_PB : D * 64;
    constexpr uint32_t BLK = FT ? FT_PB : 1024;  // distance of a tile's copy blocks
    constexpr int STAGE_B = NT * TILE_B;
    constexpr int RING = 4;
    constexpr int NP = RM ? 3 : 1;         // parts a stage's copies are issued in
    __shared__ __attribute__((aligned(1024))) uint4 sRing[RING * STAGE_B / 16];

    const int lane = threadIdx.x & 63, l32 = lane & 31, g = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = a.Hq / a.Hkv;
    const TileOrder to = tile_order_grouped(blockIdx.x, a.B * a.Hkv, G, nrb, CAUSAL, gx);
    const int kvh = to.unit % a.Hkv, b = to.unit / a.Hkv, hq = kvh * G + to.gq;
    const int Sq = a.Sq, Sk = a.Sk, diag = Sk - Sq;
    const int ib0 = 32 * NW * to.qtile, iw0 = ib0 + 32 * wave, my_q = iw0 + l32;
    const int64_t qrow0 = ((int64_t)b * a.Hq + hq) * Sq;
    const int64_t krow0 = ((int64_t)b * a.Hkv + kvh) * Sk;
    const float c = a.scale * kLog2e;

    // this wave's rows, loaded before the first copy is issued
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + qrow0 * D, (uint32_t)Sq * D * 2);
    const __amdgpu_buffer_rsrc_t rdo = make_rsrc(a.dout + qrow0 * D, (uint32_t)Sq * D * 2);
    bf16x8 qf[KK], df[KK];  // row my_q, dims 16kk + 8g
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        qf[kk] = frag<D>(rq, my_q, kk, g);
        df[kk] = frag<D>(rdo, my_q, kk, g);
    }
    const bool in = my_q < Sq;
    // the row's statistics (D_i = dO_i . O_i, LSE_i log2 e), computed here and
    // written to the workspace for the dK/dV launch that follows; each row
    // belongs to exactly one wave of one workgroup
    float Di, L2;
    {
        const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.o + qrow0 * D, (uint32_t)Sq * D * 2);
        float dot = 0.f;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const bf16x8 o = frag<D>(ro, my_q, kk, g);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                dot += (float)df[kk][e] * (float)o[e];
        }
        dot += __shfl_xor(dot, 32, 64);
        // a row that sees no key (LSE = -inf) gets the lowest finite value:
        // every score of such a row is masked to -inf, and exp2 of
        // -inf * c + FLT_MAX is exactly 0
        const float L = in ? a.lse[qrow0 + my_q] * kLog2e : 0.f;
        Di = in ? dot : 0.f;
        L2 = L == -INFINITY ? -FLT_MAX : L;
        if (in)
            a.dsum[2 * (qrow0 + my_q) + g] = g == 0 ? Di : L2;
    }
    // at 256 (one wave per SIMD) the fixed operands go to AGPRs, the VGPRs to
    // the accumulator
    settle<D == 256>(qf);
    settle<D == 256>(df);
    asm volatile("" : "+v"(Di), "+v"(L2));

    f32x16 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            dq[db][r] = 0.f;

    // key tiles that any row of the block sees
    const int i_last = min(ib0 + 32 * NW, Sq) - 1;
    const int kv_end = CAUSAL ? min(Sk, max(0, i_last + diag + 1)) : Sk;
    const int nkt = (kv_end + 31) / 32;

    // copy e = NCOPY w + h of a stage: tile e / KK (K frag, V frag, K tr),
    // instruction e % KK
    uint32_t coff[NCOPY], cdst[NCOPY];
    bool cv[NCOPY];
#pragma unroll
    for (int h = 0; h < NCOPY; ++h) {
        const int e = NCOPY * wave + h, x = e / KK, i = e % KK;
        coff[h] = RM ? off_rm(D, i, lane)
                     : FT ? off_ft(i, lane) : x == 2 ? off_tr(D, i, l32, g) : off_frag(D, i, l32, g);
        cdst[h] = (uint32_t)(x * TILE_B + BLK * i);
        cv[h] = x == 1;
    }
    // row-major read offsets (see the dK/dV kernel)
    uint32_t fro[8], tro[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        fro[i] = RM ? rm_frag_off(D, i, lane) : 0u;
        tro[i] = RM ? rm_tr_off(D, i >> 2, i & 3, lane) : 0u;
    }
    const uint32_t fto[2] = {FT ? ft_frag_off(lane, 0) : 0u, FT ? ft_frag_off(lane, 1) : 0u};
    const uint32_t tto[2] = {FT ? ft_tr_off(lane, 0) : 0u, FT ? ft_tr_off(lane, 1) : 0u};
    const uint32_t ring0 = lds_addr(sRing);
    u32x4 cdk, cdv;
    uint32_t cbase = 0;
    auto prep = [&](int t) __attribute__((always_inline)) {
        const uint16_t *ks = a.k, *vs = a.v;
        uint32_t n = 0;
        if (t < nkt) {
            ks = a.k + (krow0 + 32 * t) * D;
            vs = a.v + (krow0 + 32 * t) * D;
            n = (uint32_t)(kv_end - 32 * t) * (D * 2);
        }
        cdk = make_desc(ks, n);
        cdv = make_desc(vs, n);
        cbase = ring0 + (uint32_t)(t % RING) * STAGE_B;
    };
    // part p of NP of the prepared stage's copies (copy h goes in part h NP / NCOPY)
    auto issue = [&](int p, int np) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < NCOPY; ++h)
            if (h * np / NCOPY == p)
                copy_to_lds(cv[h] ? cdv : cdk, coff[h], cbase + cdst[h]);
    };

#pragma unroll
    for (int t = 0; t < RING - 1; ++t) {
        prep(t);
        issue(0, 1);
    }
    for (int t = 0; t < nkt; ++t) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((RING - 2) * NCOPY));
        ring_barrier();
        // at 256 the stage's copies go in three parts: here, after the S/dP
        // products, before the dQ products (every wave issues all three; at 64
        // and 128 the two waves of a SIMD hide a burst: no gain)
        prep(t + RING - 1);
        issue(0, NP);
        const int j0 = 32 * t;
        const bool any = iw0 < Sq && (!CAUSAL || iw0 + 31 + diag >= j0);
        if (!any) {
            issue(1, NP);
            issue(2, NP);
            continue;
        }
        const bool full = (!CAUSAL || iw0 + diag >= j0 + 31) && j0 + 31 < Sk && iw0 + 31 < Sq;
        const uint32_t sb = ring0 + (uint32_t)(t % RING) * STAGE_B;
        const uint32_t fa0 = FT ? lane_addr(sb, fto[0]) : 0u, fa1 = FT ? lane_addr(sb, fto[1]) : 0u;
        const uint32_t ta0 = FT ? lane_addr(sb, tto[0]) : 0u, ta1 = FT ? lane_addr(sb, tto[1]) : 0u;
        uint32_t fra[8], tra[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            fra[i] = RM ? lane_addr(sb, fro[i]) : 0u;
            tra[i] = RM ? lane_addr(sb, tro[i]) : 0u;
        }
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            s[r] = dp[r] = 0.f;
        // fragment kk of the tile at byte o
        auto fr = [&](uint32_t o, int kk) __attribute__((always_inline)) {
            return __builtin_bit_cast(bf16x8, RM ? lds16(fra[kk & 7] + o + 256 * (kk >> 3))
                                              : FT ? lds16((kk & 1 ? fa1 : fa0) + o + 32 * kk)
                                                   : lds16(sb + o + 1024 * kk + 16 * lane));
        };
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr(0, kk), qf[kk], s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr(TILE_B, kk), df[kk], dp, 0, 0, 0);
        }
        issue(1, NP);
        // lane: row my_q; register r: key j0 + 8(r/4) + 4g + r%4
        f32x16 ds;
        // hidden pairs get the score -inf, so that their probability is 0
        if (!full) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int j = j0 + 8 * (r >> 2) + 4 * g + (r & 3);
                const bool vis = in && j < Sk && (!CAUSAL || j <= my_q + diag);
                s[r] = vis ? s[r] : -INFINITY;
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
            ds[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -L2)) * (dp[r] - Di);
        issue(2, NP);
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
            const bf16x8 sa = pack_chunk(ds, ch);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const bf16x8 kt = RM   ? lds_tr_rm(tra[4 * ch + (db & 3)] + 256 * (db >> 2), D)
                                  : FT ? lds_tr_ft(ta0, ta1, db, ch)
                                       : lds_tr(sb + 2 * TILE_B + 8 * lane, db, ch);
                dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa, kt, dq[db], 0, 0, 0);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    // lane: dim 32 db + l32; register r: row iw0 + 8(r/4) + 4g + r%4
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = iw0 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (i < Sq)
                a.dq[(qrow0 + i) * D + 32 * db + l32] = to_bf16(dq[db][r] * a.scale);
        }
}

template <auto Kernel>
hipError_t launch_dkdv(const BwdArgs &a, long long grid, int nkb, hipStream_t stream)
{
    const int gx = max(1, resident_workgroups<Kernel>(256) / 8);
    hipLaunchKernelGGL(Kernel, dim3((unsigned)grid), dim3(256), 0, stream, a, nkb, gx);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t stream)
{
    // workgroups sharing a copy ring: dK/dV per 128-key block, dQ per block of
    // 32 NWQ rows
    constexpr int NWQ = D == 128 ? 8 : 4;
    const int nkb = (a.Sk + 127) / 128, nrb = (a.Sq + 32 * NWQ - 1) / (32 * NWQ);
    const long long g1 = (long long)a.B * a.Hkv * nkb;
    const long long g2 = (long long)a.B * a.Hq * nrb;
    if (g1 > 0x7fffffffLL || g2 > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;
    // dQ first: its workgroups also write every row's (D_i, LSE_i log2 e),
    // which the dK/dV launch reads
    if (g2 > 0) {
        constexpr auto kernel = bwd_dq_ring_kernel<D, CAUSAL, NWQ>;
        const int gx = max(1, resident_workgroups<kernel>(64 * NWQ) / 8);
        hipLaunchKernelGGL(kernel, dim3((unsigned)g2), dim3(64 * NWQ), 0, stream, a, nrb, gx);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    if (g1 > 0) {
        // dK and dV: one launch, or at 256 one for dK and one for dV
        hipError_t e;
        if constexpr (D == 256) {
            e = launch_dkdv<bwd_dkdv_ring_kernel<D, CAUSAL, 2>>(a, g1, nkb, stream);
            if (e == hipSuccess)
                e = launch_dkdv<bwd_dkdv_ring_kernel<D, CAUSAL, 1>>(a, g1, nkb, stream);
        } else {
            e = launch_dkdv<bwd_dkdv_ring_kernel<D, CAUSAL, 0>>(a, g1, nkb, stream);
        }
        if (e != hipSuccess)
            return e;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs &a, int d, bool causal, hipStream_t stream)
{
    switch (d) {
    case 64:
        return causal ? launch_bwd_t<64, true>(a, stream) : launch_bwd_t<64, false>(a, stream);
    case 128:
        return causal ? launch_bwd_t<128, true>(a, stream) : launch_bwd_t<128, false>(a, stream);
    case 256:
        return causal ? launch_bwd_t<256, true>(a, stream) : launch_bwd_t<256, false>(a, stream);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace miattn
