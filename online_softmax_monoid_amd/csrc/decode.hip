// decode.hip -- split-KV decode attention on gfx950: a bandwidth-bound split
// kernel and a small combine kernel, both the online-softmax monoid.
//
// Split kernel (a7): one workgroup per (stream b, kv-head, chunk of up to 16
// query heads, split s). The split covers keys [floor(s*len/S),
// floor((s+1)*len/S)) of the stream's cache. Every row of K and V is read
// from HBM once and serves all query heads of its kv-head: the heads are the
// columns of the MFMA tiles (the paper's decode kernel likewise shares one
// pass over K and V between the GQA heads, §7.4). The unnormalised partial
// state (m, l, acc[d]) of the split goes to the workspace.
//
// Combine kernel (a8): one wave per (b, query head) folds the S partial states
// with the monoid combine (rescale to the largest max, add) and finishes
// O = acc / l and LSE = m + ln l; a stream with no key gets O = +0, LSE = -inf.
// Splitting is valid because the combine is associative (§2.5 "Schedules":
// split on any associative monoid).
//
// Paged caches (the paper's gather view: a paged KV cache is an ordinary read
// whose source row comes from an index tensor, §2.1 "Views"): key row r of
// stream b and kv-head g is row r % P of page table[b][r / P] of a pool
// [num_pages, Hkv, P, d]. Only the address of each copied row changes; the
// kernels are otherwise the same, so a paged cache gives bit for bit the
// result of the contiguous cache holding the same rows.
//
// Partial maxima are kept in log2 units (scores times scale*log2(e)), so every
// exponential is one v_exp_f32.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "launch.h"

namespace miattn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
    bf16x2 p;
    p[0] = (__bf16)lo;
    p[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, p);
}

// kv length of stream b, clamped to [0, S_cap]
__device__ __forceinline__ int clamped_len(const DecodeArgs &a, int b)
{
    const int len = a.lens[b];
    return len < 0 ? 0 : (len > a.S_cap ? a.S_cap : len);
}

// Workgroups take streams longest first (ties by index), so the short
// streams' splits come last and fill the gaps instead of a long stream's
// splits running alone at the end. Up to 64 streams every wave ranks them
// itself (lane i holds stream i's length); beyond that streams go in index
// order.
// The stream's clamped length comes back in len (read from the lane that
// ranked it, so that no second load of the lengths delays the first copies).
__device__ __forceinline__ int stream_by_rank(const DecodeArgs &a, int rank, int lane, int &len)
{
    if (a.B > 64) {
        len = __builtin_amdgcn_readfirstlane(clamped_len(a, rank));
        return rank;
    }
    const int mine = lane < a.B ? clamped_len(a, lane) : -1;
    int my_rank = 0;
    for (int o = 0; o < a.B; ++o) {
        const int lo = __builtin_amdgcn_readlane(mine, o);
        my_rank += (lo > mine) || (lo == mine && o < lane);
    }
    const unsigned long long hit = __ballot(lane < a.B && my_rank == rank);
    const int b = hit ? (int)__builtin_ctzll(hit) : rank;  // exactly one lane matches
    len = __builtin_amdgcn_readlane(mine, b);
    return b;
}

// ---- split kernel on MFMA ----------------------------------------------------
// One workgroup of NW waves per (stream b, kv-head, chunk of up to 16 query
// heads, split). The split's keys go in blocks of 32, block n to wave n % NW,
// so no wave walks a whole long split alone (the long streams' splits
// would otherwise leave a tail of lone waves). Per block:
//   * K and V rows go global -> LDS by buffer DMA in whole rows (reading
//     the cache in 16-row x 64-byte fragment shapes directly runs at about
//     70% of the contiguous read rate).
//   * K fragments from LDS are the A operands of v_mfma_f32_16x16x32_bf16
//     (lane l holds dims 8(l/16)..+7 of key l%16 of a 32-dim slice), and
//     S^T = K Q^T puts the query heads in the 16 columns, so the dot
//     products need no cross-lane sums; columns past the chunk's heads see
//     zero queries and are never written out.
//   * Transposing 8-byte LDS reads of V give lane l four consecutive keys of
//     dim l%16 (+16 per d-block), the A operand of O^T += V^T P^T.
//   * The probabilities stay in registers as the B operand: lane l's eight
//     keys are 4(l/16)+{0..3} of both 16-key halves, exactly the rows its
//     score accumulators hold, and V^T is read with the same key order.
// K and V of a wave's next block are in flight while a block computes. The
// reference maximum moves lazily (only past a margin of 8 in log2 units), as
// in the prefill kernels. At the end the NW waves' states are folded through
// LDS with the monoid combine and written as the split's partial state.
template <int D, int NW, bool PAGED>
__global__ void __launch_bounds__(64 * NW)
decode_mfma_kernel(DecodeArgs a, int hchunks)
{
    constexpr int KK = D / 32;  // 32-dim slices of a key row
    constexpr int DB = D / 16;  // 16-dim blocks of the output = V DMA instructions per block
    constexpr int BK = 32;      // keys per block
    typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
    typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) void lds_void;
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

    // per wave: one K and one V block (32 keys x D bf16 each); at the end the
    // V block holds the wave's accumulator (16 columns x D f32 -- the same
    // 64 D bytes) and the K block its 16 references and row sums. Nothing
    // else, so that a workgroup takes exactly 32 D bytes per wave of LDS and
    // five two-wave workgroups fit on a CU at head dimension 128.
    __shared__ __attribute__((aligned(16))) uint4 sKall[NW][BK * D / 8];
    __shared__ __attribute__((aligned(16))) uint4 sVall[NW][BK * D / 8];
    auto s_mc = [&](int w_) __attribute__((always_inline)) { return (float *)&sKall[w_][0]; };
    auto s_l = [&](int w_) __attribute__((always_inline)) { return (float *)&sKall[w_][0] + 16; };

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15, r4 = lane >> 4;
    uint4 *const sK = sKall[wave];
    uint4 *const sV = sVall[wave];

    int id = blockIdx.x;
    const int split = id % a.splits;
    id /= a.splits;
    const int hc = id % hchunks;
    id /= hchunks;
    const int kvh = id % a.Hkv;
    const int sr = id / a.Hkv;  // stream rank
    int len;
    const int b = stream_by_rank(a, sr, lane, len);
    const int G = a.Hq / a.Hkv;
    const int h0 = kvh * G + 16 * hc;
    const int GH = min(16, G - 16 * hc);  // query heads of this chunk

    const int k_lo = (int)(((int64_t)split * len) / a.splits);
    const int k_hi = (int)(((int64_t)(split + 1) * len) / a.splits);
    const int nb = (k_hi - k_lo + BK - 1) / BK;

    // Q^T fragments (B operand): column l%16 is query head h0 + l%16
    bf16x8 qf[KK];
    {
        const bool live = l16 < GH;
        const uint16_t *qrow = a.q + ((int64_t)b * a.Hq + h0 + (live ? l16 : 0)) * D + 8 * r4;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const uint4 w = live ? *(const uint4 *)(qrow + 32 * kk) : make_uint4(0, 0, 0, 0);
            qf[kk] = __builtin_bit_cast(bf16x8, w);
        }
    }

    const int64_t row0 = ((int64_t)b * a.Hkv + kvh) * a.S_cap;
    const uint16_t *const kbase = a.k + row0 * D;
    const uint16_t *const vbase = a.v + row0 * D;
    auto block_rsrc = [&](const uint16_t *base, int kb) __attribute__((always_inline)) {
        const int keys = __builtin_amdgcn_readfirstlane(min(k_hi - kb, BK));
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base + (int64_t)kb * D),
                                                 (short)0, keys * (D * 2), 0x00020000);
    };
    // K and V blocks go global -> LDS by buffer DMA, each instruction four
    // (head dim 128) whole key rows, so every read is a contiguous 1 KB. A
    // row's 16-byte chunk c sits at slot c ^ swz(row) of the row, which keeps
    // the fragment reads below free of bank conflicts.
    // Instruction i, lane l: row RPI i + l / CPR, slot (l % CPR) ^ swz(row).
    constexpr int CPR = D / 8;     // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;  // rows per DMA instruction
    constexpr int NI = BK / RPI;   // DMA instructions per block
    // Row key of the swizzle. LDS serves a 16-byte read in four passes of 16
    // lanes: lanes l % 16 < 8 of one lane row with lanes l % 16 >= 8 of
    // another, the two rows differing in bit 0 (measured: the bank-conflict
    // counter of every layout tried matches this grouping), and a
    // transposing 8-byte read in two passes of 32 lanes. From head
    // dimension 128 on, key 2 row (mod chunks per row) makes both reads
    // conflict-free: a V read's 32 lanes (rows 4G + j, G in {0, 1} or {2, 3},
    // two chunks each) reach 16 different slots, and in a K read the
    // lanes of the two lane rows reach slots of opposite parity. At head
    // dimension 64 (two rows per 256 bytes) the row index itself does that.
    auto swz = [](int row) __attribute__((always_inline)) {
        return D == 64 ? row % CPR : (2 * row) % CPR;
    };
    // Every copy carries the non-temporal hint: each K and V row is read
    // once. Measured at the batched decode workload (Sigma len 137,467,
    // 16 splits): 98.6 against 110.4 us for split + combine, 5.7 against
    // 5.1 TB/s; a read-only probe of the same blocks goes from 95.7 to
    // 84.8 us with it. It also keeps the stream from pushing other data out
    // of the caches: without it, a decode right after a prefill paid for
    // the prefill's output still waiting there to be written back (117
    // against 111 us); with it the two take the same time.
    constexpr int kNT = 2;  // cache-policy bits of the copies: nt
    auto dma = [&](uint4 *buf, const uint16_t *base, int kb) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t r = block_rsrc(base, kb);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int row = RPI * i + lane / CPR;
            const int off = (row * CPR + ((lane % CPR) ^ swz(row))) * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(buf + 64 * i), 16, off, 0, 0, kNT);
        }
    };
    // Paged: the element offset in the pool of each lane's 16 bytes of block
    // kb (the same for K and V). Its 32 rows lie in at most three pages (page
    // size >= 16), whose table entries are read once per block (clamped to the
    // table row and to the pool, so that no entry can send a copy outside
    // it). Rows past the split repeat its last row instead of reading zeros:
    // their scores are masked and their probabilities are exactly 0.
    auto table_pages = [&](int kb, int (&pg)[3]) __attribute__((always_inline)) {
        const int lp0 = kb >> a.page_shift;
        const int *trow = a.table + (int64_t)b * a.max_pages;
#pragma unroll
        for (int t = 0; t < 3; ++t)
            pg[t] = trow[min(lp0 + t, a.max_pages - 1)];
    };
    auto paged_offsets = [&](int kb, const int (&pe)[3], int64_t (&off)[NI]) __attribute__((always_inline)) {
        const int sh = a.page_shift;
        const int lp0 = kb >> sh;
        int pg[3];
#pragma unroll
        for (int t = 0; t < 3; ++t)
            pg[t] = min(max(pe[t], 0), a.num_pages - 1);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int rb = RPI * i + lane / CPR;  // row in the block
            const int r = min(kb + rb, k_hi - 1);
            const int t = (r >> sh) - lp0;
            const int p = t == 0 ? pg[0] : (t == 1 ? pg[1] : pg[2]);
            off[i] = ((((int64_t)p * a.Hkv + kvh) << sh) + (r & ((1 << sh) - 1))) * D +
                     8 * ((lane % CPR) ^ swz(rb));
        }
    };
    auto dma_paged = [&](uint4 *buf, const uint16_t *pool, const int64_t (&off)[NI])
                         __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
            __builtin_amdgcn_global_load_lds((const void *)(pool + off[i]), (lds_void *)(buf + 64 * i),
                                             16, 0, kNT);
    };
    // (paged: the block's table entries pe, read beforehand by table_pages)
    auto copy_block = [&](int kb, const int (&pe)[3]) __attribute__((always_inline)) {
        if constexpr (PAGED) {
            int64_t off[NI];
            paged_offsets(kb, pe, off);
            dma_paged(sK, a.k, off);
            dma_paged(sV, a.v, off);
        } else {
            dma(sK, kbase, kb);
            dma(sV, vbase, kb);
        }
    };
    // K A fragments: lane l holds dims 32kk + 8(l/16) .. +7 of key 16 half + l%16
    uint4 kf[2][KK];
    auto read_k = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int row = 16 * half + l16;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                kf[half][kk] = sK[row * CPR + ((4 * kk + r4) ^ swz(row))];
        }
    };
    // V^T A fragments by transposing reads: for d-block db and half hh, lane
    // L = 16 G + 4 j + q supplies the 8 bytes V[16 hh + 4 G + j][16 db + 4 q .. +3];
    // lane l receives dim 16 db + l%16 of keys 16 hh + 4(l/16) + 0..3
    bf16x8 vf[DB];
    auto read_v = [&]() __attribute__((always_inline)) {
        const int j = (lane >> 2) & 3, q = lane & 3;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            i16x4 h2[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int row = 16 * hh + 4 * r4 + j;
                const int chunk = 2 * db + (q >> 1);
                const char *p = (const char *)sV + row * (2 * D) + 16 * (chunk ^ swz(row)) + 8 * (q & 1);
                h2[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(const_cast<char *>(p)));
            }
            vf[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(h2[0], h2[1], 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };

    const float c = a.scale * kLog2e;
    const float thr = 8.f / c;
    float m_ref = -INFINITY, nmc = 0.f, m_thr = -INFINITY, l_lane = 0.f;
    f32x4 acc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i)
        acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    int pe[3] = {0, 0, 0};  // paged: table entries of the wave's next block
    if (wave < nb) {
        if constexpr (PAGED)
            table_pages(k_lo + BK * wave, pe);
        copy_block(k_lo + BK * wave, pe);
    }
    for (int n = wave; n < nb; n += NW) {
        const int kb = k_lo + BK * n;
        // paged: the next block's table entries are read now, so that they
        // land with this block's copies instead of costing a memory round
        // trip of their own before the next copies can be issued
        if (PAGED && n + NW < nb)
            table_pages(kb + BK * NW, pe);
        // this block's copies have landed (nothing newer is in flight); take
        // it into registers, then start the copies of this wave's next block
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        read_k();
        read_v();
        if (n + NW < nb) {
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the block is in registers
            copy_block(kb + BK * NW, pe);
        }
        // S^T for the two 16-key halves: lane l holds keys 16 half + 4(l/16) + i
        // for the query head in column l%16
        f32x4 s[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            s[half] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, kf[half][0]), qf[0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
            for (int kk = 1; kk < KK; ++kk)
                s[half] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, kf[half][kk]), qf[kk], s[half], 0, 0, 0);
        }

        // mask keys past the split, row maximum per query column
        const int rel = k_hi - kb - 4 * r4;  // key 16 half + 4 r4 + i valid iff 16 half + i < rel
        float mx = -INFINITY;
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s[half][i] = (16 * half + i < rel) ? s[half][i] : -INFINITY;
                mx = fmaxf(mx, s[half][i]);
            }
        {
            auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
            auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(r2[0]), __uint_as_float(r2[1]));
        }
        if (__any(mx > m_thr)) {
            const float m_new = fmaxf(m_ref, mx);
            const float alpha = (m_new == m_ref) ? 1.f : __builtin_amdgcn_exp2f((m_ref - m_new) * c);
            l_lane *= alpha;
#pragma unroll
            for (int i = 0; i < DB; ++i)
                acc[i] *= alpha;
            m_ref = m_new;
            nmc = (m_new == -INFINITY) ? 0.f : -(m_new * c);
            m_thr = m_new + thr;
        }
        float p[2][4];
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[half][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[half][i], c, nmc));
                l_lane += p[half][i];
            }
        uint4 pw;
        pw.x = pack_bf16x2(p[0][0], p[0][1]);
        pw.y = pack_bf16x2(p[0][2], p[0][3]);
        pw.z = pack_bf16x2(p[1][0], p[1][1]);
        pw.w = pack_bf16x2(p[1][2], p[1][3]);
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
        for (int i = 0; i < DB; ++i)
            acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[i], pb, acc[i], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // no copy may still target LDS

    // this wave's state -> LDS: reference (log2 units), row sum over the four
    // lane rows of each column, accumulator [column][dim]
    {
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(l_lane), __float_as_uint(l_lane), false, false);
        l_lane = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_lane), __float_as_uint(l_lane), false, false);
        l_lane = __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
    }
    // [16][D], the 16-byte chunk c of column col at chunk c ^ col: the 16
    // lanes of a write (one column each, same chunk) then reach 16 different
    // bank groups instead of one
    float *const s_acc = (float *)sV;
    if (r4 == 0) {
        s_mc(wave)[l16] = (m_ref == -INFINITY) ? -INFINITY : m_ref * c;
        s_l(wave)[l16] = l_lane;
    }
#pragma unroll
    for (int i = 0; i < DB; ++i)
        *(float4 *)(s_acc + l16 * D + 4 * ((4 * i + r4) ^ l16)) =
            make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
    __syncthreads();

    // fold the waves' states (rescale to the largest reference, add) and
    // write the split's partial; thread t covers column t / (D/4), dims
    // 4 (t % (D/4)) .. +3 of it, for the chunk's GH columns
    const int64_t part0 = ((int64_t)b * a.Hq + h0) * a.splits + split;
    for (int e = threadIdx.x; e < GH * (D / 4); e += 64 * NW) {
        const int col = e / (D / 4), d4 = 4 * (e % (D / 4));
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            M = fmaxf(M, s_mc(w)[col]);
        float L = 0.f;
        float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float mw = s_mc(w)[col];
                const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
                L = __builtin_fmaf(f, s_l(w)[col], L);
                const float4 v = *(const float4 *)((const float *)sVall[w] + col * D + 4 * ((d4 / 4) ^ col));
                A.x = __builtin_fmaf(f, v.x, A.x);
                A.y = __builtin_fmaf(f, v.y, A.y);
                A.z = __builtin_fmaf(f, v.z, A.z);
                A.w = __builtin_fmaf(f, v.w, A.w);
            }
        }
        const int64_t p = part0 + (int64_t)col * a.splits;
        *(float4 *)(a.part_acc + p * D + d4) = A;
        if (d4 == 0) {
            a.part_ml[2 * p] = M;
            a.part_ml[2 * p + 1] = L;
        }
    }
}

// One 64-lane wave per (b, query head); lane handles d/64 output dims. The
// splits' partial states are read in one round of loads issued together (one
// split per lane for the references and sums; every lane's dims of up to 16
// splits), and each split's weight is computed once, in its lane, then
// broadcast, so the kernel costs about one memory latency (more only past 16
// or 64 splits).
__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        x = fmaxf(x, __shfl_xor(x, off, 64));
    return x;
}

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        x += __shfl_xor(x, off, 64);
    return x;
}

template <int D>
__global__ void __launch_bounds__(64)
decode_combine_kernel(DecodeArgs a)
{
    constexpr int PER = D / 64;
    constexpr int CH = 16;  // splits per batch of accumulator loads
    const int lane = threadIdx.x;
    const int64_t bh = blockIdx.x;
    const int S = a.splits;
    const float *ml = a.part_ml + bh * S * 2;
    const float *pa = a.part_acc + bh * S * D + PER * lane;

    // one round of loads: the first CH splits' accumulator slices and, one
    // split per lane, the references and sums
    float v[CH][PER];
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
        for (int i = 0; i < PER; ++i)
            v[j][i] = j < S ? pa[(int64_t)j * D + i] : 0.f;
    const float m0 = lane < S ? ml[2 * lane] : -INFINITY;
    const float l0 = lane < S ? ml[2 * lane + 1] : 0.f;

    float mloc = m0;
    for (int s = lane + 64; s < S; s += 64)
        mloc = fmaxf(mloc, ml[2 * s]);
    const float M = wave_max(mloc);
    // weight of split `lane` (splits past 64 are reloaded below)
    const float w0 = (M == -INFINITY || m0 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m0 - M);
    float lloc = w0 * l0;
    for (int s = lane + 64; s < S; s += 64) {
        const float ms = ml[2 * s];
        lloc += (M == -INFINITY || ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - M) * ml[2 * s + 1];
    }
    const float L = wave_sum(lloc);

    float o[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i)
        o[i] = 0.f;
    if (M != -INFINITY) {
        for (int s0 = 0; s0 < S; s0 += CH) {
            if (s0 > 0) {
#pragma unroll
                for (int j = 0; j < CH; ++j)
#pragma unroll
                    for (int i = 0; i < PER; ++i)
                        v[j][i] = s0 + j < S ? pa[(int64_t)(s0 + j) * D + i] : 0.f;
            }
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const int s = s0 + j;
                if (s < S) {
                    float w;
                    if (s < 64) {
                        w = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(w0), s));
                    } else {
                        const float ms = ml[2 * s];
                        w = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - M);
                    }
#pragma unroll
                    for (int i = 0; i < PER; ++i)
                        o[i] = __builtin_fmaf(w, v[j][i], o[i]);
                }
            }
        }
    }
    // no key at all (L = 0 exactly); a NaN sum (NaN in visible inputs)
    // propagates to O and LSE instead of passing for an empty stream
    const bool empty = L == 0.f;
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

template <int D, bool PAGED>
hipError_t launch_d(const DecodeArgs &a, hipStream_t stream)
{
    const int G = a.Hq / a.Hkv;
    hipError_t e;
    {
        const int hchunks = (G + 15) / 16;
        const long long grid = (long long)a.B * a.Hkv * hchunks * a.splits;
        if (grid > 0x7fffffffLL)
            return hipErrorInvalidConfiguration;
        constexpr int NW = 2;  // waves per split: LDS (16 KB per wave) allows 10 waves per CU
        hipLaunchKernelGGL((decode_mfma_kernel<D, NW, PAGED>), dim3((unsigned)grid), dim3(64 * NW), 0,
                           stream, a, hchunks);
        e = hipGetLastError();
    }
    if (e != hipSuccess)
        return e;
    const long long grid = (long long)a.B * a.Hq;
    if (grid > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)grid), dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

namespace {

// Split partials of the entry point for callers that cannot allocate
// (attn_fwd_decode_noalloc): a fixed array in device memory instead of a
// caller workspace. Every device the library runs on holds its own copy
// until the process ends. Host code never passes the array's name to a
// kernel: the name is a host-side stand-in, the device address comes from
// hipGetSymbolAddress below.
constexpr size_t kScratchBytes = size_t(16) << 20;
__device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

}  // namespace

size_t decode_scratch_bytes() { return kScratchBytes; }

// Device address of `scratch` on the current device, looked up once per
// device (the first call on a device, with that device current) and kept.
hipError_t decode_scratch(float **out)
{
    constexpr int kMaxDev = 64;
    static std::atomic<float *> addr[kMaxDev];
    static std::mutex mu;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDev)
        return hipErrorInvalidDevice;
    float *p = addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(mu);
        p = addr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            void *sym = nullptr;
            e = hipGetSymbolAddress(&sym, HIP_SYMBOL(scratch));
            if (e != hipSuccess)
                return e;
            if (sym == nullptr)
                return hipErrorInvalidSymbol;
            p = static_cast<float *>(sym);
            addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs &a, int d, hipStream_t stream)
{
    const bool paged = a.table != nullptr;
    switch (d) {
    case 64:
        return paged ? launch_d<64, true>(a, stream) : launch_d<64, false>(a, stream);
    case 128:
        return paged ? launch_d<128, true>(a, stream) : launch_d<128, false>(a, stream);
    case 256:
        return paged ? launch_d<256, true>(a, stream) : launch_d<256, false>(a, stream);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace miattn
