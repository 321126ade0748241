/*
 * miattn.h -- C ABI of libmiattn, fused softmax attention for AMD Instinct
 * MI355X (gfx950): prefill forward (with window, score-modifier and packed
 * variants), split-KV decode over contiguous or paged caches, and the
 * prefill backward.
 *
 * The operation is O = softmax(scale * Q K^T + mask) V together with the
 * per-row log-sum-exp, computed as one tiled reduction under the
 * online-softmax monoid: the state of a row is (running max m, running sum l
 * rescaled to m, value accumulator rescaled to m), two states combine by
 * rescaling both to the larger max and adding (the tang paper,
 * muni.works/research/tang, §2.2 "Comprehensions and monoids" and §2.3
 * "Rewrites": the max and both exponential sums of softmax merge into this
 * one reduction, so the score matrix is never materialised). The final map
 * O = acc / l runs on the thread that holds the accumulator (§2.3, epilogues
 * run on the reducing thread), and LSE = m + ln l is the same monoid's
 * logsumexp.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers into caller-owned memory; the
 *     library allocates nothing and keeps no state between calls, apart from
 *     a thread-local copy of the last error message and a per-device cache
 *     of how many prefill workgroups fit on the device at once.
 *   - Tensors are dense, row-major, contiguous. bf16 tensors are raw IEEE
 *     bfloat16 bit patterns (uint16); q, k, v, o and the workspace must be
 *     16-byte aligned. lse, kv_lens, block tables, prefix sums and ALiBi
 *     slopes need only 4-byte alignment: they are read and written one
 *     4-byte element at a time, so a view into a larger f32 or int32 tensor
 *     can be passed directly.
 *   - Work is enqueued on `stream` and the call returns without waiting;
 *     nothing is synchronised. Calls on different streams are independent.
 *   - Every logical output element is written (including rows that see no
 *     key), and nothing outside the logical outputs is written.
 *   - A row with no visible key gets O = +0.0 and LSE = -inf: the finished
 *     identity of the monoid (§2.1 "Views": a guarded read yields the
 *     reduction's identity). Masked keys are excluded by a select, never by
 *     an additive bias, so values stored at masked or out-of-range positions
 *     cannot reach any output -- with one caveat for causal prefill: a key
 *     that lies in a partially visible tile and is masked for some rows is
 *     multiplied by an exact zero weight, so its V row must hold finite
 *     values (NaN/inf there would propagate as 0 * NaN).
 *   - Accumulation is float32: scores and the monoid state in f32. In both
 *     the prefill and the decode kernels the probabilities are rounded to
 *     bf16 (round to nearest even) before the value contraction, while the
 *     row sum l that normalises O and gives LSE adds the unrounded f32
 *     probabilities. O is rounded to bf16 (RNE) and LSE is stored as f32.
 *   - Return value: MIATTN_OK, or an error code with the message available
 *     from miattn_last_error(). Argument checks happen on the host before
 *     anything is enqueued; on error nothing is launched.
 */
#ifndef MIATTN_H
#define MIATTN_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#if defined(__GNUC__)
#define MIATTN_API __attribute__((visibility("default")))
#else
#define MIATTN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MIATTN_OK = 0,
    MIATTN_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, bad scale */
    MIATTN_ERR_UNSUPPORTED = 2, /* head dimension not in {64, 128, 256}, or a
                                   prefill head slice of 2 GiB or more */
    MIATTN_ERR_HIP = 3          /* the HIP runtime reported a launch error */
} miattn_status;

/*
 * Prefill / full attention forward.
 *
 *   q   bf16 [B, Hq,  Sq, d]       queries
 *   k   bf16 [B, Hkv, Sk, d]       keys
 *   v   bf16 [B, Hkv, Sk, d]       values
 *   o   bf16 [B, Hq,  Sq, d]       output (written)
 *   lse f32  [B, Hq,  Sq]          natural-log log-sum-exp of the scaled,
 *                                  masked scores of each row (written)
 *
 * Query head h reads kv-head h / (Hq / Hkv): grouped-query attention as two
 * head dimensions (kv-head, group), §2.1 "Views". `causal` != 0 applies the
 * bottom-right aligned mask: key j is visible to query i iff
 * j <= i + (Sk - Sq); for Sq == Sk this is the usual lower-triangular
 * (upper-triangle-masked) pattern. scale multiplies Q K^T before the mask and
 * must be finite and > 0.
 *
 * Sizes: B, Sq, Sk >= 0 (B == 0 or Sq == 0: nothing to do, pointers unused;
 * Sk == 0: every row is empty, k and v unused); Hq, Hkv >= 1 with
 * Hq % Hkv == 0; d in {64, 128, 256}. One head's slice of Q and of K / V
 * must stay below 2 GiB (Sq * d * 2 and Sk * d * 2 < 2^31; Sq, Sk < 4M at
 * d = 256): the kernels address within a head with 32-bit buffer offsets.
 * Offsets across heads and batches are 64-bit.
 */
MIATTN_API int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
             int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal,
             float scale, hipStream_t stream);

/*
 * Prefill forward with a sliding window: attn_fwd with the further mask
 *
 *   key j is visible to query i only if  j >= i + (Sk - Sq) - window_left
 *
 * (window_left >= 0; with causal != 0 a row then sees its own aligned key and
 * the window_left keys before it). Every other argument, size limit and error
 * is attn_fwd's. The window only changes the mask, so the reduction is the
 * same online-softmax monoid (the tang paper, §2.3 "Rewrites": a change of
 * the score or the mask leaves the monoid alone); key tiles that the window
 * hides from every row of a query tile are skipped, not computed under the
 * mask (the cost §7.3 of the paper measures when they are not). A row that
 * sees no key gets O = +0 and LSE = -inf.
 */
MIATTN_API int attn_fwd_window(const void *q, const void *k, const void *v, void *o,
                    float *lse, int B, int Hq, int Hkv, int Sq, int Sk, int d,
                    int causal, int window_left, float scale, hipStream_t stream);

/*
 * Prefill forward with the score and mask variants: attn_fwd with
 *
 *   window_left   >= 0: the sliding window of attn_fwd_window; < 0: none
 *   softcap       > 0: every scaled score s becomes softcap * tanh(s / softcap)
 *                 (the soft cap of the paper's variant table, §7.3); 0: none
 *   alibi_slopes  DEVICE float [Hq] or NULL: the scaled score of query i and
 *                 key j of query head h gets - alibi_slopes[h] * |i + Sk - Sq - j|
 *                 added (ALiBi, §7.3); the slopes are not inspected on the host
 *
 * applied in that order: the soft cap to the scaled score, then the ALiBi
 * term (both may be given), then the mask. LSE is the log-sum-exp of the
 * modified scores. Only the score changes, so the reduction is the same
 * online-softmax monoid (§2.3 "Rewrites"). softcap must be finite and >= 0.
 * Every other argument, limit and error is attn_fwd's.
 */
MIATTN_API int attn_fwd_ext(const void *q, const void *k, const void *v, void *o, float *lse,
                 int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal,
                 int window_left, float softcap, const float *alibi_slopes,
                 float scale, hipStream_t stream);

/*
 * Prefill forward over a packed batch of sequences of different lengths
 * (chunked prefill of several streams at once): attn_fwd applied to each
 * sequence b on its own, with
 *
 *   q, o  bf16 [Hq,  total_q, d]   rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 *                                  of each head are sequence b's queries
 *   k, v  bf16 [Hkv, total_k, d]   rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1
 *                                  are its keys
 *   lse   f32  [Hq,  total_q]
 *   cu_seqlens_q, cu_seqlens_k   int32 [B + 1] DEVICE arrays, non-decreasing,
 *                                  starting at 0 and ending at total_q /
 *                                  total_k. They are not inspected on the
 *                                  host; on the device each sequence's range
 *                                  is clamped into [0, total) and to
 *                                  max_seqlen_q / max_seqlen_k rows, so bad
 *                                  offsets give wrong values but no access
 *                                  outside the tensors.
 *
 * Each sequence has its own Sq = its query count and Sk = its key count,
 * with attn_fwd's bottom-right causal alignment (a chunk of new queries
 * against its cached prefix plus itself when Sk > Sq). max_seqlen_q must be
 * at least the longest query count (it sizes the launch). Head dimensions
 * 64, 128 and 256; total_q * d * 2 and
 * total_k * d * 2 below 2^31. B == 0, total_q == 0 or max_seqlen_q == 0:
 * nothing to do.
 */
MIATTN_API int attn_fwd_varlen(const void *q, const void *k, const void *v, void *o,
                    float *lse, const int *cu_seqlens_q, const int *cu_seqlens_k,
                    int B, int total_q, int total_k, int max_seqlen_q,
                    int max_seqlen_k, int Hq, int Hkv, int d, int causal,
                    float scale, hipStream_t stream);

/*
 * A packed variable-length batch with the score and mask variants:
 * attn_fwd_varlen with window_left, softcap and alibi_slopes as in
 * attn_fwd_ext, each sequence taking them against its own lengths (its
 * Sq, Sk: key j of the sequence is visible to its query i only if
 * j >= i + Sk - Sq - window_left, and the ALiBi distance is
 * |i + Sk - Sq - j|). Every sequence is an attention of its own, and a
 * change of the score or the mask leaves the monoid alone (the tang paper,
 * §2.3 "Rewrites"), so the kernel is the packed batch's with the variant's
 * score and mask. softcap must be finite and >= 0; every other argument,
 * limit and error is attn_fwd_varlen's.
 */
MIATTN_API int attn_fwd_varlen_ext(const void *q, const void *k, const void *v, void *o,
                    float *lse, const int *cu_seqlens_q, const int *cu_seqlens_k,
                    int B, int total_q, int total_k, int max_seqlen_q,
                    int max_seqlen_k, int Hq, int Hkv, int d, int causal,
                    int window_left, float softcap, const float *alibi_slopes,
                    float scale, hipStream_t stream);

/*
 * Prefill backward: the gradients of attn_fwd's O with respect to Q, K and V,
 * given the forward's O and LSE and the upstream gradient dout (the flash
 * backward: P is recomputed from LSE, and the softmax gradient uses
 * D_i = dout_i . O_i; the tang paper, §3 "Gradients are comprehensions").
 *
 *   q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, causal, scale: as for attn_fwd
 *              (o and lse are attn_fwd's outputs for these inputs)
 *   dout  bf16 [B, Hq,  Sq, d]   upstream gradient
 *   dq    bf16 [B, Hq,  Sq, d]   written
 *   dk    bf16 [B, Hkv, Sk, d]   written (summed over the Hq/Hkv query heads
 *   dv    bf16 [B, Hkv, Sk, d]   written  that read each kv-head)
 *   workspace  device scratch of at least attn_bwd_workspace_size(B, Hq, Sq)
 *              bytes (per row the f32 pair D_i, LSE_i log2 e, written by the
 *              dQ kernel and read by the dK/dV kernel that follows it);
 *              4-byte aligned; contents on entry do not matter. Two calls
 *              sharing one workspace must be ordered.
 *
 * f32 accumulation, bf16 results; P and dS are rounded to bf16 for their
 * matrix products. Head dimensions 64, 128 and 256. Keys no query sees get
 * zero gradients; rows with no visible key (LSE = -inf) contribute nothing.
 */
MIATTN_API int attn_bwd(const void *q, const void *k, const void *v, const void *o,
             const float *lse, const void *dout, void *dq, void *dk, void *dv,
             int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal,
             float scale, void *workspace, size_t workspace_bytes,
             hipStream_t stream);

/* Bytes of workspace attn_bwd needs: B * Hq * Sq * 8. 0 for invalid sizes. */
MIATTN_API size_t attn_bwd_workspace_size(int B, int Hq, int Sq);

/*
 * Bytes of workspace attn_fwd_decode needs: B * Hq * num_splits * (d + 2) * 4
 * (one f32 partial state (m, l, acc[d]) per stream, head and split).
 * Returns 0 for invalid arguments.
 */
MIATTN_API size_t attn_fwd_decode_workspace_size(int B, int Hq, int d, int num_splits);

/*
 * Decode forward (one query row per stream and head) with split-KV.
 *
 *   q        bf16  [B, Hq, d]
 *   k_cache  bf16  [B, Hkv, S_cap, d]   rows >= kv_lens[b] are never read
 *   v_cache  bf16  [B, Hkv, S_cap, d]
 *   kv_lens  int32 [B]  DEVICE array of valid cache lengths; values are not
 *                        inspected on the host and are clamped to [0, S_cap]
 *                        on the device
 *   o        bf16  [B, Hq, d]           (written)
 *   lse      f32   [B, Hq]              (written)
 *   workspace         device scratch of at least
 *                     attn_fwd_decode_workspace_size(B, Hq, d, num_splits)
 *                     bytes; its contents on entry do not matter and are
 *                     overwritten.
 *
 * Attention is non-causal over keys [0, kv_lens[b]). The keys of each stream
 * are cut into num_splits balanced ranges, split s covering
 * [floor(s*len/num_splits), floor((s+1)*len/num_splits)). A first kernel
 * reduces each range to a partial monoid state (one read of each K/V row
 * serves all Hq/Hkv query heads of its kv-head); a second kernel folds the
 * partials with the monoid's combine and finishes O and LSE. The split is
 * the paper's split schedule, valid for any associative monoid (§2.5
 * "Schedules"). Two calls sharing one workspace must be ordered (same stream
 * or synchronised).
 *
 * Sizes: B >= 0 (0: nothing to do); Hq, Hkv >= 1, Hq % Hkv == 0; S_cap >= 0;
 * d in {64, 128, 256}; num_splits >= 1.
 */
MIATTN_API int attn_fwd_decode(const void *q, const void *k_cache, const void *v_cache,
                    const int *kv_lens, void *o, float *lse, int B, int Hq,
                    int Hkv, int S_cap, int d, int num_splits, float scale,
                    void *workspace, size_t workspace_bytes,
                    hipStream_t stream);

/*
 * Decode forward that allocates nothing and takes no workspace, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. It is attn_fwd_decode (same
 * arguments without the workspace, same kernels, bit-identical results) with
 * the split partials in a fixed scratch array of 16 MiB that the library
 * holds in device memory: each device the library runs on keeps its own copy
 * from the first call on that device until the process ends (that first call
 * looks up the array's device address, so make it before any graph
 * capture).
 *
 *   q, k_cache, v_cache, kv_lens, o, lse, B, Hq, Hkv, S_cap, d, num_splits,
 *   scale, stream: as for attn_fwd_decode.
 *
 * Limit: attn_fwd_decode_workspace_size(B, Hq, d, num_splits) must be at most
 * 16 MiB (e.g. B = 32, Hq = 32, d = 128, 16 splits takes 8.5 MB), else
 * MIATTN_ERR_UNSUPPORTED and nothing is launched. Every call on one device
 * shares that device's scratch and needs no clearing (each call writes every
 * partial it reads), but calls that may overlap on one device (different
 * streams, or threads without ordering) race on it and must be serialised
 * by the caller.
 */
MIATTN_API int attn_fwd_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                            const int *kv_lens, void *o, float *lse, int B, int Hq,
                            int Hkv, int S_cap, int d, int num_splits, float scale,
                            hipStream_t stream);

/*
 * Decode forward over a paged KV cache: attn_fwd_decode with each stream's
 * cache rows read through a block table. A paged cache is the paper's gather
 * view (§2.1 "Views": one source coordinate of a read comes from an index
 * tensor; the paged KV cache of vLLM is its example), so the operation is
 * attn_fwd_decode on the gathered cache
 *
 *   K[b, g, r, :] = k_pages[block_table[b, r / page_size], g, r % page_size, :]
 *
 * (V likewise) for r < kv_lens[b]. The keys, splits and results are those of
 * attn_fwd_decode on that cache, bit for bit.
 *
 *   k_pages, v_pages  bf16  [num_pages, Hkv, page_size, d]  page pool
 *   block_table       int32 [B, max_pages_per_seq]  DEVICE; entry p of stream
 *                     b is the pool page holding its keys
 *                     [p * page_size, (p + 1) * page_size). Only the entries
 *                     that cover keys < kv_lens[b] are used; entries outside
 *                     [0, num_pages) are clamped into it on the device, so a
 *                     bad entry gives wrong values but never a read outside
 *                     the pool.
 *   kv_lens           int32 [B] DEVICE, clamped on the device to
 *                     [0, max_pages_per_seq * page_size]
 *   q, o, lse, num_splits, scale, workspace: as for attn_fwd_decode (the
 *                     workspace size is attn_fwd_decode_workspace_size's)
 *
 * Sizes: B >= 0 (0: nothing to do); num_pages >= 1 unless
 * max_pages_per_seq == 0 (then every stream is empty and the pools and table
 * are unused); page_size a power of two in [16, 2^20];
 * max_pages_per_seq * page_size < 2^31; Hq, Hkv, d as for attn_fwd_decode.
 * Two calls sharing one workspace must be ordered.
 */
MIATTN_API int attn_fwd_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                          const int *block_table, const int *kv_lens, void *o,
                          float *lse, int B, int Hq, int Hkv, int num_pages,
                          int page_size, int max_pages_per_seq, int d,
                          int num_splits, float scale, void *workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* Message for the last non-OK status returned on the calling thread. */
MIATTN_API const char *miattn_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
MIATTN_API int miattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MIATTN_H */
