// api.cpp -- the C ABI of libmiattn: argument validation, error reporting and
// dispatch to the kernel launchers. Nothing here allocates or synchronises.

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string>

#include "launch.h"
#include "miattn.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_ptr(const void *p, const char *name, uintptr_t align)
{
    if (p == nullptr)
        return fail(MIATTN_ERR_INVALID_ARG, "%s is NULL", name);
    if (!aligned(p, align))
        return fail(MIATTN_ERR_INVALID_ARG, "%s is not %u-byte aligned", name, (unsigned)align);
    return MIATTN_OK;
}

int check_heads_dim(int Hq, int Hkv, int d)
{
    if (Hq < 1 || Hkv < 1)
        return fail(MIATTN_ERR_INVALID_ARG, "head counts must be >= 1 (Hq=%d, Hkv=%d)", Hq, Hkv);
    if (Hq % Hkv != 0)
        return fail(MIATTN_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if (d != 64 && d != 128 && d != 256)
        return fail(MIATTN_ERR_UNSUPPORTED, "head dimension %d not supported (64, 128, 256)", d);
    return MIATTN_OK;
}

int check_scale(float scale)
{
    if (!(scale > 0.f) || !isfinite(scale))
        return fail(MIATTN_ERR_INVALID_ARG, "scale must be finite and > 0 (got %g)", (double)scale);
    return MIATTN_OK;
}

int hip_status(hipError_t e, const char *what)
{
    if (e == hipSuccess)
        return MIATTN_OK;
    return fail(MIATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

#define MIATTN_TRY(expr)                 \
    do {                                 \
        int rc_ = (expr);                \
        if (rc_ != MIATTN_OK)            \
            return rc_;                  \
    } while (0)

extern "C" {

static int fwd_impl(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                    int Hq, int Hkv, int Sq, int Sk, int d, int causal, int window, float scale,
                    hipStream_t stream, const char *what, float softcap = 0.f,
                    const float *alibi = nullptr)
{
    if (B < 0 || Sq < 0 || Sk < 0)
        return fail(MIATTN_ERR_INVALID_ARG, "sizes must be >= 0 (B=%d, Sq=%d, Sk=%d)", B, Sq, Sk);
    MIATTN_TRY(check_heads_dim(Hq, Hkv, d));
    MIATTN_TRY(check_scale(scale));
    if ((int64_t)Sq * d * 2 >= ((int64_t)1 << 31) || (int64_t)Sk * d * 2 >= ((int64_t)1 << 31))
        return fail(MIATTN_ERR_UNSUPPORTED,
                    "one head's Q or K/V slice reaches 2 GiB (Sq=%d, Sk=%d, d=%d)", Sq, Sk, d);
    if (B == 0 || Sq == 0)
        return MIATTN_OK;
    MIATTN_TRY(check_ptr(q, "q", 16));
    MIATTN_TRY(check_ptr(o, "o", 16));
    MIATTN_TRY(check_ptr(lse, "lse", 4));
    if (Sk > 0) {
        MIATTN_TRY(check_ptr(k, "k", 16));
        MIATTN_TRY(check_ptr(v, "v", 16));
    }
    miattn::FwdArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.o = static_cast<uint16_t *>(o);
    a.lse = lse;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.Sq = Sq;
    a.Sk = Sk;
    a.scale = scale;
    a.window = window;
    a.softcap = softcap;
    a.alibi = alibi;
    return hip_status(miattn::launch_fwd(a, d, causal != 0, stream), what);
}

int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq,
             int Hkv, int Sq, int Sk, int d, int causal, float scale, hipStream_t stream)
{
    return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, causal, -1, scale, stream,
                    "attn_fwd launch");
}

int attn_fwd_window(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                    int Hq, int Hkv, int Sq, int Sk, int d, int causal, int window_left,
                    float scale, hipStream_t stream)
{
    if (window_left < 0)
        return fail(MIATTN_ERR_INVALID_ARG, "window_left must be >= 0 (got %d)", window_left);
    return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, causal, window_left, scale, stream,
                    "attn_fwd_window launch");
}

int attn_fwd_ext(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq,
                 int Hkv, int Sq, int Sk, int d, int causal, int window_left, float softcap,
                 const float *alibi_slopes, float scale, hipStream_t stream)
{
    if (!(softcap >= 0.f) || !isfinite(softcap))
        return fail(MIATTN_ERR_INVALID_ARG, "softcap must be finite and >= 0 (got %g)",
                    (double)softcap);
    if (alibi_slopes != nullptr && !aligned(alibi_slopes, 4))
        return fail(MIATTN_ERR_INVALID_ARG, "alibi_slopes is not 4-byte aligned");
    return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, causal, window_left < 0 ? -1 : window_left,
                    scale, stream, "attn_fwd_ext launch", softcap, alibi_slopes);
}

size_t attn_fwd_decode_workspace_size(int B, int Hq, int d, int num_splits)
{
    if (B < 0 || Hq < 1 || d < 1 || num_splits < 1)
        return 0;
    return (size_t)B * (size_t)Hq * (size_t)num_splits * (size_t)(d + 2) * sizeof(float);
}

// Checks shared by the contiguous decode entry points; fills everything of
// `a` but the partials' location. *done: nothing to launch (B == 0).
static int decode_common(const void *q, const void *k_cache, const void *v_cache,
                         const int *kv_lens, void *o, float *lse, int B, int Hq, int Hkv,
                         int S_cap, int d, int num_splits, float scale, miattn::DecodeArgs &a,
                         bool *done)
{
    *done = false;
    if (B < 0 || S_cap < 0)
        return fail(MIATTN_ERR_INVALID_ARG, "sizes must be >= 0 (B=%d, S_cap=%d)", B, S_cap);
    MIATTN_TRY(check_heads_dim(Hq, Hkv, d));
    MIATTN_TRY(check_scale(scale));
    if (num_splits < 1)
        return fail(MIATTN_ERR_INVALID_ARG, "num_splits must be >= 1 (got %d)", num_splits);
    if (B == 0) {
        *done = true;
        return MIATTN_OK;
    }
    MIATTN_TRY(check_ptr(q, "q", 16));
    MIATTN_TRY(check_ptr(o, "o", 16));
    MIATTN_TRY(check_ptr(lse, "lse", 4));
    MIATTN_TRY(check_ptr(kv_lens, "kv_lens", 4));
    if (S_cap > 0) {
        MIATTN_TRY(check_ptr(k_cache, "k_cache", 16));
        MIATTN_TRY(check_ptr(v_cache, "v_cache", 16));
    }
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k_cache);
    a.v = static_cast<const uint16_t *>(v_cache);
    a.lens = kv_lens;
    a.o = static_cast<uint16_t *>(o);
    a.lse = lse;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.S_cap = S_cap;
    a.splits = num_splits;
    a.scale = scale;
    return MIATTN_OK;
}

int attn_fwd_decode(const void *q, const void *k_cache, const void *v_cache, const int *kv_lens,
                    void *o, float *lse, int B, int Hq, int Hkv, int S_cap, int d,
                    int num_splits, float scale, void *workspace, size_t workspace_bytes,
                    hipStream_t stream)
{
    miattn::DecodeArgs a;
    bool done = false;
    MIATTN_TRY(decode_common(q, k_cache, v_cache, kv_lens, o, lse, B, Hq, Hkv, S_cap, d,
                             num_splits, scale, a, &done));
    if (done)
        return MIATTN_OK;
    MIATTN_TRY(check_ptr(workspace, "workspace", 16));
    const size_t need = attn_fwd_decode_workspace_size(B, Hq, d, num_splits);
    if (workspace_bytes < need)
        return fail(MIATTN_ERR_INVALID_ARG, "workspace too small: %zu bytes, need %zu",
                    workspace_bytes, need);
    // workspace layout: acc partials [B,Hq,S,d] first (16-byte aligned rows),
    // then (m, l) pairs [B,Hq,S,2]
    a.part_acc = static_cast<float *>(workspace);
    a.part_ml = a.part_acc + (size_t)B * Hq * num_splits * d;
    return hip_status(miattn::launch_decode(a, d, stream), "attn_fwd_decode launch");
}

int attn_fwd_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                            const int *kv_lens, void *o, float *lse, int B, int Hq, int Hkv,
                            int S_cap, int d, int num_splits, float scale, hipStream_t stream)
{
    miattn::DecodeArgs a;
    bool done = false;
    MIATTN_TRY(decode_common(q, k_cache, v_cache, kv_lens, o, lse, B, Hq, Hkv, S_cap, d,
                             num_splits, scale, a, &done));
    if (done)
        return MIATTN_OK;
    const size_t need = attn_fwd_decode_workspace_size(B, Hq, d, num_splits);
    if (need > miattn::decode_scratch_bytes())
        return fail(MIATTN_ERR_UNSUPPORTED,
                    "attn_fwd_decode_noalloc needs %zu bytes of partials; its fixed scratch "
                    "holds %zu (B * Hq * num_splits * (d + 2) * 4 must fit; "
                    "attn_fwd_decode takes a caller workspace of any size)",
                    need, miattn::decode_scratch_bytes());
    float *ws = nullptr;
    MIATTN_TRY(hip_status(miattn::decode_scratch(&ws), "attn_fwd_decode_noalloc scratch"));
    // the same layout as the workspace of attn_fwd_decode
    a.part_acc = ws;
    a.part_ml = a.part_acc + (size_t)B * Hq * num_splits * d;
    return hip_status(miattn::launch_decode(a, d, stream), "attn_fwd_decode_noalloc launch");
}

int attn_fwd_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                          const int *block_table, const int *kv_lens, void *o, float *lse,
                          int B, int Hq, int Hkv, int num_pages, int page_size,
                          int max_pages_per_seq, int d, int num_splits, float scale,
                          void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (B < 0 || num_pages < 0 || max_pages_per_seq < 0)
        return fail(MIATTN_ERR_INVALID_ARG,
                    "sizes must be >= 0 (B=%d, num_pages=%d, max_pages_per_seq=%d)", B, num_pages,
                    max_pages_per_seq);
    if (page_size < 16 || page_size > (1 << 20) || (page_size & (page_size - 1)) != 0)
        return fail(MIATTN_ERR_INVALID_ARG, "page_size must be a power of two in [16, 2^20] (got %d)",
                    page_size);
    if ((int64_t)max_pages_per_seq * page_size >= ((int64_t)1 << 31))
        return fail(MIATTN_ERR_INVALID_ARG,
                    "max_pages_per_seq * page_size must stay below 2^31 (%d * %d)",
                    max_pages_per_seq, page_size);
    MIATTN_TRY(check_heads_dim(Hq, Hkv, d));
    MIATTN_TRY(check_scale(scale));
    if (num_splits < 1)
        return fail(MIATTN_ERR_INVALID_ARG, "num_splits must be >= 1 (got %d)", num_splits);
    if (B == 0)
        return MIATTN_OK;
    if (max_pages_per_seq > 0 && num_pages == 0)
        return fail(MIATTN_ERR_INVALID_ARG, "num_pages must be >= 1 when max_pages_per_seq > 0");
    MIATTN_TRY(check_ptr(q, "q", 16));
    MIATTN_TRY(check_ptr(o, "o", 16));
    MIATTN_TRY(check_ptr(lse, "lse", 4));
    MIATTN_TRY(check_ptr(kv_lens, "kv_lens", 4));
    if (max_pages_per_seq > 0) {
        MIATTN_TRY(check_ptr(k_pages, "k_pages", 16));
        MIATTN_TRY(check_ptr(v_pages, "v_pages", 16));
        MIATTN_TRY(check_ptr(block_table, "block_table", 4));
    }
    MIATTN_TRY(check_ptr(workspace, "workspace", 16));
    const size_t need = attn_fwd_decode_workspace_size(B, Hq, d, num_splits);
    if (workspace_bytes < need)
        return fail(MIATTN_ERR_INVALID_ARG, "workspace too small: %zu bytes, need %zu",
                    workspace_bytes, need);
    int shift = 0;
    while ((1 << shift) < page_size)
        ++shift;
    miattn::DecodeArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k_pages);
    a.v = static_cast<const uint16_t *>(v_pages);
    a.lens = kv_lens;
    a.o = static_cast<uint16_t *>(o);
    a.lse = lse;
    a.part_acc = static_cast<float *>(workspace);
    a.part_ml = a.part_acc + (size_t)B * Hq * num_splits * d;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.S_cap = max_pages_per_seq * page_size;
    a.splits = num_splits;
    a.scale = scale;
    if (max_pages_per_seq > 0) {
        a.table = block_table;
        a.max_pages = max_pages_per_seq;
        a.num_pages = num_pages;
        a.page_shift = shift;
    }
    // without pages every stream is empty: the contiguous path with S_cap = 0
    return hip_status(miattn::launch_decode(a, d, stream), "attn_fwd_decode_paged launch");
}

static int varlen_impl(const void *q, const void *k, const void *v, void *o, float *lse,
                       const int *cu_seqlens_q, const int *cu_seqlens_k, int B, int total_q,
                       int total_k, int max_seqlen_q, int max_seqlen_k, int Hq, int Hkv, int d,
                       int causal, int window, float softcap, const float *alibi, float scale,
                       hipStream_t stream, const char *what)
{
    if (B < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
        return fail(MIATTN_ERR_INVALID_ARG,
                    "sizes must be >= 0 (B=%d, total_q=%d, total_k=%d, max_seqlen_q=%d, "
                    "max_seqlen_k=%d)", B, total_q, total_k, max_seqlen_q, max_seqlen_k);
    MIATTN_TRY(check_heads_dim(Hq, Hkv, d));
    MIATTN_TRY(check_scale(scale));
    if ((int64_t)total_q * d * 2 >= ((int64_t)1 << 31) || (int64_t)total_k * d * 2 >= ((int64_t)1 << 31))
        return fail(MIATTN_ERR_UNSUPPORTED,
                    "one head's packed Q or K/V reaches 2 GiB (total_q=%d, total_k=%d, d=%d)",
                    total_q, total_k, d);
    if (B == 0 || total_q == 0 || max_seqlen_q == 0)
        return MIATTN_OK;
    MIATTN_TRY(check_ptr(q, "q", 16));
    MIATTN_TRY(check_ptr(o, "o", 16));
    MIATTN_TRY(check_ptr(lse, "lse", 4));
    MIATTN_TRY(check_ptr(cu_seqlens_q, "cu_seqlens_q", 4));
    MIATTN_TRY(check_ptr(cu_seqlens_k, "cu_seqlens_k", 4));
    if (total_k > 0) {
        MIATTN_TRY(check_ptr(k, "k", 16));
        MIATTN_TRY(check_ptr(v, "v", 16));
    }
    miattn::FwdArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.o = static_cast<uint16_t *>(o);
    a.lse = lse;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.Sq = max_seqlen_q;
    a.Sk = max_seqlen_k;
    a.scale = scale;
    a.cu_q = cu_seqlens_q;
    a.cu_k = cu_seqlens_k;
    a.total_q = total_q;
    a.total_k = total_k;
    a.window = window;
    a.softcap = softcap;
    a.alibi = alibi;
    return hip_status(miattn::launch_fwd(a, d, causal != 0, stream), what);
}

int attn_fwd_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                    const int *cu_seqlens_q, const int *cu_seqlens_k, int B, int total_q,
                    int total_k, int max_seqlen_q, int max_seqlen_k, int Hq, int Hkv, int d,
                    int causal, float scale, hipStream_t stream)
{
    return varlen_impl(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, total_q, total_k,
                       max_seqlen_q, max_seqlen_k, Hq, Hkv, d, causal, -1, 0.f, nullptr, scale,
                       stream, "attn_fwd_varlen launch");
}

int attn_fwd_varlen_ext(const void *q, const void *k, const void *v, void *o, float *lse,
                        const int *cu_seqlens_q, const int *cu_seqlens_k, int B, int total_q,
                        int total_k, int max_seqlen_q, int max_seqlen_k, int Hq, int Hkv, int d,
                        int causal, int window_left, float softcap, const float *alibi_slopes,
                        float scale, hipStream_t stream)
{
    if (!(softcap >= 0.f) || !isfinite(softcap))
        return fail(MIATTN_ERR_INVALID_ARG, "softcap must be finite and >= 0 (got %g)",
                    (double)softcap);
    if (alibi_slopes != nullptr && !aligned(alibi_slopes, 4))
        return fail(MIATTN_ERR_INVALID_ARG, "alibi_slopes is not 4-byte aligned");
    return varlen_impl(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, total_q, total_k,
                       max_seqlen_q, max_seqlen_k, Hq, Hkv, d, causal,
                       window_left < 0 ? -1 : window_left, softcap, alibi_slopes, scale, stream,
                       "attn_fwd_varlen_ext launch");
}

size_t attn_bwd_workspace_size(int B, int Hq, int Sq)
{
    if (B < 0 || Hq < 1 || Sq < 0)
        return 0;
    return (size_t)B * (size_t)Hq * (size_t)Sq * 2 * sizeof(float);
}

int attn_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
             const void *dout, void *dq, void *dk, void *dv, int B, int Hq, int Hkv, int Sq,
             int Sk, int d, int causal, float scale, void *workspace, size_t workspace_bytes,
             hipStream_t stream)
{
    if (B < 0 || Sq < 0 || Sk < 0)
        return fail(MIATTN_ERR_INVALID_ARG, "sizes must be >= 0 (B=%d, Sq=%d, Sk=%d)", B, Sq, Sk);
    MIATTN_TRY(check_heads_dim(Hq, Hkv, d));
    MIATTN_TRY(check_scale(scale));
    if ((int64_t)Sq * d * 2 >= ((int64_t)1 << 31) || (int64_t)Sk * d * 2 >= ((int64_t)1 << 31))
        return fail(MIATTN_ERR_UNSUPPORTED,
                    "one head's Q or K/V slice reaches 2 GiB (Sq=%d, Sk=%d, d=%d)", Sq, Sk, d);
    if (B == 0 || (Sq == 0 && Sk == 0))
        return MIATTN_OK;
    if (Sq > 0) {
        MIATTN_TRY(check_ptr(q, "q", 16));
        MIATTN_TRY(check_ptr(o, "o", 16));
        MIATTN_TRY(check_ptr(dout, "dout", 16));
        MIATTN_TRY(check_ptr(lse, "lse", 4));
        MIATTN_TRY(check_ptr(dq, "dq", 16));
        MIATTN_TRY(check_ptr(workspace, "workspace", 4));
        const size_t need = attn_bwd_workspace_size(B, Hq, Sq);
        if (workspace_bytes < need)
            return fail(MIATTN_ERR_INVALID_ARG, "workspace too small: %zu bytes, need %zu",
                        workspace_bytes, need);
    }
    if (Sk > 0) {
        MIATTN_TRY(check_ptr(k, "k", 16));
        MIATTN_TRY(check_ptr(v, "v", 16));
        MIATTN_TRY(check_ptr(dk, "dk", 16));
        MIATTN_TRY(check_ptr(dv, "dv", 16));
    }
    miattn::BwdArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.o = static_cast<const uint16_t *>(o);
    a.dout = static_cast<const uint16_t *>(dout);
    a.lse = lse;
    a.dq = static_cast<uint16_t *>(dq);
    a.dk = static_cast<uint16_t *>(dk);
    a.dv = static_cast<uint16_t *>(dv);
    a.dsum = static_cast<float *>(workspace);
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.Sq = Sq;
    a.Sk = Sk;
    a.scale = scale;
    return hip_status(miattn::launch_bwd(a, d, causal != 0, stream), "attn_bwd launch");
}

const char *miattn_last_error(void) { return g_last_error.c_str(); }

int miattn_version(void) { return 700; }

}  // extern "C"
