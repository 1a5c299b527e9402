// sdpa_api.cpp -- the C-ABI entry points of libsdpa.so (include/sdpa.h).
//
// Validates every argument on the host before anything is enqueued (a
// rejected call enqueues nothing: cuDNN Frontend v1.31.0 Release Notes,
// "Compatibility and numerical behavior", omission of the split workspace
// raises before launch), then launches the HIP kernels on the caller's
// stream.  Never allocates device memory, never reads device memory, never
// synchronizes the host.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "sdpa.h"
#include "sdpa_launch.h"

namespace {

thread_local char g_detail[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_detail, sizeof g_detail, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_detail[0] = '\0';
    return SDPA_OK;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(SDPA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kMaxTokens = (int64_t)1 << 31;
// rows of a split merge: its grid of rows / 4 work-groups of 256 work-items
// stays below 2^32 work-items
constexpr int64_t kMaxCombineRows = (int64_t)1 << 26;

}  // namespace

extern "C" {

int sdpa_version(void) { return 100; }

const char* sdpa_status_string(int status) {
    switch (status) {
        case SDPA_OK: return "SDPA_OK";
        case SDPA_ERR_NULL: return "SDPA_ERR_NULL: a required pointer is NULL";
        case SDPA_ERR_SHAPE: return "SDPA_ERR_SHAPE: inconsistent or out-of-range extents/strides";
        case SDPA_ERR_UNSUPPORTED: return "SDPA_ERR_UNSUPPORTED: request declined by this build";
        case SDPA_ERR_WORKSPACE: return "SDPA_ERR_WORKSPACE: workspace missing or too small";
        case SDPA_ERR_LSE_LAYOUT: return "SDPA_ERR_LSE_LAYOUT: bad LSE layout or padded capacity";
        case SDPA_ERR_HIP: return "SDPA_ERR_HIP: a HIP launch failed";
        default: return "unknown sdpa status";
    }
}

const char* sdpa_last_error_detail(void) { return g_detail; }

static int prefill_impl(const void* q, int64_t q_st, int64_t q_sh, const void* k, int64_t k_st,
                        int64_t k_sh, const void* v, int64_t v_st, int64_t v_sh, void* o,
                        int64_t o_st, int64_t o_sh, const int32_t* cu_seqlens_q,
                        const int32_t* cu_seqlens_kv, int32_t batch, int32_t max_seqlen_q,
                        int32_t max_seqlen_kv, int32_t h_q, int32_t h_kv, int32_t d_qk,
                        int32_t d_v, float scale, int32_t causal, float* lse, int32_t lse_layout,
                        int32_t lse_s_max, int32_t window, const float* sinks, int32_t stats_log2,
                        int32_t dtype, const float* descale_q, const float* descale_k,
                        const float* descale_v, void* stream) {
    const bool fp8 = dtype == SDPA_FP8_E4M3;
    if (batch < 0 || batch > 65535) return fail(SDPA_ERR_SHAPE, "batch=%d outside [0, 65535]", batch);
    if (h_q <= 0 || h_kv <= 0 || h_q % h_kv != 0)
        return fail(SDPA_ERR_SHAPE, "h_q=%d must be a positive multiple of h_kv=%d", h_q, h_kv);
    if (h_q > 65535) return fail(SDPA_ERR_SHAPE, "h_q=%d > 65535", h_q);
    if (d_qk <= 0 || d_v <= 0) return fail(SDPA_ERR_SHAPE, "head dims must be positive");
    if (max_seqlen_q < 0 || max_seqlen_kv < 0)
        return fail(SDPA_ERR_SHAPE, "max_seqlen_q/kv must be >= 0");
    if (causal != 0 && causal != 1) return fail(SDPA_ERR_SHAPE, "causal must be 0 or 1");
    if (lse_layout != SDPA_LSE_NONE && lse_layout != SDPA_LSE_PACKED &&
        lse_layout != SDPA_LSE_PADDED && lse_layout != SDPA_LSE_HEAD_MAJOR)
        return fail(SDPA_ERR_LSE_LAYOUT, "unknown lse_layout %d", lse_layout);
    if (lse_layout == SDPA_LSE_HEAD_MAJOR && lse_s_max <= 0)
        return fail(SDPA_ERR_LSE_LAYOUT, "head-major LSE needs its per-head stride in lse_s_max");
    if (stats_log2 != 0 && stats_log2 != 1) return fail(SDPA_ERR_SHAPE, "stats_log2 must be 0 or 1");
    const bool variant = window > 0 || sinks != nullptr || stats_log2 != 0 ||
                         lse_layout == SDPA_LSE_HEAD_MAJOR;
    if (variant && dtype != SDPA_BF16 && !fp8)
        return fail(SDPA_ERR_UNSUPPORTED,
                    "windows, sinks, base-2 and head-major LSE are served for bf16 and FP8 only");
    if (lse_layout != SDPA_LSE_NONE && lse == nullptr)
        return fail(SDPA_ERR_NULL, "lse is NULL but lse_layout=%d requests Stats", lse_layout);
    if (lse_layout == SDPA_LSE_PADDED && lse_s_max < max_seqlen_q)
        return fail(SDPA_ERR_LSE_LAYOUT, "padded LSE capacity lse_s_max=%d < max_seqlen_q=%d",
                    lse_s_max, max_seqlen_q);
    if (q_st <= 0 || q_sh <= 0 || k_st <= 0 || k_sh <= 0 || v_st <= 0 || v_sh <= 0 || o_st <= 0 ||
        o_sh <= 0)
        return fail(SDPA_ERR_SHAPE, "token/head strides must be positive");
    if (dtype == SDPA_BF16) {
        if (k_st < d_qk || v_st < d_v)
            return fail(SDPA_ERR_SHAPE, "K/V token rows overlap: k_st=%lld < d_qk or v_st=%lld < d_v",
                        (long long)k_st, (long long)v_st);
        if (k_st >= ((int64_t)1 << 22) || v_st >= ((int64_t)1 << 22))
            return fail(SDPA_ERR_UNSUPPORTED, "bf16 prefill K/V token strides must be below 2^22");
        if (d_qk != d_v || (d_qk != 64 && d_qk != 128 && d_qk != 256))
            return fail(SDPA_ERR_UNSUPPORTED,
                        "bf16 prefill serves d_qk == d_v in {64, 128, 256}; got (%d, %d)", d_qk,
                        d_v);
        const int64_t st[8] = {q_st, q_sh, k_st, k_sh, v_st, v_sh, o_st, o_sh};
        for (int64_t s : st)
            if (s % 8 != 0)
                return fail(SDPA_ERR_UNSUPPORTED,
                            "bf16 prefill needs strides that are multiples of 8 elements");
    } else if (fp8) {
        if (d_qk != 128 || d_v != 128)
            return fail(SDPA_ERR_UNSUPPORTED, "FP8 prefill serves d_qk == d_v == 128; got (%d, %d)",
                        d_qk, d_v);
        if (k_st < d_qk || v_st < d_v)
            return fail(SDPA_ERR_SHAPE, "K/V token rows overlap: k_st=%lld < d_qk or v_st=%lld < d_v",
                        (long long)k_st, (long long)v_st);
        if (k_st >= ((int64_t)1 << 22) || v_st >= ((int64_t)1 << 22))
            return fail(SDPA_ERR_UNSUPPORTED, "FP8 prefill K/V token strides must be below 2^22");
        const int64_t st8[6] = {q_st, q_sh, k_st, k_sh, v_st, v_sh};
        for (int64_t x : st8)
            if (x % 16 != 0)
                return fail(SDPA_ERR_UNSUPPORTED,
                            "FP8 prefill needs Q/K/V strides that are multiples of 16 elements");
        if (o_st % 8 != 0 || o_sh % 8 != 0)
            return fail(SDPA_ERR_UNSUPPORTED, "FP8 prefill writes bf16 O: strides multiples of 8");
    } else if (dtype == SDPA_FP32) {
        if (d_qk > 256 || d_v > 256)
            return fail(SDPA_ERR_UNSUPPORTED, "fp32 prefill serves head dims <= 256");
    } else {
        return fail(SDPA_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
    }
    if (batch == 0) return ok();
    if (!q || !k || !v || !o || !cu_seqlens_q || !cu_seqlens_kv)
        return fail(SDPA_ERR_NULL, "q/k/v/o/cu_seqlens_q/cu_seqlens_kv must be non-NULL");
    if (fp8 && (!descale_q || !descale_k || !descale_v))
        return fail(SDPA_ERR_NULL, "FP8 prefill needs descale_q, descale_k and descale_v");
    if (fp8 && (!aligned(descale_q, 4) || !aligned(descale_k, 4) || !aligned(descale_v, 4)))
        return fail(SDPA_ERR_UNSUPPORTED, "descale pointers must be 4-byte aligned");
    const size_t align = dtype == SDPA_FP32 ? 4 : 16;
    if (!aligned(q, align) || !aligned(k, align) || !aligned(v, align) || !aligned(o, align) ||
        (lse && !aligned(lse, 4)) || !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_kv, 4) ||
        (sinks && !aligned(sinks, 4)))
        return fail(SDPA_ERR_UNSUPPORTED, "pointer alignment: need %zu bytes for q/k/v/o", align);

    sdpa::PrefillArgs a;
    a.q = q;
    a.q_st = q_st;
    a.q_sh = q_sh;
    a.k = k;
    a.k_st = k_st;
    a.k_sh = k_sh;
    a.v = v;
    a.v_st = v_st;
    a.v_sh = v_sh;
    a.o = o;
    a.o_st = o_st;
    a.o_sh = o_sh;
    a.cu_q = cu_seqlens_q;
    a.cu_kv = cu_seqlens_kv;
    a.batch = batch;
    a.max_q = max_seqlen_q;
    a.max_kv = max_seqlen_kv;
    a.hq = h_q;
    a.hkv = h_kv;
    a.dqk = d_qk;
    a.dv = d_v;
    a.scale = scale;
    a.causal = causal;
    a.lse = lse_layout == SDPA_LSE_NONE ? nullptr : lse;
    a.lse_layout = lse_layout;
    a.lse_s_max = lse_s_max;
    a.window = window > 0 ? window : 0;
    a.sinks = sinks;
    a.stats_log2 = stats_log2;
    a.fp8 = fp8 ? 1 : 0;
    a.descale_q = fp8 ? descale_q : nullptr;
    a.descale_k = fp8 ? descale_k : nullptr;
    a.descale_v = fp8 ? descale_v : nullptr;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (lse_layout == SDPA_LSE_PADDED) {
        hipError_t e = sdpa::launch_fill_neg_inf(lse, (int64_t)batch * lse_s_max * h_q, s);
        if (e != hipSuccess) return hip_fail(e, "padded LSE -inf fill");
    }
    hipError_t e = dtype == SDPA_FP32 ? sdpa::launch_prefill_f32(a, s)
                                      : sdpa::launch_prefill_bf16(a, s);
    if (e != hipSuccess) return hip_fail(e, "prefill launch");
    return ok();
}

int sdpa_prefill_thd(const void* q, int64_t q_st, int64_t q_sh, const void* k, int64_t k_st,
                     int64_t k_sh, const void* v, int64_t v_st, int64_t v_sh, void* o,
                     int64_t o_st, int64_t o_sh, const int32_t* cu_seqlens_q,
                     const int32_t* cu_seqlens_kv, int32_t batch, int32_t max_seqlen_q,
                     int32_t max_seqlen_kv, int32_t h_q, int32_t h_kv, int32_t d_qk,
                     int32_t d_v, float scale, int32_t causal, float* lse, int32_t lse_layout,
                     int32_t lse_s_max, int32_t dtype, void* stream) {
    if (dtype == SDPA_FP8_E4M3)
        return fail(SDPA_ERR_UNSUPPORTED, "per-tensor FP8 needs its descales: sdpa_prefill_thd_fp8");
    return prefill_impl(q, q_st, q_sh, k, k_st, k_sh, v, v_st, v_sh, o, o_st, o_sh, cu_seqlens_q,
                        cu_seqlens_kv, batch, max_seqlen_q, max_seqlen_kv, h_q, h_kv, d_qk, d_v,
                        scale, causal, lse, lse_layout, lse_s_max, 0, nullptr, 0, dtype, nullptr,
                        nullptr, nullptr, stream);
}

int sdpa_prefill_thd_ex(const void* q, int64_t q_st, int64_t q_sh, const void* k, int64_t k_st,
                        int64_t k_sh, const void* v, int64_t v_st, int64_t v_sh, void* o,
                        int64_t o_st, int64_t o_sh, const int32_t* cu_seqlens_q,
                        const int32_t* cu_seqlens_kv, int32_t batch, int32_t max_seqlen_q,
                        int32_t max_seqlen_kv, int32_t h_q, int32_t h_kv, int32_t d_qk,
                        int32_t d_v, float scale, int32_t causal, int32_t window_left,
                        const float* sinks, float* lse, int32_t lse_layout, int32_t lse_s_max,
                        int32_t stats_log2, int32_t dtype, void* stream) {
    if (dtype == SDPA_FP8_E4M3)
        return fail(SDPA_ERR_UNSUPPORTED, "per-tensor FP8 needs its descales: sdpa_prefill_thd_fp8");
    if (window_left < 0) return fail(SDPA_ERR_SHAPE, "window_left=%d < 0", window_left);
    return prefill_impl(q, q_st, q_sh, k, k_st, k_sh, v, v_st, v_sh, o, o_st, o_sh, cu_seqlens_q,
                        cu_seqlens_kv, batch, max_seqlen_q, max_seqlen_kv, h_q, h_kv, d_qk, d_v,
                        scale, causal, lse, lse_layout, lse_s_max, window_left, sinks, stats_log2,
                        dtype, nullptr, nullptr, nullptr, stream);
}

int sdpa_prefill_thd_fp8(const void* q, int64_t q_st, int64_t q_sh, const void* k, int64_t k_st,
                         int64_t k_sh, const void* v, int64_t v_st, int64_t v_sh, void* o,
                         int64_t o_st, int64_t o_sh, const int32_t* cu_seqlens_q,
                         const int32_t* cu_seqlens_kv, int32_t batch, int32_t max_seqlen_q,
                         int32_t max_seqlen_kv, int32_t h_q, int32_t h_kv, int32_t d_qk,
                         int32_t d_v, float scale, int32_t causal, int32_t window_left,
                         const float* sinks, float* lse, int32_t lse_layout, int32_t lse_s_max,
                         int32_t stats_log2, const float* descale_q, const float* descale_k,
                         const float* descale_v, void* stream) {
    if (window_left < 0) return fail(SDPA_ERR_SHAPE, "window_left=%d < 0", window_left);
    return prefill_impl(q, q_st, q_sh, k, k_st, k_sh, v, v_st, v_sh, o, o_st, o_sh, cu_seqlens_q,
                        cu_seqlens_kv, batch, max_seqlen_q, max_seqlen_kv, h_q, h_kv, d_qk, d_v,
                        scale, causal, lse, lse_layout, lse_s_max, window_left, sinks, stats_log2,
                        SDPA_FP8_E4M3, descale_q, descale_k, descale_v, stream);
}

size_t sdpa_decode_workspace_bytes(int32_t batch, int32_t s_q, int32_t h_q, int32_t d_v,
                                   int32_t num_splits) {
    if (batch <= 0 || s_q <= 0 || h_q <= 0 || d_v <= 0 || num_splits <= 1) return 0;
    const size_t rows = (size_t)batch * s_q * h_q;
    size_t o_bytes = (size_t)num_splits * rows * d_v * sizeof(float);
    o_bytes = (o_bytes + 255) / 256 * 256;
    return o_bytes + (size_t)num_splits * rows * sizeof(float);
}

int sdpa_decode_path(int32_t batch, int32_t s_q, int32_t h_q, int32_t h_kv, int32_t d_qk,
                     int32_t d_v, int32_t page_size, int64_t k_st, int64_t v_st,
                     int32_t num_splits, int32_t dtype) {
    const bool fp8 = dtype == SDPA_FP8_E4M3;
    if (!fp8 && dtype != SDPA_BF16) return 0;
    if (batch < 0 || s_q <= 0 || h_q <= 0 || h_kv <= 0 || h_q % h_kv != 0) return 0;
    if (!sdpa::decode_supported(d_qk, d_v) || page_size <= 0 || page_size % 16 != 0) return 0;
    if (num_splits < 1 || num_splits > 256 || k_st < d_qk || v_st < d_v) return 0;
    if (fp8 && (k_st % 16 != 0 || v_st % 16 != 0)) return 0;
    sdpa::DecodeArgs a{};
    a.batch = batch;
    a.sq = s_q;
    a.hq = h_q;
    a.hkv = h_kv;
    a.dqk = d_qk;
    a.dv = d_v;
    a.page = page_size;
    a.k_st = k_st;
    a.v_st = v_st;
    a.splits = num_splits;
    a.fp8 = fp8 ? 1 : 0;
    if ((int64_t)s_q * (h_q / h_kv) > 512 && !sdpa::prefill_paged_supported(a)) return 0;
    return (int)sdpa::decode_path(a);
}

static int decode_impl(const void* q, const void* k_pool, int64_t k_sp, int64_t k_st,
                       int64_t k_sh, const void* v_pool, int64_t v_sp, int64_t v_st, int64_t v_sh,
                       const int32_t* page_table_k, const int32_t* page_table_v,
                       int32_t table_stride, const int32_t* seq_lens, int32_t max_seqlen_kv,
                       int32_t batch, int32_t s_q, int32_t h_q, int32_t h_kv, int32_t d_qk,
                       int32_t d_v, int32_t page_size, float scale, int32_t causal,
                       int32_t num_splits, void* workspace, size_t workspace_bytes, void* o,
                       float* lse, int32_t dtype, const float* descale_q,
                       const float* descale_k, const float* descale_v, void* stream,
                       bool use_scratch = false, int32_t window = 0,
                       const float* sinks = nullptr, int32_t stats_log2 = 0) {
    const bool fp8 = dtype == SDPA_FP8_E4M3;
    if (batch < 0) return fail(SDPA_ERR_SHAPE, "batch=%d < 0", batch);
    if (window < 0) return fail(SDPA_ERR_SHAPE, "window_left=%d < 0", window);
    if (stats_log2 != 0 && stats_log2 != 1) return fail(SDPA_ERR_SHAPE, "stats_log2 must be 0 or 1");
    if (s_q <= 0) return fail(SDPA_ERR_SHAPE, "s_q=%d must be >= 1", s_q);
    if (h_q <= 0 || h_kv <= 0 || h_q % h_kv != 0)
        return fail(SDPA_ERR_SHAPE, "h_q=%d must be a positive multiple of h_kv=%d", h_q, h_kv);
    if (!sdpa::decode_supported(d_qk, d_v))
        return fail(SDPA_ERR_UNSUPPORTED,
                    "paged decode serves (d_qk, d_v) in {(64,64), (128,128), (256,256), "
                    "(192,128), (576,512)}; got (%d, %d)",
                    d_qk, d_v);
    if (page_size <= 0 || page_size % 16 != 0)
        return fail(SDPA_ERR_UNSUPPORTED, "page_size=%d must be a positive multiple of 16",
                    page_size);
    if (num_splits < 1 || num_splits > 256)
        return fail(SDPA_ERR_SHAPE, "num_splits=%d outside [1, 256]", num_splits);
    if (fp8) {
        // per-tensor FP8 K/V rows are DMA'd and loaded in 16-byte pieces
        const int64_t st[6] = {k_sp, k_st, k_sh, v_sp, v_st, v_sh};
        for (int64_t x : st)
            if (x % 16 != 0)
                return fail(SDPA_ERR_UNSUPPORTED, "FP8 K/V pool strides must be multiples of 16");
    }
    {
        // more than 512 query rows per KV head: only the chunked-prefill path
        // (prefill kernel over the page tables, bf16 or FP8) serves them
        sdpa::DecodeArgs probe{};
        probe.dqk = d_qk;
        probe.dv = d_v;
        probe.page = page_size;
        probe.k_st = k_st;
        probe.v_st = v_st;
        probe.sq = s_q;
        probe.hq = h_q;
        probe.hkv = h_kv;
        probe.fp8 = fp8 ? 1 : 0;  // the FP8 prefill kernel serves d = 128 only
        if ((int64_t)s_q * (h_q / h_kv) > 512 && !sdpa::prefill_paged_supported(probe))
            return fail(SDPA_ERR_UNSUPPORTED,
                        "s_q * (h_q / h_kv) = %lld query rows per KV head > 512 (more need "
                        "d_qk = d_v = 64 or 128 with page_size %% 64 == 0, or bf16 "
                        "d_qk = d_v = 256 with page_size %% 32 == 0)",
                        (long long)s_q * (h_q / h_kv));
    }
    if (causal != 0 && causal != 1) return fail(SDPA_ERR_SHAPE, "causal must be 0 or 1");
    // Window, sinks and base-2 Stats are not served at d = 256: the first GPU
    // run of the few-row kernel at d = 256 with a window and sinks faulted, and
    // the cause is not yet found, so the combination is declined before launch.
    if ((window > 0 || sinks != nullptr || stats_log2 != 0) && (d_qk == 256 || d_v == 256))
        return fail(SDPA_ERR_UNSUPPORTED,
                    "left windows, sinks and base-2 Stats are not served for d = 256 decode");
    if (table_stride <= 0) return fail(SDPA_ERR_SHAPE, "table_stride must be positive");
    if (max_seqlen_kv < 0 || (int64_t)max_seqlen_kv > (int64_t)table_stride * page_size)
        return fail(SDPA_ERR_SHAPE, "max_seqlen_kv=%d exceeds table_stride*page_size=%lld",
                    max_seqlen_kv, (long long)table_stride * page_size);
    if (k_sp <= 0 || k_st <= 0 || k_sh <= 0 || v_sp <= 0 || v_st <= 0 || v_sh <= 0)
        return fail(SDPA_ERR_SHAPE, "pool strides must be positive");
    if (k_st < d_qk || v_st < d_v)
        return fail(SDPA_ERR_SHAPE, "pool token rows overlap: k_st=%lld < d_qk or v_st=%lld < d_v",
                    (long long)k_st, (long long)v_st);
    if (k_st >= ((int64_t)1 << 26) || v_st >= ((int64_t)1 << 26))
        return fail(SDPA_ERR_UNSUPPORTED, "pool token strides must be below 2^26 elements");
    const int64_t st[6] = {k_sp, k_st, k_sh, v_sp, v_st, v_sh};
    for (int64_t x : st)
        if (x % 8 != 0)
            return fail(SDPA_ERR_UNSUPPORTED, "pool strides must be multiples of 8 elements");
    if ((int64_t)batch * h_kv * num_splits >= kMaxTokens)
        return fail(SDPA_ERR_SHAPE, "batch * h_kv * num_splits too large");
    if (num_splits > 1 && (int64_t)batch * s_q * h_q >= kMaxCombineRows)
        return fail(SDPA_ERR_SHAPE, "batch * s_q * h_q = %lld rows to merge >= 2^26",
                    (long long)batch * s_q * h_q);
    if (batch == 0) return ok();
    if (!q || !k_pool || !v_pool || !page_table_k || !page_table_v || !seq_lens || !o)
        return fail(SDPA_ERR_NULL, "q/k_pool/v_pool/page tables/seq_lens/o must be non-NULL");
    if (fp8 && (!descale_q || !descale_k || !descale_v))
        return fail(SDPA_ERR_NULL, "FP8 decode needs descale_q, descale_k and descale_v");
    if (fp8 && (!aligned(descale_q, 4) || !aligned(descale_k, 4) || !aligned(descale_v, 4)))
        return fail(SDPA_ERR_UNSUPPORTED, "descale pointers must be 4-byte aligned");
    if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(o, 16) ||
        (lse && !aligned(lse, 4)) || (sinks && !aligned(sinks, 4)))
        return fail(SDPA_ERR_UNSUPPORTED, "q/pools/o must be 16-byte aligned (lse, sinks 4)");
    const size_t need = sdpa_decode_workspace_bytes(batch, s_q, h_q, d_v, num_splits);
    if (use_scratch) {
        // the library-owned workspace: bounded, looked up without allocating
        if (need > sdpa::kDecodeScratchBytes)
            return fail(SDPA_ERR_WORKSPACE,
                        "the split workspace of this call (%zu bytes) exceeds the library-owned "
                        "%zu bytes; use sdpa_decode_paged with a caller workspace",
                        need, sdpa::kDecodeScratchBytes);
        workspace = nullptr;
        workspace_bytes = 0;
        if (need > 0) {
            hipError_t e = sdpa::decode_scratch(&workspace);
            if (e != hipSuccess) return hip_fail(e, "library-owned decode workspace lookup");
            workspace_bytes = sdpa::kDecodeScratchBytes;
        }
    }
    if (num_splits > 1) {
        if (workspace == nullptr)
            return fail(SDPA_ERR_WORKSPACE, "num_splits=%d needs %zu bytes of workspace, got NULL",
                        num_splits, need);
        if (workspace_bytes < need)
            return fail(SDPA_ERR_WORKSPACE, "workspace of %zu bytes < %zu required",
                        workspace_bytes, need);
        if (!aligned(workspace, 256))
            return fail(SDPA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    }
    sdpa::DecodeArgs a;
    a.q = q;
    a.k_pool = k_pool;
    a.k_sp = k_sp;
    a.k_st = k_st;
    a.k_sh = k_sh;
    a.v_pool = v_pool;
    a.v_sp = v_sp;
    a.v_st = v_st;
    a.v_sh = v_sh;
    a.pt_k = page_table_k;
    a.pt_v = page_table_v;
    a.table_stride = table_stride;
    a.seq_lens = seq_lens;
    a.batch = batch;
    a.sq = s_q;
    a.hq = h_q;
    a.hkv = h_kv;
    a.dqk = d_qk;
    a.dv = d_v;
    a.page = page_size;
    a.scale = scale;
    a.causal = causal;
    a.splits = num_splits;
    const int64_t rows = (int64_t)batch * s_q * h_q;
    a.o_part = nullptr;
    a.lse_part = nullptr;
    if (num_splits > 1) {
        size_t o_bytes = (size_t)num_splits * rows * d_v * sizeof(float);
        o_bytes = (o_bytes + 255) / 256 * 256;
        a.o_part = static_cast<float*>(workspace);
        a.lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + o_bytes);
    }
    a.o = o;
    a.lse = lse;
    a.fp8 = fp8 ? 1 : 0;
    a.descale_q = fp8 ? descale_q : nullptr;
    a.descale_k = fp8 ? descale_k : nullptr;
    a.descale_v = fp8 ? descale_v : nullptr;
    a.window = window;
    a.sinks = sinks;
    a.stats_log2 = stats_log2;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = fp8 ? sdpa::launch_decode_fp8(a, s) : sdpa::launch_decode_bf16(a, s);
    if (e != hipSuccess) return hip_fail(e, "paged decode launch");
    if (num_splits > 1) {
        e = sdpa::launch_combine(a.o_part, a.lse_part, num_splits, rows, d_v, o, lse, 0, s, sinks,
                                 h_q, stats_log2);
        if (e != hipSuccess) return hip_fail(e, "split-KV combine launch");
    }
    return ok();
}

int sdpa_decode_paged(const void* q, const void* k_pool, int64_t k_sp, int64_t k_st,
                      int64_t k_sh, const void* v_pool, int64_t v_sp, int64_t v_st, int64_t v_sh,
                      const int32_t* page_table_k, const int32_t* page_table_v,
                      int32_t table_stride, const int32_t* seq_lens, int32_t max_seqlen_kv,
                      int32_t batch, int32_t s_q, int32_t h_q, int32_t h_kv, int32_t d_qk,
                      int32_t d_v, int32_t page_size, float scale, int32_t causal,
                      int32_t num_splits, void* workspace, size_t workspace_bytes, void* o,
                      float* lse, int32_t dtype, void* stream) {
    if (dtype == SDPA_FP8_E4M3)
        return fail(SDPA_ERR_UNSUPPORTED, "per-tensor FP8 needs its descales: sdpa_decode_paged_fp8");
    if (dtype != SDPA_BF16) return fail(SDPA_ERR_UNSUPPORTED, "paged decode serves bf16 only");
    return decode_impl(q, k_pool, k_sp, k_st, k_sh, v_pool, v_sp, v_st, v_sh, page_table_k,
                       page_table_v, table_stride, seq_lens, max_seqlen_kv, batch, s_q, h_q, h_kv,
                       d_qk, d_v, page_size, scale, causal, num_splits, workspace,
                       workspace_bytes, o, lse, SDPA_BF16, nullptr, nullptr, nullptr, stream);
}

int sdpa_decode_paged_fp8(const void* q, const void* k_pool, int64_t k_sp, int64_t k_st,
                          int64_t k_sh, const void* v_pool, int64_t v_sp, int64_t v_st,
                          int64_t v_sh, const int32_t* page_table_k, const int32_t* page_table_v,
                          int32_t table_stride, const int32_t* seq_lens, int32_t max_seqlen_kv,
                          int32_t batch, int32_t s_q, int32_t h_q, int32_t h_kv, int32_t d_qk,
                          int32_t d_v, int32_t page_size, float scale, int32_t causal,
                          int32_t num_splits, void* workspace, size_t workspace_bytes,
                          const float* descale_q, const float* descale_k,
                          const float* descale_v, void* o, float* lse, void* stream) {
    return decode_impl(q, k_pool, k_sp, k_st, k_sh, v_pool, v_sp, v_st, v_sh, page_table_k,
                       page_table_v, table_stride, seq_lens, max_seqlen_kv, batch, s_q, h_q, h_kv,
                       d_qk, d_v, page_size, scale, causal, num_splits, workspace,
                       workspace_bytes, o, lse, SDPA_FP8_E4M3, descale_q, descale_k, descale_v,
                       stream);
}

int sdpa_decode_paged_noalloc(const void* q, const void* k_pool, int64_t k_sp, int64_t k_st,
                              int64_t k_sh, const void* v_pool, int64_t v_sp, int64_t v_st,
                              int64_t v_sh, const int32_t* page_table_k,
                              const int32_t* page_table_v, int32_t table_stride,
                              const int32_t* seq_lens, int32_t max_seqlen_kv, int32_t batch,
                              int32_t s_q, int32_t h_q, int32_t h_kv, int32_t d_qk, int32_t d_v,
                              int32_t page_size, float scale, int32_t causal, int32_t num_splits,
                              void* o, float* lse, int32_t dtype, void* stream) {
    if (dtype != SDPA_BF16) return fail(SDPA_ERR_UNSUPPORTED, "paged decode serves bf16 only");
    return decode_impl(q, k_pool, k_sp, k_st, k_sh, v_pool, v_sp, v_st, v_sh, page_table_k,
                       page_table_v, table_stride, seq_lens, max_seqlen_kv, batch, s_q, h_q, h_kv,
                       d_qk, d_v, page_size, scale, causal, num_splits, nullptr, 0, o, lse,
                       SDPA_BF16, nullptr, nullptr, nullptr, stream, /*use_scratch=*/true);
}

int sdpa_decode_paged_ex(const void* q, const void* k_pool, int64_t k_sp, int64_t k_st,
                         int64_t k_sh, const void* v_pool, int64_t v_sp, int64_t v_st,
                         int64_t v_sh, const int32_t* page_table_k, const int32_t* page_table_v,
                         int32_t table_stride, const int32_t* seq_lens, int32_t max_seqlen_kv,
                         int32_t batch, int32_t s_q, int32_t h_q, int32_t h_kv, int32_t d_qk,
                         int32_t d_v, int32_t page_size, float scale, int32_t causal,
                         int32_t window_left, const float* sinks, int32_t stats_log2,
                         int32_t num_splits, void* workspace, size_t workspace_bytes,
                         const float* descale_q, const float* descale_k, const float* descale_v,
                         void* o, float* lse, int32_t dtype, void* stream) {
    if (dtype != SDPA_BF16 && dtype != SDPA_FP8_E4M3)
        return fail(SDPA_ERR_UNSUPPORTED, "paged decode serves bf16 and FP8 E4M3; got %d", dtype);
    return decode_impl(q, k_pool, k_sp, k_st, k_sh, v_pool, v_sp, v_st, v_sh, page_table_k,
                       page_table_v, table_stride, seq_lens, max_seqlen_kv, batch, s_q, h_q, h_kv,
                       d_qk, d_v, page_size, scale, causal, num_splits, workspace,
                       workspace_bytes, o, lse, dtype,
                       dtype == SDPA_FP8_E4M3 ? descale_q : nullptr,
                       dtype == SDPA_FP8_E4M3 ? descale_k : nullptr,
                       dtype == SDPA_FP8_E4M3 ? descale_v : nullptr, stream,
                       /*use_scratch=*/false, window_left, sinks, stats_log2);
}

int sdpa_splitkv_combine(const float* o_part, const float* lse_part, int32_t num_splits,
                         int64_t rows, int32_t d_v, void* o, float* lse, int32_t dtype,
                         void* stream) {
    if (num_splits < 1 || num_splits > 256)
        return fail(SDPA_ERR_SHAPE, "num_splits=%d outside [1, 256]", num_splits);
    if (rows < 0 || rows >= kMaxCombineRows)
        return fail(SDPA_ERR_SHAPE, "rows=%lld outside [0, 2^26)", (long long)rows);
    if (d_v <= 0 || d_v > 1024) return fail(SDPA_ERR_SHAPE, "d_v=%d outside [1, 1024]", d_v);
    if (dtype != SDPA_BF16 && dtype != SDPA_FP32)
        return fail(SDPA_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
    if (rows == 0) return ok();
    if (!o_part || !lse_part || !o) return fail(SDPA_ERR_NULL, "o_part/lse_part/o must be non-NULL");
    if (!aligned(o_part, 4) || !aligned(lse_part, 4) || !aligned(o, dtype == SDPA_BF16 ? 2 : 4))
        return fail(SDPA_ERR_UNSUPPORTED, "misaligned pointer");
    hipError_t e = sdpa::launch_combine(o_part, lse_part, num_splits, rows, d_v, o, lse,
                                        dtype == SDPA_FP32 ? 1 : 0,
                                        static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    return ok();
}

}  // extern "C"
