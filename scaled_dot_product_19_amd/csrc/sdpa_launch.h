// sdpa_launch.h -- internal host-side launcher interface between the C-ABI
// layer (sdpa_api.cpp) and the kernel translation units.  Arguments arrive
// here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

struct PrefillArgs {
    const void* q;
    int64_t q_st, q_sh;
    const void* k;
    int64_t k_st, k_sh;
    const void* v;
    int64_t v_st, v_sh;
    void* o;
    int64_t o_st, o_sh;
    const int32_t* cu_q;
    const int32_t* cu_kv;
    int32_t batch, max_q, max_kv;
    int32_t hq, hkv, dqk, dv;
    float scale;
    int32_t causal;
    float* lse;
    int32_t lse_layout, lse_s_max;  // layout 3 (head-major): lse_s_max = per-head stride
    int32_t window;                 // left sliding window (<= 0: none)
    const float* sinks;             // [hq] sink logits or nullptr
    int32_t stats_log2;             // LSE in base 2
    int32_t fp8;                    // Q/K/V are E4M3 codes (per-tensor descales below)
    const float* descale_q;
    const float* descale_k;
    const float* descale_v;
};

struct DecodeArgs {
    const void* q;
    const void* k_pool;
    int64_t k_sp, k_st, k_sh;
    const void* v_pool;
    int64_t v_sp, v_st, v_sh;
    const int32_t* pt_k;
    const int32_t* pt_v;
    int32_t table_stride;
    const int32_t* seq_lens;
    int32_t batch, sq, hq, hkv, dqk, dv, page;
    float scale;
    int32_t causal, splits;
    float* o_part;    // [splits, rows, dv] when splits > 1
    float* lse_part;  // [splits, rows]
    void* o;          // final output when splits == 1
    float* lse;
    int32_t fp8;      // Q/K/V are E4M3 codes (per-tensor descales below)
    const float* descale_q;
    const float* descale_k;
    const float* descale_v;
    int32_t window;       // left sliding window (<= 0: none)
    const float* sinks;   // [hq] sink logits or nullptr (folded once: in the combine when split)
    int32_t stats_log2;   // final LSE in base 2 (split partials stay natural-log)
};

// Each returns hipSuccess or the launch error.
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s);
// per-tensor FP8: the few-row kernel up to 32 rows per KV head, the FP8 paged
// prefill kernel (D = 128), the absorbed-MLA wide kernel (576/512), the few-row
// kernel up to 64 rows, else the general kernel
hipError_t launch_decode_fp8(const DecodeArgs& a, hipStream_t s);
// The kernel both decode launchers pick for a call (values as SDPA_PATH_* in sdpa.h).
enum class DecodePath : int32_t {
    kFewRow = 1, kRowGroups = 2, kPrefill = 3, kPrefillFolded = 4, kWide = 5, kGeneral = 6
};
DecodePath decode_path(const DecodeArgs& a);
// The paged prefill kernel would fold the call's (token, head) rows.
bool prefill_paged_folds(const DecodeArgs& d);
// sinks (optional): [hq] sink logits merged once per row (row % hq is its head);
// stats_log2: write the merged LSE in base 2.
hipError_t launch_combine(const float* o_part, const float* lse_part, int32_t splits,
                          int64_t rows, int32_t dv, void* o, float* lse, int32_t out_f32,
                          hipStream_t s, const float* sinks = nullptr, int32_t hq = 1,
                          int32_t stats_log2 = 0);
hipError_t launch_fill_neg_inf(float* p, int64_t n, hipStream_t s);

// Library-owned split workspace of sdpa_decode_paged_noalloc: bytes per GPU,
// and its device address on the current device (looked up once per device).
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
hipError_t decode_scratch(void** ptr);

// Decode row-group geometry shared by the launcher and the workspace query.
bool decode_supported(int32_t dqk, int32_t dv);

// Few-row decode (s_q * G <= 16 query rows per KV head, d_qk == d_v in
// {64, 128, 256}): the HBM-streaming kernel of decode_small.hip.
// query rows per KV head the few-row decode kernel serves (in groups of 16)
constexpr int kSmallRowsMax = 64;
bool decode_small_supported(int32_t dqk, int32_t dv, int32_t rows);
hipError_t launch_decode_small(const DecodeArgs& a, hipStream_t s);

// The prefill kernels over the paged cache (d_qk = d_v = 64, 128 or 256; s_q
// of at least one work item, or folded rows past 16 per KV head): K/V tiles
// addressed through the page tables, each wave's 8 rows from its own page.
bool prefill_paged_supported(const DecodeArgs& a);
hipError_t launch_prefill_paged(const DecodeArgs& a, hipStream_t s);

// Absorbed-MLA decode (d_qk = 576, d_v = 512, any page size, any
// number of query rows per KV head): the MFMA kernel of decode_wide.hip.
bool decode_wide_supported(const DecodeArgs& a);
hipError_t launch_decode_wide(const DecodeArgs& a, hipStream_t s);

}  // namespace sdpa
