/*
 * sdpa.h -- C-ABI of the MI355X (gfx950) fused scaled-dot-product-attention
 * forward library (libsdpa.so).
 *
 * Three operations, each a set of HIP kernels enqueued on the caller's stream:
 *   sdpa_prefill_thd      packed THD ragged prefill (causal or not), GQA,
 *                         FP32 natural-log LSE Stats, packed or padded rows;
 *   sdpa_decode_paged     paged-KV decode through independent K and V page
 *                         tables, split-KV partials merged by LSE;
 *   sdpa_splitkv_combine  the LSE merge of split partials on its own.
 *
 * Conventions shared by every entry point
 *   - Pointers named q/k/v/o/lse/cu_seqlens/page tables/seq_lens/workspace
 *     are DEVICE pointers; the caller owns every buffer.  The library never
 *     allocates device memory, never reads device memory on the host and
 *     never synchronizes the host (THD metadata is consumed on the device:
 *     cuDNN Frontend v1.28.0 release notes, "New: FROST SDPA on Ampere,
 *     Ada/Blackwell-consumer, and Rubin", paragraph "Ragged / THD, with zero
 *     host reads").
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  All
 *     work, including the -inf seeding of padded LSE rows, is enqueued on it
 *     in order.
 *   - Every extent and stride is a runtime argument; strides are in
 *     ELEMENTS and 64-bit (v1.30.0 Release Notes, "New: prepared launches --
 *     the execute fast path", int64 stride leaves).  The last (head-dim) axis
 *     of every tensor is contiguous.
 *   - All argument checks run before anything is enqueued.  On any error the
 *     call returns a nonzero sdpa_status_t, enqueues nothing, and
 *     sdpa_last_error_detail() (thread-local) says why.  Unsupported
 *     combinations are declined, never served with a silently different
 *     computation (v1.30.0 "New: decode tiles", Partial PackGQA bullet).
 *   - scale is always explicit; 0 and negative values are honoured
 *     (v1.31.0 Release Notes, "Compatibility and numerical behavior";
 *     v1.32.0 Release Notes, "SDPA: backward and numerical fixes").
 *   - LSE (softmax Stats) is always FP32 and natural-log: max + ln(sum exp)
 *     of the scaled logits (v1.28.0 "Updates to Graph API -- SDPA", Stats
 *     must be FP32; v1.30.0 "New: stats_use_log2 -- LSE in base 2").
 *     lse == NULL skips the Stats stores.
 *   - A query row with no visible key gets O = 0 and LSE = -inf (v1.32.0
 *     "New: Rubin triangle operations").
 *   - GQA: query head h reads KV head h / (h_q / h_kv); h_q % h_kv must be 0.
 *   - Causal masks are bottom-right aligned per sequence: query i of a
 *     sequence with Lq queries and Lk keys sees key j iff j <= i + Lk - Lq
 *     (v1.28.0 "New: FROST SDPA ...", per-sequence THD bottom-right
 *     diagonals).
 *   - Thread-safe.  Mutable global state: the thread-local error detail;
 *     the work-queue counters of the persistent prefill and decode grids
 *     (small static device arrays per GPU, 1024 slots each); and the
 *     library-owned split workspace of sdpa_decode_paged_noalloc.  Each
 *     launch takes the next slot with a launch tag of its own; a counter
 *     still carrying another launch's tag (left behind by a launch that
 *     never finished) is taken over rather than trusted, and a launch that
 *     finishes returns its slot to zero, so a replayed captured launch finds
 *     it free.  Up to 1024 prefill calls and 1024 decode calls may be in
 *     flight on one GPU at once (different streams); a 1025th concurrent
 *     call would share a slot with the first.
 */
#ifndef SDPA_MI355X_H
#define SDPA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SDPA_OK = 0,
    SDPA_ERR_NULL = 1,         /* a required pointer is NULL                        */
    SDPA_ERR_SHAPE = 2,        /* inconsistent or out-of-range extents / strides     */
    SDPA_ERR_UNSUPPORTED = 3,  /* valid request this build does not serve (declined) */
    SDPA_ERR_WORKSPACE = 4,    /* workspace missing or smaller than required         */
    SDPA_ERR_LSE_LAYOUT = 5,   /* unknown LSE layout or bad padded-row capacity      */
    SDPA_ERR_HIP = 6           /* a HIP launch failed                                */
} sdpa_status_t;

typedef enum {
    SDPA_BF16 = 0,     /* Q/K/V/O bfloat16, FP32 accumulation (MFMA)              */
    SDPA_FP32 = 1,     /* Q/K/V/O float32, FP32 arithmetic (VALU)                 */
    SDPA_FP8_E4M3 = 2  /* Q/K/V OCP E4M3 codes with per-tensor descales, O bf16;
                          sdpa_prefill_thd_fp8 / sdpa_decode_paged_fp8 only       */
} sdpa_dtype_t;

typedef enum {
    SDPA_LSE_NONE = 0,    /* no Stats written (lse may be NULL)                         */
    SDPA_LSE_PACKED = 1,  /* token-major packed rows: lse[(cu_seqlens_q[b] + i) * h_q + h] */
    SDPA_LSE_PADDED = 2,  /* per-batch padded rows: lse[(b * lse_s_max + i) * h_q + h];
                             the library first fills all batch*lse_s_max*h_q entries with
                             -inf on `stream`, so rows i >= Lq_b read -inf           */
    SDPA_LSE_HEAD_MAJOR = 3 /* head-major rows [h_q, total]: lse[h * lse_s_max +
                             cu_seqlens_q[b] + i]; lse_s_max is the per-head stride,
                             at least cu_seqlens_q[batch] (bf16 and FP8 prefill:
                             sdpa_prefill_thd, _ex, _fp8; v1.28.0 release notes, Bug
                             Fixes, head-major stats)                                */
} sdpa_lse_layout_t;

/*
 * Packed THD ragged prefill.
 *
 * Defines: for every sequence b, query row i in [0, Lq_b) and query head h,
 *   O[i,h,:] = softmax_j(scale * <Q[i,h,:], K[j,h/G,:]>) V[j,h/G,:] over the
 *   visible keys j, and LSE[i,h] = natural-log log-sum-exp of those logits.
 *   Packed THD layout (head dim innermost, then heads, then tokens; the batch
 *   stride is never read, every sequence base comes from the offset table):
 *   v1.30.0 Release Notes, "New: the FlashInfer serving path runs on FROST";
 *   prefix-sum offsets: v1.28.0 "New: FROST SDPA ...", THD paragraph.
 *
 * q  [Tq, h_q,  d_qk] at q + t*q_st + h*q_sh   (t = packed token row)
 * k  [Tk, h_kv, d_qk] at k + t*k_st + h*k_sh
 * v  [Tk, h_kv, d_v ] at v + t*v_st + h*v_sh
 * o  [Tq, h_q,  d_v ] at o + t*o_st + h*o_sh   (written for rows of real tokens only)
 * cu_seqlens_q / cu_seqlens_kv: int32 [batch+1] prefix sums on the device;
 *   sequence b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key
 *   rows cu_seqlens_kv[b] .. cu_seqlens_kv[b+1]-1.
 * max_seqlen_q / max_seqlen_kv: host-known upper bounds of Lq_b / Lk_b (they
 *   size the grid).  The grid covers ceil(max_seqlen_q / R) * R query rows of
 *   every sequence (R = 64 for bf16 d 64/128 and FP8, 32 for bf16 d 256, 1 for
 *   fp32); rows of a longer sequence past that are written as NaN (O and LSE),
 *   never left unwritten or partly computed.
 * causal: 0 or 1 (bottom-right).  lse_layout: sdpa_lse_layout_t; lse_s_max:
 *   padded row capacity (>= max_seqlen_q) for SDPA_LSE_PADDED, the per-head
 *   stride for SDPA_LSE_HEAD_MAJOR, else ignored.
 * dtype: SDPA_BF16 (d_qk == d_v in {64, 128, 256}; rows 16-byte aligned: base
 *   pointers 16-byte aligned and strides multiples of 8) or SDPA_FP32
 *   (d_qk, d_v <= 256; 4-byte aligned).
 * Reads of K/V stop at each sequence's Lk: unwritten capacity rows past the
 * last sequence are never read.
 */
int sdpa_prefill_thd(const void* q, int64_t q_st, int64_t q_sh,
                     const void* k, int64_t k_st, int64_t k_sh,
                     const void* v, int64_t v_st, int64_t v_sh,
                     void* o, int64_t o_st, int64_t o_sh,
                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, int32_t batch,
                     int32_t max_seqlen_q, int32_t max_seqlen_kv,
                     int32_t h_q, int32_t h_kv, int32_t d_qk, int32_t d_v,
                     float scale, int32_t causal,
                     float* lse, int32_t lse_layout, int32_t lse_s_max,
                     int32_t dtype, void* stream);

/*
 * Packed THD ragged prefill with the mask and Stats variants (bf16 only).
 * Same arguments and layouts as sdpa_prefill_thd, plus:
 * window_left: 0 = none; W > 0 = left sliding window: row i of sequence b
 *   sees only keys j >= i + Lk_b - Lq_b - W + 1 (the W keys ending at its
 *   bottom-right diagonal position when causal).  Left sliding windows:
 *   v1.32.0 Release Notes, "SDPA: backward and numerical fixes".  Negative
 *   values are rejected (SDPA_ERR_SHAPE).
 * sinks: NULL, or device fp32 [h_q] attention-sink logits, in the units of
 *   scale*<q,k>: head h's sink joins the softmax denominator of every row
 *   and carries no value, so O = sum_j e^{s_j} v_j / (sum_j e^{s_j} + e^{sink_h})
 *   and LSE = ln(sum_j e^{s_j} + e^{sink_h}); a row with no visible key gets
 *   O = 0, LSE = sink_h (sinks: v1.32.0 "SDPA: wider native forward support",
 *   v1.30.0 Release Notes, sinks with paged KV and sliding window; the pages
 *   print no formula, the denominator-only reading is taken).
 * stats_log2: 0 = natural-log LSE; 1 = base 2, LSE2 = max + log2(sum_exp) =
 *   LSE * log2(e) (v1.30.0 Release Notes, "New: stats_use_log2 -- LSE in
 *   base 2").
 */
int sdpa_prefill_thd_ex(const void* q, int64_t q_st, int64_t q_sh,
                        const void* k, int64_t k_st, int64_t k_sh,
                        const void* v, int64_t v_st, int64_t v_sh,
                        void* o, int64_t o_st, int64_t o_sh,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                        int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_kv,
                        int32_t h_q, int32_t h_kv, int32_t d_qk, int32_t d_v,
                        float scale, int32_t causal, int32_t window_left, const float* sinks,
                        float* lse, int32_t lse_layout, int32_t lse_s_max, int32_t stats_log2,
                        int32_t dtype, void* stream);

/*
 * Per-tensor FP8 (E4M3) packed THD ragged prefill: sdpa_prefill_thd_ex with
 * Q, K and V holding one-byte OCP E4M3 codes, each standing for its tensor's
 * descale times its value (per-tensor FP8 forward: v1.31.0 Release Notes,
 * SM100 per-tensor FP8 D128; the SM120 per-tensor FP8 (E4M3) forward engine;
 * v1.32.0 Known issues on negative descale_q * descale_k, which is served
 * here).  The pages print no scale formula; the per-tensor reading is taken:
 *   s_ij = scale * descale_q * descale_k * <q8_i, k8_j>,
 *   O_i  = descale_v * sum_j softmax_j(s_i) v8_j   (bf16),  LSE natural log
 *   (or base 2), with the window, sinks and Stats layouts of _ex.
 * descale_q / descale_k / descale_v: device pointers to one fp32 each, read by
 * the kernel.  Q/K/V strides count elements (= bytes); o is bf16 as in
 * sdpa_prefill_thd.
 * Supported: d_qk == d_v == 128; Q/K/V strides multiples of 16, O strides
 * multiples of 8; q/k/v/o 16-byte aligned.  Else SDPA_ERR_UNSUPPORTED.
 */
int sdpa_prefill_thd_fp8(const void* q, int64_t q_st, int64_t q_sh,
                         const void* k, int64_t k_st, int64_t k_sh,
                         const void* v, int64_t v_st, int64_t v_sh,
                         void* o, int64_t o_st, int64_t o_sh,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                         int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_kv,
                         int32_t h_q, int32_t h_kv, int32_t d_qk, int32_t d_v,
                         float scale, int32_t causal, int32_t window_left, const float* sinks,
                         float* lse, int32_t lse_layout, int32_t lse_s_max, int32_t stats_log2,
                         const float* descale_q, const float* descale_k,
                         const float* descale_v, void* stream);

/*
 * Bytes of caller workspace sdpa_decode_paged needs for these extents
 * (0 when num_splits == 1).  Caller-owned split workspace: v1.31.0 Release
 * Notes, "Compatibility and numerical behavior" (direct split-attention calls
 * require caller workspace; omission is rejected before launch).
 * Layout: o_part fp32 [num_splits, rows, d_v] at offset 0, then lse_part fp32
 * [num_splits, rows] at the next 256-byte boundary; rows = batch*s_q*h_q,
 * row = (b*s_q + t)*h_q + h.
 */
size_t sdpa_decode_workspace_bytes(int32_t batch, int32_t s_q, int32_t h_q, int32_t d_v,
                                   int32_t num_splits);

/*
 * The kernel a paged decode call with these extents runs on: sdpa_decode_paged
 * (and _ex, _noalloc) for dtype SDPA_BF16, sdpa_decode_paged_fp8 for
 * SDPA_FP8_E4M3.  Host-only; reads no memory and makes no GPU call.  Returns
 * one of SDPA_PATH_*, or 0 when those entry points decline the extents (the
 * checks made here: dtype, head counts, (d_qk, d_v), page_size, num_splits,
 * row strides, the 512-row limit; pointers, alignment, page-table and
 * length arguments are checked only by the entry points themselves).
 */
enum {
    SDPA_PATH_FEW_ROW = 1,         /* few-row streaming kernel, one 16-row group     */
    SDPA_PATH_ROW_GROUPS = 2,      /* few-row kernel, 16-row groups (up to 64 rows)  */
    SDPA_PATH_PREFILL = 3,         /* prefill kernel over the page tables            */
    SDPA_PATH_PREFILL_FOLDED = 4,  /* the same with (token, head) rows folded        */
    SDPA_PATH_WIDE = 5,            /* absorbed-MLA 576/512 MFMA kernel               */
    SDPA_PATH_GENERAL = 6          /* general decode kernel                          */
};
int sdpa_decode_path(int32_t batch, int32_t s_q, int32_t h_q, int32_t h_kv, int32_t d_qk,
                     int32_t d_v, int32_t page_size, int64_t k_st, int64_t v_st,
                     int32_t num_splits, int32_t dtype);

/*
 * Paged-KV decode with split-KV.
 *
 * Defines: query token t of sequence b sits at key position seq_lens[b]-s_q+t
 * and, per head h, attends to keys j of that sequence (all j < seq_lens[b],
 * or j <= seq_lens[b]-s_q+t when causal).  Logical key j lives in physical
 * page page_table_k[b*table_stride + j/page_size] of the K pool (and
 * page_table_v[...] of the V pool) at slot j % page_size: independent K and
 * V page tables and pools (v1.31.0 "SDPA: paged KV, split-KV, and engine
 * selection"; v1.32.0 "SDPA: wider native forward support", Q/K 576 with
 * V 512 and independent K/V tables and layouts).
 * The keys of each (b, KV head) are cut into num_splits contiguous chunks of
 * ceil(ceil(L/S)/page_size)*page_size keys; each chunk's normalized partial
 * (O_c, LSE_c) goes to the workspace and a second kernel merges them by LSE
 * (sdpa_splitkv_combine).  One exception: with (d_qk, d_v) = (576, 512) and
 * more than 16 query rows per KV head, when the chunks would give the GPU more
 * than two work-groups per compute unit, m = floor(batch * h_kv * num_splits *
 * ceil(rows / 128) / (2 * CUs)) adjacent chunks share one work-group: slot
 * c * m holds the partial of chunks c*m .. c*m+m-1 together and the group's
 * other slots are empty partials (LSE -inf, O not written).  The merge of all
 * num_splits slots is the same attention either way ("fewer, longer splits").  num_splits == 1 writes O/LSE directly and needs
 * no workspace.  seq_lens need not be multiples of anything (v1.30.0 "New:
 * the FlashInfer serving path ...", split-KV kept for non-128-multiple KV max).
 *
 * q       [batch, s_q, h_q, d_qk] dense, bf16.
 * k_pool  K rows at k_pool + page*k_sp + slot*k_st + head*k_sh, d_qk wide.
 * v_pool  V rows at v_pool + page*v_sp + slot*v_st + head*v_sh, d_v wide
 *         (K and V pools may alias).  Token rows of one page must not
 *         overlap (k_st >= d_qk, v_st >= d_v) and k_st, v_st < 2^26.
 * page_table_k / page_table_v: int32 [batch, table_stride]; entries past a
 *         sequence's last page are never read.
 * seq_lens int32 [batch]; max_seqlen_kv: host-known upper bound (must be
 *         <= table_stride*page_size).  A seq_lens[b] beyond the table's reach
 *         (table_stride*page_size keys) cannot be computed: the table is read
 *         only within its reach and every output row of sequence b is NaN (O
 *         and LSE; its split partials too, and the merge propagates them).
 * o       [batch, s_q, h_q, d_v] dense bf16; lse [batch, s_q, h_q] fp32 or NULL.
 * Supported: dtype SDPA_BF16; (d_qk, d_v) in {(64,64), (128,128), (256,256),
 * (192,128), (576,512)}; page_size a multiple of 16; 1 <= num_splits <= 256;
 * s_q * (h_q/h_kv) <= 512 query rows per KV head, or any larger s_q when
 * d_qk = d_v is 64, 128 or 256 and k_st, v_st < 2^22, or with (576, 512).
 *
 * Chunked prefill over the paged cache is this same call with s_q = the
 * chunk's tokens (the last s_q of each cache; v1.31.0 "SDPA: paged KV,
 * split-KV, and engine selection", paged D128 prefill and chunked-prefill
 * selection; the context phase of v1.28.0 "Samples, Benchmarks, and Tests",
 * 512/1024-token chunks against 64k/128k caches).  With d_qk = d_v = 128,
 * k_st, v_st < 2^22 and s_q of at least one prefill work item (64 tokens when
 * h_q/h_kv is a multiple of 4, 128 when it is 2 mod 4, 256 when odd) it runs
 * on the prefill kernel, which reads its 64-key K/V tiles through the page
 * tables (each wave its 8 rows from the page that holds them, so any page
 * size serves); num_splits > 1 then writes the same partials as decode.
 * d_qk = d_v = 256 likewise runs on the D = 256 prefill kernel (32-key tiles,
 * items of 32, 64 or 128 tokens), and d_qk = d_v = 64 on the D = 64 one.  With fewer tokens and more than 16 query rows per KV head
 * (s_q * h_q/h_kv, e.g. multi-token decode over a wide GQA group), the same
 * kernel takes the call with the (token, head) rows of each KV head's group
 * folded, token-major, into its 256-row items.
 */
int sdpa_decode_paged(const void* q,
                      const void* k_pool, int64_t k_sp, int64_t k_st, int64_t k_sh,
                      const void* v_pool, int64_t v_sp, int64_t v_st, int64_t v_sh,
                      const int32_t* page_table_k, const int32_t* page_table_v,
                      int32_t table_stride, const int32_t* seq_lens, int32_t max_seqlen_kv,
                      int32_t batch, int32_t s_q, int32_t h_q, int32_t h_kv,
                      int32_t d_qk, int32_t d_v, int32_t page_size,
                      float scale, int32_t causal, int32_t num_splits,
                      void* workspace, size_t workspace_bytes,
                      void* o, float* lse, int32_t dtype, void* stream);

/*
 * Per-tensor FP8 (E4M3) paged decode: sdpa_decode_paged with Q, the K pool and
 * the V pool holding one-byte OCP E4M3 codes (sign, 4 exponent bits biased by
 * 7, 3 mantissa bits, S.1111.111 the only NaN), each standing for its tensor's
 * descale times its value.  Per-tensor FP8 paged KV: v1.31.0 Release Notes,
 * paged KV (SM100 per-tensor FP8 D128); v1.32.0 "SDPA: wider native forward
 * support" (paged per-tensor FP8 D256); the pages print no scale formula, the
 * per-tensor reading is taken:
 *   s_tj = scale * descale_q * descale_k * <q8_t, k8_j>,
 *   O_t  = descale_v * sum_j softmax_j(s_t) v8_j   (bf16),  LSE natural log.
 * descale_q / descale_k / descale_v: device pointers to one fp32 each, read by
 * the kernel (so a captured launch picks up new values).  Strides count
 * elements (= bytes).  Other arguments, the split workspace and its layout
 * are those of sdpa_decode_paged.
 * Supported: the (d_qk, d_v) pairs of sdpa_decode_paged ({64, 128, 256} square,
 * (192,128), (576,512); native D64 per-tensor FP8 and Q/K 576 with V 512 are
 * in v1.32.0 "SDPA: wider native forward support"); s_q * (h_q/h_kv) <= 512
 * query rows per KV head, or any larger s_q when d_qk = d_v = 128, page_size
 * and k_st, v_st < 2^22 (the FP8 chunked-prefill path);
 * page_size a multiple of 16; K and V pool strides multiples of 16; q and the
 * pools 16-byte aligned.  Else SDPA_ERR_UNSUPPORTED.
 * Kernels: up to 32 rows per KV head (and up to 64 off the next path) at
 * d = 64, 128, 256 or 192/128, the FP8-MFMA few-row kernel in groups of 16
 * rows.  Past 32 rows at d_qk = d_v = 128, the FP8
 * prefill kernel over the page tables (FP8 MFMA for Q K^T, V codes widened
 * to bf16 in LDS), either for s_q of at least one work item or, with fewer
 * tokens, with the (token, head) rows of each KV head's group folded into
 * its 256-row items.  (576, 512), any page size: the absorbed-MLA
 * wide kernel, its tiles DMA'd as codes, Q K^T on the FP8 MFMA and V widened
 * exactly to bf16 in LDS for a bf16 P V.
 * The rest widen the codes exactly to bf16 as they are loaded and use bf16
 * MFMA.
 */
int sdpa_decode_paged_fp8(const void* q,
                          const void* k_pool, int64_t k_sp, int64_t k_st, int64_t k_sh,
                          const void* v_pool, int64_t v_sp, int64_t v_st, int64_t v_sh,
                          const int32_t* page_table_k, const int32_t* page_table_v,
                          int32_t table_stride, const int32_t* seq_lens, int32_t max_seqlen_kv,
                          int32_t batch, int32_t s_q, int32_t h_q, int32_t h_kv,
                          int32_t d_qk, int32_t d_v, int32_t page_size,
                          float scale, int32_t causal, int32_t num_splits,
                          void* workspace, size_t workspace_bytes,
                          const float* descale_q, const float* descale_k,
                          const float* descale_v, void* o, float* lse, void* stream);

/*
 * Paged-KV decode with the mask and Stats variants: sdpa_decode_paged (dtype
 * SDPA_BF16) or sdpa_decode_paged_fp8 (dtype SDPA_FP8_E4M3, descales as
 * there; NULL for bf16) plus:
 * window_left: 0 = none; W > 0 = left sliding window: query token t of
 *   sequence b (at key position seq_lens[b] - s_q + t) sees only keys
 *   j >= seq_lens[b] - s_q + t - W + 1, the W keys ending at its own position
 *   when causal (left sliding windows: v1.32.0 Release Notes, "SDPA: backward
 *   and numerical fixes"; decode with a sliding window: v1.30.0 Release Notes,
 *   "New: decode tiles").  Negative values are rejected (SDPA_ERR_SHAPE).
 *   With num_splits > 1 the keys cut into chunks start at the page holding
 *   the first key any token of the sequence sees, so no chunk is spent on
 *   keys outside every window.
 * sinks: NULL, or device fp32 [h_q] attention-sink logits in the units of the
 *   scaled logits: head h's sink joins every row's softmax denominator once
 *   and carries no value (as in sdpa_prefill_thd_ex); a row with no visible
 *   key gets O = 0 and LSE = sink_h.  With num_splits > 1 the partials carry
 *   no sink and the merge adds it (sinks at S_q == 1 with paged KV and a
 *   sliding window: v1.30.0 "New: decode tiles"; split-KV and paged FP8 with
 *   sinks: v1.32.0 "SDPA: wider native forward support").
 * stats_log2: 0 = natural-log LSE; 1 = base 2 (v1.30.0 "New: stats_use_log2").
 *   The split workspace partials stay natural-log.
 * Supported shapes are those of sdpa_decode_paged (bf16) or
 * sdpa_decode_paged_fp8 (FP8), every variant with each of them.
 */
int sdpa_decode_paged_ex(const void* q,
                         const void* k_pool, int64_t k_sp, int64_t k_st, int64_t k_sh,
                         const void* v_pool, int64_t v_sp, int64_t v_st, int64_t v_sh,
                         const int32_t* page_table_k, const int32_t* page_table_v,
                         int32_t table_stride, const int32_t* seq_lens, int32_t max_seqlen_kv,
                         int32_t batch, int32_t s_q, int32_t h_q, int32_t h_kv,
                         int32_t d_qk, int32_t d_v, int32_t page_size,
                         float scale, int32_t causal, int32_t window_left, const float* sinks,
                         int32_t stats_log2, int32_t num_splits,
                         void* workspace, size_t workspace_bytes,
                         const float* descale_q, const float* descale_k, const float* descale_v,
                         void* o, float* lse, int32_t dtype, void* stream);

/*
 * sdpa_decode_paged for callers that cannot allocate device memory around a
 * call (code under stream capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, results and kernels, without the workspace
 * arguments.  The split partials go to a library-owned device array of
 * 32 MiB per GPU (each GPU the library runs on holds it until the process
 * ends); a call whose split workspace (sdpa_decode_workspace_bytes) exceeds
 * it is declined with SDPA_ERR_WORKSPACE before anything is enqueued.  The
 * array's device address on the current device is looked up on the first
 * call on that device (no allocation); a failed lookup returns SDPA_ERR_HIP.
 * The call allocates nothing.  All calls on one GPU share the array and it
 * keeps the last call's contents (nothing needs clearing: every partial the
 * combine reads is written first), so calls that overlap on one GPU, on
 * different streams, race on it and must not be issued.
 * dtype: SDPA_BF16 only.
 */
int sdpa_decode_paged_noalloc(const void* q,
                              const void* k_pool, int64_t k_sp, int64_t k_st, int64_t k_sh,
                              const void* v_pool, int64_t v_sp, int64_t v_st, int64_t v_sh,
                              const int32_t* page_table_k, const int32_t* page_table_v,
                              int32_t table_stride, const int32_t* seq_lens,
                              int32_t max_seqlen_kv, int32_t batch, int32_t s_q, int32_t h_q,
                              int32_t h_kv, int32_t d_qk, int32_t d_v, int32_t page_size,
                              float scale, int32_t causal, int32_t num_splits,
                              void* o, float* lse, int32_t dtype, void* stream);

/*
 * LSE merge of split-KV partials: the second step of split-KV (cuDNN Frontend
 * v1.31.0 Release Notes, "SDPA: paged KV, split-KV, and engine selection";
 * v1.32.0 "SDPA: wider native forward support", split-KV with sinks).  The
 * notes use the merge but never print it; the textbook log-sum-exp merge is
 * taken:
 *   M = max_c lse_part[c,r];  LSE[r] = M + ln sum_c exp(lse_part[c,r] - M);
 *   O[r,:] = sum_c exp(lse_part[c,r] - LSE[r]) * o_part[c,r,:];
 *   every split empty (-inf) -> O[r,:] = 0, LSE[r] = -inf;
 *   any lse_part[c,r] NaN (a split that could not be computed) -> O[r,:] and
 *   LSE[r] NaN.
 * o_part fp32 [num_splits, rows, d_v] (each partial already normalized),
 * lse_part fp32 [num_splits, rows] natural log; o [rows, d_v] in `dtype`
 * (SDPA_BF16 or SDPA_FP32); lse fp32 [rows] or NULL.  d_v <= 1024.
 */
int sdpa_splitkv_combine(const float* o_part, const float* lse_part, int32_t num_splits,
                         int64_t rows, int32_t d_v, void* o, float* lse, int32_t dtype,
                         void* stream);

/* Static description of a status code. */
const char* sdpa_status_string(int status);

/* Detail of the last error returned on this thread ("" if none). */
const char* sdpa_last_error_detail(void);

/* Library version, major*10000 + minor*100 + patch. */
int sdpa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_MI355X_H */
