/*
 * sdpa_oracle.c -- plain, slow, fp64 CPU definition of the fused
 * scaled-dot-product-attention (SDPA) forward.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness oracle for the HIP
 * library.  Only the test suite, the smoke entry point and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header, table or helper
 * with the GPU path, and the GPU path never calls it.
 *
 * What it computes (the plain definition; the fused online-softmax method
 * reaches the same value up to rounding order):
 *
 *   For a query row q_i (head h) and the keys k_j / values v_j of KV head
 *   kvh = h / G, G = Hq / Hkv:
 *     s_ij   = scale * <q_i, k_j>                         (fp64)
 *     V_i    = { j : j < Lk  and (not causal or j <= i + Lk - Lq)
 *                     and (W <= 0 or j >= i + Lk - Lq - W + 1) }
 *     m      = max of { s_ij : j in V_i } and, with a sink, sink_h
 *     l      = sum_{j in V_i} exp(s_ij - m)  [+ exp(sink_h - m)]
 *     O_i    = sum_{j in V_i} exp(s_ij - m) * v_j / l
 *     LSE_i  = m + ln(l)                                   (natural log)
 *     V_i empty and no sink  ->  O_i = 0, LSE_i = -inf.
 *   W is the left sliding window (prefill only): a row sees at most the W
 *   keys that end at its bottom-right diagonal position.  sink_h is a
 *   per-head logit in the units of s_ij that joins the softmax denominator
 *   and carries no value.
 *
 * Passages followed:
 *   - natural-log FP32 Stats "max + ln(sum_exp)": cuDNN Frontend v1.30.0
 *     Release Notes, "New: stats_use_log2 -- LSE in base 2"; Stats are FP32:
 *     v1.28.0 release notes, "Updates to Graph API -- SDPA".
 *   - bottom-right causal diagonal per THD sequence: v1.28.0 release notes,
 *     "New: FROST SDPA on Ampere, Ada/Blackwell-consumer, and Rubin"
 *     (paragraph "Masking, splitting, and heuristics"), and the bottom-right
 *     causal context benchmark in "Samples, Benchmarks, and Tests".
 *   - packed THD addressing (head dim innermost, then heads, then tokens;
 *     every sequence base from the offset table): v1.30.0 Release Notes,
 *     "New: the FlashInfer serving path runs on FROST".
 *   - GQA group G = H_q / H_kv: v1.30.0 Release Notes, "New: decode tiles"
 *     (Partial PackGQA bullet).  Reading taken: q head h uses KV head h / G.
 *   - rows with no live key give O = 0 and LSE = -inf: v1.32.0 Release
 *     Notes, "New: Rubin triangle operations".
 *   - explicit scale, zero preserved: v1.31.0 Release Notes, "Compatibility
 *     and numerical behavior".
 *   - paged K/V with independent K and V page tables, Q/K 576 with V 512:
 *     v1.31.0 Release Notes, "SDPA: paged KV, split-KV, and engine
 *     selection"; v1.32.0 Release Notes, "SDPA: wider native forward support".
 *   - split-KV partials merged by LSE: v1.31.0 "SDPA: paged KV, split-KV, and
 *     engine selection"; the merge formula is not printed on the pages, the
 *     textbook log-sum-exp merge is taken (oracle_combine below).
 *   - left sliding windows: v1.32.0 Release Notes, "SDPA: backward and
 *     numerical fixes" (left sliding windows for dense D64/D128); attention
 *     sinks: v1.32.0 "SDPA: wider native forward support" (masks, sinks) and
 *     v1.30.0 Release Notes (sinks at S_q == 1 with paged KV and sliding
 *     window).  The pages print no formula for either; the readings taken
 *     are the ones stated above (window counted from the diagonal key
 *     inclusive; sink = an extra logit in the denominator only).
 *
 *   - per-tensor FP8 (E4M3) forward and paged KV: v1.31.0 Release Notes,
 *     paged KV (per-tensor FP8 D128 paged KV); v1.32.0 "SDPA: wider native
 *     forward support" (paged per-tensor FP8 D256); the SM120 per-tensor FP8
 *     (E4M3) forward engine; v1.32.0 Known issues (descale_q * descale_k).
 *     The pages print no scale formula; the reading taken is the per-tensor
 *     one: each stored code x8 stands for descale_x * E4M3(x8), so
 *     s_ij = scale * descale_q * descale_k * <q8_i, k8_j> and the values are
 *     descale_v * v8_j.  E4M3 is the OCP 8-bit format (sign, 4 exponent bits
 *     with bias 7, 3 mantissa bits, subnormals at exponent 0, S.1111.111 the
 *     only NaN, no infinities).
 *
 * Inputs are read as bf16 (raw 16-bit patterns, widened exactly: a bf16 is
 * the top half of an IEEE binary32), as fp32, or as E4M3 codes, then
 * widened to double (every E4M3 value is exact in double, and so is its
 * product with an fp32 descale).
 * Nothing is ever rounded on the oracle side.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_BF16 0
#define ORACLE_F32 1
#define ORACLE_E4M3 2

/* ---- element access ---------------------------------------------------- */

/* OCP E4M3 code -> value: (-1)^s * 2^(e-7) * (1 + m/8) for e = 1..15,
   (-1)^s * 2^-6 * (m/8) for e = 0; e = 15 with m = 7 is NaN. */
double oracle_e4m3_value(uint8_t code) {
    int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double v = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

static double load_elem(const void* base, int dtype, int64_t idx) {
    if (dtype == ORACLE_F32) return (double)((const float*)base)[idx];
    if (dtype == ORACLE_E4M3) return oracle_e4m3_value(((const uint8_t*)base)[idx]);
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* ---- the definition, for one query row ---------------------------------
 * q: the query row (already widened), dqk long.
 * koff/voff: element offsets of the n visible key / value rows.
 * s: scratch of n doubles.  p_out (optional): the n softmax weights.
 * kscale / vscale: per-tensor descales of the stored K and V codes (1 for
 * bf16 and fp32 inputs).
 */
static void attend_row(const double* q, int dqk, int dv, const void* k, const void* v,
                       const int64_t* koff, const int64_t* voff, int64_t n, int dtype,
                       double kscale, double vscale, double scale, double sink, double* s,
                       double* o, double* lse, double* p_out) {
    /* sink = -inf: no sink */
    if (n == 0 && sink == -INFINITY) {
        for (int d = 0; d < dv; ++d) o[d] = 0.0;
        *lse = -INFINITY;
        return;
    }
    double m = sink;
    for (int64_t j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int d = 0; d < dqk; ++d) dot += q[d] * (kscale * load_elem(k, dtype, koff[j] + d));
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
    }
    double l = sink == -INFINITY ? 0.0 : exp(sink - m);
    for (int64_t j = 0; j < n; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    for (int d = 0; d < dv; ++d) o[d] = 0.0;
    for (int64_t j = 0; j < n; ++j)
        for (int d = 0; d < dv; ++d) o[d] += s[j] * (vscale * load_elem(v, dtype, voff[j] + d));
    for (int d = 0; d < dv; ++d) o[d] /= l;
    *lse = m + log(l);
    if (p_out)
        for (int64_t j = 0; j < n; ++j) p_out[j] = s[j] / l;
}

/* ---- a minimal thread pool over independent row units ------------------ */

typedef void (*unit_fn)(void* ctx, int64_t unit, double* scratch);

typedef struct {
    unit_fn fn;
    void* ctx;
    int64_t n_units;
    int64_t next;
    size_t scratch_len;
    pthread_mutex_t lock;
} pool_t;

static void* pool_worker(void* arg) {
    pool_t* p = (pool_t*)arg;
    double* scratch = (double*)malloc((p->scratch_len ? p->scratch_len : 1) * sizeof(double));
    if (!scratch) return (void*)1;
    for (;;) {
        pthread_mutex_lock(&p->lock);
        int64_t u = p->next++;
        pthread_mutex_unlock(&p->lock);
        if (u >= p->n_units) break;
        p->fn(p->ctx, u, scratch);
    }
    free(scratch);
    return NULL;
}

static int run_pool(unit_fn fn, void* ctx, int64_t n_units, size_t scratch_len, int nthreads) {
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > n_units) nthreads = n_units > 0 ? (int)n_units : 1;
    pool_t p = {fn, ctx, n_units, 0, scratch_len, PTHREAD_MUTEX_INITIALIZER};
    pthread_t th[256];
    int started = 0, rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, pool_worker, &p) != 0) { rc = -1; break; }
        ++started;
    }
    for (int t = 0; t < started; ++t) {
        void* ret = NULL;
        pthread_join(th[t], &ret);
        if (ret) rc = -1;
    }
    return rc;
}

int oracle_nproc(void) { return (int)sysconf(_SC_NPROCESSORS_ONLN); }

/* ---- packed THD ragged prefill ------------------------------------------ */

typedef struct {
    int dtype;
    const void *q, *k, *v;
    int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh;
    const int32_t *cu_q, *cu_kv;
    int32_t batch, hq, hkv, dqk, dv, causal;
    double scale;
    int64_t n_sel;
    const int64_t* sel_tok;
    const int32_t* sel_head;
    double *o, *lse, *p_out;
    int64_t max_lk;
    int32_t window;        /* left window W (<= 0: none) */
    const double* sinks;   /* [hq] sink logits, or NULL */
    double q_descale, k_descale, v_descale;  /* per-tensor descales (1 unless E4M3) */
} prefill_ctx;

/* Sequence b that owns packed query row t: cu_q[b] <= t < cu_q[b+1]. */
static int32_t owner_seq(const int32_t* cu, int32_t batch, int64_t t) {
    for (int32_t b = 0; b < batch; ++b)
        if (t >= cu[b] && t < cu[b + 1]) return b;
    return -1;
}

static void prefill_unit(void* vctx, int64_t unit, double* scratch) {
    prefill_ctx* c = (prefill_ctx*)vctx;
    int64_t t;
    int32_t h;
    if (c->n_sel < 0) {
        t = unit / c->hq;
        h = (int32_t)(unit % c->hq);
    } else {
        t = c->sel_tok[unit];
        h = c->sel_head[unit];
    }
    double* o = c->o + unit * c->dv;
    double* lse = c->lse + unit;
    int32_t b = owner_seq(c->cu_q, c->batch, t);
    if (b < 0) {  /* a row outside every sequence: nothing attends */
        for (int d = 0; d < c->dv; ++d) o[d] = 0.0;
        *lse = -INFINITY;
        return;
    }
    int64_t i = t - c->cu_q[b];
    int64_t lq = c->cu_q[b + 1] - c->cu_q[b];
    int64_t lk = c->cu_kv[b + 1] - c->cu_kv[b];
    int32_t kvh = h / (c->hq / c->hkv);
    /* visible keys j0 <= j < j1: j < lk; j <= i + lk - lq when causal;
       j >= i + lk - lq - W + 1 with a left window W */
    const int64_t diag = i + lk - lq;  /* the row's bottom-right diagonal key */
    int64_t j1 = lk;
    if (c->causal && diag + 1 < j1) j1 = diag + 1;
    int64_t j0 = 0;
    if (c->window > 0 && diag - c->window + 1 > j0) j0 = diag - c->window + 1;
    int64_t n = j1 > j0 ? j1 - j0 : 0;
    double* qrow = scratch;
    int64_t* koff = (int64_t*)(scratch + c->dqk);
    int64_t* voff = koff + c->max_lk;
    double* s = (double*)(voff + c->max_lk);
    for (int d = 0; d < c->dqk; ++d)
        qrow[d] = c->q_descale * load_elem(c->q, c->dtype, t * c->q_st + (int64_t)h * c->q_sh + d);
    for (int64_t j = 0; j < n; ++j) {
        koff[j] = (c->cu_kv[b] + j0 + j) * c->k_st + (int64_t)kvh * c->k_sh;
        voff[j] = (c->cu_kv[b] + j0 + j) * c->v_st + (int64_t)kvh * c->v_sh;
    }
    double* p_out = NULL;
    double* p_row = NULL;
    if (c->p_out) { /* probabilities for every key of the sequence, 0 when masked */
        p_out = c->p_out + unit * c->max_lk;
        for (int64_t j = 0; j < c->max_lk; ++j) p_out[j] = 0.0;
        p_row = p_out + j0;
    }
    const double sink = c->sinks ? c->sinks[h] : -INFINITY;
    attend_row(qrow, c->dqk, c->dv, c->k, c->v, koff, voff, n, c->dtype, c->k_descale,
               c->v_descale, c->scale, sink, s, o, lse, p_row);
}

/*
 * Packed THD prefill.  Q [Tq, Hq, Dqk], K [Tk, Hkv, Dqk], V [Tk, Hkv, Dv]
 * with element strides (token, head); D innermost and contiguous.
 * Sequence b holds query rows cu_q[b]..cu_q[b+1]-1 and key rows
 * cu_kv[b]..cu_kv[b+1]-1.
 *
 * n_sel < 0: every (token, head) row; o is [Tq*Hq, Dv] (row t*Hq + h), lse
 * [Tq*Hq].  n_sel >= 0: only the listed rows (sel_tok[r], sel_head[r]); o is
 * [n_sel, Dv], lse [n_sel].  p_out (optional, may be NULL) receives, per
 * computed row, max_lk softmax weights (key index j of the row's sequence).
 * window > 0 is the left sliding window W; sinks (optional) holds Hq sink
 * logits.  dtype ORACLE_E4M3: Q, K and V are E4M3 codes standing for
 * descale_q/k/v times their values (per-tensor FP8); other dtypes take
 * descales of 1.  Returns 0, or -1 on a bad argument / failed allocation.
 */
int oracle_prefill_thd_scaled(int dtype, const void* q, int64_t q_st, int64_t q_sh,
                              const void* k, int64_t k_st, int64_t k_sh, const void* v,
                              int64_t v_st, int64_t v_sh, const int32_t* cu_q,
                              const int32_t* cu_kv, int32_t batch, int32_t hq, int32_t hkv,
                              int32_t dqk, int32_t dv, double scale, int32_t causal,
                              int32_t window, const double* sinks, double descale_q,
                              double descale_k, double descale_v, int64_t n_sel,
                              const int64_t* sel_tok, const int32_t* sel_head, double* o,
                              double* lse, double* p_out, int32_t nthreads) {
    if (batch < 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0 || dqk <= 0 || dv <= 0) return -1;
    int64_t max_lk = 1;
    for (int32_t b = 0; b < batch; ++b) {
        int64_t lk = cu_kv[b + 1] - cu_kv[b];
        if (lk < 0 || cu_q[b + 1] < cu_q[b]) return -1;
        if (lk > max_lk) max_lk = lk;
    }
    prefill_ctx c = {dtype, q, k, v, q_st, q_sh, k_st, k_sh, v_st, v_sh, cu_q, cu_kv, batch,
                     hq, hkv, dqk, dv, causal, scale, n_sel, sel_tok, sel_head, o, lse, p_out,
                     max_lk, window, sinks, descale_q, descale_k, descale_v};
    int64_t tq = batch > 0 ? cu_q[batch] : 0;
    int64_t n_units = n_sel < 0 ? tq * hq : n_sel;
    size_t scratch = (size_t)dqk + 3 * (size_t)max_lk;
    return run_pool(prefill_unit, &c, n_units, scratch, nthreads);
}

/* bf16 / fp32 prefill: the same definition with descales of 1. */
int oracle_prefill_thd(int dtype, const void* q, int64_t q_st, int64_t q_sh, const void* k,
                       int64_t k_st, int64_t k_sh, const void* v, int64_t v_st, int64_t v_sh,
                       const int32_t* cu_q, const int32_t* cu_kv, int32_t batch, int32_t hq,
                       int32_t hkv, int32_t dqk, int32_t dv, double scale, int32_t causal,
                       int32_t window, const double* sinks, int64_t n_sel,
                       const int64_t* sel_tok, const int32_t* sel_head, double* o, double* lse,
                       double* p_out, int32_t nthreads) {
    if (dtype == ORACLE_E4M3) return -1;  /* E4M3 needs its descales */
    return oracle_prefill_thd_scaled(dtype, q, q_st, q_sh, k, k_st, k_sh, v, v_st, v_sh, cu_q,
                                     cu_kv, batch, hq, hkv, dqk, dv, scale, causal, window, sinks,
                                     1.0, 1.0, 1.0, n_sel, sel_tok, sel_head, o, lse, p_out,
                                     nthreads);
}

/* ---- paged-KV decode ------------------------------------------------------ */

typedef struct {
    int dtype;
    const void *q, *kp, *vp;
    int64_t k_sp, k_st, k_sh, v_sp, v_st, v_sh;
    const int32_t *pt_k, *pt_v, *seq_lens;
    int32_t table_stride, batch, sq, hq, hkv, dqk, dv, page, causal, num_splits;
    int32_t window;            /* left window W (<= 0: none) */
    const double* sinks;       /* [hq] sink logits, or NULL */
    double scale;
    double dq, dk, dv_scale;   /* per-tensor descales of Q, K, V (1 unless E4M3) */
    int64_t n_sel;
    const int64_t* sel_row;
    double *o, *lse;       /* merged output (or unsplit) */
    double *o_part, *lse_part; /* optional per-split partials, [S, rows, dv] / [S, rows] */
    int64_t max_lk;
} decode_ctx;

/* Chunk length for split-KV: ceil(ceil(L/S) / page) * page keys, chunks
 * contiguous from key 0.  (The pages print no chunking rule; any chunking
 * gives the same merged result, which the test suite checks.) */
static int64_t split_chunk(int64_t L, int32_t S, int32_t page) {
    if (S <= 1) return L > 0 ? L : 1;
    int64_t per = (L + S - 1) / S;
    int64_t pages = (per + page - 1) / page;
    int64_t c = pages * page;
    return c > 0 ? c : page;
}

static void decode_unit(void* vctx, int64_t unit, double* scratch) {
    decode_ctx* c = (decode_ctx*)vctx;
    int64_t row = c->n_sel < 0 ? unit : c->sel_row[unit];
    int32_t h = (int32_t)(row % c->hq);
    int32_t tq = (int32_t)((row / c->hq) % c->sq);
    int32_t b = (int32_t)(row / ((int64_t)c->hq * c->sq));
    int32_t kvh = h / (c->hq / c->hkv);
    int64_t L = c->seq_lens[b];
    /* query token tq sits at position pos = L - sq + tq (bottom-right alignment);
       it sees keys first <= j <= last */
    const int64_t pos = L - c->sq + tq;
    int64_t last = c->causal ? pos : (L - 1);
    int64_t first = 0;
    if (c->window > 0 && pos - c->window + 1 > first) first = pos - c->window + 1;
    /* split mode cuts the keys [base, L) into chunks, base = the start of the page
       that holds the first key any query token of the sequence can see (0 without
       a window) */
    int64_t base = 0;
    if (c->window > 0 && L - c->sq - c->window + 1 > 0)
        base = ((L - c->sq - c->window + 1) / c->page) * c->page;
    const double sink = c->sinks ? c->sinks[h] : -INFINITY;
    double* qrow = scratch;
    int64_t* koff = (int64_t*)(scratch + c->dqk);
    int64_t* voff = koff + c->max_lk;
    double* s = (double*)(voff + c->max_lk);
    for (int d = 0; d < c->dqk; ++d)
        qrow[d] = c->dq * load_elem(c->q, c->dtype, row * c->dqk + d);

    int32_t S = c->num_splits < 1 ? 1 : c->num_splits;
    int64_t chunk = split_chunk(L - base, S, c->page);
    double* o = c->o + unit * c->dv;
    double* lse = c->lse + unit;
    /* per-split partials: the merge below is the textbook LSE merge */
    double m_all = -INFINITY;
    double* ol = (double*)malloc(sizeof(double) * (size_t)c->dv * (size_t)S);
    double* ll = (double*)malloc(sizeof(double) * (size_t)S);
    if (!ol || !ll) { free(ol); free(ll); *lse = NAN; return; }
    for (int32_t sp = 0; sp < S; ++sp) {
        int64_t lo = base + (int64_t)sp * chunk;
        int64_t hi = lo + chunk;
        if (S == 1) { lo = 0; hi = L; }
        if (hi > L) hi = L;
        if (hi > last + 1) hi = last + 1;
        if (lo < first) lo = first;
        int64_t n = 0;
        for (int64_t j = lo; j < hi; ++j, ++n) {
            int64_t pg = j / c->page, slot = j % c->page;
            int64_t kpage = c->pt_k[(int64_t)b * c->table_stride + pg];
            int64_t vpage = c->pt_v[(int64_t)b * c->table_stride + pg];
            koff[n] = kpage * c->k_sp + slot * c->k_st + (int64_t)kvh * c->k_sh;
            voff[n] = vpage * c->v_sp + slot * c->v_st + (int64_t)kvh * c->v_sh;
        }
        /* one split: the plain definition, sink included; several: each chunk's
           partial without the sink, which joins the merge below */
        attend_row(qrow, c->dqk, c->dv, c->kp, c->vp, koff, voff, n, c->dtype, c->dk, c->dv_scale,
                   c->scale, S == 1 ? sink : -INFINITY, s,
                   ol + (size_t)sp * c->dv, ll + sp, NULL);
        if (ll[sp] > m_all) m_all = ll[sp];
        if (c->o_part) {
            int64_t rows = (int64_t)c->batch * c->sq * c->hq;
            for (int d = 0; d < c->dv; ++d)
                c->o_part[((int64_t)sp * rows + row) * c->dv + d] = ol[(size_t)sp * c->dv + d];
            c->lse_part[(int64_t)sp * rows + row] = ll[sp];
        }
    }
    /* the sink takes part in the merge as one more term of the denominator
       with no value: a partial whose LSE is the sink logit and whose O is 0 */
    if (S > 1 && sink > m_all) m_all = sink;
    if (S == 1) {
        for (int d = 0; d < c->dv; ++d) o[d] = ol[d];
        *lse = ll[0];
    } else if (m_all == -INFINITY) {
        for (int d = 0; d < c->dv; ++d) o[d] = 0.0;
        *lse = -INFINITY;
    } else {
        double w_sum = 0.0;
        for (int32_t sp = 0; sp < S; ++sp) w_sum += exp(ll[sp] - m_all);
        if (sink != -INFINITY) w_sum += exp(sink - m_all);
        double L_all = m_all + log(w_sum);
        for (int d = 0; d < c->dv; ++d) o[d] = 0.0;
        for (int32_t sp = 0; sp < S; ++sp) {
            double w = exp(ll[sp] - L_all);
            for (int d = 0; d < c->dv; ++d) o[d] += w * ol[(size_t)sp * c->dv + d];
        }
        *lse = L_all;
    }
    free(ol);
    free(ll);
}

/*
 * Paged decode.  Q [B, sq, Hq, Dqk] dense.  Pools addressed by element
 * strides (page, token-in-page, head); logical key j of sequence b lives in
 * page pt_k[b*table_stride + j/page] (K) and pt_v[...] (V) at slot j%page.
 * seq_lens[b] = KV length, including the sq new tokens.  Query token t of
 * sequence b sits at key position seq_lens[b] - sq + t.
 *
 * Token t sees keys j < seq_lens[b] with j <= seq_lens[b] - sq + t when
 * causal and, with a left window W > 0, j >= seq_lens[b] - sq + t - W + 1
 * (the W keys ending at its own position).  sinks (optional): Hq per-head
 * sink logits that join every row's softmax denominator with no value.
 *
 * num_splits <= 1: the plain definition over all visible keys (sink included).
 * num_splits  > 1: keys [base, L) split into contiguous chunks (split_chunk
 *   above; base = 0, or with a window the start of the page holding key
 *   L - sq - W + 1, the first key any token of the sequence sees), each
 *   chunk's normalized partial (O_c, LSE_c) computed by the definition without
 *   the sink, then merged with the sink as one more term of no value:
 *   M = max(LSE_c, sink), LSE = M + ln(sum exp(LSE_c - M) + exp(sink - M)),
 *   O = sum exp(LSE_c - LSE) O_c; all-empty and no sink -> (0, -inf).
 *   o_part/lse_part (optional) receive the partials, [S, rows, Dv]/[S, rows],
 *   row = (b*sq + t)*Hq + h.
 * n_sel < 0: all rows; else only rows sel_row[r] (same row numbering).
 * dtype ORACLE_E4M3: Q, K and V are E4M3 codes standing for descale_q/k/v
 * times their values (per-tensor FP8); other dtypes take descales of 1.
 */
int oracle_decode_paged_scaled(int dtype, const void* q, const void* kpool, int64_t k_sp,
                               int64_t k_st, int64_t k_sh, const void* vpool, int64_t v_sp,
                               int64_t v_st, int64_t v_sh, const int32_t* pt_k,
                               const int32_t* pt_v, int32_t table_stride,
                               const int32_t* seq_lens, int32_t batch, int32_t sq, int32_t hq,
                               int32_t hkv, int32_t dqk, int32_t dv, int32_t page, double scale,
                               int32_t causal, int32_t num_splits, int32_t window,
                               const double* sinks, double descale_q, double descale_k,
                               double descale_v, int64_t n_sel, const int64_t* sel_row,
                               double* o, double* lse, double* o_part, double* lse_part,
                               int32_t nthreads) {
    if (batch < 0 || sq <= 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0 || page <= 0) return -1;
    if (o_part && n_sel >= 0) return -1;
    int64_t max_lk = 1;
    for (int32_t b = 0; b < batch; ++b) {
        if (seq_lens[b] < 0) return -1;
        if (seq_lens[b] > max_lk) max_lk = seq_lens[b];
    }
    decode_ctx c = {dtype, q, kpool, vpool, k_sp, k_st, k_sh, v_sp, v_st, v_sh, pt_k, pt_v,
                    seq_lens, table_stride, batch, sq, hq, hkv, dqk, dv, page, causal,
                    num_splits, window, sinks, scale, descale_q, descale_k, descale_v, n_sel,
                    sel_row, o, lse, o_part, lse_part, max_lk};
    int64_t rows = (int64_t)batch * sq * hq;
    int64_t n_units = n_sel < 0 ? rows : n_sel;
    size_t scratch = (size_t)dqk + 3 * (size_t)max_lk;
    return run_pool(decode_unit, &c, n_units, scratch, nthreads);
}

/* bf16 / fp32 paged decode: the same definition with descales of 1. */
int oracle_decode_paged(int dtype, const void* q, const void* kpool, int64_t k_sp, int64_t k_st,
                        int64_t k_sh, const void* vpool, int64_t v_sp, int64_t v_st,
                        int64_t v_sh, const int32_t* pt_k, const int32_t* pt_v,
                        int32_t table_stride, const int32_t* seq_lens, int32_t batch,
                        int32_t sq, int32_t hq, int32_t hkv, int32_t dqk, int32_t dv,
                        int32_t page, double scale, int32_t causal, int32_t num_splits,
                        int64_t n_sel, const int64_t* sel_row, double* o, double* lse,
                        double* o_part, double* lse_part, int32_t nthreads) {
    if (dtype == ORACLE_E4M3) return -1;  /* E4M3 needs its descales */
    return oracle_decode_paged_scaled(dtype, q, kpool, k_sp, k_st, k_sh, vpool, v_sp, v_st, v_sh,
                                      pt_k, pt_v, table_stride, seq_lens, batch, sq, hq, hkv,
                                      dqk, dv, page, scale, causal, num_splits, 0, NULL, 1.0, 1.0,
                                      1.0, n_sel, sel_row, o, lse, o_part, lse_part, nthreads);
}

/*
 * LSE merge of split partials, the textbook definition.
 * o_part [S, rows, dv] (each partial already normalized), lse_part [S, rows]
 * natural log, -inf marks an empty split.
 */
void oracle_combine(const double* o_part, const double* lse_part, int32_t S, int64_t rows,
                    int32_t dv, double* o, double* lse) {
    for (int64_t r = 0; r < rows; ++r) {
        double m = -INFINITY;
        for (int32_t s = 0; s < S; ++s)
            if (lse_part[(int64_t)s * rows + r] > m) m = lse_part[(int64_t)s * rows + r];
        if (m == -INFINITY) {
            for (int d = 0; d < dv; ++d) o[r * dv + d] = 0.0;
            lse[r] = -INFINITY;
            continue;
        }
        double w_sum = 0.0;
        for (int32_t s = 0; s < S; ++s) w_sum += exp(lse_part[(int64_t)s * rows + r] - m);
        double L = m + log(w_sum);
        for (int d = 0; d < dv; ++d) {
            double acc = 0.0;
            for (int32_t s = 0; s < S; ++s) {
                double w = exp(lse_part[(int64_t)s * rows + r] - L);
                if (w != 0.0) acc += w * o_part[((int64_t)s * rows + r) * dv + d];
            }
            o[r * dv + d] = acc;
        }
        lse[r] = L;
    }
}
