// decode_paged.hip -- paged-KV decode with split-KV partials.
//
// For every sequence b, KV head kvh and split c, a work-group streams the
// chunk's keys through the K and V page tables (independent tables and
// pools: cuDNN Frontend v1.31.0 Release Notes, "SDPA: paged KV, split-KV, and
// engine selection"; v1.32.0 Release Notes, "SDPA: wider native forward
// support", Q/K 576 with V 512; the non-absorbed MLA pools d_qk 192 / d_v 128:
// v1.28.0 release notes, "New: FROST SDPA on Ampere, Ada/Blackwell-consumer,
// and Rubin", SM120 bullet) and computes, for the s_q * G query rows that
// share the KV head, the normalized partial O_c and its natural-log LSE_c.
// With one split the result is final and goes straight to O / LSE.
//
// Decode tiles are sized to the live rows (s_q * G, padded to 32 per wave),
// not to a prefill tile: running decode through a prefill-sized tile wastes
// most of every matrix op on dead rows (v1.30.0 Release Notes, "New: decode
// tiles -- SDPA decode stops running the prefill pipeline").  Rows beyond
// 32 * NW per work-group go to sibling work-groups of the same split whose ids
// are congruent mod 8, so the round-robin dispatcher places them on the same
// XCD and they share that XCD's L2 copy of the chunk.
#include "sdpa_device.h"
#include "sdpa_launch.h"

namespace sdpa {
namespace {

struct DecodeKArgs {
    const void* q;   // bf16, or E4M3 codes (F8)
    const void* kp;
    int64_t k_sp, k_st, k_sh;
    const void* vp;
    int64_t v_sp, v_st, v_sh;
    const int32_t* pt_k;
    const int32_t* pt_v;
    int32_t table_stride;
    const int32_t* seq_lens;
    int32_t sq, hq, hkv, group, page, splits, n_rg, n_units;
    int32_t rows;        // s_q * G query rows per KV head
    int64_t total_rows;  // batch * s_q * h_q
    float scale_log2;
    int32_t causal;
    float* o_part;
    float* lse_part;
    bf16_t* o;
    float* lse;
    int32_t window;      // left sliding window (0: none)
    const float* sinks;  // [hq] sink logits (natural-log units) or nullptr
    int32_t stats_log2;  // final LSE in base 2
    const float* descale_q;  // F8 only: one fp32 each, read on the device
    const float* descale_k;
    const float* descale_v;
};

constexpr int BK = 32;

// F8: per-tensor FP8 (E4M3) Q, K and V standing for descale_{q,k,v} times
// their codes (cuDNN Frontend v1.31.0 Release Notes, per-tensor FP8 D128 paged
// KV; v1.32.0 "SDPA: wider native forward support", native D64 per-tensor
// FP8, paged per-tensor FP8 D256).  Codes are widened exactly to bf16 as they
// are loaded, so the tile and MFMA path is the bf16 one; descale_q descale_k
// joins the logit scale and descale_v multiplies the normalized output.
template <int DQK, int DV, int NW, bool PREFETCH, bool F8>
__global__ __launch_bounds__(NW * 64, (DQK + DV > 512 ? 1 : 2)) void decode_kernel(DecodeKArgs a) {
    constexpr int NT = NW * 64;
    using G = TileGeom<DQK, DV, BK>;
    using SH = TileShare<DQK, DV, BK, NT>;
    extern __shared__ __attribute__((aligned(16))) bf16_t smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // work-group id -> (unit, row group); the n_rg row groups of one unit
    // have ids congruent mod 8 (same XCD) and within 8 * n_rg of each other.
    const int bid = blockIdx.x;
    const int blk = bid / (8 * a.n_rg), w8 = bid % (8 * a.n_rg);
    const int rg = w8 / 8;
    const int unit = blk * 8 + (w8 % 8);
    if (unit >= a.n_units) return;
    const int split = unit % a.splits;
    const int bh = unit / a.splits;
    const int kvh = bh % a.hkv, b = bh / a.hkv;

    // a length past the table's reach is clamped (the table is never read out of
    // bounds) and the sequence's rows are written as NaN
    const bool trunc = a.seq_lens[b] > a.table_stride * a.page;
    const int L = min(a.seq_lens[b], a.table_stride * a.page);
    // keys [base, L) are cut into the splits; with a left window, base is the
    // start of the page holding the first key any token of the sequence sees
    int base = 0;
    if (a.window > 0 && L - a.sq - a.window + 1 > 0) base = ((L - a.sq - a.window + 1) / a.page) * a.page;
    int lo = base, hi = L;
    if (a.splits > 1) {
        const int per = (L - base + a.splits - 1) / a.splits;
        const int chunk = ((per + a.page - 1) / a.page) * a.page;
        lo = min(L, base + split * chunk);
        hi = min(L, lo + chunk);
    }
    const int row0_wg = rg * NW * 32;
    const int row0 = row0_wg + wave * 32;
    const int col = lane & 31, half = lane >> 5;
    const int r = row0 + col;
    const bool row_ok = r < a.rows;
    const int t = (row_ok ? r : a.rows - 1) / a.group;
    const int h = kvh * a.group + (row_ok ? r : a.rows - 1) % a.group;
    // last key each row may see: its causal position, and the chunk's end
    auto last_key = [&](int tok) { return a.causal ? L - a.sq + tok : L - 1; };
    const int lim = min(hi - 1, last_key(t));
    const int t_max_wg = (min(a.rows, row0_wg + NW * 32) - 1) / a.group;
    const int kv_end = max(lo, min(hi, last_key(t_max_wg) + 1));
    int kv_end_w = lo, nomask_end = lo;
    if (row0 < a.rows) {
        kv_end_w = max(lo, min(hi, last_key((min(a.rows, row0 + 32) - 1) / a.group) + 1));
        nomask_end = max(lo, min(hi, last_key(row0 / a.group) + 1));
    }
    // first key each row may see (left window): this lane's, and the largest of
    // the wave's rows (its last token's); tiles starting below it need the mask
    auto first_key = [&](int tok) { return a.window > 0 ? L - a.sq + tok - a.window + 1 : INT32_MIN; };
    const int first = first_key(t);
    const int first_w = first_key((min(a.rows, row0 + 32) - 1) / a.group);

    bf16x8 qf[DQK / 16];
    const int64_t grow = ((int64_t)b * a.sq + t) * a.hq + h;  // global row id
    load_q<DQK, F8>(qf, static_cast<const char*>(a.q) + grow * DQK * (F8 ? 1 : 2), row_ok, lane);
    float scale_log2 = a.scale_log2;
    float o_mul = 1.f;
    if constexpr (F8) {
        scale_log2 *= a.descale_q[0] * a.descale_k[0];
        o_mul = a.descale_v[0];
    }

    RowState<DV> st;
    row_state_init<DV>(st);

    const int32_t* ptk = a.pt_k + (int64_t)b * a.table_stride;
    const int32_t* ptv = a.pt_v + (int64_t)b * a.table_stride;
    const char* kbase = static_cast<const char*>(a.kp) + (int64_t)kvh * a.k_sh * (F8 ? 1 : 2);
    const char* vbase = static_cast<const char*>(a.vp) + (int64_t)kvh * a.v_sh * (F8 ? 1 : 2);
    auto koff = [&](int k0) {
        return [=](int j) -> int64_t {
            const int key = k0 + j;
            if (key >= kv_end) return -1;
            return (int64_t)ptk[key / a.page] * a.k_sp + (int64_t)(key % a.page) * a.k_st;
        };
    };
    auto voff = [&](int k0) {
        return [=](int j) -> int64_t {
            const int key = k0 + j;
            if (key >= kv_end) return -1;
            return (int64_t)ptv[key / a.page] * a.v_sp + (int64_t)(key % a.page) * a.v_st;
        };
    };

    const int n_tiles = (kv_end - lo + BK - 1) / BK;
    if constexpr (PREFETCH) {
        KRegs<SH::KC> kr;
        VRegs<SH::VU> vr;
        if (n_tiles > 0) {
            load_k_part<DQK, DV, BK, NT, F8>(kr, kbase, tid, koff(lo));
            load_v_part<DQK, DV, BK, NT, F8>(vr, vbase, tid, voff(lo));
            store_k_part<DQK, DV, BK, NT>(kr, smem, tid);
            store_v_part<DQK, DV, BK, NT>(vr, smem, tid);
        }
        __syncthreads();
        for (int it = 0; it < n_tiles; ++it) {
            const int key0 = lo + it * BK;
            const bool more = it + 1 < n_tiles;
            if (more) {
                load_k_part<DQK, DV, BK, NT, F8>(kr, kbase, tid, koff(key0 + BK));
                load_v_part<DQK, DV, BK, NT, F8>(vr, vbase, tid, voff(key0 + BK));
            }
            const bf16_t* buf = smem + (it & 1) * G::BUF_ELEMS;
            if (key0 < kv_end_w)
                tile_step<DQK, DV, BK>(buf, buf + G::K_ELEMS, qf, st, key0, lim, first,
                                       key0 + BK > nomask_end || key0 < first_w, scale_log2,
                                       lane);
            if (more) {
                bf16_t* nb = smem + ((it + 1) & 1) * G::BUF_ELEMS;
                store_k_part<DQK, DV, BK, NT>(kr, nb, tid);
                store_v_part<DQK, DV, BK, NT>(vr, nb, tid);
            }
            __syncthreads();
        }
    } else {
        for (int it = 0; it < n_tiles; ++it) {
            const int key0 = lo + it * BK;
            {
                KRegs<SH::KC> kr;
                load_k_part<DQK, DV, BK, NT, F8>(kr, kbase, tid, koff(key0));
                store_k_part<DQK, DV, BK, NT>(kr, smem, tid);
            }
            {
                VRegs<SH::VU> vr;
                load_v_part<DQK, DV, BK, NT, F8>(vr, vbase, tid, voff(key0));
                store_v_part<DQK, DV, BK, NT>(vr, smem, tid);
            }
            __syncthreads();
            if (key0 < kv_end_w)
                tile_step<DQK, DV, BK>(smem, smem + G::K_ELEMS, qf, st, key0, lim, first,
                                       key0 + BK > nomask_end || key0 < first_w, scale_log2,
                                       lane);
            __syncthreads();
        }
    }

    float l_tot = row_total<DV>(st);
    if (!row_ok) return;
    float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float m = st.m;
    if (a.sinks != nullptr && a.splits == 1) {
        // head h's sink joins the denominator with no value (log2 units); split
        // partials leave it to the combine
        const float sk = a.sinks[h] * kLog2e;
        const float m2 = fmaxf(m, sk);
        if (m2 != neg_inf()) {
            const float alpha = fast_exp2(m - m2);  // 0 when no key is visible
            l_tot = l_tot * alpha + fast_exp2(sk - m2);
            inv = alpha / l_tot;
            m = m2;
        }
    }
    const float lse2 = l_tot > 0.f ? m + fast_log2(l_tot) : neg_inf();
    // partials stay natural-log; the final Stats may be base 2
    float lse = a.stats_log2 && a.splits == 1 ? lse2 : kLn2 * lse2;
    inv *= o_mul;  // descale_v (1 unless FP8)
    if (trunc) inv = lse = nan_f();
    if (a.splits > 1) {
        float* orow = a.o_part + ((int64_t)split * a.total_rows + grow) * DV;
#pragma unroll
        for (int nb = 0; nb < DV / 32; ++nb) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = nb * 32 + 8 * g + 4 * half;
                float4 w;
                w.x = st.acc[nb][4 * g] * inv;
                w.y = st.acc[nb][4 * g + 1] * inv;
                w.z = st.acc[nb][4 * g + 2] * inv;
                w.w = st.acc[nb][4 * g + 3] * inv;
                *reinterpret_cast<float4*>(orow + n) = w;
            }
        }
        if (half == 0) a.lse_part[(int64_t)split * a.total_rows + grow] = lse;
    } else {
        bf16_t* orow = a.o + grow * DV;
#pragma unroll
        for (int nb = 0; nb < DV / 32; ++nb) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = nb * 32 + 8 * g + 4 * half;
                uint2 w;
                w.x = pack_bf16x2(st.acc[nb][4 * g] * inv, st.acc[nb][4 * g + 1] * inv);
                w.y = pack_bf16x2(st.acc[nb][4 * g + 2] * inv, st.acc[nb][4 * g + 3] * inv);
                *reinterpret_cast<uint2*>(orow + n) = w;
            }
        }
        if (half == 0 && a.lse != nullptr) a.lse[grow] = lse;
    }
}

template <int DQK, int DV, int NW, bool F8>
hipError_t launch_nw(const DecodeKArgs& a, hipStream_t s) {
    constexpr bool PREFETCH = DQK + DV <= 256;
    using G = TileGeom<DQK, DV, BK>;
    const size_t lds = (PREFETCH ? 2 : 1) * (size_t)G::BUF_BYTES;
    const int64_t n_wg = (int64_t)((a.n_units + 7) / 8) * 8 * a.n_rg;
    if (n_wg == 0) return hipSuccess;
    hipError_t e = hipFuncSetAttribute((const void*)decode_kernel<DQK, DV, NW, PREFETCH, F8>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_kernel<DQK, DV, NW, PREFETCH, F8>), dim3((unsigned)n_wg),
                       dim3(NW * 64), lds, s, a);
    return hipGetLastError();
}

template <int DQK, int DV, bool F8>
hipError_t launch_dims(DecodeKArgs& a, hipStream_t s) {
    const int nw = a.rows <= 32 ? 1 : (a.rows <= 64 ? 2 : 4);
    a.n_rg = (a.rows + nw * 32 - 1) / (nw * 32);
    switch (nw) {
        case 1: return launch_nw<DQK, DV, 1, F8>(a, s);
        case 2: return launch_nw<DQK, DV, 2, F8>(a, s);
        default: return launch_nw<DQK, DV, 4, F8>(a, s);
    }
}

// The general decode kernel for the shapes the specialized kernels leave.
hipError_t launch_generic(const DecodeArgs& da, hipStream_t s, bool f8) {
    DecodeKArgs a;
    a.q = da.q;
    a.kp = da.k_pool;
    a.k_sp = da.k_sp;
    a.k_st = da.k_st;
    a.k_sh = da.k_sh;
    a.vp = da.v_pool;
    a.v_sp = da.v_sp;
    a.v_st = da.v_st;
    a.v_sh = da.v_sh;
    a.pt_k = da.pt_k;
    a.pt_v = da.pt_v;
    a.table_stride = da.table_stride;
    a.seq_lens = da.seq_lens;
    a.sq = da.sq;
    a.hq = da.hq;
    a.hkv = da.hkv;
    a.group = da.hq / da.hkv;
    a.page = da.page;
    a.splits = da.splits;
    a.n_units = da.batch * da.hkv * da.splits;
    a.rows = da.sq * a.group;
    a.total_rows = (int64_t)da.batch * da.sq * da.hq;
    a.scale_log2 = da.scale * kLog2e;
    a.causal = da.causal;
    a.o_part = da.o_part;
    a.lse_part = da.lse_part;
    a.o = static_cast<bf16_t*>(da.o);
    a.lse = da.lse;
    // a window of 2^30 keys covers every key the int32 lengths can describe
    a.window = da.window > 0 ? min(da.window, 1 << 30) : 0;
    a.sinks = da.sinks;
    a.stats_log2 = da.stats_log2;
    a.descale_q = f8 ? da.descale_q : nullptr;
    a.descale_k = f8 ? da.descale_k : nullptr;
    a.descale_v = f8 ? da.descale_v : nullptr;
    a.n_rg = 1;
    if (a.n_units == 0) return hipSuccess;
    // the kernel's per-work-group state is sized for 512 query rows per KV head; the
    // entry points decline more before they get here
    if (a.rows > 512) return hipErrorInvalidValue;
    if (f8) {
        if (da.dqk == 64) return launch_dims<64, 64, true>(a, s);
        if (da.dqk == 128) return launch_dims<128, 128, true>(a, s);
        if (da.dqk == 256) return launch_dims<256, 256, true>(a, s);
        if (da.dqk == 192) return launch_dims<192, 128, true>(a, s);
        if (da.dqk == 576) return launch_dims<576, 512, true>(a, s);
    } else {
        if (da.dqk == 64) return launch_dims<64, 64, false>(a, s);
        if (da.dqk == 128) return launch_dims<128, 128, false>(a, s);
        if (da.dqk == 256) return launch_dims<256, 256, false>(a, s);
        if (da.dqk == 192) return launch_dims<192, 128, false>(a, s);
        if (da.dqk == 576) return launch_dims<576, 512, false>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool decode_supported(int32_t dqk, int32_t dv) {
    return (dqk == 64 && dv == 64) || (dqk == 128 && dv == 128) || (dqk == 256 && dv == 256) ||
           (dqk == 192 && dv == 128) || (dqk == 576 && dv == 512);
}

// The few-row kernel takes up to kSmallRowsMax rows per KV head, in groups
// of 16 that each read the chunk's K/V (the general kernel reads it once
// but ran 4x slower at 32 rows); its unit count must fit an int.
static bool small_fits(const DecodeArgs& da) {
    const int rows = da.sq * (da.hq / da.hkv);
    return decode_small_supported(da.dqk, da.dv, rows) &&
           (int64_t)da.batch * da.hkv * da.splits * ((rows + 15) / 16) <= INT32_MAX;
}

// The kernel a decode call runs on (the order below is the selection order):
// few-row kernel up to 16 rows per KV head (FP8: up to 32, in row groups
// past 16), the paged prefill kernel (D 64 / 128 / 256 on suitable pages;
// folded rows when the call has fewer tokens than an item), the absorbed-MLA
// wide kernel, the few-row kernel in row groups up to kSmallRowsMax rows, and
// the general kernel for the rest.
DecodePath decode_path(const DecodeArgs& da) {
    const int rows = da.sq * (da.hq / da.hkv);
    const bool small = small_fits(da);
    if (small && rows <= (da.fp8 ? 32 : 16)) return rows <= 16 ? DecodePath::kFewRow : DecodePath::kRowGroups;
    if (prefill_paged_supported(da)) return prefill_paged_folds(da) ? DecodePath::kPrefillFolded : DecodePath::kPrefill;
    if (decode_wide_supported(da)) return DecodePath::kWide;
    if (small) return DecodePath::kRowGroups;
    return DecodePath::kGeneral;
}

static hipError_t launch_decode_path(const DecodeArgs& da, hipStream_t s, bool f8) {
    switch (decode_path(da)) {
        case DecodePath::kFewRow:
        case DecodePath::kRowGroups: return launch_decode_small(da, s);
        case DecodePath::kPrefill:
        case DecodePath::kPrefillFolded: return launch_prefill_paged(da, s);
        case DecodePath::kWide: return launch_decode_wide(da, s);
        default: return launch_generic(da, s, f8);
    }
}

hipError_t launch_decode_bf16(const DecodeArgs& da, hipStream_t s) { return launch_decode_path(da, s, false); }

// FP8: up to 32 rows per KV head two 16-row groups, each reading the codes,
// beat the FP8 prefill kernel's folded items (0.51 against 0.62 ms at 32 rows
// on B = 32 of the decode workload's sequences; 0.98 against 0.65 at 64)
hipError_t launch_decode_fp8(const DecodeArgs& da, hipStream_t s) { return launch_decode_path(da, s, true); }

}  // namespace sdpa
