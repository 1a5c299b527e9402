// prefill_bf16.hip -- packed THD ragged prefill, bf16 in/out, FP32 LSE.
//
// Computes, for every sequence b of a packed THD batch (offsets from the
// device-side prefix sums cu_q / cu_kv), O = softmax(scale * Q K^T) V over
// the visible keys (bottom-right causal diagonal when causal) and the
// natural-log LSE per (token, head).  Packed THD addressing and padded
// (b, s_max, h) Stats: cuDNN Frontend v1.30.0 Release Notes, "New: the
// FlashInfer serving path runs on FROST"; zero host reads, prefix-sum
// offsets, bottom-right THD diagonals, pack_gqa: v1.28.0 release notes,
// "New: FROST SDPA on Ampere, Ada/Blackwell-consumer, and Rubin".
//
// Work-group = 4 waves = 128 query rows sharing one KV head.  The rows are
// NH query heads of one GQA group x (4/NH) blocks of 32 consecutive tokens,
// NH = gcd(G, 4): every K/V tile staged in LDS is reused by NH heads
// (partial GQA packing when G is not a multiple of 4: v1.30.0 "New: decode
// tiles", Partial PackGQA bullet).  K/V tiles are double-buffered in LDS;
// the next tile's HBM loads are in flight while the current one is on MFMA.
// Work-groups are issued longest-causal-tile first.
#include "sdpa_device.h"
#include "sdpa_launch.h"

namespace sdpa {
namespace {

struct PrefillKArgs {
    const bf16_t* q;
    int64_t q_st, q_sh;
    const bf16_t* k;
    int64_t k_st, k_sh;
    const bf16_t* v;
    int64_t v_st, v_sh;
    bf16_t* o;
    int64_t o_st, o_sh;
    const int32_t* cu_q;
    const int32_t* cu_kv;
    int32_t batch, hq, group, nh, n_hg, n_qtiles;
    float scale_log2;
    int32_t causal;
    float* lse;
    int32_t lse_layout, lse_s_max;
};

constexpr int kThreads = 256;

// D <= 128 fits two work-groups per CU (<= 256 registers per lane); D = 256
// needs the whole 512-entry register file (accumulators in AGPRs) at one.
template <int D, int BK>
__global__ __launch_bounds__(kThreads, (D <= 128 ? 2 : 1)) void prefill_bf16_kernel(PrefillKArgs a) {
    using G = TileGeom<D, D, BK>;
    using SH = TileShare<D, D, BK, kThreads>;
    extern __shared__ __attribute__((aligned(16))) bf16_t smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bid = blockIdx.x;
    const int b = bid % a.batch;
    const int rest = bid / a.batch;
    const int hg = rest % a.n_hg;
    const int qt = a.n_qtiles - 1 - rest / a.n_hg;

    const int q_beg = a.cu_q[b], lq = a.cu_q[b + 1] - q_beg;
    const int kv_beg = a.cu_kv[b], lk = a.cu_kv[b + 1] - kv_beg;
    const int nt = 4 / a.nh;
    const int q0 = qt * 32 * nt;
    if (q0 >= lq) return;  // uniform across the work-group

    const int hw = wave % a.nh, tb = wave / a.nh;
    const int h = hg * a.nh + hw;
    const int kvh = h / a.group;
    const int i0 = q0 + tb * 32;
    const int col = lane & 31, half = lane >> 5;
    const int i = i0 + col;
    const bool row_ok = i < lq;
    const int shift = lk - lq;  // bottom-right diagonal offset

    // key extents: the work-group's, this wave's, and this lane's
    const int last_wg = min(q0 + 32 * nt, lq) - 1;
    const int kv_end = a.causal ? max(0, min(lk, last_wg + shift + 1)) : lk;
    int kv_end_w = 0, nomask_end = 0;
    if (i0 < lq) {
        const int last_w = min(i0 + 32, lq) - 1;
        kv_end_w = a.causal ? max(0, min(lk, last_w + shift + 1)) : lk;
        nomask_end = a.causal ? max(0, min(lk, i0 + shift + 1)) : lk;
    }
    const int lim = a.causal ? min(lk - 1, i + shift) : lk - 1;

    bf16x8 qf[D / 16];
    load_q<D>(qf, a.q + (int64_t)(q_beg + i) * a.q_st + (int64_t)h * a.q_sh, row_ok, lane);

    RowState<D> st;
    row_state_init<D>(st);

    const int n_tiles = (kv_end + BK - 1) / BK;
    const bf16_t* kb0 = a.k + (int64_t)kv_beg * a.k_st + (int64_t)kvh * a.k_sh;
    const bf16_t* vb0 = a.v + (int64_t)kv_beg * a.v_st + (int64_t)kvh * a.v_sh;
    const int64_t k_st = a.k_st, v_st = a.v_st;

    KRegs<SH::KC> kr;
    VRegs<SH::VU> vr;
    auto load = [&](int k0) {
        load_k_part<D, D, BK, kThreads>(kr, kb0, tid, [&](int j) -> int64_t {
            return k0 + j < kv_end ? (int64_t)(k0 + j) * k_st : -1;
        });
        load_v_part<D, D, BK, kThreads>(vr, vb0, tid, [&](int j) -> int64_t {
            return k0 + j < kv_end ? (int64_t)(k0 + j) * v_st : -1;
        });
    };
    auto store = [&](bf16_t* buf) {
        store_k_part<D, D, BK, kThreads>(kr, buf, tid);
        store_v_part<D, D, BK, kThreads>(vr, buf, tid);
    };
    if (n_tiles > 0) {
        load(0);
        store(smem);
    }
    __syncthreads();

    for (int t = 0; t < n_tiles; ++t) {
        const int key0 = t * BK;
        const bool more = t + 1 < n_tiles;
        if (more) load(key0 + BK);  // next tile's HBM loads in flight during the MFMAs
        const bf16_t* buf = smem + (t & 1) * G::BUF_ELEMS;
        if (key0 < kv_end_w) {
            const bool need_mask = key0 + BK > nomask_end;
            tile_step<D, D, BK>(buf, buf + G::K_ELEMS, qf, st, key0, lim, need_mask,
                                a.scale_log2, lane);
        }
        if (more) store(smem + ((t + 1) & 1) * G::BUF_ELEMS);
        __syncthreads();
    }

    // epilogue: O = O^T / l written as bf16, LSE = ln2 * (m + log2 l)
    const float l_tot = row_total<D>(st);
    if (!row_ok) return;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    bf16_t* orow = a.o + (int64_t)(q_beg + i) * a.o_st + (int64_t)h * a.o_sh;
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int n = nb * 32 + 8 * g + 4 * half;
            uint2 w;
            w.x = pack_bf16x2(st.acc[nb][4 * g] * inv, st.acc[nb][4 * g + 1] * inv);
            w.y = pack_bf16x2(st.acc[nb][4 * g + 2] * inv, st.acc[nb][4 * g + 3] * inv);
            *reinterpret_cast<uint2*>(orow + n) = w;
        }
    }
    if (a.lse != nullptr && half == 0) {
        const float lse = l_tot > 0.f ? kLn2 * (st.m + fast_log2(l_tot)) : neg_inf();
        if (a.lse_layout == 1) {
            a.lse[(int64_t)(q_beg + i) * a.hq + h] = lse;
        } else if (a.lse_layout == 2 && i < a.lse_s_max) {
            a.lse[((int64_t)b * a.lse_s_max + i) * a.hq + h] = lse;
        }
    }
}

template <int D, int BK>
hipError_t launch_d(const PrefillArgs& pa, hipStream_t s) {
    using G = TileGeom<D, D, BK>;
    PrefillKArgs a;
    a.q = static_cast<const bf16_t*>(pa.q);
    a.q_st = pa.q_st;
    a.q_sh = pa.q_sh;
    a.k = static_cast<const bf16_t*>(pa.k);
    a.k_st = pa.k_st;
    a.k_sh = pa.k_sh;
    a.v = static_cast<const bf16_t*>(pa.v);
    a.v_st = pa.v_st;
    a.v_sh = pa.v_sh;
    a.o = static_cast<bf16_t*>(pa.o);
    a.o_st = pa.o_st;
    a.o_sh = pa.o_sh;
    a.cu_q = pa.cu_q;
    a.cu_kv = pa.cu_kv;
    a.batch = pa.batch;
    a.hq = pa.hq;
    a.group = pa.hq / pa.hkv;
    a.nh = (a.group % 4 == 0) ? 4 : (a.group % 2 == 0 ? 2 : 1);
    a.n_hg = pa.hq / a.nh;
    const int tile_rows = 32 * (4 / a.nh);
    a.n_qtiles = (pa.max_q + tile_rows - 1) / tile_rows;
    a.scale_log2 = pa.scale * kLog2e;
    a.causal = pa.causal;
    a.lse = pa.lse;
    a.lse_layout = pa.lse_layout;
    a.lse_s_max = pa.lse_s_max;
    const int64_t n_wg = (int64_t)a.n_qtiles * a.n_hg * a.batch;
    if (n_wg == 0) return hipSuccess;
    const size_t lds = 2 * (size_t)G::BUF_BYTES;
    // more than 64 KiB of dynamic LDS must be requested per kernel
    hipError_t e = hipFuncSetAttribute((const void*)prefill_bf16_kernel<D, BK>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prefill_bf16_kernel<D, BK>), dim3((unsigned)n_wg), dim3(kThreads), lds, s,
                       a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
    switch (a.dqk) {
        case 64: return launch_d<64, 64>(a, s);
        case 128: return launch_d<128, 64>(a, s);
        case 256: return launch_d<256, 32>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sdpa
