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
// Work-group = 4 waves = 128 query rows sharing one KV head: NH query heads
// of one GQA group x (4 / NH) blocks of 32 consecutive tokens, NH = largest
// of {4, 2, 1} dividing G, so every K/V tile staged in LDS serves NH heads
// (partial GQA packing: v1.30.0 "New: decode tiles", Partial PackGQA bullet).
// Work-groups are issued longest causal row block first.
//
// Per wave and KV tile of BN keys (v_mfma_f32_32x32x16_bf16, wave64):
//   S^T[key][q] = K Q^T  -- A = K rows from LDS, B = the wave's Q^T held in
//                           registers; each lane ends up holding scores of
//                           ONE query (column lane % 32) for 16 keys per block;
//   online softmax       -- raw row max (3-input max), one lane-half exchange
//                           (v_permlane32_swap), p = exp2(s * c - m) as one
//                           FMA + exp, running sums per lane half; the output
//                           rescale is lazy: the running max only moves when a
//                           tile's max exceeds it by more than 8 (log2 units),
//                           which leaves the result exactly the same;
//   O^T[n][q] += V^T P^T -- B = P^T straight from the score accumulators
//                           (bf16), A = V^T from LDS, stored transposed with
//                           the keys of each 16-key step permuted to match.
// K/V tiles are double-buffered in LDS: the next tile's global loads are in
// flight while the current one is on the MFMA units.
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
    float c;          // |scale| * log2(e)
    uint32_t q_sign;  // 0x80008000 when scale < 0 (Q is negated on load), else 0
    int32_t causal;
    float* lse;
    int32_t lse_layout, lse_s_max;
};

constexpr int kThreads = 256;
constexpr float kLazyRescale = 8.f;  // log2 units the running max may lag behind
constexpr int kWin = 4;              // LDS operand fragments read ahead of the MFMAs
// Fourth word of a raw buffer resource on gfx9-family parts (CDNA): the
// range check returns zeros past num_records.
constexpr int kRsrcWord3 = 0x00020000;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <int D, int BN>
struct PCfg {
    static constexpr int KP = D + 8;             // K tile pitch (elements)
    static constexpr int VP = BN + 8;            // V^T tile pitch (elements)
    static constexpr int K_ELEMS = BN * KP;
    static constexpr int V_ELEMS = D * VP;
    static constexpr int BUF = K_ELEMS + V_ELEMS;
    static constexpr int LDS_BYTES = 2 * BUF * 2;
    static constexpr int KC = BN * D / 8 / kThreads;   // 16-byte K chunks per thread
    static constexpr int VU = BN * D / 32 / kThreads;  // V units (4 keys x 8 columns) per thread
    static constexpr int NKB = BN / 32;                // 32-key blocks of a tile
    static constexpr int NB = D / 32;                  // 32-row blocks of O^T
    static_assert(KC >= 1 && VU >= 1 && BN % 32 == 0 && D % 32 == 0, "tile shape");
    static_assert((BN / 4) * (D / 8) % kThreads == 0, "V units must tile the work-group");
};

// Lane-half exchange with v_permlane32_swap: on two copies a = b = v the
// swap leaves a = v of lanes 0..31 and b = v of lanes 32..63 in every lane,
// so a reduction of a and b is the reduction over the lane pair (l, l ^ 32).
// Written as inline asm because the compiler folds the two results of the
// builtin into one when both of its inputs are the same value.  The s_nop
// covers the VALU-write -> permlane-read hazard on the copies.
__device__ __forceinline__ void half_swap(float& a, float& b) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
// 3-input max without the NaN-quieting copies the compiler adds around fmaxf
__device__ __forceinline__ float max3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float half_max(float v) {
    float a = v, b = v;
    half_swap(a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float half_sum(float v) {
    float a = v, b = v;
    half_swap(a, b);
    return a + b;
}

template <int D, int BN>
struct Stage {
    uint4 k[PCfg<D, BN>::KC];
    uint4 v[PCfg<D, BN>::VU][4];
};

// D <= 128: two work-groups per CU (<= 256 registers per lane).  D = 256:
// one, with the O^T accumulators in the second half of the register file.
template <int D, int BN>
__global__ __launch_bounds__(kThreads, (D <= 128 ? 2 : 1)) void prefill_bf16_kernel(PrefillKArgs a) {
    using C = PCfg<D, BN>;
    extern __shared__ __attribute__((aligned(16))) bf16_t smem[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Work items: levels of equal causal row block qt, longest first; inside a
    // level the batch x head-group items are rotated by the level, so one
    // sequence's items do not stay on the same XCDs (the dispatcher sends
    // work-group id g to XCD g % 8) and ragged batches spread over the chip.
    const int bid = blockIdx.x;
    const int n_items = a.batch * a.n_hg;
    const int level = bid / n_items;
    const int item = (bid % n_items + level) % n_items;
    const int b = item / a.n_hg;
    const int hg = item % a.n_hg;
    const int qt = a.n_qtiles - 1 - level;

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

    // Q^T operand: lane (col, half) holds d = 16 kk + 8 half .. +8 of row i
    bf16x8 qf[D / 16];
    {
        const bf16_t* qrow = a.q + (int64_t)(q_beg + i) * a.q_st + (int64_t)h * a.q_sh + 8 * half;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            uint4 w = {0u, 0u, 0u, 0u};
            if (row_ok) w = *reinterpret_cast<const uint4*>(qrow + 16 * kk);
            w.x ^= a.q_sign;
            w.y ^= a.q_sign;
            w.z ^= a.q_sign;
            w.w ^= a.q_sign;
            qf[kk] = __builtin_bit_cast(bf16x8, w);
        }
    }

    f32x16 acc[C::NB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[nb][r] = 0.f;
    float m = neg_inf();  // running max (log2 units) of this lane's query
    float l = 0.f;        // this lane half's running sum

    const int n_tiles = (kv_end + BN - 1) / BN;
    const bf16_t* kb0 = a.k + (int64_t)kv_beg * a.k_st + (int64_t)kvh * a.k_sh;
    const bf16_t* vb0 = a.v + (int64_t)kv_beg * a.v_st + (int64_t)kvh * a.v_sh;

    // staging maps: K chunk idx -> (row idx / (D/8), 16-byte column idx % (D/8));
    // V unit idx -> (key quad idx % (BN/4), column chunk idx / (BN/4)).  The V
    // map makes 16 consecutive lanes write one V^T row (no LDS bank conflict).
    // Tiles are read with raw buffer loads: the resource of a tile starts at
    // its first row and ends with its last row below kv_end, so rows past the
    // end read as zeros with no predicate, and every lane offset is fixed.
    const int k_st2 = 2 * (int)a.k_st, v_st2 = 2 * (int)a.v_st;
    int k_off[C::KC], v_off[C::VU];
#pragma unroll
    for (int cc = 0; cc < C::KC; ++cc) {
        const int idx = tid + kThreads * cc;
        k_off[cc] = (idx / (D / 8)) * k_st2 + 16 * (idx % (D / 8));
    }
#pragma unroll
    for (int u = 0; u < C::VU; ++u) {
        const int idx = tid + kThreads * u;
        v_off[u] = 4 * (idx % (BN / 4)) * v_st2 + 16 * (idx / (BN / 4));
    }
    Stage<D, BN> st;
    auto load = [&](int k0) {
        const int nvalid = min(BN, kv_end - k0);
        const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(kb0 + (int64_t)k0 * a.k_st), (short)0, (nvalid - 1) * k_st2 + 2 * D,
            kRsrcWord3);
        const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(vb0 + (int64_t)k0 * a.v_st), (short)0, (nvalid - 1) * v_st2 + 2 * D,
            kRsrcWord3);
#pragma unroll
        for (int cc = 0; cc < C::KC; ++cc)
            st.k[cc] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, k_off[cc], 0, 0));
#pragma unroll
        for (int u = 0; u < C::VU; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                st.v[u][e] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(vr, v_off[u], e * v_st2, 0));
    };
    auto store = [&](bf16_t* buf) {
#pragma unroll
        for (int cc = 0; cc < C::KC; ++cc) {
            const int idx = tid + kThreads * cc;
            const int row = idx / (D / 8), ch = idx % (D / 8);
            *reinterpret_cast<uint4*>(buf + row * C::KP + 8 * ch) = st.k[cc];
        }
        bf16_t* vt = buf + C::K_ELEMS;
#pragma unroll
        for (int u = 0; u < C::VU; ++u) {
            const int idx = tid + kThreads * u;
            const int kq = idx % (BN / 4), ch = idx / (BN / 4);
            const int key0 = 4 * kq;
            const int pos = (key0 & ~15) + vt_pos(key0 & 15);
            const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&st.v[u][0]);
            const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&st.v[u][1]);
            const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&st.v[u][2]);
            const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&st.v[u][3]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint2 even, odd;
                even.x = __builtin_amdgcn_perm(w1[j], w0[j], 0x05040100u);
                even.y = __builtin_amdgcn_perm(w3[j], w2[j], 0x05040100u);
                odd.x = __builtin_amdgcn_perm(w1[j], w0[j], 0x07060302u);
                odd.y = __builtin_amdgcn_perm(w3[j], w2[j], 0x07060302u);
                const int n = 8 * ch + 2 * j;
                *reinterpret_cast<uint2*>(vt + n * C::VP + pos) = even;
                *reinterpret_cast<uint2*>(vt + (n + 1) * C::VP + pos) = odd;
            }
        }
    };

    // one KV tile for this wave
    auto tile = [&](const bf16_t* __restrict__ ks, const bf16_t* __restrict__ vt, int key0,
                    bool need_mask) {
        // S^T = K Q^T.  MFMA o works on key block o % NKB (consecutive MFMAs use
        // independent accumulators) and reads its K fragment kWin steps ahead.
        constexpr int NQK = C::NKB * (D / 16);
        auto kfrag = [&](int o) {
            return *reinterpret_cast<const bf16x8*>(
                ks + ((o % C::NKB) * 32 + col) * C::KP + 8 * half + 16 * (o / C::NKB));
        };
        f32x16 s[C::NKB];
        const f32x16 zero = {};
        bf16x8 fk[kWin];
#pragma unroll
        for (int w = 0; w < kWin; ++w) fk[w] = kfrag(w);
#pragma unroll
        for (int o = 0; o < NQK; ++o) {
            // the first MFMA of each key block starts from the constant 0
            s[o % C::NKB] = mfma_32x32x16(fk[o % kWin], qf[o / C::NKB],
                                          o < C::NKB ? zero : s[o % C::NKB]);
            if (o + kWin < NQK) fk[o % kWin] = kfrag(o + kWin);
        }
        // keep the reads kWin ahead: kWin reads, then alternate MFMA / read
        __builtin_amdgcn_sched_group_barrier(0x100, kWin, 0);
#pragma unroll
        for (int o = 0; o < NQK; ++o) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (o + kWin < NQK) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        // the first V^T fragments load while the softmax runs
        constexpr int NPV = C::NB * (BN / 16);
        auto vfrag = [&](int o) {
            return *reinterpret_cast<const bf16x8*>(
                vt + ((o % C::NB) * 32 + col) * C::VP + 8 * half + 16 * (o / C::NB));
        };
        bf16x8 fv[kWin];
#pragma unroll
        for (int w = 0; w < kWin; ++w) fv[w] = vfrag(w);
        // raw tile max of this lane's query (masked scores -> -inf)
        float mx = neg_inf();
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
            if (need_mask) {
                // key = key0 + 4 half + (compile-time offset); masked iff offset > dl
                const int dl = lim - key0 - 4 * half;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
                    s[kb][r] = off > dl ? neg_inf() : s[kb][r];
                }
            }
#pragma unroll
            for (int r = 0; r < 16; r += 2) mx = max3(mx, s[kb][r], s[kb][r + 1]);
        }
        mx = half_max(mx);
        const float mt = mx == neg_inf() ? neg_inf() : mx * a.c;
        // lazy rescale: move the running max only when the tile's exceeds it by > 8
        const bool grow = mt > m + kLazyRescale;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            // lanes that keep their max (possibly still -inf) rescale by exactly 1
            const float alpha = grow ? fast_exp2(m - mt) : 1.f;  // 0 when m = -inf
            m = grow ? mt : m;
            l *= alpha;
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[nb][r] *= alpha;
        }
        // a lane whose max is still -inf has every key masked: any finite shift
        // gives p = exp2(-inf) = 0 (c > 0) instead of exp2(-inf + inf) = NaN
        const float nm = m == neg_inf() ? 0.f : -m;
        float lsum = 0.f;
        bf16x8 pb[BN / 16];
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                float p0 = fast_exp2(__builtin_fmaf(s[kb][r], a.c, nm));
                float p1 = fast_exp2(__builtin_fmaf(s[kb][r + 1], a.c, nm));
                if (need_mask && a.c == 0.f) {  // c > 0: exp2(-inf) is already 0
                    p0 = s[kb][r] == neg_inf() ? 0.f : p0;
                    p1 = s[kb][r + 1] == neg_inf() ? 0.f : p1;
                }
                lsum += p0 + p1;
                const bf16x2 pp = __builtin_convertvector(f32x2{p0, p1}, bf16x2);
                pb[kb * 2 + (r >> 3)][r & 7] = pp[0];
                pb[kb * 2 + (r >> 3)][(r & 7) + 1] = pp[1];
            }
        }
        l += lsum;
        // O^T += V^T P^T: MFMA o works on output block o % NB
#pragma unroll
        for (int o = 0; o < NPV; ++o) {
            acc[o % C::NB] = mfma_32x32x16(fv[o % kWin], pb[o / C::NB], acc[o % C::NB]);
            if (o + kWin < NPV) fv[o % kWin] = vfrag(o + kWin);
        }
#pragma unroll
        for (int o = 0; o < NPV; ++o) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
            if (o + kWin < NPV) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
        }
    };

    if (n_tiles > 0) {
        load(0);
        store(smem);
    }
    __syncthreads();
    for (int t = 0; t < n_tiles; ++t) {
        const int key0 = t * BN;
        const bool more = t + 1 < n_tiles;
        if (more) load(key0 + BN);  // next tile's HBM loads in flight during the MFMAs
        const bf16_t* buf = smem + (t & 1) * C::BUF;
        if (key0 < kv_end_w) tile(buf, buf + C::K_ELEMS, key0, key0 + BN > nomask_end);
        if (more) store(smem + ((t + 1) & 1) * C::BUF);
        __syncthreads();
    }

    // epilogue: O = O^T / l written as bf16, LSE = ln2 * (m + log2 l)
    const float l_tot = half_sum(l);
    if (!row_ok) return;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    bf16_t* orow = a.o + (int64_t)(q_beg + i) * a.o_st + (int64_t)h * a.o_sh;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int n = nb * 32 + 8 * g + 4 * half;
            uint2 w;
            w.x = pack_bf16x2(acc[nb][4 * g] * inv, acc[nb][4 * g + 1] * inv);
            w.y = pack_bf16x2(acc[nb][4 * g + 2] * inv, acc[nb][4 * g + 3] * inv);
            *reinterpret_cast<uint2*>(orow + n) = w;
        }
    }
    if (a.lse != nullptr && half == 0) {
        const float lse = l_tot > 0.f ? kLn2 * (m + fast_log2(l_tot)) : neg_inf();
        if (a.lse_layout == 1) {
            a.lse[(int64_t)(q_beg + i) * a.hq + h] = lse;
        } else if (a.lse_layout == 2 && i < a.lse_s_max) {
            a.lse[((int64_t)b * a.lse_s_max + i) * a.hq + h] = lse;
        }
    }
}

template <int D, int BN>
hipError_t launch_d(const PrefillArgs& pa, hipStream_t s) {
    using C = PCfg<D, BN>;
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
    a.c = (pa.scale < 0.f ? -pa.scale : pa.scale) * kLog2e;
    a.q_sign = pa.scale < 0.f ? 0x80008000u : 0u;
    a.causal = pa.causal;
    a.lse = pa.lse;
    a.lse_layout = pa.lse_layout;
    a.lse_s_max = pa.lse_s_max;
    const int64_t n_wg = (int64_t)a.n_qtiles * a.n_hg * a.batch;
    if (n_wg == 0) return hipSuccess;
    // more than 64 KiB of dynamic LDS must be requested per kernel
    hipError_t e = hipFuncSetAttribute((const void*)prefill_bf16_kernel<D, BN>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prefill_bf16_kernel<D, BN>), dim3((unsigned)n_wg), dim3(kThreads),
                       (size_t)C::LDS_BYTES, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
    switch (a.dqk) {
        case 64: return launch_d<64, 128>(a, s);
        case 128: return launch_d<128, 64>(a, s);
        case 256: return launch_d<256, 32>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sdpa
