// sdpa_device.h -- gfx950 device building blocks shared by the prefill and
// decode kernels: bf16 MFMA operand types, the LDS tile layouts, the
// cooperative HBM->LDS staging of a K/V tile, and the per-wave tile step
// (S^T = K Q^T on MFMA, online softmax in registers, O^T += V^T P^T on MFMA).
//
// Layout choice (CDNA4, wave64, v_mfma_f32_32x32x16_bf16):
//   A wave owns 32 query rows.  The score tile is computed TRANSPOSED,
//   S^T[key][query] = K Q^T, so that in the MFMA accumulator layout every
//   lane holds scores of ONE query (column = lane % 32) for 16 keys.  Row
//   max / row sum are then register reductions plus a single exchange with
//   lane ^ 32.  The output is likewise kept transposed, O^T[n][query] =
//   V^T P^T, so each lane's accumulators all belong to its own query and the
//   softmax rescale is a per-lane scalar multiply.  P^T feeds the second
//   MFMA straight from the first one's accumulators (converted to bf16), with
//   no LDS round trip; V is stored transposed in LDS with the keys of each
//   16-key group permuted to match the accumulator order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // storage type of a bfloat16 in memory

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }
// quiet NaN: the value of output rows a call cannot compute (a sequence longer
// than its page table reaches, THD rows past the grid that max_seqlen_q sizes)
__device__ __forceinline__ float nan_f() { return __builtin_nanf(""); }

// 8 OCP E4M3 codes -> 8 bf16 (gfx950's FP8 conversions read OCP E4M3), two
// codes per v_cvt_scalef32_pk_bf16_fp8 at scale 1.  Every E4M3 value has at
// most 4 significant bits and an exponent in [-9, 8], so it is exact in bf16;
// an in-bounds probe on gfx950 matched an exact host decode for all 256 codes
// in all four byte positions (the NaN code gives NaN).  (The older route,
// v_cvt_pk_f32_fp8 and the top halves of the two floats, takes twice the
// instructions, and in one probe kernel the compiler merged its two results
// into one operand of the packing v_perm.)
__device__ __forceinline__ uint4 e4m3x8_to_bf16(uint2 w) {
#define SDPA_E4M3X2(x, hi) __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((x), 1.0f, (hi)))
    return uint4{SDPA_E4M3X2(w.x, false), SDPA_E4M3X2(w.x, true), SDPA_E4M3X2(w.y, false),
                 SDPA_E4M3X2(w.y, true)};
#undef SDPA_E4M3X2
}

// Round-to-nearest-even float -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __builtin_bit_cast(float, b << 16);
}

__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32, 64); }

// ---- LDS tile geometry ---------------------------------------------------
// K tile: BK keys x DQK, row-major, pitch DQK + 8 elements (the 16-byte pad
// makes the 32 rows read by one MFMA operand fetch hit distinct banks).
// V^T tile: DV rows (n) x BK keys, pitch BK + 8; inside each 16-key group the
// 4-key runs are stored in the order 0, 2, 1, 3 (see vt_pos).
template <int DQK, int DV, int BK>
struct TileGeom {
    static constexpr int KP = DQK + 8;
    static constexpr int VP = BK + 8;
    static constexpr int K_ELEMS = BK * KP;
    static constexpr int V_ELEMS = DV * VP;
    static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
    static constexpr int BUF_BYTES = BUF_ELEMS * 2;
    static constexpr int K_CHUNKS = BK * DQK / 8;   // 16-byte pieces of a K tile
    static constexpr int V_UNITS = (BK / 4) * (DV / 8);  // 4 keys x 8 columns pieces
    static_assert(DQK % 16 == 0 && DV % 32 == 0 && BK % 32 == 0, "tile shape");
};

// Position of key kappa (0..15, relative to its 16-key group) inside the
// group in V^T: the MFMA accumulator of S^T gives lane half h the keys
// {4h..4h+3, 8+4h..8+4h+3} of each 16-key slice, in that order.
__device__ __forceinline__ int vt_pos(int kappa) {
    int a = kappa >> 2;
    return ((a & 1) << 3) | ((a >> 1) << 2) | (kappa & 3);
}

// Registers holding one thread's share of a K tile / a V tile between the
// HBM load and the LDS store.
template <int N>
struct KRegs {
    uint4 k[N > 0 ? N : 1];
};
template <int N>
struct VRegs {
    uint4 v[N > 0 ? N : 1][4];
};

template <int DQK, int DV, int BK, int NTHREADS>
struct TileShare {
    using G = TileGeom<DQK, DV, BK>;
    static constexpr int KC = (G::K_CHUNKS + NTHREADS - 1) / NTHREADS;
    static constexpr int VU = (G::V_UNITS + NTHREADS - 1) / NTHREADS;
};

// 8 elements of a row at element offset off: bf16, or (F8) 8 E4M3 codes
// widened exactly to bf16.
template <bool F8>
__device__ __forceinline__ uint4 load8(const void* __restrict__ base, int64_t off) {
    if constexpr (F8) {
        return e4m3x8_to_bf16(*reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(base) + off));
    } else {
        return *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(base) + off);
    }
}

// Issue the HBM loads of one thread's share of the K tile.  koff(j) returns
// the element offset of tile key j's K row, or -1 when key j is not to be
// read (past the range); such rows are zero-filled.  F8: the pool holds E4M3
// codes (one byte per element), widened to bf16 as they arrive.
template <int DQK, int DV, int BK, int NTHREADS, bool F8 = false, class KOff>
__device__ __forceinline__ void load_k_part(KRegs<TileShare<DQK, DV, BK, NTHREADS>::KC>& r,
                                            const void* __restrict__ kbase, int tid, KOff koff) {
    using G = TileGeom<DQK, DV, BK>;
    constexpr int KC = TileShare<DQK, DV, BK, NTHREADS>::KC;
    const uint4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
        int chunk = tid + c * NTHREADS;
        r.k[c] = zero;
        if (chunk < G::K_CHUNKS) {
            int row = chunk / (DQK / 8), cc = chunk % (DQK / 8);
            int64_t off = koff(row);
            if (off >= 0) r.k[c] = load8<F8>(kbase, off + cc * 8);
        }
    }
}

// Same for the V tile: a thread loads 4 consecutive keys x 8 columns.  Rows
// not read are zero: masked probabilities are exact zeros and must never
// multiply NaN garbage (0 * NaN = NaN).
template <int DQK, int DV, int BK, int NTHREADS, bool F8 = false, class VOff>
__device__ __forceinline__ void load_v_part(VRegs<TileShare<DQK, DV, BK, NTHREADS>::VU>& r,
                                            const void* __restrict__ vbase, int tid, VOff voff) {
    using G = TileGeom<DQK, DV, BK>;
    constexpr int VU = TileShare<DQK, DV, BK, NTHREADS>::VU;
    const uint4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < VU; ++u) {
        int unit = tid + u * NTHREADS;
#pragma unroll
        for (int e = 0; e < 4; ++e) r.v[u][e] = zero;
        if (unit < G::V_UNITS) {
            int ncc = unit % (DV / 8), kq = unit / (DV / 8);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                int64_t off = voff(kq * 4 + e);
                if (off >= 0) r.v[u][e] = load8<F8>(vbase, off + ncc * 8);
            }
        }
    }
}

// Store a K share into an LDS buffer (row-major, padded pitch).
template <int DQK, int DV, int BK, int NTHREADS>
__device__ __forceinline__ void store_k_part(const KRegs<TileShare<DQK, DV, BK, NTHREADS>::KC>& r,
                                             bf16_t* buf, int tid) {
    using G = TileGeom<DQK, DV, BK>;
    constexpr int KC = TileShare<DQK, DV, BK, NTHREADS>::KC;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
        int chunk = tid + c * NTHREADS;
        if (chunk < G::K_CHUNKS) {
            int row = chunk / (DQK / 8), cc = chunk % (DQK / 8);
            *reinterpret_cast<uint4*>(buf + row * G::KP + cc * 8) = r.k[c];
        }
    }
}

// Store a V share transposed (and key-permuted): for each of the 8 columns,
// the 4 keys' values go out as one 8-byte LDS store.
template <int DQK, int DV, int BK, int NTHREADS>
__device__ __forceinline__ void store_v_part(const VRegs<TileShare<DQK, DV, BK, NTHREADS>::VU>& r,
                                             bf16_t* buf, int tid) {
    using G = TileGeom<DQK, DV, BK>;
    constexpr int VU = TileShare<DQK, DV, BK, NTHREADS>::VU;
    bf16_t* vt = buf + G::K_ELEMS;
#pragma unroll
    for (int u = 0; u < VU; ++u) {
        int unit = tid + u * NTHREADS;
        if (unit < G::V_UNITS) {
            int ncc = unit % (DV / 8), kq = unit / (DV / 8);
            int key0 = kq * 4;
            int pos = (key0 & ~15) + vt_pos(key0 & 15);
            const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&r.v[u][0]);
            const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&r.v[u][1]);
            const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&r.v[u][2]);
            const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&r.v[u][3]);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                // columns n = ncc*8 + 2w (low halves) and 2w+1 (high halves)
                uint2 even, odd;
                even.x = (w0[w] & 0xffffu) | (w1[w] << 16);
                even.y = (w2[w] & 0xffffu) | (w3[w] << 16);
                odd.x = (w0[w] >> 16) | (w1[w] & 0xffff0000u);
                odd.y = (w2[w] >> 16) | (w3[w] & 0xffff0000u);
                int n = ncc * 8 + 2 * w;
                *reinterpret_cast<uint2*>(vt + n * G::VP + pos) = even;
                *reinterpret_cast<uint2*>(vt + (n + 1) * G::VP + pos) = odd;
            }
        }
    }
}

// Per-wave running state of 32 query rows (one per lane column; the two
// lane halves hold partial row sums over disjoint key subsets).
template <int DV>
struct RowState {
    f32x16 acc[DV / 32];  // O^T accumulators: n = nb*32 + 8*(r/4) + 4*half + r%4
    float m;              // running max of the log2-domain logits
    float l;              // this half's running sum of exp2(x - m)
};

template <int DV>
__device__ __forceinline__ void row_state_init(RowState<DV>& st) {
#pragma unroll
    for (int nb = 0; nb < DV / 32; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.acc[nb][r] = 0.f;
    st.m = neg_inf();
    st.l = 0.f;
}

// One KV tile for one wave.
//   ks/vt: the LDS tile; qf: the wave's Q^T operand (DQK/16 fragments);
//   key0: absolute index of the tile's first key; lim / first: last and first
//   key index this lane's query may see (keys > lim or < first are masked);
//   need_mask: false when every key of the tile is visible to every row.
template <int DQK, int DV, int BK>
__device__ __forceinline__ void tile_step(const bf16_t* __restrict__ ks,
                                          const bf16_t* __restrict__ vt, const bf16x8* qf,
                                          RowState<DV>& st, int key0, int lim, int first,
                                          bool need_mask, float scale_log2, int lane) {
    using G = TileGeom<DQK, DV, BK>;
    const int col = lane & 31, half = lane >> 5;
    constexpr int NB = BK / 32;
    f32x16 s[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
        const bf16_t* krow = ks + (kb * 32 + col) * G::KP + half * 8;
#pragma unroll
        for (int kk = 0; kk < DQK / 16; ++kk) {
            bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + kk * 16);
            s[kb] = mfma_32x32x16(a, qf[kk], s[kb]);
            // bound how far the scheduler hoists operand reads (register pressure)
            if ((kk & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
    }
    // log2-domain logits, masking, tile max
    float mt = neg_inf();
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float x = s[kb][r] * scale_log2;
            if (need_mask) {
                int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                x = (key > lim || key < first) ? neg_inf() : x;
            }
            s[kb][r] = x;
            mt = fmaxf(mt, x);
        }
    }
    mt = fmaxf(mt, xor32(mt));
    const float m_new = fmaxf(st.m, mt);
    const float m_use = m_new == neg_inf() ? 0.f : m_new;
    const float alpha = fast_exp2(st.m - m_use);
    st.m = m_new;
    float lsum = 0.f;
    bf16x8 pb[BK / 16];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float p = fast_exp2(s[kb][r] - m_use);
            lsum += p;
            pb[kb * 2 + (r >> 3)][r & 7] = (__bf16)p;
        }
    }
    st.l = st.l * alpha + lsum;
#pragma unroll
    for (int nb = 0; nb < DV / 32; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.acc[nb][r] *= alpha;
#pragma unroll
    for (int nb = 0; nb < DV / 32; ++nb) {
        const bf16_t* vrow = vt + (nb * 32 + col) * G::VP + half * 8;
#pragma unroll
        for (int kst = 0; kst < BK / 16; ++kst) {
            bf16x8 a = *reinterpret_cast<const bf16x8*>(vrow + kst * 16);
            st.acc[nb] = mfma_32x32x16(a, pb[kst], st.acc[nb]);
        }
        if ((nb & 1) == 1) __builtin_amdgcn_sched_barrier(0);
    }
}

// Load the wave's Q^T operand: lane (col, half) gets query row `col`'s
// elements kk*16 + half*8 .. +8 for every kk (F8: codes widened to bf16).
// Rows not present are zero.
template <int DQK, bool F8 = false>
__device__ __forceinline__ void load_q(bf16x8* qf, const void* qrow, bool ok, int lane) {
    const int half = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < DQK / 16; ++kk) {
        uint4 w = {0u, 0u, 0u, 0u};
        if (ok) w = load8<F8>(qrow, kk * 16 + half * 8);
        qf[kk] = __builtin_bit_cast(bf16x8, w);
    }
}

// Final row sum (both halves) of a lane's query.
template <int DV>
__device__ __forceinline__ float row_total(const RowState<DV>& st) {
    return st.l + xor32(st.l);
}

}  // namespace sdpa
