// decode_small.hip -- paged-KV decode for few query rows per KV head
// (s_q * G <= 16) at d_qk = d_v in {64, 128, 256}, e.g. single-token GQA
// decode: the HBM-streaming case.
//
// Same result as decode_paged.hip (per (b, KV head, split): the normalized
// partial O_c and its natural-log LSE_c over the chunk's visible keys, read
// through independent K and V page tables: cuDNN Frontend v1.31.0 Release
// Notes, "SDPA: paged KV, split-KV, and engine selection"), but the tile is
// sized to the live rows (v1.30.0 Release Notes, "New: decode tiles -- SDPA
// decode stops running the prefill pipeline"): 16 query columns on the
// 16x16 MFMA instead of 32-row prefill blocks.
//
// Work decomposition: one work-group (4 waves) per (b, KV head, split).  The
// four waves stream disjoint tiles of the chunk (wave w takes tiles w, w+4,
// ...) with no block-level barrier in the loop, each with its own online
// softmax state, and merge by LSE through LDS at the end.  Per tile of TK
// keys (TK * D = 4096, so one tile is 8 KB of K plus 8 KB of V):
//   - K goes straight from HBM into the MFMA A-operand registers
//     (S^T = K Q^T: lane (key, d-group) loads 16 contiguous bytes of its key
//     row), no LDS;
//   - V is loaded row-coalesced (16 lanes read one 256-byte row) and stored
//     as it is to a wave-private LDS tile (rows padded by 32 bytes, so the
//     4 rows x 32 bytes one 16-lane group reads below fall in distinct
//     banks); the second MFMA (O^T += V^T P^T) reads its A operand with
//     ds_read_b64_tr_b16, which hands each lane 4 consecutive keys of one
//     column (an earlier version transposed V in registers with v_perm and
//     wrote V^T: 16 more VALU and twice the LDS writes per 4 x 8 unit; the
//     FP8 decode workload ran 0.496 ms with it, 0.431 ms without);
//   - the next tile's loads are issued before the current tile is computed
//     (register double buffer) and page ids are fetched two tiles ahead with
//     scalar loads, so a wave keeps 16 KB in flight.
//
// Per-tensor FP8 (E4M3) instantiation (F8): Q, K and V are E4M3 codes that
// stand for descale_{q,k,v} times their values (cuDNN Frontend v1.31.0
// Release Notes, per-tensor FP8 D128 paged KV; v1.32.0 "SDPA: wider native
// forward support", paged per-tensor FP8 D256).  A tile holds the same keys
// as in bf16 at D = 128 (8 KB in flight) and twice the keys at D = 256 (16 KB
// in flight); S^T = K Q^T runs on the FP8 MFMA
// (v_mfma_f32_16x16x32_fp8_fp8, FP32 accumulator; its dot products are not
// fp32-exact, up to ~4e-5 of the sum of |products| off) with
// scale * descale_q * descale_k folded into the exponent; V codes are widened
// exactly to bf16 on their way into the V tile, so P V stays on the bf16
// MFMA with P in bf16, and descale_v multiplies the normalized output.
#include "sdpa_device.h"
#include "sdpa_launch.h"

#include <atomic>
#include <type_traits>

namespace sdpa {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16_k32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16_k16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// 16x16x32 on E4M3 codes: lane (row l % 16, k-group l / 16) holds 8 codes
__device__ __forceinline__ f32x4 mfma16_fp8(uint64_t a, uint64_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8((long)a, (long)b, c, 0, 0, 0);
}
struct SmallKArgs {
    const void* q;   // bf16, or E4M3 codes (F8)
    const void* kp;
    int64_t k_sp, k_st, k_sh;
    const void* vp;
    int64_t v_sp, v_st, v_sh;
    const int32_t* pt_k;
    const int32_t* pt_v;
    int32_t table_stride;
    const int32_t* seq_lens;
    int32_t batch, sq, hq, hkv, group, page, page_shift, splits, rows, n_units;
    int32_t n_rg;  // groups of 16 query rows per KV head (units per chunk)
    int32_t slot;  // work-queue counters used by this launch
    uint32_t gen;  // this launch's tag on those counters (never 0)
    int64_t total_rows;
    float scale_log2;
    int32_t causal;
    float* o_part;
    float* lse_part;
    bf16_t* o;
    float* lse;
    const float* descale_q;  // F8 only: one fp32 each
    const float* descale_k;
    const float* descale_v;
    int32_t window;          // left sliding window (0: none)
    const float* sinks;      // [hq] sink logits (natural-log units) or nullptr
    int32_t stats_log2;      // final LSE in base 2
};

constexpr int kWaves = 4;

// Work queue of the persistent decode grid: counter [slot][0] hands out
// units (ticket t: the t-th (sequence, KV head, split) in order of
// decreasing sequence length), counter [slot][1] counts work-groups that
// are done; the last one returns both to 0.  Every counter word carries the
// tag of the launch that owns it (high 32 bits) next to its count (low 32
// bits); launches take tags 1, 2, 3, ... and slot = tag % kQueueSlots, and a
// launch that finds a counter with another tag (0 after a reset, or left
// behind by a launch that never finished) takes it over (own_ticket).  Up to
// kQueueSlots decode calls may run at once on one device.
constexpr int kQueueSlots = 1024;
constexpr int kRankMax = 256;  // longest-first order for batches up to this size
__device__ __align__(256) uint64_t g_decode_queue[kQueueSlots][4];

// Launch tags 1, 2, 3, ... (0 marks a free counter), one sequence for every
// instantiation of the kernel: they all share g_decode_queue, so two launches
// in flight must never be handed the same tag and slot.
std::atomic<uint32_t> g_decode_seq{0};
uint32_t next_decode_tag() {
    uint32_t g = g_decode_seq.fetch_add(1u, std::memory_order_relaxed) + 1u;
    while (g == 0u) g = g_decode_seq.fetch_add(1u, std::memory_order_relaxed) + 1u;
    return g;
}

// Ticket request on a work-queue counter: the counter word before adding 1.
// A plain one-lane atomicAdd: this file is compiled without the wave-level
// atomic optimizer, so the compiler waits for the returned value only where
// it is used and keeps its register reserved until then.  (An asm atomic
// would hide the pending write from the register allocator, which could
// hand the register to another value before the atomic returns.)
__device__ __forceinline__ uint64_t ticket_async(uint64_t* ctr) {
    return atomicAdd(reinterpret_cast<unsigned long long*>(ctr), 1ull);
}
// The ticket that `old` (a value ticket_async returned) stands for in the
// launch tagged gen.  A counter that still carries another tag is taken
// over: replaced by (gen, 1), which hands out ticket 0.
__device__ __forceinline__ uint32_t own_ticket(uint64_t* ctr, uint64_t old, uint32_t gen) {
    auto* c = reinterpret_cast<unsigned long long*>(ctr);
    while ((uint32_t)(old >> 32) != gen) {
        const unsigned long long seen = old + 1;  // the word after our add, if untouched since
        const unsigned long long prev = atomicCAS(c, seen, ((unsigned long long)gen << 32) | 1ull);
        if (prev == seen) return 0u;
        // another work-group of this launch took the counter over (ask again), or
        // another request landed on the old value (retry the take-over on it)
        old = (uint32_t)(prev >> 32) == gen ? atomicAdd(c, 1ull) : prev - 1;
    }
    return (uint32_t)old;
}

// Fourth word of a raw buffer resource on gfx9-family parts (CDNA): no
// swizzle, 32-bit data format; the range check returns zeros past num_records.
constexpr int kRsrcWord3 = 0x00020000;
// Cache policy of the K/V loads: nontemporal (the nt bit).  Every K/V byte
// is read once per call, so keeping it in the caches only evicts other data:
// on an MI355X the paged decode workload ran at 75 % of HBM with nt loads
// against 69 % without (and a plain 4.45 GB read kernel at 92 % against 80 %).
constexpr int kStream = 2;

// Load of a kernel-invariant int32 (page table, lengths) at a wave-uniform
// index through the constant address space, so it becomes a scalar load.
__device__ __forceinline__ int32_t load_uniform(const int32_t* p, int64_t i) {
    return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

// D: the Q/K head dim; DV: the V/O head dim
template <int D, bool F8, int DV = D>
struct SmallCfg {
    static constexpr int EB = F8 ? 1 : 2;    // bytes per stored element
    // keys per wave tile: about 8 KB of K, in whole 16-key sub-blocks; 4 KB for
    // E4M3 at D <= 128 (32 keys at D = 128: the FP8 decode workload ran 0.416 ms
    // with them against 0.435 ms with 64)
    static constexpr int TK = (F8 && D <= 128 ? 4096 : 8192) / (EB * D) / 16 * 16;
    static constexpr int SB = TK / 16;       // 16-key sub-blocks per tile
    static constexpr int KK = D / 32;        // k-steps of S^T = K Q^T
    static constexpr int KL = EB * D / 64;   // 16-byte K loads per lane and sub-block
    static constexpr int NB = DV / 16;       // 16-row blocks of O^T
    static constexpr int VR = DV + 16;       // V row pitch in LDS (elements): 32 bytes of pad
    static constexpr int VU = TK * DV / 32 / 64;  // V units (4 keys x 8 columns) per lane
    static constexpr int WAVE_LDS = TK * VR;  // elements of one wave's V tile
    static constexpr int MERGE_BYTES = kWaves * 16 * DV * 4 + 2 * kWaves * 16 * 4;
    static constexpr int LDS_BYTES =
        (kWaves * WAVE_LDS * 2 > MERGE_BYTES) ? kWaves * WAVE_LDS * 2 : MERGE_BYTES;
    static_assert(SB >= 1 && VU >= 1, "tile shape");
};

// One wave's registers for one tile: K operands and raw V rows (8 columns of
// 4 keys per unit: 16 bytes a row in bf16, 8 in E4M3).
template <int D, bool F8, int DV>
struct TileRegs {
    uint4 k[SmallCfg<D, F8, DV>::SB][SmallCfg<D, F8, DV>::KL];
    typename std::conditional<F8, uint2, uint4>::type v[SmallCfg<D, F8, DV>::VU][4];
};

// One unit: the keys of split `split` of sequence b for KV head kvh.  The
// next unit's ticket (lane 0 of wave 0) is requested at the start and turned
// into next_unit during the merge; returns that unit (-1: none left).
template <int D, bool F8, int DV, class NextOf>
__device__ __attribute__((always_inline)) int decode_unit(const SmallKArgs& a, bf16_t* smem, const int b,
                                                          const int kvh, const int split, const int rg,
                                                          uint64_t* ctr, int* next_unit, NextOf&& next_of) {
    using C = SmallCfg<D, F8, DV>;
    constexpr int EB = C::EB;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15, g = lane >> 4;
    uint64_t ticket = 0;
    if (threadIdx.x == 0) ticket = ticket_async(ctr);

    // a length past the table's reach is clamped (the table is never read out of
    // bounds) and the sequence's rows are written as NaN (see the epilogue)
    const int L = min(load_uniform(a.seq_lens, b), a.table_stride * a.page);
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
    // query column c of the tile = row r0 + c of this KV head (row group rg): token
    // (r0 + c) / G, head kvh*G + (r0 + c) % G
    const int r0 = 16 * rg;
    const int nr = min(16, a.rows - r0);  // rows of this unit
    const bool row_ok = c < nr;
    const int rr = r0 + (row_ok ? c : 0);
    const int tok = rr / a.group;
    const int64_t grow = ((int64_t)b * a.sq + tok) * a.hq + kvh * a.group + rr % a.group;
    const int lim = min(hi - 1, a.causal ? L - a.sq + tok : L - 1);
    // keys every live row sees (the unit's first token has the earliest causal limit)
    const int nomask_end = max(lo, min(hi, a.causal ? L - a.sq + r0 / a.group + 1 : hi));
    // first key this lane's token sees (left window), and the largest first key
    // of the live tokens (the last token's): tiles starting below it need the
    // lower mask
    const int first = a.window > 0 ? L - a.sq + tok - a.window + 1 : INT32_MIN;
    const int first_max = a.window > 0 ? L - a.window : INT32_MIN;

    // Q^T operand, 16 bytes per load.  bf16: lane (q = c, d-group g) holds
    // d = 32 kl + 8 g .. +8 of its row for k-step kl.  E4M3: load kl holds
    // d = 64 kl + 16 g .. +16, its low / high 8 codes feed k-steps 2 kl and
    // 2 kl + 1 (K fragments are split the same way, so the dot product sums
    // every d once).
    uint4 qf[C::KL];
    {
        const char* qrow = reinterpret_cast<const char*>(a.q) + (grow * D) * EB + 16 * g;
#pragma unroll
        for (int kl = 0; kl < C::KL; ++kl) {
            uint4 w = {0u, 0u, 0u, 0u};
            if (row_ok) w = *reinterpret_cast<const uint4*>(qrow + 64 * kl);
            qf[kl] = w;
        }
    }
    // log2-domain logit scale: scale (x descale_q x descale_k for E4M3)
    float scale_log2 = a.scale_log2;
    float o_mul = 1.f;  // descale_v
    if constexpr (F8) {
        scale_log2 *= a.descale_q[0] * a.descale_k[0];
        o_mul = a.descale_v[0];
    }

    f32x4 acc[C::NB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = neg_inf(), l = 0.f;

    const int n_tiles = (hi - lo + C::TK - 1) / C::TK;
    const int32_t* ptk = a.pt_k + (int64_t)b * a.table_stride;
    const int32_t* ptv = a.pt_v + (int64_t)b * a.table_stride;
    const char* kbase = reinterpret_cast<const char*>(a.kp) + (int64_t)kvh * a.k_sh * EB;
    const char* vbase = reinterpret_cast<const char*>(a.vp) + (int64_t)kvh * a.v_sh * EB;
    // byte strides
    const int64_t k_sp2 = EB * a.k_sp, v_sp2 = EB * a.v_sp;
    const int k_st2 = EB * (int)a.k_st, v_st2 = EB * (int)a.v_st;
    bf16_t* vt = smem + wave * C::WAVE_LDS;
    // the last key index whose page may be looked up (the table is never read past it)
    const int last_key = max(hi - 1, 0);

    // Per-lane byte offsets inside a 16-key sub-block; all loop-invariant.
    //   K (A operand of S^T = K Q^T): lane (key c, d-group g) -> row c, bytes 16 g + 64 kl.
    //   V (row-coalesced 4 keys x 8 columns units): unit lane + 64 u.
    const int k_off = c * k_st2 + 16 * g;
    int v_off[C::VU], v_kt[C::VU], v_n8[C::VU];
#pragma unroll
    for (int u = 0; u < C::VU; ++u) {
        const int unitv = lane + 64 * u;
        v_n8[u] = unitv % (DV / 8);
        v_kt[u] = 4 * (unitv / (DV / 8));           // first key of the unit in the tile
        v_off[u] = (v_kt[u] & 15) * v_st2 + 8 * EB * v_n8[u];
    }

    // Buffer resources of one tile's 16-key sub-blocks.  The range of a
    // sub-block covers exactly its keys below hi, so lanes of masked keys
    // read zeros and a tile past the chunk moves no data at all.
    struct Rsrc {
        __amdgpu_buffer_rsrc_t k[C::SB], v[C::SB];
    };
    auto make_rsrc = [&](int t, Rsrc& rs) {
#pragma unroll
        for (int sb = 0; sb < C::SB; ++sb) {
            const int ks = lo + t * C::TK + 16 * sb;
            const int nvalid = min(max(hi - ks, 0), 16);
            const int kc = min(ks, last_key);
            const int pidx = a.page_shift >= 0 ? (kc >> a.page_shift) : kc / a.page;
            const int slot = ks - pidx * a.page;    // in [0, page) whenever nvalid > 0
            const int32_t pk = load_uniform(ptk, pidx);
            const int32_t pv = load_uniform(ptv, pidx);
            const int k_bytes = nvalid > 0 ? (nvalid - 1) * k_st2 + EB * D : 0;
            const int v_bytes = nvalid > 0 ? (nvalid - 1) * v_st2 + EB * DV : 0;
            rs.k[sb] = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(kbase + (int64_t)pk * k_sp2 + (int64_t)slot * k_st2), (short)0, k_bytes,
                kRsrcWord3);
            rs.v[sb] = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(vbase + (int64_t)pv * v_sp2 + (int64_t)slot * v_st2), (short)0, v_bytes,
                kRsrcWord3);
        }
    };
    auto issue = [&](const Rsrc& rs, TileRegs<D, F8, DV>& r) {
#pragma unroll
        for (int sb = 0; sb < C::SB; ++sb) {
#pragma unroll
            for (int kl = 0; kl < C::KL; ++kl)
                r.k[sb][kl] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(rs.k[sb], k_off + 64 * kl, 0, kStream));
        }
#pragma unroll
        for (int u = 0; u < C::VU; ++u) {
            // the 16-key sub-block of this lane's unit: one per 64 lanes for D >= 128;
            // at D = 64 a sub-block holds 32 units, so lanes 32..63 read the next one
            const int sb = (64 * u) / (DV / 2);
            auto vload = [&](const __amdgpu_buffer_rsrc_t& rv, int e) {
                if constexpr (F8)
                    r.v[u][e] = __builtin_bit_cast(
                        uint2, __builtin_amdgcn_raw_buffer_load_b64(rv, v_off[u], e * v_st2, kStream));
                else
                    r.v[u][e] = __builtin_bit_cast(
                        uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, v_off[u], e * v_st2, kStream));
            };
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (DV / 2 >= 64) {
                    vload(rs.v[sb], e);
                } else {
                    if (lane < 32)
                        vload(rs.v[sb], e);
                    else
                        vload(rs.v[sb + 1], e);
                }
            }
        }
    };
    auto compute = [&](int t, const TileRegs<D, F8, DV>& r) {
        const int key0 = lo + t * C::TK;
        // V rows -> this wave's LDS tile, row-major (E4M3 rows widened to bf16 first)
#pragma unroll
        for (int u = 0; u < C::VU; ++u) {
            const int kt = v_kt[u];
            uint4 vr[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (F8)
                    vr[e] = e4m3x8_to_bf16(r.v[u][e]);
                else
                    vr[e] = r.v[u][e];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
                *reinterpret_cast<uint4*>(vt + (kt + e) * C::VR + 8 * v_n8[u]) = vr[e];
        }
        // S^T = K Q^T: s[sb][r] is key key0 + 16 sb + 4 g + r of query c
        f32x4 s[C::SB];
#pragma unroll
        for (int sb = 0; sb < C::SB; ++sb) {
            s[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kl = 0; kl < C::KL; ++kl) {
                if constexpr (F8) {
                    const uint4 kw = r.k[sb][kl], qw = qf[kl];
                    s[sb] = mfma16_fp8((uint64_t)kw.y << 32 | kw.x, (uint64_t)qw.y << 32 | qw.x, s[sb]);
                    s[sb] = mfma16_fp8((uint64_t)kw.w << 32 | kw.z, (uint64_t)qw.w << 32 | qw.z, s[sb]);
                } else {
                    s[sb] = mfma16_k32(__builtin_bit_cast(bf16x8, r.k[sb][kl]),
                                       __builtin_bit_cast(bf16x8, qf[kl]), s[sb]);
                }
            }
        }
        const bool need_mask = key0 + C::TK > nomask_end || key0 < first_max;
        float mt = neg_inf();
#pragma unroll
        for (int sb = 0; sb < C::SB; ++sb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float x = s[sb][i] * scale_log2;
                if (need_mask) {
                    const int key = key0 + 16 * sb + 4 * g + i;
                    x = (key > lim || key < first) ? neg_inf() : x;
                }
                s[sb][i] = x;
                mt = fmaxf(mt, x);
            }
        }
        mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float m_new = fmaxf(m, mt);
        const float m_use = m_new == neg_inf() ? 0.f : m_new;
        const float alpha = fast_exp2(m - m_use);
        m = m_new;
        float lsum = 0.f;
        s16x4 pb[C::SB];
#pragma unroll
        for (int sb = 0; sb < C::SB; ++sb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = fast_exp2(s[sb][i] - m_use);
                lsum += p;
                pb[sb][i] = (short)f32_to_bf16_bits(p);
            }
        }
        l = l * alpha + lsum;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) acc[nb] *= alpha;
        // the V stores of all lanes land before any lane reads them
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        // O^T += V^T P^T: A = V^T[n = 16 nb + c][keys 16 sb + 4 g .. +4], read
        // transposed from the row-major tile
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
#pragma unroll
            for (int sb = 0; sb < C::SB; ++sb) {
                // lane (c, g) addresses row 16 sb + 4 g + c / 4, columns 16 nb + 4 (c % 4)
                // .. +3 and receives column 16 nb + c of rows 16 sb + 4 g .. +3
                const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)(vt + (16 * sb + 4 * g + c / 4) * C::VR + 16 * nb + 4 * (c % 4)));
                acc[nb] = mfma16_k16(va, pb[sb], acc[nb]);
            }
        }
        // keep the next tile's V stores behind this tile's reads
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    };

    // wave-private stream over tiles wave, wave + 4, ...; the loads of the
    // next tile are in flight while this one is computed.  Loop invariant at
    // the top: r0 holds (or is loading) tile t, ra is the resource set of
    // tile t + 4.
    {
        TileRegs<D, F8, DV> r0, r1;
        Rsrc ra, rb;
        int t = wave;
        make_rsrc(t, rb);
        make_rsrc(t + kWaves, ra);
        issue(rb, r0);
        while (t < n_tiles) {
            make_rsrc(t + 2 * kWaves, rb);
            issue(ra, r1);
            compute(t, r0);
            t += kWaves;
            if (t >= n_tiles) break;
            // r1 holds tile t, rb the resources of tile t + 4
            make_rsrc(t + 2 * kWaves, ra);
            issue(rb, r0);
            compute(t, r1);
            t += kWaves;
        }
    }

    // ---- merge the four waves by LSE and store -----------------------------
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    __syncthreads();  // every wave is done with its V tile
    float* red_o = reinterpret_cast<float*>(smem);              // [wave][q][n]
    float* red_m = red_o + kWaves * 16 * DV;                     // [wave][q]
    float* red_l = red_m + kWaves * 16;                          // [wave][q]
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
        *reinterpret_cast<f32x4*>(red_o + (wave * 16 + c) * DV + 16 * nb + 4 * g) = acc[nb];
    if (g == 0) {
        red_m[wave * 16 + c] = m;
        red_l[wave * 16 + c] = l;
    }
    // lane 0 of wave 0: the unit after this one (its ticket has returned:
    // every vector-memory operation of the wave is done by now)
    if (threadIdx.x == 0) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        *next_unit = next_of(ticket);
    }
    __syncthreads();
    const int nxt = *next_unit;
    const int items = nr * (DV / 4);
    for (int it = threadIdx.x; it < items; it += 256) {
        const int q = it / (DV / 4), n = 4 * (it % (DV / 4));
        float mw[kWaves];
        float M = neg_inf();
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            mw[w] = red_m[w * 16 + q];
            M = fmaxf(M, mw[w]);
        }
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
        float tot = 0.f;
        if (M != neg_inf()) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float sc = fast_exp2(mw[w] - M);  // exactly 0 for an empty wave
                tot += sc * red_l[w * 16 + q];
                o += sc * *reinterpret_cast<const f32x4*>(red_o + (w * 16 + q) * DV + n);
            }
        }
        const int t2 = (r0 + q) / a.group;
        const int hh = kvh * a.group + (r0 + q) % a.group;
        const int64_t row = ((int64_t)b * a.sq + t2) * a.hq + hh;
        float o_scale = o_mul;  // descale_v (1 unless FP8)
        if (a.sinks != nullptr && a.splits == 1) {
            // head hh's sink joins the denominator with no value (log2 units);
            // split partials leave it to the combine
            const float sk = a.sinks[hh] * kLog2e;
            const float M2 = fmaxf(M, sk);
            if (M2 != neg_inf()) {
                const float al = fast_exp2(M - M2);  // 0 when no key is visible
                tot = tot * al + fast_exp2(sk - M2);
                o_scale *= al;
                M = M2;
            }
        }
        float lse = neg_inf();
        if (tot > 0.f) {
            o *= o_scale / tot;
            const float lse2 = M + fast_log2(tot);
            // partials stay natural-log; the final Stats may be base 2
            lse = a.stats_log2 && a.splits == 1 ? lse2 : kLn2 * lse2;
        }
        if (load_uniform(a.seq_lens, b) > a.table_stride * a.page) {  // truncated: NaN rows
            o = f32x4{nan_f(), nan_f(), nan_f(), nan_f()};
            lse = nan_f();
        }
        if (a.splits > 1) {
            *reinterpret_cast<f32x4*>(a.o_part + ((int64_t)split * a.total_rows + row) * DV + n) = o;
            if (n == 0) a.lse_part[(int64_t)split * a.total_rows + row] = lse;
        } else {
            uint2 w;
            w.x = pack_bf16x2(o[0], o[1]);
            w.y = pack_bf16x2(o[2], o[3]);
            *reinterpret_cast<uint2*>(a.o + row * DV + n) = w;
            if (n == 0 && a.lse != nullptr) a.lse[row] = lse;
        }
    }
    return nxt;
}

// Persistent grid: each work-group runs units until the queue is empty,
// longest sequences first (every unit of a sequence has the same number of
// keys but the last split).
template <int D, bool F8, int DV>
__global__ __launch_bounds__(256, (D <= 192 ? 2 : 1)) void decode_small_kernel(SmallKArgs a) {
    extern __shared__ __attribute__((aligned(16))) bf16_t smem[];
    __shared__ int next_unit;
    __shared__ int by_len[kRankMax];  // by_len[r] = sequence with the r-th largest length
    uint64_t* const ctr = g_decode_queue[a.slot];
    const int per_kvh = a.splits * a.n_rg;
    const int per_seq = a.hkv * per_kvh;
    const bool ranked = a.batch <= kRankMax;
    if (ranked && (int)threadIdx.x < a.batch) {
        const int me = threadIdx.x;
        const int lm = a.seq_lens[me];
        int r = 0;
        for (int j = 0; j < a.batch; ++j) {
            const int lj = a.seq_lens[j];
            r += (lj > lm) || (lj == lm && j < me);
        }
        by_len[r] = me;
    }
    // unit of the ticket request `raw` (-1: the queue is empty)
    auto next_of = [&](uint64_t raw) -> int {
        const uint32_t t = own_ticket(&ctr[0], raw, a.gen);
        return t < (uint32_t)a.n_units ? (int)t : -1;
    };
    if (threadIdx.x == 0) next_unit = next_of(ticket_async(&ctr[0]));
    __syncthreads();
    int unit = next_unit;
    while (unit >= 0) {
        const int r = unit / per_seq, rem = unit - r * per_seq;
        const int b = ranked ? by_len[r] : r;
        // the row groups of a chunk take consecutive tickets (they read the same K/V)
        const int kvh = rem / per_kvh, rem2 = rem - kvh * per_kvh;
        const int split = rem2 / a.n_rg, rg = rem2 - split * a.n_rg;
        const int nxt = decode_unit<D, F8, DV>(a, smem, b, kvh, split, rg, &ctr[0], &next_unit, next_of);
        __syncthreads();  // the merge's LDS reads are done before the next unit's V stores
        unit = nxt;
    }
    if (threadIdx.x == 0 && own_ticket(&ctr[1], ticket_async(&ctr[1]), a.gen) == gridDim.x - 1) {
        // every work-group has taken its last ticket: the slot is free again
        atomicExch(reinterpret_cast<unsigned long long*>(&ctr[0]), 0ull);
        atomicExch(reinterpret_cast<unsigned long long*>(&ctr[1]), 0ull);
    }
}

template <int D, bool F8, int DV = D>
hipError_t launch_small_d(SmallKArgs a, hipStream_t s) {
    using C = SmallCfg<D, F8, DV>;
    if (a.n_units == 0) return hipSuccess;
    const void* kernel = (const void*)decode_small_kernel<D, F8, DV>;
    hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    // resident work-groups: per CU (computed once) x CUs of the device
    static std::atomic<int> per_cu{0};
    int occ = per_cu.load(std::memory_order_relaxed);
    if (occ == 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, 256, C::LDS_BYTES) != hipSuccess || occ < 1)
            occ = 1;
        per_cu.store(occ, std::memory_order_relaxed);
    }
    int dev = 0, n_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu < 1)
        n_cu = 1;
    const int64_t slots = (int64_t)occ * n_cu;
    const uint32_t gen = next_decode_tag();
    a.gen = gen;
    a.slot = (int32_t)(gen % kQueueSlots);
    hipLaunchKernelGGL((decode_small_kernel<D, F8, DV>), dim3((unsigned)(a.n_units < slots ? a.n_units : slots)), dim3(256),
                       (size_t)C::LDS_BYTES, s, a);
    return hipGetLastError();
}

}  // namespace

bool decode_small_supported(int32_t dqk, int32_t dv, int32_t rows) {
    return ((dqk == dv && (dqk == 64 || dqk == 128 || dqk == 256)) || (dqk == 192 && dv == 128)) &&
           rows <= kSmallRowsMax;
}

hipError_t launch_decode_small(const DecodeArgs& da, hipStream_t s) {
    SmallKArgs a;
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
    a.batch = da.batch;
    a.sq = da.sq;
    a.hq = da.hq;
    a.hkv = da.hkv;
    a.group = da.hq / da.hkv;
    a.page = da.page;
    a.page_shift = -1;
    for (int sh = 4; sh < 31; ++sh)
        if (da.page == (1 << sh)) a.page_shift = sh;
    a.splits = da.splits;
    a.rows = da.sq * a.group;
    a.n_rg = (a.rows + 15) / 16;
    a.n_units = da.batch * da.hkv * da.splits * a.n_rg;
    a.total_rows = (int64_t)da.batch * da.sq * da.hq;
    a.scale_log2 = da.scale * kLog2e;
    a.causal = da.causal;
    a.o_part = da.o_part;
    a.lse_part = da.lse_part;
    a.o = static_cast<bf16_t*>(da.o);
    a.lse = da.lse;
    a.descale_q = da.descale_q;
    a.descale_k = da.descale_k;
    a.descale_v = da.descale_v;
    // a window of 2^30 keys covers every key the int32 lengths can describe;
    // the clamp keeps L - s_q + t - W + 1 in range
    a.window = da.window > 0 ? min(da.window, 1 << 30) : 0;
    a.sinks = da.sinks;
    a.stats_log2 = da.stats_log2;
    if (da.fp8) {
        switch (da.dqk) {
            case 64: return launch_small_d<64, true>(a, s);
            case 192: return launch_small_d<192, true, 128>(a, s);
            case 128: return launch_small_d<128, true>(a, s);
            case 256: return launch_small_d<256, true>(a, s);
            default: return hipErrorInvalidValue;
        }
    }
    switch (da.dqk) {
        case 64: return launch_small_d<64, false>(a, s);
        case 192: return launch_small_d<192, false, 128>(a, s);
        case 128: return launch_small_d<128, false>(a, s);
        case 256: return launch_small_d<256, false>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sdpa
