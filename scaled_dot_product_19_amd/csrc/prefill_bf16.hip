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
// Work-group = NW waves of 32 query rows sharing one KV head (NW = 8 for
// D <= 128, 4 for D = 256): NH query heads of one GQA group x (NW / NH)
// blocks of 32 consecutive tokens, NH = largest of {4, 2, 1} dividing G, so
// every K/V tile staged in LDS serves NH heads (partial GQA packing: v1.30.0
// "New: decode tiles", Partial PackGQA bullet).  Items are handed out
// longest causal row block first.
//
// K/V staging (gfx950 LDS DMA).  Tiles of BN keys go from HBM straight into
// LDS with buffer_load_dwordx4 ... lds: each lane's 16 bytes land at
// LDS base + 16 * lane, so a wave instruction fills 1 KB.  Both tiles stay
// row-major; bank conflicts are avoided by choosing, per lane, which 16-byte
// chunk of which row it fetches (an XOR swizzle of the chunk index by the
// row).  The buffer range of a tile ends with its last row below kv_end, so
// rows past it arrive as zeros and a tile past the end moves no data.  An
// S-stage LDS ring keeps S - 1 tiles in flight.
//
// Per wave and tile (v_mfma_f32_32x32x16_bf16, wave64):
//   S^T[key][q] = K Q^T  -- A = K rows (ds_read_b128), B = the wave's Q^T in
//                           registers; each lane holds the scores of ONE
//                           query (column lane % 32);
//   online softmax       -- raw row max (3-input max), one lane-half exchange
//                           (v_permlane32_swap), p = exp2(s * c - m) as one
//                           FMA + exp; the running max only moves when a
//                           tile's max exceeds it by more than 8 (log2 units),
//                           which leaves the result exactly the same;
//   O^T[n][q] += V^T P^T -- B = P^T straight from the score accumulators
//                           (bf16); A = V^T read from the row-major V tile
//                           with ds_read_b64_tr_b16, which hands each lane
//                           four consecutive keys of one column.
//
// Per-tensor FP8 (E4M3) instantiation (F8, D = 128): Q, K and V are E4M3
// codes standing for descale_{q,k,v} times their values (cuDNN Frontend
// v1.31.0 Release Notes, per-tensor FP8 D128; the SM120 per-tensor E4M3
// forward engine).  K and V tiles arrive as codes (half the DMA bytes);
// S^T = K Q^T runs on the FP8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4 with
// unit scales: four times the K depth of the bf16 MFMA per instruction),
// scale * descale_q * descale_k folded into the exponent.  Each V tile is
// widened exactly to a bf16 V tile in LDS, half by each wave group during
// its softmax phase, so P V stays on the bf16 MFMA with P in bf16;
// descale_v multiplies the normalized output.
#include "sdpa_device.h"
#include "sdpa_launch.h"
#include "tile_ops.h"

#include <atomic>
#include <type_traits>

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
    uint32_t q_sign;  // sign bits of every element when scale < 0 (Q is negated on load), else 0
    const float* descale_q;  // F8 only: one fp32 each, read on the device
    const float* descale_k;
    const float* descale_v;
    int32_t causal;
    float* lse;
    int32_t lse_layout, lse_s_max;  // layout 3 (head-major): lse_s_max = per-head stride
    int32_t window;                 // left sliding window (0: none)
    const float* sinks;             // [hq] sink logits (natural-log units) or nullptr
    int32_t stats_log2;             // LSE in base 2
    int32_t slot;    // work-queue counters used by this launch
    uint32_t gen;    // this launch's tag on those counters (never 0)
    // paged mode (chunked prefill over a paged cache; see launch_prefill_paged):
    // Q [batch, sq, hq, D] dense, K/V rows through independent page tables,
    // key range split in `splits` chunks, fp32 partials when splits > 1
    const int32_t* pt_k;
    const int32_t* pt_v;
    const int32_t* seq_lens;
    int64_t k_sp, v_sp;      // page strides (elements)
    int32_t table_stride, page, sq, splits;
    // folded rows: the item's rows are (token, head) pairs of `fold` heads,
    // token-major (row r = token r / fold of head fold hg + r % fold), so that
    // few query tokens of a whole GQA group still fill the 32-row blocks;
    // 1 = one head per wave, rows = tokens
    int32_t fold = 1;
    int64_t total_rows;      // batch * sq * hq
    float* o_part;           // [splits, total_rows, D]
    float* lse_part;         // [splits, total_rows]
};

// Work queues of the persistent prefill grid, one per XCD.  Pair p = (b, hg)
// lives on XCD p % 8, so the K/V of a head group stays in one XCD's L2; the
// queue of XCD x hands out its items level by level (longest causal row
// blocks first): ticket t -> level t / m, pair x + 8 (t % m), with m the
// number of pairs of XCD x.  A work-group takes tickets from the queue of
// the XCD it runs on and, once that is empty, from the other seven in turn.
// Counter [slot][8] counts work-groups that are done; the last one returns
// all counters of the slot to 0.
//
// Every counter word carries the tag of the launch that owns it (high 32
// bits) next to its count (low 32 bits).  Launches take tags 1, 2, 3, ...
// and slot = tag % kQueueSlots; a launch that finds a counter with another
// tag (0 after a reset, or left behind by a launch that never finished)
// takes it over (own_ticket), so no earlier launch can leave a slot that
// makes a later one skip work.  Up to kQueueSlots prefill calls may run at
// once on one device.
constexpr int kQueueSlots = 1024;
constexpr int kXcds = 8;
__device__ __align__(256) uint64_t g_prefill_queue[kQueueSlots][16];

constexpr float kLazyRescale = 8.f;  // log2 units the running max may lag behind

typedef int i32x8 __attribute__((ext_vector_type(8)));
// 32x32x64 on E4M3 codes (format 0 for A and B), unit block scales (E8M0 127)
__device__ __forceinline__ f32x16 mfma_32x32x64_fp8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0x7f7f7f7f, 0, 0x7f7f7f7f);
}
constexpr int kWin = 4;              // LDS operand fragments read ahead of the MFMAs
template <int D, int BN, int S, int NW, bool F8 = false>
struct PCfg {
    static constexpr int THREADS = 64 * NW;
    static constexpr int EB = F8 ? 1 : 2;              // bytes per stored element
    static constexpr int CPR = EB * D / 16;            // 16-byte chunks per stored row
    static constexpr int ROW_B = EB * D;               // bytes per stored row
    static constexpr int TILE_B = BN * ROW_B;          // bytes of a stored K (or V) tile
    static constexpr int VROW_B = 2 * D;               // bytes per bf16 V row
    static constexpr int VCPR = D / 8;                 // 16-byte chunks per bf16 V row
    // stage: K tile, V tile (as stored), then for F8 the V tile widened to bf16
    static constexpr int VOFF = F8 ? 2 * TILE_B : TILE_B;  // bf16 V tile in a stage
    static constexpr int STAGE_B = F8 ? 2 * TILE_B + BN * VROW_B : 2 * TILE_B;
    static constexpr int LDS_BYTES = S * STAGE_B;
    static constexpr int KK8 = D / 64;                 // k-steps of the FP8 MFMA
    static constexpr int NI = TILE_B / 1024 / NW;      // LDS DMA instructions per wave per tile
    static constexpr int NKB = BN / 32;                // 32-key blocks of a tile
    static constexpr int NB = D / 32;                  // 32-row blocks of O^T
    static constexpr int KK = D / 16;                  // k-steps of S^T = K Q^T
    static_assert(NI >= 1 && TILE_B % (1024 * NW) == 0, "tile must fill whole DMA instructions");
    static_assert(BN % 32 == 0 && D % 32 == 0 && CPR >= 8, "tile shape");
};

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
__device__ __forceinline__ uint32_t own_ticket_slow(uint64_t* ctr, uint64_t old, uint32_t gen) {
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
__device__ __forceinline__ uint32_t own_ticket(uint64_t* ctr, uint64_t old, uint32_t gen) {
    return (uint32_t)(old >> 32) == gen ? (uint32_t)old : own_ticket_slow(ctr, old, gen);
}

// D <= 128: compiled for at least two waves per SIMD (the launch bound's
// second argument), i.e. up to 256 VGPR + AGPR per lane; the 4-stage 128 KiB
// ring admits one work-group per CU, whose 8 waves run two per SIMD.  D = 256:
// one 4-wave work-group per CU, one wave per SIMD, with the O^T accumulators
// in AGPRs.
// NW waves = 32 NW query rows per work-group, each wave 32 rows.
// CZ: the scale is 0 (every logit is 0; masked keys need explicit zeros)
// PP: ping-pong schedule (NW = 8, two waves per SIMD); otherwise sequential.
// One work item: NH heads x NW / NH blocks of 32 query rows of one sequence,
// all keys it sees.  Uniform across the work-group (every exit is taken by
// all waves).  On return every LDS DMA of the item has landed.  An item with
// rows calls before_epilogue() once its last tile is done and before any of
// its stores are issued.
template <int D, int BN, int S, int NW, bool PP, bool CZ, bool PAGED, bool F8, typename Hook>
__device__ __attribute__((always_inline)) void prefill_item(const PrefillKArgs& a, const int item,
                                                            char* const lds, const uint32_t lds_base,
                                                            uint64_t* const tctr, uint64_t& ticket,
                                                            Hook&& before_epilogue) {
    static_assert(!PP || (NW == 8 && S >= 4), "ping-pong needs two wave groups and S >= 4");
    static_assert(!F8 || (PP && D == 128), "FP8: the D = 128 ping-pong kernel");
    using C = PCfg<D, BN, S, NW, F8>;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // item = level * n_pairs + pair: level = causal row block counted from
    // the last (longest first), pair = b * n_hg + hg (paged: (b * n_hg + hg)
    // * splits + split)
    const int bid = __builtin_amdgcn_readfirstlane(item);
    const int n_pairs = a.batch * a.n_hg * (PAGED ? a.splits : 1);
    const int level = bid / n_pairs;
    const int pair = bid - level * n_pairs;
    const int bh = PAGED ? pair / a.splits : pair;
    const int split = PAGED ? pair - bh * a.splits : 0;
    const int b = bh / a.n_hg;
    const int hg = bh - b * a.n_hg;
    const int qt = a.n_qtiles - 1 - level;

    // rows [q_beg, q_beg + lq) and keys [kv_beg, kv_beg + lk) of the sequence;
    // this item sees keys [lo, hi) of it (the split's chunk when paged)
    int q_beg, lq, kv_beg, lk, lo = 0, hi;
    bool trunc = false;  // paged: seq_lens past the table's reach (rows become NaN)
    if constexpr (PAGED) {
        q_beg = b * a.sq;
        lq = a.sq;
        kv_beg = 0;
        // a length past the table's reach is clamped (the table is never read
        // out of bounds) and the sequence's rows are written as NaN
        const int len = load_uniform(a.seq_lens, b);
        trunc = len > a.table_stride * a.page;
        lk = min(len, a.table_stride * a.page);
        hi = lk;
        if (a.splits > 1) {
            // keys [base, lk) are cut into the splits; with a left window, base is
            // the start of the page holding the first key any query token sees
            int base = 0;
            if (a.window > 0 && lk - lq - a.window + 1 > 0) base = ((lk - lq - a.window + 1) / a.page) * a.page;
            const int per = (lk - base + a.splits - 1) / a.splits;
            const int chunk = ((per + a.page - 1) / a.page) * a.page;
            lo = min(lk, base + split * chunk);
            hi = min(lk, lo + chunk);
        }
    } else {
        q_beg = load_uniform(a.cu_q, b);
        lq = load_uniform(a.cu_q, b + 1) - q_beg;
        kv_beg = load_uniform(a.cu_kv, b);
        lk = load_uniform(a.cu_kv, b + 1) - kv_beg;
        hi = lk;
    }
    const int nt = NW / a.nh;
    // rows of the sequence for one head (fg = 1) or one head group (folded)
    const int fg = PAGED ? a.fold : 1;
    const int n_rows = lq * fg;
    const int q0 = qt * 32 * nt;  // the item's first row
    if (q0 >= n_rows) {  // uniform across the work-group
        if (tid == 0) ticket = ticket_async(tctr);
        wait_vmcnt<0>();
        return;
    }

    const int hw = wave % a.nh, tb = wave / a.nh;
    const int hb = (hg * a.nh + hw) * fg;  // the wave's head, or first head of its group
    const int kvh = hb / a.group;
    const int i0 = q0 + tb * 32;  // the wave's first row
    const int col = lane & 31, half = lane >> 5;
    const int ri = i0 + col;  // this lane's row: query token i of head h
    const int i = ri / fg;
    const int h = hb + (ri - i * fg);
    const bool row_ok = ri < n_rows;
    // a wave without rows (a folded item's or a sequence's last row block)
    // still issues its share of every tile's DMA but runs no MFMA
    const bool idle = i0 >= n_rows;
    const int shift = lk - lq;  // bottom-right diagonal offset

    // left sliding window: row i sees keys >= i + shift - W + 1, so the item
    // starts at the first tile holding a key of its first row's window
    if (a.window > 0) lo = max(lo, ((max(0, (q0 / fg) + shift - a.window + 1)) / BN) * BN);
    // key extents within [lo, hi): the work-group's, this wave's, and this lane's
    // (from the query tokens of their first and last rows)
    const int last_wg = (min(q0 + 32 * nt, n_rows) - 1) / fg;
    const int kv_end = a.causal ? max(lo, min(hi, last_wg + shift + 1)) : hi;
    int kv_end_w = lo, nomask_end = lo, kv_beg_w = lo;
    if (i0 < n_rows) {
        const int first_w = i0 / fg;
        // with a window, tiles that end before the wave's first visible key are skipped
        if (a.window > 0) kv_beg_w = max(lo, first_w + shift - a.window + 1);
        const int last_w = (min(i0 + 32, n_rows) - 1) / fg;
        kv_end_w = a.causal ? max(lo, min(hi, last_w + shift + 1)) : hi;
        nomask_end = a.causal ? max(lo, min(hi, first_w + shift + 1)) : hi;
    }
    const int lim = a.causal ? min(hi - 1, i + shift) : hi - 1;
    // first visible key of this lane's row, and the largest of the wave's rows:
    // tiles starting below it need the lower mask
    const int first = i + shift - a.window + 1;  // used only with a window
    const int first_w_max = a.window > 0 ? (min(i0 + 31, n_rows - 1) / fg) + shift - a.window + 1 : INT32_MIN;
    // the tile starting at key0 holds keys of this wave, and needs the mask
    auto sees = [&](int key0) __attribute__((always_inline)) {
        return key0 < kv_end_w && key0 + BN > kv_beg_w;
    };
    auto masked = [&](int key0) __attribute__((always_inline)) {
        return key0 + BN > nomask_end || key0 < first_w_max;
    };
    const int n_tiles = (kv_end - lo + BN - 1) / BN;  // tile t: keys lo + t BN ..

    // ---- LDS DMA of the K/V tiles -------------------------------------------
    // Wave w's instruction j fills bytes [(w NI + j) KiB, +1 KiB) of a tile;
    // lane L of it writes chunk position p = (w NI + j) * 64 + L, i.e. row
    // p / CPR, physical chunk p % CPR, and so fetches logical chunk
    // swz(row, p % CPR) of that row.  These byte offsets never change.
    const char* kb0 = reinterpret_cast<const char*>(a.k) + C::EB * ((int64_t)kv_beg * a.k_st + (int64_t)kvh * a.k_sh);
    const char* vb0 = reinterpret_cast<const char*>(a.v) + C::EB * ((int64_t)kv_beg * a.v_st + (int64_t)kvh * a.v_sh);
    const int k_st2 = C::EB * (int)a.k_st, v_st2 = C::EB * (int)a.v_st;  // byte strides
    // Paged: a wave's instructions cover exactly its 8 rows 8 w .. 8 w + 7 of
    // a tile, which lie in one page (page_size % 8 == 0, tiles start on
    // multiples of 8 keys), so each wave reads through its own page and its
    // source offsets count from its first row; the swizzle follows the row
    // within the tile.
    constexpr int RW = C::NI * 64 / C::CPR;  // tile rows per wave
    static_assert(!PAGED || RW == 8, "paged DMA: 8 rows per wave");
    const int row0 = PAGED ? RW * wave : 0;
    int k_src[C::NI], v_src[C::NI];
#pragma unroll
    for (int j = 0; j < C::NI; ++j) {
        const int p = (wave * C::NI + j) * 64 + lane;
        const int row = p / C::CPR, pc = p % C::CPR;
        k_src[j] = (row - row0) * k_st2 + 16 * swz_k<C::CPR>(row, pc);
        // an FP8 V tile stays unswizzled: it is only read row-contiguously, by the widening
        v_src[j] = (row - row0) * v_st2 + 16 * (F8 ? pc : swz_v<C::CPR>(row, pc));
    }
    // Paged: the K and V page ids of the next tile to be issued (scalar
    // loads).  An outstanding scalar load makes every later LDS wait a full
    // lgkmcnt(0), so in the ping-pong schedule the loads are started at the
    // beginning of a VALU phase (which reads no LDS) and waited for at its end.
    int pk_nx = 0, pv_nx = 0;
    const int32_t* const ptk_b = PAGED ? a.pt_k + (int64_t)b * a.table_stride : nullptr;
    const int32_t* const ptv_b = PAGED ? a.pt_v + (int64_t)b * a.table_stride : nullptr;
    auto page_ids = [&](int t) __attribute__((always_inline)) {
        if constexpr (PAGED) {
            const int k0 = lo + t * BN + row0;  // the wave's first key of the tile
            const int e = k0 < kv_end ? k0 / a.page : 0;  // rows past the end read no page
            pk_nx = load_uniform(ptk_b, e);
            pv_nx = load_uniform(ptv_b, e);
        }
    };
    auto page_ids_ready = [&]() __attribute__((always_inline)) {
        if constexpr (PAGED) asm volatile("" ::"s"(pk_nx), "s"(pv_nx));
    };
    auto issue = [&](int t) __attribute__((always_inline)) {
        // a tile at or past kv_end gets an empty range: its DMA writes zeros
        // and reads nothing
        const int k0 = lo + t * BN + row0;  // paged: the wave's first key
        const int nvalid = min(PAGED ? RW : BN, kv_end - k0);
        const void* kt;
        const void* vt;
        if constexpr (PAGED) {
            // the wave's rows lie in one page (K and V pages looked up
            // independently)
            const int64_t in_page = nvalid > 0 ? k0 % a.page : 0;
            kt = reinterpret_cast<const char*>(a.k) +
                 C::EB * ((int64_t)pk_nx * a.k_sp + in_page * a.k_st + (int64_t)kvh * a.k_sh);
            vt = reinterpret_cast<const char*>(a.v) +
                 C::EB * ((int64_t)pv_nx * a.v_sp + in_page * a.v_st + (int64_t)kvh * a.v_sh);
        } else {
            kt = kb0 + (int64_t)k0 * k_st2;
            vt = vb0 + (int64_t)k0 * v_st2;
        }
        const u32x4 kr = make_rsrc(kt, nvalid > 0 ? (nvalid - 1) * k_st2 + C::ROW_B : 0);
        const u32x4 vr = make_rsrc(vt, nvalid > 0 ? (nvalid - 1) * v_st2 + C::ROW_B : 0);
        const uint32_t st = lds_base + (t % S) * C::STAGE_B + wave * C::NI * 1024;
#pragma unroll
        for (int j = 0; j < C::NI; ++j) dma16(kr, st + j * 1024, k_src[j]);
#pragma unroll
        for (int j = 0; j < C::NI; ++j) dma16(vr, st + C::TILE_B + j * 1024, v_src[j]);
    };
    // start the first tiles before the Q load so they overlap it (S - 1 ahead
    // in the sequential ring, S - 2 in the ping-pong one)
#pragma unroll
    for (int t = 0; t < (PP ? S - 2 : S - 1); ++t) {
        page_ids(t);
        page_ids_ready();
        issue(t);
    }
    if constexpr (PP) page_ids(S - 2);  // for M(0)

    // log2-domain logit scale and the sign flip of Q; FP8 folds in
    // descale_q * descale_k (a negative product flips Q like a negative scale)
    float c = a.c;
    uint32_t q_sign = a.q_sign;
    float o_mul = 1.f;  // descale_v
    if constexpr (F8) {
        const float dqk = a.descale_q[0] * a.descale_k[0];
        c *= fabsf(dqk);
        if (dqk < 0.f) q_sign ^= 0x80808080u;
        o_mul = a.descale_v[0];
    }
    // Q^T operand.  bf16: lane (col, half) holds d = 16 kk + 8 half .. +8 of
    // row i.  FP8: for k-step kk it holds the 32 codes d = 64 kk + 32 half ..
    // +32; the K fragment of the same lane half covers the same d (the FP8
    // MFMA pairs the bytes of A and B lanes of equal half one to one).
    constexpr int NQF = F8 ? 1 : C::KK;
    constexpr int NQF8 = F8 ? C::KK8 : 1;
    bf16x8 qf[NQF];
    i32x8 qf8[NQF8];
    {
        const char* qrow = reinterpret_cast<const char*>(a.q) +
                           C::EB * ((int64_t)(q_beg + i) * a.q_st + (int64_t)h * a.q_sh);
        if constexpr (F8) {
#pragma unroll
            for (int kk = 0; kk < C::KK8; ++kk) {
                uint4 w0 = {0u, 0u, 0u, 0u}, w1 = {0u, 0u, 0u, 0u};
                if (row_ok) {
                    w0 = *reinterpret_cast<const uint4*>(qrow + 64 * kk + 32 * half);
                    w1 = *reinterpret_cast<const uint4*>(qrow + 64 * kk + 32 * half + 16);
                }
                qf8[kk] = i32x8{(int)(w0.x ^ q_sign), (int)(w0.y ^ q_sign), (int)(w0.z ^ q_sign),
                                (int)(w0.w ^ q_sign), (int)(w1.x ^ q_sign), (int)(w1.y ^ q_sign),
                                (int)(w1.z ^ q_sign), (int)(w1.w ^ q_sign)};
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < C::KK; ++kk) {
                uint4 w = {0u, 0u, 0u, 0u};
                if (row_ok) w = *reinterpret_cast<const uint4*>(qrow + 32 * kk + 16 * half);
                w.x ^= q_sign;
                w.y ^= q_sign;
                w.z ^= q_sign;
                w.w ^= q_sign;
                qf[kk] = __builtin_bit_cast(bf16x8, w);
            }
        }
    }

    // ---- per-lane LDS read offsets (bytes within a stage) -------------------
    // K fragment (A of S^T): lane (key = col, half) reads logical chunk
    // 2 kk + half of row 32 kb + col.  The swizzle depends on the row only
    // modulo 16, so block kb adds 32 rows and kk >= 8 adds 16 chunks exactly.
    constexpr int KKW = C::KK < 8 ? C::KK : 8;
    int k_rd[KKW];
#pragma unroll
    for (int kk = 0; kk < KKW; ++kk)
        k_rd[kk] = col * C::ROW_B + 16 * swz_k<C::CPR>(col, 2 * kk + half);
    // FP8 K fragment: lane (key = col, half) reads logical chunks 4 kk + 2 half
    // and + 1 (32 codes) of row 32 kb + col; the swizzle depends on the row
    // modulo 16 only, so block kb adds 32 rows exactly.
    constexpr int NK8 = F8 ? 2 * C::KK8 : 1;
    int k_rd8[NK8];
#pragma unroll
    for (int j = 0; j < NK8; ++j)
        k_rd8[j] = col * C::ROW_B + 16 * swz_k<C::CPR>(col, 4 * (j / 2) + 2 * half + (j % 2));
    // V^T fragment (A of O^T), two transpose reads per 16-key step: lane l of
    // 16-lane group G = l / 16 supplies row 16 kst + 4 half + (l % 16) / 4
    // (+8 for the second read) and the 4 columns starting at
    // 32 nb + 16 (G % 2) + 4 (l % 4); it receives 4 consecutive keys of
    // column 32 nb + l % 32.  The swizzle depends on the row modulo 4 only,
    // and 32-column blocks nb >= 4 sit 16 chunks further.
    constexpr int NBW = C::NB < 4 ? C::NB : 4;
    int v_rd[NBW];
    {
        const int r0 = 4 * half + (lane & 15) / 4;
        const int cg = 2 * ((lane >> 4) & 1) + (lane & 3) / 2;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
            v_rd[nb] = C::VOFF + r0 * C::VROW_B + 16 * swz_v<C::VCPR>(r0, 4 * nb + cg) +
                       8 * (lane & 1);
    }

    f32x16 acc[C::NB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[nb][r] = 0.f;
    float m = neg_inf();  // running max (log2 units) of this lane's query
    float l = 0.f;        // this lane half's running sum

    // ---- the three parts of a tile for this wave ------------------------------
    // QK: s = S^T = K Q^T of the tile in stage st.  MFMA o works on key block
    // o % NKB (consecutive MFMAs use independent accumulators) and reads its
    // K fragment kWin steps ahead.
    constexpr int NQK = C::NKB * C::KK;
    constexpr int NPV = C::NB * (BN / 16);
    // K fragment of QK MFMA o (key block o % NKB, k-step o / NKB) in stage st
    auto kfrag_at = [&](const char* st, int o) __attribute__((always_inline)) {
        const int kb = o % C::NKB, kk = o / C::NKB;
        return *reinterpret_cast<const bf16x8*>(st + k_rd[kk % KKW] + kb * 32 * C::ROW_B + (kk / KKW) * 256);
    };
    // V^T fragment of PV MFMA o (output block o % NB, 16-key step o / NB):
    // two transpose reads
    auto vfrag_at = [&](const char* st, int o) __attribute__((always_inline)) {
        const int nb = o % C::NB, kst = o / C::NB;
        const char* vp = st + v_rd[nb % NBW] + (nb / NBW) * 256 + kst * 16 * C::VROW_B;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 8 * C::VROW_B));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto qk = [&](const char* st, f32x16(&s)[C::NKB]) __attribute__((always_inline)) {
        auto kfrag = [&](int o) __attribute__((always_inline)) { return kfrag_at(st, o); };
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
        __builtin_amdgcn_sched_group_barrier(0x100, kWin, 0);
#pragma unroll
        for (int o = 0; o < NQK; ++o) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (o + kWin < NQK) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    };
    // FP8 QK: NKB x KK8 MFMAs of 32x32x64, each with a 32-code K fragment
    // (two 16-byte reads); all fragments are read first.
    auto qk8 = [&](const char* st, f32x16(&s)[C::NKB]) __attribute__((always_inline)) {
        if constexpr (F8) {
            constexpr int N8 = C::NKB * C::KK8;
            const f32x16 zero = {};
            i32x8 fk[N8];
#pragma unroll
            for (int o = 0; o < N8; ++o) {
                const int kb = o % C::NKB, kk = o / C::NKB;
                const char* kp = st + kb * 32 * C::ROW_B;
                const uint4 w0 = *reinterpret_cast<const uint4*>(kp + k_rd8[2 * kk]);
                const uint4 w1 = *reinterpret_cast<const uint4*>(kp + k_rd8[2 * kk + 1]);
                fk[o] = i32x8{(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w,
                              (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
            }
#pragma unroll
            for (int o = 0; o < N8; ++o)
                s[o % C::NKB] = mfma_32x32x64_fp8(fk[o], qf8[o / C::NKB], o < C::NKB ? zero : s[o % C::NKB]);
            // Keep the scores' MFMAs in this (MFMA) phase: left alone, the
            // compiler sinks them into the branch of the next phase that
            // reads them (the softmax), where they no longer overlap the
            // other wave group's softmax.  An empty asm that only USES the
            // scores pins them here; it must not redefine them, or the
            // compiler would lose track of the MFMA results its softmax reads
            // and would not put the MFMA -> VALU wait states in front of them.
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb) asm volatile("" ::"v"(s[kb]));
        }
    };
    // softmax: scores s of the tile whose first key is key0 -> P^T operands pb
    // (bf16), running max / sums, lazy rescale of the O^T accumulators.
    auto softmax = [&](f32x16(&s)[C::NKB], bf16x8(&pb)[BN / 16], int key0,
                       bool need_mask) __attribute__((always_inline)) {
        // raw tile max of this lane's query (masked scores -> -inf)
        float mx = neg_inf();
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
            if (need_mask) {
                // key = key0 + 4 half + (compile-time offset); masked iff the
                // offset is above dl (causal / end) or below dl_lo (window)
                const int dl = lim - key0 - 4 * half;
                const int dl_lo = a.window > 0 ? first - key0 - 4 * half : -1;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
                    s[kb][r] = (off > dl || off < dl_lo) ? neg_inf() : s[kb][r];
                }
            }
#pragma unroll
            for (int r = 0; r < 16; r += 2) mx = max3(mx, s[kb][r], s[kb][r + 1]);
        }
        mx = half_max(mx);
        const float mt = mx == neg_inf() ? neg_inf() : mx * c;
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
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                float p0 = fast_exp2(__builtin_fmaf(s[kb][r], c, nm));
                float p1 = fast_exp2(__builtin_fmaf(s[kb][r + 1], c, nm));
                // c > 0: exp2(-inf) is already 0; FP8's c comes from device
                // descales and may be 0
                if ((CZ || F8) && need_mask) {
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
    };
    // PV: O^T += V^T P^T for the tile in stage st.  MFMA o works on output
    // block o % NB, 16-key step o / NB; V^T fragments are two transpose reads.
    auto pv = [&](const char* st, const bf16x8(&pb)[BN / 16]) __attribute__((always_inline)) {
        auto vfrag = [&](int o) __attribute__((always_inline)) { return vfrag_at(st, o); };
        bf16x8 fv[kWin];
#pragma unroll
        for (int w = 0; w < kWin; ++w) fv[w] = vfrag(w);
#pragma unroll
        for (int o = 0; o < NPV; ++o) {
            acc[o % C::NB] = mfma_32x32x16(fv[o % kWin], pb[o / C::NB], acc[o % C::NB]);
            if (o + kWin < NPV) fv[o % kWin] = vfrag(o + kWin);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kWin, 1);
#pragma unroll
        for (int o = 0; o < NPV; ++o) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
            if (o + kWin < NPV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        }
    };
    // PV of the tile in stage sv, then QK of the tile in stage sk, as one MFMA
    // stream whose operand read-ahead window runs across the boundary; hook()
    // (the DMA issue) comes after the first window of reads so that its
    // scalar work overlaps their latency instead of delaying the first MFMA.
    auto pv_qk = [&](const char* sv, const bf16x8(&pb)[BN / 16], const char* sk, f32x16(&s)[C::NKB],
                     auto&& hook) __attribute__((always_inline)) {
        constexpr int NM = NPV + NQK;
        static_assert(NPV >= kWin, "read-ahead window within PV");
        auto frag = [&](int o) __attribute__((always_inline)) {
            return o < NPV ? vfrag_at(sv, o) : kfrag_at(sk, o - NPV);
        };
        const f32x16 zero = {};
        bf16x8 fr[kWin];
#pragma unroll
        for (int w = 0; w < kWin; ++w) fr[w] = frag(w);
        hook();
#pragma unroll
        for (int o = 0; o < NM; ++o) {
            if (o < NPV) {
                acc[o % C::NB] = mfma_32x32x16(fr[o % kWin], pb[o / C::NB], acc[o % C::NB]);
            } else {
                const int k = o - NPV;
                s[k % C::NKB] = mfma_32x32x16(fr[o % kWin], qf[k / C::NKB], k < C::NKB ? zero : s[k % C::NKB]);
            }
            if (o + kWin < NM) fr[o % kWin] = frag(o + kWin);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kWin, 2);
#pragma unroll
        for (int o = 0; o < NM; ++o) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
            if (o + kWin < NPV) {
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);
            } else if (o + kWin < NM) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 2);
            }
        }
    };
    auto stage_ptr = [&](int t) __attribute__((always_inline)) {
        return lds + (t % S) * C::STAGE_B;
    };
    constexpr int PER_TILE = 2 * C::NI;  // vector-memory operations per tile and wave
    f32x16 s[C::NKB];
    bf16x8 pb[BN / 16];

    // The next item's ticket: it returns while this item runs (the wait
    // before the epilogue covers it).  Q is needed first, so that the wait
    // for it does not include the atomic's round trip.
    if constexpr (F8) {
#pragma unroll
        for (int kk = 0; kk < NQF8; ++kk) asm volatile("" ::"v"(qf8[kk]));
    } else {
#pragma unroll
        for (int kk = 0; kk < NQF; ++kk) asm volatile("" ::"v"(qf[kk]));
    }
    if (tid == 0) ticket = ticket_async(tctr);

    if constexpr (!PP) {
        // Sequential ring: at iteration t tile t is complete in stage t % S,
        // tiles up to t + S - 2 are in flight; the DMA of tile t + S - 1
        // reuses the stage tile t - 1 occupied (every wave passed the barrier
        // after it).
        wait_vmcnt<PER_TILE * (S - 2)>();
        __syncthreads();
        auto step = [&](int t, auto stage) __attribute__((always_inline)) {
            page_ids(t + S - 1);
            page_ids_ready();
            issue(t + S - 1);
            const int key0 = lo + t * BN;
            if (sees(key0)) {
                const char* st = lds + decltype(stage)::value * C::STAGE_B;
                qk(st, s);
                softmax(s, pb, key0, masked(key0));
                pv(st, pb);
            }
            wait_vmcnt<PER_TILE * (S - 2)>();
            __syncthreads();
        };
        // unrolled by S so that each stage's LDS offsets are compile-time constants
        for (int t = 0; t < n_tiles; t += S) {
            step(t, std::integral_constant<int, 0>{});
            if (t + 1 < n_tiles) step(t + 1, std::integral_constant<int, 1 % S>{});
            if constexpr (S > 2) {
                if (t + 2 < n_tiles) step(t + 2, std::integral_constant<int, 2 % S>{});
                if (t + 3 < n_tiles) step(t + 3, std::integral_constant<int, 3 % S>{});
            }
        }
    } else {
        // Ping-pong: waves w and w + 4 share a SIMD.  Each wave alternates an
        // MFMA phase M(t) = [PV of tile t - 1, QK of tile t] and a VALU phase
        // V(t) = [softmax of tile t], with a barrier after every phase; group
        // 1 (waves 4..7) takes one extra barrier first, so between any two
        // barriers one group runs MFMAs while the other runs the softmax.
        // DMA: M(t) issues tile t + S - 2 into the stage tile t - 2 used
        // (its last reader, PV(t - 2) of the late group, ended a window
        // earlier).  Tile t is read first in window 2t; each wave has waited
        // for its own part of it before the barrier that opens that window
        // (group 0 after V(t - 1), group 1 after M(t - 1)).
        //
        // FP8: the bf16 V tile of tile t is written in the MFMA phases M(t),
        // where the VALU is otherwise idle: rows 0..31 by the early group
        // (window 2t), rows 32..63 by the late group (window 2t + 1), each
        // after issuing its PV(t - 1) MFMAs.  Tile t has landed by window 2t
        // and its first P V (early group) runs in window 2t + 2.
        const bool late = wave >= NW / 2;
        // rows 32 part .. +32 of tile t: E4M3 codes -> the stage's bf16 V tile
        // (one 16-code chunk per thread of the group)
        auto convert_v = [&](int t, int part) __attribute__((always_inline)) {
            if constexpr (F8) {
                char* st = lds + (t % S) * C::STAGE_B;
                const int tt = tid & (NW / 2 * 64 - 1);
                const int row = 32 * part + tt / C::CPR, ch = tt % C::CPR;
                const uint4 w = *reinterpret_cast<const uint4*>(st + C::TILE_B + row * C::ROW_B + 16 * ch);
                char* vrow = st + C::VOFF + row * C::VROW_B;
                *reinterpret_cast<uint4*>(vrow + 16 * swz_v<C::VCPR>(row, 2 * ch)) = e4m3x8_to_bf16(uint2{w.x, w.y});
                *reinterpret_cast<uint4*>(vrow + 16 * swz_v<C::VCPR>(row, 2 * ch + 1)) = e4m3x8_to_bf16(uint2{w.z, w.w});
            }
        };
        static_assert(!F8 || (BN == 64 && 32 * C::CPR == NW / 2 * 64), "one chunk per thread of a group");
        wait_vmcnt<PER_TILE * (S - 3)>();
        __syncthreads();
        if (late) __syncthreads();
        // end of an MFMA phase / of a VALU phase
        auto m_end = [&]() __attribute__((always_inline)) {
            __builtin_amdgcn_s_setprio(0);
            if (late) wait_vmcnt<PER_TILE>();
            __syncthreads();
        };
        // V(t): softmax of tile t, or P = 0 for a wave that sees none of its keys
        auto v_phase = [&](int t) __attribute__((always_inline)) {
            page_ids(t + S - 1);  // issued by M(t + 1)
            const int key0 = lo + t * BN;
            if (sees(key0)) {
                softmax(s, pb, key0, masked(key0));
            } else {
#pragma unroll
                for (int j = 0; j < BN / 16; ++j) pb[j] = bf16x8{};
            }
            page_ids_ready();
            if (!late) wait_vmcnt<PER_TILE>();
            __syncthreads();
        };
        if (n_tiles > 0) {
            // M(0): QK of tile 0
            __builtin_amdgcn_s_setprio(1);
            page_ids_ready();
            issue(S - 2);
            if constexpr (F8) {
                if (!idle) qk8(stage_ptr(0), s);
                convert_v(0, late ? 1 : 0);
            } else {
                if (!idle) qk(stage_ptr(0), s);
            }
            m_end();
            v_phase(0);
            // M(t) = PV(t - 1) and QK(t) as one MFMA stream (one code path:
            // a wave whose keys end before tile t computes QK(t) and drops it)
            for (int t = 1; t < n_tiles; ++t) {
                __builtin_amdgcn_s_setprio(1);
                if constexpr (F8) {
                    issue(t + S - 2);
                    if (!idle) pv(stage_ptr(t - 1), pb);
                    convert_v(t, late ? 1 : 0);
                    if (!idle) qk8(stage_ptr(t), s);
                } else if (idle) {
                    issue(t + S - 2);
                } else {
                    pv_qk(stage_ptr(t - 1), pb, stage_ptr(t), s,
                          [&]() __attribute__((always_inline)) { issue(t + S - 2); });
                }
                m_end();
                v_phase(t);
            }
            // M(n_tiles): PV of the last tile
            __builtin_amdgcn_s_setprio(1);
            if (!idle) pv(stage_ptr(n_tiles - 1), pb);
            m_end();
        }
        if (!late) __syncthreads();
    }

    // The DMA of tiles past the end writes zeros into LDS: let all of it land
    // before this work-group can finish and its LDS be handed to another.
    wait_vmcnt<0>();
    before_epilogue();

    if constexpr (!PAGED) {
        // THD rows past the grid (a sequence longer than max_seqlen_q allows
        // for, rounded up to whole row blocks): the item of the last row block
        // writes them, for its heads, as NaN O and NaN LSE
        const int cover = a.n_qtiles * 32 * nt;
        if (qt == a.n_qtiles - 1 && lq > cover) {  // uniform
            const int chunks = D / 8;  // 16-byte chunks of an O row
            const int n = (lq - cover) * a.nh * chunks;
            const uint4 nan8 = {0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};
            for (int e = tid; e < n; e += C::THREADS) {
                const int r = cover + e / (a.nh * chunks);
                const int hh = hg * a.nh + (e / chunks) % a.nh;
                bf16_t* orow = a.o + (int64_t)(q_beg + r) * a.o_st + (int64_t)hh * a.o_sh;
                *reinterpret_cast<uint4*>(orow + 8 * (e % chunks)) = nan8;
                if (a.lse != nullptr && e % chunks == 0) {
                    if (a.lse_layout == 1) {
                        a.lse[(int64_t)(q_beg + r) * a.hq + hh] = nan_f();
                    } else if (a.lse_layout == 2 && r < a.lse_s_max) {
                        a.lse[((int64_t)b * a.lse_s_max + r) * a.hq + hh] = nan_f();
                    } else if (a.lse_layout == 3) {
                        a.lse[(int64_t)hh * a.lse_s_max + q_beg + r] = nan_f();
                    }
                }
            }
        }
    }

    // epilogue: O = O^T / l written as bf16, LSE = ln2 * (m + log2 l); a
    // split of a paged call writes its normalized fp32 partial and LSE_c
    // (-inf and zeros when it sees no key of the row)
    float l_tot = half_sum(l);
    float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (trunc) inv = nan_f();
    if constexpr (PAGED) {
        if (a.splits > 1) {  // uniform
            if (!row_ok) return;
            const int64_t grow = (int64_t)(q_beg + i) * a.hq + h;
            float* prow = a.o_part + ((int64_t)split * a.total_rows + grow) * D;
            inv *= o_mul;  // descale_v (1 unless FP8)
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int n = nb * 32 + 8 * g + 4 * half;
                    *reinterpret_cast<f32x4*>(prow + n) = f32x4{acc[nb][4 * g] * inv, acc[nb][4 * g + 1] * inv,
                                                               acc[nb][4 * g + 2] * inv, acc[nb][4 * g + 3] * inv};
                }
            }
            if (half == 0)
                a.lse_part[(int64_t)split * a.total_rows + grow] =
                    trunc ? nan_f() : (l_tot > 0.f ? kLn2 * (m + fast_log2(l_tot)) : neg_inf());
            return;
        }
    }
    if (a.sinks != nullptr) {
        // head h's sink: one more logit (log2 units below) in the denominator
        // only.  m2 = max(m, sink); O^T stays relative to m and is scaled by
        // alpha / l_tot; a row without keys (l = 0) keeps O = 0, LSE = sink.
        const float sk = a.sinks[h] * kLog2e;
        const float m2 = max(m, sk);
        if (m2 != neg_inf()) {
            const float alpha = fast_exp2(m - m2);  // 0 when m = -inf
            l_tot = l_tot * alpha + fast_exp2(sk - m2);
            inv = alpha / l_tot;
            m = m2;
        }
    }
    inv *= o_mul;  // descale_v (1 unless FP8)
    // Ping-pong kernels: O goes out through LDS, so that every store writes
    // whole rows.  The wave's 32 x D bf16 block is written to its own part of
    // the (now idle) ring as this lane's column of O^T, 16-byte chunks
    // XOR-swizzled by the row so that neither side conflicts, and read back
    // as 16-byte row chunks.  Each global store then covers 64 / (D / 8) full
    // rows instead of 16 bytes of each of 32 rows.
    if constexpr (PP) {
        constexpr int OROW_B = 2 * D;      // bytes per O row
        constexpr int OCPR = D / 8;        // 16-byte chunks per O row
        constexpr int RPI = 64 / OCPR;     // rows per 64-lane read
        static_assert((OCPR & (OCPR - 1)) == 0 && OCPR <= 64, "O row chunks");
        static_assert(NW * 32 * OROW_B <= C::LDS_BYTES, "O staging fits the ring");
        __syncthreads();  // every wave's DMAs have landed and its ring reads are done
        char* const ow = lds + wave * 32 * OROW_B;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                // d = nb 32 + 8 g + 4 half .. +4: chunk 4 nb + g, bytes 8 half ..
                const int pc = (4 * nb + g) ^ (col & (OCPR - 1));
                uint2 w;
                w.x = pack_bf16x2(acc[nb][4 * g] * inv, acc[nb][4 * g + 1] * inv);
                w.y = pack_bf16x2(acc[nb][4 * g + 2] * inv, acc[nb][4 * g + 3] * inv);
                *reinterpret_cast<uint2*>(ow + col * OROW_B + 16 * pc + 8 * half) = w;
            }
        }
        const int rc = lane % OCPR;  // the chunk this lane moves
#pragma unroll
        for (int j = 0; j < 32 / RPI; ++j) {
            const int r = j * RPI + lane / OCPR;
            const uint4 w = *reinterpret_cast<const uint4*>(ow + r * OROW_B + 16 * (rc ^ (r & (OCPR - 1))));
            const int rr = i0 + r;
            if (rr < n_rows) {
                // nontemporal: O is not read again by this call, and cached
                // dirty lines would be written back while later items stream
                // K/V (2 % on the THD prefill workload)
                const int tr = rr / fg;
                bf16_t* orow = a.o + (int64_t)(q_beg + tr) * a.o_st + (int64_t)(hb + rr - tr * fg) * a.o_sh;
                __builtin_nontemporal_store(u32x4{w.x, w.y, w.z, w.w}, reinterpret_cast<u32x4*>(orow + 8 * rc));
            }
        }
    }
    if (!row_ok) return;
    if constexpr (!PP) {
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
    }
    if (a.lse != nullptr && half == 0) {
        // natural log, or base 2 (the running statistics are already log2)
        const float lse2 = l_tot > 0.f ? m + fast_log2(l_tot) : neg_inf();
        const float lse = trunc ? nan_f() : (a.stats_log2 ? lse2 : kLn2 * lse2);
        if (a.lse_layout == 1) {
            a.lse[(int64_t)(q_beg + i) * a.hq + h] = lse;
        } else if (a.lse_layout == 2 && i < a.lse_s_max) {
            a.lse[((int64_t)b * a.lse_s_max + i) * a.hq + h] = lse;
        } else if (a.lse_layout == 3) {
            a.lse[(int64_t)h * a.lse_s_max + q_beg + i] = lse;
        }
    }
}

// Persistent grid: each work-group runs items until every queue is empty.
// The ticket of the next item is fetched (one atomic of wave 0) while the
// current item runs and handed to the other waves through LDS.
template <int D, int BN, int S, int NW, bool PP, bool CZ, bool PAGED, bool F8>
__global__ __launch_bounds__(64 * NW, (D <= 128 ? 2 : 1)) void prefill_bf16_kernel(PrefillKArgs a) {
    extern __shared__ __attribute__((aligned(16))) bf16_t smem[];
    __shared__ int next_item;
    char* const lds = reinterpret_cast<char*>(smem);
    const uint32_t lds_base = lds_addr(smem);
    uint64_t* const ctr = g_prefill_queue[a.slot];
    const int n_pairs = a.batch * a.n_hg * (PAGED ? a.splits : 1);
    // Only lane 0 of wave 0 talks to the queues: q is the queue it draws
    // from, tries the number of queues it has found empty.
    int q = 0, tries = 0;
    // item of ticket t of queue x, or -1 when the queue is exhausted
    auto item_of = [&](int x, uint32_t t) -> int {
        const int m = n_pairs > x ? (n_pairs - x + kXcds - 1) / kXcds : 0;
        if (m == 0 || t >= (uint32_t)(m * a.n_qtiles)) return -1;
        const int level = (int)t / m;
        return level * n_pairs + x + kXcds * ((int)t - level * m);
    };
    // next item after the ticket request `raw` on queue q, moving on to the
    // other queues
    auto next_of = [&](uint64_t raw) -> int {
        for (;;) {
            const int it = item_of(q, own_ticket(&ctr[q], raw, a.gen));
            if (it >= 0 || ++tries >= kXcds) return it;
            q = (q + 1) % kXcds;
            raw = ticket_async(&ctr[q]);
        }
    };
    uint64_t ticket = 0;
    if (threadIdx.x == 0) {
        unsigned xcc;
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
        q = (int)(xcc % kXcds);
        ticket = ticket_async(&ctr[q]);
    }
    // The next item is resolved (lane 0 of wave 0) before the current item's
    // epilogue: waiting for the ticket there costs nothing, while after the
    // epilogue the wait would also cover its stores (one memory counter).
    int nxt = -1;
    bool resolved = false;
    for (;;) {
        if (threadIdx.x == 0) next_item = resolved ? nxt : next_of(ticket);
        __syncthreads();
        const int item = next_item;
        if (item < 0) break;
        resolved = false;
        prefill_item<D, BN, S, NW, PP, CZ, PAGED, F8>(a, item, lds, lds_base, &ctr[q], ticket,
                                                      [&]() __attribute__((always_inline)) {
                                                          if (threadIdx.x == 0) nxt = next_of(ticket);
                                                          resolved = true;
                                                      });
        __syncthreads();  // every wave has read next_item before it is replaced
    }
    if (threadIdx.x == 0 && own_ticket(&ctr[kXcds], ticket_async(&ctr[kXcds]), a.gen) == gridDim.x - 1) {
        // every work-group has taken its last ticket: the slot is free again
        for (int x = 0; x <= kXcds; ++x) atomicExch(reinterpret_cast<unsigned long long*>(&ctr[x]), 0ull);
    }
}

// Resident work-groups per CU of a kernel (computed once per kernel: the Tag
// is the kernel's own template) x CUs of the device.
template <typename Tag, typename K>
int resident_slots(K kernel, int threads, int lds_bytes) {
    static std::atomic<int> per_cu{0};
    int occ = per_cu.load(std::memory_order_relaxed);
    if (occ == 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void*)kernel, threads, lds_bytes) != hipSuccess ||
            occ < 1)
            occ = 1;
        per_cu.store(occ, std::memory_order_relaxed);
    }
    int dev = 0, n_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu < 1)
        n_cu = 1;
    return occ * n_cu;
}

// Launch tags of the prefill work queues: 1, 2, 3, ... (0 marks a free counter).
std::atomic<uint32_t> g_launch_seq{0};
uint32_t next_launch_tag() {
    uint32_t g = g_launch_seq.fetch_add(1u, std::memory_order_relaxed) + 1u;
    while (g == 0u) g = g_launch_seq.fetch_add(1u, std::memory_order_relaxed) + 1u;
    return g;
}

template <int D, int BN, int S, int NW, bool PP, bool CZ, bool PAGED, bool F8>
struct KernelTag {};

template <int D, int BN, int S, int NW, bool PP, bool CZ, bool PAGED, bool F8 = false>
hipError_t launch_dz(PrefillKArgs a, int64_t n_wg, hipStream_t s) {
    using C = PCfg<D, BN, S, NW, F8>;
    auto kernel = prefill_bf16_kernel<D, BN, S, NW, PP, CZ, PAGED, F8>;
    // more than 64 KiB of dynamic LDS must be requested per kernel
    hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    const int64_t slots =
        resident_slots<KernelTag<D, BN, S, NW, PP, CZ, PAGED, F8>>(kernel, C::THREADS, C::LDS_BYTES);
    a.gen = next_launch_tag();
    a.slot = (int32_t)(a.gen % kQueueSlots);
    hipLaunchKernelGGL(kernel, dim3((unsigned)(n_wg < slots ? n_wg : slots)), dim3(C::THREADS),
                       (size_t)C::LDS_BYTES, s, a);
    return hipGetLastError();
}

template <int D, int BN, int S, int NW, bool PP, bool F8 = false>
hipError_t launch_d(const PrefillArgs& pa, hipStream_t s) {
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
    const int tile_rows = 32 * (NW / a.nh);
    a.n_qtiles = (pa.max_q + tile_rows - 1) / tile_rows;
    a.c = (pa.scale < 0.f ? -pa.scale : pa.scale) * kLog2e;
    a.q_sign = pa.scale < 0.f ? (F8 ? 0x80808080u : 0x80008000u) : 0u;
    a.descale_q = F8 ? pa.descale_q : nullptr;
    a.descale_k = F8 ? pa.descale_k : nullptr;
    a.descale_v = F8 ? pa.descale_v : nullptr;
    a.causal = pa.causal;
    a.lse = pa.lse;
    a.lse_layout = pa.lse_layout;
    a.lse_s_max = pa.lse_s_max;
    // a window of 2^30 keys covers every key of any sequence the int32
    // offsets can describe; the clamp keeps i + shift - W + 1 in range
    a.window = pa.window > 0 ? min(pa.window, 1 << 30) : 0;
    a.sinks = pa.sinks;
    a.stats_log2 = pa.stats_log2;
    a.pt_k = a.pt_v = a.seq_lens = nullptr;
    a.k_sp = a.v_sp = 0;
    a.table_stride = a.page = a.sq = 0;
    a.splits = 1;
    a.total_rows = 0;
    a.o_part = a.lse_part = nullptr;
    const int64_t n_wg = (int64_t)a.n_qtiles * a.n_hg * a.batch;
    if (n_wg == 0) return hipSuccess;
    if (n_wg > INT32_MAX) return hipErrorInvalidValue;
    return a.c == 0.f ? launch_dz<D, BN, S, NW, PP, true, false, F8>(a, n_wg, s)
                      : launch_dz<D, BN, S, NW, PP, false, false, F8>(a, n_wg, s);
}

// Waves (32 rows each) of the paged kernel for head dim d: the D = 128
// ping-pong kernel has 8, the D = 256 sequential one 4.
int paged_waves(int d) { return d == 256 ? 4 : 8; }

// Query tokens per work item of the paged kernel (its waves of 32 rows over
// NH heads of a GQA group).
int paged_item_tokens(int group, int nw) {
    const int nh = (group % 4 == 0) ? 4 : (group % 2 == 0 ? 2 : 1);
    return 32 * (nw / nh);
}

// Fewer query tokens than an item holds: the rows of a whole GQA group are
// folded, token-major, into the item's 256 rows.  Returns the group size, or
// 0 when the call does not fold.  Up to 16 rows per KV head the few-row
// decode kernel reads the K/V once and is the better fit; past that it reads
// them once per 16-row group, and the folded item (K/V read once, MFMA work
// of 256 rows) is 1.5x faster at 32 rows and 2.8x at 64.
constexpr int kFoldRowsMin = 17;
int paged_fold(const DecodeArgs& d) {
    const int group = d.hq / d.hkv;
    if (d.sq >= paged_item_tokens(group, paged_waves(d.dqk))) return 0;
    const int64_t rows = (int64_t)d.sq * group;
    return rows < kFoldRowsMin || rows > (1 << 24) ? 0 : group;
}

}  // namespace

bool prefill_paged_supported(const DecodeArgs& d) {
    // D = 128 (bf16 or FP8), D = 64 and D = 256 (bf16); any page size of a
    // multiple of 8 keys (each wave's 8 rows of a tile lie in one page)
    if (d.dqk != d.dv || d.page % 8 != 0) return false;
    if (!(d.dqk == 128 || (d.dqk == 64 && !d.fp8) || (d.dqk == 256 && !d.fp8))) return false;
    if (d.k_st >= (1 << 22) || d.v_st >= (1 << 22)) return false;
    return d.sq >= paged_item_tokens(d.hq / d.hkv, paged_waves(d.dqk)) || paged_fold(d) > 0;
}

bool prefill_paged_folds(const DecodeArgs& d) { return prefill_paged_supported(d) && paged_fold(d) > 0; }

template <int D, int BN, int S, int NW, bool PP, bool F8>
hipError_t launch_prefill_paged_t(const DecodeArgs& d, hipStream_t s) {
    static_assert(NW == (D == 256 ? 4 : 8), "the waves paged_waves assumes");
    PrefillKArgs a;
    a.q = static_cast<const bf16_t*>(d.q);
    a.q_st = (int64_t)d.hq * D;
    a.q_sh = D;
    a.k = static_cast<const bf16_t*>(d.k_pool);
    a.k_st = d.k_st;
    a.k_sh = d.k_sh;
    a.v = static_cast<const bf16_t*>(d.v_pool);
    a.v_st = d.v_st;
    a.v_sh = d.v_sh;
    a.o = static_cast<bf16_t*>(d.o);
    a.o_st = (int64_t)d.hq * D;
    a.o_sh = D;
    a.cu_q = a.cu_kv = nullptr;
    a.batch = d.batch;
    a.hq = d.hq;
    a.group = d.hq / d.hkv;
    const int fold = paged_fold(d);
    if (fold > 0) {
        // one head group per item, its sq * group rows in blocks of 256
        a.fold = fold;
        a.nh = 1;
        a.n_hg = d.hkv;
        a.n_qtiles = (int)(((int64_t)d.sq * a.group + 32 * NW - 1) / (32 * NW));
    } else {
        a.fold = 1;
        a.nh = (a.group % 4 == 0) ? 4 : (a.group % 2 == 0 ? 2 : 1);
        a.n_hg = d.hq / a.nh;
        const int tokens = paged_item_tokens(a.group, NW);
        a.n_qtiles = (d.sq + tokens - 1) / tokens;
    }
    a.c = (d.scale < 0.f ? -d.scale : d.scale) * kLog2e;
    a.q_sign = d.scale < 0.f ? (F8 ? 0x80808080u : 0x80008000u) : 0u;
    a.descale_q = F8 ? d.descale_q : nullptr;
    a.descale_k = F8 ? d.descale_k : nullptr;
    a.descale_v = F8 ? d.descale_v : nullptr;
    a.causal = d.causal;
    a.lse = d.lse;
    a.lse_layout = d.lse != nullptr ? 1 : 0;  // [B, s_q, Hq] = token-major
    a.lse_s_max = 0;
    // a window of 2^30 keys covers every key of any sequence the int32
    // lengths can describe; the clamp keeps i + shift - W + 1 in range
    a.window = d.window > 0 ? min(d.window, 1 << 30) : 0;
    a.sinks = d.sinks;  // folded in the epilogue with one split, by the combine otherwise
    a.stats_log2 = d.stats_log2;
    a.pt_k = d.pt_k;
    a.pt_v = d.pt_v;
    a.seq_lens = d.seq_lens;
    a.k_sp = d.k_sp;
    a.v_sp = d.v_sp;
    a.table_stride = d.table_stride;
    a.page = d.page;
    a.sq = d.sq;
    a.splits = d.splits;
    a.total_rows = (int64_t)d.batch * d.sq * d.hq;
    a.o_part = d.o_part;
    a.lse_part = d.lse_part;
    const int64_t n_wg = (int64_t)a.n_qtiles * a.n_hg * a.batch * a.splits;
    if (n_wg == 0) return hipSuccess;
    if (n_wg > INT32_MAX) return hipErrorInvalidValue;
    return a.c == 0.f ? launch_dz<D, BN, S, NW, PP, true, true, F8>(a, n_wg, s)
                      : launch_dz<D, BN, S, NW, PP, false, true, F8>(a, n_wg, s);
}

hipError_t launch_prefill_paged(const DecodeArgs& d, hipStream_t s) {
    if (d.dqk == 256) return launch_prefill_paged_t<256, 32, 4, 4, false, false>(d, s);
    if (d.dqk == 64) return launch_prefill_paged_t<64, 64, 4, 8, true, false>(d, s);
    return d.fp8 ? launch_prefill_paged_t<128, 64, 4, 8, true, true>(d, s)
                 : launch_prefill_paged_t<128, 64, 4, 8, true, false>(d, s);
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
    if (a.fp8) return a.dqk == 128 ? launch_d<128, 64, 4, 8, true, true>(a, s) : hipErrorInvalidValue;
    switch (a.dqk) {
        case 64: return launch_d<64, 128, 4, 8, true>(a, s);
        case 128: return launch_d<128, 64, 4, 8, true>(a, s);
        case 256: return launch_d<256, 32, 4, 4, false>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sdpa
