// decode_wide.hip -- paged-KV decode with many query rows per KV head, bf16.
//
// Serves every s_q * G query rows per KV head with d_qk = 576, d_v = 512: the
// absorbed-MLA decode shape with independent K/V page tables (cuDNN Frontend
// v1.32.0 Release Notes, "SDPA: wider native forward support"; paged K/V and
// split-KV: v1.31.0 "SDPA: paged KV, split-KV, and engine selection").  With
// hundreds of rows sharing one KV head every key costs rows x 1088 MACs, so
// the work is a dense contraction per K/V tile and runs on MFMA:
//
// Work-group = 4 waves = 128 query rows (row r of a KV head is query token
// r / G, head kvh G + r % G) x one split-KV chunk of one sequence; chunks of
// the longest sequences are dispatched first.  Per tile of 32 keys (tiles
// start on multiples of 16 keys and may span pages when page_size is 16):
//   K tile (32 x 576) and V tile (32 x 512) gathered from their pages into
//   LDS by buffer_load_dwordx4 ... lds (lane L's 16 bytes land at M0 + 16 L),
//   each wave its own 8 rows (which lie in one page: page_size % 8 == 0),
//   one 1 KB row per instruction, in a ring of two K and two V slots that
//   refill independently.  Bank conflicts are
//   avoided by a 16-byte pad after dims 0..511 of each K row, an XOR swizzle
//   of the 8 chunks of dims 512..575 (kept in a region of their own) and an
//   XOR swizzle of the V chunks;
//   S^T = K Q^T: 36 v_mfma_f32_32x32x16_bf16 per wave for its 32 rows, A = K
//   rows (ds_read_b128), B = the wave's Q^T held in registers, so each lane
//   holds the scores of one query;
//   online softmax in registers (row max: 3-input max + one lane-half
//   exchange) in a fixed per-lane frame, the chunk run a second time when a
//   later tile's max outgrows it (the softmax frame below);
//   P^T goes through LDS (1 KB per 32 rows x 16 keys) and each wave owns 128
//   columns of O^T for all 128 rows: O^T += V^T P^T is 32 MFMAs per wave
//   whose operands are each read once and used four times (A = V^T via
//   ds_read_b64_tr_b16 from the row-major V tile, B = P^T), half the LDS
//   reads of a wave owning whole rows.
// The chunk's normalized partial (O_c, LSE_c) goes to the split workspace,
// or O / LSE directly when num_splits == 1.
//
// Fewer, longer chunks: each work-group carries a fixed cost of about eight
// tiles (the length rank, page ids, Q and the first K/V tiles before its
// first MFMA; the partial's stores after its last), and one work-group per
// CU runs at a time.  When num_splits would give more than two work-groups
// per CU, `merge` adjacent chunks go to one work-group: it computes the
// partial of their union into the slot of the first and marks the others
// empty (LSE -inf, O not written; the LSE merge neither reads nor weighs
// them), so the merge over all num_splits slots is the same attention.
//
// Per-tensor FP8 (E4M3 Q, K and V codes; F8 = true): the tiles arrive by the
// same LDS DMA as codes, half the bytes.  K rows are 512 + 64 codes (region
// A: 32 chunks per row, chunk XOR row mod 8; region B: 4 chunks, chunk XOR
// (row / 2) mod 4).  S^T = K Q^T runs on the FP8 MFMA (32x32x64, unit block
// scales): 9 k-steps of 64 codes, a lane's K fragment two 16-code reads (d =
// 64 kk + 32 half .. +32) and Q^T held as codes.  P V stays on the bf16
// MFMA: each wave widens its own 128 columns of the V codes exactly into a
// bf16 V tile outside the ring (the only wave that reads them), laid out as
// the bf16 kernel's V tile.  descale_q * descale_k joins the logit scale and
// descale_v the output.
#include "sdpa_device.h"
#include "sdpa_launch.h"
#include "tile_ops.h"

namespace sdpa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));  // 32 E4M3 codes

struct WideArgs {
    const void* q;       // bf16 or E4M3 codes
    const void* k_pool;
    int64_t k_sp, k_st, k_sh;
    const void* v_pool;
    int64_t v_sp, v_st, v_sh;
    const int32_t* pt_k;
    const int32_t* pt_v;
    int32_t table_stride;
    const int32_t* seq_lens;
    int32_t batch, sq, hq, hkv, group, page, splits;
    int32_t merge;    // adjacent chunks per work-group (>= 1)
    int32_t n_cg;     // ceil(splits / merge) chunk groups per (sequence, KV head)
    int32_t rows;     // s_q * group query rows per KV head
    int32_t n_rb;     // 128-row blocks per KV head
    int32_t n_g;      // batch * hkv * splits chunks
    float c;          // |scale| * log2(e)
    uint32_t q_sign;  // 0x80008000 when scale < 0 (Q negated on load), else 0
    int32_t causal;
    float* o_part;    // [splits, batch*sq*hq, 512] when splits > 1
    float* lse_part;  // [splits, batch*sq*hq]
    bf16_t* o;        // [batch, sq, hq, 512] when splits == 1
    float* lse;       // [batch, sq, hq] or null
    int32_t window;   // left sliding window (0: none)
    const float* sinks;  // [hq] sink logits (natural-log units) or null
    int32_t stats_log2;  // final LSE in base 2
    const float* descale_q;  // FP8 only: one fp32 each, read on the device
    const float* descale_k;
    const float* descale_v;
};

// LDS: two ring stages, each K region A (dims 0..511 of 32 rows, pitch
// 1040 B: 1 KB + a 16-byte pad), K region B (dims 512..575, 32 rows x 128 B,
// chunk XOR row mod 8), V (32 rows x 1 KB, chunk XOR 4 (row mod 4)); then
// the P^T exchange: one 1 KB MFMA operand per (32-row block, 16-key step),
// lane l's 16 bytes at 16 l.
// FP8: region A rows of 512 codes (no pad, chunks swizzled), region B rows
// of 64 codes, V rows of 512 codes; after the two stages the widened bf16 V
// tile (32 rows x 1 KB, chunk XOR 4 (row mod 4) as the bf16 V tile).
template <int DQK, int DV, bool F8>
struct WCfg {
    static constexpr int NW = 4;                    // waves, 32 query rows each
    static constexpr int BN = 32;                   // keys per tile
    static constexpr int EB = F8 ? 1 : 2;           // bytes per element
    static constexpr int KA_PITCH = F8 ? 512 : 1040;
    static constexpr int KA_B = BN * KA_PITCH;      // region A bytes
    static constexpr int KB_OFF = KA_B;             // region B
    static constexpr int KB_ROW = 64 * EB;
    static constexpr int KB_B = BN * KB_ROW;
    static constexpr int V_OFF = KB_OFF + KB_B;     // V tile (codes for FP8)
    static constexpr int VROW_B = EB * DV;
    static constexpr int STAGE_B = V_OFF + BN * VROW_B;
    static constexpr int VB_OFF = 2 * STAGE_B;      // FP8: widened bf16 V tile
    static constexpr int VBROW_B = 2 * DV;          // bf16 V rows, wherever they are read
    static constexpr int P_OFF = VB_OFF + (F8 ? BN * VBROW_B : 0);  // P^T exchange
    static constexpr int LDS_BYTES = P_OFF + NW * (BN / 16) * 1024;
    static constexpr int RPW = BN / NW;             // tile rows per wave (one DMA each)
    static constexpr int KK = DQK / 16;             // k-steps of S^T = K Q^T
    static constexpr int KKA = 32;                  // k-steps in region A
    static constexpr int NBW = DV / 32 / NW;        // 32-column blocks of O^T per wave
    static constexpr int NQK = KK;                  // QK MFMAs per tile
    static_assert(DQK == 576 && DV == 512, "geometry below is written for the 576/512 shape");
    static_assert(BN * 8 == 64 * NW, "region B: one DMA instruction per wave");
    static_assert(NBW == 4 && NW == 4, "O^T: 4 column blocks x 4 row blocks per wave");
};
constexpr int kTxPitch = 528;      // bytes per row of the output transpose (512 + 16)

constexpr int kWideRankMax = 256;  // longest-first order for batches up to this size
static_assert(4 * 32 * kTxPitch <= WCfg<576, 512, false>::P_OFF, "output transpose fits in the ring");
static_assert(4 * 32 * kTxPitch <= WCfg<576, 512, true>::P_OFF, "output transpose fits below P^T");

constexpr int kWinW = 4;  // LDS operand fragments read ahead of the MFMAs

// S^T MFMAs are written as inline asm with VGPR operands: the 256 O^T
// accumulators then take the whole AGPR file (compiler-selected MFMAs) while
// the score accumulator and Q^T stay in VGPRs.  The compiler's hazard model
// does not see MFMAs inside asm, so the chain carries its own wait states:
// the even and odd k-steps accumulate into two register sets (so adjacent
// MFMAs are independent; each set is only read back as the srcC of an MFMA
// into exactly the same registers, which needs no wait), each MFMA first
// covers a VALU write of its A/B operands (s_nop 1), and qk_fence() puts 24
// wait states between the last MFMAs and any VALU read of the scores (an
// 8-pass MFMA result needs fewer).
__device__ __forceinline__ void qk_first(f32x16& d, bf16x8 a, bf16x8 b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk_next(f32x16& d, bf16x8 a, bf16x8 b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
// The FP8 form (v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 x E4M3, block scales
// 2^0 from `sc`) under the same rules; it takes 16 passes, so the 24-wait-
// state fence still covers the VALU reads after it.
__device__ __forceinline__ void qk8_first(f32x16& d, i32x8 a, i32x8 b, int sc) {
    asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %3 op_sel_hi:[0,0,0]"
                 : "=&v"(d) : "v"(a), "v"(b), "v"(sc));
}
__device__ __forceinline__ void qk8_next(f32x16& d, i32x8 a, i32x8 b, int sc) {
    asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
                 : "+v"(d) : "v"(a), "v"(b), "v"(sc));
}
__device__ __forceinline__ void qk_fence(f32x16& d0, f32x16& d1) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(d0), "+v"(d1));
}

// Softmax frame.  O^T is never rescaled inside the tile loop (any VALU work
// on the 256 accumulators there makes the compiler move them out of the
// AGPRs): each lane fixes its reference max m at its first visible tile and
// adds p = exp2(s c - m) of later tiles in that frame.  Those p stay below
// 2^kMaxExcess unless a tile's max exceeds m by more than kMaxExcess; the
// work-group then runs the chunk once more with every lane's reference set to
// the largest tile max it saw, so p <= 1 throughout.  Either way O = O^T / l
// and LSE = ln2 (m + log2 l) are the softmax of the chunk.
constexpr float kMaxExcess = 32.f;

// DMA source offsets v + s and (v ^ x) + s, computed where they are used: as
// volatile asm the compiler cannot hoist them out of the tile loop (and then
// spill them for lack of VGPRs).
__device__ __forceinline__ uint32_t add_here(uint32_t v, uint32_t s) {
    uint32_t r;
    asm volatile("v_add_u32 %0, %1, %2" : "=v"(r) : "s"(s), "v"(v));
    return r;
}
__device__ __forceinline__ uint32_t xor_add_here(uint32_t v, uint32_t x, uint32_t s) {
    uint32_t r;
    asm volatile("v_xor_b32 %0, %1, %2\n\tv_add_u32 %0, %3, %0" : "=&v"(r) : "s"(x), "v"(v), "s"(s));
    return r;
}
// (v ^ x) + w + s with a per-lane w
__device__ __forceinline__ uint32_t xor_add3_here(uint32_t v, uint32_t x, uint32_t w, uint32_t s) {
    uint32_t r;
    asm volatile("v_xor_b32 %0, %1, %2\n\tv_add3_u32 %0, %0, %3, %4" : "=&v"(r) : "s"(x), "v"(v), "v"(w), "s"(s));
    return r;
}

// VAR: a left window, sinks or base-2 Stats are requested (their masks and
// epilogue cost registers the plain instantiation has none to spare for).
// NRB: 32-row blocks of O^T each wave computes: 4, or 1 when a KV head has at
// most 32 query rows (waves 1..3 then hold no rows, and the O^T MFMAs of the
// three empty row blocks are not issued).
template <int DQK, int DV, bool VAR, bool F8, int NRB>
__global__ __launch_bounds__(256, 1) void decode_wide_kernel(WideArgs a) {
    using C = WCfg<DQK, DV, F8>;
    static_assert(NRB == 1 || NRB == C::NW, "one row block, or all of them");
    extern __shared__ __attribute__((aligned(16))) bf16_t smem[];
    char* const lds = reinterpret_cast<char*>(smem);
    const uint32_t lds_base = lds_addr(smem);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // chunk group g = (b, kvh, cg); the n_rb row blocks of a group are 8 work-
    // groups apart, i.e. on the same XCD (work-group i runs on XCD i % 8)
    const int bid = blockIdx.x;
    const int g = (bid / (8 * a.n_rb)) * 8 + bid % 8;
    const int rb = (bid / 8) % a.n_rb;
    if (g >= a.n_g) return;
    const int cg = g % a.n_cg;  // chunk group: chunks cg * merge .. + merge - 1
    const int bk = g / a.n_cg;
    const int kvh = bk % a.hkv;
    // the (bk / hkv)-th longest sequence (ties by index): work-groups are
    // dispatched about in index order, so the longest chunks start first and
    // the short ones fill the tail
    int b = bk / a.hkv;
    int len_b;
    if (a.batch <= kWideRankMax) {
        __shared__ __attribute__((aligned(16))) int lens_x[kWideRankMax];
        __shared__ int seq_of;
        // lengths to LDS (padded to a multiple of 4 with INT32_MIN, below any length)
        if (tid < ((a.batch + 3) & ~3)) lens_x[tid] = tid < a.batch ? a.seq_lens[tid] : INT32_MIN;
        __syncthreads();
        if (tid < a.batch) {
            const int lm = lens_x[tid];
            int rk = 0;
            for (int j = 0; j < a.batch; j += 4) {
                const int4 q4 = *reinterpret_cast<const int4*>(lens_x + j);
                rk += (q4.x > lm) || (q4.x == lm && j < tid);
                rk += (q4.y > lm) || (q4.y == lm && j + 1 < tid);
                rk += (q4.z > lm) || (q4.z == lm && j + 2 < tid);
                rk += (q4.w > lm) || (q4.w == lm && j + 3 < tid);
            }
            if (rk == b) seq_of = tid;
        }
        __syncthreads();
        b = __builtin_amdgcn_readfirstlane(seq_of);
        len_b = __builtin_amdgcn_readfirstlane(lens_x[b]);
    } else {
        len_b = load_uniform(a.seq_lens, b);
    }

    // keys of this chunk: [lo, hi).  Keys [base, L) are cut into the splits;
    // with a left window, base is the start of the page holding the first key
    // any token of the sequence sees.
    // a length past the table's reach is clamped (the table is never read out of
    // bounds) and the sequence's rows are written as NaN
    const bool trunc = len_b > a.table_stride * a.page;
    const int L = min(len_b, a.table_stride * a.page);
    int base = 0;
    if (VAR && a.window > 0 && L - a.sq - a.window + 1 > 0) base = ((L - a.sq - a.window + 1) / a.page) * a.page;
    int lo = base, hi = L;
    if (a.splits > 1) {
        const int per = (L - base + a.splits - 1) / a.splits;
        const int chunk = ((per + a.page - 1) / a.page) * a.page;
        lo = min(L, base + cg * a.merge * chunk);
        hi = min(L, lo + a.merge * chunk);
    }

    // rows of this lane / wave / work-group
    const int col = lane & 31, half = lane >> 5;
    const int r = rb * 128 + wave * 32 + col;
    const bool row_ok = r < a.rows;
    const int tq = (row_ok ? r : a.rows - 1) / a.group;  // query token
    const int h = kvh * a.group + (row_ok ? r : a.rows - 1) % a.group;
    const int r_w0 = min(rb * 128 + wave * 32, a.rows - 1);        // first row of the wave
    const int r_w1 = min(rb * 128 + wave * 32 + 31, a.rows - 1);   // last
    const int r_g1 = min(rb * 128 + 127, a.rows - 1);
    // key j is visible to token t iff j <= L - sq + t (causal) / j < L
    auto end_of = [&](int row) { return a.causal ? min(hi, L - a.sq + row / a.group + 1) : hi; };
    const int kv_end = max(lo, end_of(r_g1));
    const bool wave_rows = rb * 128 + wave * 32 < a.rows;
    const int kv_end_w = wave_rows ? max(lo, end_of(r_w1)) : lo;
    const int nomask_end = wave_rows ? max(lo, end_of(r_w0)) : lo;
    // last visible key of this lane within the chunk (a chunk of 16-key pages can
    // end inside a tile: the keys past hi are masked, not merely zero-filled)
    const int lim = min(hi - 1, a.causal ? L - a.sq + tq : L - 1);
    // first visible key of this lane (left window), and the largest of the
    // wave's rows (its last token's): tiles starting below it need the lower mask
    const bool win = VAR && a.window > 0;
    const int first = win ? L - a.sq + tq - a.window + 1 : INT32_MIN;
    const int first_w = win ? L - a.sq + r_w1 / a.group - a.window + 1 : INT32_MIN;
    const int n_tiles = (kv_end - lo + C::BN - 1) / C::BN;

    // ---- LDS DMA of the K/V tiles -------------------------------------------
    // Wave w moves rows 8 w .. 8 w + 7 of each tile: per row one instruction
    // for K dims 0..511 (lane L: chunk L) and one for V (lane L: chunk
    // L ^ 4 (row mod 4)); one more instruction covers its 8 rows of K dims
    // 512..575 (lane L: row 8 w + L / 8, chunk (L mod 8) ^ (row mod 8)).
    // FP8: per wave 4 instructions of 2 rows each for region A (lane L: row
    // + L / 32, physical chunk L % 32 = logical chunk (L % 32) ^ (row mod 8)),
    // lanes 0..31 of one for its 8 rows of region B (lane L: row + L / 4,
    // physical chunk L % 4 = logical (L % 4) ^ ((row / 2) mod 4)), and 4 of 2
    // rows each for V (unswizzled).
    const uint32_t k_st2 = C::EB * (uint32_t)a.k_st, v_st2 = C::EB * (uint32_t)a.v_st;
    const uint32_t l16 = 16u * (uint32_t)lane;
    const int rb_row = wave * C::RPW + lane / (F8 ? 4 : 8);
    // (source offsets count from the wave's first row of the tile; the
    // swizzles follow the row within the tile)
    const uint32_t rb_rel = (uint32_t)(rb_row - wave * C::RPW);
    const uint32_t kb_src =
        F8 ? rb_rel * k_st2 + 512u + 16u * (uint32_t)((lane & 3) ^ ((rb_row >> 1) & 3))
           : rb_rel * k_st2 + 1024u + 16u * (uint32_t)((lane & 7) ^ (rb_row & 7));
    const uint32_t hl = (uint32_t)(lane >> 5);  // FP8: second row of a 2-row instruction
    const uint32_t ka_v = 16u * (((uint32_t)lane & 31u) ^ hl), ka_w = hl * k_st2;
    const uint32_t va_v = hl * v_st2 + 16u * ((uint32_t)lane & 31u);
    // Physical pages of the chunk's first 64 pages (lane i: page lo/page + i);
    // a chunk of more pages reloads the window when it gets there.
    const int pg0 = lo / a.page;
    const int64_t pt_row = (int64_t)b * a.table_stride;
    const int n_pages = (kv_end - lo + a.page - 1) / a.page;
    int pwin = 0;  // first page (relative to pg0) of the loaded window
    int pk = 0, pv = 0;
    auto load_window = [&](int first) __attribute__((always_inline)) {
        const int i = min(first + lane, max(n_pages - 1, 0));
        pk = a.pt_k[pt_row + pg0 + i];
        pv = a.pt_v[pt_row + pg0 + i];
        pwin = first;
        // use the ids at once: the compiler waits for them here, where the
        // window is (re)loaded, and not (conservatively, for every pending
        // DMA) before each later readlane of a window that arrived long ago
        asm volatile("" ::"v"(pk), "v"(pv));
    };
    if (n_pages > 0) load_window(0);
    const char* const kbase = static_cast<const char*>(a.k_pool) + (int64_t)C::EB * kvh * a.k_sh;
    const char* const vbase = static_cast<const char*>(a.v_pool) + (int64_t)C::EB * kvh * a.v_sh;
    // The 17 DMA instructions of a tile (per wave: 8 rows of K dims 0..511,
    // its rows of K dims 512..575, 8 rows of V) are issued in two bursts, V
    // and K, each right after the barrier that frees its slot: spread between
    // the MFMAs, the data arriving in LDS throughout slows every phase's
    // operand reads more.  A tile at or past the end gets an empty buffer
    // range: its DMA writes zeros and reads nothing.  The loads are
    // nontemporal: 2 % faster on the MLA decode workload than cached ones.
    struct DmaPlan {
        u32x4 kr, vr;
        uint32_t st;
    };
    // Each wave moves its own 8 rows of a tile (keys key0 + 8 w ..), which lie
    // in one page (page_size % 8 == 0 and tiles start on multiples of 16), so
    // a tile may span pages; the wave's buffer resource starts at its first row.
    auto plan = [&](int t, int stage) __attribute__((always_inline)) {
        const int keyw = lo + t * C::BN + wave * C::RPW;
        const int nvalid = min(C::RPW, kv_end - keyw);
        const int rel = min(keyw / a.page - pg0, n_pages - 1);
        // uniform; the second pass of a chunk starts again below the window
        if (rel - pwin >= 64 || rel < pwin) load_window(rel);
        const int pkp = __builtin_amdgcn_readlane(pk, rel - pwin);
        const int pvp = __builtin_amdgcn_readlane(pv, rel - pwin);
        const int slot = keyw % a.page;
        // rows at or past nvalid fall outside the buffer range and arrive as zeros
        const uint32_t kn = nvalid > 0 ? (uint32_t)(nvalid - 1) * k_st2 + C::EB * DQK : 0u;
        const uint32_t vn = nvalid > 0 ? (uint32_t)(nvalid - 1) * v_st2 + C::EB * DV : 0u;
        DmaPlan d;
        d.kr = make_rsrc(kbase + (int64_t)C::EB * ((int64_t)pkp * a.k_sp + (int64_t)slot * a.k_st), kn);
        d.vr = make_rsrc(vbase + (int64_t)C::EB * ((int64_t)pvp * a.v_sp + (int64_t)slot * a.v_st), vn);
        d.st = lds_base + stage * C::STAGE_B;
        return d;
    };
    // K of a tile is NK pieces (8 rows of dims 0..511, then the wave's rows of
    // dims 512..575), V is NV pieces (8 rows); FP8: 4 + 1 and 4
    constexpr int NA = F8 ? C::RPW / 2 : C::RPW;  // region A pieces
    constexpr int NK = NA + 1, NV = NA;
    auto k_piece = [&](const DmaPlan& d, int j) __attribute__((always_inline)) {
        if constexpr (F8) {
            if (j < NA) {
                const int row = wave * C::RPW + 2 * j;
                dma16_stream(d.kr, d.st + row * C::KA_PITCH,
                             xor_add3_here(ka_v, 32u * (uint32_t)j, ka_w, (uint32_t)(2 * j) * k_st2));
            } else if (lane < 32) {
                dma16_stream(d.kr, d.st + C::KB_OFF + wave * 512, kb_src);
            }
        } else {
            if (j < C::RPW) {
                const int row = wave * C::RPW + j;
                dma16_stream(d.kr, d.st + row * C::KA_PITCH, add_here(l16, (uint32_t)j * k_st2));
            } else {
                dma16_stream(d.kr, d.st + C::KB_OFF + wave * 1024, kb_src);
            }
        }
    };
    auto v_piece = [&](const DmaPlan& d, int j) __attribute__((always_inline)) {
        if constexpr (F8) {
            const int row = wave * C::RPW + 2 * j;
            dma16_stream(d.vr, d.st + C::V_OFF + row * C::VROW_B, add_here(va_v, (uint32_t)(2 * j) * v_st2));
        } else {
            const int row = wave * C::RPW + j;
            dma16_stream(d.vr, d.st + C::V_OFF + row * C::VROW_B,
                  xor_add_here(l16, 64u * (uint32_t)(row & 3), (uint32_t)j * v_st2));
        }
    };
    // the ring's first tiles: K and V of tile 0, K of tile 1
    auto prologue = [&]() __attribute__((always_inline)) {
        const DmaPlan d0 = plan(0, 0);
#pragma unroll
        for (int j = 0; j < NK; ++j) k_piece(d0, j);
#pragma unroll
        for (int j = 0; j < NV; ++j) v_piece(d0, j);
        const DmaPlan d1 = plan(1, 1);
#pragma unroll
        for (int j = 0; j < NK; ++j) k_piece(d1, j);
    };
    if (n_tiles > 0) prologue();  // overlaps the Q load below

    // log2-domain logit scale and Q's sign flip; FP8 folds in descale_q *
    // descale_k (a negative product flips Q like a negative scale)
    float c = a.c;
    uint32_t q_sign = a.q_sign;
    float o_mul = 1.f;  // descale_v (1 unless FP8)
    if constexpr (F8) {
        const float dqk = a.descale_q[0] * a.descale_k[0];
        c *= fabsf(dqk);
        if (dqk < 0.f) q_sign ^= 0x80008000u;
        o_mul = a.descale_v[0];
    }
    // Q^T operand: lane (col, half) holds d = 16 kk + 8 half .. +8 of row r
    // (rows past the end read the last row and are zeroed).  FP8: the codes
    // d = 64 kk + 32 half .. +32 of k-step kk (sign bits flipped per byte).
    constexpr int KK8 = DQK / 64;
    bf16x8 qf[F8 ? 1 : C::KK];
    i32x8 qf8[F8 ? KK8 : 1];
    {
        const uint32_t keep = row_ok ? 0xffffffffu : 0u;
        const int64_t qoff = ((int64_t)(b * a.sq + tq) * a.hq + h) * DQK;
        if constexpr (F8) {
            const uint32_t sg = q_sign != 0u ? 0x80808080u : 0u;
            const char* qrow = static_cast<const char*>(a.q) + qoff + 32 * half;
#pragma unroll
            for (int kk = 0; kk < KK8; ++kk) {
                const uint4 w0 = *reinterpret_cast<const uint4*>(qrow + 64 * kk);
                const uint4 w1 = *reinterpret_cast<const uint4*>(qrow + 64 * kk + 16);
                qf8[kk] = i32x8{(int)((w0.x & keep) ^ sg), (int)((w0.y & keep) ^ sg), (int)((w0.z & keep) ^ sg),
                                (int)((w0.w & keep) ^ sg), (int)((w1.x & keep) ^ sg), (int)((w1.y & keep) ^ sg),
                                (int)((w1.z & keep) ^ sg), (int)((w1.w & keep) ^ sg)};
            }
        } else {
            const bf16_t* qrow = static_cast<const bf16_t*>(a.q) + qoff + 8 * half;
#pragma unroll
            for (int kk = 0; kk < C::KK; ++kk) {
                uint4 w = *reinterpret_cast<const uint4*>(qrow + 16 * kk);
                w.x = (w.x & keep) ^ q_sign;
                w.y = (w.y & keep) ^ q_sign;
                w.z = (w.z & keep) ^ q_sign;
                w.w = (w.w & keep) ^ q_sign;
                qf[kk] = __builtin_bit_cast(bf16x8, w);
            }
        }
    }

    // ---- per-lane LDS read offsets (bytes within a stage) -------------------
    // K fragment of k-step kk: lane (key = col, half) reads chunk 2 kk + half
    // of row col: in region A at col * pitch + 32 kk + 16 half, in region B
    // at chunk (2 (kk - 32) + half) ^ (col mod 8).
    const int k_ra = col * C::KA_PITCH + 16 * half;
    int k_rb[C::KK - C::KKA];
#pragma unroll
    for (int kk = C::KKA; kk < C::KK; ++kk)
        k_rb[kk - C::KKA] = C::KB_OFF + col * 128 + 16 * ((2 * (kk - C::KKA) + half) ^ (col & 7));
    // V^T fragment (A of O^T), two transpose reads per 16-key step: lane l of
    // 16-lane group G = l / 16 supplies row 16 kst + 4 half + (l % 16) / 4
    // (+8 for the second read) and 4 columns starting at 32 nb + 16 (G % 2) +
    // 4 (l % 4); it receives 4 consecutive keys of column 32 nb + l % 32.
    // Wave w reads the column blocks nb = 4 w + j (bytes 256 w .. of a row).
    // FP8 K codes of k-step kk: lane (col, half) reads logical chunks
    // 4 kk + 2 half + e (e = 0, 1) of row col; in region A (kk < 8) the
    // physical chunk is that XOR (col mod 8), i.e. block kk / 2 of 8 chunks
    // and within it (4 (kk mod 2) + 2 half + e) ^ (col mod 8); in region B
    // (kk = 8) it is (2 half + e) XOR ((col / 2) mod 4).
    int k8a[2][2], k8b[2];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int e = 0; e < 2; ++e) k8a[p][e] = col * 512 + 16 * ((4 * p + 2 * half + e) ^ (col & 7));
#pragma unroll
    for (int e = 0; e < 2; ++e) k8b[e] = C::KB_OFF + col * 64 + 16 * ((2 * half + e) ^ ((col >> 1) & 3));
    int v_rd[C::NBW];
    {
        const int r0 = 4 * half + (lane & 15) / 4;
        const int cg = 2 * ((lane >> 4) & 1) + (lane & 3) / 2;
#pragma unroll
        for (int j = 0; j < C::NBW; ++j)
            v_rd[j] = (F8 ? C::VB_OFF : C::V_OFF) + r0 * C::VBROW_B + 16 * swz_v<64>(r0, 4 * j + cg) +
                      8 * (lane & 1) + 256 * wave;
    }
    auto kfrag = [&](const char* st, int kk) __attribute__((always_inline)) {
        const int off = kk < C::KKA ? k_ra + 32 * kk : k_rb[kk - C::KKA];
        return *reinterpret_cast<const bf16x8*>(st + off);
    };
    auto kfrag8 = [&](const char* st, int kk) __attribute__((always_inline)) {
        const int o0 = kk < 8 ? k8a[kk % 2][0] + 128 * (kk / 2) : k8b[0];
        const int o1 = kk < 8 ? k8a[kk % 2][1] + 128 * (kk / 2) : k8b[1];
        const uint4 w0 = *reinterpret_cast<const uint4*>(st + o0);
        const uint4 w1 = *reinterpret_cast<const uint4*>(st + o1);
        return i32x8{(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w, (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
    };
    const int unit_scales = 0x7f7f7f7f;  // E8M0 block scales of 2^0
    // the bf16 V^T operands: in the stage, or (FP8) in the widened tile
    auto vfrag = [&](const char* st, int j, int kst) __attribute__((always_inline)) {
        const char* vp = (F8 ? lds : st) + v_rd[j] + kst * 16 * C::VBROW_B;
        const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp));
        const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 8 * C::VBROW_B));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // P^T operand of (row block rbk, key step kst): the score-accumulator
    // layout of wave rbk, lane l's 16 bytes at 16 l (conflict-free both ways)
    char* const p_x = lds + C::P_OFF + 16 * lane;
    auto pslot = [&](int rbk, int kst) __attribute__((always_inline)) {
        return reinterpret_cast<bf16x8*>(p_x + (rbk * 2 + kst) * 1024);
    };

    // O^T accumulators of this wave: acc[j][rbk] = columns 128 w + 32 j x rows 32 rbk
    f32x16 acc[C::NBW][NRB];
#pragma unroll
    for (int j = 0; j < C::NBW; ++j)
#pragma unroll
        for (int rbk = 0; rbk < NRB; ++rbk)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[j][rbk][i] = 0.f;
    float m = neg_inf();      // reference max (log2 units) of this lane's query
    float l = 0.f;            // this lane half's sum of p
    float mx_all = neg_inf(); // largest tile max seen (log2 units)

    // One tile: S^T and the softmax of this wave's 32 rows (when one of them
    // sees a key of the tile; else P = 0), P^T to LDS, mid() (the barrier
    // that publishes P^T), then this wave's 128 columns of O^T for all rows.
    auto tile = [&](const char* st, int key0, bool vis, bool need_mask, auto&& mid)
                    __attribute__((always_inline)) {
        bf16x8 pb[2];
        if (vis) {
            // S^T = K Q^T
            f32x16 s;
            if constexpr (F8) {
                // 9 FP8 k-steps, two fragments read ahead
                f32x16 s0, s1;
                constexpr int W8 = 2;
                i32x8 fk8[W8];
#pragma unroll
                for (int w = 0; w < W8; ++w) fk8[w] = kfrag8(st, w);
#pragma unroll
                for (int o = 0; o < KK8; ++o) {
                    f32x16& d = (o & 1) ? s1 : s0;
                    if (o < 2) {
                        qk8_first(d, fk8[o % W8], qf8[o], unit_scales);
                    } else {
                        qk8_next(d, fk8[o % W8], qf8[o], unit_scales);
                    }
                    if (o + W8 < KK8) fk8[o % W8] = kfrag8(st, o + W8);
                }
                qk_fence(s0, s1);
                s = s0 + s1;
            } else {
                f32x16 s0, s1;
                bf16x8 fk[kWinW];
#pragma unroll
                for (int w = 0; w < kWinW; ++w) fk[w] = kfrag(st, w);
#pragma unroll
                for (int o = 0; o < C::NQK; ++o) {
                    f32x16& d = (o & 1) ? s1 : s0;
                    if (o < 2) {
                        qk_first(d, fk[o % kWinW], qf[o]);
                    } else {
                        qk_next(d, fk[o % kWinW], qf[o]);
                    }
                    if (o + kWinW < C::NQK) fk[o % kWinW] = kfrag(st, o + kWinW);
                }
                qk_fence(s0, s1);
                s = s0 + s1;
            }
            // online softmax; lane (col, half) holds keys key0 + 8 (i / 4) + 4 half + i % 4
            float mx = neg_inf();
            if (need_mask) {
                // key = key0 + 4 half + (compile-time offset): masked above the causal
                // bound dl or below the window's first key dlo
                const int dl = lim - key0 - 4 * half;
                const int dlo = win ? first - key0 - 4 * half : -1;  // first is INT32_MIN without a window
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int off = 8 * (i >> 2) + (i & 3);
                    s[i] = (off > dl || (VAR && off < dlo)) ? neg_inf() : s[i];
                }
            }
#pragma unroll
            for (int i = 0; i < 16; i += 2) mx = max3(mx, s[i], s[i + 1]);
            mx = half_max(mx);
            const float mt = mx == neg_inf() ? neg_inf() : mx * c;
            mx_all = fmaxf(mx_all, mt);
            m = m == neg_inf() ? mt : m;  // first visible tile fixes the frame
            const float nm = m == neg_inf() ? 0.f : -m;
            float lsum = 0.f;
#pragma unroll
            for (int i = 0; i < 16; i += 2) {
                float p0 = fast_exp2(__builtin_fmaf(s[i], c, nm));
                float p1 = fast_exp2(__builtin_fmaf(s[i + 1], c, nm));
                if (need_mask) {  // exact zeros also when c = 0 (-inf * 0 = NaN)
                    p0 = s[i] == neg_inf() ? 0.f : p0;
                    p1 = s[i + 1] == neg_inf() ? 0.f : p1;
                }
                lsum += p0 + p1;
                const bf16x2 pp = __builtin_convertvector(f32x2{p0, p1}, bf16x2);
                pb[i >> 3][i & 7] = pp[0];
                pb[i >> 3][(i & 7) + 1] = pp[1];
            }
            l += lsum;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) pb[0][i] = pb[1][i] = bf16_t(0.f);
        }
        *pslot(wave, 0) = pb[0];
        *pslot(wave, 1) = pb[1];
        mid();
        if constexpr (F8) {
            // this wave's 128 columns of the V codes (every row) -> the bf16 V
            // tile; no other wave reads or writes them.  Lane l: rows 8 i + l / 8,
            // codes 16 (8 w + l mod 8) .. +16 -> bf16 chunks 16 w + 2 (l mod 8)
            // and + 1, XOR 4 (row mod 4) as the reads expect.
            const char* vc = st + C::V_OFF + 16 * (8 * wave + (lane & 7));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 8 * i + (lane >> 3);
                const uint4 w = *reinterpret_cast<const uint4*>(vc + row * C::VROW_B);
                char* vb = lds + C::VB_OFF + row * C::VBROW_B + 16 * ((16 * wave + 2 * (lane & 7)) ^ (4 * (row & 3)));
                *reinterpret_cast<uint4*>(vb) = e4m3x8_to_bf16(uint2{w.x, w.y});
                *reinterpret_cast<uint4*>(vb + 16) = e4m3x8_to_bf16(uint2{w.z, w.w});
            }
        }
        // O^T += V^T P^T: per key step 4 V^T and 4 P^T operands, 16 MFMAs
#pragma unroll
        for (int kst = 0; kst < C::BN / 16; ++kst) {
            bf16x8 fv[C::NBW], fp[NRB];
#pragma unroll
            for (int j = 0; j < C::NBW; ++j) fv[j] = vfrag(st, j, kst);
#pragma unroll
            for (int rbk = 0; rbk < NRB; ++rbk) fp[rbk] = *pslot(rbk, kst);
#pragma unroll
            for (int j = 0; j < C::NBW; ++j)
#pragma unroll
                for (int rbk = 0; rbk < NRB; ++rbk)
                    acc[j][rbk] = mfma_32x32x16(fv[j], fp[rbk], acc[j][rbk]);
        }
    };

    // Ring of two K and two V slots that refill independently: tile t uses
    // slot t % 2 of each.  V of tile t + 1 is issued right after the barrier
    // that opens tile t (its slot held V of tile t - 1, whose O^T MFMAs every
    // wave has passed), K of tile t + 2 right after the barrier between the
    // softmax and O^T (its slot is the one S^T just read).  Each piece thus
    // has about a whole tile of compute to land.  Issue order per wave:
    // ... V(t), K(t+1), V(t+1), K(t+2) ...: when K(t) (or V(t)) is needed,
    // the NV + NK pieces issued after it may still be in flight.
    auto step = [&](int t, auto stage) __attribute__((always_inline)) {
        constexpr int ST = decltype(stage)::value;
        const DmaPlan dv = plan(t + 1, ST ^ 1);
        wait_vmcnt<NK + NV>();  // K of tile t
        __syncthreads();        // (also: every wave is done with P^T and V of tile t - 1)
#pragma unroll
        for (int j = 0; j < NV; ++j) v_piece(dv, j);
        auto mid = [&]() __attribute__((always_inline)) {
            const DmaPlan dk = plan(t + 2, ST);
            wait_vmcnt<NK + NV>();  // V of tile t
            __syncthreads();        // P^T of tile t is in LDS; S^T is done with K of tile t
#pragma unroll
            for (int j = 0; j < NK; ++j) k_piece(dk, j);
        };
        const int key0 = lo + t * C::BN;
        tile(lds + ST * C::STAGE_B, key0, key0 < kv_end_w,
             key0 + C::BN > nomask_end || (VAR && key0 < first_w), mid);
    };
    auto run_tiles = [&]() __attribute__((always_inline)) {
        for (int t = 0; t < n_tiles; t += 2) {
            step(t, std::integral_constant<int, 0>{});
            if (t + 1 < n_tiles) step(t + 1, std::integral_constant<int, 1>{});
        }
        // the pieces past the last tile (zeros) land before the slots are reused
        wait_vmcnt<0>();
        __syncthreads();
    };
    run_tiles();
    // Another pass if any lane of the work-group saw a tile max beyond its
    // reference by more than kMaxExcess.  (Written out as a second copy of the
    // loop: zeroing the accumulators on the back edge of one loop over both
    // passes would move them out of the AGPRs.)
    __shared__ int rerun;
    if (tid == 0) rerun = 0;
    __syncthreads();
    if (__builtin_amdgcn_ballot_w64(mx_all > m + kMaxExcess) != 0 && lane == 0) rerun = 1;
    __syncthreads();
    if (rerun != 0) {
        m = mx_all;
        l = 0.f;
#pragma unroll
        for (int j = 0; j < C::NBW; ++j)
#pragma unroll
            for (int rbk = 0; rbk < NRB; ++rbk)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[j][rbk][i] = 0.f;
        if (n_tiles > 0) prologue();
        run_tiles();
    }

    // epilogue: O = O^T / l, LSE = ln2 * (m + log2 l); with one split the sink
    // of head h joins the denominator (split partials leave it to the combine).
    // The owner of row r's scores publishes 1 / l of it for the waves that
    // hold its columns (the P^T exchange is free: the loop ended on a barrier).
    float l_tot = half_sum(l);
    float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (VAR && a.sinks != nullptr && a.splits == 1) {
        const float sk = a.sinks[h] * kLog2e;
        const float m2 = fmaxf(m, sk);
        if (m2 != neg_inf()) {
            const float alpha = fast_exp2(m - m2);  // 0 when no key is visible
            l_tot = l_tot * alpha + fast_exp2(sk - m2);
            inv = alpha / l_tot;
            m = m2;
        }
    }
    inv *= o_mul;  // descale_v (1 unless FP8)
    const float lse2 = l_tot > 0.f ? m + fast_log2(l_tot) : neg_inf();
    // partials stay natural-log; the final Stats may be base 2
    float lse = VAR && a.stats_log2 && a.splits == 1 ? lse2 : kLn2 * lse2;
    if (trunc) inv = lse = nan_f();
    const int64_t rows_all = (int64_t)a.batch * a.sq * a.hq;
    auto row_global = [&](int rr) {  // (b, token, head) row of row rr of this KV head
        return (int64_t)(b * a.sq + rr / a.group) * a.hq + kvh * a.group + rr % a.group;
    };
    const int slot = cg * a.merge;  // workspace slot of the group's partial
    if (row_ok && half == 0) {
        const int64_t row_g = row_global(r);
        if (a.splits > 1) {
            a.lse_part[(int64_t)slot * rows_all + row_g] = lse;
            // the group's other chunks are empty slots
            for (int c = slot + 1; c < min(a.splits, slot + a.merge); ++c)
                a.lse_part[(int64_t)c * rows_all + row_g] = neg_inf();
        } else if (a.lse != nullptr) {
            a.lse[row_g] = lse;
        }
    }
    // (1 / l, output row) of every row of the block, -1 past the end
    int2* const row_x = reinterpret_cast<int2*>(lds + C::P_OFF);
    if (half == 0) row_x[wave * 32 + col] = make_int2(__float_as_int(inv), row_ok ? (int)row_global(r) : -1);
    __syncthreads();
    // O rows go out through a wave-private LDS transpose (32 rows x 128
    // columns fp32 at a time, pitch 528 B): written in the accumulator layout
    // (one row per lane pair), read back two whole rows per instruction, so
    // every store writes 2 x 512 contiguous bytes (2 x 256 as bf16).
    char* const tx = lds + wave * (32 * kTxPitch);
    auto write_rows = [&](auto&& store) __attribute__((always_inline)) {
#pragma unroll
        for (int rbk = 0; rbk < NRB; ++rbk) {
#pragma unroll
            for (int j = 0; j < C::NBW; ++j)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const f32x16& c = acc[j][rbk];
                    const f32x4 w = {c[4 * gq], c[4 * gq + 1], c[4 * gq + 2], c[4 * gq + 3]};
                    *reinterpret_cast<f32x4*>(tx + col * kTxPitch + 4 * (32 * j + 8 * gq + 4 * half)) = w;
                }
            // lane l: row 2 i + l / 32 of the block, columns 4 (l % 32) .. + 3;
            // every read first, then the stores
            f32x4 v[16];
            int2 rx[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int rr_b = 2 * i + (lane >> 5);
                v[i] = *reinterpret_cast<const f32x4*>(tx + rr_b * kTxPitch + 16 * (lane & 31));
                rx[i] = row_x[rbk * 32 + rr_b];
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float iv = __int_as_float(rx[i].x);
                if (rx[i].y >= 0)
                    store((int64_t)rx[i].y, 128 * wave + 4 * (lane & 31),
                          f32x4{v[i][0] * iv, v[i][1] * iv, v[i][2] * iv, v[i][3] * iv});
            }
        }
    };
    if (a.splits > 1) {
        float* const op = a.o_part + (int64_t)slot * rows_all * DV;
        write_rows([&](int64_t row_g, int n, f32x4 w) __attribute__((always_inline)) {
            *reinterpret_cast<f32x4*>(op + row_g * DV + n) = w;
        });
    } else {
        write_rows([&](int64_t row_g, int n, f32x4 w) __attribute__((always_inline)) {
            uint2 u;
            u.x = pack_bf16x2(w[0], w[1]);
            u.y = pack_bf16x2(w[2], w[3]);
            *reinterpret_cast<uint2*>(a.o + row_g * DV + n) = u;
        });
    }
}

}  // namespace

bool decode_wide_supported(const DecodeArgs& a) {
    const int rows = a.sq * (a.hq / a.hkv);
    return a.dqk == 576 && a.dv == 512 && rows > 0 && a.page % 16 == 0;
}

namespace {
template <bool VAR, bool F8, int NRB>
hipError_t launch_wide_t(const WideArgs& a, int64_t n_wg, hipStream_t s) {
    using C = WCfg<576, 512, F8>;
    const void* kernel = (const void*)decode_wide_kernel<576, 512, VAR, F8, NRB>;
    hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_wide_kernel<576, 512, VAR, F8, NRB>), dim3((unsigned)n_wg), dim3(256),
                       (size_t)C::LDS_BYTES, s, a);
    return hipGetLastError();
}
template <bool VAR, bool F8>
hipError_t launch_wide_rows(const WideArgs& a, int64_t n_wg, hipStream_t s) {
    return a.rows <= 32 ? launch_wide_t<VAR, F8, 1>(a, n_wg, s) : launch_wide_t<VAR, F8, 4>(a, n_wg, s);
}
}  // namespace

hipError_t launch_decode_wide(const DecodeArgs& d, hipStream_t s) {
    WideArgs a;
    a.q = d.q;
    a.k_pool = d.k_pool;
    a.k_sp = d.k_sp;
    a.k_st = d.k_st;
    a.k_sh = d.k_sh;
    a.v_pool = d.v_pool;
    a.v_sp = d.v_sp;
    a.v_st = d.v_st;
    a.v_sh = d.v_sh;
    a.pt_k = d.pt_k;
    a.pt_v = d.pt_v;
    a.table_stride = d.table_stride;
    a.seq_lens = d.seq_lens;
    a.batch = d.batch;
    a.sq = d.sq;
    a.hq = d.hq;
    a.hkv = d.hkv;
    a.group = d.hq / d.hkv;
    a.page = d.page;
    a.splits = d.splits;
    a.rows = d.sq * a.group;
    a.n_rb = (a.rows + 127) / 128;
    // chunks per work-group: enough that the grid holds about two work-groups per CU
    a.merge = 1;
    if (d.splits > 1) {
        int dev = 0, n_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu < 1)
            n_cu = 1;
        const int64_t wgs = (int64_t)d.batch * d.hkv * d.splits * a.n_rb;
        const int64_t m = wgs / (2 * (int64_t)n_cu);
        a.merge = m < 1 ? 1 : (m > d.splits ? d.splits : (int32_t)m);
    }
    a.n_cg = (d.splits + a.merge - 1) / a.merge;
    const int64_t n_g = (int64_t)d.batch * d.hkv * a.n_cg;
    a.n_g = (int32_t)n_g;
    a.c = (d.scale < 0.f ? -d.scale : d.scale) * kLog2e;
    a.q_sign = d.scale < 0.f ? 0x80008000u : 0u;
    a.causal = d.causal;
    a.o_part = d.o_part;
    a.lse_part = d.lse_part;
    a.o = static_cast<bf16_t*>(d.o);
    a.lse = d.lse;
    // a window of 2^30 keys covers every key the int32 lengths can describe
    a.window = d.window > 0 ? min(d.window, 1 << 30) : 0;
    a.sinks = d.sinks;
    a.stats_log2 = d.stats_log2;
    a.descale_q = d.fp8 ? d.descale_q : nullptr;
    a.descale_k = d.fp8 ? d.descale_k : nullptr;
    a.descale_v = d.fp8 ? d.descale_v : nullptr;
    const int64_t n_wg = (n_g + 7) / 8 * 8 * a.n_rb;
    if (n_g == 0) return hipSuccess;
    // the epilogue passes output row indices as int32
    if (n_wg > INT32_MAX || (int64_t)d.batch * d.sq * d.hq > INT32_MAX) return hipErrorInvalidValue;
    const bool var = a.window > 0 || a.sinks != nullptr || a.stats_log2 != 0;
    if (d.fp8) return var ? launch_wide_rows<true, true>(a, n_wg, s) : launch_wide_rows<false, true>(a, n_wg, s);
    return var ? launch_wide_rows<true, false>(a, n_wg, s) : launch_wide_rows<false, false>(a, n_wg, s);
}

}  // namespace sdpa
