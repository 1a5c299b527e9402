// combine.hip -- LSE merge of split-KV partials, and the -inf seeding of
// padded LSE rows.
//
// Merge (the notes use split-KV partials merged by LSE -- cuDNN Frontend
// v1.31.0 Release Notes, "SDPA: paged KV, split-KV, and engine selection" --
// but print no formula; the textbook log-sum-exp merge is taken):
//   M = max_c LSE_c, LSE = M + ln sum_c exp(LSE_c - M),
//   O = sum_c exp(LSE_c - LSE) * O_c; every split empty -> O = 0, LSE = -inf.
// A split with LSE_c = -inf gets weight exactly 0 and its partial is not
// read (neither its bytes fetched nor its values used), so an empty split
// never contributes 0 * NaN and costs no traffic.  With attention sinks
// (decode with split-KV: v1.32.0 Release Notes, "SDPA: wider native forward
// support", split-KV supports sinks) the sink of the row's head joins the
// merge once, as one more term with no value: M = max(M, sink), the sum gains
// exp(sink - M), and no partial is scaled by it.
//
// -inf seeding: a padded (b, s_max, h) Stats buffer under THD is filled with
// -inf on the launch stream before the prefill writes the real rows (v1.30.0
// Release Notes, "New: the FlashInfer serving path runs on FROST").
#include "sdpa_device.h"
#include "sdpa_launch.h"

namespace sdpa {
namespace {

constexpr int kMaxSplits = 256;

// One wave per row; each lane owns columns lane, lane+64, ... (coalesced).
template <bool OUT_F32>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o_part,
                                                      const float* __restrict__ lse_part,
                                                      int splits, int64_t rows, int dv, void* o,
                                                      float* lse, int vec,
                                                      const float* __restrict__ sinks, int hq,
                                                      int stats_log2) {
    __shared__ float w_s[4][kMaxSplits];
    __shared__ float cw_s[4][kMaxSplits];  // the nonzero weights, in split order
    __shared__ int ci_s[4][kMaxSplits];    // and their splits
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t row = (int64_t)blockIdx.x * 4 + wave;
    const bool valid = row < rows;  // no early return: every wave reaches the barrier
    float* w = w_s[wave];
    float* cw = cw_s[wave];
    int* ci = ci_s[wave];
    int nz = 0;  // splits of nonzero weight (NaN counts as nonzero); uniform in the wave
    float lse_row = neg_inf();
    if (valid) {
        // row = (b * s_q + t) * hq + h: the sink of head h (natural-log units)
        const float sk = sinks != nullptr ? sinks[row % hq] : neg_inf();
        float m = sk;
        bool bad = false;  // a NaN partial (a split that could not be computed)
        for (int c = lane; c < splits; c += 64) {
            const float x = lse_part[(int64_t)c * rows + row];
            bad |= x != x;
            m = fmaxf(m, x);
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
        if (__builtin_amdgcn_ballot_w64(bad) != 0) {
            // the row's O and LSE become NaN too (fmaxf above skips NaN)
            lse_row = nan_f();
            for (int c = lane; c < splits; c += 64) w[c] = nan_f();
        } else if (m == neg_inf()) {
            for (int c = lane; c < splits; c += 64) w[c] = 0.f;
        } else {
            float sum = lane == 0 ? fast_exp2((sk - m) * kLog2e) : 0.f;  // 0 without a sink
            for (int c = lane; c < splits; c += 64)
                sum += fast_exp2((lse_part[(int64_t)c * rows + row] - m) * kLog2e);
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
            lse_row = m + kLn2 * fast_log2(sum);
            for (int c = lane; c < splits; c += 64)
                w[c] = fast_exp2((lse_part[(int64_t)c * rows + row] - lse_row) * kLog2e);
        }
        // compact the splits whose partial is read (lane c % 64 wrote w[c])
        const uint64_t below = (1ull << lane) - 1ull;
        for (int c0 = 0; c0 < splits; c0 += 64) {
            const int c = c0 + lane;
            const bool keep = c < splits && w[c] != 0.f;
            const uint64_t bal = __builtin_amdgcn_ballot_w64(keep);
            if (keep) {
                const int pos = nz + __builtin_popcountll(bal & below);
                cw[pos] = w[c];
                ci[pos] = c;
            }
            nz += __builtin_popcountll(bal);
        }
    }
    __syncthreads();
    if (!valid) return;
    if (vec) {  // d_v % 4 == 0, o_part 16-byte and o 8/16-byte aligned
        // 4 columns per lane and step over the splits of nonzero weight
        // only, in split order; the loads of 8 of them are issued together
        const f32x4* src = reinterpret_cast<const f32x4*>(o_part) + row * (dv / 4);
        const int64_t cstride = rows * (dv / 4);
        for (int n4 = lane; n4 < dv / 4; n4 += 64) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            int k = 0;
            for (; k + 8 <= nz; k += 8) {
                f32x4 x[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) x[j] = src[(int64_t)ci[k + j] * cstride + n4];
#pragma unroll
                for (int j = 0; j < 8; ++j) acc = acc + cw[k + j] * x[j];
            }
            for (; k < nz; ++k) acc = acc + cw[k] * src[(int64_t)ci[k] * cstride + n4];
            if (OUT_F32) {
                reinterpret_cast<f32x4*>(o)[row * (dv / 4) + n4] = acc;
            } else {
                uint2 u;
                u.x = pack_bf16x2(acc[0], acc[1]);
                u.y = pack_bf16x2(acc[2], acc[3]);
                reinterpret_cast<uint2*>(o)[row * (dv / 4) + n4] = u;
            }
        }
    } else {
        for (int n = lane; n < dv; n += 64) {
            float acc = 0.f;
            for (int k = 0; k < nz; ++k)
                acc = fmaf(cw[k], o_part[((int64_t)ci[k] * rows + row) * dv + n], acc);
            if (OUT_F32)
                static_cast<float*>(o)[row * dv + n] = acc;
            else
                static_cast<bf16_t*>(o)[row * dv + n] = (bf16_t)f32_to_bf16_bits(acc);
        }
    }
    if (lse != nullptr && lane == 0) lse[row] = stats_log2 ? lse_row * kLog2e : lse_row;
}

__global__ void fill_kernel(float* p, int64_t n, float value) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) p[i] = value;
}

}  // namespace

hipError_t launch_combine(const float* o_part, const float* lse_part, int32_t splits,
                          int64_t rows, int32_t dv, void* o, float* lse, int32_t out_f32,
                          hipStream_t s, const float* sinks, int32_t hq, int32_t stats_log2) {
    if (rows == 0) return hipSuccess;
    const int64_t blocks = (rows + 3) / 4;
    const int vec = (dv % 4 == 0) && reinterpret_cast<uintptr_t>(o_part) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(o) % (out_f32 ? 16 : 8) == 0;
    if (sinks == nullptr) hq = 1;
    if (out_f32)
        hipLaunchKernelGGL(combine_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, o_part,
                           lse_part, (int)splits, rows, (int)dv, o, lse, vec, sinks, (int)hq,
                           (int)stats_log2);
    else
        hipLaunchKernelGGL(combine_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, o_part,
                           lse_part, (int)splits, rows, (int)dv, o, lse, vec, sinks, (int)hq,
                           (int)stats_log2);
    return hipGetLastError();
}

hipError_t launch_fill_neg_inf(float* p, int64_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n,
                       -__builtin_inff());
    return hipGetLastError();
}

}  // namespace sdpa
