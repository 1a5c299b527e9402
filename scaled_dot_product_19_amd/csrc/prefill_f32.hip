// prefill_f32.hip -- packed THD ragged prefill with fp32 inputs and outputs.
//
// Same operation and conventions as the bf16 prefill (packed THD rows from
// device prefix sums, bottom-right causal, GQA h -> h / G, FP32 natural-log
// LSE), computed entirely in fp32 on the vector ALUs: rounding fp32 inputs
// to bf16 for the matrix cores would move the logits by ~1e-3 and break the
// LSE accuracy the fp32 workload asks for.  Intended for small problems.
//
// One wave per (sequence, query row, head).  Keys are processed 64 at a time
// (one per lane): lane-parallel dot products, a wave-wide max / sum, then
// each lane accumulates its share of the output columns.
#include "sdpa_device.h"
#include "sdpa_launch.h"

namespace sdpa {
namespace {

constexpr int kMaxD = 256;

struct F32Args {
    const float* q;
    int64_t q_st, q_sh;
    const float* k;
    int64_t k_st, k_sh;
    const float* v;
    int64_t v_st, v_sh;
    float* o;
    int64_t o_st, o_sh;
    const int32_t* cu_q;
    const int32_t* cu_kv;
    int32_t hq, group, dqk, dv;
    float scale_log2;
    int32_t causal;
    float* lse;
    int32_t lse_layout, lse_s_max;
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__global__ __launch_bounds__(64) void prefill_f32_kernel(F32Args a) {
    __shared__ float qs[kMaxD];
    __shared__ float ps[64];
    const int lane = threadIdx.x;
    const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int q_beg = a.cu_q[b], lq = a.cu_q[b + 1] - q_beg;
    if (i == gridDim.x - 1) {
        // rows past the grid (a sequence longer than max_seqlen_q): NaN O and LSE
        for (int r = i + 1; r < lq; ++r) {
            float* orow = a.o + (int64_t)(q_beg + r) * a.o_st + (int64_t)h * a.o_sh;
            for (int n = lane; n < a.dv; n += 64) orow[n] = nan_f();
            if (a.lse != nullptr && lane == 0) {
                if (a.lse_layout == 1)
                    a.lse[(int64_t)(q_beg + r) * a.hq + h] = nan_f();
                else if (a.lse_layout == 2 && r < a.lse_s_max)
                    a.lse[((int64_t)b * a.lse_s_max + r) * a.hq + h] = nan_f();
            }
        }
    }
    if (i >= lq) return;
    const int kv_beg = a.cu_kv[b], lk = a.cu_kv[b + 1] - kv_beg;
    const int kvh = h / a.group;
    const int lim = a.causal ? min(lk - 1, i + lk - lq) : lk - 1;  // last visible key
    const float* qrow = a.q + (int64_t)(q_beg + i) * a.q_st + (int64_t)h * a.q_sh;
    for (int d = lane; d < a.dqk; d += 64) qs[d] = qrow[d];
    __syncthreads();

    constexpr int NPER = kMaxD / 64;  // output columns per lane
    float acc[NPER];
#pragma unroll
    for (int c = 0; c < NPER; ++c) acc[c] = 0.f;
    float m = neg_inf(), l = 0.f;
    for (int j0 = 0; j0 <= lim; j0 += 64) {
        const int j = j0 + lane;
        float x = neg_inf();
        if (j <= lim) {
            const float* krow = a.k + (int64_t)(kv_beg + j) * a.k_st + (int64_t)kvh * a.k_sh;
            float dot = 0.f;
            for (int d = 0; d < a.dqk; ++d) dot = fmaf(qs[d], krow[d], dot);
            x = dot * a.scale_log2;
        }
        const float m_new = fmaxf(m, wave_max(x));
        const float m_use = m_new == neg_inf() ? 0.f : m_new;
        const float alpha = fast_exp2(m - m_use);
        const float p = fast_exp2(x - m_use);
        l = l * alpha + wave_sum(p);
        m = m_new;
        ps[lane] = p;
        __syncthreads();
        const int nk = min(64, lim + 1 - j0);
#pragma unroll
        for (int c = 0; c < NPER; ++c) {
            const int n = lane + 64 * c;
            if (n < a.dv) {
                float s = acc[c] * alpha;
                for (int jj = 0; jj < nk; ++jj)
                    s = fmaf(ps[jj],
                             a.v[(int64_t)(kv_beg + j0 + jj) * a.v_st + (int64_t)kvh * a.v_sh + n],
                             s);
                acc[c] = s;
            }
        }
        __syncthreads();
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* orow = a.o + (int64_t)(q_beg + i) * a.o_st + (int64_t)h * a.o_sh;
#pragma unroll
    for (int c = 0; c < NPER; ++c) {
        const int n = lane + 64 * c;
        if (n < a.dv) orow[n] = acc[c] * inv;
    }
    if (a.lse != nullptr && lane == 0) {
        const float lse = l > 0.f ? kLn2 * (m + fast_log2(l)) : neg_inf();
        if (a.lse_layout == 1)
            a.lse[(int64_t)(q_beg + i) * a.hq + h] = lse;
        else if (a.lse_layout == 2 && i < a.lse_s_max)
            a.lse[((int64_t)b * a.lse_s_max + i) * a.hq + h] = lse;
    }
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& pa, hipStream_t s) {
    if (pa.batch == 0 || pa.max_q == 0) return hipSuccess;
    F32Args a;
    a.q = static_cast<const float*>(pa.q);
    a.q_st = pa.q_st;
    a.q_sh = pa.q_sh;
    a.k = static_cast<const float*>(pa.k);
    a.k_st = pa.k_st;
    a.k_sh = pa.k_sh;
    a.v = static_cast<const float*>(pa.v);
    a.v_st = pa.v_st;
    a.v_sh = pa.v_sh;
    a.o = static_cast<float*>(pa.o);
    a.o_st = pa.o_st;
    a.o_sh = pa.o_sh;
    a.cu_q = pa.cu_q;
    a.cu_kv = pa.cu_kv;
    a.hq = pa.hq;
    a.group = pa.hq / pa.hkv;
    a.dqk = pa.dqk;
    a.dv = pa.dv;
    a.scale_log2 = pa.scale * kLog2e;
    a.causal = pa.causal;
    a.lse = pa.lse;
    a.lse_layout = pa.lse_layout;
    a.lse_s_max = pa.lse_s_max;
    hipLaunchKernelGGL(prefill_f32_kernel, dim3(pa.max_q, pa.hq, pa.batch), dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace sdpa
