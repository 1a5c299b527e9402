// tile_ops.h -- gfx950 building blocks of the LDS-DMA attention kernels:
// raw buffer resources, 16-byte LDS DMA (buffer_load_dwordx4 ... lds), the
// XOR chunk swizzles of row-major K/V tiles, explicit vmcnt waits, uniform
// scalar loads and the wave64 lane-half reductions.
#ifndef SDPA_TILE_OPS_H
#define SDPA_TILE_OPS_H

#include "sdpa_device.h"

namespace sdpa {

// Fourth word of a raw buffer resource on gfx9-family parts (CDNA): the
// range check returns zeros past num_records (also for loads into LDS).
constexpr int kRsrcWord3 = 0x00020000;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Swizzled position of 16-byte chunk lc of a K row: 16 lanes reading the
// same chunk of 16 consecutive rows hit 16 different 16-byte bank groups.
template <int CPR>
__device__ __forceinline__ int swz_k(int row, int lc) {
    return CPR >= 16 ? (lc ^ (row & 15)) : (lc ^ ((row >> 1) & 7));
}
// Swizzled chunk of a V row: the transpose reads of 32 lanes touch 4
// consecutive rows x 4 consecutive chunks, which then cover all banks.
template <int CPR>
__device__ __forceinline__ int swz_v(int row, int lc) {
    return CPR >= 16 ? (lc ^ (4 * (row & 3))) : (lc ^ (4 * ((row >> 1) & 1)));
}

// Lane-half exchange with v_permlane32_swap: on two copies a = b = v the
// swap leaves a = v of lanes 0..31 and b = v of lanes 32..63 in every lane,
// so a reduction of a and b is the reduction over the lane pair (l, l ^ 32).
// Written as inline asm because the compiler folds the two results of the
// builtin into one when both of its inputs are the same value.  The s_nop
// covers the VALU-write -> permlane-read hazard on the copies.
__device__ __forceinline__ void half_swap(float& a, float& b) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
// 3-input max (v_max3_f32).  Written in plain C so that the compiler sees
// every read of its operands: the scores come straight out of MFMA
// accumulators, and a VALU read of an MFMA result needs wait states after the
// MFMA that only the compiler's hazard recognizer inserts (an asm v_max3_f32
// would be issued right behind the MFMA and could read stale registers).
__device__ __forceinline__ float max3(float a, float b, float c) {
    return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource (no stride) over [base, base + nbytes).
__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint32_t nbytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    return u32x4{(uint32_t)p, (uint32_t)(p >> 32) & 0xffffu, (uint32_t)nbytes, (uint32_t)kRsrcWord3};
}

// LDS byte address of a pointer into this work-group's LDS.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p);
}

// 16-byte LDS DMA: lane L's 16 bytes at rsrc + voff land at LDS address
// lds + 16 L.  Issued as inline asm so the compiler does not hold LDS reads
// back behind every pending DMA (its alias model cannot tell the ring stages
// apart); completion is awaited explicitly with wait_vmcnt + a barrier.  The
// s_nop covers the M0-write -> LDS-DMA hazard.  M0 is declared clobbered;
// nothing else in these kernels keeps a value in M0 (the compiler only uses
// it for LDS DMA, interpolation and indexed moves, none of which occur).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t lds, int voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}
// The same with the nontemporal cache policy, for data read once per call
// (decode K/V streams): it does not displace reused lines from the caches.
__device__ __forceinline__ void dma16_stream(u32x4 rsrc, uint32_t lds, int voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Uniform 32-bit load through the scalar cache (read-only data).
__device__ __forceinline__ int32_t load_uniform(const int32_t* p, int64_t i) {
    return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

// Wait until at most N vector-memory operations of this wave are pending.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace sdpa

#endif  // SDPA_TILE_OPS_H
