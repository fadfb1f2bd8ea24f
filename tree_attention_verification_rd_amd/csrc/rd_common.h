// Shared device helpers for the gfx950 kernels of librd.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
// finite stand-in for -infinity in running maxima: exp2(x - kNegBig) never
// produces NaN and exp2(kNegBig - finite) underflows to 0
constexpr float kNegBig = -1.0e30f;

// bf16 bits -> float (exact)
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float -> bf16 bits, round to nearest, ties to even (inputs are finite)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// v_mfma_f32_16x16x32_bf16: D[16x16] += A[16x32] * B[32x16].
// Lane l holds A row (l%16) and B column (l%16), eight consecutive k-slots
// each for k-group l/16; D: lane l holds column l%16, rows 4*(l/16)+i.
__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Raw buffer loads: a 128-bit resource (base, byte range) plus a 32-bit
// per-lane byte offset.  Offsets at or past the range read as zero, which is
// how out-of-range rows and columns are filled without branches.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;        // an offset past every range
constexpr uint32_t kMaxRange = 0x7FFFFFFFu;   // largest range a resource may cover

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    // dword 3 = 0x00020000: raw 32-bit data format, the CDNA3/CDNA4 setting
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                             static_cast<int>(bytes < kMaxRange ? bytes : kMaxRange), 0x00020000);
}

__device__ __forceinline__ bf16x8 as_bf16(const u32x4 &v) {
    bf16x8 r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}

__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Explicitly counted loads.  The compiler inserts conservative "wait for
// every outstanding load" points at loop back-edges and before any LDS read
// that might alias a direct-to-LDS load, which would drain a multi-stage
// prefetch ring once per trip.  Ring loads are therefore issued with inline
// asm, invisible to the compiler's wait tracking, and the consumer waits
// explicitly with vm_wait<N>(), N = number of ring loads issued after the
// ones being waited for.  Loads complete in issue order, and any other load
// the compiler adds in between only makes the wait stronger.
typedef int i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4_t make_srsrc(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4_t r;
    r.x = __builtin_amdgcn_readfirstlane(static_cast<int>(a & 0xFFFFFFFFu));
    r.y = __builtin_amdgcn_readfirstlane(static_cast<int>((a >> 32) & 0xFFFFu));  // stride 0
    r.z = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes < kMaxRange ? bytes : kMaxRange));
    r.w = 0x00020000;
    return r;
}

template <int N>
__device__ __forceinline__ void vm_wait() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Direct global->LDS load (gfx950 buffer_load_dwordx4 ... lds): lane i's 16
// bytes land at LDS byte address m0 + 16*i, with the wave-uniform m0 set just
// before the load; an offset past the resource's range writes zeros.  No
// register receives the data.  It is counted explicitly (see above): the
// consumer waits with vm_wait<N>() and then a workgroup barrier before
// reading the LDS it fills.
__device__ __forceinline__ void lds_dma16(uint32_t lds_addr, const i32x4_t &rs, uint32_t off) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 ::"v"(off), "s"(rs), "s"(lds_addr)
                 : "memory", "m0");
}

// LDS byte address of a __shared__ object (the low half of its flat address)
__device__ __forceinline__ uint32_t lds_addr_of(const void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
    return __shfl_xor(v, mask, kWave);
}

// XCD-aware tile order.  Workgroups are dispatched round-robin over the 8
// XCDs (block i goes to XCD i % 8); this maps block ids so that each XCD
// receives one contiguous range of natural tile indices, keeping tiles that
// share data in one L2.  Bijective for any ntiles.
__device__ __forceinline__ int xcd_tile(int block, int ntiles) {
    constexpr int kXcd = 8;
    const int xcd = block % kXcd;
    const int j = block / kXcd;
    const int per = ntiles / kXcd;
    const int rem = ntiles % kXcd;
    return (xcd < rem) ? xcd * (per + 1) + j : rem * (per + 1) + (xcd - rem) * per + j;
}

}  // namespace rd
