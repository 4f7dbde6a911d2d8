// Device helpers shared by the gfx950 kernels of libkvq.so.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

constexpr int WAVE = 64;

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// fp32 -> fp16 bits, round to nearest even (v_cvt_f16_f32).
__device__ __forceinline__ uint16_t float_to_half_bits(float f) { return __half_as_ushort(__float2half_rn(f)); }
__device__ __forceinline__ float half_bits_to_float(uint32_t h) { return __half2float(__ushort_as_half((uint16_t)h)); }

__device__ __forceinline__ float load_as_float(const void *p, int dtype, int64_t idx) {
    if (dtype == KVQ_F32) return ((const float *)p)[idx];
    if (dtype == KVQ_F16) return half_bits_to_float(((const uint16_t *)p)[idx]);
    return bf16_bits_to_float(((const uint16_t *)p)[idx]);
}

// Workgroup barrier that orders LDS accesses only: this wave's LDS operations
// complete, then all waves meet. Global loads in flight (direct-to-LDS
// prefetches included) are not waited for, unlike __syncthreads(), whose fence
// drains the vector memory counter. The memory clobber keeps the compiler from
// moving memory accesses across it. A direct-to-LDS copy must be waited for
// explicitly (s_waitcnt vmcnt) before the barrier that publishes it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Read-only kernel input read through the constant address space, so that a
// wave-uniform index becomes a scalar load (the kernel never writes these).
template <typename V>
__device__ __forceinline__ V load_const(const V *p, int64_t i) {
    return ((const __attribute__((address_space(4))) V *)(uintptr_t)p)[i];
}

// Word 3 of a raw buffer resource on gfx9 (32-bit data format, no swizzle, no
// stride): loads at offsets past num_records bytes return zero.
constexpr int BUF_DWORD3 = 0x00020000;

// Butterfly partner exchange inside a group of lanes (xor pattern).
__device__ __forceinline__ float xor_shfl(float v, int mask) { return __shfl_xor(v, mask, WAVE); }

}  // namespace kvq
