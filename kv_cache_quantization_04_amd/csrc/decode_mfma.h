// Device helpers of the GQA decode kernels (gfx950): code unpacking into exact fp16
// matrix-core operands, power-of-two operand scaling, fp16 hi + lo splitting, page
// images and their prefetch.
#pragma once

#include "xlane.h"

#include "common.h"
#include "launch.h"

namespace kvq {

// 2^x as the bare v_exp_f32: exp2f adds a range split (two selects, an add and a
// ldexp) to return denormal results, and the weights here are at most 1, so one
// below 2^-126 flushing to zero changes nothing; exp2_fast(-inf) = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int MD = 128;      // head_dim of this kernel
constexpr int MNT = 256;     // threads per workgroup (4 waves)

__device__ __forceinline__ half2v as_h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }
// a * b with a an fp16 value: one mixed-precision FMA (v_fma_mix_f32) instead of a
// conversion and a multiply
__device__ __forceinline__ float mul_h(_Float16 a, float b) { return __builtin_fmaf((float)a, b, 0.f); }
__device__ __forceinline__ uint32_t as_u(half2v h) { return __builtin_bit_cast(uint32_t, h); }

// Eight codes of one lane chunk -> half8 in MFMA element order kk, where element
// kk holds chunk position e(kk) = (kk >> 1) + 4 (kk & 1) as the fp16 bit pattern
// code << (10 - B): the subnormal code * 2^(-14 - B), exact in the matrix cores.
// (The top of the subnormal range: accumulating products of the bare bit pattern,
// code * 2^-24, loses low-order bits.) The power of two goes into the fp32 scale
// factors. `lo` holds the chunk's bits starting at bit 0 (b * 8 bits used).
template <int B>
__device__ __forceinline__ half8 unpack8(uint32_t lo) {
    constexpr int K = 10 - B;
    constexpr uint32_t M = ((1u << B) - 1u) * 0x00010001u << K;
    uint32_t s = lo;
    // codes 4..7 to bits 16..: one bitfield insert; the other bits it leaves above the
    // low codes (copies of lower codes, or of bits past the chunk) are never shifted
    // into the mask below
    if constexpr (B == 2) s = (lo & 0xFFu) | ((lo << 8) & ~0xFFu);
    if constexpr (B == 3) s = (lo & 0xFFFu) | ((lo << 4) & ~0xFFFu);
    uint32_t p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int sh = K - B * i;  // compile-time after unrolling
        p[i] = (sh >= 0 ? (s << sh) : (s >> -sh)) & M;
    }
    return __builtin_bit_cast(half8, uint4{p[0], p[1], p[2], p[3]});
}
template <int B> constexpr int CODE_EXP = 14 + B;  // unpacked code n is n * 2^-CODE_EXP

// 2^(14 - floor(log2 m)) for m > 0 (1 for m == 0 or not finite): scales values
// with maximum magnitude m into [2^14, 2^15).
__device__ __forceinline__ float pow2_scale_for(float m) {
    const int e = (int)((__float_as_uint(m) >> 23) & 0xffu);
    if (e == 0 || e == 0xff) return 1.f;
    const int se = min(254, 268 - e);  // biased exponent of 2^(14 - (e - 127))
    return __uint_as_float((uint32_t)se << 23);
}

// 2^E / x for x a power of two from pow2_scale_for (exact; saturates at 2^127)
template <int E>
__device__ __forceinline__ float pow2_over(float x) {
    return __uint_as_float((uint32_t)min(254, 254 + E - (int)(__float_as_uint(x) >> 23)) << 23);
}

// fp16 hi + lo parts of the product a b: hi = f16(a b), lo = f16(a b - hi). Each is
// one mixed-precision FMA (v_fma_mixlo/mixhi_f16: b may be an fp16 value, the product
// is formed exactly inside the FMA), so lo carries the exact residual of hi.
__device__ __forceinline__ void split_prod(float a, float b, _Float16 &hi, _Float16 &lo) {
    hi = (_Float16)__builtin_fmaf(a, b, 0.f);
    lo = (_Float16)__builtin_fmaf(a, b, -(float)hi);
}

// Sum / max over the 4 lanes sharing lane & 15, by permlane swaps (VALU, no LDS
// round trip on the dependency chain); every lane gets the same bits.
__device__ __forceinline__ float xlane_sum_q(float v) { return sum_x4rows(v); }
__device__ __forceinline__ float xlane_max_q(float v) { return max_x4rows(v); }

// The 24 bits of eight 3-bit codes starting at byte-aligned bit `bit0`
// (three byte loads: never reads past the chunk).
__device__ __forceinline__ uint32_t load_bits3(const uint8_t *base, int64_t bit0) {
    const uint8_t *p = base + (bit0 >> 3);
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16);
}

// Page image of one (page, kv head) for the staged path (small pages): K codes,
// K (S, Z), K normalizer, V codes, V (S, Z), V normalizer, as laid out in HBM.
// 3-bit V codes are also re-aligned into a second buffer: the 24 bits of each
// 8-token chunk of a channel get a 32-bit word of their own.
template <int T, int KB, int VB>
struct PageImage {
    static constexpr int KC = T * MD * KB / 8, SZ = T * 4, CN = MD * 2, VC = T * MD * VB / 8;
    static constexpr int O_KC = 0, O_KSZ = KC, O_KCN = KC + SZ, O_VC = KC + SZ + CN;
    static constexpr int O_VSZ = O_VC + VC, O_VCN = O_VSZ + SZ, BYTES = O_VCN + CN;
    static constexpr int NPRE = (BYTES / 16 + 63) / 64;         // 16-byte chunks per lane
    static constexpr int VCW = VB == 3 ? MD * (T / 8) * 4 : 16;  // re-aligned V codes
};

// Copy N bytes from global memory into LDS with the wave's direct-to-LDS loads,
// every lane active in every instruction: 16-byte loads (1 KB per instruction)
// when N is a multiple of 1 KB, else 4-byte loads (256 B per instruction). No lane
// guard: the compiler has merged guarded direct-to-LDS loads of different regions
// across divergent branches into one instruction with one LDS base.
template <int N>
__device__ __forceinline__ void copy_region(const uint8_t *src, uint8_t *dst, int lane) {
    constexpr int W = N % 1024 == 0 ? 16 : 4;
    static_assert(N % (64 * W) == 0, "region size");
#pragma unroll
    for (int k = 0; k < N / (64 * W); ++k) {
        const void *g = (const void *)(src + 64 * W * k + W * lane);
        auto *l = (__attribute__((address_space(3))) void *)(dst + 64 * W * k);
        if constexpr (W == 16) __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
        else __builtin_amdgcn_global_load_lds(g, l, 4, 0, 0);
    }
}

// Direct-to-LDS load instructions that copy_region<N> issues.
template <int N>
constexpr int copy_instrs() { return N / (64 * (N % 1024 == 0 ? 16 : 4)); }

// s_waitcnt for at most N vector-memory operations outstanding (the other counters
// left alone)
template <int N>
__device__ __forceinline__ void wait_vm_upto() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int N>
struct Chunks {
    uint4 v[N];
};

// Where this lane's 16-byte chunks lane + 64 k of a page image come from: chunk k of
// block blk is at base[k] + blk * stride[k] (the region the chunk falls in, resolved
// once per kernel; lanes past the image re-read its last chunk, unused).
template <int T, int KB, int VB>
struct PageSrc {
    static constexpr int N = PageImage<T, KB, VB>::NPRE;
    uint64_t base[N];
    uint32_t stride[N];
};
template <int T, int KB, int VB>
__device__ __forceinline__ PageSrc<T, KB, VB> page_src(const DecodeArgs &a, int lane) {
    using PI = PageImage<T, KB, VB>;
    PageSrc<T, KB, VB> r;
#pragma unroll
    for (int k = 0; k < PI::NPRE; ++k) {
        const int off = min(1024 * k + 16 * lane, PI::BYTES - 16);
        uintptr_t src = (uintptr_t)(a.kcodes + off);
        uint32_t st = PI::KC;
        if (off >= PI::O_KSZ) src = (uintptr_t)a.ksz + (off - PI::O_KSZ), st = PI::SZ;
        if (off >= PI::O_KCN) src = (uintptr_t)a.kcn + (off - PI::O_KCN), st = PI::CN;
        if (off >= PI::O_VC) src = (uintptr_t)a.vcodes + (off - PI::O_VC), st = PI::VC;
        if (off >= PI::O_VSZ) src = (uintptr_t)a.vsz + (off - PI::O_VSZ), st = PI::SZ;
        if (off >= PI::O_VCN) src = (uintptr_t)a.vcn + (off - PI::O_VCN), st = PI::CN;
        r.base[k] = src;
        r.stride[k] = st;
    }
    return r;
}

// This lane's chunks of the page image of block `blk` (blk < 2^32, checked at launch).
template <int T, int KB, int VB>
__device__ __forceinline__ Chunks<PageImage<T, KB, VB>::NPRE> fetch_page(const PageSrc<T, KB, VB> &ps, uint32_t blk) {
    Chunks<PageImage<T, KB, VB>::NPRE> r;
#pragma unroll
    for (int k = 0; k < PageImage<T, KB, VB>::NPRE; ++k) {
        // a global-memory load (an integer address alone would make it a flat load, which
        // also holds the LDS counter until it returns)
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 v = *(const __attribute__((address_space(1))) u32x4 *)(ps.base[k] + (uint64_t)blk * ps.stride[k]);
        r.v[k] = uint4{v.x, v.y, v.z, v.w};
    }
    return r;
}

}  // namespace kvq
