// Cross-lane helpers of the gfx950 quantizers: DPP row operations and the
// ds_swizzle crossbar (no LDS memory, no VALU slot).
#pragma once

#include <hip/hip_runtime.h>

namespace kvq {

// DPP controls (gfx9 encoding)
constexpr int DPP_QUAD_XOR1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int DPP_ROR4 = 0x124;      // lane i <- lane (i - 4) mod 16
constexpr int DPP_ROR8 = 0x128;      // lane i <- lane (i - 8) mod 16

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// Partner value across lanes, lane ^ M within 32-lane groups (ds_swizzle bit mode).
template <int M>
__device__ __forceinline__ float swz_xor(float v) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (M << 10) | 0x1F));
}

// Value of lane K of the lane's 16-lane row (ds_swizzle broadcast mode: and-mask 0x10,
// or-mask K within each 32-lane group).
template <int K>
__device__ __forceinline__ float row_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x10 | (K << 5)));
}

// Walsh-Hadamard butterflies over the 16 lanes of a DPP row, all in DPP-fused
// FMAs, t <- t + s partner: stage 1 pairs lane l with l ^ 15 (row mirror, s = -1
// on lanes with bit 3 set), stage 2 with l ^ 7 (half-row mirror, bit 2), stage 3
// with l ^ 1 (bit 0), stage 4 with l ^ 2 (bit 1). The mirror pairings are linearly
// independent over the lane bits, so the four stages compute the 16-point Sylvester
// transform with its outputs relabelled and signed: lane l ends with
// hsign16(l) * (H16 x)[hperm16(l)] (checked against the plain transform on the CPU).
// The compiler does not fold a DPP move into an FMA, hence asm: one block per
// stage and eight independent values, led by the two wait states a DPP read needs
// after a VALU write of its source.
__device__ __forceinline__ int hperm16(int l) { return (int)((0x7214BED8FA9C3650ull >> (4 * l)) & 15); }
__device__ __forceinline__ float hsign16(int l) { return ((0xF9F6u >> l) & 1) ? -1.f : 1.f; }

#define KVQ_DPP_FMAC8(CTRL)                                                                                         \
    asm volatile("s_nop 1\n\t"                                                                                      \
                 "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                               \
                 "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                               \
                 "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                               \
                 "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                               \
                 "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                               \
                 "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                               \
                 "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                               \
                 "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf"                                     \
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])   \
                 : "v"(s))

// the four stages on eight values per lane; cc = lane & 15
__device__ __forceinline__ void hadamard16_lanes(float *v, int cc) {
    float s = (cc & 8) ? -1.f : 1.f;
    KVQ_DPP_FMAC8("row_mirror");
    s = (cc & 4) ? -1.f : 1.f;
    KVQ_DPP_FMAC8("row_half_mirror");
    s = (cc & 1) ? -1.f : 1.f;
    KVQ_DPP_FMAC8("quad_perm:[1,0,3,2]");
    s = (cc & 2) ? -1.f : 1.f;
    KVQ_DPP_FMAC8("quad_perm:[2,3,0,1]");
}
#undef KVQ_DPP_FMAC8

// Sum over the 16 lanes of a DPP row of four independent values, and min and max
// of four more, in DPP-fused instructions (t <- op(partner, t)): the stages rotate
// by 8 and by 4 inside the row, then swap lanes 2 and 1 apart inside each quad.
// Each instruction's DPP source was written one stage (four or eight instructions)
// earlier, so only the first stage needs the two wait states after the caller's
// writes.
#define KVQ_DPP_OP4(OP, CTRL)                                                                     \
    OP "_dpp %0, %0, %0 " CTRL " row_mask:0xf bank_mask:0xf\n\t" OP "_dpp %1, %1, %1 " CTRL \
       " row_mask:0xf bank_mask:0xf\n\t" OP "_dpp %2, %2, %2 " CTRL                           \
       " row_mask:0xf bank_mask:0xf\n\t" OP "_dpp %3, %3, %3 " CTRL " row_mask:0xf bank_mask:0xf\n\t"
__device__ __forceinline__ void row_sum16_x4(float (&v)[4]) {
    asm volatile("s_nop 1\n\t" KVQ_DPP_OP4("v_add_f32", "row_ror:8") KVQ_DPP_OP4("v_add_f32", "row_ror:4")
                     KVQ_DPP_OP4("v_add_f32", "quad_perm:[2,3,0,1]") KVQ_DPP_OP4("v_add_f32", "quad_perm:[1,0,3,2]")
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
}
#define KVQ_DPP_MINMAX(CTRL)                                                                              \
    "v_min_f32_dpp %0, %0, %0 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                                 \
    "v_min_f32_dpp %1, %1, %1 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                                 \
    "v_min_f32_dpp %2, %2, %2 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                                 \
    "v_min_f32_dpp %3, %3, %3 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                                 \
    "v_max_f32_dpp %4, %4, %4 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                                 \
    "v_max_f32_dpp %5, %5, %5 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                                 \
    "v_max_f32_dpp %6, %6, %6 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                                 \
    "v_max_f32_dpp %7, %7, %7 " CTRL " row_mask:0xf bank_mask:0xf\n\t"
__device__ __forceinline__ void row_minmax16_x4(float (&mn)[4], float (&mx)[4]) {
    asm volatile("s_nop 1\n\t" KVQ_DPP_MINMAX("row_ror:8") KVQ_DPP_MINMAX("row_ror:4")
                     KVQ_DPP_MINMAX("quad_perm:[2,3,0,1]") KVQ_DPP_MINMAX("quad_perm:[1,0,3,2]")
                 : "+v"(mn[0]), "+v"(mn[1]), "+v"(mn[2]), "+v"(mn[3]), "+v"(mx[0]), "+v"(mx[1]), "+v"(mx[2]),
                   "+v"(mx[3]));
}
#undef KVQ_DPP_OP4
#undef KVQ_DPP_MINMAX

// One packed bf16 pair (x0 in the low half, x1 in the high half) -> x0 + x1 and
// x0 - x1 in fp32, the first Walsh-Hadamard butterfly straight from the loaded word:
// v_dot2_f32_bf16 against the pair (1, 1), the second with the upper product negated.
// A sum whose exact value needs more than 24 bits (exponents more than 14 apart) is
// truncated rather than rounded to nearest (checked on the box): at most 1 ulp.
__device__ __forceinline__ void bf16_pair_butterfly(uint32_t w, float &sum, float &dif) {
    const uint32_t one2 = 0x3F803F80u;  // bf16 (1, 1)
    asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(sum) : "v"(w), "s"(one2));
    asm("v_dot2_f32_bf16 %0, %1, %2, 0 neg_hi:[0,1,0]" : "=v"(dif) : "v"(w), "s"(one2));
}
// acc + x0^2 + x1^2 of a packed bf16 pair (the products are exact in fp32)
__device__ __forceinline__ float bf16_pair_sumsq(uint32_t w, float acc) {
    asm("v_dot2_f32_bf16 %0, %1, %1, %0" : "+v"(acc) : "v"(w));
    return acc;
}

// Lanes 16 and 32 apart, through the gfx950 permlane swaps (VALU, no LDS round trip).
// Swapping x with itself leaves in `lo` the value of the even 16-lane row (pair16) or
// of the lower 32 lanes (pair32) of the lane's pair, and in `hi` the odd / upper one:
// lo + hi is the pair's sum in both lanes (same bits), and lo + s hi with s = -1 on the
// odd / upper member is the Walsh-Hadamard butterfly (even: x + partner, odd: partner - x).
__device__ __forceinline__ void pair16(float x, float &lo, float &hi) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair32(float x, float &lo, float &hi) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
}
// sum / max over the four lanes l, l ^ 16, l ^ 32, l ^ 48
__device__ __forceinline__ float sum_x4rows(float v) {
    float lo, hi;
    pair16(v, lo, hi);
    v = lo + hi;
    pair32(v, lo, hi);
    return lo + hi;
}
__device__ __forceinline__ float max_x4rows(float v) {
    float lo, hi;
    pair16(v, lo, hi);
    v = fmaxf(lo, hi);
    pair32(v, lo, hi);
    return fmaxf(lo, hi);
}

// Sum / min / max over the 16 lanes of a DPP row; every lane gets the same bits.
__device__ __forceinline__ float row_sum16(float s) {
    s += dpp<DPP_ROR8>(s);
    s += dpp<DPP_ROR4>(s);
    s += dpp<DPP_QUAD_XOR2>(s);
    s += dpp<DPP_QUAD_XOR1>(s);
    return s;
}
__device__ __forceinline__ float row_min16(float s) {
    s = fminf(s, dpp<DPP_ROR8>(s));
    s = fminf(s, dpp<DPP_ROR4>(s));
    s = fminf(s, dpp<DPP_QUAD_XOR2>(s));
    return fminf(s, dpp<DPP_QUAD_XOR1>(s));
}
__device__ __forceinline__ float row_max16(float s) {
    s = fmaxf(s, dpp<DPP_ROR8>(s));
    s = fmaxf(s, dpp<DPP_ROR4>(s));
    s = fmaxf(s, dpp<DPP_QUAD_XOR2>(s));
    return fmaxf(s, dpp<DPP_QUAD_XOR1>(s));
}

// 32 byte codes (each < 2^BITS) in stream order, four per word (code 4 i + b in byte
// b of bw[i]) -> the BITS words of their little-endian bitstream. Within a word the
// four codes are joined in parallel (SWAR): (w | w >> (8 - BITS)) puts bytes 1 and 3
// next to bytes 0 and 2, the mask keeps the two 2 BITS-bit fields, and a shift by
// 16 - 2 BITS joins them: 4 BITS bits per word in four instructions.
template <int BITS>
__device__ __forceinline__ void pack32_codes(const uint32_t (&bw)[8], uint32_t (&out)[BITS]) {
    constexpr uint32_t F = (1u << (2 * BITS)) - 1u;
#pragma unroll
    for (int d = 0; d < BITS; ++d) out[d] = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t v = (bw[i] | (bw[i] >> (8 - BITS))) & (F * 0x00010001u);
        const uint32_t x = (v & F) | (v >> (16 - 2 * BITS));
        constexpr int W = 4 * BITS;  // bits per word of codes
        const int pos = W * i;       // compile-time after unrolling
        out[pos >> 5] |= x << (pos & 31);
        if ((pos & 31) + W > 32) out[(pos >> 5) + 1] |= x >> (32 - (pos & 31));
    }
}

}  // namespace kvq
