// The 128-point Walsh-Hadamard transform of 16 rows as bf16 matrix-core products
// (gfx950 v_mfma_f32_16x16x32_bf16): X' = X H with H[k][j] = (-1)^popcount(k & j),
// the Sylvester matrix in natural order, unnormalized. The entries of H are +-1,
// exact in bf16, so every product of a bf16 input with H is exact and the matrix
// cores accumulate in fp32: the result differs from an fp32 butterfly only by the
// order of the additions.
//
// Operands (M = 16 rows, N = 16 output channels per tile, K = 32 input channels per
// step): lane l supplies A[row l & 15][k = 32 s + 8 (l >> 4) + e], e = 0..7, in step s
// (16 contiguous bytes of a bf16 row), and B[k][j = 16 t + (l & 15)] for output tile
// t. With k = 32 s + 8 kg + e and j = 16 t + n:
//   popcount(k & j) = popcount(e & n & 7) + (kg & 1)(n >> 3) + (kg >> 1)(t & 1)
//                     + popcount(s & (t >> 1)),
// so B(s, t) is one of two per-lane patterns (t & 1) times a sign that depends on s
// and t only: four operand registers of 8 bf16 cover all 32 (s, t) pairs. Lane l
// receives X'[4 (l >> 4) + i][16 t + (l & 15)] in element i of output tile t.
// The output channels may also be permuted by the B columns at no cost as long as
// the pattern count stays two. The pair order used by the 128-token kernel puts
// channel j = 32 (t >> 1) + 2 n + (t & 1) in column n of tile t, so that each lane
// holds adjacent channel pairs: then
//   popcount(k & j) = (e & 1)(t & 1) + popcount((e >> 1) & n & 3) + popcount(kg & (n >> 2))
//                     + popcount(s & (t >> 1)),
// again two per-lane patterns (t & 1) and a sign of s and t.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Had128B {
    uint4 p0, p1;  // the two per-lane patterns (t & 1 = 0, 1), + sign; - is the sign bits flipped
};

// PAIRS = false: natural order, channel 16 t + n; true: pair order (above)
template <bool PAIRS = false>
__device__ __forceinline__ Had128B had128_operands(int lane) {
    const int n = lane & 15, kg = lane >> 4;
    uint32_t w[2][4];
#pragma unroll
    for (int t0 = 0; t0 < 2; ++t0)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            uint32_t word = 0;
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int e = 2 * h + b;
                const int par = PAIRS ? ((e & 1 & t0) + __builtin_popcount((e >> 1) & n & 3) +
                                         __builtin_popcount(kg & (n >> 2))) & 1
                                      : (__builtin_popcount(e & n & 7) + ((kg & 1) & (n >> 3)) + ((kg >> 1) & t0)) & 1;
                word |= (par ? 0xBF80u : 0x3F80u) << (16 * b);  // bf16 -1 / +1
            }
            w[t0][h] = word;
        }
    return Had128B{uint4{w[0][0], w[0][1], w[0][2], w[0][3]}, uint4{w[1][0], w[1][1], w[1][2], w[1][3]}};
}

// Makes the patterns opaque to the compiler where called (inside an item loop): the
// sign-flipped copies formed from them are then recomputed per call (8 instructions)
// instead of being hoisted and held, 16 more registers, across the whole loop.
__device__ __forceinline__ void opaque(Had128B &b) {
    asm volatile("" : "+v"(b.p0.x), "+v"(b.p0.y), "+v"(b.p0.z), "+v"(b.p0.w), "+v"(b.p1.x), "+v"(b.p1.y),
                 "+v"(b.p1.z), "+v"(b.p1.w));
}

// x[s]: the lane's 8 bf16 of step s (see above). out[t][i] = X'[4 (lane >> 4) + i][channel of
// (lane & 15, t)] in the order the operands were built for.
__device__ __forceinline__ void had128_rows16(const uint4 (&x)[4], const Had128B &hb, f32x4 (&out)[8]) {
    bf16x8 a[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = __builtin_bit_cast(bf16x8, x[s]);
    // the negated patterns exist only while the products run (8 sign flips per call)
    const uint32_t f = 0x80008000u;
    struct {
        bf16x8 p0, n0, p1, n1;
    } b = {__builtin_bit_cast(bf16x8, hb.p0),
           __builtin_bit_cast(bf16x8, uint4{hb.p0.x ^ f, hb.p0.y ^ f, hb.p0.z ^ f, hb.p0.w ^ f}),
           __builtin_bit_cast(bf16x8, hb.p1),
           __builtin_bit_cast(bf16x8, uint4{hb.p1.x ^ f, hb.p1.y ^ f, hb.p1.z ^ f, hb.p1.w ^ f})};
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const bool neg = __builtin_popcount(s & (t >> 1)) & 1;
            const bf16x8 bo = (t & 1) ? (neg ? b.n1 : b.p1) : (neg ? b.n0 : b.p0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], bo, acc, 0, 0, 0);
        }
        out[t] = acc;
    }
}

}  // namespace kvq
