// Split-K decode attention over a quantized MLA latent cache on the int8 matrix
// cores (gfx950): 512 latent channels (4-bit codes, token-major, one scale group
// per token), a 64-channel bf16 rope part, 128-token pages, and query heads that
// share one latent per kv head (absorbed MLA: the latent is both key and value).
//
// Method: "KVarN" project review, Key Features (rotation, normalization rounds,
// asymmetric RTN with fp16 scale/zero/normalizer); the decode folds the rotation
// and normalizers into query and output and the per-token scales into scores.
//
// Per page, with qbar = q Q over the latent, q'_j = qbar_j c_j (c of this page):
//   score_t = sm * ( S_t * [A . q']_t + Z_t * sum_j q'_j + <q_rope, k_rope_t> )
//   o'_j   += c_j * ( [A^T . P~]_j + sum_t p_t Z_t ),  P~_t = p_t S_t
// with A the codes (integers 0..15). Both products run on
// v_mfma_i32_16x16x64_i8: the codes are exact int8 operands, and q' and P~ enter
// as 16-bit fixed-point integers (a power-of-two scale per page puts the largest
// possible magnitude just under 2^15 for q', 2^14 for P~) split into two signed
// int8 limbs x = 256 s1 + s0, each limb its own product, the two joined in int32
// (exact). One mixed-precision FMA against the constant 1.5 2^23 (+128) rounds
// a product to that integer and leaves it, biased by 128, in the low 16 bits of
// the result: its bytes are the limbs. sum_j q'_j is taken from the same rounded
// integers (v_dot4 on the limbs), so the rounding enters the score as
// sum_j d_j (S_t a_tj + Z_t), an error on the centered key. The rope product runs
// as v_mfma_f32_16x16x32_bf16 (query rope part split into bf16 hi + lo unless
// the query is bf16).
//
// Per page the workgroup unpacks the 4-bit codes once into an int8 image in LDS
// (token rows of 512 bytes, 16-byte slots XOR-swizzled); the score product reads
// it row-wise (16 channels of one token per lane), the value product through
// ds_read_b64_tr_b8 (8 tokens of one channel per lane and read), both without
// unpacking in the waves.
//
// Work split: a workgroup (8 waves) serves 64 query heads of one (sequence,
// kv head, page range). Waves w and w + 4 own the same 16 heads (the N dimension
// of every tile) and split the latent: wave half h = w / 4 takes channels
// 256 h .. 256 h + 255 of both products (and rope half h). The two partial scores
// meet through LDS; both waves then run the same softmax. Scores are computed
// transposed (tokens x heads): lane (head l16, group lq) holds tokens
// 16 j + 4 lq + i of tile j, which is the B operand layout of the value product
// with K-step k taking tiles 4 k .. 4 k + 3. The next page's codes, scales and
// normalizers are copied HBM -> LDS staging by direct-to-LDS loads during the
// current page's scores, its rope part after them.
#include "common.h"
#include "launch.h"
#include "xlane.h"

namespace kvq {

// 2^x as the bare v_exp_f32: exp2f adds a range split (two selects, an add and a
// ldexp) to return denormal results, and the weights here are at most 1, so one
// below 2^-126 flushing to zero changes nothing; exp2_fast(-inf) = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));

constexpr int XD = 512;    // latent channels
constexpr int XR = 64;     // rope channels
constexpr int XT = 128;    // tokens per page
constexpr int XNT = 512;   // threads per workgroup (8 waves)
constexpr int XHG = 64;    // query heads per workgroup

// Staging image of the next page (direct-to-LDS copies, natural chunk order):
// codes (token rows of 256 B), (S, Z) fp16 pairs per token, normalizer c.
constexpr int S_SZ = XT * XD / 2;           // 32768
constexpr int S_CN = S_SZ + XT * 4;         // 33280
constexpr int S_BYTES = S_CN + XD * 2;      // 34304
constexpr int S_CHUNKS = S_BYTES / 16;      // 2144 16-byte chunks
constexpr int S_COPIES = (S_CHUNKS + 63) / 64;  // 34 wave-wide copies
// Rope image (bf16 rows of 128 B; chunk g of row r at slot g ^ rswz(r), placed by
// the copy's source addresses): 1024 chunks, 16 wave-wide copies.
constexpr int R_BYTES = XT * XR * 2;
constexpr int R_COPIES = R_BYTES / 1024;
// Working image: int8 codes (token rows of 512 B, 16-channel slot g of row r at
// g ^ i8swz(r), bytes of a slot in channel order pi), (S, Z), normalizer in the
// same per-16-channel order pi.
constexpr int W_SZ = XT * XD;               // 65536
constexpr int W_CN = W_SZ + XT * 4;         // 66048
constexpr int W_BYTES = W_CN + XD * 2;      // 67072
constexpr int XCH_WORDS = 32 * 64;          // partial scores of one wave pair (32 per lane)

// Byte p of an int8 slot holds channel pi(p) of its 16 (the 4-bit unpack of a
// dword gives the even channels, then the odd ones):
// pi = 0 2 4 6 1 3 5 7 8 10 12 14 9 11 13 15.
__host__ __device__ constexpr int pi16(int p) { return 8 * (p >> 3) + 2 * (p & 3) + ((p >> 2) & 1); }

// Slot swizzle of an int8 code row. A score read takes one slot of 16 rows
// 16 j + 0..15; a transposing read takes one slot of the 8 rows r0 + {0,1,2,3,16,
// 17,18,19} in each 16-lane group: both land in distinct slots modulo 16.
__device__ __forceinline__ int i8swz(int r) { return (r & 3) | ((((r >> 2) & 3) ^ (((r >> 4) & 1) * 3)) << 2); }
// Rope rows are 128 B, two to a 256-byte bank window: the 16 rows of a score tile
// differ in (r & 1, rswz(r)).
__device__ __forceinline__ int rswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ half2v as_h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }

// a * b with a an fp16 value: one mixed-precision FMA (v_fma_mix_f32)
__device__ __forceinline__ float mul_h(_Float16 a, float b) { return __builtin_fmaf((float)a, b, 0.f); }
// fp16 hi + lo parts of the product a b: hi = f16(a b), lo = f16(a b - hi), each one
// mixed-precision FMA (the product is formed exactly inside it)
__device__ __forceinline__ void split_prod(float a, float b, _Float16 &hi, _Float16 &lo) {
    hi = (_Float16)__builtin_fmaf(a, b, 0.f);
    lo = (_Float16)__builtin_fmaf(a, b, -(float)hi);
}

// ((a << 8) + b) << 8 + c as two shift-adds: the inner sum made opaque, so that the
// compiler does not re-associate it into a << 16 + b << 8 + c (three instructions)
__device__ __forceinline__ int limbs3_combine(int a, int b, int c) {
    int t = (a << 8) + b;
    asm("" : "+v"(t));
    return (t << 8) + c;
}

// v_perm_b32: byte k of the result is byte sel_k of the pair (lo: bytes 0..3,
// hi: bytes 4..7)
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Eight int8 codes (two words) -> fp16 operands code 2^-18 (the bit pattern code << 6,
// a subnormal the matrix cores take exactly): each code byte becomes the low byte of a
// half (v_perm with zero bytes), and one shift moves both halves' codes up by 6 bits
__device__ __forceinline__ half8 codes_sub18(uint32_t w0, uint32_t w1) {
    return __builtin_bit_cast(half8, uint4{perm(0u, w0, 0x0C010C00u) << 6, perm(0u, w0, 0x0C030C02u) << 6,
                                           perm(0u, w1, 0x0C010C00u) << 6, perm(0u, w1, 0x0C030C02u) << 6});
}
constexpr float CODE_UNIT_INV = 262144.f;  // 2^18

// The two int8 limbs of four integers x_k, each given as y_k with (x_k + 128) in
// its low 16 bits: limb 1 (byte 1 of y_k) = (x_k + 128) >> 8, limb 0 = low byte
// of y_k minus 128 (byte k of each result word is element k).
__device__ __forceinline__ void limbs4(float y0, float y1, float y2, float y3, uint32_t &l1, uint32_t &l0) {
    const uint32_t p01 = perm(__float_as_uint(y1), __float_as_uint(y0), 0x05010400u);  // y0.b0 y1.b0 y0.b1 y1.b1
    const uint32_t p23 = perm(__float_as_uint(y3), __float_as_uint(y2), 0x05010400u);
    l0 = perm(p23, p01, 0x05040100u) ^ 0x80808080u;
    l1 = perm(p23, p01, 0x07060302u);
}

// The three int8 limbs of four integers 0 <= x_k < 2^19, each given as y_k with
// (x_k + 32896) in its low mantissa bits: with u = x + 32896, limb 2 = u >> 16
// (byte 2 of y minus 64), limb 1 = byte 1 of u minus 128, limb 0 = byte 0 minus 128.
__device__ __forceinline__ void limbs4x3(float y0, float y1, float y2, float y3, uint32_t &l2, uint32_t &l1,
                                         uint32_t &l0) {
    const uint32_t p01 = perm(__float_as_uint(y1), __float_as_uint(y0), 0x05010400u);  // y0.b0 y1.b0 y0.b1 y1.b1
    const uint32_t p23 = perm(__float_as_uint(y3), __float_as_uint(y2), 0x05010400u);
    const uint32_t q01 = perm(__float_as_uint(y1), __float_as_uint(y0), 0x0c0c0602u);  // y0.b2 y1.b2 0 0
    const uint32_t q23 = perm(__float_as_uint(y3), __float_as_uint(y2), 0x0c0c0602u);
    l0 = perm(p23, p01, 0x05040100u) ^ 0x80808080u;
    l1 = perm(p23, p01, 0x07060302u) ^ 0x80808080u;
    l2 = perm(q23, q01, 0x05040100u) ^ 0x40404040u;
}

// 1.5 2^23 + 128: an FMA result near this constant has an ulp of 1 and holds
// round(product) + 128 in its low mantissa bits (for |product| < 2^22)
constexpr float MAGIC_B = 12583040.0f;
// 1.5 2^23 + 32896: the same with the bias of the three-limb split
constexpr float MAGIC_P = 12615808.0f;

// Scale 2^k of the query fold: the largest power of two with b 2^k <= 32639, so
// that |x| + 128 stays below 2^15 (1 for b == 0 or not finite)
__device__ __forceinline__ float qfold_scale(float b) {
    const uint32_t u = __float_as_uint(b);
    const int e = (int)((u >> 23) & 0xffu);
    if (e == 0 || e == 0xff) return 1.f;
    int k = 141 - e;                           // b 2^k in [2^14, 2^15)
    if ((u & 0x7fffffu) > 0x7EFE00u) k -= 1;   // mantissa above 32639 / 16384
    k = max(-100, min(100, k));
    return __uint_as_float((uint32_t)(127 + k) << 23);
}
// 2^(18 - floor(log2 m)) for m > 0 (1 for m == 0 or not finite): m times it is below 2^19
__device__ __forceinline__ float pfold_scale(float m) {
    const int e = (int)((__float_as_uint(m) >> 23) & 0xffu);
    if (e == 0 || e == 0xff) return 1.f;
    const int k = max(-100, min(100, 145 - e));
    return __uint_as_float((uint32_t)(127 + k) << 23);
}
// 1 / x for x a power of two from the two functions above (exact)
__device__ __forceinline__ float pow2_inv(float x) { return __uint_as_float((uint32_t)(254 - (int)(__float_as_uint(x) >> 23)) << 23); }

// both bf16 halves of w times a power of two (exact for finite results)
__device__ __forceinline__ uint32_t bf16x2_scale(uint32_t w, float f) {
    const float lo = __uint_as_float(w << 16) * f, hi = __uint_as_float(w & 0xffff0000u) * f;
    return perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

__device__ __forceinline__ float lq_sum(float v) { return sum_x4rows(v); }  // the 4 lanes sharing lane & 15
__device__ __forceinline__ float lq_max(float v) { return max_x4rows(v); }

__device__ __forceinline__ uint16_t bf16_rn(float f) {  // fp32 -> bf16 bits, nearest even (finite inputs)
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// largest fp16 value (all >= 0) among the low halves (lo) and among the high halves
// with their sign bits cleared (hi) of four words
__device__ __forceinline__ void max_h4_words(const uint32_t (&w)[4], float &lo, float &hi) {
    u16x2 m = __builtin_bit_cast(u16x2, w[0] & 0x7fff7fffu);
#pragma unroll
    for (int i = 1; i < 4; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7fff7fffu));
    lo = half_bits_to_float(m.x);
    hi = half_bits_to_float(m.y);
}

}  // namespace

// Raw words of 8 consecutive query elements from element offset i (16-byte aligned for
// 16-bit types: 32 bytes of fp32 as two loads)
template <int QDT>
struct Q8 {
    uint4 w[QDT == KVQ_F32 ? 2 : 1];
};
template <int QDT>
__device__ __forceinline__ Q8<QDT> load_q8(const void *q, int64_t i) {
    Q8<QDT> r;
    if constexpr (QDT == KVQ_F32) {
        const uint4 *p = reinterpret_cast<const uint4 *>(reinterpret_cast<const float *>(q) + i);
        r.w[0] = p[0];
        r.w[1] = p[1];
    } else {
        r.w[0] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(q) + i);
    }
    return r;
}
template <int QDT>
__device__ __forceinline__ float q8_at(const Q8<QDT> &r, int e) {
    if constexpr (QDT == KVQ_F32) {
        const uint4 w = r.w[e >> 2];
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
        return __uint_as_float(u[e & 3]);
    } else {
        const uint4 w = r.w[0];
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
        const uint32_t b = (e & 1) ? u[e >> 1] >> 16 : u[e >> 1] & 0xffffu;
        return QDT == KVQ_F16 ? half_bits_to_float((uint16_t)b) : __uint_as_float(b << 16);
    }
}

// One workgroup's pages. The shared-memory regions come in as restrict pointers:
// after inlining, the compiler knows that the direct-to-LDS copies into `stage`
// and `ropeb` touch neither `work` nor `xch`, and lets them stay in flight while
// the current page is processed.
template <int QDT>
__device__ __forceinline__ void mla_body(const DecodeArgs &a, int units, int nhg, uint8_t *__restrict__ stage,
                                         uint8_t *__restrict__ ropeb, uint8_t *__restrict__ work,
                                         float *__restrict__ xch, uint32_t *__restrict__ qrl_lds) {
    constexpr bool QLO = QDT != KVQ_BF16;  // the rope query needs a bf16 lo part
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hs = wave & 3, half = wave >> 2;
    const int l16 = lane & 15, lq = lane >> 4;

    // Workgroup id -> (unit = (sequence, kv head, split), head group). The head
    // groups of one unit get ids that are equal modulo 8, so they run on the same
    // XCD and share its L2 for the page they all read.
    const int id = blockIdx.x;
    const int rest = id >> 3;
    const int hgi = rest % nhg;
    const int unit = (rest / nhg) * 8 + (id & 7);
    if (unit >= units) return;
    const int split = unit % a.splits;
    const int sk = unit / a.splits;
    const int hk = sk % a.Hkv, s = sk / a.Hkv;
    const int L = load_const(a.seq_lens, s);
    const int npages = min((L + XT - 1) / XT, a.bt_stride);
    const int pps = (npages + a.splits - 1) / a.splits;
    const int p0 = split * pps, p1 = min(npages, p0 + pps);
    const int hl0 = hgi * XHG + 16 * hs;                    // first head of this wave within the kv group
    const bool active = hl0 < a.grp;                        // uniform per wave
    const bool hq_ok = active && hl0 + l16 < a.grp;
    const int hq = hk * a.grp + hl0 + l16;                  // this lane's head (columns of every tile)

    auto page_blk = [&](int pi) {
        const int page = load_const(a.bt, (int64_t)s * a.bt_stride + pi);
        return (int64_t)page * a.Hkv + hk;
    };
    // codes, (S, Z) and normalizer of page pi -> staging image: wave w issues
    // wave-wide copies w, w + 8, ...; lane l of copy k moves chunk 64 k + l
    auto fetch_codes = [&](int pi) {
        const int64_t blk = page_blk(pi);
        const uint8_t *gcodes = a.kcodes + blk * (XT * XD / 2);
        const uint8_t *gsz = reinterpret_cast<const uint8_t *>(a.ksz + blk * (XT * 2));
        const uint8_t *gcn = reinterpret_cast<const uint8_t *>(a.kcn + blk * XD);
        for (int k = wave; k < S_COPIES; k += 8) {
            const int c = 64 * k + lane;
            const uint8_t *src = c < 2048 ? gcodes + 16 * c : c < 2080 ? gsz + 16 * (c - 2048) : gcn + 16 * (c - 2080);
            if (c < S_CHUNKS)
                __builtin_amdgcn_global_load_lds((const void *)src, (__attribute__((address_space(3))) void *)(stage + 1024 * k),
                                                 16, 0, 0);
        }
    };
    // rope part of page pi -> rope image, swizzled: LDS chunk p (row p >> 3, slot
    // p & 7) takes the row's chunk (p & 7) ^ rswz(row)
    auto fetch_rope = [&](int pi) {
        const uint8_t *grope = reinterpret_cast<const uint8_t *>(a.krope + page_blk(pi) * (XT * XR));
        for (int k = wave; k < R_COPIES; k += 8) {
            const int p = 64 * k + lane, r = p >> 3;
            const uint8_t *src = grope + 128 * r + 16 * ((p & 7) ^ rswz(r));
            __builtin_amdgcn_global_load_lds((const void *)src, (__attribute__((address_space(3))) void *)(ropeb + 1024 * k),
                                             16, 0, 0);
        }
    };
    auto page_ok = [&](int pi) {
        const int page = load_const(a.bt, (int64_t)s * a.bt_stride + pi);
        return page >= 0 && page < a.num_pages;
    };
    // The lane's query words are requested before the first page: 16 wide loads, issued
    // together, ahead of the page copies (the vector-memory count is in order, so waiting
    // for them leaves the copies in flight). Lanes past the kv group's heads read the
    // group's first head and use zeros.
    Q8<QDT> qraw[8][2], rraw;
    {
        const int64_t qb = ((int64_t)s * a.Hq + (hq_ok ? hq : hk * a.grp)) * (XD + XR);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int h = 0; h < 2; ++h) qraw[ks][h] = load_q8<QDT>(a.q, qb + 64 * ks + 16 * lq + 8 * h);
        rraw = load_q8<QDT>(a.q, qb + XD + 32 * half + 8 * lq);
    }
    asm volatile("" ::: "memory");  // keep the query loads ahead of the page requests
    int pi = p0;
    while (pi < p1 && !page_ok(pi)) ++pi;
    if (pi < p1) {
        fetch_codes(pi);
        fetch_rope(pi);
    }

    // ---- rotated query of the lane's head over all 512 channels (c = 64 ks + 16 lq + f);
    // the wave keeps its half: qv[ks][f] = qbar[256 half + 64 ks + 16 lq + f] / sqrt(512)
    float qv[4][16];
    // rope dims 32 half + 8 lq + 0..7 as bf16 pairs: hi words in LDS (wave-major, then
    // word, then lane; a fifth word holds the lane's mean square of qbar), lo words in
    // registers (bf16 queries have none)
    uint32_t *qrw = qrl_lds + wave * 5 * 64 + lane;
    uint32_t qrl[4];
    float qmax = 0.f;
    {
        float q[8][16];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int f = 0; f < 16; ++f) q[ks][f] = hq_ok ? q8_at<QDT>(qraw[ks][f >> 3], f & 7) : 0.f;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            uint32_t hw = 0, lw = 0;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float x = hq_ok ? q8_at<QDT>(rraw, 2 * e2 + h) : 0.f;
                const uint16_t hb = bf16_rn(x);
                const uint16_t lb = bf16_rn(x - bf16_bits_to_float(hb));
                hw |= (uint32_t)hb << (16 * h);
                lw |= (uint32_t)lb << (16 * h);
            }
            qrw[e2 * 64] = hw;
            qrl[e2] = lw;
        }
        // Walsh-Hadamard transform: bits of f and ks in registers, bits of lq
        // across lanes (lane bits 4 and 5)
#pragma unroll
        for (int b = 1; b < 16; b <<= 1)
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
#pragma unroll
                for (int f = 0; f < 16; ++f)
                    if (!(f & b)) {
                        const float x = q[ks][f], y = q[ks][f | b];
                        q[ks][f] = x + y;
                        q[ks][f | b] = x - y;
                    }
#pragma unroll
        for (int b = 1; b < 8; b <<= 1)
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
                if (!(ks & b))
#pragma unroll
                    for (int f = 0; f < 16; ++f) {
                        const float x = q[ks][f], y = q[ks | b][f];
                        q[ks][f] = x + y;
                        q[ks | b][f] = x - y;
                    }
        const float s16 = (lq & 1) ? -1.f : 1.f, s32 = (lq & 2) ? -1.f : 1.f;
        constexpr float INV_SQRT = 0.04419417382415922f;  // 1 / sqrt(512)
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int f = 0; f < 16; ++f) {
                float v = q[ks][f], lo, hi;
                pair16(v, lo, hi);
                v = __builtin_fmaf(s16, hi, lo);
                pair32(v, lo, hi);
                v = __builtin_fmaf(s32, hi, lo);
                v *= INV_SQRT;
                qmax = fmaxf(qmax, fabsf(v));
                q[ks][f] = v;
            }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int f = 0; f < 16; ++f) qv[ks][f] = half ? q[ks + 4][f] : q[ks][f];
    }
    qmax = lq_max(qmax);
    // mean square of qbar over the head's 512 channels (the score product's range test)
    float qms = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int f = 0; f < 16; ++f) qms = __builtin_fmaf(qv[ks][f], qv[ks][f], qms);
    qms = lq_sum(qms);  // this half's 256 channels
    qrw[4 * 64] = __float_as_uint(qms);  // kept in LDS beside the rope query words (registers are tight)

    const float sml2 = a.sm * 1.4426950408889634f;  // scores in log2 units
    float m_run = -INFINITY, l_run = 0.f;
    float psc_run = 1.f;  // o holds the page-weighted sums times psc_run
    f32x4 o[16];
#pragma unroll
    for (int mc = 0; mc < 16; ++mc) o[mc] = f32x4{0.f, 0.f, 0.f, 0.f};
    float *xp = xch + hs * XCH_WORDS;  // this pair's exchange slot

    while (pi < p1) {
        const int cur = pi;
        __builtin_amdgcn_s_waitcnt(0);  // this wave's copies into the staging and rope images have landed
        lds_barrier();                  // every wave's, and every wave is done with the working image
        // ---- staging -> working image: 4-bit code chunks unpacked to int8 slots;
        // (S, Z) copied; the normalizer rearranged to the slot channel order
        {
            const int r0 = tid >> 4, g = tid & 15;  // chunk tid + 512 k: row r0 + 32 k, 32 channels 32 g ..
            const int sw = i8swz(r0);               // rows 32 apart share the swizzle
            const int off0 = r0 * 512 + 16 * ((2 * g) ^ sw), off1 = r0 * 512 + 16 * ((2 * g + 1) ^ sw);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint4 w = *reinterpret_cast<const uint4 *>(stage + 16 * (tid + 512 * k));
                constexpr uint32_t M = 0x0F0F0F0Fu;
                *reinterpret_cast<uint4 *>(work + off0 + 16384 * k) = uint4{w.x & M, (w.x >> 4) & M, w.y & M, (w.y >> 4) & M};
                *reinterpret_cast<uint4 *>(work + off1 + 16384 * k) = uint4{w.z & M, (w.z >> 4) & M, w.w & M, (w.w >> 4) & M};
            }
            if (tid < 32) {
                *reinterpret_cast<uint4 *>(work + W_SZ + 16 * tid) = *reinterpret_cast<const uint4 *>(stage + S_SZ + 16 * tid);
            } else if (tid < 96) {
                // eight channels 8 q .. 8 q + 7 stay in their 16 bytes: halves 0 2 4 6 1 3 5 7
                const int qk = tid - 32;
                const uint4 w = *reinterpret_cast<const uint4 *>(stage + S_CN + 16 * qk);
                *reinterpret_cast<uint4 *>(work + W_CN + 16 * qk) =
                    uint4{perm(w.y, w.x, 0x05040100u), perm(w.w, w.z, 0x05040100u), perm(w.y, w.x, 0x07060302u),
                          perm(w.w, w.z, 0x07060302u)};
            }
        }
        lds_barrier();  // working image complete, staging image free
        // the next valid page's codes and side data travel during this page's scores
        ++pi;
        while (pi < p1 && !page_ok(pi)) ++pi;
        const bool more = pi < p1;
        if (more) fetch_codes(pi);
        const int rows = min(XT, L - cur * XT);

        // Per-lane byte offsets, made opaque here so that the per-step addresses
        // below are formed next to their reads rather than hoisted out of the loop.
        int lo = lane;
        asm volatile("" : "+v"(lo));
        const int ol16 = lo & 15, olq = lo >> 4;
        // score read of tile j, K-step ks: row 16 j + l16, slot (16 half | 4 ks | lq) ^ i8swz(row)
        const int ibase = 512 * ol16 + 16 * ((16 * half + olq) ^ ol16);
        // rope read of tile j: row 16 j + l16, chunk 4 half + lq
        const int rbase = 128 * ol16 + 16 * ((4 * half + olq) ^ ((ol16 & 7) ^ (ol16 >> 3)));
        // transposing read (K-step kk, read rr, channel tile mc): this lane supplies row
        // 64 kk + 32 rr + 16 (l16 >> 3) + 4 lq + ((l16 >> 1) & 3), half (l16 & 1) of slot
        // (16 half + mc) ^ i8swz(row)
        const int trow = 16 * (ol16 >> 3) + 4 * olq + ((ol16 >> 1) & 3);
        const int tsw = ((ol16 >> 1) & 3) | ((olq ^ (3 * (ol16 >> 3))) << 2);
        const int tbase = 512 * trow + 16 * ((16 * half) ^ tsw) + 8 * (ol16 & 1);

        // page bounds: the largest normalizer (query fold scale), the largest scale
        // and |zero point| (value fold scale); every lane takes two words of each
        float cmax, smax, zmax, cms;
        {
            const uint4 cw = *reinterpret_cast<const uint4 *>(work + W_CN + 16 * lane);
            const uint32_t c4[4] = {cw.x, cw.y, cw.z, cw.w};
            float c0, c1;
            max_h4_words(c4, c0, c1);
            cmax = max_x4rows(row_max16(fmaxf(c0, c1)));
            float cs = 0.f;  // sum of c^2 over the page's 512 channels (eight per lane)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const half2v c2 = as_h2(c4[i]);
                cs = __builtin_fmaf((float)c2.x, (float)c2.x, cs);
                cs = __builtin_fmaf((float)c2.y, (float)c2.y, cs);
            }
            cms = lq_sum(row_sum16(cs));
            const uint2 zw = *reinterpret_cast<const uint2 *>(work + W_SZ + 8 * lane);
            const uint32_t z4[4] = {zw.x, zw.y, zw.x, zw.y};
            float s0, z0;
            max_h4_words(z4, s0, z0);
            smax = max_x4rows(row_max16(s0));
            zmax = max_x4rows(row_max16(z0));
        }
        const float qsc = qfold_scale(qmax * cmax), qinv = pow2_inv(qsc);
        const float magic_q = MAGIC_B * qinv;

        f32x4 sc[8];
        if (active) {
            // Range test: the fixed-point fold gives every channel the page's one scale 2^k,
            // set by max |qbar| max c; channels far below that bound (a latent with a large
            // mean puts one rotated channel's normalizer far above the rest) keep few bits.
            // Pages where the bound exceeds 16 times rms(qbar) rms(c) take the fp16 product.
            const bool fp16 = __builtin_amdgcn_ballot_w64(qmax * qmax * cmax * cmax > 256.f * (__uint_as_float(qrw[4 * 64]) * (1.f / 256.f)) * (cms * (1.f / 512.f))) != 0;
            if (fp16) {
                // ---- scores^T from fp16 products: K-step ks2 takes 32 channels, lane lq the
                // eight of slot (16 half | 4 (ks2 >> 1) | lq), half ks2 & 1; the codes enter as
                // code 2^-18, the query as fp16 hi + lo of x 2^k
#pragma unroll
                for (int j = 0; j < 8; ++j) sc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
                float qc = 0.f;
#pragma unroll
                for (int ks2 = 0; ks2 < 8; ++ks2) {
                    const int ks = ks2 >> 1, hh = ks2 & 1;
                    const uint4 cw = *reinterpret_cast<const uint4 *>(work + W_CN + 32 * (16 * half + 4 * ks + olq) + 16 * hh);
                    const uint32_t c4[4] = {cw.x, cw.y, cw.z, cw.w};
                    half8 bh, bl;
#pragma unroll
                    for (int p = 0; p < 8; ++p) {
                        const half2v c2 = as_h2(c4[p >> 1]);
                        const float x = mul_h((p & 1) ? c2.y : c2.x, qv[ks][pi16(8 * hh + p)]);
                        qc += x;
                        _Float16 hi, lo;
                        split_prod(x, qsc, hi, lo);
                        bh[p] = hi;
                        bl[p] = lo;
                    }
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int off = 8192 * j + (ibase ^ ((64 * ks) ^ (192 * (j & 1)))) + 8 * hh;
                        const uint2 w = *reinterpret_cast<const uint2 *>(work + off);
                        const half8 av = codes_sub18(w.x, w.y);
                        sc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bh, sc[j], 0, 0, 0);
                        sc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bl, sc[j], 0, 0, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);  // one K-step's operands in flight at a time
                }
                const float qcx = lq_sum(qc) * qsc;  // sum_j x_j 2^k of the half
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint4 zw = *reinterpret_cast<const uint4 *>(work + W_SZ + 4 * (16 * j + 4 * olq));
                    const uint32_t z4[4] = {zw.x, zw.y, zw.z, zw.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const half2v sz = as_h2(z4[i]);  // (S, Z)
                        sc[j][i] = __builtin_fmaf((float)sz.x * CODE_UNIT_INV, sc[j][i], (float)sz.y * qcx);
                    }
                }
            } else {
                // ---- fold: q' = qbar o c for the wave's 256 channels as int8 limbs (B
                // operands of the four K-steps); sum_j x_j from the same limbs
                v4i B1[4], B0[4];
                int qc1 = 0, qc0 = 0;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const uint8_t *cp = work + W_CN + 32 * (16 * half + 4 * ks + olq);
                    const uint4 cwa = *reinterpret_cast<const uint4 *>(cp), cwb = *reinterpret_cast<const uint4 *>(cp + 16);
                    const uint32_t cw[8] = {cwa.x, cwa.y, cwa.z, cwa.w, cwb.x, cwb.y, cwb.z, cwb.w};
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        float y[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int p = 4 * d + i;
                            const half2v c2 = as_h2(cw[p >> 1]);
                            y[i] = __builtin_fmaf((float)((p & 1) ? c2.y : c2.x), qv[ks][pi16(p)], magic_q);
                        }
                        uint32_t l1, l0;
                        limbs4(y[0], y[1], y[2], y[3], l1, l0);
                        B1[ks][d] = (int)l1;
                        B0[ks][d] = (int)l0;
                        qc1 = __builtin_amdgcn_sdot4((int)l1, 0x01010101, qc1, false);
                        qc0 = __builtin_amdgcn_sdot4((int)l0, 0x01010101, qc0, false);
                    }
                }
                const float qcx = lq_sum((float)(256 * qc1 + qc0));  // sum_j x_j of the half (units of 2^-k)

                // ---- partial scores^T in units of 2^-k: tile j holds tokens 16 j + row;
                // y = S R + Z sum x, then + 2^k rope
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    v4i a1 = {0, 0, 0, 0}, a0 = {0, 0, 0, 0};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const int off = 8192 * j + (ibase ^ ((64 * ks) ^ (192 * (j & 1))));
                        const v4i av = *reinterpret_cast<const v4i *>(work + off);
                        a1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, B1[ks], a1, 0, 0, 0);
                        a0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, B0[ks], a0, 0, 0, 0);
                    }
                    const uint4 zw = *reinterpret_cast<const uint4 *>(work + W_SZ + 4 * (16 * j + 4 * olq));
                    const uint32_t z4[4] = {zw.x, zw.y, zw.z, zw.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const half2v sz = as_h2(z4[i]);  // (S, Z)
                        const float rf = (float)((a1[i] << 8) + a0[i]);
                        sc[j][i] = __builtin_fmaf((float)sz.x, rf, (float)sz.y * qcx);
                    }
                    __builtin_amdgcn_sched_barrier(0);  // one tile's operands in flight at a time
                }
            }
            // the rope query times 2^k, so that the rope product lands in the same units
            const bf16x8 rqh = __builtin_bit_cast(bf16x8, uint4{bf16x2_scale(qrw[0], qsc), bf16x2_scale(qrw[64], qsc),
                                                                 bf16x2_scale(qrw[128], qsc), bf16x2_scale(qrw[192], qsc)});
            bf16x8 rql;
            if constexpr (QLO)
                rql = __builtin_bit_cast(bf16x8, uint4{bf16x2_scale(qrl[0], qsc), bf16x2_scale(qrl[1], qsc),
                                                        bf16x2_scale(qrl[2], qsc), bf16x2_scale(qrl[3], qsc)});
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const bf16x8 ar = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(ropeb + rbase + 2048 * j));
                sc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar, rqh, sc[j], 0, 0, 0);
                if constexpr (QLO) sc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar, rql, sc[j], 0, 0, 0);
            }
            // the low half publishes its partial sums
            if (half == 0) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) xp[(4 * j + i) * 64 + lane] = sc[j][i];
            }
        }
        lds_barrier();
        // every wave's rope reads are done: the next page's rope part may land
        if (more) fetch_rope(pi);
        if (active && half == 1) {  // the high half completes the sums and publishes them
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sc[j][i] += xp[(4 * j + i) * 64 + lane];
                    xp[(4 * j + i) * 64 + lane] = sc[j][i];
                }
        }
        lds_barrier();
        if (!active) continue;
        if (half == 0) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) sc[j][i] = xp[(4 * j + i) * 64 + lane];
        }

        // ---- online softmax; lane (head l16, lq) holds tokens 16 j + 4 lq + i
        if (rows < XT) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * j + 4 * olq + i >= rows) sc[j][i] = -INFINITY;
        }
        float pmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) pmax = fmaxf(pmax, sc[j][i]);
        const float sml2q = sml2 * qinv;  // scores are in units of 2^-k
        pmax = lq_max(pmax) * sml2q;
        const float m_new = fmaxf(m_run, pmax);
        const float alpha = exp2_fast(m_run - m_new);
        m_run = m_new;
        // P~ = p S psc below 2^19 (three limbs); the zero-point sum sum_t p Z psc stays
        // below 2^29 in the int32 accumulator (|Z| / 8 enters the bound)
        // kept from page to page unless this page needs a smaller one or allows one 4x larger
        // (each change rescales o')
        const float psc_pg = pfold_scale(fmaxf(smax, zmax * 0.125f));
        const float psc = (psc_pg < psc_run || psc_pg >= 4.f * psc_run) ? psc_pg : psc_run;
        // the scaling enters the exponent: ps = p psc = 2^(score - m + log2 psc)
        const float m_ps = m_new - (float)((int)(__float_as_uint(psc) >> 23) - 127);
        float psum = 0.f, zs = 0.f;
        uint32_t pl2[8], pl1[8], pl0[8];  // P~ limbs of tile j, elements i in bytes i
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint4 zw = *reinterpret_cast<const uint4 *>(work + W_SZ + 4 * (16 * j + 4 * olq));
            const uint32_t z4[4] = {zw.x, zw.y, zw.z, zw.w};
            float y[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const half2v sz = as_h2(z4[i]);  // (S, Z)
                const float ps = exp2_fast(__builtin_fmaf(sc[j][i], sml2q, -m_ps));
                psum += ps;
                zs = __builtin_fmaf((float)sz.y, ps, zs);
                y[i] = __builtin_fmaf(ps, (float)sz.x, MAGIC_P);
            }
            limbs4x3(y[0], y[1], y[2], y[3], pl2[j], pl1[j], pl0[j]);
        }
        l_run = __builtin_fmaf(l_run, alpha, psum * pow2_inv(psc));
        const int zi = (int)rintf(lq_sum(zs));
        // o' is kept times the page's psc: rescaled when a head's maximum moved or psc changed
        const float beta = alpha * (psc * pow2_inv(psc_run));
        psc_run = psc;
        if (__builtin_amdgcn_ballot_w64(beta != 1.f) != 0)
#pragma unroll
            for (int mc = 0; mc < 16; ++mc)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[mc][i] *= beta;

        // ---- values^T over this wave's latent half: tile mc has channels 256 half + 16 mc
        // + pi(row) as A rows (rows 4 lq + i of the lane: cnp entries 16 mc + 4 lq + i);
        // K-step kk takes tokens 64 kk .. 64 kk + 63 in the order of score tiles 4 kk .. 4 kk + 3
        const v4i P2[2] = {{(int)pl2[0], (int)pl2[1], (int)pl2[2], (int)pl2[3]}, {(int)pl2[4], (int)pl2[5], (int)pl2[6], (int)pl2[7]}};
        const v4i P1[2] = {{(int)pl1[0], (int)pl1[1], (int)pl1[2], (int)pl1[3]}, {(int)pl1[4], (int)pl1[5], (int)pl1[6], (int)pl1[7]}};
        const v4i P0[2] = {{(int)pl0[0], (int)pl0[1], (int)pl0[2], (int)pl0[3]}, {(int)pl0[4], (int)pl0[5], (int)pl0[6], (int)pl0[7]}};
        const v4i zi4 = {zi, zi, zi, zi};
        const uint8_t *cnp = work + W_CN + 2 * (256 * half + 4 * olq);
#pragma unroll
        for (int mc = 0; mc < 16; ++mc) {
            v4i a2 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0}, a0 = zi4;
            const int toff = tbase ^ (16 * mc);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const v2i t0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) v2i *)(work + toff + 32768 * kk));
                const v2i t1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) v2i *)(work + toff + 32768 * kk + 16384));
                const v4i av = {t0.x, t0.y, t1.x, t1.y};
                a2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, P2[kk], a2, 0, 0, 0);
                a1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, P1[kk], a1, 0, 0, 0);
                a0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, P0[kk], a0, 0, 0, 0);
            }
            const uint2 cv2 = *reinterpret_cast<const uint2 *>(cnp + 32 * mc);
            const half2v c01 = as_h2(cv2.x), c23 = as_h2(cv2.y);
            const _Float16 cvv[4] = {c01.x, c01.y, c23.x, c23.y};
#pragma unroll
            for (int i = 0; i < 4; ++i) o[mc][i] = __builtin_fmaf((float)cvv[i], (float)limbs3_combine(a2[i], a1[i], a0[i]), o[mc][i]);
            if (mc & 1) __builtin_amdgcn_sched_barrier(0);  // at most two tiles' operands in flight
        }
    }

    // ---- split partial of the lane's head: o' (channels 256 half + 16 mc + pi(4 lq + i)),
    // m (natural log), l
    if (!hq_ok) return;
    l_run = lq_sum(l_run);
    const float oinv = pow2_inv(psc_run);
    // a partial row is XD + 2 = 514 floats
    float *wsr = a.ws + (((int64_t)s * a.Hq + hq) * a.splits + split) * (XD + 2);
#pragma unroll
    for (int mc = 0; mc < 16; ++mc)
#pragma unroll
        for (int i = 0; i < 4; ++i) wsr[256 * half + 16 * mc + pi16(4 * lq + i)] = o[mc][i] * oinv;
    if (lq == 0 && half == 0) {
        wsr[XD] = m_run == -INFINITY ? -INFINITY : m_run * 0.6931471805599453f;
        wsr[XD + 1] = l_run;
    }
}

template <int QDT>
__global__ void __launch_bounds__(XNT, 1) decode_mla_kernel(DecodeArgs a, int units, int nhg) {
    // Separate LDS variables: each gets its own alias scope, which lets the
    // compiler keep the direct-to-LDS copies into `stage` and `ropeb` in flight
    // across the accesses to the others.
    __shared__ __attribute__((aligned(16))) uint8_t stage[S_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t ropeb[R_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t work[W_BYTES];
    __shared__ float xch[4 * XCH_WORDS];
    __shared__ uint32_t qr[8 * 5 * 64];
    mla_body<QDT>(a, units, nhg, stage, ropeb, work, xch, qr);
}

bool decode_mla_supported(const DecodeArgs &a) {
    auto al16 = [](const void *p) { return ((uintptr_t)p & 15) == 0; };
    return al16(a.q) && al16(a.kcodes) && al16(a.ksz) && al16(a.kcn) && al16(a.krope) && a.D == XD && a.R == XR && a.Dv == XD && a.T == XT && a.kbits == 4 && a.kG == XD && a.kh == XD &&
           a.klayout == KVQ_TOKEN_MAJOR && a.vcodes == a.kcodes && a.grp % 16 == 0 && a.krope != nullptr;
}

// workgroups per (sequence, kv head, split): one per 64 query heads
int decode_mla_head_groups(const DecodeArgs &a) { return (a.grp + XHG - 1) / XHG; }

bool launch_decode_mla(const DecodeArgs &a, hipStream_t stream) {
    const int nhg = decode_mla_head_groups(a);
    const int units = a.B * a.Hkv * a.splits;
    const int grid = ((units + 7) / 8) * 8 * nhg;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(grid), dim3(XNT), 0, stream, a, units, nhg);
        return true;
    };
    switch (a.q_dtype) {
    case KVQ_F32: return go(decode_mla_kernel<KVQ_F32>);
    case KVQ_F16: return go(decode_mla_kernel<KVQ_F16>);
    default: return go(decode_mla_kernel<KVQ_BF16>);
    }
}

}  // namespace kvq
