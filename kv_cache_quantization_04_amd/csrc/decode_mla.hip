// Split-K decode attention over a quantized MLA latent cache with MFMA (gfx950):
// 512 latent channels (4-bit codes, token-major, one scale group per token),
// a 64-channel bf16 rope part, 128-token pages, and query heads that share one
// latent per kv head (absorbed MLA: the latent is both key and value).
//
// Method: "KVarN" project review, Key Features (rotation, normalization rounds,
// asymmetric RTN with fp16 scale/zero/normalizer); the decode folds the rotation
// and normalizers into query and output and the per-token scales into scores.
//
// Per page, with qbar = q Q over the latent, q'_j = qbar_j c_j (c of this page):
//   score_t = sm * ( S_t * [A . q']_t + Z_t * sum_j q'_j + <q_rope, k_rope_t> )
//   o'_j   += c_j * ( [A^T . P~]_j + sum_t p_t Z_t ),  P~_t = p_t S_t
// with A the codes, exact in fp16 (as subnormals n 2^-18). Both products run as
// v_mfma_f32_16x16x32_f16 with q' and P~ split into fp16 hi + lo parts after a
// power-of-two scaling; the rope product runs as v_mfma_f32_16x16x32_bf16 with
// the query's rope part split into bf16 hi + lo.
//
// Work split: a workgroup (8 waves) serves 64 query heads of one (sequence,
// kv head, page range). Waves w and w + 4 own the same 16 heads, which form the
// N dimension of every tile, and split the latent: wave half h = w / 4 takes
// channels 256 h .. 256 h + 255 of the score product (and rope half h), and the
// same channels of the value product. The two partial scores meet through LDS;
// both waves then run the same softmax. Scores are computed transposed (tokens
// x heads), so the probability tile lands, lane for lane, in the B operand of
// the value product (latent x heads); that product's A operand (the latent
// transposed to 16 tokens of one channel per lane) comes from LDS by
// ds_read_b64_tr_b4. Each thread prefetches its share of the next page into
// registers while the current page is processed from LDS.
#include "common.h"
#include "launch.h"
#include "xlane.h"

namespace kvq {

// 2^x as the bare v_exp_f32: exp2f adds a range split (two selects, an add and a
// ldexp) to return denormal results, and the weights here are at most 1, so one
// below 2^-126 flushing to zero changes nothing; exp2_fast(-inf) = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// a * b with a an fp16 value: one mixed-precision FMA (v_fma_mix_f32) instead of a
// conversion and a multiply
__device__ __forceinline__ float mul_h(_Float16 a, float b) { return __builtin_fmaf((float)a, b, 0.f); }
// fp16 hi + lo parts of the product a b: hi = f16(a b), lo = f16(a b - hi). Each is
// one mixed-precision FMA (v_fma_mixlo/mixhi_f16: b may be an fp16 value, the product
// is formed exactly inside the FMA), so lo carries the exact residual of hi.
__device__ __forceinline__ void split_prod(float a, float b, _Float16 &hi, _Float16 &lo) {
    hi = (_Float16)__builtin_fmaf(a, b, 0.f);
    lo = (_Float16)__builtin_fmaf(a, b, -(float)hi);
}
// largest of the fp16 values (all >= 0) in the low and high halves of four words,
// taken on the bit patterns (the order of non-negative fp16 values)
__device__ __forceinline__ float max_h8(const uint32_t (&w)[4]) {
    u16x2 m = __builtin_bit_cast(u16x2, w[0]);
#pragma unroll
    for (int i = 1; i < 4; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i]));
    return half_bits_to_float(m.x > m.y ? m.x : m.y);
}

constexpr int XD = 512;    // latent channels
constexpr int XR = 64;     // rope channels
constexpr int XT = 128;    // tokens per page
constexpr int XNT = 512;   // threads per workgroup (8 waves)
constexpr int XHG = 64;    // query heads per workgroup

// LDS image of one page (bytes). Codes: token row r (256 B) holds its 16-byte
// chunk g at slot g ^ swz(r); rope: row r (128 B) holds chunk g at slot g ^ rswz(r);
// (S, Z) pairs and the normalizer in natural order.
constexpr int L_CODES = 0;
constexpr int L_ROPE = XT * XD / 2;             // 32768
constexpr int L_SZ = L_ROPE + XT * XR * 2;      // 49152
constexpr int L_CN = L_SZ + XT * 4;             // 49664
constexpr int L_BYTES = L_CN + XD * 2;          // 50688
constexpr int NCHUNK = L_BYTES / 16;            // 3168 16-byte chunks per page
constexpr int CPT = (NCHUNK + XNT - 1) / XNT;   // 7 chunks per thread in the staging copy
constexpr int NDMA = (NCHUNK + 63) / 64;        // 50 wave-wide direct-to-LDS copies per page
// shared memory: staging image (natural chunk order, written by direct-to-LDS
// copies), working image (swizzled), score exchange [pair][33][64] floats, and
// each wave's rope query (bf16 hi / lo words, lane-major): 151552 bytes
constexpr int XCH_WORDS = 33 * 64;

// Slot swizzle of a code row: the 16 rows read together by either product land
// in 16 different 16-byte slots (rows 4b + i + 16 q of a score tile, and rows
// 16 lq + i of a transposed read).
__device__ __forceinline__ int swz(int r) { return (r & 15) ^ ((r >> 2) & 12); }
// Rope rows are 128 B, two to a bank window: the 16 rows of a score tile (rows
// 4 b + i + 16 q) differ in (r & 1, rswz(r)).
__device__ __forceinline__ int rswz(int r) { return ((r >> 1) & 1) | ((r >> 3) & 6); }

__device__ __forceinline__ half2v as_h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }

// Eight 4-bit codes of one dword -> half8 in MFMA element order kk, element kk
// holding nibble e(kk) = (kk >> 1) + 4 (kk & 1). Each code n becomes the fp16 bit
// pattern n << 6, the subnormal n * 2^-18, which the matrix cores take exactly
// (with the bare pattern n * 2^-24 their accumulation loses low-order bits); the
// factor 2^18 goes into the fp32 scale of the product.
__device__ __forceinline__ half8 unpack8_4(uint32_t w) {
    constexpr uint32_t M = 0x000F000Fu << 6;
    const uint32_t p0 = (w << 6) & M, p1 = (w << 2) & M, p2 = (w >> 2) & M, p3 = (w >> 6) & M;
    return __builtin_bit_cast(half8, uint4{p0, p1, p2, p3});
}
constexpr int CODE_EXP = 18;  // unpacked code n is n * 2^-18

// 2^(14 - floor(log2 m)) for m > 0 (1 for m == 0 or not finite).
__device__ __forceinline__ float pow2_scale(float m) {
    const int e = (int)((__float_as_uint(m) >> 23) & 0xffu);
    if (e == 0 || e == 0xff) return 1.f;
    const int se = min(254, 268 - e);
    return __uint_as_float((uint32_t)se << 23);
}

// 2^CODE_EXP / x for x a power of two from pow2_scale (exact; saturates at 2^127)
__device__ __forceinline__ float code_over(float x) {
    return __uint_as_float((uint32_t)min(254, 254 + CODE_EXP - (int)(__float_as_uint(x) >> 23)) << 23);
}

__device__ __forceinline__ float lq_sum(float v) { return sum_x4rows(v); }  // the 4 lanes sharing lane & 15
__device__ __forceinline__ float lq_max(float v) { return max_x4rows(v); }

__device__ __forceinline__ uint16_t bf16_rn(float f) {  // fp32 -> bf16 bits, nearest even (finite inputs)
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

}  // namespace

template <int QDT>
__device__ __forceinline__ float load_q(const void *q, int64_t i) {
    if constexpr (QDT == KVQ_F32) return reinterpret_cast<const float *>(q)[i];
    else if constexpr (QDT == KVQ_F16) return half_bits_to_float(reinterpret_cast<const uint16_t *>(q)[i]);
    else return bf16_bits_to_float(reinterpret_cast<const uint16_t *>(q)[i]);
}

// One workgroup's pages. The three shared-memory regions come in as restrict
// pointers: after inlining, the compiler knows that the direct-to-LDS copies
// into `stage` touch neither `work` nor `xch`, and lets them stay in flight while
// the current page is processed.
template <int QDT>
__device__ __forceinline__ void mla_body(const DecodeArgs &a, int units, int nhg, uint8_t *__restrict__ stage,
                                         uint8_t *__restrict__ work, float *__restrict__ xch,
                                         uint32_t *__restrict__ qrl_lds) {
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

    // ---- page copy HBM -> staging image: wave w issues wave-wide copies w, w + 8, ...;
    // lane l of copy k moves chunk 64 k + l
    auto fetch = [&](int pi) {
        const int page = load_const(a.bt, (int64_t)s * a.bt_stride + pi);
        const int64_t blk = (int64_t)page * a.Hkv + hk;
        const uint8_t *gcodes = a.kcodes + blk * (XT * XD / 2);
        const uint8_t *grope = reinterpret_cast<const uint8_t *>(a.krope + blk * (XT * XR));
        const uint8_t *gsz = reinterpret_cast<const uint8_t *>(a.ksz + blk * (XT * 2));
        const uint8_t *gcn = reinterpret_cast<const uint8_t *>(a.kcn + blk * XD);
        for (int k = wave; k < NDMA; k += 8) {
            const int c = 64 * k + lane;
            const uint8_t *src = c < 2048 ? gcodes + 16 * c
                               : c < 3072 ? grope + 16 * (c - 2048)
                               : c < 3104 ? gsz + 16 * (c - 3072)
                                          : gcn + 16 * (c - 3104);
            if (c < NCHUNK)
                __builtin_amdgcn_global_load_lds((const void *)src, (__attribute__((address_space(3))) void *)(stage + 1024 * k),
                                                 16, 0, 0);
        }
    };
    auto page_ok = [&](int pi) {
        const int page = load_const(a.bt, (int64_t)s * a.bt_stride + pi);
        return page >= 0 && page < a.num_pages;
    };
    int pi = p0;
    while (pi < p1 && !page_ok(pi)) ++pi;
    if (pi < p1) fetch(pi);

    // ---- rotated query of the lane's head over all 512 channels (c = 32 st + 8 lq + e);
    // the wave keeps its half: qv[st'][e] = qbar[256 half + 32 st' + 8 lq + e] / sqrt(512)
    float qv[8][8];
    uint32_t *qr = qrl_lds + wave * 8 * 64 + lane;  // rope dims 32 half + 8 lq + 0..7: bf16 hi words 0..3, lo 4..7
    float qmax = 0.f;
    {
        const int64_t qb = ((int64_t)s * a.Hq + hq) * (XD + XR);
        float q[16][8];
#pragma unroll
        for (int st = 0; st < 16; ++st)
#pragma unroll
            for (int e = 0; e < 8; ++e) q[st][e] = hq_ok ? load_q<QDT>(a.q, qb + 32 * st + 8 * lq + e) : 0.f;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            uint32_t hw = 0, lw = 0;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float x = hq_ok ? load_q<QDT>(a.q, qb + XD + 32 * half + 8 * lq + 2 * e2 + h) : 0.f;
                const uint16_t hb = bf16_rn(x);
                const uint16_t lb = bf16_rn(x - bf16_bits_to_float(hb));
                hw |= (uint32_t)hb << (16 * h);
                lw |= (uint32_t)lb << (16 * h);
            }
            qr[e2 * 64] = hw;
            qr[(4 + e2) * 64] = lw;
        }
        // Walsh-Hadamard transform: bits of e and st in registers, bits of lq
        // across lanes (lane bits 4 and 5)
#pragma unroll
        for (int b = 1; b < 8; b <<= 1)
#pragma unroll
            for (int st = 0; st < 16; ++st)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (!(e & b)) {
                        const float x = q[st][e], y = q[st][e | b];
                        q[st][e] = x + y;
                        q[st][e | b] = x - y;
                    }
#pragma unroll
        for (int b = 1; b < 16; b <<= 1)
#pragma unroll
            for (int st = 0; st < 16; ++st)
                if (!(st & b))
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float x = q[st][e], y = q[st | b][e];
                        q[st][e] = x + y;
                        q[st | b][e] = x - y;
                    }
        const float s16 = (lq & 1) ? -1.f : 1.f, s32 = (lq & 2) ? -1.f : 1.f;
        constexpr float INV_SQRT = 0.04419417382415922f;  // 1 / sqrt(512)
#pragma unroll
        for (int st = 0; st < 16; ++st)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float v = q[st][e], lo, hi;
                pair16(v, lo, hi);
                v = __builtin_fmaf(s16, hi, lo);
                pair32(v, lo, hi);
                v = __builtin_fmaf(s32, hi, lo);
                v *= INV_SQRT;
                qmax = fmaxf(qmax, fabsf(v));
                q[st][e] = v;
            }
#pragma unroll
        for (int st = 0; st < 8; ++st)
#pragma unroll
            for (int e = 0; e < 8; ++e) qv[st][e] = half ? q[st + 8][e] : q[st][e];
    }
    qmax = lq_max(qmax);

    const float sml2 = a.sm * 1.4426950408889634f;  // scores in log2 units
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[16];
#pragma unroll
    for (int mc = 0; mc < 16; ++mc) o[mc] = f32x4{0.f, 0.f, 0.f, 0.f};
    float *xp = xch + hs * XCH_WORDS;  // this pair's exchange slot
    const uint16_t *cn = reinterpret_cast<const uint16_t *>(work + L_CN);

    while (pi < p1) {
        const int cur = pi;
        __builtin_amdgcn_s_waitcnt(0);  // this wave's copies into the staging image have landed
        lds_barrier();                  // every wave's, and every wave is done with the working image
        // staging -> working image, swizzled
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const int c = tid + XNT * k;
            if (c < NCHUNK) {
                int off;
                if (c < 2048) {
                    const int r = c >> 4, g = c & 15;
                    off = L_CODES + r * 256 + 16 * (g ^ swz(r));
                } else if (c < 3072) {
                    const int r = (c - 2048) >> 3, g = (c - 2048) & 7;
                    off = L_ROPE + r * 128 + 16 * (g ^ rswz(r));
                } else {
                    off = L_SZ + 16 * (c - 3072);  // (S, Z) then normalizer, contiguous
                }
                *reinterpret_cast<uint4 *>(work + off) = *reinterpret_cast<const uint4 *>(stage + 16 * c);
            }
        }
        lds_barrier();  // working image complete, staging image free
        const int rows = min(XT, L - cur * XT);
        // Per-lane byte addresses of the code rows this lane reads, made opaque here
        // so that the per-K-step addresses below are formed next to their reads
        // rather than hoisted out of the page loop (64 live registers otherwise).
        // Score tile j reads row r = 64 pi2 + 16 q + 4 b + i: address r * 256 + 4 lq,
        // XOR 16 (chunk ^ swz(r)); the transposed reads use rows 64 pi2 + 16 lq + l16.
        int lo = lane;  // the lane id, opaque: addresses derived from it stay inside the loop
        asm volatile("" : "+v"(lo));
        const int ol16 = lo & 15, olq = lo >> 4;
        // rows 64 apart share the swizzle, so the second half of the page is a
        // constant 16 KB further (an immediate offset of the read)
        int sbase[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int r = 16 * (ol16 >> 2) + 4 * b + (ol16 & 3);
            sbase[b] = L_CODES + r * 256 + 16 * swz(r) + 4 * olq;
        }
        const int tr0 = 16 * olq + ol16;
        const int tbase = L_CODES + tr0 * 256 + 16 * swz(tr0);

        // page-wide bound of the query-side scaling: max c
        float cmax = 0.f;
        {
            const uint4 cw = *reinterpret_cast<const uint4 *>(work + L_CN + 16 * lane);
            const uint32_t w4[4] = {cw.x, cw.y, cw.z, cw.w};
            cmax = max_x4rows(row_max16(max_h8(w4)));  // all 64 lanes (normalizers are > 0)
        }
        const float qsc = pow2_scale(qmax * cmax);
        const float qinv = code_over(qsc);  // undoes the query scaling and the code unit
        // the next valid page, copied into the staging image while this one is processed
        ++pi;
        while (pi < p1 && !page_ok(pi)) ++pi;
        if (pi < p1) fetch(pi);

        // ---- partial scores^T over this wave's latent half: tile j = (pi2 = j >> 2, b = j & 3)
        // holds tokens 64 pi2 + 16 q + 4 b + i (row 4 q + i); A rows come from lane l16 = 4 q + i
        f32x4 sc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) sc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        float qc = 0.f;
        if (active) {
#pragma unroll
            for (int st = 0; st < 8; ++st) {
                const int chunk = 8 * half + st;  // 16-byte chunk of a code row: channels 32 chunk ..
                const uint4 cw = *reinterpret_cast<const uint4 *>(work + L_CN + 2 * (32 * chunk + 8 * lq));
                const uint32_t c4[4] = {cw.x, cw.y, cw.z, cw.w};
                half8 bh, bl;
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) {
                    const int e = (kk >> 1) + 4 * (kk & 1);
                    const half2v c2 = as_h2(c4[e >> 1]);
                    const float x = mul_h((e & 1) ? c2.y : c2.x, qv[st][e]);
                    qc += x;
                    _Float16 hi, lo;
                    split_prod(x, qsc, hi, lo);
                    bh[kk] = hi;
                    bl[kk] = lo;
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t w =
                        *reinterpret_cast<const uint32_t *>(work + (sbase[j & 3] ^ (16 * chunk)) + 16384 * (j >> 2));
                    const half8 av = unpack8_4(w);
                    sc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bh, sc[j], 0, 0, 0);
                    sc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bl, sc[j], 0, 0, 0);
                }
                // keep the next K-step's operands from being hoisted here (register pressure)
                __builtin_amdgcn_sched_barrier(0);
            }
            // rope half, then y = S qinv sc + rope
            const bf16x8 bh = __builtin_bit_cast(bf16x8, uint4{qr[0], qr[64], qr[128], qr[192]});
            const bf16x8 bl = __builtin_bit_cast(bf16x8, uint4{qr[256], qr[320], qr[384], qr[448]});
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int r = 64 * (j >> 2) + 16 * (ol16 >> 2) + 4 * (j & 3) + (ol16 & 3);
                const uint4 rw = *reinterpret_cast<const uint4 *>(work + L_ROPE + r * 128 + 16 * ((4 * half + olq) ^ rswz(r)));
                const bf16x8 av = __builtin_bit_cast(bf16x8, rw);
                f32x4 rp = {0.f, 0.f, 0.f, 0.f};
                rp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bh, rp, 0, 0, 0);
                rp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bl, rp, 0, 0, 0);
                const int t0 = 64 * (j >> 2) + 16 * olq + 4 * (j & 3);
                const uint4 zw = *reinterpret_cast<const uint4 *>(work + L_SZ + 4 * t0);
                const uint32_t z4[4] = {zw.x, zw.y, zw.z, zw.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) sc[j][i] = __builtin_fmaf((float)as_h2(z4[i]).x, qinv * sc[j][i], rp[i]);  // qinv: a power of two
            }
            // the low half publishes its partial sums
            if (half == 0) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) xp[(4 * j + i) * 64 + lane] = sc[j][i];
                xp[32 * 64 + lane] = qc;
            }
        }
        lds_barrier();
        if (active && half == 1) {  // the high half completes the sums and publishes them
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sc[j][i] += xp[(4 * j + i) * 64 + lane];
                    xp[(4 * j + i) * 64 + lane] = sc[j][i];
                }
            qc += xp[32 * 64 + lane];
            xp[32 * 64 + lane] = qc;
        }
        lds_barrier();
        if (!active) continue;
        if (half == 0) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) sc[j][i] = xp[(4 * j + i) * 64 + lane];
            qc = xp[32 * 64 + lane];
        }
        qc = lq_sum(qc);

        // ---- online softmax; lane (head l16, lq) holds tokens 64 pi2 + 16 lq + 4 b + i of tile (pi2, b)
        // scales are >= 0: their largest is the largest fp16 bit pattern (packed u16
        // maxima; the zero points in the upper halves are ignored)
        uint32_t smaxw = 0;
        float pmax = -INFINITY;
        const float a_z = sml2 * qc;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int t0 = 64 * (j >> 2) + 16 * olq + 4 * (j & 3);
            const uint4 zw = *reinterpret_cast<const uint4 *>(work + L_SZ + 4 * t0);
            const uint32_t z4[4] = {zw.x, zw.y, zw.z, zw.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                smaxw = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, smaxw),
                                                                               __builtin_bit_cast(u16x2, z4[i])));
                float x = __builtin_fmaf((float)as_h2(z4[i]).y, a_z, sml2 * sc[j][i]);
                if (t0 + i >= rows) x = -INFINITY;
                sc[j][i] = x;
                pmax = fmaxf(pmax, x);
            }
        }
        pmax = lq_max(pmax);
        const float smax = lq_max(half_bits_to_float(smaxw & 0x7fffu));
        const float m_new = fmaxf(m_run, pmax);
        const float alpha = exp2_fast(m_run - m_new);
        // the rescaling of o' runs only when some head's running maximum moved (most
        // pages once the first few are seen leave every alpha at exactly 1)
        const bool rescale = __builtin_amdgcn_ballot_w64(alpha != 1.f) != 0;
        m_run = m_new;
        const float psc = pow2_scale(smax), pinv = code_over(psc);
        // the scaling enters the exponent: ps = p psc = 2^(score - m + log2 psc), and the
        // sums over ps are scaled back once (powers of two: the same values as unscaled)
        const float m_ps = m_new - (float)((int)(__float_as_uint(psc) >> 23) - 127);
        const float pscinv = __uint_as_float((uint32_t)(254 - (int)(__float_as_uint(psc) >> 23)) << 23);
        float psum = 0.f, zs = 0.f;
        // P~ = p S psc straight into the B operand of the value product: K-step
        // kap = 2 pi2 + beta covers tokens 64 pi2 + 16 lq + 8 beta + e(kk); element
        // kk = 2 i + (j & 1) comes from tile j = 4 pi2 + 2 beta + (j & 1), row i
        half8 pbh[4], pbl[4];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int t0 = 64 * (j >> 2) + 16 * olq + 4 * (j & 3);
            const int kap = 2 * (j >> 2) + ((j >> 1) & 1);
            const uint4 zw = *reinterpret_cast<const uint4 *>(work + L_SZ + 4 * t0);
            const uint32_t z4[4] = {zw.x, zw.y, zw.z, zw.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const half2v sz = as_h2(z4[i]);  // (S, Z)
                const float ps = exp2_fast(sc[j][i] - m_ps);
                psum += ps;
                zs = __builtin_fmaf((float)sz.y, ps, zs);
                _Float16 hi, lo;
                split_prod(ps, (float)sz.x, hi, lo);
                pbh[kap][2 * i + (j & 1)] = hi;
                pbl[kap][2 * i + (j & 1)] = lo;
            }
        }
        l_run = __builtin_fmaf(l_run, alpha, psum * pscinv);
        zs = lq_sum(zs) * pscinv;

        if (rescale)
#pragma unroll
            for (int m2 = 0; m2 < 16; ++m2)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[m2][i] *= alpha;
        // ---- values^T over this wave's latent half: tile mc (channels 16 mc + l16 as A rows);
        // the transposed read gives lane (l16, lq) channel 16 mc + l16 of tokens 64 pi2 + 16 lq + 0..15
#pragma unroll
        for (int m2 = 0; m2 < 16; ++m2) {
            const int mc = 16 * half + m2;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p2 = 0; p2 < 2; ++p2) {
                const int off = (tbase ^ (16 * (mc >> 1))) + 16384 * p2 + 8 * (mc & 1);  // this lane's row of the group's read
                const v2i tw = __builtin_amdgcn_ds_read_tr4_b64_v2i32((__attribute__((address_space(3))) v2i *)(work + off));
#pragma unroll
                for (int beta = 0; beta < 2; ++beta) {
                    const half8 av = unpack8_4((uint32_t)tw[beta]);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pbh[2 * p2 + beta], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pbl[2 * p2 + beta], acc, 0, 0, 0);
                }
            }
            // fold (o' rescaled above): rows 4 lq + i of tile mc are channels 16 mc + 4 lq + i
            const uint2 cv2 = *reinterpret_cast<const uint2 *>(cn + 16 * mc + 4 * lq);
            const half2v c01 = as_h2(cv2.x), c23 = as_h2(cv2.y);
            const _Float16 cvv[4] = {c01.x, c01.y, c23.x, c23.y};
#pragma unroll
            for (int i = 0; i < 4; ++i) o[m2][i] = __builtin_fmaf((float)cvv[i], __builtin_fmaf(acc[i], pinv, zs), o[m2][i]);
            if (m2 & 1) __builtin_amdgcn_sched_barrier(0);  // at most two tiles' operands in flight
        }
    }

    // ---- split partial of the lane's head: o' (channels 16 mc + 4 lq + i of this half), m (natural log), l
    if (!hq_ok) return;
    l_run = lq_sum(l_run);
    // a partial row is XD + 2 = 514 floats: rows start 8-byte aligned only, so the stores are float2
    float *wsr = a.ws + (((int64_t)s * a.Hq + hq) * a.splits + split) * (XD + 2);
#pragma unroll
    for (int m2 = 0; m2 < 16; ++m2) {
        float2 *dst = reinterpret_cast<float2 *>(wsr + 16 * (16 * half + m2) + 4 * lq);
        dst[0] = float2{o[m2][0], o[m2][1]};
        dst[1] = float2{o[m2][2], o[m2][3]};
    }
    if (lq == 0 && half == 0) {
        wsr[XD] = m_run == -INFINITY ? -INFINITY : m_run * 0.6931471805599453f;
        wsr[XD + 1] = l_run;
    }
}

template <int QDT>
__global__ void __launch_bounds__(XNT, 1) decode_mla_kernel(DecodeArgs a, int units, int nhg) {
    // Separate LDS variables: each gets its own alias scope, which lets the
    // compiler keep the direct-to-LDS copies into `stage` in flight across the
    // accesses to the others.
    __shared__ __attribute__((aligned(16))) uint8_t stage[L_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t work[L_BYTES];
    __shared__ float xch[4 * XCH_WORDS];
    __shared__ uint32_t qr[8 * 8 * 64];
    mla_body<QDT>(a, units, nhg, stage, work, xch, qr);
}

bool decode_mla_supported(const DecodeArgs &a) {
    auto al16 = [](const void *p) { return ((uintptr_t)p & 15) == 0; };
    return al16(a.kcodes) && al16(a.ksz) && al16(a.kcn) && al16(a.krope) && a.D == XD && a.R == XR && a.Dv == XD && a.T == XT && a.kbits == 4 && a.kG == XD && a.kh == XD &&
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
