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
//   score_t = sm * ( S_t * [A . q']_t + (Z_t + 8 S_t) * sum_j q'_j + <q_rope, k_rope_t> )
//   o'_j   += c_j * ( [A^T . P~]_j + sum_t p_t (Z_t + 8 S_t) ),  P~_t = p_t S_t
// with A the centred codes (code - 8), exact in fp16. Both products run as
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

namespace kvq {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

constexpr int XD = 512;    // latent channels
constexpr int XR = 64;     // rope channels
constexpr int XT = 128;    // tokens per page
constexpr int XNT = 512;   // threads per workgroup (8 waves)
constexpr int XHG = 64;    // query heads per workgroup

// LDS image of one page (bytes). Codes: token row r (256 B) holds its 16-byte
// chunk g at slot g ^ swz(r); rope: row r (128 B) holds chunk g at slot g ^ (r & 7);
// (S, Z) pairs and the normalizer in natural order.
constexpr int L_CODES = 0;
constexpr int L_ROPE = XT * XD / 2;             // 32768
constexpr int L_SZ = L_ROPE + XT * XR * 2;      // 49152
constexpr int L_CN = L_SZ + XT * 4;             // 49664
constexpr int L_BYTES = L_CN + XD * 2;          // 50688
constexpr int NCHUNK = L_BYTES / 16;            // 3168 16-byte chunks per page
constexpr int PRE = (NCHUNK + XNT - 1) / XNT;   // 7 per thread
// score exchange between the two waves of a pair: [wave][33][64] floats
constexpr int L_XCH = L_BYTES;
constexpr int XCH_WORDS = 33 * 64;
constexpr int L_TOTAL = L_XCH + 8 * XCH_WORDS * 4;  // 118272

// Slot swizzle of a code row: the 16 rows read together by either product land
// in 16 different 16-byte slots (rows 4b + i + 16 q of a score tile, and rows
// 16 lq + i of a transposed read).
__device__ __forceinline__ int swz(int r) { return (r & 15) ^ ((r >> 2) & 12); }

__device__ __forceinline__ half2v as_h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }

// Eight 4-bit codes of one dword -> half8 in MFMA element order kk, element kk
// holding nibble e(kk) = (kk >> 1) + 4 (kk & 1), centred by 8.
__device__ __forceinline__ half8 unpack8_4(uint32_t w) {
    constexpr uint32_t MAGIC = 0x64006400u;  // fp16 1024 in both halves
    const half2v bias = {(_Float16)1032.f, (_Float16)1032.f};
    half8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const half2v h = as_h2(((w >> (4 * i)) & 0x000F000Fu) | MAGIC) - bias;
        r[2 * i] = h[0];
        r[2 * i + 1] = h[1];
    }
    return r;
}

// 2^(14 - floor(log2 m)) for m > 0 (1 for m == 0 or not finite).
__device__ __forceinline__ float pow2_scale(float m) {
    const int e = (int)((__float_as_uint(m) >> 23) & 0xffu);
    if (e == 0 || e == 0xff) return 1.f;
    const int se = min(254, 268 - e);
    return __uint_as_float((uint32_t)se << 23);
}

__device__ __forceinline__ float lq_sum(float v) {  // over the 4 lanes sharing lane & 15
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}
__device__ __forceinline__ float lq_max(float v) {
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    v = fmaxf(v, __shfl_xor(v, 32, 64));
    return v;
}

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

template <int QDT>
__global__ void __launch_bounds__(XNT, 1) decode_mla_kernel(DecodeArgs a, int units, int nhg) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // L_TOTAL bytes

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

    // ---- page prefetch: thread t moves chunks t + 512 k of the page image
    uint4 pre[PRE];
    auto fetch = [&](int pi) {
        const int page = load_const(a.bt, (int64_t)s * a.bt_stride + pi);
        const int64_t blk = (int64_t)page * a.Hkv + hk;
        const uint4 *gcodes = reinterpret_cast<const uint4 *>(a.kcodes + blk * (XT * XD / 2));
        const uint4 *grope = reinterpret_cast<const uint4 *>(a.krope + blk * (XT * XR));
        const uint4 *gsz = reinterpret_cast<const uint4 *>(a.ksz + blk * (XT * 2));
        const uint4 *gcn = reinterpret_cast<const uint4 *>(a.kcn + blk * XD);
#pragma unroll
        for (int k = 0; k < PRE; ++k) {
            const int c = tid + XNT * k;
            if (c < 2048) pre[k] = gcodes[c];
            else if (c < 3072) pre[k] = grope[c - 2048];
            else if (c < 3104) pre[k] = gsz[c - 3072];
            else if (c < NCHUNK) pre[k] = gcn[c - 3104];
        }
    };
    auto stash = [&]() {  // registers -> LDS image, swizzled
#pragma unroll
        for (int k = 0; k < PRE; ++k) {
            const int c = tid + XNT * k;
            int off;
            if (c < 2048) {
                const int r = c >> 4, g = c & 15;
                off = L_CODES + r * 256 + 16 * (g ^ swz(r));
            } else if (c < 3072) {
                const int r = (c - 2048) >> 3, g = (c - 2048) & 7;
                off = L_ROPE + r * 128 + 16 * (g ^ (r & 7));
            } else {
                off = L_SZ + 16 * (c - 3072);  // (S, Z) then normalizer, contiguous
            }
            if (c < NCHUNK) *reinterpret_cast<uint4 *>(lds + off) = pre[k];
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
    uint32_t qrh[4], qrl[4];  // rope dims 32 half + 8 lq + 0..7 as bf16 hi / lo pairs
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
            qrh[e2] = hw;
            qrl[e2] = lw;
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
                float v = q[st][e];
                v = __builtin_fmaf(s16, v, __shfl_xor(v, 16, 64));
                v = __builtin_fmaf(s32, v, __shfl_xor(v, 32, 64));
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
    float *xmine = reinterpret_cast<float *>(lds + L_XCH) + wave * XCH_WORDS;
    const float *xpart = reinterpret_cast<const float *>(lds + L_XCH) + (wave ^ 4) * XCH_WORDS;

    while (pi < p1) {
        const int cur = pi;
        lds_barrier();  // every wave is done with the previous page image
        stash();
        lds_barrier();  // the page image is complete
        ++pi;
        while (pi < p1 && !page_ok(pi)) ++pi;
        if (pi < p1) fetch(pi);
        const int rows = min(XT, L - cur * XT);

        // page-wide bound of the query-side scaling: max c
        const uint16_t *cn = reinterpret_cast<const uint16_t *>(lds + L_CN);
        float cmax = 0.f;
        {
            const uint4 cw = *reinterpret_cast<const uint4 *>(lds + L_CN + 16 * lane);
            const uint32_t w4[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                cmax = fmaxf(cmax, fmaxf(fabsf(half_bits_to_float(w4[i] & 0xffffu)), fabsf(half_bits_to_float(w4[i] >> 16))));
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) cmax = fmaxf(cmax, __shfl_xor(cmax, m, 64));
        }
        const float qsc = pow2_scale(qmax * cmax);
        const float qinv = 1.0f / qsc;

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
                const uint4 cw = *reinterpret_cast<const uint4 *>(lds + L_CN + 2 * (32 * chunk + 8 * lq));
                const uint32_t c4[4] = {cw.x, cw.y, cw.z, cw.w};
                half8 bh, bl;
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) {
                    const int e = (kk >> 1) + 4 * (kk & 1);
                    const uint32_t w = c4[e >> 1];
                    const float x = qv[st][e] * half_bits_to_float((e & 1) ? (w >> 16) : (w & 0xffffu));
                    qc += x;
                    const float xs = x * qsc;
                    const _Float16 hi = (_Float16)xs;
                    bh[kk] = hi;
                    bl[kk] = (_Float16)(xs - (float)hi);
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int r = 64 * (j >> 2) + 16 * (l16 >> 2) + 4 * (j & 3) + (l16 & 3);
                    const uint32_t w =
                        *reinterpret_cast<const uint32_t *>(lds + L_CODES + r * 256 + 16 * (chunk ^ swz(r)) + 4 * lq);
                    const half8 av = unpack8_4(w);
                    sc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bh, sc[j], 0, 0, 0);
                    sc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bl, sc[j], 0, 0, 0);
                }
            }
            // rope half, then y = S qinv sc + rope, published for the partner wave
            const bf16x8 bh = __builtin_bit_cast(bf16x8, uint4{qrh[0], qrh[1], qrh[2], qrh[3]});
            const bf16x8 bl = __builtin_bit_cast(bf16x8, uint4{qrl[0], qrl[1], qrl[2], qrl[3]});
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int r = 64 * (j >> 2) + 16 * (l16 >> 2) + 4 * (j & 3) + (l16 & 3);
                const uint4 rw = *reinterpret_cast<const uint4 *>(lds + L_ROPE + r * 128 + 16 * ((4 * half + lq) ^ (r & 7)));
                const bf16x8 av = __builtin_bit_cast(bf16x8, rw);
                f32x4 rp = {0.f, 0.f, 0.f, 0.f};
                rp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bh, rp, 0, 0, 0);
                rp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bl, rp, 0, 0, 0);
                const int t0 = 64 * (j >> 2) + 16 * lq + 4 * (j & 3);
                const uint4 zw = *reinterpret_cast<const uint4 *>(lds + L_SZ + 4 * t0);
                const uint32_t z4[4] = {zw.x, zw.y, zw.z, zw.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float S = half_bits_to_float(z4[i] & 0xffffu);
                    sc[j][i] = __builtin_fmaf(S * qinv, sc[j][i], rp[i]);
                    xmine[(4 * j + i) * 64 + lane] = sc[j][i];
                }
            }
            xmine[32 * 64 + lane] = qc;
        }
        lds_barrier();  // partial scores of both halves published
        if (!active) continue;
        qc += xpart[32 * 64 + lane];
        qc = lq_sum(qc);

        // ---- online softmax; lane (head l16, lq) holds tokens 64 pi2 + 16 lq + 4 b + i of tile (pi2, b)
        float smax = 0.f, pmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int t0 = 64 * (j >> 2) + 16 * lq + 4 * (j & 3);
            const uint4 zw = *reinterpret_cast<const uint4 *>(lds + L_SZ + 4 * t0);
            const uint32_t z4[4] = {zw.x, zw.y, zw.z, zw.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float S = half_bits_to_float(z4[i] & 0xffffu), Z = half_bits_to_float(z4[i] >> 16);
                smax = fmaxf(smax, fabsf(S));
                const float y = sc[j][i] + xpart[(4 * j + i) * 64 + lane];
                float x = sml2 * __builtin_fmaf(__builtin_fmaf(8.f, S, Z), qc, y);
                if (t0 + i >= rows) x = -INFINITY;
                sc[j][i] = x;
                pmax = fmaxf(pmax, x);
            }
        }
        pmax = lq_max(pmax);
        smax = lq_max(smax);
        const float m_new = fmaxf(m_run, pmax);
        const float alpha = exp2f(m_run - m_new);
        m_run = m_new;
        const float psc = pow2_scale(smax), pinv = 1.0f / psc;
        float psum = 0.f, zs = 0.f;
        // P~ = p S psc straight into the B operand of the value product: K-step
        // kap = 2 pi2 + beta covers tokens 64 pi2 + 16 lq + 8 beta + e(kk); element
        // kk = 2 i + (j & 1) comes from tile j = 4 pi2 + 2 beta + (j & 1), row i
        half8 pbh[4], pbl[4];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int t0 = 64 * (j >> 2) + 16 * lq + 4 * (j & 3);
            const int kap = 2 * (j >> 2) + ((j >> 1) & 1);
            const uint4 zw = *reinterpret_cast<const uint4 *>(lds + L_SZ + 4 * t0);
            const uint32_t z4[4] = {zw.x, zw.y, zw.z, zw.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float S = half_bits_to_float(z4[i] & 0xffffu), Z = half_bits_to_float(z4[i] >> 16);
                const float p = exp2f(sc[j][i] - m_new);
                psum += p;
                zs = __builtin_fmaf(p, __builtin_fmaf(8.f, S, Z), zs);
                const float xs = p * S * psc;
                const _Float16 hi = (_Float16)xs;
                pbh[kap][2 * i + (j & 1)] = hi;
                pbl[kap][2 * i + (j & 1)] = (_Float16)(xs - (float)hi);
            }
        }
        l_run = __builtin_fmaf(l_run, alpha, psum);
        zs = lq_sum(zs);

        // ---- values^T over this wave's latent half: tile mc (channels 16 mc + l16 as A rows);
        // the transposed read gives lane (l16, lq) channel 16 mc + l16 of tokens 64 pi2 + 16 lq + 0..15
#pragma unroll
        for (int m2 = 0; m2 < 16; ++m2) {
            const int mc = 16 * half + m2;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p2 = 0; p2 < 2; ++p2) {
                const int r = 64 * p2 + 16 * lq + l16;  // row addressed by this lane for the group's read
                const int off = L_CODES + r * 256 + 16 * ((mc >> 1) ^ swz(r)) + 8 * (mc & 1);
                const v2i tw = __builtin_amdgcn_ds_read_tr4_b64_v2i32((__attribute__((address_space(3))) v2i *)(lds + off));
#pragma unroll
                for (int beta = 0; beta < 2; ++beta) {
                    const half8 av = unpack8_4((uint32_t)tw[beta]);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pbh[2 * p2 + beta], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pbl[2 * p2 + beta], acc, 0, 0, 0);
                }
            }
            // fold: rows 4 lq + i of tile mc are channels 16 mc + 4 lq + i
            const uint2 cv2 = *reinterpret_cast<const uint2 *>(cn + 16 * mc + 4 * lq);
            const float cvv[4] = {half_bits_to_float(cv2.x & 0xffffu), half_bits_to_float(cv2.x >> 16),
                                  half_bits_to_float(cv2.y & 0xffffu), half_bits_to_float(cv2.y >> 16)};
#pragma unroll
            for (int i = 0; i < 4; ++i) o[m2][i] = __builtin_fmaf(o[m2][i], alpha, cvv[i] * __builtin_fmaf(acc[i], pinv, zs));
        }
    }

    // ---- split partial of the lane's head: o' (channels 16 mc + 4 lq + i of this half), m (natural log), l
    if (!hq_ok) return;
    l_run = lq_sum(l_run);
    float *wsr = a.ws + (((int64_t)s * a.Hq + hq) * a.splits + split) * (XD + 2);
#pragma unroll
    for (int m2 = 0; m2 < 16; ++m2)
        *reinterpret_cast<float4 *>(wsr + 16 * (16 * half + m2) + 4 * lq) = float4{o[m2][0], o[m2][1], o[m2][2], o[m2][3]};
    if (lq == 0 && half == 0) {
        wsr[XD] = m_run == -INFINITY ? -INFINITY : m_run * 0.6931471805599453f;
        wsr[XD + 1] = l_run;
    }
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
        // the LDS image plus the score exchange exceed the default 64 KB
        if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, L_TOTAL) != hipSuccess)
            return false;
        hipLaunchKernelGGL(kern, dim3(grid), dim3(XNT), L_TOTAL, stream, a, units, nhg);
        return true;
    };
    switch (a.q_dtype) {
    case KVQ_F32: return go(decode_mla_kernel<KVQ_F32>);
    case KVQ_F16: return go(decode_mla_kernel<KVQ_F16>);
    default: return go(decode_mla_kernel<KVQ_BF16>);
    }
}

}  // namespace kvq
