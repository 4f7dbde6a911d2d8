// Tile quantizer for 512-channel tiles of 128 tokens (the MLA latent: Hadamard
// block 512, one scale group per token, optional bf16 rope part copied through),
// gfx950. Same method and results as the other quantizer kernels.
//
// Workgroup = 8 waves, one (tile, head) item at a time, persistent. Lane l of wave
// w loads the 32 consecutive channels 32 (l & 15) .. + 31 of the four rows
// 4 rg .. + 3, rg = 4 w + (l >> 4). The 16 lanes of a DPP row cover one token's
// 512 channels: five Hadamard stages run in registers, four across lanes (after
// which the lane holds rotated channel group hperm16(l & 15)), and every
// per-token reduction is a row operation. Column partials are reduced over
// the four row groups of a wave by permlane swaps and over the 8 waves through
// LDS. The 128 values per lane leave no room for their squares, which are
// recomputed in every round. Codes of a row leave as one 16-byte store per lane.
// The next item's latent rows travel HBM -> LDS by direct-to-LDS copies while the
// current item is processed.
//
// Method: "KVarN" project review, Key Features ("Variance-Normalized
// Quantization Pipeline", "MLA Model Support"): rotate, run row/column RMS
// normalization rounds, asymmetric round-to-nearest with fp16 scale, zero point
// and normalizer; the rope part is kept in bf16, unrotated.
#include "common.h"
#include "launch.h"
#include "xlane.h"

namespace kvq {

namespace {

constexpr int LD = 512;    // latent channels
constexpr int LT = 128;    // tokens per tile
constexpr int LNT = 512;   // 8 waves
constexpr int LPAD = 576;  // per-channel LDS arrays: 4 floats of padding after every 32 channels
static_assert(4 * LPAD == 2304, "row stride of the asm column-sum reads");
// native vector type for 16-byte LDS accesses: one access keeps its aliasing
// information, where a struct-typed one is split and merged back without it
typedef float f32x4 __attribute__((ext_vector_type(4)));

// LDS offset of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// A few LDS accesses are written in asm. The compiler's merged forms of them carry
// no aliasing information, so it would wait for the direct-to-LDS copies in flight
// (which fill only `stage`) before each; the asm forms are not taken as touching
// `stage`. Loads wait for their own results inside the block.
__device__ __forceinline__ void lds_store_f32(float *p, float v) {
    asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}

// p[0..7] = h[0..7] (p 16-byte aligned)
__device__ __forceinline__ void lds_store_8f32(float *p, const float *h) {
    const f32x4 lo = {h[0], h[1], h[2], h[3]}, hi = {h[4], h[5], h[6], h[7]};
    asm volatile("ds_write_b128 %0, %1\n\tds_write_b128 %0, %2 offset:16" ::"v"(lds_addr(p)), "v"(lo), "v"(hi) : "memory");
}

// sum of p[0], p[LPAD], ..., p[7 LPAD]
__device__ __forceinline__ float lds_sum8_stride(const float *p) {
    float r[8];
    asm volatile(
        "ds_read_b32 %0, %8\n\t"
        "ds_read_b32 %1, %8 offset:2304\n\t"
        "ds_read_b32 %2, %8 offset:4608\n\t"
        "ds_read_b32 %3, %8 offset:6912\n\t"
        "ds_read_b32 %4, %8 offset:9216\n\t"
        "ds_read_b32 %5, %8 offset:11520\n\t"
        "ds_read_b32 %6, %8 offset:13824\n\t"
        "ds_read_b32 %7, %8 offset:16128\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(lds_addr(p))
        : "memory");
    float acc = 0.f;
#pragma unroll
    for (int v = 0; v < 8; ++v) acc += r[v];
    return acc;
}

// padded index of channel ch: the 16 lanes reading 32 consecutive channels each
// then hit 16 different bank groups
__device__ __forceinline__ int pch(int ch) { return ch + ((ch >> 5) << 2); }

// 16-byte slot of a staged row that holds chunk g of the row (an involution):
// a lane's four consecutive chunks, read by the 16 lanes of a DPP row, fall in
// 16 different bank groups.
__device__ __forceinline__ int slot(int g) { return g ^ ((g >> 4) & 3); }

}  // namespace

// The LDS buffers come in as restrict pointers to separate variables: after
// inlining, the compiler knows that no access to the others touches `stage` and
// keeps the direct-to-LDS copies into it in flight across them.
template <int BITS, int NIT>
__device__ __forceinline__ void quantize_d512_body(const QuantArgs &a, int num_items, uint8_t *__restrict__ stage,
                                                   float (*__restrict__ colsum)[LPAD], float *__restrict__ wsh0,
                                                   float *__restrict__ wsh1, float *__restrict__ multsh) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cc = lane & 15, rr = lane >> 4;
    const int rg = 4 * wave + rr;
    constexpr float LEVELS = (float)((1 << BITS) - 1);
    constexpr float TINY = 1e-30f;
    constexpr float INV_SQRT_H = 0.04419417382415922f;  // 1 / sqrt(512)
    const int iters = NIT >= 0 ? NIT : a.iters;
    const int pcc = hperm16(cc);      // rotated channel group held after the lane stages
    const float sigma = hsign16(cc);  // and its sign
    const int W = LD + a.R;  // source channels per token

    // rows 16 w .. 16 w + 15 of item itm: one wave-wide copy (1 KB) per row,
    // lane l -> slot l <- chunk slot(l)
    auto fetch = [&](int itm) {
        const int tl = itm / a.H, hd = itm % a.H;
        const int nv = load_const(a.tile_valid, tl);
        const char *src = reinterpret_cast<const char *>(a.src) +
                          2 * (hd * a.stride_head + (int64_t)load_const(a.tile_src_token, tl) * a.stride_token);
        const uint32_t loff = 16u * (uint32_t)slot(lane);
        if (nv <= 0) return;
#pragma unroll
        for (int i = 0; i < 16; ++i) {  // rows past the valid ones repeat the last valid row (never read)
            const int row = 16 * wave + i, srow = min(row, nv - 1);
            __builtin_amdgcn_global_load_lds((const void *)(src + (int64_t)srow * a.stride_token * 2 + loff),
                                             (__attribute__((address_space(3))) void *)(stage + 1024 * row), 16, 0, 0);
        }
    };
    int item = blockIdx.x;
    if (item < num_items) fetch(item);
    for (; item < num_items; item += gridDim.x) {
        const int tile = item / a.H, head = item % a.H;
        const int dst_page = load_const(a.tile_dst_page, tile);
        const int n = load_const(a.tile_valid, tile);
        const int64_t tok0 = load_const(a.tile_src_token, tile);
        const int64_t blk = (int64_t)dst_page * a.H + head;
        __builtin_amdgcn_s_waitcnt(0);  // this wave's copies have landed
        lds_barrier();                  // and every other wave's
        float y[4][32];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int row = 4 * rg + k;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 v = row < n ? *reinterpret_cast<const uint4 *>(stage + 1024 * row + 16 * slot(4 * cc + i))
                                        : uint4{0, 0, 0, 0};
                const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int h = 0; h < 4; ++h) bf16_pair_butterfly(w4[h], y[k][8 * i + 2 * h], y[k][8 * i + 2 * h + 1]);
            }
        }
        // rope part (bf16, copied unrotated): two 16-byte chunks per thread, loaded now, stored at the end
        uint4 rp[2] = {uint4{0, 0, 0, 0}, uint4{0, 0, 0, 0}};
        uint32_t bad = 0;
        if (a.R == 64 && n > 0) {
            int ot = tid;  // opaque: the addresses are formed here, not kept across the item
            asm volatile("" : "+v"(ot));
#pragma unroll
            for (int m = 0; m < 2; ++m) {  // branch-free: padding rows read the last valid row, zeroed below
                const int q = ot + LNT * m, row = min(q >> 3, n - 1), part = q & 7;
                rp[m] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(a.src) + head * a.stride_head +
                                                         (tok0 + row) * a.stride_token + LD + 8 * part);
            }
        }
        lds_barrier();  // the staging buffer is free again
        if (item + (int)gridDim.x < num_items) fetch(item + gridDim.x);
        if (dst_page < 0 || dst_page >= a.num_pages) continue;  // invalid destination: tile skipped (uniform)

        // ---- unnormalized Walsh-Hadamard transform along the 512 channels: bit 0
        // straight from the packed source pairs (above), bits 1..4 in registers, bits
        // 5..8 across lanes (DPP-fused multiply-adds); afterwards the lane holds
        // sigma * Y of channels 32 pcc .. 32 pcc + 31
#pragma unroll
        for (int s = 2; s < 32; s <<= 1)
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int e = 0; e < 32; ++e)
                    if (!(e & s)) {
                        const float p = y[k][e], q = y[k][e | s];
                        y[k][e] = p + q;
                        y[k][e | s] = p - q;
                    }
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int e = 0; e < 32; e += 8) hadamard16_lanes(&y[k][e], cc);

        // ---- normalization rounds on A = Y^2 (recomputed): u = 1/r^2 per row, w = 1/c^2 per channel
        if (iters == 0) {
            float ssq = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int e = 0; e < 32; ++e) ssq = __builtin_fmaf(y[k][e], y[k][e], ssq);
            if (!isfinite(ssq)) bad |= KVQ_FLAG_NONFINITE;
        }
        // w holds 1 / c^2 before the first round and 1 / (512 c^2) after it (the mean over
        // the 512 channels folded in: powers of two, so the row sums and u = 1 / r^2 are
        // the same bits as with the plain mean)
        float u[4];
        const float fn = (float)n, fn_d = fn * (1.0f / LD);
        constexpr float HUGE_F = 3.4028234663852886e38f;
        float t_own = 0.f;  // column sum of channel tid (last round)
#pragma unroll
        for (int it = 0; it < iters; ++it) {
            // row step: r^2 = mean_j A_ij / c_j^2, the lane's w read four at a time (w = 1 before the first round)
            float sk[4] = {0.f, 0.f, 0.f, 0.f};
            const float *wprev = (it & 1) ? wsh0 : wsh1;  // written by the previous round
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const f32x4 q = it == 0 ? f32x4{1.f, 1.f, 1.f, 1.f}
                                        : *reinterpret_cast<const f32x4 *>(&wprev[pch(32 * pcc) + 4 * i]);
                const float w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int h = 0; h < 4; ++h) sk[k] = __builtin_fmaf(y[k][4 * i + h] * w4[h], y[k][4 * i + h], sk[k]);
            }
            row_sum16_x4(sk);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (it == 0 && !isfinite(sk[k])) bad |= KVQ_FLAG_NONFINITE;
                // max(s, tiny) as a median with the largest float: one instruction (fmaxf
                // would first quiet the value the DPP asm produced); a NaN sum is flagged
                u[k] = it == 0 ? (float)LD * __builtin_amdgcn_rcpf(__builtin_amdgcn_fmed3f(sk[k], TINY, HUGE_F))
                               : __builtin_amdgcn_rcpf(__builtin_amdgcn_fmed3f(sk[k], TINY * (1.0f / LD), HUGE_F));
            }
            float t[32];
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                float acc = 0.f;
#pragma unroll
                for (int k = 0; k < 4; ++k) acc = __builtin_fmaf(y[k][e] * u[k], y[k][e], acc);
                t[e] = acc;
            }
            // across the four row groups of the wave: lane (cc, rr) ends with channels 32 pcc + 8 rr + j
            float h16[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(t[j]), __float_as_uint(t[j + 16]), false, false);
                h16[j] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            }
            float h8[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(h16[j]), __float_as_uint(h16[j + 8]), false, false);
                h8[j] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            }
            lds_store_8f32(&colsum[wave][pch(32 * pcc + 8 * rr)], h8);
            lds_barrier();
            float *wsh = (it & 1) ? wsh1 : wsh0;
            {
                const int pc = pch(tid);
                t_own = lds_sum8_stride(&colsum[0][pc]);
                // a zero column keeps a large finite w (its A entries are all zero); the
                // last round's sums go straight to the normalizer below (no w)
                if (it + 1 < iters) lds_store_f32(&wsh[pc], fn_d * __builtin_amdgcn_rcpf(fmaxf(t_own, TINY)));
            }
            if (it + 1 < iters) lds_barrier();  // w of this round visible to every lane
        }

        // ---- fp16 normalizer c16 (thread tid owns channel tid) and the multiplier
        // sigma / (sqrt(512) c16); a column whose sum of squares is 0 or not finite keeps c = 1
        {
            const float csq = (iters > 0 && n > 0 && t_own > 0.f && t_own < INFINITY) ? t_own / fn : 1.f;
            const uint16_t c16 = float_to_half_bits(sqrtf(csq));
            const float cv = half_bits_to_float(c16);
            if (!(cv > 0.f && cv < INFINITY)) bad |= KVQ_FLAG_SIDE_OVERFLOW;
            // reciprocal, then one Newton correction of the quotient (Markstein): within an
            // ulp of the rounded quotient
            const float rc = __builtin_amdgcn_rcpf(cv), q0 = INV_SQRT_H * rc;
            lds_store_f32(&multsh[pch(tid)], __builtin_fmaf(__builtin_fmaf(-cv, q0, INV_SQRT_H), rc, q0));
            a.cnorm[blk * LD + tid] = c16;
        }
        lds_barrier();
        // y <- y * multiplier (read four at a time)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const f32x4 q = *reinterpret_cast<const f32x4 *>(&multsh[pch(32 * pcc) + 4 * i]);
            const float m4[4] = {q.x * sigma, q.y * sigma, q.z * sigma, q.w * sigma};
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int h = 0; h < 4; ++h) y[k][4 * i + h] *= m4[h];
        }

        // ---- per token: asymmetric RTN with fp16 (S, Z); 32 codes per lane and row
        uint8_t *codes = a.codes + blk * (LT * LD * BITS / 8);
        float mnr[4], mxr[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float mn = y[k][0], mx = y[k][0];
#pragma unroll
            for (int e = 1; e < 32; ++e) {
                mn = fminf(mn, y[k][e]);
                mx = fmaxf(mx, y[k][e]);
            }
            mnr[k] = mn;
            mxr[k] = mx;
        }
        row_minmax16_x4(mnr, mxr);
        // per token: lane cc = k of each row group computes (S16, Z16) of its row 4 rg + k
        // (k < 4) and writes them; the rows' 1 / S and -Z / S return to the 16 lanes by
        // broadcasts (the other lanes' results are not used)
        float inv4[4], zi4[4];
        bool clamp;
        {
            const float mn = cc == 0 ? mnr[0] : cc == 1 ? mnr[1] : cc == 2 ? mnr[2] : mnr[3];
            const float mx = cc == 0 ? mxr[0] : cc == 1 ? mxr[1] : cc == 2 ? mxr[2] : mxr[3];
            const int row = 4 * rg + (cc & 3);
            const bool own = cc < 4;
            uint16_t S16 = 0, Z16 = 0;
            if (row < n) {
                S16 = float_to_half_bits((mx - mn) * (1.0f / LEVELS));
                Z16 = float_to_half_bits(mn);
            }
            const float Sv = half_bits_to_float(S16), Zv = half_bits_to_float(Z16);
            if (own && (!(Sv < INFINITY) || !(fabsf(Zv) < INFINITY))) bad |= KVQ_FLAG_SIDE_OVERFLOW;
            const float inv = Sv != 0.f ? __builtin_amdgcn_rcpf(Sv) : 0.f;
            const float zi = -Zv * inv;
            if (own) reinterpret_cast<uint32_t *>(a.sz)[blk * LT + row] = (uint32_t)S16 | ((uint32_t)Z16 << 16);
            // (y - Z) / S; v_cvt_pk_u8_f32 rounds to nearest even and clamps below at 0.
            // The upper clamp changes a code only for a value at or above LEVELS + 1/2, and
            // the map is monotone (inv >= 0), so only when a row's largest value gets there
            // (fp16 rounding of S and Z far larger than usual, or a non-finite value): the
            // packing runs in one of two copies, with and without it, chosen for the whole
            // wave (the clamp leaves every other code as it is)
            clamp = __ballot(bad != 0 || (own && !(__builtin_fmaf(mx, inv, zi) < LEVELS + 0.5f))) != 0;
            inv4[0] = row_bcast<0>(inv), zi4[0] = row_bcast<0>(zi);
            inv4[1] = row_bcast<1>(inv), zi4[1] = row_bcast<1>(zi);
            inv4[2] = row_bcast<2>(inv), zi4[2] = row_bcast<2>(zi);
            inv4[3] = row_bcast<3>(inv), zi4[3] = row_bcast<3>(zi);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int row = 4 * rg + k;
            const float inv = inv4[k], zi = zi4[k];
            auto pack_row = [&](auto clamp_c) {
                auto code = [&](float v) {
                    const float q = __builtin_fmaf(v, inv, zi);
                    return decltype(clamp_c)::value ? fminf(q, LEVELS) : q;
                };
                uint32_t word[BITS];
                if constexpr (BITS == 4) {
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        uint32_t ev = 0, od = 0;
#pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            ev = __builtin_amdgcn_cvt_pk_u8_f32(code(y[k][8 * d + 2 * b]), b, ev);
                            od = __builtin_amdgcn_cvt_pk_u8_f32(code(y[k][8 * d + 2 * b + 1]), b, od);
                        }
                        word[d] = ev | (od << 4);
                    }
                    *reinterpret_cast<uint4 *>(codes + row * (LD / 2) + 16 * pcc) = uint4{word[0], word[1], word[2], word[3]};
                } else {  // BITS == 2: 16 codes per word
#pragma unroll
                    for (int d = 0; d < 2; ++d) {
                        uint32_t q4[4] = {0, 0, 0, 0};
#pragma unroll
                        for (int b = 0; b < 4; ++b)
#pragma unroll
                            for (int m = 0; m < 4; ++m)
                                q4[m] = __builtin_amdgcn_cvt_pk_u8_f32(code(y[k][16 * d + 4 * b + m]), b, q4[m]);
                        word[d] = q4[0] | (q4[1] << 2) | (q4[2] << 4) | (q4[3] << 6);
                    }
                    *reinterpret_cast<uint2 *>(codes + row * (LD / 4) + 8 * pcc) = uint2{word[0], word[1]};
                }
            };
            if (clamp) pack_row(std::true_type{});
            else pack_row(std::false_type{});
        }
        if (a.R == 64) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int q = tid + LNT * m, row = q >> 3, part = q & 7;
                if (row >= n) rp[m] = uint4{0, 0, 0, 0};
                const uint32_t w4[4] = {rp[m].x, rp[m].y, rp[m].z, rp[m].w};
#pragma unroll
                for (int h = 0; h < 4; ++h)
                    if (((w4[h] & 0x7f80u) == 0x7f80u) || ((w4[h] & 0x7f800000u) == 0x7f800000u)) bad |= KVQ_FLAG_NONFINITE;
                *reinterpret_cast<uint4 *>(a.rope + (blk * LT + row) * 64 + 8 * part) = rp[m];
            }
        }
        if (a.flags) {  // one atomic per wave that saw a condition
            const bool nf = __ballot((bad & KVQ_FLAG_NONFINITE) != 0) != 0;
            const bool so = __ballot((bad & KVQ_FLAG_SIDE_OVERFLOW) != 0) != 0;
            if (lane == 0 && (nf || so))
                atomicOr(a.flags, (nf ? (uint32_t)KVQ_FLAG_NONFINITE : 0u) | (so ? (uint32_t)KVQ_FLAG_SIDE_OVERFLOW : 0u));
        }
    }
}

template <int BITS, int NIT>
__global__ void __launch_bounds__(LNT) quantize_d512_kernel(QuantArgs a, int num_items) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[LT * LD * 2];  // 128 rows x 1 KB (bf16)
    __shared__ __attribute__((aligned(16))) float colsum[8][LPAD];
    __shared__ __attribute__((aligned(16))) float wsh0[LPAD], wsh1[LPAD];
    __shared__ __attribute__((aligned(16))) float multsh[LPAD];
    quantize_d512_body<BITS, NIT>(a, num_items, stage, colsum, wsh0, wsh1, multsh);
}

bool quantize_d512_supported(int D, int T, const QuantArgs &a) {
    auto al16 = [](const void *p) { return ((uintptr_t)p & 15) == 0; };
    return D == LD && T == LT && a.h == LD && a.G == LD && (a.R == 0 || a.R == 64) && a.dtype == KVQ_BF16 &&
           a.center == 0 &&
           (a.bits == 2 || a.bits == 4) && a.layout == KVQ_TOKEN_MAJOR && a.stride_token < (int64_t(1) << 40) &&
           al16(a.codes) && (a.R == 0 || al16(a.rope));
}

template <int BITS, int NIT>
static void d512_launch(int num_tiles, const QuantArgs &a, hipStream_t stream) {
    const int items = num_tiles * a.H;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    const int grid = items < cus ? items : cus;  // one workgroup per compute unit (LDS)
    hipLaunchKernelGGL((quantize_d512_kernel<BITS, NIT>), dim3(grid), dim3(LNT), 0, stream, a, items);
}

void launch_quantize_d512(int num_tiles, const QuantArgs &a, hipStream_t stream) {
    if (a.bits == 4) {
        if (a.iters == 4) d512_launch<4, 4>(num_tiles, a, stream);
        else d512_launch<4, -1>(num_tiles, a, stream);
    } else {
        if (a.iters == 4) d512_launch<2, 4>(num_tiles, a, stream);
        else d512_launch<2, -1>(num_tiles, a, stream);
    }
}

}  // namespace kvq
