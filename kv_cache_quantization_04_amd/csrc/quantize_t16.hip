// Tile quantizer for 16-token tiles of head_dim 128 (Hadamard block 128, one
// scale group per token), gfx950: one wave per (tile, head), no workgroup
// barriers. Same method and results as the other quantizer kernels.
//
// Lane l of a wave loads the 8 consecutive channels 8 (l & 15) .. + 7 of the four
// rows 4 (l >> 4) .. + 3. The 16 lanes of a DPP row cover one token's 128
// channels: Hadamard butterflies on channel bits 3..6 (after which the lane holds
// rotated channel group hperm16(l & 15)) and all per-token reductions are row
// operations. Column sums finish inside the wave (permlane
// swaps across the four row groups) and come back to the lanes through a small
// per-wave LDS array. Codes go to a per-wave LDS byte image in bitstream order
// (token-major t * 128 + j, channel-major j * 16 + t); each lane then packs 32
// consecutive codes into the little-endian bitstream, and the block leaves with
// one store per lane. The next tile is loaded into registers meanwhile.
//
// Method: "KVarN" project review, Key Features ("Variance-Normalized
// Quantization Pipeline"): rotate, run row/column RMS normalization rounds,
// asymmetric round-to-nearest with fp16 scale, zero point and normalizer.
#include "common.h"
#include "launch.h"
#include "xlane.h"

namespace kvq {

namespace {

constexpr int ZD = 128;   // head_dim
constexpr int ZT = 16;    // tokens per tile
constexpr int ZNT = 256;  // 4 waves, one tile each

struct Rows {
    uint4 v[4];  // four rows x 8 bf16 channels
};

// The lane's 4 rows x 8 channels of an item (rows >= nv read as zero).
__device__ __forceinline__ Rows load_rows(const QuantArgs &a, int item, int lane) {
    Rows r;
    const int tl = item / a.H, hd = item % a.H;
    const int nv = load_const(a.tile_valid, tl);
    const uint16_t *src = reinterpret_cast<const uint16_t *>(a.src) + hd * a.stride_head +
                          (int64_t)load_const(a.tile_src_token, tl) * a.stride_token + 8 * (lane & 15);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int row = 4 * (lane >> 4) + k;
        r.v[k] = row < nv ? *reinterpret_cast<const uint4 *>(src + (int64_t)row * a.stride_token) : uint4{0, 0, 0, 0};
    }
    return r;
}

}  // namespace

template <int BITS, int LAYOUT, int NIT>
__global__ void __launch_bounds__(ZNT, 4) quantize_t16_kernel(QuantArgs a, int num_items) {
    __shared__ float chv[4][ZD];                                // per wave: one value per channel
    __shared__ __attribute__((aligned(16))) uint8_t img[4][ZT * ZD];  // per wave: codes in stream order

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int cc = lane & 15, rr = lane >> 4;
    constexpr float LEVELS = (float)((1 << BITS) - 1);
    constexpr float TINY = 1e-30f;
    constexpr float INV_SQRT_H = 0.08838834764831845f;  // 1 / sqrt(128)
    const int iters = NIT >= 0 ? NIT : a.iters;
    // after the lane stages of the rotation the lane holds sigma * Y of channel
    // group pcc: channels 8 pcc .. 8 pcc + 7
    const int pcc = hperm16(cc);
    const float sigma = hsign16(cc);
    float *cv = chv[wave];
    uint8_t *im = img[wave];

    int item = blockIdx.x * 4 + wave;
    const int stride = gridDim.x * 4;
    Rows nxt{};
    if (item < num_items) nxt = load_rows(a, item, lane);
    for (; item < num_items; item += stride) {
        const int tile = item / a.H, head = item % a.H;
        const int dst_page = load_const(a.tile_dst_page, tile);
        const int n = load_const(a.tile_valid, tile);
        float y[4][8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t w4[4] = {nxt.v[k].x, nxt.v[k].y, nxt.v[k].z, nxt.v[k].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) bf16_pair_butterfly(w4[i], y[k][2 * i], y[k][2 * i + 1]);
        }
        if (item + stride < num_items) nxt = load_rows(a, item + stride, lane);  // travels meanwhile
        if (dst_page < 0 || dst_page >= a.num_pages) continue;  // invalid destination: tile skipped (uniform)
        const int64_t blk = (int64_t)dst_page * a.H + head;

        // ---- unnormalized Walsh-Hadamard transform along the 128 channels: bit 0
        // straight from the packed source pairs (above), bits 1..2 in registers, bits
        // 3..6 across lanes (DPP-fused multiply-adds)
#pragma unroll
        for (int s = 2; s < 8; s <<= 1)
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (!(j & s)) {
                        const float p = y[k][j], q = y[k][j | s];
                        y[k][j] = p + q;
                        y[k][j | s] = p - q;
                    }
#pragma unroll
        for (int k = 0; k < 4; ++k) hadamard16_lanes(y[k], cc);

        // ---- normalization rounds on A = Y^2: u = 1/r^2 per row, w = 1/c^2 per channel
        float A[4][8];
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int j = 0; j < 8; ++j) A[k][j] = y[k][j] * y[k][j];
        uint32_t bad = 0;
        if (iters == 0) {
            float ssq = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int j = 0; j < 8; ++j) ssq += A[k][j];
            if (!isfinite(ssq)) bad |= KVQ_FLAG_NONFINITE;
        }
        // w holds 1 / c^2 in the first round and 1 / (128 c^2) after it (the mean over
        // the 128 channels folded in: powers of two, so the row sums and u = 1 / r^2 are
        // the same bits as with the plain mean)
        float w[8], u[4];
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = 1.f;
        const float fn = (float)n, fn_d = fn * (1.0f / ZD);
        constexpr float HUGE_F = 3.4028234663852886e38f;
        float t_own[2] = {0.f, 0.f};  // column sums of channels 8 cc + 2 rr + {0, 1} (last round)
#pragma unroll
        for (int it = 0; it < iters; ++it) {
            // row step: r^2 = mean_j A_ij / c_j^2 over the 128 channels
            float rs[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) s = __builtin_fmaf(A[k][j], w[j], s);
                rs[k] = s;
            }
            row_sum16_x4(rs);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (it == 0 && !isfinite(rs[k])) bad |= KVQ_FLAG_NONFINITE;
                // max(s, tiny) as a median with the largest float: one instruction (fmaxf
                // would first quiet the value the DPP asm produced); a NaN sum is flagged
                u[k] = it == 0 ? (float)ZD * __builtin_amdgcn_rcpf(__builtin_amdgcn_fmed3f(rs[k], TINY, HUGE_F))
                               : __builtin_amdgcn_rcpf(__builtin_amdgcn_fmed3f(rs[k], TINY * (1.0f / ZD), HUGE_F));
            }
            // column step: c^2 = mean_i A_ij u_i over the n valid rows (padding rows are zero)
            float t[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float acc = 0.f;
#pragma unroll
                for (int k = 0; k < 4; ++k) acc = __builtin_fmaf(A[k][j], u[k], acc);
                t[j] = acc;
            }
            float h4[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(t[j]), __float_as_uint(t[j + 4]), false, false);
                h4[j] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);  // ch j (lanes < 32) / j + 4 (lanes >= 32)
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(h4[j]), __float_as_uint(h4[j + 2]), false, false);
                t_own[j] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);  // channel 8 pcc + 2 rr + j
            }
            // a zero column keeps a large finite w (its A entries are all zero)
            *reinterpret_cast<float2 *>(&cv[8 * pcc + 2 * rr]) =
                float2{fn_d * __builtin_amdgcn_rcpf(fmaxf(t_own[0], TINY)), fn_d * __builtin_amdgcn_rcpf(fmaxf(t_own[1], TINY))};
            const float4 w0 = *reinterpret_cast<const float4 *>(&cv[8 * pcc]);
            const float4 w1 = *reinterpret_cast<const float4 *>(&cv[8 * pcc + 4]);
            w[0] = w0.x; w[1] = w0.y; w[2] = w0.z; w[3] = w0.w;
            w[4] = w1.x; w[5] = w1.y; w[6] = w1.z; w[7] = w1.w;
        }

        // ---- fp16 normalizer c16 of the lane's two channels and the multiplier
        // sigma / (sqrt(128) c16); a column whose sum of squares is 0 or not finite keeps c = 1
        {
            uint32_t c2 = 0;
            float m2[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float tj = t_own[j];
                const float csq = (iters > 0 && n > 0 && tj > 0.f && tj < INFINITY) ? tj / fn : 1.f;
                const uint16_t c16 = float_to_half_bits(sqrtf(csq));
                const float cvj = half_bits_to_float(c16);
                if (!(cvj > 0.f && cvj < INFINITY)) bad |= KVQ_FLAG_SIDE_OVERFLOW;
                m2[j] = INV_SQRT_H / cvj;
                c2 |= (uint32_t)c16 << (16 * j);
            }
            *reinterpret_cast<uint32_t *>(a.cnorm + blk * ZD + 8 * pcc + 2 * rr) = c2;
            *reinterpret_cast<float2 *>(&cv[8 * pcc + 2 * rr]) = float2{m2[0], m2[1]};
        }
        float mult[8];
        {
            const float4 m0 = *reinterpret_cast<const float4 *>(&cv[8 * pcc]);
            const float4 m1 = *reinterpret_cast<const float4 *>(&cv[8 * pcc + 4]);
            mult[0] = m0.x * sigma; mult[1] = m0.y * sigma; mult[2] = m0.z * sigma; mult[3] = m0.w * sigma;
            mult[4] = m1.x * sigma; mult[5] = m1.y * sigma; mult[6] = m1.z * sigma; mult[7] = m1.w * sigma;
        }

        // ---- per token: asymmetric RTN with fp16 (S, Z); byte codes into the image
        uint32_t cm[8];  // channel-major: bytes of rows 4 rr .. + 3 of channel 8 cc + j
#pragma unroll
        for (int j = 0; j < 8; ++j) cm[j] = 0;
        // y -> y / c16 (scaled, signed), in place; row minima and maxima over the 128 channels
        float mnr[4], mxr[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
#pragma unroll
            for (int j = 0; j < 8; ++j) y[k][j] *= mult[j];
            float mn = y[k][0], mx = y[k][0];
#pragma unroll
            for (int j = 1; j < 8; ++j) {
                mn = fminf(mn, y[k][j]);
                mx = fmaxf(mx, y[k][j]);
            }
            mnr[k] = mn;
            mxr[k] = mx;
        }
        row_minmax16_x4(mnr, mxr);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int row = 4 * rr + k;
            const float mn = mnr[k], mx = mxr[k];
            uint16_t S16 = 0, Z16 = 0;
            if (row < n) {
                S16 = float_to_half_bits((mx - mn) * (1.0f / LEVELS));
                Z16 = float_to_half_bits(mn);
            }
            const float Sv = half_bits_to_float(S16), Zv = half_bits_to_float(Z16);
            if (!(Sv < INFINITY) || !(fabsf(Zv) < INFINITY)) bad |= KVQ_FLAG_SIDE_OVERFLOW;
            const float inv = Sv != 0.f ? __builtin_amdgcn_rcpf(Sv) : 0.f;
            const float zi = -Zv * inv;
            // (y - Z) / S; cvt_pk_u8 rounds to nearest even and clamps below at 0. The upper
            // clamp changes a code only for a value at or above LEVELS + 1/2, and the map
            // is monotone (inv >= 0), so only when the row's largest value gets there
            float q[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) q[j] = __builtin_fmaf(y[k][j], inv, zi);
            if (bad || !(__builtin_fmaf(mx, inv, zi) < LEVELS + 0.5f))
#pragma unroll
                for (int j = 0; j < 8; ++j) q[j] = fminf(q[j], LEVELS);
            if (cc == 0)
                reinterpret_cast<uint32_t *>(a.sz)[blk * ZT + row] = (uint32_t)S16 | ((uint32_t)Z16 << 16);
            if constexpr (LAYOUT == KVQ_TOKEN_MAJOR) {
                uint32_t lo = 0, hi = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    lo = __builtin_amdgcn_cvt_pk_u8_f32(q[b], b, lo);
                    hi = __builtin_amdgcn_cvt_pk_u8_f32(q[b + 4], b, hi);
                }
                *reinterpret_cast<uint2 *>(&im[row * ZD + 8 * pcc]) = uint2{lo, hi};
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) cm[j] = __builtin_amdgcn_cvt_pk_u8_f32(q[j], k, cm[j]);
            }
        }
        if constexpr (LAYOUT == KVQ_CHANNEL_MAJOR) {
#pragma unroll
            for (int j = 0; j < 8; ++j) *reinterpret_cast<uint32_t *>(&im[(8 * pcc + j) * ZT + 4 * rr]) = cm[j];
        }

        // ---- pack: lane l takes stream positions 32 l .. 32 l + 31 -> BITS words
        {
            const uint4 b0 = *reinterpret_cast<const uint4 *>(&im[32 * lane]);
            const uint4 b1 = *reinterpret_cast<const uint4 *>(&im[32 * lane + 16]);
            const uint32_t bw[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
            uint32_t out[BITS];
#pragma unroll
            for (int d = 0; d < BITS; ++d) out[d] = 0;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                const uint32_t c = (bw[i >> 2] >> (8 * (i & 3))) & 0xFFu;
                const int bit = BITS * i;
                out[bit >> 5] |= c << (bit & 31);
                if ((bit & 31) + BITS > 32) out[(bit >> 5) + 1] |= c >> (32 - (bit & 31));
            }
            uint32_t *dst = reinterpret_cast<uint32_t *>(a.codes + blk * (ZT * ZD * BITS / 8)) + BITS * lane;
            if constexpr (BITS == 4) *reinterpret_cast<uint4 *>(dst) = uint4{out[0], out[1], out[2], out[3]};
            else if constexpr (BITS == 2) *reinterpret_cast<uint2 *>(dst) = uint2{out[0], out[1]};
            else {
#pragma unroll
                for (int d = 0; d < BITS; ++d) dst[d] = out[d];
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

bool quantize_t16_supported(int D, int T, const QuantArgs &a) {
    return D == ZD && T == ZT && a.h == ZD && a.G == ZD && a.R == 0 && a.dtype == KVQ_BF16 && a.center == 0 &&
           (a.bits == 2 || a.bits == 3 || a.bits == 4) &&
           (a.layout == KVQ_TOKEN_MAJOR || a.layout == KVQ_CHANNEL_MAJOR) && a.stride_token < (int64_t(1) << 40) &&
           ((uintptr_t)a.codes & 15) == 0 && ((uintptr_t)a.cnorm & 3) == 0;
}

template <int BITS, int LAYOUT, int NIT>
static void t16_launch(int num_tiles, const QuantArgs &a, hipStream_t stream) {
    const int items = num_tiles * a.H;
    int dev = 0, cus = 256, per_cu = 1;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, quantize_t16_kernel<BITS, LAYOUT, NIT>, ZNT, 0) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    const int waves_needed = (items + 3) / 4;
    const int grid = waves_needed < cus * per_cu ? waves_needed : cus * per_cu;
    hipLaunchKernelGGL((quantize_t16_kernel<BITS, LAYOUT, NIT>), dim3(grid), dim3(ZNT), 0, stream, a, items);
}

template <int BITS, int LAYOUT>
static void t16_launch_n(int num_tiles, const QuantArgs &a, hipStream_t stream) {
    if (a.iters == 2) t16_launch<BITS, LAYOUT, 2>(num_tiles, a, stream);
    else if (a.iters == 4) t16_launch<BITS, LAYOUT, 4>(num_tiles, a, stream);
    else t16_launch<BITS, LAYOUT, -1>(num_tiles, a, stream);
}

template <int BITS>
static void t16_launch_l(int num_tiles, const QuantArgs &a, hipStream_t stream) {
    if (a.layout == KVQ_TOKEN_MAJOR) t16_launch_n<BITS, KVQ_TOKEN_MAJOR>(num_tiles, a, stream);
    else t16_launch_n<BITS, KVQ_CHANNEL_MAJOR>(num_tiles, a, stream);
}

void launch_quantize_t16(int num_tiles, const QuantArgs &a, hipStream_t stream) {
    if (a.bits == 2) t16_launch_l<2>(num_tiles, a, stream);
    else if (a.bits == 3) t16_launch_l<3>(num_tiles, a, stream);
    else t16_launch_l<4>(num_tiles, a, stream);
}

}  // namespace kvq
