// Tile quantizer for 16-token tiles of head_dim 128 (Hadamard block 128, one
// scale group per token), gfx950: one wave per (tile, head), no workgroup
// barriers. Same method and results as the other quantizer kernels.
//
// The 128-point rotation runs on the matrix cores (mfma_hadamard.h): lane l loads
// the bf16 source of token l & 15, channels 32 s + 8 (l >> 4) .. + 7 for s = 0..3,
// as the A operand, and receives the rotated rows 4 (l >> 4) .. + 3 at channels
// 16 j + (l & 15), j = 0..7. The 16 lanes of a DPP row thus cover one token's 128
// channels, and all per-token reductions are row operations. Column sums finish
// inside the wave (permlane swaps across the four row groups) and the per-channel
// factors go back to the four row groups through a small per-wave LDS buffer.
// Per-token scale and zero are computed by one lane per row and broadcast. Codes go
// to a per-wave LDS byte image in bitstream order (token-major t * 128 + j,
// channel-major j * 16 + t); each lane then packs 32 consecutive codes into the
// little-endian bitstream, and the block leaves with one store per lane. The next
// tile is loaded into registers meanwhile.
//
// Method: "KVarN" project review, Key Features ("Variance-Normalized
// Quantization Pipeline"): rotate, run row/column RMS normalization rounds,
// asymmetric round-to-nearest with fp16 scale, zero point and normalizer.
#include "common.h"
#include "launch.h"
#include "mfma_hadamard.h"
#include "xlane.h"

namespace kvq {

namespace {

constexpr int ZD = 128;   // head_dim
constexpr int ZT = 16;    // tokens per tile
constexpr int ZNT = 256;  // 4 waves, one tile each

struct Rows {
    uint4 v[4];  // token lane & 15: 8 bf16 channels 32 s + 8 (lane >> 4) .. + 7 for s = 0..3
};

// The lane's A operands of an item. The loads go through a buffer resource that
// covers the tile's nv valid rows only (nv row strides from its first row; a row
// stride is at least 128 channels), so a row >= nv falls outside it and reads as zero
// without a branch.
__device__ __forceinline__ Rows load_rows(const QuantArgs &a, int item, int lane) {
    Rows r;
    const int tl = item / a.H, hd = item % a.H;
    const int nv = load_const(a.tile_valid, tl);
    const uint16_t *base = reinterpret_cast<const uint16_t *>(a.src) + hd * a.stride_head +
                           (int64_t)load_const(a.tile_src_token, tl) * a.stride_token;
    const int rec = (int)(nv * a.stride_token * 2);  // bytes; < 2^31 (checked at launch)
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base), (short)0, rec,
                                                                        BUF_DWORD3);
    const int off = (int)((lane & 15) * a.stride_token * 2) + 16 * (lane >> 4);
#pragma unroll
    for (int s = 0; s < 4; ++s) r.v[s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 64 * s, 0, 0));
    return r;
}

// The values of the lane's 8 local channels (t = 0..7, channel 16 t + (lane & 15)) from
// their owners: after the column-sum swaps, lane (cc, rr) holds local channels 2 rr and
// 2 rr + 1 (o0, o1).
// Through the wave's own 512-byte LDS buffer: lane (cc, rr) writes its pair to row cc,
// slots 2 rr, 2 rr + 1, and reads row cc back (a wave's LDS operations run in order, so
// no barrier is needed). The permlane swaps would do it in registers, but a swap of a
// value with itself first needs a register copy: 12 VALU instructions against none.
__device__ __forceinline__ void bcast_owned(float o0, float o1, float (&v)[8], float *buf, int cc, int rr) {
    *reinterpret_cast<float2 *>(&buf[8 * cc + 2 * rr]) = float2{o0, o1};
    const float4 lo = *reinterpret_cast<const float4 *>(&buf[8 * cc]);
    const float4 hi = *reinterpret_cast<const float4 *>(&buf[8 * cc + 4]);
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
}

}  // namespace

template <int BITS, int LAYOUT, int NIT>
__global__ void __launch_bounds__(ZNT, 4) quantize_t16_kernel(QuantArgs a, int num_items) {
    __shared__ __attribute__((aligned(16))) uint8_t img[4][ZT * ZD];  // per wave: codes in stream order
    __shared__ uint4 hbtab[2 * 64];  // the two per-lane Hadamard operand patterns, read per item
    __shared__ __attribute__((aligned(16))) float bcb[4][16 * 8];  // per wave: channel factors, row cc = lane & 15

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    constexpr float LEVELS = (float)((1 << BITS) - 1);
    constexpr float TINY = 1e-30f;
    constexpr float INV_SQRT_H = 0.08838834764831845f;  // 1 / sqrt(128)
    const int iters = NIT >= 0 ? NIT : a.iters;
    if (threadIdx.x < 64) {
        const Had128B hb = had128_operands(lane);
        hbtab[lane] = hb.p0;
        hbtab[64 + lane] = hb.p1;
    }
    __syncthreads();
    uint8_t *im = img[wave];

    int item = blockIdx.x * 4 + wave;
    const int stride = gridDim.x * 4;
    Rows nxt{};
    if (item < num_items) nxt = load_rows(a, item, lane);
    for (; item < num_items; item += stride) {
        // lane id made opaque: the LDS and global addresses derived from it are formed
        // inside the item, not hoisted out of the loop (held across it they spill, and a
        // spill reload waits for the next item's loads in flight)
        int ol = lane;
        asm volatile("" : "+v"(ol));
        // after the rotation the lane holds channels 16 j + cc, j = 0..7, of rows 4 rr + k
        const int cc = ol & 15, rr = ol >> 4;
        const int tile = item / a.H, head = item % a.H;
        const int dst_page = load_const(a.tile_dst_page, tile);
        const int n = load_const(a.tile_valid, tile);
        // ---- unnormalized Walsh-Hadamard transform along the 128 channels (matrix cores)
        float y[4][8];
        {
            f32x4 xr[8];
            const Had128B hb{hbtab[ol], hbtab[64 + ol]};  // held across the loop, the patterns spill
            had128_rows16(nxt.v, hb, xr);
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int j = 0; j < 8; ++j) y[k][j] = xr[j][k];
        }
        if (item + stride < num_items) nxt = load_rows(a, item + stride, lane);  // travels meanwhile
        if (dst_page < 0 || dst_page >= a.num_pages) continue;  // invalid destination: tile skipped (uniform)
        const int64_t blk = (int64_t)dst_page * a.H + head;

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
        float t_own[2] = {0.f, 0.f};  // column sums of channels 16 (2 rr + {0, 1}) + cc (last round)
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
                t_own[j] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);  // channel 16 (2 rr + j) + cc
            }
            // a zero column keeps a large finite w (its A entries are all zero)
            bcast_owned(fn_d * __builtin_amdgcn_rcpf(fmaxf(t_own[0], TINY)),
                        fn_d * __builtin_amdgcn_rcpf(fmaxf(t_own[1], TINY)), w, bcb[wave], cc, rr);
        }

        // ---- fp16 normalizer c16 of the lane's two channels and the multiplier
        // 1 / (sqrt(128) c16); a column whose sum of squares is 0 or not finite keeps c = 1
        float mult[8];
        {
            float m2[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float tj = t_own[j];
                // mean over the n valid rows by a reciprocal of n (exact for a full tile,
                // n = 16; within an ulp of the quotient otherwise)
                const float csq = (iters > 0 && n > 0 && tj > 0.f && tj < INFINITY) ? tj * __builtin_amdgcn_rcpf(fn) : 1.f;
                const uint16_t c16 = float_to_half_bits(__builtin_amdgcn_sqrtf(csq));
                const float cvj = half_bits_to_float(c16);
                if (!(cvj > 0.f && cvj < INFINITY)) bad |= KVQ_FLAG_SIDE_OVERFLOW;
                const int ch = 16 * (2 * rr + j) + cc;
                a.cnorm[blk * ZD + ch] = c16;
                // 1 / (sqrt(128) c16): reciprocal, then one Newton correction of the quotient
                // (Markstein), within an ulp of the rounded quotient
                const float rc = __builtin_amdgcn_rcpf(cvj), q0 = INV_SQRT_H * rc;
                m2[j] = __builtin_fmaf(__builtin_fmaf(-cvj, q0, INV_SQRT_H), rc, q0);
            }
            bcast_owned(m2[0], m2[1], mult, bcb[wave], cc, rr);
        }

        // ---- per token: asymmetric RTN with fp16 (S, Z); byte codes into the image
        uint32_t cm[8];  // channel-major: bytes of rows 4 rr .. + 3 of channel 16 j + cc
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
        // per token: lane cc = k of each row group computes (S16, Z16) of its row 4 rr + k
        // (k < 4) and stores them; the rows' 1 / S and -Z / S return to the 16 lanes by
        // broadcasts. The other lanes' results are not used.
        float inv4[4], zi4[4];
        bool clamp;
        {
            const float mn = cc == 0 ? mnr[0] : cc == 1 ? mnr[1] : cc == 2 ? mnr[2] : mnr[3];
            const float mx = cc == 0 ? mxr[0] : cc == 1 ? mxr[1] : cc == 2 ? mxr[2] : mxr[3];
            const int row = 4 * rr + (cc & 3);
            uint16_t S16 = 0, Z16 = 0;
            if (row < n) {
                S16 = float_to_half_bits((mx - mn) * (1.0f / LEVELS));
                Z16 = float_to_half_bits(mn);
            }
            const float Sv = half_bits_to_float(S16), Zv = half_bits_to_float(Z16);
            const bool own = cc < 4;
            if (own && (!(Sv < INFINITY) || !(fabsf(Zv) < INFINITY))) bad |= KVQ_FLAG_SIDE_OVERFLOW;
            const float inv = Sv != 0.f ? __builtin_amdgcn_rcpf(Sv) : 0.f;
            const float zi = -Zv * inv;
            if (own) reinterpret_cast<uint32_t *>(a.sz)[blk * ZT + row] = (uint32_t)S16 | ((uint32_t)Z16 << 16);
            // (y - Z) / S; cvt_pk_u8 rounds to nearest even and clamps below at 0. The upper
            // clamp changes a code only for a value at or above LEVELS + 1/2, and the map
            // is monotone (inv >= 0), so only when a row's largest value gets there; it is
            // then applied to the whole wave (it leaves every other code as it is)
            clamp = __ballot(bad != 0 || (own && !(__builtin_fmaf(mx, inv, zi) < LEVELS + 0.5f))) != 0;
            inv4[0] = row_bcast<0>(inv), zi4[0] = row_bcast<0>(zi);
            inv4[1] = row_bcast<1>(inv), zi4[1] = row_bcast<1>(zi);
            inv4[2] = row_bcast<2>(inv), zi4[2] = row_bcast<2>(zi);
            inv4[3] = row_bcast<3>(inv), zi4[3] = row_bcast<3>(zi);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int row = 4 * rr + k;
            float q[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) q[j] = __builtin_fmaf(y[k][j], inv4[k], zi4[k]);
            if (clamp)
#pragma unroll
                for (int j = 0; j < 8; ++j) q[j] = fminf(q[j], LEVELS);
            if constexpr (LAYOUT == KVQ_TOKEN_MAJOR) {
#pragma unroll
                for (int j = 0; j < 8; ++j) im[row * ZD + 16 * j + cc] = (uint8_t)__builtin_amdgcn_cvt_pk_u8_f32(q[j], 0, 0);
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) cm[j] = __builtin_amdgcn_cvt_pk_u8_f32(q[j], k, cm[j]);
            }
        }
        if constexpr (LAYOUT == KVQ_CHANNEL_MAJOR) {
#pragma unroll
            for (int j = 0; j < 8; ++j) *reinterpret_cast<uint32_t *>(&im[(16 * j + cc) * ZT + 4 * rr]) = cm[j];
        }

        // ---- pack: lane l takes stream positions 32 l .. 32 l + 31 -> BITS words
        {
            const uint4 b0 = *reinterpret_cast<const uint4 *>(&im[32 * ol]);
            const uint4 b1 = *reinterpret_cast<const uint4 *>(&im[32 * ol + 16]);
            const uint32_t bw[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
            uint32_t out[BITS];
            pack32_codes<BITS>(bw, out);
            uint32_t *dst = reinterpret_cast<uint32_t *>(a.codes + blk * (ZT * ZD * BITS / 8)) + BITS * ol;
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
           (a.layout == KVQ_TOKEN_MAJOR || a.layout == KVQ_CHANNEL_MAJOR) && a.stride_token >= ZD &&
           a.stride_token < (int64_t(1) << 26) &&
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
