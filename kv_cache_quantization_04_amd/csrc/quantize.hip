// Tile quantizer and dequantizer kernels (gfx950).
//
// One workgroup owns one (tile, head): T tokens x D channels held in registers.
// Thread layout: 2*D threads; thread (rg, cc) with cc = tid % (D/8) holds the 8
// consecutive channels 8cc..8cc+7 of the T/16 consecutive rows rg*T/16 + k.
// A 16-byte load per row and thread; the D/8 lanes of a row group cover a
// token's channels contiguously.
//
// Method: "KVarN" project review, Key Features ("Variance-Normalized
// Quantization Pipeline"): Hadamard rotation along channels, iterative
// Sinkhorn-like row/column variance normalization over the tile, asymmetric
// round-to-nearest. Rotation here is the unnormalized Walsh-Hadamard butterfly
// Y = X H; the 1/sqrt(h) factor is applied together with 1/c at the end (the
// normalizers are invariant to a common scale of the tile once one round has
// run, and equal 1 when none has).
#include "common.h"
#include "launch.h"

namespace kvq {

// Load 8 consecutive channels (16-byte aligned) as fp32.
__device__ __forceinline__ void load8(const void *src, int dtype, int64_t idx, float (&v)[8]) {
    if (dtype == KVQ_F32) {
        const float4 a = *reinterpret_cast<const float4 *>((const float *)src + idx);
        const float4 b = *reinterpret_cast<const float4 *>((const float *)src + idx + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        const uint4 a = *reinterpret_cast<const uint4 *>((const uint16_t *)src + idx);
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
        if (dtype == KVQ_BF16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = __uint_as_float(w[i] << 16);
                v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = half_bits_to_float(w[i] & 0xffffu);
                v[2 * i + 1] = half_bits_to_float(w[i] >> 16);
            }
        }
    }
}

// Unnormalized Walsh-Hadamard transform of blocks of h channels, Sylvester
// order: channel bits 0..2 inside the thread, bits 3.. across lanes cc.
template <int RR>
__device__ __forceinline__ void fwht_rows(float (&y)[RR][8], int h, int cc) {
#pragma unroll
    for (int s = 1; s < 8; s <<= 1) {
        if (s < h) {
#pragma unroll
            for (int k = 0; k < RR; ++k)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (!(j & s)) {
                        const float a = y[k][j], b = y[k][j | s];
                        y[k][j] = a + b;
                        y[k][j | s] = a - b;
                    }
        }
    }
    for (int m = 1; 8 * m < h; m <<= 1) {
        const bool upper = (cc & m) != 0;
#pragma unroll
        for (int k = 0; k < RR; ++k)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float pv = xor_shfl(y[k][j], m);
                y[k][j] = upper ? pv - y[k][j] : y[k][j] + pv;
            }
    }
}

template <int D, int T>
__global__ void __launch_bounds__(2 * D) quantize_kernel(QuantArgs a) {
    constexpr int NT = 2 * D;
    constexpr int LPR = D / 8;   // lanes per row group
    constexpr int NRG = 16;      // row groups
    constexpr int RR = T / NRG;  // rows per thread
    static_assert(NT == LPR * NRG, "layout");

    __shared__ float colpart[NRG][D];
    __shared__ float wsh[D];
    __shared__ float multsh[D];
    __shared__ uint8_t codesh[T * D];

    const int tid = threadIdx.x;
    const int cc = tid % LPR, rg = tid / LPR;
    const int tile = blockIdx.x, head = blockIdx.y;
    const int dst_page = a.tile_dst_page[tile];
    if (dst_page < 0 || dst_page >= a.num_pages) return;  // invalid destination: tile skipped
    const int n = a.tile_valid[tile];
    const int64_t tok0 = a.tile_src_token[tile];
    const int64_t blk = (int64_t)dst_page * a.H + head;

    float y[RR][8];
#pragma unroll
    for (int k = 0; k < RR; ++k) {
        const int row = rg * RR + k;
        if (row < n) {
            load8(a.src, a.dtype, (tok0 + row) * a.stride_token + head * a.stride_head + cc * 8, y[k]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) y[k][j] = 0.f;
        }
    }

    fwht_rows<RR>(y, a.h, cc);

    uint32_t bad = 0;
#pragma unroll
    for (int k = 0; k < RR; ++k)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (!isfinite(y[k][j])) bad |= KVQ_FLAG_NONFINITE;

    // ---- normalization rounds on A = Y^2: u = 1/r^2, w = 1/c^2 --------------
    // A = Y^2 is kept in registers when it fits, otherwise recomputed
    constexpr bool KEEP_A = D <= 256;
    float A[KEEP_A ? RR : 1][8];
    if constexpr (KEEP_A) {
#pragma unroll
        for (int k = 0; k < RR; ++k)
#pragma unroll
            for (int j = 0; j < 8; ++j) A[k][j] = y[k][j] * y[k][j];
    }
    auto sq = [&](int k, int j) -> float {
        if constexpr (KEEP_A) return A[k][j];
        else return y[k][j] * y[k][j];
    };
    float w[8], u[RR];
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = 1.f;
#pragma unroll
    for (int k = 0; k < RR; ++k) u[k] = 1.f;
    float csq = 1.f;  // c^2 of channel tid (tid < D)

    if (a.center) {
        // Centered rounds: each step divides by the standard deviation about the
        // row's (column's) mean. With sr = 1/r and vc = 1/c, Z = Y sr vc; a row step
        // sets sr_i = 1 / std_j(Y_ij vc_j), a column step vc_j = 1 / std_i(Y_ij sr_i)
        // over the n valid rows (two passes each: mean, then squared deviations).
        float sr[RR], vc[8];
#pragma unroll
        for (int k = 0; k < RR; ++k) sr[k] = 1.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) vc[j] = 1.f;
        for (int it = 0; it < a.iters; ++it) {
#pragma unroll
            for (int k = 0; k < RR; ++k) {
                float m = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) m += y[k][j] * vc[j];
#pragma unroll
                for (int mm = 1; mm < LPR; mm <<= 1) m += xor_shfl(m, mm);
                m *= 1.0f / (float)D;
                float v = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float d = y[k][j] * vc[j] - m;  // z - mean, as rounded z: exact 0 for a constant row
                    v = __builtin_fmaf(d, d, v);
                }
#pragma unroll
                for (int mm = 1; mm < LPR; mm <<= 1) v += xor_shfl(v, mm);
                v *= 1.0f / (float)D;
                if (v > 0.f && isfinite(v)) sr[k] = 1.0f / sqrtf(v);
            }
            // column mean over the valid rows
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float t = 0.f;
#pragma unroll
                for (int k = 0; k < RR; ++k)
                    if (rg * RR + k < n) t += y[k][j] * sr[k];
                colpart[rg][cc * 8 + j] = t;
            }
            __syncthreads();
            if (tid < D) {
                float t = 0.f;
#pragma unroll
                for (int g = 0; g < NRG; ++g) t += colpart[g][tid];
                wsh[tid] = n > 0 ? t / (float)n : 0.f;
            }
            __syncthreads();
            float cm[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) cm[j] = wsh[cc * 8 + j];
            // column variance about that mean
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float t = 0.f;
#pragma unroll
                for (int k = 0; k < RR; ++k)
                    if (rg * RR + k < n) {
                        const float d = y[k][j] * sr[k] - cm[j];  // exact 0 for a single valid row
                        t = __builtin_fmaf(d, d, t);
                    }
                colpart[rg][cc * 8 + j] = t;
            }
            __syncthreads();
            if (tid < D) {
                float t = 0.f;
#pragma unroll
                for (int g = 0; g < NRG; ++g) t += colpart[g][tid];
                if (n > 0 && t > 0.f && isfinite(t)) csq = t / (float)n;  // c_j = std (new)
                wsh[tid] = 1.0f / sqrtf(csq);
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < 8; ++j) vc[j] = wsh[cc * 8 + j];
        }
    }
    for (int it = 0; it < (a.center ? 0 : a.iters); ++it) {
        // row step: r_i^2 = mean_j A_ij / c_j^2
#pragma unroll
        for (int k = 0; k < RR; ++k) {
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) s = __builtin_fmaf(sq(k, j), w[j], s);
#pragma unroll
            for (int m = 1; m < LPR; m <<= 1) s += xor_shfl(s, m);
            if (s > 0.f && isfinite(s)) u[k] = (float)D / s;
        }
        // column step: c_j^2 = mean_i A_ij / r_i^2 over the n valid rows
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float t = 0.f;
#pragma unroll
            for (int k = 0; k < RR; ++k) t = __builtin_fmaf(sq(k, j), u[k], t);
            colpart[rg][cc * 8 + j] = t;
        }
        __syncthreads();
        if (tid < D) {
            float t = 0.f;
#pragma unroll
            for (int g = 0; g < NRG; ++g) t += colpart[g][tid];
            if (n > 0 && t > 0.f && isfinite(t)) csq = t / (float)n;
            wsh[tid] = 1.f / csq;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = wsh[cc * 8 + j];
    }

    // ---- fp16 normalizer and the per-channel multiplier 1 / (sqrt(h) c16) ----
    if (tid < D) {
        const uint16_t c16 = float_to_half_bits(sqrtf(csq));
        const float cv = half_bits_to_float(c16);
        if (!isfinite(cv) || cv == 0.f) bad |= KVQ_FLAG_SIDE_OVERFLOW;
        a.cnorm[blk * D + tid] = c16;
        multsh[tid] = (1.0f / sqrtf((float)a.h)) / cv;
    }
    __syncthreads();

    // ---- per token and group: asymmetric RTN with fp16 (S, Z) ----------------
    const int levels = (1 << a.bits) - 1;
    const int lpg = a.G / 8;  // lanes per group
    float mult[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) mult[j] = multsh[cc * 8 + j];
    const int ng = D / a.G;
#pragma unroll
    for (int k = 0; k < RR; ++k) {
        const int row = rg * RR + k;
        float mn = INFINITY, mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            y[k][j] = y[k][j] * mult[j];
            mn = fminf(mn, y[k][j]);
            mx = fmaxf(mx, y[k][j]);
        }
        for (int m = 1; m < lpg; m <<= 1) {
            mn = fminf(mn, xor_shfl(mn, m));
            mx = fmaxf(mx, xor_shfl(mx, m));
        }
        uint16_t S16 = 0, Z16 = 0;
        if (row < n) {
            S16 = float_to_half_bits((mx - mn) / (float)levels);
            Z16 = float_to_half_bits(mn);
        }
        const float Sv = half_bits_to_float(S16), Zv = half_bits_to_float(Z16);
        if (!isfinite(Sv) || !isfinite(Zv)) bad |= KVQ_FLAG_SIDE_OVERFLOW;
        const float inv = 1.0f / Sv;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float q = 0.f;
            if (Sv != 0.f) {
                const float d = y[k][j] - Zv;
                q = fminf(fmaxf(rintf(d * inv), 0.f), (float)levels);
            }
            const int ch = cc * 8 + j;
            const int idx = a.layout == KVQ_TOKEN_MAJOR ? row * D + ch : ch * T + row;
            codesh[idx] = (uint8_t)q;
        }
        if (cc % lpg == 0) {
            const int g = cc / lpg;
            reinterpret_cast<uint32_t *>(a.sz)[(blk * T + row) * ng + g] = (uint32_t)S16 | ((uint32_t)Z16 << 16);
        }
    }
    __syncthreads();

    // ---- pack the block as one little-endian bitstream ----------------------
    const int bits = a.bits;
    constexpr int NCODE = T * D;
    const int ndw = NCODE * bits / 32;
    uint32_t *out = reinterpret_cast<uint32_t *>(a.codes + blk * (int64_t)(NCODE * bits / 8));
    for (int wd = tid; wd < ndw; wd += NT) {
        const int b0 = 32 * wd;
        const int i0 = b0 / bits, i1 = min((b0 + 31) / bits, NCODE - 1);
        uint64_t acc = 0;
        for (int i = i0; i <= i1; ++i) acc |= (uint64_t)codesh[i] << (bits * i - b0 + 32);
        out[wd] = (uint32_t)(acc >> 32);
    }

    // ---- rope channels (MLA): bf16 copy, unrotated --------------------------
    if (a.R > 0) {
        for (int e = tid; e < T * a.R; e += NT) {
            const int row = e / a.R, kk = e % a.R;
            uint16_t bv = 0;
            if (row < n) {
                const float v = load_as_float(a.src, a.dtype, (tok0 + row) * a.stride_token + head * a.stride_head + D + kk);
                if (!isfinite(v)) bad |= KVQ_FLAG_NONFINITE;
                bv = float_to_bf16_bits(v);
            }
            a.rope[(blk * T + row) * a.R + kk] = bv;
        }
    }

    if (a.flags) {
        const int nf = __syncthreads_or((int)(bad & KVQ_FLAG_NONFINITE));
        const int so = __syncthreads_or((int)(bad & KVQ_FLAG_SIDE_OVERFLOW));
        if (tid == 0 && (nf || so))
            atomicOr(a.flags, (nf ? (uint32_t)KVQ_FLAG_NONFINITE : 0u) | (so ? (uint32_t)KVQ_FLAG_SIDE_OVERFLOW : 0u));
    }
}

template <int D, int T>
__global__ void __launch_bounds__(2 * D) dequant_kernel(DequantArgs a) {
    constexpr int LPR = D / 8;
    constexpr int RR = T / 16;
    const int tid = threadIdx.x;
    const int cc = tid % LPR, rg = tid / LPR;
    const int tile = blockIdx.x, head = blockIdx.y;
    const int nvalid = a.tile_valid[tile];
    const int src_page = a.tile_page[tile];
    if (src_page < 0 || src_page >= a.num_pages) return;  // invalid page: tile skipped
    const int64_t blk = (int64_t)src_page * a.H + head;
    const int bits = a.bits;
    const int blockbytes = T * D * bits / 8;
    const uint8_t *cb = a.codes + blk * blockbytes;
    const int ng = D / a.G;

    float y[RR][8];
    float cv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) cv[j] = half_bits_to_float(a.cnorm[blk * D + cc * 8 + j]);
#pragma unroll
    for (int k = 0; k < RR; ++k) {
        const int row = rg * RR + k;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int ch = cc * 8 + j;
            const int i = a.layout == KVQ_TOKEN_MAJOR ? row * D + ch : ch * T + row;
            const int bit = bits * i;
            const int bo = bit >> 3;
            uint32_t win = cb[bo];
            if (bo + 1 < blockbytes) win |= (uint32_t)cb[bo + 1] << 8;
            const uint32_t code = (win >> (bit & 7)) & ((1u << bits) - 1);
            const uint32_t szw = reinterpret_cast<const uint32_t *>(a.sz)[(blk * T + row) * ng + ch / a.G];
            const float S = half_bits_to_float(szw & 0xffffu), Z = half_bits_to_float(szw >> 16);
            y[k][j] = __builtin_fmaf(S, (float)code, Z) * cv[j];
        }
    }
    fwht_rows<RR>(y, a.h, cc);
    const float sc = 1.0f / sqrtf((float)a.h);
    const int W = D + a.R;
#pragma unroll
    for (int k = 0; k < RR; ++k) {
        const int row = rg * RR + k;
        const int64_t o = ((int64_t)(tile * a.H + head) * T + row) * W + cc * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float v = row < nvalid ? y[k][j] * sc : 0.f;
            if (a.dtype == KVQ_F32) ((float *)a.dst)[o + j] = v;
            else if (a.dtype == KVQ_F16) ((uint16_t *)a.dst)[o + j] = float_to_half_bits(v);
            else ((uint16_t *)a.dst)[o + j] = float_to_bf16_bits(v);
        }
    }
    if (a.R > 0) {
        for (int e = tid; e < T * a.R; e += 2 * D) {
            const int row = e / a.R, kk = e % a.R;
            const float v = row < nvalid ? bf16_bits_to_float(a.rope[(blk * T + row) * a.R + kk]) : 0.f;
            const int64_t o = ((int64_t)(tile * a.H + head) * T + row) * W + D + kk;
            if (a.dtype == KVQ_F32) ((float *)a.dst)[o] = v;
            else if (a.dtype == KVQ_F16) ((uint16_t *)a.dst)[o] = float_to_half_bits(v);
            else ((uint16_t *)a.dst)[o] = float_to_bf16_bits(v);
        }
    }
}

#define KVQ_DISPATCH_DT(D_, MACRO) \
    switch (T) {                   \
    case 16: MACRO(D_, 16); break; \
    case 32: MACRO(D_, 32); break; \
    case 64: MACRO(D_, 64); break; \
    case 128: MACRO(D_, 128); break; \
    default: return false;         \
    }

#define KVQ_DISPATCH(MACRO)                      \
    switch (D) {                                 \
    case 64: KVQ_DISPATCH_DT(64, MACRO) break;   \
    case 128: KVQ_DISPATCH_DT(128, MACRO) break; \
    case 256: KVQ_DISPATCH_DT(256, MACRO) break; \
    case 512: KVQ_DISPATCH_DT(512, MACRO) break; \
    default: return false;                       \
    }

bool quantize_d128_supported(int D, int T, const QuantArgs &a);
void launch_quantize_d128(int T, int num_tiles, const QuantArgs &a, hipStream_t stream);
bool quantize_d128_pair_supported(int T, const QuantArgs &k, const QuantArgs &v);
void launch_quantize_d128_pair(int T, int num_tiles, const QuantArgs &k, const QuantArgs &v, hipStream_t stream);
bool quantize_t16_supported(int D, int T, const QuantArgs &a);
void launch_quantize_t16(int num_tiles, const QuantArgs &a, hipStream_t stream);
bool quantize_d512_supported(int D, int T, const QuantArgs &a);
void launch_quantize_d512(int num_tiles, const QuantArgs &a, hipStream_t stream);

const char *quantize_kernel_name(int D, int T, const QuantArgs &a) {
    if (quantize_d128_supported(D, T, a)) return "quantize_d128_kernel";
    if (quantize_t16_supported(D, T, a)) return "quantize_t16_kernel";
    if (quantize_d512_supported(D, T, a)) return "quantize_d512_kernel";
    return "quantize_kernel";
}

bool launch_quantize(int D, int T, int num_tiles, const QuantArgs &a, hipStream_t stream) {
    if (quantize_d128_supported(D, T, a)) {
        launch_quantize_d128(T, num_tiles, a, stream);
        return true;
    }
    if (quantize_t16_supported(D, T, a)) {
        launch_quantize_t16(num_tiles, a, stream);
        return true;
    }
    if (quantize_d512_supported(D, T, a)) {
        launch_quantize_d512(num_tiles, a, stream);
        return true;
    }
#define KVQ_LQ(D_, T_) \
    hipLaunchKernelGGL((quantize_kernel<D_, T_>), dim3(num_tiles, a.H), dim3(2 * D_), 0, stream, a)
    KVQ_DISPATCH(KVQ_LQ)
#undef KVQ_LQ
    return true;
}

bool quantize_pair_supported(int D, int T, const QuantArgs &k, const QuantArgs &v) {
    return D == 128 && k.H == v.H && quantize_d128_pair_supported(T, k, v);
}

bool launch_quantize_pair(int D, int T, int num_tiles, const QuantArgs &k, const QuantArgs &v, hipStream_t stream) {
    if (!quantize_pair_supported(D, T, k, v)) return false;
    launch_quantize_d128_pair(T, num_tiles, k, v, stream);
    return true;
}

bool launch_dequant(int D, int T, int num_tiles, const DequantArgs &a, hipStream_t stream) {
#define KVQ_LD(D_, T_) \
    hipLaunchKernelGGL((dequant_kernel<D_, T_>), dim3(num_tiles, a.H), dim3(2 * D_), 0, stream, a)
    KVQ_DISPATCH(KVQ_LD)
#undef KVQ_LD
    return true;
}

}  // namespace kvq
