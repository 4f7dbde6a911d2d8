// Split-K decode attention over the paged quantized cache (gfx950), generic path.
//
// Folded evaluation (the dequantized K and V are never formed):
//   score_t = sm * ( sum_g S_tg * <q'_g, code_tg> + Z_tg * sum_{j in g} q'_j ) [+ <q_rope, k_rope_t>]
//     with q' = (q Q) o c_K (per page: c is per tile),
//   o'      = sum_t p_t (S_tg code_tj + Z_tg) c_V,j     accumulated per page,
//   out     = (o' / sum_t p_t) Q                         in the reduce kernel.
// Grid: (split, kv head x head chunk, sequence); each workgroup walks its page
// range through the block table and writes (m, l, o') to the workspace.
#include "common.h"
#include "decode_merge.h"
#include "launch.h"
#include "xlane.h"

namespace kvq {

__device__ __forceinline__ uint32_t get_code(const uint8_t *blk, int i, int bits, int blockbytes) {
    const int bit = bits * i;
    const int bo = bit >> 3;
    uint32_t win = blk[bo];
    if (bo + 1 < blockbytes) win |= (uint32_t)blk[bo + 1] << 8;
    return (win >> (bit & 7)) & ((1u << bits) - 1);
}

// In-place Walsh-Hadamard transform of `rows` LDS rows of length n, blocks of h.
__device__ void lds_fwht(float *buf, int rows, int n, int h) {
    for (int len = 1; len < h; len <<= 1) {
        for (int e = threadIdx.x; e < rows * n / 2; e += blockDim.x) {
            const int r = e / (n / 2), pe = e % (n / 2);
            const int i = (pe / len) * 2 * len + pe % len;
            float *row = buf + r * n;
            const float x = row[i], y = row[i + len];
            row[i] = x + y;
            row[i + len] = x - y;
        }
        __syncthreads();
    }
}

constexpr int DEC_NT = 256;
constexpr int DEC_MAXO = 32;  // owned (head, channel) outputs per thread

__global__ void __launch_bounds__(DEC_NT) decode_generic_kernel(DecodeArgs a) {
    extern __shared__ float smem[];
    const int hc = a.hc, D = a.D, R = a.R, Dv = a.Dv, T = a.T;
    float *qbar = smem;                    // [hc][D]
    float *qt = qbar + hc * D;             // [hc][D]
    float *qsum = qt + hc * D;             // [hc][D/kG]
    float *qrope = qsum + hc * (D / a.kG); // [hc][R]
    float *logit = qrope + hc * R;         // [hc][T]
    float *mrow = logit + hc * T;          // [hc]
    float *lrow = mrow + hc;               // [hc]
    float *srow = lrow + hc;               // [hc]

    const int tid = threadIdx.x;
    const int split = blockIdx.x;
    const int hk = blockIdx.y / a.nhc, chunk = blockIdx.y % a.nhc;
    const int s = blockIdx.z;
    const int h0 = hk * a.grp + chunk * hc;
    const int L = a.seq_lens[s];
    const int npages = min((L + T - 1) / T, a.bt_stride);
    const int pps = (npages + a.splits - 1) / a.splits;
    const int p0 = split * pps, p1 = min(npages, p0 + pps);

    // rotated query (unnormalized transform; 1/sqrt(h) applied below)
    for (int e = tid; e < hc * D; e += DEC_NT) {
        const int hh = e / D, j = e % D;
        qbar[e] = load_as_float(a.q, a.q_dtype, ((int64_t)s * a.Hq + h0 + hh) * (D + R) + j);
    }
    for (int e = tid; e < hc * R; e += DEC_NT) {
        const int hh = e / R, j = e % R;
        qrope[e] = load_as_float(a.q, a.q_dtype, ((int64_t)s * a.Hq + h0 + hh) * (D + R) + D + j);
    }
    if (tid < hc) {
        mrow[tid] = -INFINITY;
        lrow[tid] = 0.f;
    }
    __syncthreads();
    lds_fwht(qbar, hc, D, a.kh);
    const float qscale = 1.0f / sqrtf((float)a.kh);
    for (int e = tid; e < hc * D; e += DEC_NT) qbar[e] *= qscale;

    float o[DEC_MAXO];
#pragma unroll
    for (int i = 0; i < DEC_MAXO; ++i) o[i] = 0.f;
    const int nown = hc * Dv;
    const int kblockbytes = T * D * a.kbits / 8;
    const int vblockbytes = T * Dv * a.vbits / 8;
    const int kng = D / a.kG, vng = Dv / a.vG;
    __syncthreads();

    for (int pi = p0; pi < p1; ++pi) {
        const int page = a.bt[(int64_t)s * a.bt_stride + pi];
        if (page < 0 || page >= a.num_pages) continue;  // invalid block-table entry: page skipped
        const int rows = min(T, L - pi * T);
        const int64_t kblk = (int64_t)page * a.Hkv + hk;
        for (int e = tid; e < hc * D; e += DEC_NT) qt[e] = qbar[e] * half_bits_to_float(a.kcn[kblk * D + e % D]);
        __syncthreads();
        for (int e = tid; e < hc * kng; e += DEC_NT) {
            const int hh = e / kng, g = e % kng;
            float acc = 0.f;
            for (int j = g * a.kG; j < (g + 1) * a.kG; ++j) acc += qt[hh * D + j];
            qsum[e] = acc;
        }
        __syncthreads();
        const uint8_t *kb = a.kcodes + kblk * kblockbytes;
        for (int e = tid; e < hc * T; e += DEC_NT) {
            const int hh = e / T, t = e % T;
            float acc = -INFINITY;
            if (t < rows) {
                acc = 0.f;
                for (int g = 0; g < kng; ++g) {
                    float dot = 0.f;
                    for (int j = g * a.kG; j < (g + 1) * a.kG; ++j) {
                        const int i = a.klayout == KVQ_TOKEN_MAJOR ? t * D + j : j * T + t;
                        dot = __builtin_fmaf(qt[hh * D + j], (float)get_code(kb, i, a.kbits, kblockbytes), dot);
                    }
                    const uint32_t szw = reinterpret_cast<const uint32_t *>(a.ksz)[(kblk * T + t) * kng + g];
                    acc += half_bits_to_float(szw & 0xffffu) * dot + half_bits_to_float(szw >> 16) * qsum[hh * kng + g];
                }
                for (int j = 0; j < R; ++j)
                    acc += qrope[hh * R + j] * bf16_bits_to_float(a.krope[(kblk * T + t) * R + j]);
                acc *= a.sm;
            }
            logit[e] = acc;
        }
        __syncthreads();
        if (tid < hc) {
            float mx = mrow[tid];
            for (int t = 0; t < rows; ++t) mx = fmaxf(mx, logit[tid * T + t]);
            const float sc = __expf(mrow[tid] - mx);
            float l = lrow[tid] * sc;
            for (int t = 0; t < rows; ++t) {
                const float pv = __expf(logit[tid * T + t] - mx);
                logit[tid * T + t] = pv;
                l += pv;
            }
            mrow[tid] = mx;
            lrow[tid] = l;
            srow[tid] = sc;
        }
        __syncthreads();
        const int64_t vblk = (int64_t)page * a.vH + hk;
        const uint8_t *vb = a.vcodes + vblk * vblockbytes;
#pragma unroll
        for (int i = 0; i < DEC_MAXO; ++i) {
            const int e = tid + i * DEC_NT;
            if (e < nown) {
                const int hh = e / Dv, j = e % Dv;
                const int g = j / a.vG;
                float acc = 0.f;
                for (int t = 0; t < rows; ++t) {
                    const int ci = a.vlayout == KVQ_TOKEN_MAJOR ? t * Dv + j : j * T + t;
                    const uint32_t szw = reinterpret_cast<const uint32_t *>(a.vsz)[(vblk * T + t) * vng + g];
                    const float xv = __builtin_fmaf(half_bits_to_float(szw & 0xffffu),
                                                    (float)get_code(vb, ci, a.vbits, vblockbytes),
                                                    half_bits_to_float(szw >> 16));
                    acc = __builtin_fmaf(logit[hh * T + t], xv, acc);
                }
                o[i] = __builtin_fmaf(o[i], srow[hh], acc * half_bits_to_float(a.vcn[vblk * Dv + j]));
            }
        }
        __syncthreads();
    }

    // partial result of this split: o' (unnormalized), m, l
#pragma unroll
    for (int i = 0; i < DEC_MAXO; ++i) {
        const int e = tid + i * DEC_NT;
        if (e < nown) {
            const int hh = e / Dv, j = e % Dv;
            a.ws[(((int64_t)s * a.Hq + h0 + hh) * a.splits + split) * (Dv + 2) + j] = o[i];
        }
    }
    if (tid < hc) {
        float *w = a.ws + (((int64_t)s * a.Hq + h0 + tid) * a.splits + split) * (Dv + 2) + Dv;
        w[0] = mrow[tid];
        w[1] = lrow[tid];
    }
}

__global__ void __launch_bounds__(64 * RED_WAVES) decode_reduce_kernel(DecodeArgs a) {
    __shared__ float wgt[RED_WAVES][RED_MAX_SPLITS];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nhg = (a.Hq + RED_WAVES - 1) / RED_WAVES;  // head groups per row
    const int s = blockIdx.x / nhg, hq = (blockIdx.x - s * nhg) * RED_WAVES + wave;
    if (hq >= a.Hq) return;  // whole wave
    switch (a.Dv) {
    case 64: reduce_one<1>(a, s, hq, lane, wgt[wave]); break;
    case 128: reduce_one<2>(a, s, hq, lane, wgt[wave]); break;
    case 256: reduce_one<4>(a, s, hq, lane, wgt[wave]); break;
    default: reduce_one<8>(a, s, hq, lane, wgt[wave]); break;  // 512
    }
}

static void launch_reduce(const DecodeArgs &a, hipStream_t stream) {
    // one workgroup per (row, group of RED_WAVES query heads), rows = a.B
    const int64_t nwg = (int64_t)((a.Hq + RED_WAVES - 1) / RED_WAVES) * a.B;
    hipLaunchKernelGGL(decode_reduce_kernel, dim3((unsigned)nwg), dim3(64 * RED_WAVES), 0, stream, a);
}

bool decode_mfma_supported(const DecodeArgs &a);
bool decode_pair16_supported(const DecodeArgs &a);
bool launch_decode_mfma(const DecodeArgs &a, hipStream_t stream);
bool decode_mla_supported(const DecodeArgs &a);
int decode_mla_head_groups(const DecodeArgs &a);
bool launch_decode_mla(const DecodeArgs &a, hipStream_t stream);

// Split count for `units` independent (sequence, kv head[, head group]) items: about
// `target` workgroups in all, at least `min_pages` pages per split.
static int splits_for(int64_t units, int64_t target, int64_t pages, int64_t min_pages) {
    if (units < 1) return 1;
    int64_t sp = (target + units - 1) / units;
    const int64_t cap = (pages + min_pages - 1) / min_pages;
    if (sp > cap) sp = cap;
    if (sp > RED_MAX_SPLITS) sp = RED_MAX_SPLITS;
    if (sp < 1) sp = 1;
    return (int)sp;
}

int decode_default_splits(const DecodeArgs &a, int max_seq_len) {
    const int64_t pages = (max_seq_len + a.T - 1) / a.T;
    if (decode_mla_supported(a)) {
        // one 256-thread workgroup per compute unit (its registers fill the SIMDs),
        // per (sequence, kv head, 64 query heads, split); at least 2 pages per split
        return splits_for((int64_t)a.B * a.Hkv * decode_mla_head_groups(a), 256, pages, 2);
    }
    // Four waves per workgroup walk the split's pages independently. Two bounds, the
    // larger wins: at least 512 workgroups (two per compute unit), and at most 2048
    // tokens of the longest sequence per split (512 per wave), so that with unequal
    // lengths the longest sequences do not trail; each wave keeps at least one page.
    // The paired 16-token kernel starts the longest sequences first (up to 256, one per
    // thread of its workgroup), which keeps them from trailing with splits twice as
    // long: 4096 tokens (64 sequences of 512..16384 tokens: 4 splits 238-240 us, 8 splits 262 us).
    // (Measured on the GQA workloads against 2..256 splits: best or within 2% of it.)
    const int64_t units = (int64_t)a.B * a.Hkv;
    if (units < 1) return 1;
    int64_t sp = (512 + units - 1) / units;
    const int64_t split_tokens = decode_pair16_supported(a) && a.B <= 256 ? 4096 : 2048;
    const int64_t by_len = ((int64_t)max_seq_len + split_tokens - 1) / split_tokens;
    if (sp < by_len) sp = by_len;
    sp = splits_for(1, sp, pages, 4);
    // Long splits of 64- and 128-token pages (4 or more pages per wave): one workgroup
    // per compute unit with double-buffered page images, when each wave then walks at
    // least 8 pages (the kernel picks that variant from the split length).
    if (a.T >= 64 && (pages + sp - 1) / sp >= 16) {
        const int64_t db = splits_for(units, 256, pages, 32);
        if ((pages + db - 1) / db >= 32) return (int)db;
    }
    return (int)sp;
}

int decode_chunk_splits(const DecodeArgs &a, int max_seq_len) {
    // chunked prefill (the column blocks counted as sequences): about 4 workgroups per
    // compute unit, at least 4 pages per split
    const int64_t pages = (max_seq_len + a.T - 1) / a.T;
    if (decode_mla_supported(a)) return splits_for((int64_t)a.B * a.Hkv * decode_mla_head_groups(a), 256, pages, 2);
    return splits_for((int64_t)a.B * a.Hkv, 1024, pages, 4);
}

const char *decode_kernel_name(const DecodeArgs &a) {
    if (decode_mla_supported(a)) return "decode_mla_kernel";
    if (decode_pair16_supported(a)) return "decode_pair16_kernel";
    if (decode_mfma_supported(a)) return "decode_mfma_kernel";
    return "decode_generic_kernel";
}

// chunked prefill on the MFMA kernel: a.B real sequences of a.Lq positions; the
// split partials, the reduce and the output cover a.B * a.Lq rows
bool launch_decode_chunk(const DecodeArgs &a_in, hipStream_t stream) {
    DecodeArgs a = a_in;
    a.cnt = nullptr;
    if (a.splits > RED_MAX_SPLITS || a.Lq <= 0 || !decode_mfma_supported(a)) return false;
    if (!launch_decode_mfma(a, stream)) return false;
    DecodeArgs r = a;
    r.B = a.B * a.Lq;
    r.Lq = 0;
    launch_reduce(r, stream);
    return true;
}

// The matrix-core GQA kernels merge the splits themselves (the last workgroup of each
// sequence and kv head, counted in a.cnt) when the grid is one round of workgroups on
// the chip (at most two per compute unit): the merge then replaces the reduce kernel's
// launch and ramp with a few memory round trips at the end of the last workgroups.
// Larger grids keep the reduce kernel: every workgroup would wait for its partial
// stores to complete before counting its arrival, and with several rounds of
// workgroups those waits add up to more than the launch they save. Grids beyond the
// counters, and the other kernels, use the reduce kernel too.
constexpr int64_t MERGE_MAX_WORKGROUPS = 512;

bool decode_merges_in_kernel(const DecodeArgs &a) {
    return !decode_mla_supported(a) && decode_mfma_supported(a) && a.B <= 65535 && a.splits <= RED_MAX_SPLITS &&
           (int64_t)a.B * a.Hkv <= MERGE_COUNTERS && (int64_t)a.B * a.Hkv * a.splits <= MERGE_MAX_WORKGROUPS;
}

bool launch_decode(const DecodeArgs &a_in, hipStream_t stream) {
    DecodeArgs a = a_in;
    const bool counters = a.cnt && decode_merges_in_kernel(a);
    a.cnt = nullptr;
    if (a.splits > RED_MAX_SPLITS) return false;
    if (decode_mla_supported(a)) {
        if (!launch_decode_mla(a, stream)) return false;
        launch_reduce(a, stream);
        return true;
    }
    if (a.B > 65535) return false;  // the grids below put sequences on z
    if (decode_mfma_supported(a)) {
        if (counters) a.cnt = a_in.cnt;
        if (!launch_decode_mfma(a, stream)) return false;
        if (!a.cnt) launch_reduce(a, stream);
        return true;
    }
    const size_t smem = sizeof(float) * (2 * a.hc * a.D + a.hc * (a.D / a.kG) + a.hc * a.R + a.hc * a.T + 3 * a.hc);
    if (a.hc * a.Dv > DEC_NT * DEC_MAXO) return false;
    if (smem > 64 * 1024 &&
        hipFuncSetAttribute((const void *)decode_generic_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) !=
            hipSuccess)
        return false;
    hipLaunchKernelGGL(decode_generic_kernel, dim3(a.splits, a.Hkv * a.nhc, a.B), dim3(DEC_NT), smem, stream, a);
    launch_reduce(a, stream);
    return true;
}

}  // namespace kvq
