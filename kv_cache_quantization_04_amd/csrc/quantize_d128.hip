// Tile quantizer specialised for head_dim 128, Hadamard block 128, one scale
// group per token (gfx950). Same method and results as the generic kernel; all
// cross-lane traffic stays in the VALU (DPP, permlane swaps) or the LDS
// crossbar without memory (ds_swizzle), and the codes are packed in registers.
//
// Workgroup = one (tile, head) at a time, T / (4 R) waves, wave w owning rows
// 16 w .. 16 w + 15. The 128-point rotation runs on the matrix cores
// (mfma_hadamard.h, pair order): lane l supplies the bf16 source of row 16 w + (l & 15)
// as the A operand and receives the rotated rows of row group rg = 4 w + (l >> 4)
// (R = 4 rows) at the channel pairs 32 u + 2 (l & 15) + {0, 1}, u = 0..3. The 16 lanes
// of a DPP row therefore cover one token's 128 channels: every per-token reduction is
// a DPP row operation, and 4-bit token-major codes leave each lane as whole bytes.
//
// Persistent workgroups walk items (tile, head); the next item's rows are copied
// HBM -> LDS while the current one is computed. One launch can cover the K and V
// caches of a batch (PAIR): K items first, then V items, each with its own layout
// and bit width.
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

constexpr int QD = 128;
// rows per lane: 4 (8 waves per 128-token tile, 4 per 64-token tile)
constexpr int QR = 4;

// LDS image of a code block: 16-byte slot U of the global layout lives at slot
// code_slot(U). The stores that run together (one row, or one channel, of every
// lane) then fall in distinct 16-byte bank windows, and the coalesced copy-out
// reads slot code_slot(i) for global slot i (the map is its own inverse).
//   token-major: the four row groups of a wave (rg & 3) spread over the slots of a
//     row, rg = row / R, row = U / BITS;
//   channel-major: the 16 channel groups (cc) spread over the 16 low slot bits.
template <int T, int R, int BITS, int LAYOUT>
__device__ __forceinline__ int code_slot(int U) {
    if constexpr (LAYOUT == KVQ_TOKEN_MAJOR) {
        constexpr int L = BITS == 4 ? 2 : 1;   // log2 of slots per token row
        constexpr int S = L + (R == 8 ? 3 : 2);  // log2 of slots per row group
        return U ^ (((U >> S) & 3) << L);
    } else {
        constexpr int CR = T * BITS / 128;      // slots per channel row
        constexpr int S = CR == 4 ? 5 : CR == 2 ? 4 : 3;  // log2 of slots per channel group (8 channels)
        constexpr int M = CR == 1 ? 7 : 15;
        return U ^ ((U >> S) & M);
    }
}
template <int T, int R, int BITS, int LAYOUT>
__device__ __forceinline__ int code_byte(int b) {
    return (code_slot<T, R, BITS, LAYOUT>(b >> 4) << 4) | (b & 15);
}

}  // namespace

// The LDS buffers come in as restrict pointers: after inlining, the compiler
// knows that the direct-to-LDS prefetch into `stage` touches none of the others
// and lets the prefetch stay in flight across their accesses.
//   stage  [T * 128 * 2 / 16] source rows of the next item (bf16, swizzled chunks)
//   colsum0/1 [waves][128] per-channel column partial sums, [wave][channel]; even/odd rounds
//   wsh0/1    [128]     1 / c^2 per channel; even/odd rounds
//   multsh [128]        per-channel output multiplier
//   outbuf [T * 128 * BITS / 32] LDS image of the code block
//   szbuf  [T]          (S, Z) fp16 pairs per token
//   hbtab  [2][64]      the two per-lane Hadamard operand patterns (read per item:
//                       held in registers across the item loop they spill)
template <int V>
struct IntC {
    static constexpr int value = V;
};

// Items 0 .. nk - 1 belong to cache `ak` (format BK, LK); with PAIR, items nk ..
// num_items - 1 are item - nk of cache `av` (BV, LV): the K and V caches of one batch
// in one launch, the prefetch running on from the last K item into the first V items.
template <int T, int R, int BK, int LK, int BV, int LV, int NIT, bool PAIR>
__device__ __forceinline__ void quantize_d128_body(const QuantArgs &ak, const QuantArgs &av, int nk, int num_items,
                                                   uint4 *__restrict__ stage,
                                                   float (*__restrict__ colsum0)[QD], float (*__restrict__ colsum1)[QD],
                                                   float *__restrict__ wsh0, float *__restrict__ wsh1,
                                                   float *__restrict__ multsh, uint32_t *__restrict__ outbuf,
                                                   uint32_t *__restrict__ szbuf, uint4 *__restrict__ hbtab) {
    constexpr int NWV = T / (4 * R);  // waves (4 row groups of R rows each)
    constexpr int NT = 64 * NWV;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cc = lane & 15, rr = lane >> 4;
    const int rg = wave * 4 + rr;
    if (wave == 0) {  // published by the first item's barrier
        const Had128B hb = had128_operands<true>(lane);
        hbtab[lane] = hb.p0;
        hbtab[64 + lane] = hb.p1;
    }

    // Persistent workgroups: item = tile * H + head, strided by the grid. The
    // next item's source rows are copied HBM -> LDS by direct-to-LDS loads while
    // the current item is processed in registers; only LDS-ordering barriers are
    // used until the next item starts, so the copies stay in flight. Each wave
    // load instruction moves 4 rows (1 KB): lane l -> row 4 b + (l >> 4), 16-byte
    // chunk l & 15. LDS slot (l & 15) of row r holds chunk slot ^ (r & 15), so the
    // 16 rows that the lanes of a wave read as one operand step (one chunk each) sit
    // in 16 different bank windows.
    auto fetch = [&](int gitm) {
        const bool isk = !PAIR || gitm < nk;  // uniform
        const QuantArgs &a = isk ? ak : av;
        const int itm = isk ? gitm : gitm - nk;
        const int tl = itm / a.H, hd = itm % a.H;
        const int nv = load_const(a.tile_valid, tl);
        const char *src = reinterpret_cast<const char *>(a.src) +
                          2 * (hd * a.stride_head + (int64_t)load_const(a.tile_src_token, tl) * a.stride_token);
        if (nv <= 0) return;
        // every lane takes part in every copy (rows past the valid ones repeat the last
        // valid row, never read): no guarded direct-to-LDS loads for the compiler to merge
        const int last = nv - 1;
        const uint32_t row_bytes = (uint32_t)a.stride_token * 2u;
        // lane id made opaque here: its few derived offsets are recomputed per copy
        // instead of being kept (or spilled) across the item
        int fl = tid & 63;
        asm volatile("" : "+v"(fl));
        const int fcc = fl & 15, frr = fl >> 4;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int b = wave * R + i;
            const int rb = min(4 * b, last);                // wave-uniform first row of the copy
            const int dr = min(4 * b + frr, last) - rb;     // this lane's row, 0..3 rows further
            const uint32_t off = (uint32_t)dr * row_bytes + 16u * (uint32_t)(fcc ^ ((4 * i + frr) & 15));
            __builtin_amdgcn_global_load_lds((const void *)(src + (int64_t)rb * a.stride_token * 2 + off),
                                             (__attribute__((address_space(3))) void *)(stage + b * 64), 16, 0, 0);
        }
    };
    // one item of cache `a` (local index `item`, global index `gitem`)
    auto process = [&](auto bits_c, auto layout_c, const QuantArgs &a, int item, int gitem) {
    constexpr int BITS = decltype(bits_c)::value, LAYOUT = decltype(layout_c)::value;
    constexpr float LEVELS = (float)((1 << BITS) - 1);
    // rounds: a compile-time count (fully unrolled) or, with NIT < 0, the runtime one
    const int iters = NIT >= 0 ? NIT : a.iters;
    const int tile = item / a.H, head = item % a.H;
    const int dst_page = load_const(a.tile_dst_page, tile);
    const int n = load_const(a.tile_valid, tile);
    const int64_t blk = (int64_t)dst_page * a.H + head;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies into LDS have landed
    lds_barrier();                  // and every other wave's
    // the A operands: row 16 wave + (lane & 15), chunks 4 s + (lane >> 4). Rows past the
    // valid ones hold copies of the last valid row (see fetch): read unconditionally,
    // zeroed only when the tile is partial (a uniform branch)
    uint4 x4[4];
    {
        const int arow = 16 * wave + cc;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) x4[s4] = stage[arow * 16 + ((4 * s4 + rr) ^ cc)];
        if (n < T && arow >= n)
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) x4[s4] = uint4{0, 0, 0, 0};
    }
    lds_barrier();  // the staging buffer is free again
    if (gitem + (int)gridDim.x < num_items) fetch(gitem + gridDim.x);
    if (dst_page < 0 || dst_page >= a.num_pages) return;  // invalid destination: tile skipped (uniform)

    // ---- unnormalized Walsh-Hadamard transform along the 128 channels (matrix
    // cores): lane (cc, rr) gets rows rg R + k at channels ch(t) = 32 (t >> 1) + 2 cc
    // + (t & 1), t = 0..7
    float y[R][8];
    {
        f32x4 xr[8];
        int ol = lane;  // opaque: the pattern reads stay inside the item
        asm volatile("" : "+v"(ol));
        const Had128B hbi{hbtab[ol], hbtab[64 + ol]};
        had128_rows16(x4, hbi, xr);
#pragma unroll
        for (int k = 0; k < R; ++k)
#pragma unroll
            for (int t = 0; t < 8; ++t) y[k][t] = xr[t][k];
    }

    // ---- normalization rounds on A = Y^2: u = 1/r^2 per row, w = 1/c^2 per channel
    // A = Y^2, kept in registers
    float A[R][8];
#pragma unroll
    for (int k = 0; k < R; ++k)
#pragma unroll
        for (int j = 0; j < 8; ++j) A[k][j] = y[k][j] * y[k][j];
    // non-finite detector: a row's sum of squares is finite iff the row is
    // (first round below; computed here when there is no round)
    // data conditions of this lane (lane masks: no vector registers)
    bool nonfinite = false, sideov = false;
    if (iters == 0) {
        float t = 0.f;
#pragma unroll
        for (int k = 0; k < R; ++k)
#pragma unroll
            for (int j = 0; j < 8; ++j) t += A[k][j];
        if (!isfinite(t)) nonfinite = true;
    }
    // w holds 1 / c^2 in the first round and 1 / (128 c^2) after it (the mean over
    // the 128 channels folded in: powers of two, so the row sums and u = 1 / r^2 are
    // the same bits as with the plain mean)
    float w[8], u[R];
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = 1.f;
#pragma unroll
    for (int k = 0; k < R; ++k) u[k] = 1.f;
    const float fn = (float)n, fn_d = fn * (1.0f / QD);
    // owner of channel tid (tid < 128): column sum of the last round
    float t_own = 0.f;
    constexpr float TINY = 1e-30f, HUGE_F = 3.4028234663852886e38f;

#pragma unroll
    for (int it = 0; it < iters; ++it) {
        // row step: r^2 = mean_j A_ij / c_j^2 over the 128 channels. A zero row keeps
        // a large finite u and contributes 0 * u = 0 below, as with an unchanged factor.
        // (first round: c = 1, a plain sum)
        float rs[R];
#pragma unroll
        for (int k = 0; k < R; ++k) {
            float s = 0.f;
            if (it == 0)
#pragma unroll
                for (int j = 0; j < 8; ++j) s += A[k][j];
            else
#pragma unroll
                for (int j = 0; j < 8; ++j) s = __builtin_fmaf(A[k][j], w[j], s);
            rs[k] = s;
        }
        row_sum16_x4(rs);
#pragma unroll
        for (int k = 0; k < R; ++k) {
            if (it == 0 && !isfinite(rs[k])) nonfinite = true;
            // max(s, tiny) as a median with the largest float: one instruction (fmaxf would first
            // quiet the value the DPP asm produced); a NaN sum is flagged above. First round:
            // u = 128 / sum_j Y_j^2
            u[k] = it == 0 ? (float)QD * __builtin_amdgcn_rcpf(__builtin_amdgcn_fmed3f(rs[k], TINY, HUGE_F))
                           : __builtin_amdgcn_rcpf(__builtin_amdgcn_fmed3f(rs[k], TINY * (1.0f / QD), HUGE_F));
        }
        // column step: c^2 = mean_i A_ij u_i over the n valid rows
        float t[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int k = 0; k < R; ++k) acc = __builtin_fmaf(A[k][j], u[k], acc);
            t[j] = acc;
        }
        // across the four row groups of the wave: permlane swaps pair up halves
        float h4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(t[j]), __float_as_uint(t[j + 4]), false, false);
            h4[j] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);  // ch j (lanes < 32) / j + 4 (lanes >= 32)
        }
        float h2[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(h4[j]), __float_as_uint(h4[j + 2]), false, false);
            h2[j] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);  // local t = 2 rr + j: channel 32 rr + 2 cc + j
        }
        float(*colsum)[QD] = (it & 1) ? colsum1 : colsum0;
        float *wsh = (it & 1) ? wsh1 : wsh0;
        *reinterpret_cast<float2 *>(&colsum[wave][32 * rr + 2 * cc]) = float2{h2[0], h2[1]};
        lds_barrier();
        if (tid < QD) {
            float acc[NWV / 4];
#pragma unroll
            for (int v = 0; v < NWV / 4; ++v)
                acc[v] = (colsum[4 * v][tid] + colsum[4 * v + 1][tid]) + (colsum[4 * v + 2][tid] + colsum[4 * v + 3][tid]);
            t_own = NWV == 8 ? acc[0] + acc[NWV / 8] : acc[0];
            // a zero column keeps a large finite w (its A entries are all zero)
            if (it + 1 < iters) wsh[tid] = fn_d * __builtin_amdgcn_rcpf(fmaxf(t_own, TINY));
        }
        // the last round's column sums go straight to the normalizer below (no w)
        if (it + 1 == iters) break;
        lds_barrier();
#pragma unroll
        for (int u2 = 0; u2 < 4; ++u2) {
            const float2 wv = *reinterpret_cast<const float2 *>(&wsh[32 * u2 + 2 * cc]);
            w[2 * u2] = wv.x;
            w[2 * u2 + 1] = wv.y;
        }
    }

    // ---- fp16 normalizer c16 (owner threads) and the per-channel multiplier
    // 1 / (sqrt(128) c16); a column whose sum of squares is 0 or not finite keeps c = 1
    constexpr float INV_SQRT_H = 0.08838834764831845f;  // 1 / sqrt(128)
    if (tid < QD) {
        // mean over the n valid rows by a reciprocal of n (exact for a full tile, n a
        // power of two; within an ulp of the quotient otherwise)
        const float csq = (iters > 0 && n > 0 && t_own > 0.f && t_own < INFINITY) ? t_own * __builtin_amdgcn_rcpf(fn) : 1.f;
        const uint16_t c16 = float_to_half_bits(sqrtf(csq));
        const float cv = half_bits_to_float(c16);
        if (!(cv > 0.f && cv < INFINITY)) sideov = true;
        // reciprocal, then one Newton correction of the quotient (Markstein): within an
        // ulp of the rounded quotient
        const float rc = __builtin_amdgcn_rcpf(cv), q0 = INV_SQRT_H * rc;
        multsh[tid] = __builtin_fmaf(__builtin_fmaf(-cv, q0, INV_SQRT_H), rc, q0);
        // thread id made opaque: the store address is formed here, not hoisted out of
        // the item loop (with two caches' addresses held, they would spill, and a spill
        // reload waits for the prefetch in flight)
        int otid = tid;
        asm volatile("" : "+v"(otid));
        a.cnorm[blk * QD + otid] = c16;
    }
    lds_barrier();
    float mult[8];
#pragma unroll
    for (int u2 = 0; u2 < 4; ++u2) {
        const float2 mv = *reinterpret_cast<const float2 *>(&multsh[32 * u2 + 2 * cc]);
        mult[2 * u2] = mv.x;
        mult[2 * u2 + 1] = mv.y;
    }

    // ---- per token: asymmetric RTN with fp16 (S, Z), codes packed in registers
    // channel-major: two byte-accumulators per channel (4-bit: even / odd rows,
    // 2-bit: rows 0..3 in the first), assembled into the channel's bitstream at the end
    static_assert(R == 4, "four rows per lane");
    uint32_t cma[8], cmb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) cma[j] = cmb[j] = 0;
    uint8_t *cbase = reinterpret_cast<uint8_t *>(outbuf);  // LDS image of the code block
    // y -> y / c16 (scaled), in place; row minima and maxima over the 128 channels
    float mnr[R], mxr[R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
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
    // per token: lane cc = k of each row group computes (S16, Z16) of its row rg R + k
    // and writes them; the rows' 1 / S and -Z / S return to the 16 lanes by broadcasts
    // (the other lanes' results are not used)
    float inv4[R], zi4[R];
    bool clamp;
    {
        const float mn = cc == 0 ? mnr[0] : cc == 1 ? mnr[1] : cc == 2 ? mnr[2] : mnr[3];
        const float mx = cc == 0 ? mxr[0] : cc == 1 ? mxr[1] : cc == 2 ? mxr[2] : mxr[3];
        const int row = rg * R + (cc & 3);
        const bool own = cc < 4;
        uint16_t S16 = 0, Z16 = 0;
        if (row < n) {
            S16 = float_to_half_bits((mx - mn) * (1.0f / LEVELS));
            Z16 = float_to_half_bits(mn);
        }
        const float Sv = half_bits_to_float(S16), Zv = half_bits_to_float(Z16);
        if (own && (!(Sv < INFINITY) || !(fabsf(Zv) < INFINITY))) sideov = true;
        const float inv = Sv != 0.f ? __builtin_amdgcn_rcpf(Sv) : 0.f;
        const float zi = -Zv * inv;
        if (own) szbuf[row] = (uint32_t)S16 | ((uint32_t)Z16 << 16);
        // (y - Z) / S; cvt_pk_u8 rounds to nearest even and clamps below at 0. The upper
        // clamp changes a code only for a value at or above LEVELS + 1/2 (below it the
        // rounding gives at most LEVELS), and the map is monotone (inv >= 0), so only when
        // a row's largest value gets there: fp16 rounding of S and Z far larger than
        // usual (an offset much larger than the range), or a non-finite value. It is then
        // applied to the whole wave (it leaves every other code as it is).
        clamp = __ballot(nonfinite || sideov || (own && !(__builtin_fmaf(mx, inv, zi) < LEVELS + 0.5f))) != 0;
        inv4[0] = row_bcast<0>(inv), zi4[0] = row_bcast<0>(zi);
        inv4[1] = row_bcast<1>(inv), zi4[1] = row_bcast<1>(zi);
        inv4[2] = row_bcast<2>(inv), zi4[2] = row_bcast<2>(zi);
        inv4[3] = row_bcast<3>(inv), zi4[3] = row_bcast<3>(zi);
    }
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int row = rg * R + k;
        float q[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) q[j] = __builtin_fmaf(y[k][j], inv4[k], zi4[k]);
        if (clamp)
#pragma unroll
            for (int j = 0; j < 8; ++j) q[j] = fminf(q[j], LEVELS);
        if constexpr (LAYOUT == KVQ_TOKEN_MAJOR) {
            // the lane's channel pairs 32 u + 2 cc + {0, 1}: one byte each (4-bit, the
            // even channel in the low nibble); 2-bit: the pair's nibble, joined with the
            // neighbouring lane's pair (channels 32 u + 2 (cc ^ 1) + {0, 1}) into a byte
#pragma unroll
            for (int u2 = 0; u2 < 4; ++u2) {
                const uint32_t lo = __builtin_amdgcn_cvt_pk_u8_f32(q[2 * u2], 0, 0);
                const uint32_t hi = __builtin_amdgcn_cvt_pk_u8_f32(q[2 * u2 + 1], 0, 0);
                if constexpr (BITS == 4) {
                    cbase[code_byte<T, R, BITS, LAYOUT>(row * (QD / 2) + 16 * u2 + cc)] = (uint8_t)(lo | (hi << 4));
                } else {
                    const uint32_t nib = lo | (hi << 2);
                    const uint32_t nb = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)nib, DPP_QUAD_XOR1, 0xF, 0xF, true);
                    if (!(cc & 1))
                        cbase[code_byte<T, R, BITS, LAYOUT>(row * (QD / 4) + 8 * u2 + (cc >> 1))] = (uint8_t)(nib | (nb << 4));
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if constexpr (BITS == 4) {
                    if (k & 1) cmb[j] = __builtin_amdgcn_cvt_pk_u8_f32(q[j], k >> 1, cmb[j]);
                    else cma[j] = __builtin_amdgcn_cvt_pk_u8_f32(q[j], k >> 1, cma[j]);
                } else {
                    cma[j] = __builtin_amdgcn_cvt_pk_u8_f32(q[j], k, cma[j]);
                }
            }
        }
    }
    if constexpr (LAYOUT == KVQ_CHANNEL_MAJOR) {
        // channel ch: rows rg*R .. rg*R + R - 1 are stream positions ch * T + rg * R + k
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int pos = (32 * (j >> 1) + 2 * cc + (j & 1)) * T + rg * R;
            if constexpr (BITS == 4) {
                *reinterpret_cast<uint16_t *>(cbase + code_byte<T, R, BITS, LAYOUT>(pos / 2)) =
                    (uint16_t)(cma[j] | (cmb[j] << 4));
            } else {  // four byte codes (< 4) -> one byte, LE 2-bit fields
                const uint32_t x = cma[j];
                cbase[code_byte<T, R, BITS, LAYOUT>(pos / 4)] =
                    (uint8_t)((x & 0x03u) | ((x >> 6) & 0x0Cu) | ((x >> 12) & 0x30u) | ((x >> 18) & 0xC0u));
            }
        }
    }
    // ---- coalesced stores of the code block and the (S, Z) words --------------
    lds_barrier();
    {
        constexpr int NW = T * QD * BITS / 32;  // 32-bit words of the code block
        uint4 *gcodes = reinterpret_cast<uint4 *>(a.codes + blk * (T * QD * BITS / 8));
        const uint4 *lcodes = reinterpret_cast<const uint4 *>(outbuf);
        int otid = tid;  // opaque, as for the normalizer store
        asm volatile("" : "+v"(otid));
#pragma unroll
        for (int k = 0; k < (NW / 4 + NT - 1) / NT; ++k) {
            const int i = otid + k * NT;
            if ((NW / 4) % NT == 0 || i < NW / 4) gcodes[i] = lcodes[code_slot<T, R, BITS, LAYOUT>(i)];
        }
        if (otid < T / 4)
            reinterpret_cast<uint4 *>(a.sz + blk * T * 2)[otid] = reinterpret_cast<const uint4 *>(szbuf)[otid];
    }
    if (a.flags) {  // one atomic per wave that saw a condition; no barrier
        const bool nf = __ballot(nonfinite) != 0;
        const bool so = __ballot(sideov) != 0;
        if (lane == 0 && (nf || so))
            atomicOr(a.flags, (nf ? (uint32_t)KVQ_FLAG_NONFINITE : 0u) | (so ? (uint32_t)KVQ_FLAG_SIDE_OVERFLOW : 0u));
    }
    };
    int item = blockIdx.x;
    if (item < num_items) fetch(item);
    for (; item < num_items; item += gridDim.x) {
        if (!PAIR || item < nk) process(IntC<BK>{}, IntC<LK>{}, ak, item, item);
        else process(IntC<BV>{}, IntC<LV>{}, av, item - nk, item);
    }
}

// Four waves per SIMD (the second bound: HIP passes it on as the minimum waves per
// execution unit), so at most 128 registers per lane: two 8-wave workgroups per
// compute unit for 128-token tiles. Every variant fits without spilling (the few
// addresses that would not are recomputed from an opaque lane id where used).
template <int T, int R, int BK, int LK, int BV, int LV, int NIT, bool PAIR>
__global__ void __launch_bounds__(16 * T / R, 4) quantize_d128_kernel(QuantArgs ak, QuantArgs av, int nk, int num_items) {
    constexpr int NWV = T / (4 * R);
    constexpr int MB = BK > BV ? BK : BV;
    __shared__ uint4 stage[T * QD * 2 / 16];
    __shared__ float colsum0[NWV][QD], colsum1[NWV][QD];
    __shared__ float wsh0[QD], wsh1[QD];
    __shared__ float multsh[QD];
    __shared__ uint32_t outbuf[T * QD * MB / 32];
    __shared__ uint32_t szbuf[T];
    __shared__ uint4 hbtab[2 * 64];
    quantize_d128_body<T, R, BK, LK, BV, LV, NIT, PAIR>(ak, av, nk, num_items, stage, colsum0, colsum1, wsh0, wsh1,
                                                        multsh, outbuf, szbuf, hbtab);
}

bool quantize_d128_supported(int D, int T, const QuantArgs &a) {
    // the per-lane source offset (up to 3 token strides) is kept in 32 bits
    return D == QD && (T == 64 || T == 128) && a.h == QD && a.G == QD && a.R == 0 && a.dtype == KVQ_BF16 &&
           a.center == 0 &&
           a.stride_token < (int64_t(1) << 28) &&
           (a.bits == 2 || a.bits == 4) && (a.layout == KVQ_TOKEN_MAJOR || a.layout == KVQ_CHANNEL_MAJOR);
}

static int d128_grid(int items, const void *kernel, int threads) {
    int dev = 0, cus = 256, per_cu = 2;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu < 1) per_cu = 1;
    return items < cus * per_cu ? items : cus * per_cu;
}

template <int T, int BITS, int LAYOUT, int NIT>
static void launch_one(int num_tiles, const QuantArgs &a, hipStream_t stream) {
    constexpr int R = QR;
    constexpr int NT = 16 * T / R;
    const int items = num_tiles * a.H;
    auto kern = quantize_d128_kernel<T, R, BITS, LAYOUT, BITS, LAYOUT, NIT, false>;
    hipLaunchKernelGGL(kern, dim3(d128_grid(items, (const void *)kern, NT)), dim3(NT), 0, stream, a, a, items, items);
}

template <int T, int BITS, int LAYOUT>
static void launch_n(int num_tiles, const QuantArgs &a, hipStream_t stream) {
    if (a.iters == 4) launch_one<T, BITS, LAYOUT, 4>(num_tiles, a, stream);
    else if (a.iters == 2) launch_one<T, BITS, LAYOUT, 2>(num_tiles, a, stream);
    else launch_one<T, BITS, LAYOUT, -1>(num_tiles, a, stream);
}

template <int T, int BITS>
static void launch_l(int num_tiles, const QuantArgs &a, hipStream_t stream) {
    if (a.layout == KVQ_TOKEN_MAJOR) launch_n<T, BITS, KVQ_TOKEN_MAJOR>(num_tiles, a, stream);
    else launch_n<T, BITS, KVQ_CHANNEL_MAJOR>(num_tiles, a, stream);
}

void launch_quantize_d128(int T, int num_tiles, const QuantArgs &a, hipStream_t stream) {
    if (T == 128) {
        if (a.bits == 4) launch_l<128, 4>(num_tiles, a, stream);
        else launch_l<128, 2>(num_tiles, a, stream);
    } else {
        if (a.bits == 4) launch_l<64, 4>(num_tiles, a, stream);
        else launch_l<64, 2>(num_tiles, a, stream);
    }
}

// K (token-major) and V (channel-major) caches of one batch in one launch: same
// tiles, tile size and round count; each cache's own bits
bool quantize_d128_pair_supported(int T, const QuantArgs &k, const QuantArgs &v) {
    return quantize_d128_supported(QD, T, k) && quantize_d128_supported(QD, T, v) && k.layout == KVQ_TOKEN_MAJOR &&
           v.layout == KVQ_CHANNEL_MAJOR && k.iters == v.iters;
}

template <int T, int BK, int BV, int NIT>
static void launch_pair_n(int num_tiles, const QuantArgs &k, const QuantArgs &v, hipStream_t stream) {
    constexpr int R = QR;
    constexpr int NT = 16 * T / R;
    const int nk = num_tiles * k.H, items = nk + num_tiles * v.H;
    auto kern = quantize_d128_kernel<T, R, BK, KVQ_TOKEN_MAJOR, BV, KVQ_CHANNEL_MAJOR, NIT, true>;
    hipLaunchKernelGGL(kern, dim3(d128_grid(items, (const void *)kern, NT)), dim3(NT), 0, stream, k, v, nk, items);
}

template <int T, int BK, int BV>
static void launch_pair_i(int num_tiles, const QuantArgs &k, const QuantArgs &v, hipStream_t stream) {
    if (k.iters == 4) launch_pair_n<T, BK, BV, 4>(num_tiles, k, v, stream);
    else if (k.iters == 2) launch_pair_n<T, BK, BV, 2>(num_tiles, k, v, stream);
    else launch_pair_n<T, BK, BV, -1>(num_tiles, k, v, stream);
}

template <int T>
static void launch_pair_t(int num_tiles, const QuantArgs &k, const QuantArgs &v, hipStream_t stream) {
    if (k.bits == 4) {
        if (v.bits == 4) launch_pair_i<T, 4, 4>(num_tiles, k, v, stream);
        else launch_pair_i<T, 4, 2>(num_tiles, k, v, stream);
    } else {
        if (v.bits == 4) launch_pair_i<T, 2, 4>(num_tiles, k, v, stream);
        else launch_pair_i<T, 2, 2>(num_tiles, k, v, stream);
    }
}

void launch_quantize_d128_pair(int T, int num_tiles, const QuantArgs &k, const QuantArgs &v, hipStream_t stream) {
    if (T == 128) launch_pair_t<128>(num_tiles, k, v, stream);
    else launch_pair_t<64>(num_tiles, k, v, stream);
}

}  // namespace kvq
