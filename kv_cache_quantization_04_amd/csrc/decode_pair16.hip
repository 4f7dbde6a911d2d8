// Split-K decode attention over 16-token pages with up to 8 query heads per kv head
// (gfx950): two pages per matrix-core pass.
//
// The folded evaluation is that of decode_mfma.hip (scores from the codes with the
// per-token scale and zero, the K normalizer folded into the query per page, values
// accumulated per page and scaled by the V normalizer):
//   score_t = sm * ( S_t * [A_K . q']_t + Z_t * sum_j q'_j ),  q' = (q Q) o c_K
//   o'_j   += c_V,j * ( [A_V . P~]_j + sum_t p_t Z_t ),        P~_t = p_t S_V,t
// With g <= 8 query heads per kv head, half of the 16 MFMA columns would be padding,
// and a 16-token page fills only half of the 32-token K-step of the value product.
// Here a wave takes its pages two at a time (A, B): columns 0..7 are the g heads on
// page A, columns 8..15 the same heads on page B, and
//   - the score product runs once per page on that page's codes (two 16-token M-tiles,
//     one per page; every lane folds the query for its own column's page only, so the
//     per-page query fold costs half of a one-page pass), and each column keeps the
//     result of its own page;
//   - the value product takes both pages' 16 tokens as its 32-token K-step, page A's
//     tokens in lanes 0..31 and page B's in lanes 32..63, with P~ zero where a column
//     meets the other page's tokens: one K-step per channel tile serves both pages.
// Columns c and c + 8 are two independent online-softmax streams of one head (the
// wave's even and odd pages); the workgroup merge combines them with the other waves'.
// The next pair's page images are prefetched into registers while a pair is computed
// and written to the wave's two LDS images at the top of the next pair; a wave with an
// odd number of pages ends with page A loaded again as page B, whose tokens are all masked.
#include "common.h"
#include "decode_merge.h"
#include "decode_mfma.h"
#include "launch.h"
#include "xlane.h"

namespace kvq {

// One Walsh-Hadamard stage on channel bit 4 K of a query row held four channels per lane
// (lane u of a 32-lane group holds channels 4 u .. 4 u + 3): the lower member of each
// pair takes own + partner, the upper one partner - own (stages at or above h skipped)
template <int K>
__device__ __forceinline__ void hstage(float (&x)[4], int u, int h) {
    if (4 * K < h) {
        const float sg = (u & K) ? -1.f : 1.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = __builtin_fmaf(sg, x[e], swz_xor<K>(x[e]));
    }
}

// Workgroups take their sequence in order of decreasing page count: grid row z gets the
// sequence of rank z (ties by index). Workgroups are dispatched in grid order, so the
// splits of the longest sequences start in the first rounds and the shortest fill in at
// the end: greedy list scheduling with the longest jobs first, whose tail is at most one
// short job, where the natural order can leave a long sequence's splits for last. Up to
// MNT sequences (one per thread); more keep the natural order. keys: MNT + 4 ints of LDS.
template <int T>
__device__ __forceinline__ int sequence_of_row(const DecodeArgs &a, int z, int *keys) {
    static_assert(MNT == 256, "the split rule assumes ordering up to 256 sequences");
    if (a.B > MNT) return z;
    const int t = threadIdx.x, n4 = (a.B + 3) >> 2;
    int np = 0;
    if (t < a.B) {
        const int L = a.seq_lens[t];
        np = min((L + T - 1) / T, a.bt_stride);  // the page walk's own count
        keys[t] = np;
    } else if (t < 4 * n4) {
        keys[t] = -2147483647 - 1;  // padding: below every page count (which is > INT32_MIN)
    }
    lds_barrier();
    if (t < a.B) {
        int r = 0;
        for (int u4 = 0; u4 < n4; ++u4) {
            const int4 p = *reinterpret_cast<const int4 *>(&keys[4 * u4]);
            const int u = 4 * u4;
            r += (p.x > np || (p.x == np && u < t)) + (p.y > np || (p.y == np && u + 1 < t)) +
                 (p.z > np || (p.z == np && u + 2 < t)) + (p.w > np || (p.w == np && u + 3 < t));
        }
        if (r == z) keys[MNT] = t;  // the ranks are a permutation of 0 .. B - 1
    }
    lds_barrier();
    return __builtin_amdgcn_readfirstlane(keys[MNT]);
}

template <int KB, int VB>
__global__ void __launch_bounds__(MNT, 3) decode_pair16_kernel(DecodeArgs a) {
    constexpr int T = 16;
    using PI = PageImage<T, KB, VB>;
    constexpr int KCB = 32 * KB / 8;  // bytes of one lane's 32-channel K chunk
    // pool: the four waves' two page images during the page walk, the merge after it
    constexpr int RED_O = 4 * 16 * (MD + 1) * 4, RED_BYTES = RED_O + 4 * 16 * 2 * 4;
    constexpr int IMG_BYTES = 4 * 2 * PI::BYTES;
    __shared__ __attribute__((aligned(16))) uint8_t pool[IMG_BYTES > RED_BYTES ? IMG_BYTES : RED_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t wrk[4][2][VB == 3 ? PI::VCW : 16];
    // the rotated query of the (up to 8) heads, then max |qbar| of each head
    __shared__ __attribute__((aligned(16))) float qlds[8 * MD + 8];
    float(*red_o)[16][MD + 1] = reinterpret_cast<float(*)[16][MD + 1]>(pool);
    float(*red_ml)[16][2] = reinterpret_cast<float(*)[16][2]>(pool + RED_O);

    const int tid = threadIdx.x, lane = tid & 63;
    const PageSrc<T, KB, VB> psrc = page_src<T, KB, VB>(a, lane);  // chunk sources of a page image
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint8_t *img0 = pool + wave * 2 * PI::BYTES;  // page A image; page B's follows it
    const int l16 = lane & 15, lq = lane >> 4;
    const int half = l16 >> 3;  // this lane's column: page A (0) or B (1) of the pair
    const int g = a.grp;
    __shared__ __attribute__((aligned(16))) int seq_keys[MNT + 4];
    const int split = blockIdx.x, hk = blockIdx.y, s = sequence_of_row<T>(a, blockIdx.z, seq_keys);
    const int hh = l16 & 7;  // column head
    const bool hv = hh < g;
    const int L = load_const(a.seq_lens, s);
    const int npages = min((L + T - 1) / T, a.bt_stride);
    const int pps = (npages + a.splits - 1) / a.splits;
    const int p0 = split * pps, p1 = min(npages, p0 + pps);

    auto page_of = [&](int q) { return load_const(a.bt, (int64_t)s * a.bt_stride + q); };
    auto next_valid = [&](int q) {  // first valid page >= q of this wave's stride-4 sequence, or p1
        while (q < p1) {
            const int page = page_of(q);
            if (page >= 0 && page < a.num_pages) return q;
            q += 4;
        }
        return p1;
    };

    // The query is rotated once per workgroup: thread t takes head t >> 5 (< g) and its
    // channels 4 (t & 31) .. + 3, whose raw words are loaded before the first pages are
    // requested (the vector-memory counter is in order: waiting for them leaves the
    // page loads in flight).
    // The load is unconditional (threads past the group's g heads read its first head and
    // use zeros below): a load under a divergent condition is waited for where the branch
    // joins, before the page requests.
    const int qh = tid >> 5, qu = tid & 31;
    const bool qok = qh < g;
    uint4 qraw;
    {
        const int64_t qb = ((int64_t)s * a.Hq + hk * g + (qok ? qh : 0)) * MD + 4 * qu;
        if (a.q_dtype == KVQ_F32) qraw = *reinterpret_cast<const uint4 *>(reinterpret_cast<const float *>(a.q) + qb);
        else {
            const uint2 v = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(a.q) + qb);
            qraw = uint4{v.x, v.y, 0, 0};
        }
    }
    asm volatile("" ::: "memory");  // keep the query loads ahead of the page requests
    int pa = next_valid(p0 + wave);
    int pb = pa < p1 ? next_valid(pa + 4) : p1;
    Chunks<PI::NPRE> preA{}, preB{};
    // A missing page B is page A loaded a second time (its tokens are masked): a register
    // copy of page A would wait for A's loads where it is made.
    if (pa < p1) {
        preA = fetch_page(psrc, (uint32_t)(page_of(pa) * a.Hkv + hk));
        preB = fetch_page(psrc, (uint32_t)(page_of(pb < p1 ? pb : pa) * a.Hkv + hk));
        wait_vm_upto<2 * PI::NPRE>();
    } else {
        wait_vm_upto<0>();
    }

    // ---- rotated query, once per workgroup: the Walsh-Hadamard butterflies on channel
    // bits 0 and 1 run in registers, bits 2..6 across the head's 32 lanes (xor swizzles
    // in groups of 32); blocks of h channels rotate separately
    {
        float x[4];
        if (a.q_dtype == KVQ_F32) {
            x[0] = __uint_as_float(qraw.x); x[1] = __uint_as_float(qraw.y);
            x[2] = __uint_as_float(qraw.z); x[3] = __uint_as_float(qraw.w);
        } else if (a.q_dtype == KVQ_BF16) {
            x[0] = __uint_as_float(qraw.x << 16); x[1] = __uint_as_float(qraw.x & 0xffff0000u);
            x[2] = __uint_as_float(qraw.y << 16); x[3] = __uint_as_float(qraw.y & 0xffff0000u);
        } else {
            x[0] = half_bits_to_float(qraw.x & 0xffffu); x[1] = half_bits_to_float(qraw.x >> 16);
            x[2] = half_bits_to_float(qraw.y & 0xffffu); x[3] = half_bits_to_float(qraw.y >> 16);
        }
        if (!qok) x[0] = x[1] = x[2] = x[3] = 0.f;
        if (1 < a.kh) {
            const float y0 = x[0], y2 = x[2];
            x[0] = y0 + x[1]; x[1] = y0 - x[1];
            x[2] = y2 + x[3]; x[3] = y2 - x[3];
        }
        if (2 < a.kh) {
            const float y0 = x[0], y1 = x[1];
            x[0] = y0 + x[2]; x[2] = y0 - x[2];
            x[1] = y1 + x[3]; x[3] = y1 - x[3];
        }
        hstage<1>(x, qu, a.kh);
        hstage<2>(x, qu, a.kh);
        hstage<4>(x, qu, a.kh);
        hstage<8>(x, qu, a.kh);
        hstage<16>(x, qu, a.kh);
        const float qscale = 1.0f / sqrtf((float)a.kh);
        float m = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] *= qscale;
            m = fmaxf(m, fabsf(x[e]));
        }
        m = fmaxf(m, swz_xor<1>(m));
        m = fmaxf(m, swz_xor<2>(m));
        m = fmaxf(m, swz_xor<4>(m));
        m = fmaxf(m, swz_xor<8>(m));
        m = fmaxf(m, swz_xor<16>(m));
        *reinterpret_cast<float4 *>(&qlds[qh * MD + 4 * qu]) = float4{x[0], x[1], x[2], x[3]};
        if (qu == 0) qlds[8 * MD + qh] = m;
    }
    lds_barrier();  // the page loads stay in flight
    // lane (column l16, chunk lq), K-step st covers channels lq*32 + st*8 + e(kk): columns
    // of both halves hold the same head; max |qbar| of the lane's head (all 128 channels)
    // with the page's largest c_K bounds max |q'|, which sets the power-of-two scaling of
    // the query fold
    float qv[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 v = *reinterpret_cast<const float4 *>(&qlds[hh * MD + lq * 32 + 4 * i]);
        qv[4 * i] = v.x; qv[4 * i + 1] = v.y; qv[4 * i + 2] = v.z; qv[4 * i + 3] = v.w;
    }
    const float qvmax = qlds[8 * MD + hh];

    const float sml2 = a.sm * 1.4426950408889634f;  // scores in log2 units
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[8];
#pragma unroll
    for (int mc = 0; mc < 8; ++mc) o[mc] = f32x4{0.f, 0.f, 0.f, 0.f};

    // score rows 4 lq .. + 3 hold tokens tok0 .. + 3 of the column's page; the A operand
    // row l16 of an M-tile is token ktok of its page (the order that makes the score
    // tile the value product's B operand without a transpose)
    const int tok0 = 8 * (lq & 1) + 4 * (lq >> 1);
    // P~ operand selectors (byte permutes of the swapped pairs): the low halves, or the
    // high halves, of both words; all zero for the other page's tokens
    const bool pact = (lq >> 1) == half;
    const uint32_t psel_h = pact ? 0x01000504u : 0x0C0C0C0Cu, psel_l = pact ? 0x03020706u : 0x0C0C0C0Cu;
    const int ktok = 8 * ((l16 >> 2) & 1) + 4 * (l16 >> 3) + (l16 & 3);

    while (pa < p1) {
        const int curA = pa, curB = pb;  // curB == p1: no page B (its copy of A is masked)
        pa = curB < p1 ? next_valid(curB + 4) : p1;
        pb = pa < p1 ? next_valid(pa + 4) : p1;
        // registers -> the wave's two LDS images (LDS operations of a wave stay in order)
#pragma unroll
        for (int k = 0; k < PI::NPRE; ++k) {
            const int off = 1024 * k + 16 * lane;
            if (off < PI::BYTES) {
                *reinterpret_cast<uint4 *>(&img0[off]) = preA.v[k];
                *reinterpret_cast<uint4 *>(&img0[PI::BYTES + off]) = preB.v[k];
            }
        }
        if constexpr (VB == 3) {  // four 3-byte chunks per lane -> four words, each page
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int c4 = lane; c4 < MD * (T / 8) / 4; c4 += 64) {
                    const uint32_t *sw = reinterpret_cast<const uint32_t *>(&img0[h2 * PI::BYTES + PI::O_VC + 12 * c4]);
                    const uint32_t w0 = sw[0], w1 = sw[1], w2 = sw[2];
                    const uint4 r = {w0 & 0xFFFFFFu, (w0 >> 24) | ((w1 & 0xFFFFu) << 8),
                                     (w1 >> 16) | ((w2 & 0xFFu) << 16), w2 >> 8};
                    *reinterpret_cast<uint4 *>(&wrk[wave][h2][16 * c4]) = r;
                }
        }
        // valid tokens of this lane's column page (0: the missing page B)
        const int rows = half ? (curB < p1 ? min(T, L - curB * T) : 0) : min(T, L - curA * T);
        const uint8_t *own = img0 + half * PI::BYTES;  // the column's page image

        // K code words of token ktok on both pages (A-operand rows)
        uint32_t kw[2][KB];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const uint8_t *row = img0 + h2 * PI::BYTES + PI::O_KC + ktok * (MD * KB / 8) + lq * KCB;
#pragma unroll
            for (int i = 0; i < KB; ++i) kw[h2][i] = reinterpret_cast<const uint32_t *>(row)[i];
        }
        // q' = qbar o c_K for the column's page (c_K of the lane's 32 channels), scaled by
        // 2^sq so that the bound max |qbar| max c_K lands in [2^14, 2^15), as fp16 hi + lo;
        // sum_j q'_j accumulates on the way. The normalizers are >= 0: their largest is the
        // largest fp16 bit pattern (packed u16 maxima).
        const uint4 *cp = reinterpret_cast<const uint4 *>(&own[PI::O_KCN + 64 * lq]);
        float cmax;
        {
            u16x2 m = {0, 0};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const uint4 v = cp[st];
                m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, v.x));
                m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, v.y));
                m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, v.z));
                m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, v.w));
            }
            cmax = xlane_max_q(half_bits_to_float(m.x > m.y ? m.x : m.y));
        }
        const float qsc = pow2_scale_for(qvmax * cmax);
        const float qinv = pow2_over<CODE_EXP<KB>>(qsc);
        float qc = 0.f;
        half8 qhi[4], qlo[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            uint4 v = cp[st];
            asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));  // re-read: not held from the maximum
            const uint32_t cw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const int e = (kk >> 1) + 4 * (kk & 1);
                const half2v c2 = as_h2(cw[e >> 1]);
                const float x = mul_h((e & 1) ? c2.y : c2.x, qv[st * 8 + e]);
                qc += x;
                _Float16 hi, lo;
                split_prod(x, qsc, hi, lo);
                qhi[st][kk] = hi;
                qlo[st][kk] = lo;
            }
        }
        qc = xlane_sum_q(qc);

        // ---- scores: one MFMA chain per page; each column keeps its own page's
        f32x4 scp[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const int bit = st * 8 * KB;
                uint32_t bitsv;
                if (bit % 32 == 0) bitsv = kw[h2][bit / 32];
                else
                    bitsv = __builtin_amdgcn_alignbit(kw[h2][bit / 32 + 1 < KB ? bit / 32 + 1 : bit / 32],
                                                      kw[h2][bit / 32], bit % 32);
                const half8 ak = unpack8<KB>(bitsv);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, qhi[st], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, qlo[st], acc, 0, 0, 0);
            }
            scp[h2] = acc;
        }
        f32x4 sc;
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = half ? scp[1][i] : scp[0][i];
        // the next pair travels during the softmax and the value product (issued here,
        // after the query fold, so that its registers are not live across the fold)
        if (pa < p1) {
            preA = fetch_page(psrc, (uint32_t)(page_of(pa) * a.Hkv + hk));
            preB = fetch_page(psrc, (uint32_t)(page_of(pb < p1 ? pb : pa) * a.Hkv + hk));
        }

        // ---- online softmax over the column's page
        const float a_s = sml2 * qinv, a_z = sml2 * qc;
        float pmax = -INFINITY;
        const uint4 kz = *reinterpret_cast<const uint4 *>(&own[PI::O_KSZ + 4 * tok0]);
        const uint4 vzq = *reinterpret_cast<const uint4 *>(&own[PI::O_VSZ + 4 * tok0]);
        {
            const uint32_t kzw[4] = {kz.x, kz.y, kz.z, kz.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const half2v sz = as_h2(kzw[i]);  // (S, Z)
                float x = __builtin_fmaf((float)sz.x, a_s * sc[i], mul_h(sz.y, a_z));
                if (tok0 + i >= rows) x = -INFINITY;
                sc[i] = x;
                pmax = fmaxf(pmax, x);
            }
        }
        pmax = xlane_max_q(pmax);
        // a column may see no valid token on this pass (the missing page B): exponents
        // against 0 then give alpha = 0 and p = 0, and its running maximum stays
        float m_new = fmaxf(m_run, pmax);
        m_new = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = exp2_fast(m_run - m_new);
        const bool rescale = __builtin_amdgcn_ballot_w64(alpha != 1.f) != 0;
        m_run = fmaxf(m_run, pmax);
        uint32_t smaxw = 0;
        const uint32_t vzw[4] = {vzq.x, vzq.y, vzq.z, vzq.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            smaxw = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, smaxw),
                                                                           __builtin_bit_cast(u16x2, vzw[i])));
        const float smax = half_bits_to_float(smaxw & 0x7fffu);
        const float psc = pow2_scale_for(xlane_max_q(smax));
        const float m_ps = m_new - (float)((int)(__float_as_uint(psc) >> 23) - 127);
        const float pscinv = pow2_over<0>(psc);
        float psum = 0.f, zs = 0.f;
        _Float16 phi[4], plo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const half2v sz = as_h2(vzw[i]);  // (S_V, Z_V)
            const float ps = exp2_fast(sc[i] - m_ps);
            psum += ps;
            zs = __builtin_fmaf((float)sz.y, ps, zs);
            split_prod(ps, (float)sz.x, phi[i], plo[i]);
        }
        const float pinv = pow2_over<CODE_EXP<VB>>(psc);
        l_run = __builtin_fmaf(l_run, alpha, psum * pscinv);
        zs = xlane_sum_q(zs) * pscinv;

        // ---- P~ as the B operand of the value product: K-step token 8 lq + e(kk) is token
        // 8 (lq & 1) + e of page lq >> 1; a column's values enter only on its own page.
        // The lane holds 4 of the 8 tokens (e < 4 when lq < 2, e >= 4 when lq >= 2); the
        // other 4 come from lane ^ 32
        half8 pbh, pbl;
        {
            // the partner's (hi, lo) pair, 32 lanes apart, by one permlane swap of the packed
            // pair; the swap leaves the lower lane's pair in its first result and the upper
            // lane's in its second, so one byte permute per word puts the two hi (lo) parts
            // in token order on both sides (selectors fixed per lane, zero off the page)
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const half2v mine = {phi[i], plo[i]};
                const auto sw = __builtin_amdgcn_permlane32_swap(as_u(mine), as_u(mine), false, false);
                hw[i] = __builtin_amdgcn_perm(sw[0], sw[1], psel_h);
                lw[i] = __builtin_amdgcn_perm(sw[0], sw[1], psel_l);
            }
            pbh = __builtin_bit_cast(half8, uint4{hw[0], hw[1], hw[2], hw[3]});
            pbl = __builtin_bit_cast(half8, uint4{lw[0], lw[1], lw[2], lw[3]});
        }

        // ---- values: channel tiles mc; lane (channel 16 mc + l16, page lq >> 1, tokens
        // 8 (lq & 1) ..); output lane (column l16, channels 16 mc + 4 lq + i)
        const uint8_t *vimg = img0 + (lq >> 1) * PI::BYTES;
        const uint8_t *vbase = VB == 3 ? &wrk[wave][lq >> 1][0] : &vimg[PI::O_VC];
        const uint16_t *vcn = reinterpret_cast<const uint16_t *>(&own[PI::O_VCN]);
        if (rescale)
#pragma unroll
            for (int mc = 0; mc < 8; ++mc)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[mc][i] *= alpha;
#pragma unroll
        for (int mc = 0; mc < 8; ++mc) {
            const int ch = 16 * mc + l16;
            const int64_t bit0 = ((int64_t)ch * T + 8 * (lq & 1)) * VB;
            uint32_t bitsv;
            if constexpr (VB == 4) bitsv = reinterpret_cast<const uint32_t *>(vbase)[bit0 >> 5];
            else if constexpr (VB == 2) bitsv = reinterpret_cast<const uint16_t *>(vbase)[bit0 >> 4];
            else bitsv = reinterpret_cast<const uint32_t *>(vbase)[bit0 / 24];  // re-aligned
            const half8 av = unpack8<VB>(bitsv);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pbh, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pbl, acc, 0, 0, 0);
            const uint2 cv2 = *reinterpret_cast<const uint2 *>(vcn + 16 * mc + 4 * lq);
            const half2v c01 = as_h2(cv2.x), c23 = as_h2(cv2.y);
            const _Float16 cvv[4] = {c01.x, c01.y, c23.x, c23.y};
#pragma unroll
            for (int i = 0; i < 4; ++i) o[mc][i] = __builtin_fmaf((float)cvv[i], __builtin_fmaf(acc[i], pinv, zs), o[mc][i]);
        }
    }

    // ---- merge the eight streams of each head (four waves x two column halves), write
    // the split partial (m, l in log2 units -> natural)
    l_run = xlane_sum_q(l_run);
    __syncthreads();  // the merge buffers overlay the page images
    if (lq == 0) {
        red_ml[wave][l16][0] = m_run;
        red_ml[wave][l16][1] = l_run;
    }
#pragma unroll
    for (int mc = 0; mc < 8; ++mc)
#pragma unroll
        for (int i = 0; i < 4; ++i) red_o[wave][l16][16 * mc + 4 * lq + i] = o[mc][i];
    __syncthreads();
    for (int e = tid; e < g * MD; e += MNT) {
        const int cc = e / MD, j = e % MD;
        const int64_t wrow = (int64_t)s * a.Hq + hk * g + cc;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, fmaxf(red_ml[w][cc][0], red_ml[w][cc + 8][0]));
        float acc = 0.f, lsum = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int col = cc + 8 * h2;
                const float mw = red_ml[w][col][0];
                if (mw != -INFINITY) {
                    const float f = exp2_fast(mw - M);
                    acc = __builtin_fmaf(f, red_o[w][col][j], acc);
                    lsum = __builtin_fmaf(f, red_ml[w][col][1], lsum);
                }
            }
        float *wsr = a.ws + (wrow * a.splits + split) * (MD + 2);
        // device-coherent stores when the last workgroup of the unit reads them
        auto put = [&](int i, float v) {
            if (a.cnt) store_dev(wsr + i, v);
            else wsr[i] = v;
        };
        put(j, acc);
        if (j == 0) {
            put(MD, M == -INFINITY ? -INFINITY : M * 0.6931471805599453f);
            put(MD + 1, lsum);
        }
    }
    static_assert(sizeof(pool) >= 4 * RED_MAX_SPLITS * sizeof(float), "merge weights fit the pool");
    if (a.cnt) merge_if_last<MNT, MD / 64>(a, s, hk, reinterpret_cast<float *>(pool));
}

bool decode_mfma_supported(const DecodeArgs &a);

// decode (not chunked prefill) over 16-token pages with at most 8 query heads per kv head
bool decode_pair16_supported(const DecodeArgs &a) {
    return a.T == 16 && a.Lq == 0 && a.grp <= 8 && decode_mfma_supported(a);
}

bool launch_decode_pair16(const DecodeArgs &a, hipStream_t stream) {
    const dim3 grid(a.splits, a.Hkv, a.B);
#define KVQ_P16(KB_, VB_) \
    hipLaunchKernelGGL((decode_pair16_kernel<KB_, VB_>), grid, dim3(MNT), 0, stream, a)
    switch (a.kbits * 8 + a.vbits) {
    case 2 * 8 + 2: KVQ_P16(2, 2); return true;
    case 2 * 8 + 3: KVQ_P16(2, 3); return true;
    case 2 * 8 + 4: KVQ_P16(2, 4); return true;
    case 3 * 8 + 2: KVQ_P16(3, 2); return true;
    case 3 * 8 + 3: KVQ_P16(3, 3); return true;
    case 3 * 8 + 4: KVQ_P16(3, 4); return true;
    case 4 * 8 + 2: KVQ_P16(4, 2); return true;
    case 4 * 8 + 3: KVQ_P16(4, 3); return true;
    case 4 * 8 + 4: KVQ_P16(4, 4); return true;
    }
#undef KVQ_P16
    return false;
}

}  // namespace kvq
