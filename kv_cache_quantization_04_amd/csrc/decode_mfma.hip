// Split-K decode attention over the paged quantized cache with MFMA (gfx950),
// head_dim 128, grouped-query attention with up to 16 query heads per kv head.
//
// Scores and value accumulation are dense contractions per page:
//   scores^T [tokens x heads]  = A_K [tokens x channels] . qbar^T [channels x heads]
//   o'^T     [channels x heads] = A_V [channels x tokens] . P~^T [tokens x heads]
// run as v_mfma_f32_16x16x32_f16 tiles with fp32 accumulation. The codes enter
// exactly: code n becomes the fp16 subnormal n 2^-(14+b), which the matrix cores
// take as is (the power of two goes into the fp32 scale factors); the
// K normalizer is folded into the query per page, q'_j = qbar_j c_K,j in fp32.
// Query and probability operands are split into fp16 hi + lo parts (two MFMAs
// each), about 22 significant bits, after a per-page power-of-two scaling that
// puts their largest value near 2^14 (clear of fp16 overflow, and of the
// subnormal range where lo would lose bits).
//   score_t = sm * ( S_t * [A_K . q']_t + Z_t * sum_j q'_j )
//   o'_j   += c_V,j * ( [A_V . P~]_j + sum_t p_t Z_t ),  P~_t = p_t S_t
// Each wave walks its own pages (online softmax per wave); the four waves of a
// workgroup merge before writing the split partial. Token order inside a page
// is permuted so that the score tile of two 16-token M-tiles lands, lane for
// lane, in the layout of the 32-token operand of the value product.
//
// Chunked prefill (PF) runs the same kernel with the 16 MFMA columns holding
// (query position, head) pairs, 16 / g consecutive positions of one kv head's g
// query heads, each column with its own causal length: one page read serves
// 16 / g positions and no column is padding. Workgroups that share pages (the
// column blocks of one sequence, kv head and split) are given consecutive ids
// on one XCD, so the repeated page reads hit that XCD's L2.
//
// Page staging by page size: 16-token pages are prefetched into registers one page
// ahead; 64- and 128-token pages are copied whole into a per-wave LDS image by
// direct-to-LDS loads (V codes last, waited for only before the value product),
// and with long splits (DB) into two alternating images, the next page's copies
// travelling while the current page is computed.
#include "common.h"
#include "decode_merge.h"
#include "decode_mfma.h"
#include "launch.h"

namespace kvq {

// One Walsh-Hadamard stage on channel bit 3 + log2 K of a query row held eight channels
// per lane (lane u of a 16-lane group holds channels 8 u .. 8 u + 7): the lower member
// of each pair takes own + partner, the upper one partner - own (stages at or above h
// skipped)
template <int K>
__device__ __forceinline__ void qstage(float (&x)[8], int u, int h) {
    if (8 * K < h) {
        const float sg = (u & K) ? -1.f : 1.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = __builtin_fmaf(sg, x[e], swz_xor<K>(x[e]));
    }
}

template <int T, int KB, int VB, bool PF, bool DB>
__global__ void __launch_bounds__(MNT) decode_mfma_kernel(DecodeArgs a) {
    constexpr int MT = T / 16;                 // 16-token M-tiles of the score product
    constexpr int KSV = T >= 32 ? T / 32 : 1;  // 32-token K-steps of the value product
    constexpr int KCB = 32 * KB / 8;           // bytes of one lane's 32-channel K chunk
    // 16-token pages are staged: each lane loads its share of the wave's next page into
    // registers while the current page is processed from the wave's LDS image (`stg`,
    // plus `wrk` for re-aligned 3-bit V codes).
    constexpr bool STAGED = T == 16;
    // Pages of 64 and 128 tokens are copied whole (codes, side data, normalizers) into
    // the wave's LDS image by direct-to-LDS loads at the top of the page: one HBM round
    // trip per page instead of one per tile of codes and side data.
    constexpr bool IMG = T >= 64;
    constexpr bool LDSPAGE = STAGED || IMG;
    // DB (whole-page images, several pages per wave): two images per wave; the copies of
    // the wave's next page travel while the current page is computed. The two images
    // are separate LDS arrays and the page loop is unrolled by two, so each LDS read
    // provably misses the copies in flight (no wait for them is inserted).
    static_assert(!DB || (IMG && !PF), "double-buffered images: decode, pages of 64 or 128 tokens");
    using PI = PageImage<T, KB, VB>;
    // One pool: the four waves' page images during the page walk, the split merge after
    // it (a barrier separates the two uses).
    constexpr int RED_O = 4 * 16 * (MD + 1) * 4, RED_BYTES = RED_O + 4 * 16 * 2 * 4;
    constexpr int IMG_BYTES = LDSPAGE ? 4 * PI::BYTES : 0;
    __shared__ __attribute__((aligned(16))) uint8_t pool[IMG_BYTES > RED_BYTES ? IMG_BYTES : RED_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t pool2[DB ? 4 * PI::BYTES : 16];
    __shared__ __attribute__((aligned(16))) uint8_t wrk[4][STAGED ? PI::VCW : 16];
    // the rotated query of the workgroup's 16 columns (row stride padded against bank
    // conflicts); with two images per wave it borrows the second ones, which receive
    // nothing before the page walk
    constexpr int QLD = MD + 4;
    static_assert(!DB || 4 * PI::BYTES >= 16 * QLD * 4, "query rows fit the second images");
    __shared__ __attribute__((aligned(16))) float qlds_own[DB ? 4 : 16 * QLD];
    float *qlds = DB ? reinterpret_cast<float *>(pool2) : qlds_own;
    float(*red_o)[16][MD + 1] = reinterpret_cast<float(*)[16][MD + 1]>(pool);
    float(*red_ml)[16][2] = reinterpret_cast<float(*)[16][2]>(pool + RED_O);

    const int tid = threadIdx.x, lane = tid & 63;
    const PageSrc<T, KB, VB> psrc = page_src<T, KB, VB>(a, lane);  // staged path: chunk sources
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint8_t *stg = pool + wave * (LDSPAGE ? PI::BYTES : 0);  // this wave's page image
    uint8_t *stg2 = pool2 + wave * (DB ? PI::BYTES : 0);     // its second image (DB)
    const int l16 = lane & 15, lq = lane >> 4;
    const int g = a.grp;
    int split, hk, s, cb = 0;
    if constexpr (PF) {
        // work item n = ((s * Hkv + hk) * splits + split) * ncb + cb; XCD x (= id mod 8
        // under round-robin dispatch) takes items x * chunk .. in id order
        const int ncb = (a.Lq * g + 15) / 16;
        const int64_t W = (int64_t)a.B * a.Hkv * a.splits * ncb, chunk = (W + 7) / 8;
        const int64_t n = (int64_t)(blockIdx.x & 7) * chunk + (blockIdx.x >> 3);
        if (n >= W) return;  // whole workgroup, before any barrier
        cb = (int)(n % ncb);
        int64_t t = n / ncb;
        split = (int)(t % a.splits);
        t /= a.splits;
        hk = (int)(t % a.Hkv);
        s = (int)(t / a.Hkv);
    } else {
        split = blockIdx.x;
        hk = blockIdx.y;
        s = blockIdx.z;
    }
    // column l16: decode, query head hk g + l16 (l16 < g); prefill, position
    // pos = cb (16 / g) + l16 / g of the chunk and query head hk g + l16 mod g
    const int ppb = PF ? 16 / g : 1;
    const int pos = PF ? cb * ppb + l16 / g : 0;
    const int hh = PF ? l16 - (l16 / g) * g : l16;
    const bool hv = PF ? pos < a.Lq : l16 < g;
    const int Ls = load_const(a.seq_lens, s);
    // tokens the workgroup attends (the longest column) and this lane's column
    const int L = PF ? max(0, Ls - a.Lq + min(a.Lq, (cb + 1) * ppb)) : Ls;
    const int Lc = PF ? (hv ? Ls - a.Lq + pos + 1 : 0) : Ls;
    const int npages = min((L + T - 1) / T, a.bt_stride);
    const int pps = (npages + a.splits - 1) / a.splits;
    const int p0 = split * pps, p1 = min(npages, p0 + pps);

    auto page_of = [&](int q) { return load_const(a.bt, (int64_t)s * a.bt_stride + q); };
    auto valid = [&](int q) {
        const int page = page_of(q);
        return page >= 0 && page < a.num_pages;
    };
    // The query rows are loaded before the first page is requested: the vector-memory
    // counter is in order, so waiting for the query then leaves the page's loads in
    // flight while the query is converted and rotated. The workgroup rotates each of
    // its 16 columns once (all four waves read the same columns): thread t holds
    // channels 8 (t mod 16) .. + 7 of column t / 16.
    const int qcol = tid >> 4, qu = tid & 15;
    uint4 qraw[2];
    const int qpos = PF ? cb * ppb + qcol / g : 0;
    const bool qok = PF ? qpos < a.Lq : qcol < g;
    {
        const int qhh = PF ? qcol - (qcol / g) * g : qcol;
        const int64_t qrow = PF ? (int64_t)s * a.Lq + (qok ? qpos : 0) : s;
        const int64_t qb = (qrow * a.Hq + hk * g + (qok ? qhh : 0)) * MD + 8 * qu;
        if (a.q_dtype == KVQ_F32) {
            const uint4 *p4 = reinterpret_cast<const uint4 *>(reinterpret_cast<const float *>(a.q) + qb);
            qraw[0] = p4[0];
            qraw[1] = p4[1];
        } else {
            qraw[0] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(a.q) + qb);
            qraw[1] = uint4{0, 0, 0, 0};
        }
    }
    asm volatile("" ::: "memory");  // keep the query loads ahead of the page requests
    // staged path: the next page's image chunks, in registers
    Chunks<STAGED ? PI::NPRE : 1> pre{};
    int pi = p0 + wave;
    while (pi < p1 && !valid(pi)) pi += 4;
    // (each path waits for the query loads itself, leaving the page's loads in flight:
    // the compiler cannot count the outstanding loads past a conditional request)
    if constexpr (STAGED) {
        if (pi < p1) {
            pre = fetch_page(psrc, (uint32_t)(page_of(pi) * a.Hkv + hk));
            wait_vm_upto<PI::NPRE>();
        } else {
            wait_vm_upto<0>();
        }
    }
    // whole-page images: the copies of the wave's first page travel while the query
    // is loaded and rotated
    auto copy_page = [&](int64_t kblk, uint8_t *__restrict__ dst) {
        if constexpr (IMG) {
        copy_region<PI::KC>(a.kcodes + kblk * PI::KC, dst + PI::O_KC, lane);
        copy_region<PI::SZ>(reinterpret_cast<const uint8_t *>(a.ksz) + kblk * PI::SZ, dst + PI::O_KSZ, lane);
        copy_region<PI::CN>(reinterpret_cast<const uint8_t *>(a.kcn) + kblk * PI::CN, dst + PI::O_KCN, lane);
        // V codes last: the scores need everything else, the value product these
        copy_region<PI::SZ>(reinterpret_cast<const uint8_t *>(a.vsz) + kblk * PI::SZ, dst + PI::O_VSZ, lane);
        copy_region<PI::CN>(reinterpret_cast<const uint8_t *>(a.vcn) + kblk * PI::CN, dst + PI::O_VCN, lane);
        copy_region<PI::VC>(a.vcodes + kblk * PI::VC, dst + PI::O_VC, lane);
        }
    };
    const int first = pi;
    if constexpr (IMG) {
        if (pi < p1) {
            copy_page((int64_t)page_of(pi) * a.Hkv + hk, stg);
            wait_vm_upto<2 * copy_instrs<PI::SZ>() + 2 * copy_instrs<PI::CN>() + copy_instrs<PI::KC>() +
                         copy_instrs<PI::VC>()>();
        } else {
            wait_vm_upto<0>();
        }
    }

    // ---- rotated query qbar = q Q / sqrt(h), once per workgroup: the Walsh-Hadamard
    // butterflies on channel bits 0..2 run in registers, bits 3..6 across the column's
    // 16 lanes (xor swizzles); blocks of h channels rotate separately. Columns without a
    // query (no head, or past the chunk) are zero.
    {
        float x[8];
        if (a.q_dtype == KVQ_F32) {
            x[0] = __uint_as_float(qraw[0].x); x[1] = __uint_as_float(qraw[0].y);
            x[2] = __uint_as_float(qraw[0].z); x[3] = __uint_as_float(qraw[0].w);
            x[4] = __uint_as_float(qraw[1].x); x[5] = __uint_as_float(qraw[1].y);
            x[6] = __uint_as_float(qraw[1].z); x[7] = __uint_as_float(qraw[1].w);
        } else {
            const uint32_t w[4] = {qraw[0].x, qraw[0].y, qraw[0].z, qraw[0].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (a.q_dtype == KVQ_BF16) {
                    x[2 * k] = __uint_as_float(w[k] << 16);
                    x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
                } else {
                    x[2 * k] = half_bits_to_float(w[k] & 0xffffu);
                    x[2 * k + 1] = half_bits_to_float(w[k] >> 16);
                }
            }
        }
        if (!qok)
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = 0.f;
#pragma unroll
        for (int b = 1; b < 8; b <<= 1)
            if (b < a.kh)
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    if (!(i & b)) {
                        const float y0 = x[i], y1 = x[i | b];
                        x[i] = y0 + y1;
                        x[i | b] = y0 - y1;
                    }
        qstage<1>(x, qu, a.kh);
        qstage<2>(x, qu, a.kh);
        qstage<4>(x, qu, a.kh);
        qstage<8>(x, qu, a.kh);
        const float qscale = 1.0f / sqrtf((float)a.kh);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= qscale;
        float *qd = &qlds[qcol * QLD + 8 * qu];
        *reinterpret_cast<float4 *>(qd) = float4{x[0], x[1], x[2], x[3]};
        *reinterpret_cast<float4 *>(qd + 4) = float4{x[4], x[5], x[6], x[7]};
    }
    lds_barrier();  // the page loads stay in flight
    // B-operand layout: lane (column l16, chunk lq), K-step st covers channels
    // lq*32 + st*8 + e(kk); qv[st*8 + e] = qbar[lq*32 + st*8 + e]
    float qv[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 v = *reinterpret_cast<const float4 *>(&qlds[l16 * QLD + lq * 32 + 4 * i]);
        qv[4 * i] = v.x; qv[4 * i + 1] = v.y; qv[4 * i + 2] = v.z; qv[4 * i + 3] = v.w;
    }
    if constexpr (DB) lds_barrier();  // every wave has its rows before the next pages' copies land

    const float sml2 = a.sm * 1.4426950408889634f;  // scores in log2 units
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[8];
#pragma unroll
    for (int mc = 0; mc < 8; ++mc) o[mc] = f32x4{0.f, 0.f, 0.f, 0.f};

    // one page: `img` holds it (whole-page images), `nimg` receives the next (DB)
    auto page_step = [&](uint8_t *__restrict__ img, uint8_t *__restrict__ nimg) {
        const int cur = pi;
        const int page = page_of(cur);
        pi += 4;
        while (pi < p1 && !valid(pi)) pi += 4;
        if constexpr (STAGED) {
            // registers -> this wave's LDS image (LDS operations of a wave stay in order)
#pragma unroll
            for (int k = 0; k < PI::NPRE; ++k) {
                const int off = 1024 * k + 16 * lane;
                if (off < PI::BYTES) *reinterpret_cast<uint4 *>(&img[off]) = pre.v[k];
            }
            if constexpr (VB == 3) {  // four 3-byte chunks per lane -> four words
#pragma unroll
                for (int c4 = lane; c4 < MD * (T / 8) / 4; c4 += 64) {
                    const uint32_t *sw = reinterpret_cast<const uint32_t *>(&img[PI::O_VC + 12 * c4]);
                    const uint32_t w0 = sw[0], w1 = sw[1], w2 = sw[2];
                    const uint4 r = {w0 & 0xFFFFFFu, (w0 >> 24) | ((w1 & 0xFFFFu) << 8), (w1 >> 16) | ((w2 & 0xFFu) << 16),
                                     w2 >> 8};
                    *reinterpret_cast<uint4 *>(&wrk[wave][16 * c4]) = r;
                }
            }
            if (pi < p1) pre = fetch_page(psrc, (uint32_t)(page_of(pi) * a.Hkv + hk));  // travels meanwhile
        }
        const int rows = min(T, Lc - cur * T);  // valid tokens of this column (may be <= 0 in PF)
        const int64_t kblk = (int64_t)page * a.Hkv + hk;
        if constexpr (DB) {
            __builtin_amdgcn_s_waitcnt(0);  // this page's copies, issued one page earlier, have landed
            if (pi < p1) {
                // the other image's LDS reads (the previous page) have returned; make sure
                // before the copies overwrite it
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                copy_page((int64_t)page_of(pi) * a.Hkv + hk, nimg);
            }
        } else if constexpr (IMG) {
            if (cur != first) {
                // the previous page's LDS reads have returned (their values were consumed);
                // make sure before the copies overwrite the image
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                copy_page(kblk, img);
            }
            // all but the V code copies have landed (in order; the wave alone reads its
            // image): the scores run while the V codes travel
            wait_vm_upto<copy_instrs<PI::VC>()>();
        }
        // the page's K code words of every M-tile, issued now so that they travel
        // while the query is folded (a page in HBM, not staged)
        const uint8_t *kbase = LDSPAGE ? &img[PI::O_KC] : a.kcodes + kblk * (T * MD * KB / 8);
        uint32_t kpre[MT][KB];
#pragma unroll
        for (int j = 0; j < MT; ++j) {
            int tok;
            if constexpr (T >= 32) tok = 32 * (j >> 1) + 8 * (l16 >> 2) + 4 * (j & 1) + (l16 & 3);
            else tok = 8 * ((l16 >> 2) & 1) + 4 * (l16 >> 3) + (l16 & 3);
            const uint8_t *row = kbase + tok * (MD * KB / 8) + lq * KCB;
#pragma unroll
            for (int i = 0; i < KB; ++i) kpre[j][i] = reinterpret_cast<const uint32_t *>(row)[i];
        }

        // c_K of the lane's 32 channels (lq*32 ..)
        const uint4 *cp = LDSPAGE ? reinterpret_cast<const uint4 *>(&img[PI::O_KCN + 64 * lq])
                                 : reinterpret_cast<const uint4 *>(a.kcn + kblk * MD + lq * 32);
        uint32_t cw[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 v = cp[i];
            cw[4 * i] = v.x; cw[4 * i + 1] = v.y; cw[4 * i + 2] = v.z; cw[4 * i + 3] = v.w;
        }
        // q' = qbar o c_K for this page, scaled by 2^sq, as fp16 hi + lo in MFMA element order
        float qt[32];
        float qc = 0.f, qmax = 0.f;  // sum_j q'_j and max |q'_j| over the lane's channels
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const half2v c2 = as_h2(cw[st * 4 + (e >> 1)]);
                const float x = mul_h((e & 1) ? c2.y : c2.x, qv[st * 8 + e]);
                qt[st * 8 + e] = x;
                qc += x;
                qmax = fmaxf(qmax, fabsf(x));
            }
        qc = xlane_sum_q(qc);
        const float qsc = pow2_scale_for(xlane_max_q(qmax));
        const float qinv = pow2_over<CODE_EXP<KB>>(qsc);  // undoes the query scaling and the code unit
        half8 qhi[4], qlo[4];
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const int e = (kk >> 1) + 4 * (kk & 1);
                _Float16 hi, lo;
                split_prod(qt[st * 8 + e], qsc, hi, lo);
                qhi[st][kk] = hi;
                qlo[st][kk] = lo;
            }

        // ---- scores: one MFMA chain per 16-token M-tile
        f32x4 sc[MT];
#pragma unroll
        for (int j = 0; j < MT; ++j) {
            const uint32_t *kw = kpre[j];
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                // 8 codes of K-step st start at bit st*8*KB of the chunk
                const int bit = st * 8 * KB;
                uint32_t bitsv;
                if (bit % 32 == 0) bitsv = kw[bit / 32];
                else bitsv = __builtin_amdgcn_alignbit(kw[bit / 32 + 1 < KB ? bit / 32 + 1 : bit / 32], kw[bit / 32], bit % 32);
                const half8 ak = unpack8<KB>(bitsv);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, qhi[st], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, qlo[st], acc, 0, 0, 0);
            }
            sc[j] = acc;
        }

        // ---- online softmax over this page (per head l16; lanes hold tokens)
        // score in log2 units: sm log2(e) (S qinv acc + Z sum_j q'_j)
        const float a_s = sml2 * qinv, a_z = sml2 * qc;
        float pmax = -INFINITY;
        uint4 vzq[MT];
#pragma unroll
        for (int j = 0; j < MT; ++j) {
            int tok0;
            if constexpr (T >= 32) tok0 = 32 * (j >> 1) + 8 * lq + 4 * (j & 1);
            else tok0 = 8 * (lq & 1) + 4 * (lq >> 1);
            const uint4 kz = LDSPAGE ? *reinterpret_cast<const uint4 *>(&img[PI::O_KSZ + 4 * tok0])
                                    : *reinterpret_cast<const uint4 *>(a.ksz + (kblk * T + tok0) * 2);
            vzq[j] = LDSPAGE ? *reinterpret_cast<const uint4 *>(&img[PI::O_VSZ + 4 * tok0])
                            : *reinterpret_cast<const uint4 *>(a.vsz + (kblk * T + tok0) * 2);
            const uint32_t kzw[4] = {kz.x, kz.y, kz.z, kz.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const half2v sz = as_h2(kzw[i]);  // (S, Z)
                float x = __builtin_fmaf((float)sz.x, a_s * sc[j][i], mul_h(sz.y, a_z));
                if (tok0 + i >= rows) x = -INFINITY;
                sc[j][i] = x;
                pmax = fmaxf(pmax, x);
            }
        }
        pmax = xlane_max_q(pmax);
        float m_new = fmaxf(m_run, pmax);
        // a prefill column may have seen no valid token yet: exponents against 0 then
        // give alpha = 0 and p = 0 (decode pages always hold a valid token)
        if constexpr (PF) m_new = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = exp2_fast(m_run - m_new);
        // 16-token pages: the rescaling of o' runs only when some column's running maximum
        // moved (most pages once the first few are seen leave every alpha at exactly 1);
        // larger pages keep it fused into the fold (a separate pass costs them registers,
        // and at 256 the kernel would drop to one wave per SIMD)
        constexpr bool LAZY = STAGED;
        const bool rescale = LAZY && __builtin_amdgcn_ballot_w64(alpha != 1.f) != 0;
        m_run = PF ? fmaxf(m_run, pmax) : m_new;
        // P~ = p S_V scaled by 2^sp with max_t S_V,t near 2^14 (p <= 1). The scales are
        // >= 0, so the largest is the largest fp16 bit pattern (packed u16 maxima; the
        // zero points in the upper halves are ignored)
        uint32_t smaxw = 0;
#pragma unroll
        for (int j = 0; j < MT; ++j) {
            const uint32_t vzw[4] = {vzq[j].x, vzq[j].y, vzq[j].z, vzq[j].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) smaxw = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(
                                                   __builtin_bit_cast(u16x2, smaxw), __builtin_bit_cast(u16x2, vzw[i])));
        }
        const float smax = half_bits_to_float(smaxw & 0x7fffu);
        const float psc = pow2_scale_for(xlane_max_q(smax));
        // the scaling enters the exponent: ps = p psc = 2^(score - m + log2 psc), and the
        // sums over ps are scaled back once (powers of two: the same values as unscaled)
        const float m_ps = m_new - (float)((int)(__float_as_uint(psc) >> 23) - 127);
        const float pscinv = pow2_over<0>(psc);
        float psum = 0.f, zs = 0.f;
        _Float16 phi[MT][4], plo[MT][4];
#pragma unroll
        for (int j = 0; j < MT; ++j) {
            const uint32_t vzw[4] = {vzq[j].x, vzq[j].y, vzq[j].z, vzq[j].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const half2v sz = as_h2(vzw[i]);  // (S_V, Z_V)
                const float ps = exp2_fast(sc[j][i] - m_ps);
                psum += ps;
                zs = __builtin_fmaf((float)sz.y, ps, zs);
                split_prod(ps, (float)sz.x, phi[j][i], plo[j][i]);
            }
        }
        const float pinv = pow2_over<CODE_EXP<VB>>(psc);
        l_run = __builtin_fmaf(l_run, alpha, psum * pscinv);
        zs = xlane_sum_q(zs) * pscinv;

        // ---- P~ as the B operand of the value product: K-step sv, lane (head, lq)
        // element kk <-> token 32 sv + 8 lq + e(kk), e < 4 from M-tile 2sv, e >= 4 from 2sv+1
        half8 pbh[KSV], pbl[KSV];
        if constexpr (T >= 32) {
#pragma unroll
            for (int sv = 0; sv < KSV; ++sv)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pbh[sv][2 * i] = phi[2 * sv][i];
                    pbh[sv][2 * i + 1] = phi[2 * sv + 1][i];
                    pbl[sv][2 * i] = plo[2 * sv][i];
                    pbl[sv][2 * i + 1] = plo[2 * sv + 1][i];
                }
        } else {
            // T = 16: lanes lq = 0, 1 take tokens 8 lq + e; the upper four come from lane + 32
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float hu = __shfl_xor((float)phi[0][i], 32, 64);
                const float lu = __shfl_xor((float)plo[0][i], 32, 64);
                const bool act = lq < 2;
                pbh[0][2 * i] = act ? phi[0][i] : (_Float16)0.f;
                pbh[0][2 * i + 1] = act ? (_Float16)hu : (_Float16)0.f;
                pbl[0][2 * i] = act ? plo[0][i] : (_Float16)0.f;
                pbl[0][2 * i + 1] = act ? (_Float16)lu : (_Float16)0.f;
            }
        }

        // ---- values: channel tiles mc; lane (channel 16 mc + l16, tokens 32 sv + 8 lq ..)
        // (their code words are loaded two tiles ahead of use: loading all of them
        // with the K words halves the waves per SIMD and loses more than it hides)
        if constexpr (IMG && !DB) wait_vm_upto<0>();  // the V codes have landed
        const uint8_t *vbase = STAGED ? (VB == 3 ? &wrk[wave][0] : &img[PI::O_VC])
                                      : IMG ? &img[PI::O_VC] : a.vcodes + kblk * (T * MD * VB / 8);
        constexpr bool VRING = !LDSPAGE && T >= 32 && VB != 3;
        uint32_t vw[VRING ? 8 : 1][VRING ? KSV : 1];
        auto vword = [&](int mc, int sv) -> uint32_t {
            const int64_t bit0 = ((int64_t)(16 * mc + l16) * T + 32 * sv + 8 * lq) * VB;
            if constexpr (VB == 4) return reinterpret_cast<const uint32_t *>(vbase)[bit0 >> 5];
            else return reinterpret_cast<const uint16_t *>(vbase)[bit0 >> 4];
        };
        if constexpr (VRING) {
#pragma unroll
            for (int sv = 0; sv < KSV; ++sv) {
                vw[0][sv] = vword(0, sv);
                vw[1][sv] = vword(1, sv);
            }
        }
        const uint16_t *vcn = LDSPAGE ? reinterpret_cast<const uint16_t *>(&img[PI::O_VCN]) : a.vcn + kblk * MD;
        if (rescale)
#pragma unroll
            for (int mc = 0; mc < 8; ++mc)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[mc][i] *= alpha;
#pragma unroll
        for (int mc = 0; mc < 8; ++mc) {
            const int ch = 16 * mc + l16;
            if constexpr (VRING)
                if (mc + 2 < 8)
#pragma unroll
                    for (int sv = 0; sv < KSV; ++sv) vw[mc + 2][sv] = vword(mc + 2, sv);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sv = 0; sv < KSV; ++sv) {
                half8 av;
                if (T >= 32 || lq < 2) {
                    const int64_t bit0 = ((int64_t)ch * T + 32 * sv + 8 * lq) * VB;
                    uint32_t bitsv;
                    if constexpr (VRING) bitsv = vw[mc][sv];
                    else if constexpr (VB == 4) bitsv = reinterpret_cast<const uint32_t *>(vbase)[bit0 >> 5];
                    else if constexpr (VB == 2) bitsv = reinterpret_cast<const uint16_t *>(vbase)[bit0 >> 4];
                    else if constexpr (STAGED) bitsv = reinterpret_cast<const uint32_t *>(vbase)[bit0 / 24];  // re-aligned
                    else bitsv = load_bits3(vbase, bit0);
                    av = unpack8<VB>(bitsv);
                } else {
#pragma unroll
                    for (int kk = 0; kk < 8; ++kk) av[kk] = (_Float16)0.f;
                }
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pbh[sv], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pbl[sv], acc, 0, 0, 0);
            }
            // fold: o' = alpha o' + c_V (acc + zs), or with o' rescaled above (LAZY) one mixed
            // FMA with c_V an fp16 operand; rows 4 lq + i of tile mc are channels
            const uint2 cv2 = *reinterpret_cast<const uint2 *>(vcn + 16 * mc + 4 * lq);
            const half2v c01 = as_h2(cv2.x), c23 = as_h2(cv2.y);
            const _Float16 cvv[4] = {c01.x, c01.y, c23.x, c23.y};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float t = __builtin_fmaf(acc[i], pinv, zs);
                o[mc][i] = LAZY ? __builtin_fmaf((float)cvv[i], t, o[mc][i]) : __builtin_fmaf(o[mc][i], alpha, mul_h(cvv[i], t));
            }
        }
    };
    if constexpr (DB) {
        while (pi < p1) {
            page_step(stg, stg2);
            if (!(pi < p1)) break;
            page_step(stg2, stg);
        }
    } else {
        while (pi < p1) page_step(stg, stg);
    }

    // ---- merge the four waves, write the split partial (m, l in log2 units -> natural)
    l_run = xlane_sum_q(l_run);
    if constexpr (LDSPAGE) __syncthreads();  // the merge buffers overlay the page images
    if (lq == 0) {
        red_ml[wave][l16][0] = m_run;
        red_ml[wave][l16][1] = l_run;
    }
#pragma unroll
    for (int mc = 0; mc < 8; ++mc)
#pragma unroll
        for (int i = 0; i < 4; ++i) red_o[wave][l16][16 * mc + 4 * lq + i] = o[mc][i];
    __syncthreads();
    for (int e = tid; e < (PF ? 16 : g) * MD; e += MNT) {
        const int cc = e / MD, j = e % MD;
        int64_t wrow;  // workspace row: (sequence or chunk position, query head)
        if constexpr (PF) {
            const int cpos = cb * ppb + cc / g;
            if (cpos >= a.Lq) continue;
            wrow = ((int64_t)s * a.Lq + cpos) * a.Hq + hk * g + cc % g;
        } else {
            wrow = (int64_t)s * a.Hq + hk * g + cc;
        }
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, red_ml[w][cc][0]);
        float acc = 0.f, lsum = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float mw = red_ml[w][cc][0];
            if (mw != -INFINITY) {
                const float f = exp2_fast(mw - M);
                acc = __builtin_fmaf(f, red_o[w][cc][j], acc);
                lsum = __builtin_fmaf(f, red_ml[w][cc][1], lsum);
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
            // partial max stored in natural-log units for the merge kernel
            put(MD, M == -INFINITY ? -INFINITY : M * 0.6931471805599453f);
            put(MD + 1, lsum);
        }
    }
    if constexpr (!PF) {
        static_assert(sizeof(pool) >= 4 * RED_MAX_SPLITS * sizeof(float), "merge weights fit the pool");
        if (a.cnt) merge_if_last<MNT, MD / 64>(a, s, hk, reinterpret_cast<float *>(pool));
    }
}

bool decode_mfma_supported(const DecodeArgs &a) {
    auto al16 = [](const void *p) { return ((uintptr_t)p & 15) == 0; };
    if (!al16(a.q) || !al16(a.kcodes) || !al16(a.ksz) || !al16(a.kcn) || !al16(a.vcodes) || !al16(a.vsz) || !al16(a.vcn))
        return false;
    if (a.D != MD || a.R != 0 || a.Dv != MD) return false;
    if (a.kG != MD || a.vG != MD) return false;
    if (a.grp > 16 || 16 % a.grp != 0 || a.hc != a.grp) return false;
    if (a.klayout != KVQ_TOKEN_MAJOR || a.vlayout != KVQ_CHANNEL_MAJOR || a.vH != a.Hkv) return false;
    if (!(a.kbits >= 2 && a.kbits <= 4) || !(a.vbits >= 2 && a.vbits <= 4)) return false;
    if ((int64_t)a.num_pages * a.Hkv >= (int64_t(1) << 31)) return false;  // 32-bit block ids
    return a.T == 16 || a.T == 32 || a.T == 64 || a.T == 128;
}

// Double-buffered page images (one workgroup per compute unit: the two images fill
// its LDS) for decode with pages of 64 or 128 tokens when every wave of a split walks
// at least 8 pages; below that, two single-image workgroups per compute unit hide the
// page latency better (measured on the long-context workload).
bool decode_use_db(const DecodeArgs &a, int max_seq_len) {
    if (a.Lq > 0 || a.T < 64) return false;
    const int64_t pages = (max_seq_len + a.T - 1) / a.T;
    return (pages + a.splits - 1) / a.splits >= 32;
}

template <int T, int KB, bool PF, bool DB>
static bool launch_vb2(const DecodeArgs &a, dim3 grid, hipStream_t stream) {
    switch (a.vbits) {
    case 2: hipLaunchKernelGGL((decode_mfma_kernel<T, KB, 2, PF, DB>), grid, dim3(MNT), 0, stream, a); return true;
    case 3: hipLaunchKernelGGL((decode_mfma_kernel<T, KB, 3, PF, DB>), grid, dim3(MNT), 0, stream, a); return true;
    case 4: hipLaunchKernelGGL((decode_mfma_kernel<T, KB, 4, PF, DB>), grid, dim3(MNT), 0, stream, a); return true;
    }
    return false;
}

template <int T, int KB, bool PF>
static bool launch_vb(const DecodeArgs &a, hipStream_t stream) {
    dim3 grid(a.splits, a.Hkv, a.B);
    if constexpr (PF) {
        const int64_t W = (int64_t)a.B * a.Hkv * a.splits * ((a.Lq * a.grp + 15) / 16);
        if (W > ((int64_t)1 << 30)) return false;
        grid = dim3((unsigned)(8 * ((W + 7) / 8)));
        return launch_vb2<T, KB, PF, false>(a, grid, stream);
    } else {
        if constexpr (T >= 64)
            if (decode_use_db(a, a.max_len)) return launch_vb2<T, KB, false, true>(a, grid, stream);
        return launch_vb2<T, KB, false, false>(a, grid, stream);
    }
}

template <int T, bool PF>
static bool launch_kb(const DecodeArgs &a, hipStream_t stream) {
    switch (a.kbits) {
    case 2: return launch_vb<T, 2, PF>(a, stream);
    case 3: return launch_vb<T, 3, PF>(a, stream);
    case 4: return launch_vb<T, 4, PF>(a, stream);
    }
    return false;
}

template <bool PF>
static bool launch_t(const DecodeArgs &a, hipStream_t stream) {
    switch (a.T) {
    case 16: return launch_kb<16, PF>(a, stream);
    case 32: return launch_kb<32, PF>(a, stream);
    case 64: return launch_kb<64, PF>(a, stream);
    case 128: return launch_kb<128, PF>(a, stream);
    }
    return false;
}

bool decode_pair16_supported(const DecodeArgs &a);
bool launch_decode_pair16(const DecodeArgs &a, hipStream_t stream);

// decode (a.Lq == 0) or chunked prefill (a.Lq > 0, a.B real sequences); decode over
// 16-token pages with at most 8 query heads per kv head takes two pages per pass
bool launch_decode_mfma(const DecodeArgs &a, hipStream_t stream) {
    if (a.Lq == 0 && decode_pair16_supported(a)) return launch_decode_pair16(a, stream);
    return a.Lq > 0 ? launch_t<true>(a, stream) : launch_t<false>(a, stream);
}

}  // namespace kvq
