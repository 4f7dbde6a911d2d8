/*
 * CPU oracle for KVarN-style KV-cache quantization and quantized decode attention.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark, never by the GPU library. Plain scalar
 * loops in IEEE double precision; see oracle.h for the sources cited below.
 *
 * Build: g++ -O2 -std=c++17 -ffp-contract=off -fPIC -shared -pthread
 * (-ffp-contract=off: every double operation is rounded on its own, as
 * written; no fused multiply-adds).
 */
#include "oracle.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

namespace {

/* ------------------------------------------------------------------------ */
/* IEEE-754 binary16 and bfloat16, written from the format definitions.      */
/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits.                 */
/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits.                 */
/* Rounding is to nearest, ties to even; overflow goes to infinity.          */
/* ------------------------------------------------------------------------ */

uint16_t round_to_format(double x, int frac_bits, int min_exp, int bias, int exp_field_max,
                         double overflow_at) {
    const uint16_t sign_bit = (uint16_t)(1u << (frac_bits + (exp_field_max == 31 ? 5 : 8)));
    if (std::isnan(x)) return (uint16_t)((exp_field_max << frac_bits) | (1u << (frac_bits - 1)));
    uint16_t sign = std::signbit(x) ? sign_bit : 0;
    double a = std::fabs(x);
    if (a == 0.0) return sign;
    if (a >= overflow_at) return (uint16_t)(sign | (exp_field_max << frac_bits));
    int e2 = 0;
    std::frexp(a, &e2);           /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;
    if (E < min_exp) E = min_exp; /* subnormals share the quantum of the lowest binade */
    const double quantum = std::ldexp(1.0, E - frac_bits);
    double q = std::nearbyint(a / quantum); /* exact quotient; default mode = ties-to-even */
    const double one = std::ldexp(1.0, frac_bits);
    if (q >= 2.0 * one) { /* rounding carried into the next binade */
        q = one;
        E += 1;
    }
    if (q < one) return (uint16_t)(sign | (uint16_t)q); /* subnormal (E == min_exp) */
    const int field = E + bias;
    if (field >= exp_field_max) return (uint16_t)(sign | (exp_field_max << frac_bits));
    return (uint16_t)(sign | (field << frac_bits) | (uint16_t)(q - one));
}

double decode_format(uint16_t v, int frac_bits, int exp_bits, int bias) {
    const int exp_max = (1 << exp_bits) - 1;
    const int e = (v >> frac_bits) & exp_max;
    const int m = v & ((1 << frac_bits) - 1);
    const double s = (v >> (frac_bits + exp_bits)) & 1 ? -1.0 : 1.0;
    if (e == 0) return s * std::ldexp((double)m, 1 - bias - frac_bits);
    if (e == exp_max) return m ? std::nan("") : s * INFINITY;
    return s * std::ldexp((double)((1 << frac_bits) + m), e - bias - frac_bits);
}

double half_val(uint16_t h) { return decode_format(h, 10, 5, 15); }
uint16_t to_half(double x) { return round_to_format(x, 10, -14, 15, 31, 65520.0); }
double bf16_val(uint16_t b) { return decode_format(b, 7, 8, 127); }
uint16_t to_bf16(double x) {
    /* largest finite bf16 is (2 - 2^-7) * 2^127; halfway to 2^128 rounds up (odd fraction) */
    return round_to_format(x, 7, -126, 127, 255, std::ldexp(2.0 - std::ldexp(1.0, -8), 127));
}

double load_elem(const void *p, int dtype, int64_t idx) {
    switch (dtype) {
    case ORC_F32: {
        float f;
        std::memcpy(&f, (const char *)p + idx * 4, 4);
        return (double)f;
    }
    case ORC_F16: return half_val(((const uint16_t *)p)[idx]);
    default: return bf16_val(((const uint16_t *)p)[idx]);
    }
}

/* ------------------------------------------------------------------------ */
/* Sylvester Hadamard matrix in natural order: H[i][j] = (-1)^popcount(i&j). */
/* The rotation is X' = X Q with Q = blockdiag(H_h/sqrt(h), ...) along the   */
/* channel axis ([REVIEW] Key Features: a Hadamard rotation spreads channel  */
/* outliers; [SEARCH] SAW-INT4: block-diagonal Hadamard). Q is symmetric and */
/* orthogonal, hence its own inverse.                                        */
/* ------------------------------------------------------------------------ */
inline double hadamard_sign(int i, int j) { return (__builtin_popcount((unsigned)(i & j)) & 1) ? -1.0 : 1.0; }

void rotate_rows(const double *x, int n, int D, int h, double *out) {
    const double inv = 1.0 / std::sqrt((double)h);
    std::vector<double> row(D);
    for (int i = 0; i < n; ++i) {
        for (int b0 = 0; b0 < D; b0 += h) {
            for (int j = 0; j < h; ++j) {
                double acc = 0.0;
                for (int k = 0; k < h; ++k) acc += x[(size_t)i * D + b0 + k] * hadamard_sign(k, j);
                row[b0 + j] = acc * inv;
            }
        }
        std::memcpy(out + (size_t)i * D, row.data(), sizeof(double) * D);
    }
}

/* ------------------------------------------------------------------------ */
/* Sinkhorn-like dual-axis variance normalization ([REVIEW] Key Features:     */
/* iterative, equalizes variance across the tile; [TAG] KVarN item: dual-axis).*/
/* Reading: "variance" is the second moment about zero (RMS); one round is a  */
/* row step then a column step; a factor that is zero or not finite is        */
/* replaced by one. Only the valid n rows take part. With center = 1 (the     */
/* other reading of "variance") each step uses the standard deviation about   */
/* the row's / column's mean instead; the means are not removed from the data.*/
/* ------------------------------------------------------------------------ */
void normalizers(const double *xr, int n, int D, int iters, int center, double *c, double *r) {
    std::vector<double> rr(std::max(n, 1), 1.0);
    for (int j = 0; j < D; ++j) c[j] = 1.0;
    for (int it = 0; it < iters; ++it) {
        for (int i = 0; i < n; ++i) { /* row step: each row of Z = X'/(r c) to unit RMS (or std) */
            double mu = 0.0;
            if (center) {
                for (int j = 0; j < D; ++j) mu += xr[(size_t)i * D + j] / (rr[i] * c[j]);
                mu /= D;
            }
            double s = 0.0;
            for (int j = 0; j < D; ++j) {
                const double z = xr[(size_t)i * D + j] / (rr[i] * c[j]) - mu;
                s += z * z;
            }
            double rho = std::sqrt(s / D);
            if (!(rho > 0.0) || !std::isfinite(rho)) rho = 1.0;
            rr[i] *= rho;
        }
        if (n == 0) continue;
        for (int j = 0; j < D; ++j) { /* column step: each column of Z to unit RMS (or std) */
            double mu = 0.0;
            if (center) {
                for (int i = 0; i < n; ++i) mu += xr[(size_t)i * D + j] / (rr[i] * c[j]);
                mu /= n;
            }
            double s = 0.0;
            for (int i = 0; i < n; ++i) {
                const double z = xr[(size_t)i * D + j] / (rr[i] * c[j]) - mu;
                s += z * z;
            }
            double gam = std::sqrt(s / n);
            if (!(gam > 0.0) || !std::isfinite(gam)) gam = 1.0;
            c[j] *= gam;
        }
    }
    if (r)
        for (int i = 0; i < n; ++i) r[i] = rr[i];
}

/* Asymmetric round-to-nearest of one value against the stored fp16 scale and
 * zero point ([REVIEW] Key Features: asymmetric round-to-nearest), the plain
 * definition in fp64: code = clamp(rne((y - Z) / S), 0, 2^b - 1); S == 0 gives
 * code 0 (a constant group). *quot receives (y - Z) / S before rounding (NaN
 * for S == 0), the value whose distance from a half-integer says how close the
 * decision was to a tie. */
uint16_t rtn_code(double y, double Sv, double Zv, int levels, double *quot) {
    if (Sv == 0.0) {
        if (quot) *quot = std::nan("");
        return 0;
    }
    const double qr = (y - Zv) / Sv;
    if (quot) *quot = qr;
    const double qn = std::nearbyint(qr); /* default rounding mode: ties to even */
    if (!(qn > 0.0)) return 0;
    if (qn > (double)levels) return (uint16_t)levels;
    return (uint16_t)qn;
}

int row_bytes_of(const orc_format *f) {
    return f->layout == ORC_TOKEN_MAJOR ? f->head_dim * f->bits / 8 : f->tile_tokens * f->bits / 8;
}

template <class Fn> void parallel_for(int64_t count, int nthreads, Fn fn) {
    if (nthreads <= 1 || count <= 1) {
        for (int64_t i = 0; i < count; ++i) fn(i);
        return;
    }
    std::atomic<int64_t> next(0);
    std::vector<std::thread> pool;
    const int nt = (int)std::min<int64_t>(nthreads, count);
    for (int t = 0; t < nt; ++t)
        pool.emplace_back([&]() {
            for (int64_t i; (i = next.fetch_add(1)) < count;) fn(i);
        });
    for (auto &th : pool) th.join();
}

size_t page_head_code_bytes(const orc_format *f) { return (size_t)f->tile_tokens * f->head_dim * f->bits / 8; }
size_t page_head_sz_elems(const orc_format *f) { return (size_t)f->tile_tokens * (f->head_dim / f->group) * 2; }

/* Dequantize rows of one (page, head) block to the rotated domain
 * x'_tj = (S_tg code_tj + Z_tg) c_j, then rotate back (Q^-1 = Q). */
void dequant_block(const orc_cache *cc, int page, int head, double *out /* [T][D] */) {
    const orc_format *f = &cc->fmt;
    const int T = f->tile_tokens, D = f->head_dim;
    const size_t blk = (size_t)page * cc->num_heads + head;
    std::vector<uint16_t> codes((size_t)T * D);
    orc_unpack(cc->codes + blk * page_head_code_bytes(f), f, codes.data());
    const uint16_t *sz = cc->sz + blk * page_head_sz_elems(f);
    const uint16_t *c16 = cc->cnorm + blk * D;
    std::vector<uint16_t> szv(sz, sz + page_head_sz_elems(f));
    orc_dequant_tile(codes.data(), szv.data(), c16, f, out);
}

} // namespace

extern "C" {

double orc_half_to_double(uint16_t h) { return half_val(h); }
uint16_t orc_double_to_half(double x) { return to_half(x); }
double orc_bf16_to_double(uint16_t b) { return bf16_val(b); }
uint16_t orc_double_to_bf16(double x) { return to_bf16(x); }

void orc_hadamard_matrix(int32_t h, double *out) {
    const double inv = 1.0 / std::sqrt((double)h);
    for (int i = 0; i < h; ++i)
        for (int j = 0; j < h; ++j) out[(size_t)i * h + j] = hadamard_sign(i, j) * inv;
}

void orc_rotate(const double *x, int32_t n, int32_t D, int32_t h, double *out) { rotate_rows(x, n, D, h, out); }

void orc_normalizers(const double *xr, int32_t n, int32_t D, int32_t iters, int32_t center, double *c, double *r) {
    normalizers(xr, n, D, iters, center, c, r);
}

uint32_t orc_quantize_tile(const double *x, int32_t n, const orc_format *f, uint16_t *codes, uint16_t *sz,
                           uint16_t *c16, double *c_exact, double *quot) {
    const int T = f->tile_tokens, D = f->head_dim, G = f->group, ng = D / G;
    const int levels = (1 << f->bits) - 1;
    uint32_t flags = 0;
    for (size_t i = 0; i < (size_t)n * D; ++i)
        if (!std::isfinite(x[i])) flags |= ORC_FLAG_NONFINITE;

    /* 1. rotate along channels */
    std::vector<double> xr((size_t)std::max(n, 1) * D);
    rotate_rows(x, n, D, f->hadamard_n, xr.data());
    /* 2. per-channel normalizer c (the row factors only re-scale each token,
     *    which the per-token scale and zero absorb, so they are not stored) */
    std::vector<double> c(D);
    normalizers(xr.data(), n, D, f->iters, f->center, c.data(), nullptr);
    std::vector<double> cval(D);
    for (int j = 0; j < D; ++j) {
        c16[j] = to_half(c[j]);
        cval[j] = half_val(c16[j]);
        if (!std::isfinite(cval[j]) || cval[j] == 0.0) flags |= ORC_FLAG_SIDE_OVERFLOW;
        if (c_exact) c_exact[j] = c[j];
    }
    /* 3. per-token, per-group asymmetric min-max round-to-nearest on y = X'/c16
     *    ([REVIEW] Key Features: asymmetric round-to-nearest; [SEARCH] KIVI:
     *    per-token asymmetric quantization) */
    std::memset(codes, 0, sizeof(uint16_t) * (size_t)T * D);
    std::memset(sz, 0, sizeof(uint16_t) * (size_t)T * ng * 2);
    if (quot)
        for (size_t i = 0; i < (size_t)T * D; ++i) quot[i] = std::nan("");
    std::vector<double> y(G);
    for (int t = 0; t < n; ++t) {
        for (int g = 0; g < ng; ++g) {
            double mn = INFINITY, mx = -INFINITY;
            for (int k = 0; k < G; ++k) {
                const int j = g * G + k;
                y[k] = xr[(size_t)t * D + j] / cval[j];
                mn = std::min(mn, y[k]);
                mx = std::max(mx, y[k]);
            }
            const uint16_t S16 = to_half((mx - mn) / levels);
            const uint16_t Z16 = to_half(mn);
            const double Sv = half_val(S16), Zv = half_val(Z16);
            if (!std::isfinite(Sv) || !std::isfinite(Zv)) flags |= ORC_FLAG_SIDE_OVERFLOW;
            sz[((size_t)t * ng + g) * 2 + 0] = S16;
            sz[((size_t)t * ng + g) * 2 + 1] = Z16;
            for (int k = 0; k < G; ++k) {
                const size_t e = (size_t)t * D + g * G + k;
                codes[e] = rtn_code(y[k], Sv, Zv, levels, quot ? quot + e : nullptr);
            }
        }
    }
    return flags;
}

/* Little-endian bitstream per row: code at position p occupies bits
 * [b p, b p + b), bit k of the stream being bit (k mod 8) of byte k / 8. */
void orc_pack(const uint16_t *codes, const orc_format *f, uint8_t *out) {
    const int T = f->tile_tokens, D = f->head_dim, b = f->bits;
    const int rb = row_bytes_of(f);
    std::memset(out, 0, (size_t)T * D * b / 8);
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < D; ++j) {
            const unsigned v = codes[(size_t)t * D + j];
            const int row = f->layout == ORC_TOKEN_MAJOR ? t : j;
            const int pos = f->layout == ORC_TOKEN_MAJOR ? j : t;
            for (int k = 0; k < b; ++k)
                if ((v >> k) & 1u) {
                    const long bit = (long)pos * b + k;
                    out[(size_t)row * rb + bit / 8] |= (uint8_t)(1u << (bit % 8));
                }
        }
}

void orc_unpack(const uint8_t *in, const orc_format *f, uint16_t *codes) {
    const int T = f->tile_tokens, D = f->head_dim, b = f->bits;
    const int rb = row_bytes_of(f);
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < D; ++j) {
            const int row = f->layout == ORC_TOKEN_MAJOR ? t : j;
            const int pos = f->layout == ORC_TOKEN_MAJOR ? j : t;
            unsigned v = 0;
            for (int k = 0; k < b; ++k) {
                const long bit = (long)pos * b + k;
                if ((in[(size_t)row * rb + bit / 8] >> (bit % 8)) & 1u) v |= 1u << k;
            }
            codes[(size_t)t * D + j] = (uint16_t)v;
        }
}

void orc_dequant_tile(const uint16_t *codes, const uint16_t *sz, const uint16_t *c16, const orc_format *f,
                      double *out) {
    const int T = f->tile_tokens, D = f->head_dim, G = f->group, ng = D / G;
    std::vector<double> xq((size_t)T * D);
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < D; ++j) {
            const int g = j / G;
            const double S = half_val(sz[((size_t)t * ng + g) * 2 + 0]);
            const double Z = half_val(sz[((size_t)t * ng + g) * 2 + 1]);
            xq[(size_t)t * D + j] = (S * codes[(size_t)t * D + j] + Z) * half_val(c16[j]);
        }
    rotate_rows(xq.data(), T, D, f->hadamard_n, out);
}

uint32_t orc_quantize_cache(const orc_cache *dst, const void *src, int32_t src_dtype, int64_t stride_token,
                            int64_t stride_head, int32_t num_tiles, const int32_t *tile_src_token,
                            const int32_t *tile_valid, const int32_t *tile_dst_page, int32_t nthreads) {
    const orc_format *f = &dst->fmt;
    const int T = f->tile_tokens, D = f->head_dim, R = f->rope_dim, H = dst->num_heads;
    std::atomic<uint32_t> flags(0);
    parallel_for((int64_t)num_tiles * H, nthreads, [&](int64_t w) {
        const int tile = (int)(w / H), head = (int)(w % H);
        const int n = tile_valid[tile];
        std::vector<double> x((size_t)std::max(n, 1) * D);
        for (int t = 0; t < n; ++t)
            for (int j = 0; j < D; ++j)
                x[(size_t)t * D + j] =
                    load_elem(src, src_dtype, (int64_t)(tile_src_token[tile] + t) * stride_token + head * stride_head + j);
        std::vector<uint16_t> codes((size_t)T * D), sz((size_t)T * (D / f->group) * 2), c16(D);
        const size_t blk = (size_t)tile_dst_page[tile] * H + head;
        double *qt = dst->quot ? dst->quot + blk * (size_t)T * D : nullptr;
        uint32_t fl = orc_quantize_tile(x.data(), n, f, codes.data(), sz.data(), c16.data(), nullptr, qt);
        orc_pack(codes.data(), f, dst->codes + blk * page_head_code_bytes(f));
        std::memcpy(dst->sz + blk * page_head_sz_elems(f), sz.data(), sizeof(uint16_t) * sz.size());
        std::memcpy(dst->cnorm + blk * D, c16.data(), sizeof(uint16_t) * D);
        if (R > 0) {
            uint16_t *rp = dst->rope + blk * (size_t)T * R;
            for (int t = 0; t < T; ++t)
                for (int k = 0; k < R; ++k) {
                    double v = 0.0;
                    if (t < n)
                        v = load_elem(src, src_dtype,
                                      (int64_t)(tile_src_token[tile] + t) * stride_token + head * stride_head + D + k);
                    if (t < n && !std::isfinite(v)) fl |= ORC_FLAG_NONFINITE;
                    rp[(size_t)t * R + k] = to_bf16(v);
                }
        }
        flags.fetch_or(fl);
    });
    return flags.load();
}

void orc_dequantize_cache(const orc_cache *src, int32_t num_tiles, const int32_t *tile_page, const int32_t *tile_valid,
                          double *out, int32_t nthreads) {
    const orc_format *f = &src->fmt;
    const int T = f->tile_tokens, D = f->head_dim, R = f->rope_dim, H = src->num_heads;
    const int W = D + R;
    parallel_for((int64_t)num_tiles * H, nthreads, [&](int64_t w) {
        const int tile = (int)(w / H), head = (int)(w % H);
        std::vector<double> blk((size_t)T * D);
        dequant_block(src, tile_page[tile], head, blk.data());
        double *o = out + ((size_t)tile * H + head) * T * W;
        const uint16_t *rp = R > 0 ? src->rope + ((size_t)tile_page[tile] * H + head) * T * R : nullptr;
        for (int t = 0; t < T; ++t)
            for (int j = 0; j < W; ++j) {
                double v = 0.0;
                if (t < tile_valid[tile]) v = j < D ? blk[(size_t)t * D + j] : bf16_val(rp[(size_t)t * R + (j - D)]);
                o[(size_t)t * W + j] = v;
            }
    });
}

void orc_decode_attn(const void *q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads, const orc_cache *k,
                     const orc_cache *v, const int32_t *block_table, int32_t block_table_stride,
                     const int32_t *seq_lens, double sm_scale, int32_t folded, double *out, int32_t nthreads) {
    const orc_format *fk = &k->fmt;
    const orc_cache *vc = v ? v : k;
    const orc_format *fv = &vc->fmt;
    const int T = fk->tile_tokens, D = fk->head_dim, R = fk->rope_dim, Dv = fv->head_dim;
    const int Hkv = k->num_heads, grp = num_q_heads / Hkv, Wq = D + R;
    /* one work item = (sequence, kv head): its pages are dequantized (or read) once
     * and shared by the query heads of the group */
    const int64_t units = (int64_t)num_seqs * Hkv;
    const int inner = (int)std::max<int64_t>(1, nthreads / std::max<int64_t>(units, 1));
    parallel_for(units, nthreads, [&](int64_t w) {
        const int s = (int)(w / Hkv), hk = (int)(w % Hkv);
        const int L = seq_lens[s];
        const int npages = (L + T - 1) / T;
        if (!folded) {
            /* softmax(q K^T * scale) V over explicitly dequantized K and V */
            std::vector<double> K((size_t)npages * T * D), V((size_t)npages * T * Dv);
            parallel_for(npages, inner, [&](int64_t pi) {
                const int page = block_table[(size_t)s * block_table_stride + pi];
                dequant_block(k, page, hk, K.data() + (size_t)pi * T * D);
                if (v) dequant_block(v, page, hk, V.data() + (size_t)pi * T * Dv);
            });
            if (!v) V = K; /* the MLA latent doubles as the value */
            parallel_for(grp, inner, [&](int64_t gi) {
                const int hq = hk * grp + (int)gi;
                const int64_t qoff = ((int64_t)s * num_q_heads + hq) * Wq;
                std::vector<double> logits(std::max(L, 1));
                double mx = -INFINITY;
                for (int t = 0; t < L; ++t) {
                    const int pi = t / T, row = t % T;
                    double acc = 0.0;
                    for (int j = 0; j < D; ++j) acc += load_elem(q, q_dtype, qoff + j) * K[((size_t)pi * T + row) * D + j];
                    if (R > 0) {
                        const int page = block_table[(size_t)s * block_table_stride + pi];
                        const uint16_t *rp = k->rope + ((size_t)page * Hkv + hk) * T * R + (size_t)row * R;
                        for (int j = 0; j < R; ++j) acc += load_elem(q, q_dtype, qoff + D + j) * bf16_val(rp[j]);
                    }
                    logits[t] = acc * sm_scale;
                    mx = std::max(mx, logits[t]);
                }
                double l = 0.0;
                std::vector<double> o(Dv, 0.0);
                for (int t = 0; t < L; ++t) {
                    const double p = std::exp(logits[t] - mx);
                    l += p;
                    for (int j = 0; j < Dv; ++j) o[j] += p * V[(size_t)t * Dv + j];
                }
                for (int j = 0; j < Dv; ++j) out[((size_t)s * num_q_heads + hq) * Dv + j] = L > 0 ? o[j] / l : 0.0;
            });
        } else {
            /* the folded evaluation: q' = (q Q) o c_K per page, scores use the
             * per-token scale and zero directly, values accumulate in the rotated
             * and normalized domain and are mapped back once at the end */
            const int Gk = fk->group, Gv = fv->group;
            parallel_for(grp, inner, [&](int64_t gi) {
                const int hq = hk * grp + (int)gi;
                std::vector<uint16_t> kc((size_t)T * D), vcodes((size_t)T * Dv);
                std::vector<double> logits(std::max(L, 1));
                const int64_t qoff = ((int64_t)s * num_q_heads + hq) * Wq;
                std::vector<double> qin(D), qbar(D);
                for (int j = 0; j < D; ++j) qin[j] = load_elem(q, q_dtype, qoff + j);
                rotate_rows(qin.data(), 1, D, fk->hadamard_n, qbar.data());
                double mx = -INFINITY;
                for (int pi = 0; pi < npages; ++pi) {
                    const int page = block_table[(size_t)s * block_table_stride + pi];
                    const size_t blk = (size_t)page * Hkv + hk;
                    orc_unpack(k->codes + blk * page_head_code_bytes(fk), fk, kc.data());
                    const uint16_t *sz = k->sz + blk * page_head_sz_elems(fk);
                    const uint16_t *c16 = k->cnorm + blk * D;
                    for (int row = 0; row < T && pi * T + row < L; ++row) {
                        double acc = 0.0;
                        for (int g = 0; g < D / Gk; ++g) {
                            double dot = 0.0, sum = 0.0;
                            for (int j = g * Gk; j < (g + 1) * Gk; ++j) {
                                const double qt = qbar[j] * half_val(c16[j]);
                                dot += qt * kc[(size_t)row * D + j];
                                sum += qt;
                            }
                            acc += half_val(sz[((size_t)row * (D / Gk) + g) * 2]) * dot +
                                   half_val(sz[((size_t)row * (D / Gk) + g) * 2 + 1]) * sum;
                        }
                        if (R > 0) {
                            const uint16_t *rp = k->rope + blk * T * R + (size_t)row * R;
                            for (int j = 0; j < R; ++j) acc += load_elem(q, q_dtype, qoff + D + j) * bf16_val(rp[j]);
                        }
                        logits[pi * T + row] = acc * sm_scale;
                        mx = std::max(mx, logits[pi * T + row]);
                    }
                }
                double l = 0.0;
                std::vector<double> o(Dv, 0.0), acc(Dv);
                for (int pi = 0; pi < npages; ++pi) {
                    const int page = block_table[(size_t)s * block_table_stride + pi];
                    const size_t blk = (size_t)page * vc->num_heads + hk;
                    orc_unpack(vc->codes + blk * page_head_code_bytes(fv), fv, vcodes.data());
                    const uint16_t *sz = vc->sz + blk * page_head_sz_elems(fv);
                    const uint16_t *c16 = vc->cnorm + blk * Dv;
                    std::fill(acc.begin(), acc.end(), 0.0);
                    for (int row = 0; row < T && pi * T + row < L; ++row) {
                        const double p = std::exp(logits[pi * T + row] - mx);
                        l += p;
                        for (int j = 0; j < Dv; ++j) {
                            const int g = j / Gv;
                            acc[j] += p * (half_val(sz[((size_t)row * (Dv / Gv) + g) * 2]) * vcodes[(size_t)row * Dv + j] +
                                           half_val(sz[((size_t)row * (Dv / Gv) + g) * 2 + 1]));
                        }
                    }
                    for (int j = 0; j < Dv; ++j) o[j] += acc[j] * half_val(c16[j]);
                }
                std::vector<double> ob(Dv);
                for (int j = 0; j < Dv; ++j) o[j] = L > 0 ? o[j] / l : 0.0;
                rotate_rows(o.data(), 1, Dv, fv->hadamard_n, ob.data());
                for (int j = 0; j < Dv; ++j) out[((size_t)s * num_q_heads + hq) * Dv + j] = ob[j];
            });
        }
    });
}

} // extern "C"
