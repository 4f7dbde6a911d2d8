/*
 * CPU oracle for KVarN-style KV-cache quantization and quantized decode attention.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. The GPU library never
 * links it, includes it or calls it; the two share no code, headers or tables.
 *
 * Everything is plain scalar code in IEEE double precision. Values are rounded
 * only where the method stores them (fp16 normalizers, scales and zero points,
 * integer codes); the code decision is the plain fp64 round-to-nearest-even of
 * (y - Z) / S.
 *
 * Sources (web pages on the subject; cited by page title and section):
 *   [REVIEW]  "KVarN" project review (open-radar), sections Overview and
 *             Key Features ("Variance-Normalized Quantization Pipeline",
 *             "Calibration-Free Operation", "MLA Model Support",
 *             "4-bit Keys, 2-bit Values Preset").
 *   [TAG]     "KV-Cache" tag page (baguaai), the KVarN item that names the
 *             dual-axis normalization and round-to-nearest quantization.
 *   [SEARCH]  the paper-search listing ("value cache amortisation"): KIVI
 *             (per-token asymmetric quantization) and SAW-INT4 (token-wise
 *             INT4 with a block-diagonal Hadamard rotation).
 * The pages fix only the stage order; every other choice is a reading that is
 * listed, with its reason, in the repository's design notes.
 */
#ifndef KVQ_ORACLE_H
#define KVQ_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Code layouts of one (page, head) block of T x D codes. */
enum { ORC_TOKEN_MAJOR = 0, ORC_CHANNEL_MAJOR = 1 };
/* Element types of inputs. */
enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };
/* Status bits mirrored from the device side. */
enum { ORC_FLAG_NONFINITE = 1, ORC_FLAG_SIDE_OVERFLOW = 2 };

typedef struct {
    int32_t head_dim;    /* D: quantized channels per token and head            */
    int32_t rope_dim;    /* R: extra bf16 channels stored as-is (MLA), else 0   */
    int32_t tile_tokens; /* T: tokens per tile = tokens per page                */
    int32_t hadamard_n;  /* h: block size of the block-diagonal Hadamard, h | D */
    int32_t group;       /* G: channels per scale/zero group, G | D             */
    int32_t bits;        /* b: code width                                       */
    int32_t iters;       /* N: row/column normalization rounds                  */
    int32_t layout;      /* ORC_TOKEN_MAJOR or ORC_CHANNEL_MAJOR                */
    int32_t center;      /* 0: rounds scale rows/columns to unit RMS about zero;
                            1: to unit standard deviation about their mean      */
} orc_format;

/* Host-memory paged quantized cache. Per (page p, head h):
 *   codes  uint8  [P][H][T*D*b/8]      token-major: T rows of D*b/8 bytes,
 *                                      channel-major: D rows of T*b/8 bytes;
 *                                      each row a little-endian bitstream
 *   sz     uint16 [P][H][T][D/G][2]    fp16 (scale, zero) per token and group
 *   cnorm  uint16 [P][H][D]            fp16 per-channel normalizer
 *   rope   uint16 [P][H][T][R]         bf16 copy of the rope channels (R > 0)
 *   quot   double [P][H][T][D]         nullable; written by orc_quantize_cache:
 *                                      the code quotient (y - Z) / S before
 *                                      rounding (NaN where S == 0 or t >= n) */
typedef struct {
    orc_format fmt;
    int32_t num_pages, num_heads;
    uint8_t *codes;
    uint16_t *sz;
    uint16_t *cnorm;
    uint16_t *rope;
    double *quot;
} orc_cache;

/* ---- number formats (IEEE-754 binary16, bfloat16) ---- */
double orc_half_to_double(uint16_t h);
uint16_t orc_double_to_half(double x);
double orc_bf16_to_double(uint16_t b);
uint16_t orc_double_to_bf16(double x);

/* ---- tile-level steps ---- */
void orc_hadamard_matrix(int32_t h, double *out /* h*h, row-major */);
void orc_rotate(const double *x, int32_t n, int32_t D, int32_t h, double *out);
void orc_normalizers(const double *xr, int32_t n, int32_t D, int32_t iters, int32_t center,
                     double *c /* [D] */, double *r /* [n] or NULL */);
/* Quantize one tile of n valid rows (n <= T) of D channels (rope excluded).
 * codes: [T][D] unpacked integer codes (rows >= n zero); sz: [T][D/G][2];
 * c16: [D]; c_exact: [D] fp64 normalizer before rounding (nullable);
 * quot: [T][D] code quotient (y - Z) / S before rounding, NaN where S == 0 or
 * t >= n (nullable). Returns status bits. */
uint32_t orc_quantize_tile(const double *x, int32_t n, const orc_format *f,
                           uint16_t *codes, uint16_t *sz, uint16_t *c16, double *c_exact,
                           double *quot);
void orc_pack(const uint16_t *codes, const orc_format *f, uint8_t *out);
void orc_unpack(const uint8_t *in, const orc_format *f, uint16_t *codes);
/* Dequantize one tile back to the input space: out [T][D]. */
void orc_dequant_tile(const uint16_t *codes, const uint16_t *sz, const uint16_t *c16,
                      const orc_format *f, double *out);

/* ---- cache-level drivers, threaded over independent tiles / outputs ---- */
uint32_t orc_quantize_cache(const orc_cache *dst, const void *src, int32_t src_dtype,
                            int64_t stride_token, int64_t stride_head, int32_t num_tiles,
                            const int32_t *tile_src_token, const int32_t *tile_valid,
                            const int32_t *tile_dst_page, int32_t nthreads);
/* out: [num_tiles][H][T][D + R] doubles (rope passes through). */
void orc_dequantize_cache(const orc_cache *src, int32_t num_tiles, const int32_t *tile_page,
                          const int32_t *tile_valid, double *out, int32_t nthreads);
/* Decode attention for one new query per sequence.
 * q: [num_seqs][num_q_heads][D + R] in q_dtype; v == NULL means the K cache
 * (the MLA latent) is also the value cache. out: [num_seqs][num_q_heads][Dv].
 * folded = 0: softmax attention over explicitly dequantized K and V.
 * folded = 1: the folded evaluation (rotation and normalizers moved onto the
 *             query and the output, per-token scales onto the scores). */
void orc_decode_attn(const void *q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                     const orc_cache *k, const orc_cache *v, const int32_t *block_table,
                     int32_t block_table_stride, const int32_t *seq_lens, double sm_scale,
                     int32_t folded, double *out, int32_t nthreads);

#ifdef __cplusplus
}
#endif
#endif
