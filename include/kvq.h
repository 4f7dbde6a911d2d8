/*
 * kvq: KVarN-style KV-cache quantization and quantized decode attention for
 * AMD Instinct MI355X (gfx950). C ABI of libkvq.so.
 *
 * The method (as described by the "KVarN" project review, section Key
 * Features, "Variance-Normalized Quantization Pipeline"; and by the KVarN item
 * of the "KV-Cache" tag page): each KV tile of T tokens x D channels is
 *   1. rotated along its channels by a block Sylvester Hadamard matrix
 *      Q = blockdiag(H_h / sqrt(h)) to spread channel outliers,
 *   2. put through `iters` Sinkhorn-like rounds that set every row, then every
 *      column, of X Q / (r c) to unit RMS (dual-axis variance equalization over
 *      the tile, computed on the fly: no calibration data),
 *   3. quantized per token and per group of `group` channels by asymmetric
 *      round-to-nearest: code = clamp(rne((y - Z) / S), 0, 2^bits - 1) with
 *      y = (X Q)_j / c_j, S = (max y - min y) / (2^bits - 1), Z = min y.
 * Stored per (page, head): packed codes, fp16 (S, Z) per token and group,
 * fp16 c per channel. The per-token row factors r are not stored: per-token
 * min-max quantization is exactly invariant to them.
 * The consumer (decode attention) never rebuilds K or V: it rotates and
 * scales the query, q' = (q Q) o c_K, takes scores from the codes with the
 * per-token (S, Z), accumulates values as sum_t p_t (S_t code_t + Z_t) o c_V
 * and rotates the result back once.
 *
 * Conventions
 *  - Every pointer inside kvq_cache and every array argument named "device"
 *    is device memory owned by the caller; kvq_cache and kvq_format structs
 *    themselves are host memory, read during the call only.
 *  - Each call validates its arguments on the host, returns a negative
 *    kvq_status without enqueuing anything when they are invalid, and otherwise
 *    enqueues its kernels on `stream` and returns KVQ_OK without synchronizing.
 *  - Data conditions found on the device (non-finite input, fp16 overflow of a
 *    scale, zero point or normalizer) set bits in *status_flags; they never
 *    abort a launch. The codes of a block with such a condition are
 *    unspecified but stay in 0 .. 2^bits - 1.
 *  - The library allocates no device memory and keeps no mutable global state
 *    (the one exception: kv_decode_attn_noalloc's per-device scratch array and its
 *    address table); calls on different streams may run concurrently, except
 *    kv_decode_attn_noalloc calls on one GPU.
 */
#ifndef KVQ_H
#define KVQ_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. Calls take them (and kvq_status_str its code) as int32_t: any
 * value may arrive through the C ABI, and an out-of-range one returns KVQ_EINVAL
 * (a parameter of enum type holding it would be undefined behaviour in C++). */
typedef enum { KVQ_F32 = 0, KVQ_F16 = 1, KVQ_BF16 = 2 } kvq_dtype;

typedef enum {
    KVQ_OK = 0,
    KVQ_EINVAL = -1,       /* null pointer, bad size, shape mismatch          */
    KVQ_EUNSUPPORTED = -2, /* valid but not built: head_dim, tile, bits, align */
    KVQ_EWORKSPACE = -3,   /* decode workspace smaller than required          */
    KVQ_ELAUNCH = -4       /* the HIP runtime refused a launch                */
} kvq_status;

/* Order of the codes inside one (page, head) block. */
enum { KVQ_TOKEN_MAJOR = 0, KVQ_CHANNEL_MAJOR = 1 };

/* Bits of *status_flags. */
enum { KVQ_FLAG_NONFINITE = 1u, KVQ_FLAG_SIDE_OVERFLOW = 2u };

typedef struct {
    int32_t head_dim;    /* D: quantized channels (MLA: the latent width)                */
    int32_t rope_dim;    /* R: channels after D kept as bf16 unrotated (MLA rope), else 0 */
    int32_t tile_tokens; /* T: tokens per tile = tokens per page                         */
    int32_t hadamard_n;  /* h: Hadamard block size; power of two dividing D              */
    int32_t group;       /* G: channels per (S, Z) pair; multiple of 8 dividing D        */
    int32_t bits;        /* code width: 2, 3, 4 or 8                                     */
    int32_t iters;       /* normalization rounds (row step then column step), >= 0       */
    int32_t layout;      /* KVQ_TOKEN_MAJOR (keys) or KVQ_CHANNEL_MAJOR (values)          */
    int32_t center;      /* 0: each round scales rows, then columns, to unit RMS about
                            zero (the default reading of the pages' "variance");
                            1: to unit standard deviation about their mean. Only the
                            quantizer reads it; the stored data mean the same either
                            way. 1 runs on the general quantizer kernel only.         */
} kvq_format;

/* One paged quantized cache (K, V, or the MLA latent). Byte layout, per
 * physical page p and head h (P = num_pages, H = num_heads):
 *   codes  [P][H][T*D*bits/8] bytes. The block is one little-endian bitstream
 *          (bit k is bit k%8 of byte k/8); code i of the stream occupies bits
 *          [bits*i, bits*i + bits). Token-major: i = t*D + j. Channel-major:
 *          i = j*T + t.
 *   sz     [P][H][T][D/G][2] fp16: (S, Z) of token t, channel group g.
 *   cnorm  [P][H][D] fp16: normalizer c_j of the tile.
 *   rope   [P][H][T][R] bf16: unrotated copy of channels D..D+R-1; NULL if R == 0.
 * Rows t >= the tile's valid count hold zero codes, S = Z = 0 and zero rope. */
typedef struct {
    kvq_format fmt;
    int32_t num_pages, num_heads;
    uint8_t *codes;
    uint16_t *sz;
    uint16_t *cnorm;
    uint16_t *rope;
} kvq_cache;

/* Parses "kvarn_k{bk}v{bv}_g{T}" (the KVarN preset string, e.g.
 * kvarn_k4v2_g128: 4-bit keys, 2-bit values, 128-token tiles; "KVarN"
 * project review, Key Features, "4-bit Keys, 2-bit Values Preset"). Sets
 * head_dim, tile_tokens and bits; hadamard_n = group = head_dim, iters = 4,
 * rope_dim = 0, center = 0; keys token-major, values channel-major.
 * Returns KVQ_EINVAL for a malformed string or null pointers. */
kvq_status kvq_format_from_preset(const char *preset, int32_t head_dim, kvq_format *k, kvq_format *v);

/* Bytes of codes, sz, cnorm and rope for one cache (the four arrays' sizes
 * summed), or 0 for an invalid format. */
size_t kvq_cache_bytes(const kvq_format *fmt, int32_t num_pages, int32_t num_heads);

/* Quantizes num_tiles tiles for every head into dst.
 * src (device): element (token tau, head h, channel c) is at
 *   src[tau * stride_token + h * stride_head + c], c < D + R, in src_dtype;
 *   strides in elements, multiples of 8, src 16-byte aligned.
 * Tile i reads tokens tile_src_token[i] .. + tile_valid[i] - 1
 *   (0 <= tile_valid[i] <= T) and writes page tile_dst_page[i] of every head;
 *   the three arrays are device int32 [num_tiles]. Statistics use the valid rows
 *   only; the rest of the page is zeroed.
 * status_flags (device, nullable): KVQ_FLAG_* bits are OR-ed in.
 * Supported: D in {64, 128, 256, 512}, T in {16, 32, 64, 128}, bits in
 *   {2, 3, 4, 8}, G a multiple of 8 dividing D, h a power of two in [8, D]
 *   or h = 1; R = 0, or R a multiple of 8 with bf16/f16/f32 input.
 * Errors: KVQ_EINVAL (nulls, negative counts, H != dst->num_heads ...),
 *   KVQ_EUNSUPPORTED (outside the list above), KVQ_ELAUNCH. */
kvq_status kv_quantize(const kvq_cache *dst, const void *src, int32_t src_dtype, int64_t stride_token,
                       int64_t stride_head, int32_t num_tiles, const int32_t *tile_src_token,
                       const int32_t *tile_valid, const int32_t *tile_dst_page, uint32_t *status_flags,
                       hipStream_t stream);

/* The K and V caches of one batch quantized by one launch: the same result as
 * kv_quantize(k_dst, k_src, ...) followed by kv_quantize(v_dst, v_src, ...) with
 * the shared tile arrays and status_flags ("KVarN" project review, Key Features,
 * "Variance-Normalized Quantization Pipeline", applied to keys and values alike).
 * Arguments per cache as for kv_quantize. Taken when both formats fit the
 * 128-channel quantizer: head_dim 128, hadamard_n = group = 128, rope_dim 0,
 * center 0, bf16 sources, 2- or 4-bit codes, 64- or 128-token tiles, keys
 * token-major and values channel-major, both caches with the same tile_tokens,
 * iters and number of heads. Otherwise KVQ_EUNSUPPORTED and nothing is launched
 * (two kv_quantize calls do the work). Errors as for kv_quantize. */
kvq_status kv_quantize_kv(const kvq_cache *k_dst, const kvq_cache *v_dst, const void *k_src, const void *v_src,
                          int32_t src_dtype, int64_t k_stride_token, int64_t k_stride_head, int64_t v_stride_token,
                          int64_t v_stride_head, int32_t num_tiles, const int32_t *tile_src_token,
                          const int32_t *tile_valid, const int32_t *tile_dst_page, uint32_t *status_flags,
                          hipStream_t stream);

/* Rebuilds tiles from the cache: x_hat = ((S code + Z) o c) Q, rope copied.
 * dst (device): [num_tiles][H][T][D + R] in dst_dtype (f32, f16 or bf16); rows
 * t >= tile_valid[i] are written as zero. tile_page, tile_valid: device int32. */
kvq_status kv_dequantize(const kvq_cache *src, int32_t num_tiles, const int32_t *tile_page,
                         const int32_t *tile_valid, void *dst, int32_t dst_dtype, hipStream_t stream);

/* Number of split-K partitions kv_decode_attn uses when num_splits == 0 for
 * these caches (k, v as passed to kv_decode_attn; host structs, device arrays
 * not read) and sizes. The count depends on the kernel the call selects: the
 * pages of each (sequence, kv head) are divided into this many ranges, each
 * producing a partial softmax state that a second pass merges. Returns 1 for
 * invalid arguments. */
int32_t kv_decode_attn_default_splits(const kvq_cache *k, const kvq_cache *v, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t max_seq_len);

/* Bytes at the head of a kv_decode_attn workspace that hold split-merge arrival
 * counters (one 32-bit counter per sequence and kv head, up to 16384 of them). */
#define KVQ_DECODE_COUNTER_BYTES (64u << 10)

/* Workspace bytes kv_decode_attn needs for these sizes (num_splits >= 1):
 * KVQ_DECODE_COUNTER_BYTES plus num_seqs * num_q_heads * num_splits *
 * (head_dim_v + 2) floats of split partials. */
size_t kv_decode_attn_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim_v,
                                      int32_t num_splits);

/* Decode attention of one new query per sequence over the paged quantized
 * cache: out[s][hq] = softmax_t(sm_scale <q[s][hq], k_t>) applied to v_t, over
 * t < seq_lens[s], with k_t, v_t the dequantized rows reached through
 * block_table[s][t / T] (row t % T). Query head hq reads kv head
 * hq / (num_q_heads / H). When v == NULL (MLA), k's latent (first D channels
 * of each dequantized row) is also the value and k's rope channels take part
 * in the score only.
 *   q (device): [num_seqs][num_q_heads][D + R] in q_dtype.
 *   block_table (device int32): [num_seqs][block_table_stride].
 *   seq_lens (device int32): [num_seqs], each in [0, max_seq_len].
 *   out (device fp32): [num_seqs][num_q_heads][Dv], Dv = (v ? v : k)->fmt.head_dim.
 *   workspace (device): at least kv_decode_attn_workspace_bytes(...) bytes,
 *     4-byte aligned. Its first KVQ_DECODE_COUNTER_BYTES bytes are counters that
 *     must be zero when the workspace is first used (a zero-filled allocation, or
 *     one clear after allocating it); every call leaves them zero, and
 *     kv_prefill_attn never writes them, so a workspace stays ready between calls
 *     of both. Other writes to those bytes require clearing them again. The rest
 *     is overwritten. On the matrix-core kernels (128-channel K and V), when the
 *     grid of num_seqs * H * splits workgroups is at most 512 (one round on the
 *     chip), the last workgroup to finish among the splits of each (sequence,
 *     kv head) merges them (it counts arrivals there); larger grids and the other
 *     kernels merge in a second kernel. Calls that overlap in time must use
 *     different workspaces.
 * The score rotation and normalizer fold is exact in real arithmetic; in fp32
 * the result differs from fp64 dequantize-then-attention by rounding only.
 * Errors: KVQ_EINVAL, KVQ_EUNSUPPORTED (layouts: K token-major, V channel-major,
 * MLA latent token-major; T in {16, 32, 64, 128}; num_seqs above 65535 except
 * for MLA), KVQ_EWORKSPACE, KVQ_ELAUNCH. */
kvq_status kv_decode_attn(const void *q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                          const kvq_cache *k, const kvq_cache *v, const int32_t *block_table,
                          int32_t block_table_stride, const int32_t *seq_lens, int32_t max_seq_len,
                          float sm_scale, int32_t num_splits, void *workspace, size_t workspace_bytes,
                          float *out, hipStream_t stream);

/* Size of kv_decode_attn_noalloc's scratch array (bytes, per GPU). */
#define KVQ_NOALLOC_SCRATCH_BYTES (64u << 20)

/* kv_decode_attn for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * result, kernels and split rule, with the split-K partials in a scratch array
 * that the library holds in every GPU's memory (KVQ_NOALLOC_SCRATCH_BYTES, held
 * until the process ends) instead of a caller workspace. The call allocates
 * nothing; the caller still passes q, the caches, the tables and out.
 * The first call on a device looks up that device's copy of the array (with the
 * device current) and clears its split-merge counters (a kernel on `stream`,
 * ahead of the decode); later calls reuse the address. The array keeps the last
 * call's partials: calls on one GPU that overlap in time (different streams, or
 * host threads) race on it and must be ordered by the caller.
 * Errors: as kv_decode_attn; KVQ_EWORKSPACE when the partials,
 * kv_decode_attn_workspace_bytes(num_seqs, num_q_heads, Dv, splits), exceed
 * KVQ_NOALLOC_SCRATCH_BYTES (nothing is launched); KVQ_ELAUNCH when the runtime
 * does not give the array's device address. */
kvq_status kv_decode_attn_noalloc(const void *q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                                  const kvq_cache *k, const kvq_cache *v, const int32_t *block_table,
                                  int32_t block_table_stride, const int32_t *seq_lens, int32_t max_seq_len,
                                  float sm_scale, int32_t num_splits, float *out, hipStream_t stream);

/* Append one new token per sequence to a paged quantized cache, keeping every
 * token in it: the token's row goes into the sequence's partial last tile and
 * that tile is quantized again from its unquantized rows (the method's
 * statistics are per tile: "KVarN" project review, Key Features,
 * "Variance-Normalized Quantization Pipeline"). After the call, page
 * block_table[s][L / T] (L = seq_lens[s]) holds the quantization of the
 * sequence's tokens T*(L/T) .. L, exactly what kv_quantize gives for that tile.
 *   tail (device, caller-owned, read and written): [num_seqs][T][H][D + R] in
 *     dtype; row r of sequence s holds token T*(L/T) + r of s. The call writes
 *     row L % T; rows below it must hold the sequence's earlier tokens of the
 *     tile (they do when every token was appended through this call, or the
 *     caller copied them in). 16-byte aligned.
 *   new_tokens (device): element (s, h, e) at s*new_stride_seq +
 *     h*new_stride_head + e, e < D + R, in dtype.
 *   seq_lens (device int32): [num_seqs], the lengths BEFORE the append; not
 *     modified (the caller increments). A negative length skips the sequence.
 *   block_table (device int32): [num_seqs][block_table_stride]; a page index
 *     L / T outside the row, or a page number outside [0, num_pages), leaves
 *     the cache unchanged for that sequence (the tail row is still written).
 *   workspace (device): at least kv_append_workspace_bytes(num_seqs) bytes,
 *     4-byte aligned; overwritten.
 *   status_flags: as for kv_quantize.
 * Errors: KVQ_EINVAL, KVQ_EUNSUPPORTED (as kv_quantize), KVQ_EWORKSPACE,
 * KVQ_ELAUNCH. Calls on one stream are ordered; two appends to one sequence
 * must not run concurrently. */
kvq_status kv_append(const kvq_cache *dst, void *tail, int32_t dtype, const void *new_tokens,
                     int64_t new_stride_seq, int64_t new_stride_head, int32_t num_seqs,
                     const int32_t *seq_lens, const int32_t *block_table, int32_t block_table_stride,
                     void *workspace, size_t workspace_bytes, uint32_t *status_flags, hipStream_t stream);

/* Workspace bytes kv_append needs for num_seqs sequences (0 for negative). */
size_t kv_append_workspace_bytes(int32_t num_seqs);

/* Name of the GPU kernel kv_quantize runs for these arguments (the same checks
 * and dispatch; nothing is launched or dereferenced): "quantize_d128_kernel",
 * "quantize_t16_kernel", "quantize_d512_kernel" (specialised tile shapes) or
 * "quantize_kernel" (any supported format). NULL where kv_quantize would
 * reject the arguments. The string is static. For profilers and benchmarks. */
const char *kv_quantize_kernel_name(const kvq_cache *dst, const void *src, int32_t src_dtype,
                                    int64_t stride_token, int64_t stride_head);

/* Name of the main GPU kernel kv_decode_attn runs for this query pointer and
 * these caches: "decode_mla_kernel", "decode_pair16_kernel" (16-token pages, at
 * most 8 query heads per kv head: two pages per matrix-core pass),
 * "decode_mfma_kernel" or "decode_generic_kernel". NULL for invalid arguments.
 * The string is static. For profilers and benchmarks. */
const char *kv_decode_attn_kernel_name(const void *q, const kvq_cache *k, const kvq_cache *v,
                                       int32_t num_q_heads);

/* Name of the split-merge kernel kv_decode_attn launches after the main kernel
 * for these arguments (num_splits as passed to it, 0 = the default rule for
 * max_seq_len): "decode_reduce_kernel", or "" when the main kernel merges the
 * splits itself (see kv_decode_attn's workspace). NULL for invalid arguments.
 * The string is static. For profilers and benchmarks. */
const char *kv_decode_attn_merge_kernel_name(const void *q, const kvq_cache *k, const kvq_cache *v,
                                             int32_t num_seqs, int32_t num_q_heads, int32_t num_splits,
                                             int32_t max_seq_len);

/* Chunked prefill attention over the paged quantized cache. Each sequence b
 * ends with a chunk of chunk_len query positions whose keys and values are
 * already in the cache (its last chunk_len tokens); position i of the chunk
 * attends causally to tokens 0 .. seq_lens[b] - chunk_len + i (a position with
 * no token left gives zeros, the result of an empty decode). The result per
 * (b, i) is kv_decode_attn's for that query over that prefix, with the same fold
 * (scores and values from the codes, normalizers folded into the query and the
 * output). Formats that kv_decode_attn runs on "decode_mfma_kernel" or
 * "decode_pair16_kernel" run decode_mfma_kernel in its chunk mode (the MFMA columns hold (position, head) pairs, so one
 * page read serves 16 / (num_q_heads / H) positions); other formats run the
 * chunk positions as chunk_len virtual sequences sharing b's block-table row.
 *   q (device): [num_seqs][chunk_len][num_q_heads][D + R] in q_dtype.
 *   seq_lens (device int32): [num_seqs], total lengths including the chunk.
 *   out (device fp32): [num_seqs][chunk_len][num_q_heads][Dv].
 *   workspace (device): at least kv_prefill_attn_workspace_bytes(...) bytes,
 *     256-byte aligned; holds the split partials, the virtual block table and
 *     the virtual lengths after KVQ_DECODE_COUNTER_BYTES bytes that it leaves
 *     untouched (kv_decode_attn's counters, when the workspace also serves it).
 *   num_splits: 0 = kv_prefill_attn_default_splits(...).
 * Other arguments and errors as kv_decode_attn; KVQ_EUNSUPPORTED when
 * num_seqs * chunk_len exceeds 2^24. */
kvq_status kv_prefill_attn(const void *q, int32_t q_dtype, int32_t num_seqs, int32_t chunk_len,
                           int32_t num_q_heads, const kvq_cache *k, const kvq_cache *v,
                           const int32_t *block_table, int32_t block_table_stride, const int32_t *seq_lens,
                           int32_t max_seq_len, float sm_scale, int32_t num_splits, void *workspace,
                           size_t workspace_bytes, float *out, hipStream_t stream);

/* Workspace bytes of kv_prefill_attn (num_splits >= 1); 0 for invalid sizes. */
size_t kv_prefill_attn_workspace_bytes(int32_t num_seqs, int32_t chunk_len, int32_t num_q_heads,
                                       int32_t head_dim_v, int32_t num_splits, int32_t block_table_stride);

/* Split count kv_prefill_attn uses for num_splits = 0 (1 for invalid arguments). */
int32_t kv_prefill_attn_default_splits(const kvq_cache *k, const kvq_cache *v, int32_t num_seqs,
                                       int32_t chunk_len, int32_t num_q_heads, int32_t max_seq_len);

/* Name of the main GPU kernel kv_prefill_attn runs for this query pointer and
 * these caches ("decode_mfma_kernel" in its chunk mode, else the decode kernel
 * the virtual sequences run on); the split merge, "decode_reduce_kernel",
 * follows it. NULL for invalid arguments. The string is static. */
const char *kv_prefill_attn_kernel_name(const void *q, const kvq_cache *k, const kvq_cache *v,
                                        int32_t num_q_heads);

/* Static description of a status code. */
const char *kvq_status_str(int32_t s);

#ifdef __cplusplus
}
#endif
#endif
