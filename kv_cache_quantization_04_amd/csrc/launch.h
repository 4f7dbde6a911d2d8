// Argument blocks and launchers shared by the host API and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

struct QuantArgs {
    const void *src;
    int dtype;
    int64_t stride_token, stride_head;
    const int32_t *tile_src_token, *tile_valid, *tile_dst_page;
    uint8_t *codes;
    uint16_t *sz, *cnorm, *rope;
    int H, h, G, bits, iters, layout, R, num_pages;
    uint32_t *flags;
    int center;  // 1: rounds use the standard deviation about the mean
};

struct DequantArgs {
    const uint8_t *codes;
    const uint16_t *sz, *cnorm, *rope;
    const int32_t *tile_page, *tile_valid;
    void *dst;
    int dtype;
    int H, h, G, bits, layout, R, num_pages;
};

struct DecodeArgs {
    const void *q;
    int q_dtype;
    int B, Hq, Hkv, grp, hc, nhc;
    // K (or MLA latent) cache
    const uint8_t *kcodes;
    const uint16_t *ksz, *kcn, *krope;
    int D, R, kG, kbits, kh, klayout;
    // V cache (the K cache itself for MLA)
    const uint8_t *vcodes;
    const uint16_t *vsz, *vcn;
    int Dv, vG, vbits, vh, vlayout, vH;
    int T, num_pages;
    const int32_t *bt;
    int bt_stride;
    const int32_t *seq_lens;
    float sm;
    int splits;
    float *ws;
    // arrival counters of the in-kernel split merge, one per (sequence, kv head), zero
    // between calls; null: the reduce kernel merges
    uint32_t *cnt;
    float *out;
    // chunked prefill on the MFMA kernel: Lq > 0 query positions per sequence (q rows
    // [B][Lq][Hq]), position i attending to tokens 0 .. seq_lens[b] - Lq + i; the
    // workspace and the reduce run over B * Lq rows. 0 for decode.
    int Lq;
    // longest sequence the caller names (host-side launch choices only)
    int max_len;
};

// append path: new token rows -> tail buffer, tile descriptors -> workspace
struct AppendArgs {
    const void *new_tokens;
    int64_t new_stride_seq, new_stride_head;  // elements
    void *tail;                               // [num_seqs][T][H][W]
    int esize;                                // bytes per element
    int num_seqs, T, H, W;                    // W = D + R
    const int32_t *seq_lens, *block_table;
    int bt_stride;
    int32_t *tile_src_token, *tile_valid, *tile_dst_page;  // [num_seqs] each
};

// chunked prefill: virtual block table and lengths for B * Lq virtual sequences
struct PrefillArgs {
    int num_seqs, Lq;
    const int32_t *seq_lens, *block_table;
    int bt_stride;
    int32_t *vbt, *vlens;  // workspace: [num_seqs * Lq][bt_stride], [num_seqs * Lq]
};

bool launch_quantize(int D, int T, int num_tiles, const QuantArgs &a, hipStream_t stream);
// K and V of one batch in one launch; false (nothing launched) outside the formats it takes
bool quantize_pair_supported(int D, int T, const QuantArgs &k, const QuantArgs &v);
bool launch_quantize_pair(int D, int T, int num_tiles, const QuantArgs &k, const QuantArgs &v, hipStream_t stream);
bool launch_append(const AppendArgs &a, int D, int T, const QuantArgs &q, hipStream_t stream);
bool launch_prefill(const PrefillArgs &p, const DecodeArgs &d, hipStream_t stream);
// split-K partitions and main kernel of a prefill call (d.B = real sequences)
int prefill_default_splits(const DecodeArgs &d, int Lq, int max_seq_len);
const char *prefill_kernel_name(const DecodeArgs &d);
bool launch_dequant(int D, int T, int num_tiles, const DequantArgs &a, hipStream_t stream);
bool launch_decode(const DecodeArgs &a, hipStream_t stream);
// split-K partitions for a decode call whose fields other than q, block table,
// lengths, splits and buffers are filled in
int decode_default_splits(const DecodeArgs &a, int max_seq_len);
int decode_chunk_splits(const DecodeArgs &a, int max_seq_len);
// name of the main kernel launch_quantize / launch_decode would run for these arguments
const char *quantize_kernel_name(int D, int T, const QuantArgs &a);
const char *decode_kernel_name(const DecodeArgs &a);

}  // namespace kvq
