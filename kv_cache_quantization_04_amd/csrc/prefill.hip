// Chunked prefill attention over the paged quantized cache: each sequence has
// a chunk of Lq new query positions whose keys and values are already in the
// cache (appended or quantized), the chunk being the last Lq tokens of the
// sequence. Position i of sequence b attends causally to the sequence's tokens
// 0 .. L_b - Lq + i.
//
// Formats of the GQA MFMA decode kernel run it in its chunk mode: the MFMA
// columns hold (position, head) pairs, so a page read serves 16 / g positions.
// Other formats run as decode attention over B * Lq virtual sequences that share
// their sequence's block-table row: a first kernel writes the virtual block
// table and lengths into the workspace, then the decode kernels (split-K, folded
// scores and values) run unchanged, in launches of at most 65535 virtual
// sequences.
#include "common.h"
#include "launch.h"

namespace kvq {

namespace {

constexpr int PNT = 256;

// one workgroup per virtual sequence v = b * Lq + i
__global__ void __launch_bounds__(PNT) prefill_prep_kernel(PrefillArgs a) {
    const int v = blockIdx.x;
    const int b = v / a.Lq, i = v - b * a.Lq;
    const int32_t *src = a.block_table + (int64_t)b * a.bt_stride;
    int32_t *dst = a.vbt + (int64_t)v * a.bt_stride;
    for (int j = threadIdx.x; j < a.bt_stride; j += PNT) dst[j] = src[j];
    if (threadIdx.x == 0) {
        const int L = a.seq_lens[b] - a.Lq + i + 1;
        a.vlens[v] = L > 0 ? L : 0;
    }
}

}  // namespace

bool decode_mfma_supported(const DecodeArgs &a);
bool launch_decode_chunk(const DecodeArgs &a, hipStream_t stream);

// d: the decode arguments over the B * Lq virtual sequences (virtual table and
// lengths in the workspace), Lq = 0
bool launch_prefill(const PrefillArgs &p, const DecodeArgs &d, hipStream_t stream) {
    if (decode_mfma_supported(d)) {
        DecodeArgs c = d;
        c.B = p.num_seqs;
        c.Lq = p.Lq;
        c.bt = p.block_table;
        c.seq_lens = p.seq_lens;
        return launch_decode_chunk(c, stream);
    }
    const int nv = p.num_seqs * p.Lq;
    hipLaunchKernelGGL(prefill_prep_kernel, dim3(nv), dim3(PNT), 0, stream, p);
    const int qw = d.D + d.R, qes = d.q_dtype == KVQ_F32 ? 4 : 2;
    for (int v0 = 0; v0 < nv; v0 += 65535) {
        DecodeArgs a = d;
        a.B = min(65535, nv - v0);
        a.q = static_cast<const uint8_t *>(d.q) + (int64_t)v0 * d.Hq * qw * qes;
        a.bt = d.bt + (int64_t)v0 * d.bt_stride;
        a.seq_lens = d.seq_lens + v0;
        a.ws = d.ws + (int64_t)v0 * d.Hq * d.splits * (d.Dv + 2);
        a.out = d.out + (int64_t)v0 * d.Hq * d.Dv;
        if (!launch_decode(a, stream)) return false;
    }
    return true;
}

int prefill_default_splits(const DecodeArgs &d, int Lq, int max_seq_len) {
    DecodeArgs a = d;
    if (decode_mfma_supported(a)) {
        // as decode, counting the chunk's column blocks as sequences
        a.B = d.B * ((Lq * d.grp + 15) / 16);
        return decode_chunk_splits(a, max_seq_len);
    }
    a.B = d.B * Lq;
    return decode_chunk_splits(a, max_seq_len);
}

// the chunk mode runs decode_mfma_kernel for every format it takes (also those whose
// decode takes two pages per pass); other formats run their decode kernel
const char *prefill_kernel_name(const DecodeArgs &d) {
    return decode_mfma_supported(d) ? "decode_mfma_kernel" : decode_kernel_name(d);
}

}  // namespace kvq
