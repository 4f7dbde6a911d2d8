// Chunked prefill attention over the paged quantized cache: each sequence has
// a chunk of Lq new query positions whose keys and values are already in the
// cache (appended or quantized), the chunk being the last Lq tokens of the
// sequence. Position i of sequence b attends causally to the sequence's tokens
// 0 .. L_b - Lq + i. It is computed as decode attention over B * Lq virtual
// sequences that share their sequence's block-table row: a first kernel writes
// the virtual block table and lengths into the workspace, then the decode
// kernels (split-K, folded scores and values) run unchanged.
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

bool launch_prefill(const PrefillArgs &p, const DecodeArgs &d, hipStream_t stream) {
    hipLaunchKernelGGL(prefill_prep_kernel, dim3(p.num_seqs * p.Lq), dim3(PNT), 0, stream, p);
    return launch_decode(d, stream);
}

}  // namespace kvq
