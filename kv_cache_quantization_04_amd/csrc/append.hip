// Append path: one new token per sequence goes into the sequence's partial last
// tile, and that tile is quantized again from its unquantized rows, so the paged
// cache always holds every token (the decode kernels read it unchanged).
//
// The unquantized rows of each sequence's current tile live in a caller-owned
// "tail" buffer [num_seqs][T][H][D + R] in the source dtype. A first kernel
// writes the new token's row into the tail at row seq_len % T and fills the
// tile descriptors of the re-quantization (source token, valid rows, destination
// page through the block table); the quantizer then runs over one tile per
// sequence. The method quantizes a tile from all of its valid rows ("KVarN"
// project review, Key Features, "Variance-Normalized Quantization Pipeline":
// statistics per tile), so a partial tile is re-encoded whole.
#include "common.h"
#include "launch.h"

namespace kvq {

namespace {

constexpr int ANT = 256;

// One workgroup per sequence: copies the new row (H * W elements) and writes
// the sequence's tile descriptor. A negative length, or a page index past the
// block table row, leaves the tile invalid (destination -1: the quantizer
// skips it).
__global__ void __launch_bounds__(ANT) append_prep_kernel(AppendArgs a) {
    const int s = blockIdx.x;
    const int len = a.seq_lens[s];
    const int rowlen = a.H * a.W;  // elements of one token row in the tail
    if (len >= 0) {
        const int pos = len % a.T;
        const int64_t dst0 = ((int64_t)s * a.T + pos) * rowlen;
        for (int i = threadIdx.x; i < rowlen; i += ANT) {
            const int h = i / a.W, e = i - h * a.W;
            const int64_t src = (int64_t)s * a.new_stride_seq + (int64_t)h * a.new_stride_head + e;
            if (a.esize == 4)
                reinterpret_cast<uint32_t *>(a.tail)[dst0 + i] = reinterpret_cast<const uint32_t *>(a.new_tokens)[src];
            else
                reinterpret_cast<uint16_t *>(a.tail)[dst0 + i] = reinterpret_cast<const uint16_t *>(a.new_tokens)[src];
        }
    }
    if (threadIdx.x == 0) {
        const int pidx = len >= 0 ? len / a.T : -1;
        a.tile_src_token[s] = s * a.T;
        a.tile_valid[s] = len >= 0 ? len % a.T + 1 : 0;
        a.tile_dst_page[s] = (pidx >= 0 && pidx < a.bt_stride) ? a.block_table[(int64_t)s * a.bt_stride + pidx] : -1;
    }
}

}  // namespace

bool launch_append(const AppendArgs &a, int D, int T, const QuantArgs &q, hipStream_t stream) {
    hipLaunchKernelGGL(append_prep_kernel, dim3(a.num_seqs), dim3(ANT), 0, stream, a);
    return launch_quantize(D, T, a.num_seqs, q, stream);
}

}  // namespace kvq
