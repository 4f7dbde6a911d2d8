// C ABI of libkvq.so: host-side validation and launch.
#include <cstdio>
#include <cstring>
#include <mutex>

#include "common.h"

#include "launch.h"

namespace kvq {
// the decode kernel merges its split partials itself (no reduce kernel follows)
bool decode_merges_in_kernel(const DecodeArgs &a);
}  // namespace kvq

namespace {

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

kvq_status check_format(const kvq_format *f) {
    if (!f) return KVQ_EINVAL;
    const int D = f->head_dim, T = f->tile_tokens;
    if (D <= 0 || T <= 0 || f->bits <= 0 || f->group <= 0 || f->hadamard_n <= 0 || f->iters < 0 ||
        f->rope_dim < 0)
        return KVQ_EINVAL;
    if (f->layout != KVQ_TOKEN_MAJOR && f->layout != KVQ_CHANNEL_MAJOR) return KVQ_EINVAL;
    if (D % f->group != 0 || D % f->hadamard_n != 0 || !is_pow2(f->hadamard_n)) return KVQ_EINVAL;
    if (!(D == 64 || D == 128 || D == 256 || D == 512)) return KVQ_EUNSUPPORTED;
    if (!(T == 16 || T == 32 || T == 64 || T == 128)) return KVQ_EUNSUPPORTED;
    if (!(f->bits == 2 || f->bits == 3 || f->bits == 4 || f->bits == 8)) return KVQ_EUNSUPPORTED;
    if (f->group % 8 != 0) return KVQ_EUNSUPPORTED;
    if (f->rope_dim % 8 != 0) return KVQ_EUNSUPPORTED;
    if (f->iters > 64) return KVQ_EUNSUPPORTED;
    if (f->center != 0 && f->center != 1) return KVQ_EINVAL;
    return KVQ_OK;
}

kvq_status check_cache(const kvq_cache *c) {
    if (!c) return KVQ_EINVAL;
    kvq_status st = check_format(&c->fmt);
    if (st != KVQ_OK) return st;
    if (c->num_pages < 0 || c->num_heads <= 0) return KVQ_EINVAL;
    if (!c->codes || !c->sz || !c->cnorm) return KVQ_EINVAL;
    if (c->fmt.rope_dim > 0 && !c->rope) return KVQ_EINVAL;
    if (((uintptr_t)c->codes & 3) || ((uintptr_t)c->sz & 3)) return KVQ_EUNSUPPORTED;
    return KVQ_OK;
}

bool valid_dtype(int d) { return d == KVQ_F32 || d == KVQ_F16 || d == KVQ_BF16; }

kvq_status launched() { return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ELAUNCH; }

// Format-dependent fields of a decode call over validated caches: GQA grouping,
// the K (or MLA latent) cache and the V cache (the latent itself when v is NULL).
kvq_status decode_layout(const kvq_cache *k, const kvq_cache *v, int32_t num_q_heads, kvq::DecodeArgs &a) {
    const kvq_format &fk = k->fmt;
    const kvq_format &fv = v ? v->fmt : k->fmt;
    if (num_q_heads <= 0 || num_q_heads % k->num_heads != 0) return KVQ_EINVAL;
    if (v) {
        if (v->num_heads != k->num_heads || fv.tile_tokens != fk.tile_tokens || v->num_pages != k->num_pages)
            return KVQ_EINVAL;
        if (fk.rope_dim != 0 || fv.rope_dim != 0) return KVQ_EUNSUPPORTED;
        if (fk.layout != KVQ_TOKEN_MAJOR || fv.layout != KVQ_CHANNEL_MAJOR) return KVQ_EUNSUPPORTED;
    } else {
        if (fk.layout != KVQ_TOKEN_MAJOR) return KVQ_EUNSUPPORTED;
    }
    a.Hq = num_q_heads;
    a.Hkv = k->num_heads;
    a.grp = num_q_heads / k->num_heads;
    a.hc = a.grp < 16 ? a.grp : 16;
    if (a.grp % a.hc != 0) return KVQ_EUNSUPPORTED;
    a.nhc = a.grp / a.hc;
    a.kcodes = k->codes;
    a.ksz = k->sz;
    a.kcn = k->cnorm;
    a.krope = k->rope;
    a.D = fk.head_dim;
    a.R = fk.rope_dim;
    a.kG = fk.group;
    a.kbits = fk.bits;
    a.kh = fk.hadamard_n;
    a.klayout = fk.layout;
    const kvq_cache *vc = v ? v : k;
    a.vcodes = vc->codes;
    a.vsz = vc->sz;
    a.vcn = vc->cnorm;
    a.Dv = fv.head_dim;
    a.vG = fv.group;
    a.vbits = fv.bits;
    a.vh = fv.hadamard_n;
    a.vlayout = fv.layout;
    a.vH = vc->num_heads;
    a.T = fk.tile_tokens;
    a.num_pages = k->num_pages;
    return KVQ_OK;
}

// checks of kv_quantize's cache and source arguments
kvq_status check_quantize_source(const kvq_cache *dst, const void *src, int32_t src_dtype, int64_t stride_token,
                                 int64_t stride_head) {
    kvq_status st = check_cache(dst);
    if (st != KVQ_OK) return st;
    if (!src || !valid_dtype(src_dtype) || stride_token < 0 || stride_head < 0) return KVQ_EINVAL;
    if (((uintptr_t)src & 15) || (stride_token % 8) || (stride_head % 8)) return KVQ_EUNSUPPORTED;
    return KVQ_OK;
}

kvq::QuantArgs quant_args(const kvq_cache *dst, const void *src, int32_t src_dtype, int64_t stride_token,
                          int64_t stride_head, const int32_t *tile_src_token, const int32_t *tile_valid,
                          const int32_t *tile_dst_page, uint32_t *status_flags) {
    const kvq_format &f = dst->fmt;
    return kvq::QuantArgs{src, (int)src_dtype, stride_token, stride_head, tile_src_token, tile_valid, tile_dst_page,
                          dst->codes, dst->sz, dst->cnorm, dst->rope, dst->num_heads, f.hadamard_n, f.group, f.bits,
                          f.iters, f.layout, f.rope_dim, dst->num_pages, status_flags, f.center};
}

// Split-K partials of kv_decode_attn_noalloc: a file-scope device array, one copy
// per GPU the library runs on, held until the process ends. In host code `scratch`
// names a host-side stand-in, never the device memory: the per-device address comes
// from hipGetSymbolAddress (taken once per device, with that device current) and only
// that address is passed to kernels. Its head holds the split-merge arrival counters,
// cleared on the device's first call (by a kernel on the caller's stream) and left at
// zero by every call; no kernel reads a partial it has not written.
static __device__ __align__(256) uint8_t scratch[KVQ_NOALLOC_SCRATCH_BYTES];

__global__ void clear_words_kernel(uint32_t *p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex scratch_mu;
void *scratch_ptr[SCRATCH_MAX_DEVICES] = {};

// Device address of `scratch` on the device `stream` belongs to (the current device
// for the null stream), or nullptr when the runtime does not give it.
void *scratch_for(hipStream_t stream) {
    int dev = -1, cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    dev = cur;
    if (stream != nullptr) {
        hipDevice_t sd;
        if (hipStreamGetDevice(stream, &sd) != hipSuccess) return nullptr;
        dev = (int)sd;
    }
    if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (scratch_ptr[dev]) return scratch_ptr[dev];
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return nullptr;
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e == hipSuccess && ptr) {
        // (a launch error surfaces in the caller's launch check)
        constexpr int nw = KVQ_DECODE_COUNTER_BYTES / 4;
        hipLaunchKernelGGL(clear_words_kernel, dim3((nw + 255) / 256), dim3(256), 0, stream, (uint32_t *)ptr, nw);
    }
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || !ptr) return nullptr;
    scratch_ptr[dev] = ptr;
    return ptr;
}

// kv_decode_attn after its workspace is known (nullptr with `have_ws` false: the
// noalloc scratch, resolved after every host-side check has passed)
kvq_status decode_attn_impl(const void *q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                            const kvq_cache *k, const kvq_cache *v, const int32_t *block_table,
                            int32_t block_table_stride, const int32_t *seq_lens, int32_t max_seq_len, float sm_scale,
                            int32_t num_splits, void *workspace, size_t workspace_bytes, bool have_ws, float *out,
                            hipStream_t stream);

}  // namespace

extern "C" {

const char *kvq_status_str(int32_t s) {
    switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_EINVAL: return "invalid argument";
    case KVQ_EUNSUPPORTED: return "unsupported configuration";
    case KVQ_EWORKSPACE: return "workspace too small";
    case KVQ_ELAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

kvq_status kvq_format_from_preset(const char *preset, int32_t head_dim, kvq_format *k, kvq_format *v) {
    if (!preset || !k || !v || head_dim <= 0) return KVQ_EINVAL;
    int bk = 0, bv = 0, T = 0, used = 0;
    if (std::sscanf(preset, "kvarn_k%dv%d_g%d%n", &bk, &bv, &T, &used) != 3 || preset[used] != '\0')
        return KVQ_EINVAL;
    if (bk <= 0 || bv <= 0 || T <= 0) return KVQ_EINVAL;
    *k = kvq_format{head_dim, 0, T, head_dim, head_dim, bk, 4, KVQ_TOKEN_MAJOR, 0};
    *v = kvq_format{head_dim, 0, T, head_dim, head_dim, bv, 4, KVQ_CHANNEL_MAJOR, 0};
    return KVQ_OK;
}

size_t kvq_cache_bytes(const kvq_format *f, int32_t num_pages, int32_t num_heads) {
    if (check_format(f) != KVQ_OK || num_pages < 0 || num_heads <= 0) return 0;
    const size_t ph = (size_t)num_pages * num_heads;
    const size_t T = f->tile_tokens, D = f->head_dim;
    return ph * (T * D * f->bits / 8 + T * (D / f->group) * 4 + D * 2 + T * f->rope_dim * 2);
}

kvq_status kv_quantize(const kvq_cache *dst, const void *src, int32_t src_dtype, int64_t stride_token,
                       int64_t stride_head, int32_t num_tiles, const int32_t *tile_src_token,
                       const int32_t *tile_valid, const int32_t *tile_dst_page, uint32_t *status_flags,
                       hipStream_t stream) {
    kvq_status st = check_quantize_source(dst, src, src_dtype, stride_token, stride_head);
    if (st != KVQ_OK) return st;
    if (num_tiles < 0) return KVQ_EINVAL;
    if (num_tiles > 0 && (!tile_src_token || !tile_valid || !tile_dst_page)) return KVQ_EINVAL;
    if (num_tiles == 0) return KVQ_OK;
    const kvq_format &f = dst->fmt;
    const kvq::QuantArgs a = quant_args(dst, src, src_dtype, stride_token, stride_head, tile_src_token, tile_valid,
                                        tile_dst_page, status_flags);
    if (!kvq::launch_quantize(f.head_dim, f.tile_tokens, num_tiles, a, stream)) return KVQ_EUNSUPPORTED;
    return launched();
}

kvq_status kv_quantize_kv(const kvq_cache *k_dst, const kvq_cache *v_dst, const void *k_src, const void *v_src,
                          int32_t src_dtype, int64_t k_stride_token, int64_t k_stride_head, int64_t v_stride_token,
                          int64_t v_stride_head, int32_t num_tiles, const int32_t *tile_src_token,
                          const int32_t *tile_valid, const int32_t *tile_dst_page, uint32_t *status_flags,
                          hipStream_t stream) {
    kvq_status st = check_quantize_source(k_dst, k_src, src_dtype, k_stride_token, k_stride_head);
    if (st != KVQ_OK) return st;
    if ((st = check_quantize_source(v_dst, v_src, src_dtype, v_stride_token, v_stride_head)) != KVQ_OK) return st;
    if (num_tiles < 0) return KVQ_EINVAL;
    if (num_tiles > 0 && (!tile_src_token || !tile_valid || !tile_dst_page)) return KVQ_EINVAL;
    const kvq_format &fk = k_dst->fmt, &fv = v_dst->fmt;
    if (fk.head_dim != fv.head_dim || fk.tile_tokens != fv.tile_tokens || k_dst->num_pages != v_dst->num_pages)
        return KVQ_EUNSUPPORTED;
    const kvq::QuantArgs ak = quant_args(k_dst, k_src, src_dtype, k_stride_token, k_stride_head, tile_src_token,
                                         tile_valid, tile_dst_page, status_flags);
    const kvq::QuantArgs av = quant_args(v_dst, v_src, src_dtype, v_stride_token, v_stride_head, tile_src_token,
                                         tile_valid, tile_dst_page, status_flags);
    if (!kvq::quantize_pair_supported(fk.head_dim, fk.tile_tokens, ak, av)) return KVQ_EUNSUPPORTED;
    if (num_tiles == 0) return KVQ_OK;
    if (!kvq::launch_quantize_pair(fk.head_dim, fk.tile_tokens, num_tiles, ak, av, stream)) return KVQ_EUNSUPPORTED;
    return launched();
}

const char *kv_quantize_kernel_name(const kvq_cache *dst, const void *src, int32_t src_dtype, int64_t stride_token,
                                    int64_t stride_head) {
    if (check_quantize_source(dst, src, src_dtype, stride_token, stride_head) != KVQ_OK) return nullptr;
    const kvq::QuantArgs a =
        quant_args(dst, src, src_dtype, stride_token, stride_head, nullptr, nullptr, nullptr, nullptr);
    return kvq::quantize_kernel_name(dst->fmt.head_dim, dst->fmt.tile_tokens, a);
}

kvq_status kv_dequantize(const kvq_cache *src, int32_t num_tiles, const int32_t *tile_page, const int32_t *tile_valid,
                         void *dst, int32_t dst_dtype, hipStream_t stream) {
    kvq_status st = check_cache(src);
    if (st != KVQ_OK) return st;
    if (!dst || num_tiles < 0 || !valid_dtype(dst_dtype)) return KVQ_EINVAL;
    if (num_tiles > 0 && (!tile_page || !tile_valid)) return KVQ_EINVAL;
    if (num_tiles == 0) return KVQ_OK;
    const kvq_format &f = src->fmt;
    kvq::DequantArgs a{src->codes, src->sz, src->cnorm, src->rope, tile_page, tile_valid, dst, (int)dst_dtype,
                       src->num_heads, f.hadamard_n, f.group, f.bits, f.layout, f.rope_dim, src->num_pages};
    if (!kvq::launch_dequant(f.head_dim, f.tile_tokens, num_tiles, a, stream)) return KVQ_EUNSUPPORTED;
    return launched();
}

size_t kv_append_workspace_bytes(int32_t num_seqs) {
    if (num_seqs < 0) return 0;
    return (size_t)3 * num_seqs * sizeof(int32_t);
}

kvq_status kv_append(const kvq_cache *dst, void *tail, int32_t dtype, const void *new_tokens,
                     int64_t new_stride_seq, int64_t new_stride_head, int32_t num_seqs, const int32_t *seq_lens,
                     const int32_t *block_table, int32_t block_table_stride, void *workspace, size_t workspace_bytes,
                     uint32_t *status_flags, hipStream_t stream) {
    kvq_status st = check_cache(dst);
    if (st != KVQ_OK) return st;
    if (!tail || !new_tokens || !valid_dtype(dtype) || num_seqs < 0) return KVQ_EINVAL;
    if (new_stride_seq < 0 || new_stride_head < 0) return KVQ_EINVAL;
    if ((uintptr_t)new_tokens & (dtype == KVQ_F32 ? 3 : 1)) return KVQ_EINVAL;
    if (num_seqs == 0) return KVQ_OK;
    if (!seq_lens || !block_table || block_table_stride <= 0) return KVQ_EINVAL;
    if (!workspace || workspace_bytes < kv_append_workspace_bytes(num_seqs)) return KVQ_EWORKSPACE;
    if ((uintptr_t)workspace & 3) return KVQ_EINVAL;
    const kvq_format &f = dst->fmt;
    const int W = f.head_dim + f.rope_dim;
    const int64_t row = (int64_t)dst->num_heads * W;  // tail elements per token
    if ((int64_t)num_seqs * f.tile_tokens * row > (int64_t(1) << 40) || (int64_t)num_seqs * f.tile_tokens >= (1 << 30))
        return KVQ_EUNSUPPORTED;
    // the tail is the quantizer's source: same alignment rules as kv_quantize
    if ((st = check_quantize_source(dst, tail, dtype, row, W)) != KVQ_OK) return st;
    int32_t *ws = (int32_t *)workspace;
    kvq::AppendArgs ap{new_tokens, new_stride_seq, new_stride_head, tail, dtype == KVQ_F32 ? 4 : 2, num_seqs,
                       f.tile_tokens, dst->num_heads, W, seq_lens, block_table, block_table_stride, ws,
                       ws + num_seqs, ws + 2 * num_seqs};
    const kvq::QuantArgs q = quant_args(dst, tail, dtype, row, W, ap.tile_src_token, ap.tile_valid, ap.tile_dst_page,
                                        status_flags);
    if (!kvq::launch_append(ap, f.head_dim, f.tile_tokens, q, stream)) return KVQ_EUNSUPPORTED;
    return launched();
}

int32_t kv_decode_attn_default_splits(const kvq_cache *k, const kvq_cache *v, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t max_seq_len) {
    kvq::DecodeArgs a{};
    if (num_seqs <= 0 || max_seq_len <= 0 || check_cache(k) != KVQ_OK || (v && check_cache(v) != KVQ_OK) ||
        decode_layout(k, v, num_q_heads, a) != KVQ_OK)
        return 1;
    a.B = num_seqs;
    return kvq::decode_default_splits(a, max_seq_len);
}

const char *kv_decode_attn_kernel_name(const void *q, const kvq_cache *k, const kvq_cache *v, int32_t num_q_heads) {
    kvq::DecodeArgs a{};
    if (!q || check_cache(k) != KVQ_OK || (v && check_cache(v) != KVQ_OK) ||
        decode_layout(k, v, num_q_heads, a) != KVQ_OK)
        return nullptr;
    a.q = q;
    return kvq::decode_kernel_name(a);
}

const char *kv_decode_attn_merge_kernel_name(const void *q, const kvq_cache *k, const kvq_cache *v, int32_t num_seqs,
                                             int32_t num_q_heads, int32_t num_splits, int32_t max_seq_len) {
    kvq::DecodeArgs a{};
    if (!q || num_seqs <= 0 || num_splits < 0 || max_seq_len < 0 || check_cache(k) != KVQ_OK ||
        (v && check_cache(v) != KVQ_OK) || decode_layout(k, v, num_q_heads, a) != KVQ_OK)
        return nullptr;
    a.q = q;
    a.B = num_seqs;
    a.splits = num_splits > 0 ? num_splits : kvq::decode_default_splits(a, max_seq_len);
    return kvq::decode_merges_in_kernel(a) ? "" : "decode_reduce_kernel";
}

size_t kv_decode_attn_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim_v,
                                      int32_t num_splits) {
    if (num_seqs < 0 || num_q_heads <= 0 || head_dim_v <= 0 || num_splits <= 0) return 0;
    return KVQ_DECODE_COUNTER_BYTES + (size_t)num_seqs * num_q_heads * num_splits * (head_dim_v + 2) * sizeof(float);
}

kvq_status kv_decode_attn(const void *q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads, const kvq_cache *k,
                          const kvq_cache *v, const int32_t *block_table, int32_t block_table_stride,
                          const int32_t *seq_lens, int32_t max_seq_len, float sm_scale, int32_t num_splits,
                          void *workspace, size_t workspace_bytes, float *out, hipStream_t stream) {
    return decode_attn_impl(q, q_dtype, num_seqs, num_q_heads, k, v, block_table, block_table_stride, seq_lens,
                            max_seq_len, sm_scale, num_splits, workspace, workspace_bytes, true, out, stream);
}

kvq_status kv_decode_attn_noalloc(const void *q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                                  const kvq_cache *k, const kvq_cache *v, const int32_t *block_table,
                                  int32_t block_table_stride, const int32_t *seq_lens, int32_t max_seq_len,
                                  float sm_scale, int32_t num_splits, float *out, hipStream_t stream) {
    return decode_attn_impl(q, q_dtype, num_seqs, num_q_heads, k, v, block_table, block_table_stride, seq_lens,
                            max_seq_len, sm_scale, num_splits, nullptr, KVQ_NOALLOC_SCRATCH_BYTES, false, out, stream);
}

size_t kv_prefill_attn_workspace_bytes(int32_t num_seqs, int32_t chunk_len, int32_t num_q_heads, int32_t head_dim_v,
                                       int32_t num_splits, int32_t block_table_stride) {
    if (num_seqs < 0 || chunk_len <= 0 || num_q_heads <= 0 || head_dim_v <= 0 || num_splits <= 0 ||
        block_table_stride <= 0 || (int64_t)num_seqs * chunk_len > (1 << 24))
        return 0;
    const int32_t nv = num_seqs * chunk_len;
    const size_t dec = (kv_decode_attn_workspace_bytes(nv, num_q_heads, head_dim_v, num_splits) + 255) & ~(size_t)255;
    return dec + (size_t)nv * block_table_stride * sizeof(int32_t) + (size_t)nv * sizeof(int32_t);
}

int32_t kv_prefill_attn_default_splits(const kvq_cache *k, const kvq_cache *v, int32_t num_seqs, int32_t chunk_len,
                                       int32_t num_q_heads, int32_t max_seq_len) {
    if (chunk_len <= 0 || num_seqs < 0 || (int64_t)num_seqs * chunk_len > (1 << 24) || max_seq_len < 0) return 1;
    kvq::DecodeArgs a{};
    if (check_cache(k) != KVQ_OK || (v && check_cache(v) != KVQ_OK) || decode_layout(k, v, num_q_heads, a) != KVQ_OK)
        return 1;
    alignas(16) static const uint8_t aligned_probe[16] = {};
    a.q = aligned_probe;  // the split count assumes a 16-byte aligned query
    a.B = num_seqs;
    return kvq::prefill_default_splits(a, chunk_len, max_seq_len);
}

const char *kv_prefill_attn_kernel_name(const void *q, const kvq_cache *k, const kvq_cache *v, int32_t num_q_heads) {
    kvq::DecodeArgs a{};
    if (!q || check_cache(k) != KVQ_OK || (v && check_cache(v) != KVQ_OK) ||
        decode_layout(k, v, num_q_heads, a) != KVQ_OK)
        return nullptr;
    a.q = q;
    return kvq::prefill_kernel_name(a);
}

kvq_status kv_prefill_attn(const void *q, int32_t q_dtype, int32_t num_seqs, int32_t chunk_len, int32_t num_q_heads,
                           const kvq_cache *k, const kvq_cache *v, const int32_t *block_table,
                           int32_t block_table_stride, const int32_t *seq_lens, int32_t max_seq_len, float sm_scale,
                           int32_t num_splits, void *workspace, size_t workspace_bytes, float *out,
                           hipStream_t stream) {
    kvq_status st = check_cache(k);
    if (st != KVQ_OK) return st;
    if (v && (st = check_cache(v)) != KVQ_OK) return st;
    if (!q || !valid_dtype(q_dtype) || num_seqs < 0 || chunk_len <= 0 || num_q_heads <= 0 || !out || max_seq_len < 0)
        return KVQ_EINVAL;
    if ((int64_t)num_seqs * chunk_len > (1 << 24)) return KVQ_EUNSUPPORTED;
    if (num_seqs == 0) return KVQ_OK;
    if (!block_table || !seq_lens || block_table_stride <= 0 || num_splits < 0) return KVQ_EINVAL;
    kvq::DecodeArgs a{};
    if ((st = decode_layout(k, v, num_q_heads, a)) != KVQ_OK) return st;
    if ((int64_t)block_table_stride * a.T < max_seq_len) return KVQ_EINVAL;
    const int32_t nv = num_seqs * chunk_len;
    a.q = q;
    a.B = num_seqs;
    const int splits = num_splits > 0 ? num_splits : kvq::prefill_default_splits(a, chunk_len, max_seq_len);
    a.B = nv;
    if (!workspace || ((uintptr_t)workspace & 255) ||
        workspace_bytes < kv_prefill_attn_workspace_bytes(num_seqs, chunk_len, num_q_heads, a.Dv, splits,
                                                          block_table_stride))
        return KVQ_EWORKSPACE;
    const size_t dec = (kv_decode_attn_workspace_bytes(nv, num_q_heads, a.Dv, splits) + 255) & ~(size_t)255;
    int32_t *vbt = (int32_t *)((char *)workspace + dec);
    int32_t *vlens = vbt + (size_t)nv * block_table_stride;
    kvq::PrefillArgs p{num_seqs, chunk_len, seq_lens, block_table, block_table_stride, vbt, vlens};
    a.q = q;
    a.q_dtype = (int)q_dtype;
    a.bt = vbt;
    a.bt_stride = block_table_stride;
    a.seq_lens = vlens;
    a.sm = sm_scale;
    a.splits = splits;
    // the counter bytes at the head stay untouched (a workspace may also serve decode)
    a.ws = (float *)((char *)workspace + KVQ_DECODE_COUNTER_BYTES);
    a.cnt = nullptr;
    a.out = out;
    if (!kvq::launch_prefill(p, a, stream)) return KVQ_EUNSUPPORTED;
    return launched();
}

}  // extern "C"

namespace {

kvq_status decode_attn_impl(const void *q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                            const kvq_cache *k, const kvq_cache *v, const int32_t *block_table,
                            int32_t block_table_stride, const int32_t *seq_lens, int32_t max_seq_len, float sm_scale,
                            int32_t num_splits, void *workspace, size_t workspace_bytes, bool have_ws, float *out,
                            hipStream_t stream) {
    kvq_status st = check_cache(k);
    if (st != KVQ_OK) return st;
    if (v && (st = check_cache(v)) != KVQ_OK) return st;
    if (!q || !valid_dtype(q_dtype) || num_seqs < 0 || num_q_heads <= 0 || !out || max_seq_len < 0) return KVQ_EINVAL;
    if (num_seqs == 0) return KVQ_OK;
    if (!block_table || !seq_lens || block_table_stride <= 0 || num_splits < 0) return KVQ_EINVAL;
    kvq::DecodeArgs a{};
    if ((st = decode_layout(k, v, num_q_heads, a)) != KVQ_OK) return st;
    if ((int64_t)block_table_stride * a.T < max_seq_len) return KVQ_EINVAL;
    a.B = num_seqs;
    const int splits = num_splits > 0 ? num_splits : kvq::decode_default_splits(a, max_seq_len);
    if (workspace_bytes < kv_decode_attn_workspace_bytes(num_seqs, num_q_heads, a.Dv, splits)) return KVQ_EWORKSPACE;
    if (have_ws) {
        if (!workspace || ((uintptr_t)workspace & 3)) return KVQ_EWORKSPACE;
    } else if (!(workspace = scratch_for(stream))) {
        return KVQ_ELAUNCH;
    }
    a.q = q;
    a.q_dtype = (int)q_dtype;
    a.bt = block_table;
    a.bt_stride = block_table_stride;
    a.seq_lens = seq_lens;
    a.sm = sm_scale;
    a.splits = splits;
    a.cnt = (uint32_t *)workspace;
    a.ws = (float *)((char *)workspace + KVQ_DECODE_COUNTER_BYTES);
    a.out = out;
    a.max_len = max_seq_len;
    if (!kvq::launch_decode(a, stream)) return KVQ_EUNSUPPORTED;
    return launched();
}

}  // namespace
