"""Python binding of libkvq.so (KVarN-style KV-cache quantization for MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels of
libkvq.so. PyTorch supplies device memory (tensor.data_ptr()) and the stream
(torch.cuda.current_stream()). The functions keep the C names:

    kvq_format_from_preset, kvq_cache_bytes, kv_quantize, kv_dequantize,
    kv_decode_attn_default_splits, kv_decode_attn_workspace_bytes,
    kv_decode_attn, kv_append, kv_append_workspace_bytes, kv_prefill_attn,
    kv_prefill_attn_workspace_bytes, kv_prefill_attn_default_splits,
    kv_quantize_kernel_name, kv_decode_attn_kernel_name,
    kv_decode_attn_merge_kernel_name, kv_prefill_attn_kernel_name, kvq_status_str

plus ``DeviceCache``, a holder of the four device arrays of one cache, and
``decode_workspace``, a workspace for kv_decode_attn with its counters cleared.
Importing this module fails if libkvq.so has not been built: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVQ_LIB: another build of the same sources (e.g. host code with sanitizers)
LIB_PATH = os.environ.get("KVQ_LIB") or os.path.join(_HERE, "libkvq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python __graft_entry__.py` (hipcc, gfx950)")

# PyTorch ships its own HIP runtime under the same soname; loading torch first
# makes libkvq.so bind to that one instance, so torch's streams and device
# memory are valid handles inside the library.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

KVQ_F32, KVQ_F16, KVQ_BF16 = 0, 1, 2
KVQ_OK, KVQ_EINVAL, KVQ_EUNSUPPORTED, KVQ_EWORKSPACE, KVQ_ELAUNCH = 0, -1, -2, -3, -4
KVQ_TOKEN_MAJOR, KVQ_CHANNEL_MAJOR = 0, 1
KVQ_FLAG_NONFINITE, KVQ_FLAG_SIDE_OVERFLOW = 1, 2

EXPORTS = ("kvq_format_from_preset", "kvq_cache_bytes", "kv_quantize", "kv_quantize_kv", "kv_dequantize",
           "kv_decode_attn_default_splits", "kv_decode_attn_workspace_bytes", "kv_decode_attn", "kv_decode_attn_noalloc", "kv_append", "kv_append_workspace_bytes", "kv_prefill_attn",
           "kv_prefill_attn_workspace_bytes", "kv_prefill_attn_default_splits",
           "kv_quantize_kernel_name", "kv_decode_attn_kernel_name", "kv_decode_attn_merge_kernel_name",
           "kv_prefill_attn_kernel_name", "kvq_status_str")


class kvq_format(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("head_dim", "rope_dim", "tile_tokens", "hadamard_n", "group", "bits", "iters", "layout", "center")]

    def __repr__(self):
        return "kvq_format(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class kvq_cache(ctypes.Structure):
    _fields_ = [("fmt", kvq_format), ("num_pages", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("codes", ctypes.c_void_p), ("sz", ctypes.c_void_p), ("cnorm", ctypes.c_void_p),
                ("rope", ctypes.c_void_p)]


_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_sig = {
    "kvq_format_from_preset": (_i32, [ctypes.c_char_p, _i32, ctypes.POINTER(kvq_format), ctypes.POINTER(kvq_format)]),
    "kvq_cache_bytes": (_sz, [ctypes.POINTER(kvq_format), _i32, _i32]),
    "kv_quantize": (_i32, [ctypes.POINTER(kvq_cache), _vp, _i32, _i64, _i64, _i32, _vp, _vp, _vp, _vp, _vp]),
    "kv_quantize_kv": (_i32, [ctypes.POINTER(kvq_cache), ctypes.POINTER(kvq_cache), _vp, _vp, _i32, _i64, _i64, _i64,
                              _i64, _i32, _vp, _vp, _vp, _vp, _vp]),
    "kv_dequantize": (_i32, [ctypes.POINTER(kvq_cache), _i32, _vp, _vp, _vp, _i32, _vp]),
    "kv_decode_attn_default_splits": (_i32, [ctypes.c_void_p, ctypes.c_void_p, _i32, _i32, _i32]),
    "kv_decode_attn_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "kv_decode_attn": (_i32, [_vp, _i32, _i32, _i32, ctypes.POINTER(kvq_cache), ctypes.POINTER(kvq_cache), _vp, _i32,
                              _vp, _i32, ctypes.c_float, _i32, _vp, _sz, _vp, _vp]),
    "kv_decode_attn_noalloc": (_i32, [_vp, _i32, _i32, _i32, ctypes.POINTER(kvq_cache), ctypes.POINTER(kvq_cache),
                                      _vp, _i32, _vp, _i32, ctypes.c_float, _i32, _vp, _vp]),
    "kv_append": (_i32, [ctypes.POINTER(kvq_cache), _vp, _i32, _vp, _i64, _i64, _i32, _vp, _vp, _i32, _vp, _sz, _vp,
                         _vp]),
    "kv_append_workspace_bytes": (_sz, [_i32]),
    "kv_prefill_attn": (_i32, [_vp, _i32, _i32, _i32, _i32, ctypes.POINTER(kvq_cache), ctypes.POINTER(kvq_cache), _vp,
                               _i32, _vp, _i32, ctypes.c_float, _i32, _vp, _sz, _vp, _vp]),
    "kv_prefill_attn_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "kv_prefill_attn_default_splits": (_i32, [ctypes.c_void_p, ctypes.c_void_p, _i32, _i32, _i32, _i32]),
    "kv_quantize_kernel_name": (ctypes.c_char_p, [ctypes.POINTER(kvq_cache), _vp, _i32, _i64, _i64]),
    "kv_decode_attn_kernel_name": (ctypes.c_char_p, [_vp, ctypes.POINTER(kvq_cache), ctypes.POINTER(kvq_cache), _i32]),
    "kv_decode_attn_merge_kernel_name": (ctypes.c_char_p, [_vp, ctypes.POINTER(kvq_cache), ctypes.POINTER(kvq_cache), _i32,
                                                           _i32, _i32, _i32]),
    "kv_prefill_attn_kernel_name": (ctypes.c_char_p, [_vp, ctypes.POINTER(kvq_cache), ctypes.POINTER(kvq_cache), _i32]),
    "kvq_status_str": (ctypes.c_char_p, [_i32]),
}
for _name, (_res, _args) in _sig.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class KvqError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {kvq_status_str(status)} ({status})")
        self.status = status


def kvq_status_str(status: int) -> str:
    return _lib.kvq_status_str(status).decode()


def _check(status: int, where: str):
    if status != KVQ_OK:
        raise KvqError(status, where)


def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    return {torch.float32: KVQ_F32, torch.float16: KVQ_F16, torch.bfloat16: KVQ_BF16}[t.dtype]


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def make_format(head_dim, rope_dim, tile_tokens, hadamard_n, group, bits, iters, layout, center=0) -> kvq_format:
    return kvq_format(head_dim, rope_dim, tile_tokens, hadamard_n, group, bits, iters, layout, center)


def kvq_format_from_preset(preset: str, head_dim: int):
    k, v = kvq_format(), kvq_format()
    _check(_lib.kvq_format_from_preset(preset.encode(), head_dim, ctypes.byref(k), ctypes.byref(v)),
           "kvq_format_from_preset")
    return k, v


def kvq_cache_bytes(fmt: kvq_format, num_pages: int, num_heads: int) -> int:
    return int(_lib.kvq_cache_bytes(ctypes.byref(fmt), num_pages, num_heads))


class DeviceCache:
    """The four device arrays of one paged quantized cache (layout in kvq.h)."""

    def __init__(self, fmt: kvq_format, num_pages: int, num_heads: int, device="cuda"):
        torch = _torch()
        self.fmt = fmt
        T, D, G, R = fmt.tile_tokens, fmt.head_dim, fmt.group, fmt.rope_dim
        self.num_pages, self.num_heads = num_pages, num_heads
        self.codes = torch.zeros((num_pages, num_heads, T * D * fmt.bits // 8), dtype=torch.uint8, device=device)
        self.sz = torch.zeros((num_pages, num_heads, T, D // G, 2), dtype=torch.int16, device=device)
        self.cnorm = torch.zeros((num_pages, num_heads, D), dtype=torch.int16, device=device)
        self.rope = (torch.zeros((num_pages, num_heads, T, R), dtype=torch.int16, device=device) if R else None)
        self.struct = kvq_cache(fmt, num_pages, num_heads, self.codes.data_ptr(), self.sz.data_ptr(),
                                self.cnorm.data_ptr(), self.rope.data_ptr() if self.rope is not None else None)

    def nbytes(self) -> int:
        n = self.codes.numel() + 2 * (self.sz.numel() + self.cnorm.numel())
        return n + (2 * self.rope.numel() if self.rope is not None else 0)


def kv_quantize(dst: DeviceCache, src, tile_src_token, tile_valid, tile_dst_page, status_flags=None, stream=None):
    """src: device tensor [tokens][H][D + R] (or any view with unit channel stride)."""
    assert src.dim() == 3 and src.stride(2) == 1
    _check(_lib.kv_quantize(ctypes.byref(dst.struct), _ptr(src), _dtype_code(src), src.stride(0), src.stride(1),
                            tile_src_token.numel(), _ptr(tile_src_token), _ptr(tile_valid), _ptr(tile_dst_page),
                            _ptr(status_flags), _stream(stream)), "kv_quantize")


def kv_quantize_kv(k_dst: DeviceCache, v_dst: DeviceCache, k_src, v_src, tile_src_token, tile_valid, tile_dst_page,
                   status_flags=None, stream=None):
    """K and V caches of one batch in one launch (same result as kv_quantize on each).
    Raises KvqError (KVQ_EUNSUPPORTED) for formats the one-launch kernel does not take."""
    assert k_src.dim() == 3 and k_src.stride(2) == 1 and v_src.dim() == 3 and v_src.stride(2) == 1
    assert k_src.dtype == v_src.dtype
    _check(_lib.kv_quantize_kv(ctypes.byref(k_dst.struct), ctypes.byref(v_dst.struct), _ptr(k_src), _ptr(v_src),
                               _dtype_code(k_src), k_src.stride(0), k_src.stride(1), v_src.stride(0), v_src.stride(1),
                               tile_src_token.numel(), _ptr(tile_src_token), _ptr(tile_valid), _ptr(tile_dst_page),
                               _ptr(status_flags), _stream(stream)), "kv_quantize_kv")


def kv_dequantize(src: DeviceCache, tile_page, tile_valid, out=None, dtype=None, stream=None):
    torch = _torch()
    f = src.fmt
    if out is None:
        out = torch.empty((tile_page.numel(), src.num_heads, f.tile_tokens, f.head_dim + f.rope_dim),
                          dtype=dtype or torch.float32, device=src.codes.device)
    _check(_lib.kv_dequantize(ctypes.byref(src.struct), tile_page.numel(), _ptr(tile_page), _ptr(tile_valid),
                              _ptr(out), _dtype_code(out), _stream(stream)), "kv_dequantize")
    return out


def kv_decode_attn_default_splits(k: DeviceCache, v: Optional[DeviceCache], num_seqs: int, num_q_heads: int,
                                  max_seq_len: int) -> int:
    return int(_lib.kv_decode_attn_default_splits(ctypes.byref(k.struct), ctypes.byref(v.struct) if v is not None else None,
                                                  num_seqs, num_q_heads, max_seq_len))


def kv_append_workspace_bytes(num_seqs: int) -> int:
    return int(_lib.kv_append_workspace_bytes(num_seqs))


def kv_append(dst: DeviceCache, tail, new_tokens, seq_lens, block_table, workspace=None, status_flags=None,
              stream=None):
    """Append new_tokens[s] ([num_seqs][H][D + R], same dtype as tail) to each sequence:
    row seq_lens[s] % T of tail[s] ([num_seqs][T][H][D + R]) and a re-quantization of
    that partial tile into page block_table[s][seq_lens[s] // T]. seq_lens are the
    lengths before the append and are not modified."""
    torch = _torch()
    B = new_tokens.shape[0]
    if tail.dtype != new_tokens.dtype:
        raise ValueError("tail and new_tokens must have the same dtype")
    if new_tokens.dim() != 3 or new_tokens.stride(2) != 1 or not tail.is_contiguous():
        raise ValueError("new_tokens must be [num_seqs][H][D + R] with unit stride in the last dimension; tail contiguous")
    if workspace is None:
        workspace = torch.empty(max(kv_append_workspace_bytes(B), 4), dtype=torch.uint8, device=new_tokens.device)
    _check(_lib.kv_append(ctypes.byref(dst.struct), _ptr(tail), _dtype_code(tail), _ptr(new_tokens),
                          new_tokens.stride(0), new_tokens.stride(1), B, _ptr(seq_lens), _ptr(block_table),
                          block_table.shape[1], _ptr(workspace), workspace.numel() * workspace.element_size(),
                          _ptr(status_flags), _stream(stream)), "kv_append")


def kv_prefill_attn_workspace_bytes(num_seqs: int, chunk_len: int, num_q_heads: int, head_dim_v: int,
                                    num_splits: int, block_table_stride: int) -> int:
    return int(_lib.kv_prefill_attn_workspace_bytes(num_seqs, chunk_len, num_q_heads, head_dim_v, num_splits,
                                                    block_table_stride))


def kv_prefill_attn_default_splits(k: DeviceCache, v: Optional[DeviceCache], num_seqs: int, chunk_len: int,
                                   num_q_heads: int, max_seq_len: int) -> int:
    return int(_lib.kv_prefill_attn_default_splits(ctypes.byref(k.struct),
                                                   ctypes.byref(v.struct) if v is not None else None,
                                                   num_seqs, chunk_len, num_q_heads, max_seq_len))


def kv_prefill_attn(q, k: DeviceCache, v: Optional[DeviceCache], block_table, seq_lens, max_seq_len: int,
                    sm_scale: float, num_splits: int = 0, workspace=None, out=None, stream=None):
    """q: [num_seqs][chunk_len][num_q_heads][D + R]; seq_lens include the chunk.
    Returns out [num_seqs][chunk_len][num_q_heads][Dv] (fp32)."""
    torch = _torch()
    if q.dim() != 4 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [num_seqs][chunk_len][num_q_heads][D + R] tensor")
    B, Lq, Hq = q.shape[0], q.shape[1], q.shape[2]
    dv = (v or k).fmt.head_dim
    if num_splits <= 0:
        num_splits = kv_prefill_attn_default_splits(k, v, B, Lq, Hq, max_seq_len)
    need = kv_prefill_attn_workspace_bytes(B, Lq, Hq, dv, num_splits, block_table.shape[1])
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Lq, Hq, dv), dtype=torch.float32, device=q.device)
    _check(_lib.kv_prefill_attn(_ptr(q), _dtype_code(q), B, Lq, Hq, ctypes.byref(k.struct),
                                ctypes.byref(v.struct) if v is not None else None, _ptr(block_table),
                                block_table.shape[1], _ptr(seq_lens), max_seq_len, sm_scale, num_splits,
                                _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out),
                                _stream(stream)), "kv_prefill_attn")
    return out


def kv_quantize_kernel_name(dst: DeviceCache, src) -> Optional[str]:
    """Kernel kv_quantize(dst, src, ...) runs, or None where it would reject the arguments."""
    r = _lib.kv_quantize_kernel_name(ctypes.byref(dst.struct), _ptr(src), _dtype_code(src), src.stride(0), src.stride(1))
    return r.decode() if r is not None else None


def kv_decode_attn_kernel_name(q, k: DeviceCache, v: Optional[DeviceCache]) -> Optional[str]:
    """Main kernel kv_decode_attn(q, k, v, ...) runs, or None for invalid arguments."""
    r = _lib.kv_decode_attn_kernel_name(_ptr(q), ctypes.byref(k.struct), ctypes.byref(v.struct) if v is not None else None,
                                        q.shape[1])
    return r.decode() if r is not None else None


def kv_decode_attn_merge_kernel_name(q, k: DeviceCache, v: Optional[DeviceCache], num_splits: int,
                                     max_seq_len: int) -> Optional[str]:
    """Split-merge kernel that follows the main kernel of kv_decode_attn(q, k, v, ...),
    "" when the main kernel merges the splits itself, None for invalid arguments."""
    r = _lib.kv_decode_attn_merge_kernel_name(_ptr(q), ctypes.byref(k.struct),
                                              ctypes.byref(v.struct) if v is not None else None, q.shape[0], q.shape[1],
                                              num_splits, max_seq_len)
    return r.decode() if r is not None else None


def kv_prefill_attn_kernel_name(q, k: DeviceCache, v: Optional[DeviceCache]) -> Optional[str]:
    """Main kernel kv_prefill_attn(q, k, v, ...) runs for q [B, Lq, Hq, D + R], or None for invalid arguments."""
    r = _lib.kv_prefill_attn_kernel_name(_ptr(q), ctypes.byref(k.struct), ctypes.byref(v.struct) if v is not None else None,
                                         q.shape[2])
    return r.decode() if r is not None else None


# bytes at the head of a decode workspace holding the split-merge arrival counters:
# zero when the workspace is first used, left zero by every call
KVQ_DECODE_COUNTER_BYTES = 64 << 10


def kv_decode_attn_workspace_bytes(num_seqs: int, num_q_heads: int, head_dim_v: int, num_splits: int) -> int:
    return int(_lib.kv_decode_attn_workspace_bytes(num_seqs, num_q_heads, head_dim_v, num_splits))


def decode_workspace(num_bytes: int, device):
    """A decode workspace of `num_bytes` bytes, ready for kv_decode_attn (its counter
    bytes cleared) and for kv_prefill_attn."""
    torch = _torch()
    ws = torch.empty(max(int(num_bytes), KVQ_DECODE_COUNTER_BYTES), dtype=torch.uint8, device=device)
    ws[:KVQ_DECODE_COUNTER_BYTES].zero_()
    return ws


def kv_decode_attn(q, k: DeviceCache, v: Optional[DeviceCache], block_table, seq_lens, max_seq_len: int,
                   sm_scale: float, num_splits: int = 0, workspace=None, out=None, stream=None):
    torch = _torch()
    B, Hq = q.shape[0], q.shape[1]
    dv = (v or k).fmt.head_dim
    if num_splits <= 0:
        num_splits = kv_decode_attn_default_splits(k, v, B, Hq, max_seq_len)
    need = kv_decode_attn_workspace_bytes(B, Hq, dv, num_splits)
    if workspace is None:
        workspace = decode_workspace(need, q.device)
    if out is None:
        out = torch.empty((B, Hq, dv), dtype=torch.float32, device=q.device)
    _check(_lib.kv_decode_attn(_ptr(q), _dtype_code(q), B, Hq, ctypes.byref(k.struct),
                               ctypes.byref(v.struct) if v is not None else None, _ptr(block_table),
                               block_table.shape[1], _ptr(seq_lens), max_seq_len, sm_scale, num_splits,
                               _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out),
                               _stream(stream)), "kv_decode_attn")
    return out


KVQ_NOALLOC_SCRATCH_BYTES = 64 << 20


def kv_decode_attn_noalloc(q, k: DeviceCache, v: Optional[DeviceCache], block_table, seq_lens, max_seq_len: int,
                           sm_scale: float, num_splits: int = 0, out=None, stream=None):
    """kv_decode_attn with the split partials in the library's per-GPU scratch array
    (the C call allocates nothing; `out` is allocated here when not given)."""
    torch = _torch()
    B, Hq = q.shape[0], q.shape[1]
    dv = (v or k).fmt.head_dim
    if out is None:
        out = torch.empty((B, Hq, dv), dtype=torch.float32, device=q.device)
    _check(_lib.kv_decode_attn_noalloc(_ptr(q), _dtype_code(q), B, Hq, ctypes.byref(k.struct),
                                       ctypes.byref(v.struct) if v is not None else None, _ptr(block_table),
                                       block_table.shape[1], _ptr(seq_lens), max_seq_len, sm_scale, num_splits,
                                       _ptr(out), _stream(stream)), "kv_decode_attn_noalloc")
    return out
