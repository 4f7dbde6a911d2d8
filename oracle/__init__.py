"""ctypes binding of the CPU oracle (``oracle.cpp``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``; never by the GPU library or its
Python binding.  All arrays are host numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

TOKEN_MAJOR, CHANNEL_MAJOR = 0, 1
F32, F16, BF16 = 0, 1, 2
FLAG_NONFINITE, FLAG_SIDE_OVERFLOW = 1, 2


class OrcFormat(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("head_dim", "rope_dim", "tile_tokens", "hadamard_n", "group", "bits", "iters", "layout", "center")]


class OrcCache(ctypes.Structure):
    _fields_ = [("fmt", OrcFormat), ("num_pages", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("codes", ctypes.c_void_p), ("sz", ctypes.c_void_p), ("cnorm", ctypes.c_void_p),
                ("rope", ctypes.c_void_p), ("quot", ctypes.c_void_p)]


def lib():
    global _LIB
    if _LIB is None:
        # KVQ_ORACLE_LIB: another build of oracle.cpp (e.g. with sanitizers), same ABI
        path = os.environ.get("KVQ_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(path)
        vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        sig = {
            "orc_half_to_double": (f64, [ctypes.c_uint16]),
            "orc_double_to_half": (ctypes.c_uint16, [f64]),
            "orc_bf16_to_double": (f64, [ctypes.c_uint16]),
            "orc_double_to_bf16": (ctypes.c_uint16, [f64]),
            "orc_hadamard_matrix": (None, [i32, vp]),
            "orc_rotate": (None, [vp, i32, i32, i32, vp]),
            "orc_normalizers": (None, [vp, i32, i32, i32, i32, vp, vp]),
            "orc_quantize_tile": (ctypes.c_uint32, [vp, i32, vp, vp, vp, vp, vp, vp]),
            "orc_pack": (None, [vp, vp, vp]),
            "orc_unpack": (None, [vp, vp, vp]),
            "orc_dequant_tile": (None, [vp, vp, vp, vp, vp]),
            "orc_quantize_cache": (ctypes.c_uint32, [vp, vp, i32, i64, i64, i32, vp, vp, vp, i32]),
            "orc_dequantize_cache": (None, [vp, i32, vp, vp, vp, i32]),
            "orc_decode_attn": (None, [vp, i32, i32, i32, vp, vp, vp, i32, vp, f64, i32, vp, i32]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def fmt_struct(f) -> OrcFormat:
    return OrcFormat(f.head_dim, f.rope_dim, f.tile_tokens, f.hadamard_n, f.group, f.bits, f.iters, f.layout,
                     getattr(f, "center", 0))


def half_to_double(h: int) -> float:
    return lib().orc_half_to_double(h)


def double_to_half(x: float) -> int:
    return lib().orc_double_to_half(x)


def bf16_to_double(b: int) -> float:
    return lib().orc_bf16_to_double(b)


def double_to_bf16(x: float) -> int:
    return lib().orc_double_to_bf16(x)


def halves(a: np.ndarray) -> np.ndarray:
    """fp16 bit patterns -> float64 values (through the oracle's own decoder)."""
    flat = np.ascontiguousarray(a, dtype=np.uint16).reshape(-1)
    out = np.array([lib().orc_half_to_double(int(v)) for v in flat], dtype=np.float64)
    return out.reshape(np.shape(a))


def hadamard(h: int) -> np.ndarray:
    out = np.empty((h, h), np.float64)
    lib().orc_hadamard_matrix(h, out.ctypes.data)
    return out


def rotate(x: np.ndarray, h: int) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    n, D = x.shape
    out = np.empty_like(x)
    lib().orc_rotate(x.ctypes.data, n, D, h, out.ctypes.data)
    return out


def normalizers(xr: np.ndarray, iters: int, center: int = 0):
    xr = np.ascontiguousarray(xr, dtype=np.float64)
    n, D = xr.shape
    c = np.empty(D, np.float64)
    r = np.empty(max(n, 1), np.float64)
    lib().orc_normalizers(xr.ctypes.data, n, D, iters, center, c.ctypes.data, r.ctypes.data)
    return c, r[:n]


def quantize_tile(x: np.ndarray, f, with_quot: bool = False):
    """x: [n][D] float64 (n <= T). Returns codes [T][D], sz [T][D/G][2], c16 [D], c [D], flags,
    and with with_quot also quot [T][D]: the code quotient (y - Z) / S before rounding."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    n = x.shape[0]
    T, D, G = f.tile_tokens, f.head_dim, f.group
    codes = np.zeros((T, D), np.uint16)
    sz = np.zeros((T, D // G, 2), np.uint16)
    c16 = np.zeros(D, np.uint16)
    c = np.zeros(D, np.float64)
    quot = np.zeros((T, D), np.float64) if with_quot else None
    fs = fmt_struct(f)
    flags = lib().orc_quantize_tile(x.ctypes.data if n else None, n, ctypes.byref(fs), codes.ctypes.data,
                                    sz.ctypes.data, c16.ctypes.data, c.ctypes.data, _p(quot))
    if with_quot:
        return codes, sz, c16, c, int(flags), quot
    return codes, sz, c16, c, int(flags)


def pack(codes: np.ndarray, f) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint16)
    out = np.zeros(f.tile_tokens * f.head_dim * f.bits // 8, np.uint8)
    fs = fmt_struct(f)
    lib().orc_pack(codes.ctypes.data, ctypes.byref(fs), out.ctypes.data)
    return out


def unpack(buf: np.ndarray, f) -> np.ndarray:
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    out = np.zeros((f.tile_tokens, f.head_dim), np.uint16)
    fs = fmt_struct(f)
    lib().orc_unpack(buf.ctypes.data, ctypes.byref(fs), out.ctypes.data)
    return out


def dequant_tile(codes, sz, c16, f) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint16)
    sz = np.ascontiguousarray(sz, dtype=np.uint16)
    c16 = np.ascontiguousarray(c16, dtype=np.uint16)
    out = np.zeros((f.tile_tokens, f.head_dim), np.float64)
    fs = fmt_struct(f)
    lib().orc_dequant_tile(codes.ctypes.data, sz.ctypes.data, c16.ctypes.data, ctypes.byref(fs), out.ctypes.data)
    return out


class HostCache:
    """Host-memory paged quantized cache in the library's byte layout.  With
    with_quot, quantize_cache also records every code's quotient (y - Z) / S before
    rounding, [P][H][T][D] float64 (NaN where S == 0 or the row is not valid)."""

    def __init__(self, f, num_pages: int, num_heads: int, with_quot: bool = False):
        self.f = f
        self.num_pages, self.num_heads = num_pages, num_heads
        T, D, G, R = f.tile_tokens, f.head_dim, f.group, f.rope_dim
        self.codes = np.zeros((num_pages, num_heads, f.code_bytes()), np.uint8)
        self.sz = np.zeros((num_pages, num_heads, T, D // G, 2), np.uint16)
        self.cnorm = np.zeros((num_pages, num_heads, D), np.uint16)
        self.rope = np.zeros((num_pages, num_heads, T, R), np.uint16) if R else None
        self.quot = np.full((num_pages, num_heads, T, D), np.nan) if with_quot else None
        self.struct = OrcCache(fmt_struct(f), num_pages, num_heads, self.codes.ctypes.data, self.sz.ctypes.data,
                               self.cnorm.ctypes.data, _p(self.rope), _p(self.quot))


def quantize_cache(cache: HostCache, src: np.ndarray, src_dtype: int, tile_src_token, tile_valid, tile_page,
                   nthreads: int = 8) -> int:
    """src: [tokens][H][width] array; tile arrays int32."""
    src = np.ascontiguousarray(src)
    tst = np.ascontiguousarray(tile_src_token, np.int32)
    tv = np.ascontiguousarray(tile_valid, np.int32)
    tp = np.ascontiguousarray(tile_page, np.int32)
    stride_token = src.shape[1] * src.shape[2]
    stride_head = src.shape[2]
    return int(lib().orc_quantize_cache(ctypes.byref(cache.struct), src.ctypes.data, src_dtype, stride_token,
                                        stride_head, tst.size, tst.ctypes.data, tv.ctypes.data, tp.ctypes.data,
                                        nthreads))


def dequantize_cache(cache: HostCache, tile_page, tile_valid, nthreads: int = 8) -> np.ndarray:
    tp = np.ascontiguousarray(tile_page, np.int32)
    tv = np.ascontiguousarray(tile_valid, np.int32)
    f = cache.f
    out = np.zeros((tp.size, cache.num_heads, f.tile_tokens, f.head_dim + f.rope_dim), np.float64)
    lib().orc_dequantize_cache(ctypes.byref(cache.struct), tp.size, tp.ctypes.data, tv.ctypes.data,
                               out.ctypes.data, nthreads)
    return out


def decode_attn(q: np.ndarray, q_dtype: int, kc: HostCache, vc: Optional[HostCache], block_table, seq_lens,
                sm_scale: float, folded: bool = False, nthreads: int = 8) -> np.ndarray:
    q = np.ascontiguousarray(q)
    B, Hq = q.shape[0], q.shape[1]
    bt = np.ascontiguousarray(block_table, np.int32)
    sl = np.ascontiguousarray(seq_lens, np.int32)
    dv = (vc or kc).f.head_dim
    out = np.zeros((B, Hq, dv), np.float64)
    lib().orc_decode_attn(q.ctypes.data, q_dtype, B, Hq, ctypes.byref(kc.struct),
                          ctypes.byref(vc.struct) if vc is not None else None, bt.ctypes.data, bt.shape[1],
                          sl.ctypes.data, sm_scale, 1 if folded else 0, out.ctypes.data, nthreads)
    return out
