"""Seeded synthetic workloads for the KV-cache quantizer and quantized decode attention.

The generator (``synth.c``) is a counter-based splitmix64 stream with Box-Muller
normals, so every slice of a workload can be regenerated on its own.  This module
turns the five workload descriptions into shapes, formats and host arrays.  It
holds none of the quantization arithmetic and is used by both the GPU path and
the CPU oracle (and by nothing else of theirs).

Recipe (seed = 1000 + config index; stream numbers below):
  K   stream 1: N(0,1) * s[h, j]; s = exp(N(0,1)) (stream 4, index h*D + j) times
      20 on 3 channels per kv head (configs 1-3), or s = 15 on 3 channels per
      head and 1 elsewhere (config 0); outlier channels are the first 3 entries of
      a seeded Fisher-Yates shuffle (stream 100 + h).
  V   stream 2: N(0,1).
  MLA latent+rope row (576 values) stream 1: N(0,1), 5 latent dims (1% of 512)
      times 10, chosen by a Fisher-Yates shuffle (stream 100).
  q   stream 3: N(0,1).
  seq lens (config 3) stream 5: uniform integers in [512, 16384] by rejection.
  page permutation (config 3) stream 6: Fisher-Yates over all physical pages.
Values are drawn in double, rounded to fp32, then to bf16 (nearest, ties even)
where the workload is bf16.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

TOKEN_MAJOR = 0
CHANNEL_MAJOR = 1
F32, F16, BF16 = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def lib():
    global _LIB
    if _LIB is None:
        # KVQ_SYNTH_LIB: another build of synth.c (e.g. with sanitizers), same ABI
        path = os.environ.get("KVQ_SYNTH_LIB") or os.path.join(_HERE, "libsynth.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(path)
        L.synth_u64.restype = ctypes.c_uint64
        L.synth_u64.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64]
        L.synth_normal.restype = None
        L.synth_normal.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64,
                                   ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64]
        _LIB = L
    return _LIB


def u64(seed: int, stream: int, index: int) -> int:
    return int(lib().synth_u64(seed, stream, index))


class _Draws:
    """Sequential bounded integers from one (seed, stream), by rejection sampling."""

    def __init__(self, seed: int, stream: int):
        self.seed, self.stream, self.i = seed, stream, 0

    def below(self, m: int) -> int:
        limit = (1 << 64) - ((1 << 64) % m)
        while True:
            x = u64(self.seed, self.stream, self.i)
            self.i += 1
            if x < limit:
                return x % m


def permutation(n: int, seed: int, stream: int) -> np.ndarray:
    """Fisher-Yates shuffle of range(n) (Durstenfeld's in-place form)."""
    d = _Draws(seed, stream)
    p = np.arange(n, dtype=np.int64)
    for i in range(n - 1, 0, -1):
        j = d.below(i + 1)
        p[i], p[j] = p[j], p[i]
    return p


def normal(n: int, seed: int, stream: int, offset: int = 0, col_scale: Optional[np.ndarray] = None,
           dtype: str = "bf16") -> np.ndarray:
    """n standard normals at counters offset..offset+n-1, times col_scale[k % len]."""
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)
    cs = None
    ncols = 1
    if col_scale is not None:
        cs = np.ascontiguousarray(col_scale, dtype=np.float32)
        ncols = cs.size
    lib().synth_normal(out.ctypes.data, 0 if dtype == "f32" else 2, n, seed, stream, offset,
                       cs.ctypes.data if cs is not None else None, ncols)
    return out


@dataclass
class Fmt:
    head_dim: int
    rope_dim: int
    tile_tokens: int
    hadamard_n: int
    group: int
    bits: int
    iters: int
    layout: int
    center: int = 0   # 1: rounds normalize to unit std about the mean (else RMS about zero)

    def code_bytes(self) -> int:          # per (page, head)
        return self.tile_tokens * self.head_dim * self.bits // 8

    def token_bytes(self) -> float:       # stored bytes per (token, head), side data included
        T, D = self.tile_tokens, self.head_dim
        return D * self.bits / 8 + 4 * (D // self.group) + 2 * D / T + 2 * self.rope_dim


@dataclass
class Config:
    index: int
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    seq_lens: np.ndarray
    fk: Fmt
    fv: Optional[Fmt]          # None: the K cache (MLA latent) is also the value
    src_dtype: str             # "f32" or "bf16"
    sm_scale: float
    min_splits: int
    seed: int
    k_outliers: int = 3
    k_outlier_mult: float = 20.0
    k_lognormal: bool = True
    mla_outliers: int = 0
    page_perm: bool = False
    # derived
    tile_src_token: np.ndarray = field(default=None)
    tile_valid: np.ndarray = field(default=None)
    tile_page: np.ndarray = field(default=None)
    block_table: np.ndarray = field(default=None)
    seq_start: np.ndarray = field(default=None)
    tile_seq: np.ndarray = field(default=None)

    @property
    def width(self) -> int:
        return self.fk.head_dim + self.fk.rope_dim

    @property
    def total_tokens(self) -> int:
        return int(self.seq_lens.sum())

    @property
    def num_pages(self) -> int:
        return int(self.tile_page.size)

    @property
    def dv(self) -> int:
        return (self.fv or self.fk).head_dim


NAMES = ["tiny", "gqa", "long", "paged", "mla"]


def _finish(cfg: Config) -> Config:
    T = cfg.fk.tile_tokens
    lens = cfg.seq_lens
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    npages = (lens + T - 1) // T
    src, valid, seq = [], [], []
    for s in range(cfg.num_seqs):
        for p in range(int(npages[s])):
            src.append(starts[s] + p * T)
            valid.append(min(T, int(lens[s]) - p * T))
            seq.append(s)
    P = len(src)
    page = permutation(P, cfg.seed, 6) if cfg.page_perm else np.arange(P, dtype=np.int64)
    bt = np.zeros((cfg.num_seqs, int(npages.max())), dtype=np.int32)
    k = 0
    for s in range(cfg.num_seqs):
        for p in range(int(npages[s])):
            bt[s, p] = page[k]
            k += 1
    cfg.tile_src_token = np.asarray(src, dtype=np.int32)
    cfg.tile_valid = np.asarray(valid, dtype=np.int32)
    cfg.tile_page = np.asarray(page, dtype=np.int32)
    cfg.tile_seq = np.asarray(seq, dtype=np.int32)
    cfg.block_table = bt
    cfg.seq_start = starts
    return cfg


def config(i: int, **overrides) -> Config:
    seed = 1000 + i
    if i == 0:
        f = Fmt(64, 0, 64, 64, 64, 4, 4, TOKEN_MAJOR)
        cfg = Config(0, "tiny: 1 seq, 2 kv heads, head_dim 64, 256 tokens, fp32, K4/V4", 1, 2, 2,
                     np.array([256], np.int64), f, Fmt(64, 0, 64, 64, 64, 4, 4, CHANNEL_MAJOR), "f32",
                     1.0 / 8.0, 1, seed, k_outliers=3, k_outlier_mult=15.0, k_lognormal=False)
    elif i == 1:
        cfg = Config(1, "gqa decode: batch 8, 32 q / 8 kv heads, head_dim 128, context 4096, bf16, K4/V4", 8,
                     32, 8, np.full(8, 4096, np.int64), Fmt(128, 0, 128, 128, 128, 4, 4, TOKEN_MAJOR),
                     Fmt(128, 0, 128, 128, 128, 4, 4, CHANNEL_MAJOR), "bf16", 1.0 / math.sqrt(128), 1, seed)
    elif i == 2:
        cfg = Config(2, "long context: batch 1, 32 q / 8 kv heads, head_dim 128, context 131072, bf16, K4/V2",
                     1, 32, 8, np.array([131072], np.int64), Fmt(128, 0, 128, 128, 128, 4, 4, TOKEN_MAJOR),
                     Fmt(128, 0, 128, 128, 128, 2, 4, CHANNEL_MAJOR), "bf16", 1.0 / math.sqrt(128), 256, seed)
    elif i == 3:
        d = _Draws(seed, 5)
        lens = np.array([512 + d.below(16384 - 512 + 1) for _ in range(64)], np.int64)
        cfg = Config(3, "paged serving: 64 seqs, lengths U[512,16384], 16-token pages, 64 q / 8 kv heads, "
                     "head_dim 128, bf16, K3/V3, 2 iters", 64, 64, 8, lens,
                     Fmt(128, 0, 16, 128, 128, 3, 2, TOKEN_MAJOR), Fmt(128, 0, 16, 128, 128, 3, 2, CHANNEL_MAJOR),
                     "bf16", 1.0 / math.sqrt(128), 1, seed, page_perm=True)
    elif i == 4:
        cfg = Config(4, "mla latent: batch 32, context 32768, 512 latent + 64 rope bf16, 128 q heads, 4-bit latent",
                     32, 128, 1, np.full(32, 32768, np.int64), Fmt(512, 64, 128, 512, 512, 4, 4, TOKEN_MAJOR),
                     None, "bf16", 1.0 / 24.0, 1, seed, k_outliers=0, k_lognormal=False, mla_outliers=5)
    else:
        raise ValueError(i)
    for k, v in overrides.items():
        setattr(cfg, k, v)
    return _finish(cfg)


def k_col_scale(cfg: Config) -> np.ndarray:
    """Per (kv head, channel) multiplier of the K stream, length H * width."""
    H, D, W = cfg.num_kv_heads, cfg.fk.head_dim, cfg.width
    s = np.ones((H, W), np.float64)
    if cfg.k_lognormal:
        z = normal(H * D, cfg.seed, 4, dtype="f32").astype(np.float64).reshape(H, D)
        s[:, :D] = np.exp(z)
    for h in range(H):
        if cfg.k_outliers:
            for j in permutation(D, cfg.seed, 100 + h)[: cfg.k_outliers]:
                s[h, j] *= cfg.k_outlier_mult
        if cfg.mla_outliers:
            for j in permutation(D, cfg.seed, 100 + h)[: cfg.mla_outliers]:
                s[h, j] *= 10.0
    return s.reshape(-1).astype(np.float32)


def gen_k(cfg: Config, t0: int = 0, t1: Optional[int] = None, col_scale=None) -> np.ndarray:
    """K source rows [t1 - t0][H][width] for global tokens t0..t1-1."""
    t1 = cfg.total_tokens if t1 is None else t1
    H, W = cfg.num_kv_heads, cfg.width
    cs = k_col_scale(cfg) if col_scale is None else col_scale
    a = normal((t1 - t0) * H * W, cfg.seed, 1, t0 * H * W, cs, cfg.src_dtype)
    return a.reshape(t1 - t0, H, W)


def gen_v(cfg: Config, t0: int = 0, t1: Optional[int] = None) -> np.ndarray:
    t1 = cfg.total_tokens if t1 is None else t1
    H, D = cfg.num_kv_heads, cfg.dv
    a = normal((t1 - t0) * H * D, cfg.seed, 2, t0 * H * D, None, cfg.src_dtype)
    return a.reshape(t1 - t0, H, D)


def gen_q(cfg: Config) -> np.ndarray:
    n = cfg.num_seqs * cfg.num_q_heads * cfg.width
    return normal(n, cfg.seed, 3, 0, None, cfg.src_dtype).reshape(cfg.num_seqs, cfg.num_q_heads, cfg.width)


def np_dtype_code(a: np.ndarray, declared: str) -> int:
    return F32 if declared == "f32" else BF16
