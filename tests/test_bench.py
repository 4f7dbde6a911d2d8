"""The benchmark's accounting, checked on the CPU: algorithmic bytes and operation
counts of the four workloads recomputed here from the formats' definitions (codes,
per-token fp16 scale and zero, per-channel fp16 normalizer, bf16 rope), and the
single-GPU guard of the command line."""
import math
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_cache_block_bytes_by_hand():
    # 128 tokens x 128 channels at 4 bits, one (S, Z) pair of fp16 per token, one fp16
    # normalizer per channel
    f = W.config(1).fk
    assert bench.block_bytes(f) == 128 * 128 // 2 + 128 * 4 + 128 * 2 == 8960
    # 16-token pages at 3 bits
    f3 = W.config(3).fk
    assert bench.block_bytes(f3) == 16 * 128 * 3 // 8 + 16 * 4 + 128 * 2 == 1088
    # MLA latent: 512 channels at 4 bits plus 64 bf16 rope channels per token
    fm = W.config(4).fk
    assert bench.block_bytes(fm) == 128 * 512 // 2 + 128 * 4 + 512 * 2 + 128 * 64 * 2 == 50688
    assert bench.block_bytes(fm, with_rope=False) == 50688 - 128 * 64 * 2


@pytest.mark.parametrize("ci", [1, 2, 3, 4])
def test_quantize_bytes_match_the_workload(ci):
    cfg = W.config(ci)
    r, w = bench.quantize_bytes(cfg, cfg.fk, cfg.width)
    tokens = int(np.sum(cfg.seq_lens))
    assert r == tokens * cfg.num_kv_heads * cfg.width * 2  # bf16 source
    # every page of every kv head is written once
    T = cfg.fk.tile_tokens
    pages = sum(-(-int(L) // T) for L in cfg.seq_lens)
    assert cfg.num_pages == pages
    assert w == pages * cfg.num_kv_heads * bench.block_bytes(cfg.fk)


def test_quantize_bytes_gqa_total():
    cfg = W.config(1)
    rk, wk = bench.quantize_bytes(cfg, cfg.fk, cfg.width)
    rv, wv = bench.quantize_bytes(cfg, cfg.fv, cfg.dv)
    # 4096 (tile, head) items per cache of 32768 + 8192 + 512 + 256 bytes
    assert rk + wk + rv + wv == 2 * 2048 * (32768 + 8192 + 512 + 256) == 170917888


@pytest.mark.parametrize("ci", [1, 2, 3, 4])
def test_decode_bytes_match_the_workload(ci):
    cfg = W.config(ci)
    T = cfg.fk.tile_tokens
    page_heads = sum(-(-int(L) // T) for L in cfg.seq_lens) * cfg.num_kv_heads
    per = bench.block_bytes(cfg.fk) + (bench.block_bytes(cfg.fv) if cfg.fv is not None else 0)
    q = cfg.num_seqs * cfg.num_q_heads * cfg.width * 2
    out = cfg.num_seqs * cfg.num_q_heads * cfg.dv * 4
    assert bench.decode_bytes(cfg) == page_heads * per + q + out


def test_decode_bytes_gqa_total():
    # 8 sequences x 32 pages x 8 kv heads of K and V blocks, plus q (bf16) and out (fp32)
    assert bench.decode_bytes(W.config(1)) == 2048 * 17920 + 8 * 32 * 128 * 2 + 8 * 32 * 128 * 4 == 36896768


def test_valu_operation_count():
    cfg = W.config(3)
    elems = int(np.sum(cfg.seq_lens)) * cfg.num_kv_heads * 128
    # log2(128) butterfly stages + 2 N row/column FMAs + 7 per element, N = 2
    assert bench.quantize_valu_ops(cfg, cfg.fk, cfg.width) == elems * (7 + 4 + 7)
    # the peak: 256 compute units x 4 SIMDs x 16 lanes at 2.4 GHz
    assert math.isclose(bench.VALU_PEAK_TOPS, 256 * 4 * 16 * 2.4e9 / 1e12)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "single GPU" in r.stderr and r.stdout == ""
