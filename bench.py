#!/usr/bin/env python3
"""Benchmark of the KV-cache quantization hot path on one MI355X.

One step = quantize the K and V of one batch (every tile and kv head of the
workload) and run quantized decode attention over one batch's quantized cache.
The default run times the four workloads (GQA decode, long context, paged
serving, MLA latent) one after the other and quotes the headline on paged
serving, the largest. Inputs are seeded synthetic data already resident in
device memory; a ring of independent copies (inputs and caches) larger than the
256 MB last-level cache makes every step read from and write to HBM: the decode
reads the cache that the quantizer wrote half a ring of steps earlier, not the
one it has just written.

Prints one JSON line: whole-step throughput in GB/s of algorithmic bytes
(inputs read + codes and side data written by the quantizer; codes and side data
of every attended page + queries + outputs for decode) on the headline workload,
the HBM roofline position of its dominant kernel (algorithmic bytes per launch
over the average duration of back-to-back launches), per-workload figures under
"detail", and the CPU oracle timed on a bounded sample of the headline workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantize GB/s (fp16 in) + quantized decode-attn GB/s, % of HBM peak"
HBM_PEAK_GBS = 8000.0
# fp32 VALU lane-operations per second with packed FP32 disabled (the build's flag):
# 256 CUs x 64 lanes x 2.4 GHz
VALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12
# dense f16 / bf16 MFMA, MI355X published
MFMA_F16_PEAK_TFLOPS = 2500.0
ESIZE = {"f32": 4, "bf16": 2}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def block_bytes(f, with_rope=True):
    T, D = f.tile_tokens, f.head_dim
    return T * D * f.bits // 8 + T * (D // f.group) * 4 + 2 * D + (T * f.rope_dim * 2 if with_rope else 0)


def quantize_bytes(cfg, f, width):
    """Algorithmic bytes of one quantizer launch: source read + cache written."""
    read = cfg.total_tokens * cfg.num_kv_heads * width * ESIZE[cfg.src_dtype]
    write = cfg.num_pages * cfg.num_kv_heads * block_bytes(f)
    return read, write


def quantize_valu_ops(cfg, f, width):
    """Algorithmic VALU lane-operations of one quantizer launch: per element log2(h)
    butterfly add/sub + 2 N row/column FMAs + 7 (square, scale, min, max, code FMA,
    clamp, round-and-pack)."""
    elements = cfg.total_tokens * cfg.num_kv_heads * f.head_dim
    return elements * (int(math.log2(f.hadamard_n)) + 2 * f.iters + 7)


def decode_bytes(cfg, seqs=None):
    """Algorithmic bytes of one decode call: every attended page of K and V
    (codes, scale/zero, normalizer, rope), the queries and the fp32 outputs."""
    T = cfg.fk.tile_tokens
    lens = cfg.seq_lens if seqs is None else cfg.seq_lens[seqs]
    pages = int(sum((int(L) + T - 1) // T for L in lens)) * cfg.num_kv_heads
    per_page = block_bytes(cfg.fk) + (block_bytes(cfg.fv) if cfg.fv is not None else 0)
    q = len(lens) * cfg.num_q_heads * cfg.width * ESIZE[cfg.src_dtype]
    out = len(lens) * cfg.num_q_heads * cfg.dv * 4
    return pages * per_page + q + out


CSRC = os.path.join(ROOT, "kv_cache_quantization_04_amd", "csrc")
KERNEL_FILE = {"quantize_d128_kernel": "quantize_d128.hip", "quantize_t16_kernel": "quantize_t16.hip",
               "quantize_d512_kernel": "quantize_d512.hip", "quantize_kernel": "quantize.hip",
               "decode_mfma_kernel": "decode_mfma.hip", "decode_pair16_kernel": "decode_pair16.hip",
               "decode_mla_kernel": "decode_mla.hip",
               "decode_generic_kernel": "decode.hip"}


def source_files(kernel):
    """The kernel's source file and the local headers it includes, transitively."""
    todo, seen = [KERNEL_FILE[kernel]], []
    while todo:
        name = todo.pop()
        if name in seen or not os.path.exists(os.path.join(CSRC, name)):
            continue
        seen.append(name)
        todo += re.findall(r'^#include "([^"]+)"', open(os.path.join(CSRC, name)).read(), re.M)
    return sorted(seen)


def source_digest(kernel):
    """First 16 hex digits of sha256 over the kernel's source files (sorted by name)."""
    h = hashlib.sha256()
    for name in source_files(kernel):
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_traffic(kernel, workload_key):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary,
    or None when there is none or the kernel's source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload_key}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_digest:\s*([0-9a-f]+)", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != source_digest(kernel):
        return None
    return float(t.group(1))


def cpu_baseline(cfg, nseq):
    """The CPU oracle, as it stands, on the first nseq sequences of the workload: fp64
    quantization of their K and V tiles and dequantize-then-softmax decode for every
    query head, on all host threads. GB/s of the same algorithmic bytes as the GPU
    figures, over the sample."""
    import oracle as O
    import workloads as W

    threads = os.cpu_count() or 1
    seqs = list(range(min(nseq, cfg.num_seqs)))
    sel = np.nonzero(np.isin(cfg.tile_seq, seqs))[0]
    t_end = int(cfg.seq_start[seqs[-1]] + cfg.seq_lens[seqs[-1]])
    ks = W.gen_k(cfg, 0, t_end)
    vs = W.gen_v(cfg, 0, t_end) if cfg.fv is not None else None
    q = W.gen_q(cfg)
    Hkv = cfg.num_kv_heads
    dt = O.F32 if cfg.src_dtype == "f32" else O.BF16
    t0 = time.perf_counter()
    kc = O.HostCache(cfg.fk, cfg.num_pages, Hkv)
    O.quantize_cache(kc, ks, dt, cfg.tile_src_token[sel], cfg.tile_valid[sel], cfg.tile_page[sel], nthreads=threads)
    vc = None
    if cfg.fv is not None:
        vc = O.HostCache(cfg.fv, cfg.num_pages, Hkv)
        O.quantize_cache(vc, vs, dt, cfg.tile_src_token[sel], cfg.tile_valid[sel], cfg.tile_page[sel],
                         nthreads=threads)
    tq = time.perf_counter() - t0
    t1 = time.perf_counter()
    O.decode_attn(q[seqs], dt, kc, vc, cfg.block_table[seqs], cfg.seq_lens[seqs], cfg.sm_scale, folded=False,
                  nthreads=threads)
    td = time.perf_counter() - t1
    tokens = int(cfg.seq_lens[seqs].sum())
    W_ = cfg.width
    qb = tokens * Hkv * W_ * ESIZE[cfg.src_dtype] + sel.size * Hkv * block_bytes(cfg.fk)
    if cfg.fv is not None:
        qb += tokens * Hkv * cfg.dv * ESIZE[cfg.src_dtype] + sel.size * Hkv * block_bytes(cfg.fv)
    db = decode_bytes(cfg, seqs)
    return {"value": round((qb + db) / (tq + td) / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{cfg.name.split(':')[0]}: first {len(seqs)} of {cfg.num_seqs} sequences ({tokens} tokens x "
                      f"{Hkv} kv heads): fp64 oracle quantize of their K and V tiles ({tq:.2f} s) and "
                      f"dequantize-then-softmax decode for all {cfg.num_q_heads} query heads ({td:.2f} s), "
                      f"{threads} threads"}


def bench_append(args, cfg, torch, K, W, dev):
    """Append path: every step appends one token to the K and V caches of every
    sequence, starting from the workload's context lengths (each sequence's tail
    holds its partial tile). Timed with HIP events on the launch stream."""
    B, H, T = cfg.num_seqs, cfg.num_kv_heads, cfg.fk.tile_tokens
    total = args.warmup + args.steps
    fmts = [cfg.fk] + ([cfg.fv] if cfg.fv is not None else [])
    widths = [cfg.width] + ([cfg.dv] if cfg.fv is not None else [])
    dt = torch.float32 if cfg.src_dtype == "f32" else torch.bfloat16
    es = ESIZE[cfg.src_dtype]
    lens0 = np.asarray(cfg.seq_lens, np.int64)
    npg = (lens0 + total + T - 1) // T
    P = int(npg.sum())
    bt = np.full((B, int(npg.max())), -1, np.int32)
    k = 0
    for s_ in range(B):
        bt[s_, :npg[s_]] = np.arange(k, k + npg[s_])
        k += int(npg[s_])
    btd = torch.from_numpy(bt).to(dev)
    caches, tails, news = [], [], []
    g = torch.Generator(device=dev)
    g.manual_seed(1000 + args.config)
    for f, w in zip(fmts, widths):
        caches.append(K.DeviceCache(K.make_format(f.head_dim, f.rope_dim, f.tile_tokens, f.hadamard_n, f.group, f.bits,
                                                  f.iters, f.layout), P, H, device=dev))
        tails.append(torch.randn((B, T, H, w), generator=g, device=dev).to(dt))
        news.append(torch.randn((total, B, H, w), generator=g, device=dev).to(dt))
    lens = [torch.from_numpy((lens0 + i).astype(np.int32)).to(dev) for i in range(total)]
    ws = torch.empty(max(K.kv_append_workspace_bytes(B), 4), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        for c, t_, n_ in zip(caches, tails, news):
            K.kv_append(c, t_, n_[i], lens[i], btd, workspace=ws, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.warmup, total):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    # algorithmic bytes per step: the re-quantized rows read, the new rows written to
    # the tails, and each touched page block written whole
    rows = sum(int(((lens0 + i) % T + 1).sum()) for i in range(args.warmup, total)) / args.steps
    byts = sum(rows * H * w * es + B * H * w * es + B * H * block_bytes(f) for f, w in zip(fmts, widths))
    gbs = byts / (ms * 1e-3) / 1e9
    res = {
        "metric": "kv_append tokens/s (one token per sequence per step, K and V re-quantized)",
        "value": round(B / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": cfg.name + " (append)", "seqs": B, "kv_heads": H, "tile_tokens": T,
                   "mean_rows_requantized": round(rows / B, 1)},
        "roofline": {"bound": "hbm", "kernel": "append_prep_kernel + " + K.kv_quantize_kernel_name(caches[0], tails[0].view(B * T, H, -1)),
                     "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 5), "traffic": None, "algorithmic_bytes_per_step": byts,
                     "note": "B x H tiles per launch: latency-bound, far from either roofline"},
    }
    print(json.dumps(res), flush=True)


def bench_prefill(args, cfg, torch, K, W, dev):
    """Chunked prefill attention: the last LQ tokens of every sequence of the workload
    are the chunk (their K and V quantized into the cache with the rest); each step
    is one kv_prefill_attn call. Timed with HIP events on the launch stream."""
    Lq = args.prefill
    B, H, Hq = cfg.num_seqs, cfg.num_kv_heads, cfg.num_q_heads

    def to_dev(a):
        if cfg.src_dtype == "f32":
            return torch.from_numpy(a).to(dev)
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)

    def kfmt(f):
        return K.make_format(f.head_dim, f.rope_dim, f.tile_tokens, f.hadamard_n, f.group, f.bits, f.iters, f.layout)

    tst, tv, tp = i32(cfg.tile_src_token), i32(cfg.tile_valid), i32(cfg.tile_page)
    kc = K.DeviceCache(kfmt(cfg.fk), cfg.num_pages, H, device=dev)
    K.kv_quantize(kc, to_dev(W.gen_k(cfg)), tst, tv, tp)
    vc = None
    if cfg.fv is not None:
        vc = K.DeviceCache(kfmt(cfg.fv), cfg.num_pages, H, device=dev)
        K.kv_quantize(vc, to_dev(W.gen_v(cfg)), tst, tv, tp)
    g = torch.Generator(device=dev)
    g.manual_seed(1000 + args.config)
    dt = torch.float32 if cfg.src_dtype == "f32" else torch.bfloat16
    q = torch.randn((B, Lq, Hq, cfg.width), generator=g, device=dev).to(dt)
    bt, sl = i32(cfg.block_table), i32(cfg.seq_lens)
    max_len = int(cfg.seq_lens.max())
    splits = K.kv_prefill_attn_default_splits(kc, vc, B, Lq, Hq, max_len)
    ws = torch.empty(K.kv_prefill_attn_workspace_bytes(B, Lq, Hq, cfg.dv, splits, bt.shape[1]), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((B, Lq, Hq, cfg.dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        K.kv_prefill_attn(q, kc, vc, bt, sl, max_len, cfg.sm_scale, num_splits=splits, workspace=ws, out=out,
                          stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    kname = K.kv_prefill_attn_kernel_name(q, kc, vc)
    chunk_mode = kname == "decode_mfma_kernel"
    kernel_label = ("" if chunk_mode else "prefill_prep_kernel + ") + kname + " + decode_reduce_kernel"
    if chunk_mode:
        ppb = 16 // (Hq // H)
        note = f"chunk mode: (position, head) MFMA columns, {ppb} positions per page read"
    else:
        note = "each chunk position runs as its own decode sequence: the pages are re-read per position"
    # algorithmic: scores over D + R and values over Dv per (query position, head, attended token)
    attended = float(sum(int(L) - Lq + i + 1 for L in cfg.seq_lens for i in range(Lq)))
    flops = 2.0 * attended * Hq * (cfg.width + cfg.dv)
    tf = flops / (ms * 1e-3) / 1e12
    res = {
        "metric": "prefill query tokens/s (causal chunk over the quantized cache)",
        "value": round(B * Lq / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": cfg.name + f" (prefill chunk {Lq})", "chunk": Lq, "decode_splits": splits},
        "roofline": {"bound": "mfma", "kernel": kernel_label,
                     "achieved": round(tf, 2), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 5), "traffic": None, "algorithmic_flops_per_step": flops,
                     "note": note},
    }
    print(json.dumps(res), flush=True)


def loop_ms(torch, stream, n, fn):
    """Average duration of fn(i), i < n, launched back to back on `stream`: two HIP
    events bracket the whole loop (none between launches)."""
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(n):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def run_config(ci, args, torch, K, W, dev):
    """One workload: quantize K and V + decode per step, on a ring of input copies and
    caches. Returns the step time and, from separate back-to-back loops of each part,
    the quantizer's and the decode call's average durations."""
    cfg = W.config(ci)
    log(f"workload {ci}: {cfg.name}")
    stream = torch.cuda.current_stream()

    def to_dev(a):
        if cfg.src_dtype == "f32":
            return torch.from_numpy(a).to(dev)
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    def kfmt(f):
        return K.make_format(f.head_dim, f.rope_dim, f.tile_tokens, f.hadamard_n, f.group, f.bits, f.iters, f.layout)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)

    tst, tv, tp = i32(cfg.tile_src_token), i32(cfg.tile_valid), i32(cfg.tile_page)
    bt, sl = i32(cfg.block_table), i32(cfg.seq_lens)
    qd = to_dev(W.gen_q(cfg))
    kin_r, kout_w = quantize_bytes(cfg, cfg.fk, cfg.width)
    vin_r, vout_w = quantize_bytes(cfg, cfg.fv, cfg.dv) if cfg.fv is not None else (0, 0)
    qbytes = kin_r + kout_w + vin_r + vout_w
    dbytes = decode_bytes(cfg)
    ring = max(2, math.ceil(args.ring_mb * 1e6 / qbytes))
    t0 = time.perf_counter()
    ksrc0 = to_dev(W.gen_k(cfg))
    vsrc0 = to_dev(W.gen_v(cfg)) if cfg.fv is not None else None
    log(f"  inputs generated and uploaded in {time.perf_counter() - t0:.1f} s; ring of {ring} copies "
        f"({ring * qbytes / 1e6:.0f} MB live)")
    ksrc = [ksrc0] + [ksrc0.clone() for _ in range(ring - 1)]
    vsrc = ([vsrc0] + [vsrc0.clone() for _ in range(ring - 1)]) if vsrc0 is not None else [None] * ring
    kcache = [K.DeviceCache(kfmt(cfg.fk), cfg.num_pages, cfg.num_kv_heads, device=dev) for _ in range(ring)]
    vcache = ([K.DeviceCache(kfmt(cfg.fv), cfg.num_pages, cfg.num_kv_heads, device=dev) for _ in range(ring)]
              if cfg.fv is not None else [None] * ring)
    max_len = int(cfg.seq_lens.max())
    splits = args.splits or K.kv_decode_attn_default_splits(kcache[0], vcache[0], cfg.num_seqs, cfg.num_q_heads, max_len)
    ws = K.decode_workspace(K.kv_decode_attn_workspace_bytes(cfg.num_seqs, cfg.num_q_heads, cfg.dv, splits), dev)
    out = torch.empty((cfg.num_seqs, cfg.num_q_heads, cfg.dv), dtype=torch.float32, device=dev)
    # K and V in one launch (kv_quantize_kv) where the library takes the pair of formats
    pair = False
    if vsrc[0] is not None:
        try:
            K.kv_quantize_kv(kcache[0], vcache[0], ksrc[0], vsrc[0], tst, tv, tp, stream=stream)
            pair = True
        except K.KvqError as e:
            if e.status != K.KVQ_EUNSUPPORTED:
                raise

    def quantize(j):
        if pair:
            K.kv_quantize_kv(kcache[j], vcache[j], ksrc[j], vsrc[j], tst, tv, tp, stream=stream)
        else:
            K.kv_quantize(kcache[j], ksrc[j], tst, tv, tp, stream=stream)
            if vsrc[j] is not None:
                K.kv_quantize(vcache[j], vsrc[j], tst, tv, tp, stream=stream)

    def decode(j):
        K.kv_decode_attn(qd, kcache[j], vcache[j], bt, sl, max_len, cfg.sm_scale, num_splits=splits, workspace=ws,
                         out=out, stream=stream)

    # Every ring slot holds a quantized cache before the first step. Step i quantizes
    # slot i mod ring and decodes the cache of slot i - ring/2, written half a ring of
    # steps earlier: neither the quantizer's source nor the decoder's cache is still in
    # the 256 MB last-level cache (at least one copy's traffic in between).
    for j in range(ring):
        quantize(j)
    lag = ring // 2

    def step(i):
        quantize(i % ring)
        decode((i - lag) % ring)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step_ms = loop_ms(torch, stream, args.steps, step)
    wall = time.perf_counter() - t0
    log(f"  timed {args.steps} steps: {step_ms * args.steps:.3f} ms on device, {wall * 1e3:.3f} ms wall")
    # each part alone, back to back over the ring (no event between launches)
    n = max(args.steps, 2 * ring)
    tq = loop_ms(torch, stream, n, lambda i: quantize(i % ring))
    td = loop_ms(torch, stream, n, lambda i: decode(i % ring))
    log(f"  quantize {tq * 1e3:.1f} us per step, decode {td * 1e3:.1f} us per call ({n} back to back)")

    nq = 2 if cfg.fv is not None and not pair else 1  # quantizer launches per step
    qnames = sorted({K.kv_quantize_kernel_name(kcache[0], ksrc[0])} |
                    ({K.kv_quantize_kernel_name(vcache[0], vsrc[0])} if vsrc[0] is not None else set()))
    dname = K.kv_decode_attn_kernel_name(qd, kcache[0], vcache[0])
    mname = K.kv_decode_attn_merge_kernel_name(qd, kcache[0], vcache[0], splits, max_len)
    qops = quantize_valu_ops(cfg, cfg.fk, cfg.width) + (quantize_valu_ops(cfg, cfg.fv, cfg.dv)
                                                        if cfg.fv is not None else 0)
    positions = int(cfg.seq_lens.sum())
    q_gbs = qbytes / (tq * 1e-3) / 1e9
    d_gbs = dbytes / (td * 1e-3) / 1e9
    r = {
        "workload": cfg.name, "key": W.NAMES[ci], "step_ms": round(step_ms, 5),
        "step_GBps": round((qbytes + dbytes) / (step_ms * 1e-3) / 1e9, 2),
        "quantize_kernels": qnames, "quantize_launches": nq, "quantize_us": round(tq * 1e3, 2),
        "quantize_GBps": round(q_gbs, 2), "quantize_frac_hbm": round(q_gbs / HBM_PEAK_GBS, 4),
        "quantize_input_GBps": round((kin_r + vin_r) / (tq * 1e-3) / 1e9, 2),
        "quantize_tokens_per_s": round((2 if cfg.fv is not None else 1) * cfg.total_tokens * cfg.num_kv_heads /
                                       (tq * 1e-3), 1),
        "quantize_valu_frac": round(qops / (tq * 1e-3) / 1e12 / VALU_PEAK_TOPS, 4),
        "decode_kernel": dname + (" + " + mname if mname else " (split merge inside)"), "decode_splits": splits, "decode_us": round(td * 1e3, 2),
        "decode_GBps": round(d_gbs, 2), "decode_frac_hbm": round(d_gbs / HBM_PEAK_GBS, 4),
        "decode_positions_per_s": round(positions / (td * 1e-3), 1),
        "decode_tokens_per_s": round(cfg.num_seqs / (td * 1e-3), 1),
        "quantize_bytes": qbytes, "decode_bytes": dbytes, "copy_ring": ring,
    }
    if dname == "decode_mla_kernel":
        # dense f16 MFMA contraction: scores over D + R channels and values over D, per head and position
        flops = 2.0 * positions * cfg.num_q_heads * (cfg.width + cfg.dv)
        r["decode_TFLOPs"] = round(flops / (td * 1e-3) / 1e12, 2)
        r["decode_frac_mfma_f16"] = round(flops / (td * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)
    # the dominant kernel of the step and its HBM roofline position: algorithmic bytes
    # per launch over the average launch duration
    if tq >= td:
        kern = qnames[0] if len(qnames) == 1 else " / ".join(qnames)
        per_launch, launch_ms = qbytes / nq, tq / nq
        other = {"valu": {"achieved": round(qops / nq / (launch_ms * 1e-3) / 1e12, 3),
                          "peak": round(VALU_PEAK_TOPS, 2), "unit": "T VALU lane-ops/s",
                          "frac": r["quantize_valu_frac"],
                          "algorithmic_ops_per_launch": qops / nq}}
        traffic = profiled_traffic(qnames[0], W.NAMES[ci]) if len(qnames) == 1 else None
    else:
        kern = dname
        per_launch, launch_ms = dbytes, td
        other = {}
        if "decode_TFLOPs" in r:
            other = {"mfma": {"achieved": r["decode_TFLOPs"], "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                              "frac": r["decode_frac_mfma_f16"]}}
        traffic = profiled_traffic(dname, W.NAMES[ci])
    gbs = per_launch / (launch_ms * 1e-3) / 1e9
    r["roofline"] = dict(bound="hbm", kernel=kern, achieved=round(gbs, 2), peak=HBM_PEAK_GBS, unit="GB/s",
                         frac=round(gbs / HBM_PEAK_GBS, 4), traffic=traffic, algorithmic_bytes_per_launch=per_launch,
                         avg_launch_us=round(launch_ms * 1e3, 3), **other)
    return r, cfg


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--splits", type=int, default=0, help="decode split count (0: the library's default rule)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--configs", default="1,2,3,4", help="workload indices timed in this run")
    ap.add_argument("--headline", type=int, default=3,
                    help="workload the headline value is quoted on (3 = paged serving, the largest)")
    ap.add_argument("--config", type=int, default=None, help="time one workload only (it is then the headline)")
    ap.add_argument("--ring-mb", type=int, default=2048, help="live bytes of the copy ring")
    ap.add_argument("--cpu-seqs", type=int, default=64, help="sequences of the headline workload the oracle times")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--append", action="store_true",
                    help="measure the append path (one token per sequence per step, K and V) instead")
    ap.add_argument("--prefill", type=int, default=0, metavar="LQ",
                    help="measure chunked prefill attention with LQ query positions per sequence instead")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures a single GPU: the quantizer and decode shard by sequence and kv head with no "
              "exchange, so no multi-GPU figure is produced; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import kv_cache_quantization_04_amd as K
    import workloads as W

    dev = torch.device("cuda:0")
    if args.append or args.prefill > 0:
        args.config = 1 if args.config is None else args.config
        cfg = W.config(args.config)
        log(f"workload: {cfg.name}")
        (bench_append if args.append else bench_prefill)(args, cfg, torch, K, W, dev)
        return
    if args.config is not None:
        configs, headline = [args.config], args.config
    else:
        configs, headline = [int(c) for c in args.configs.split(",")], args.headline
        if headline not in configs:
            configs.append(headline)
    per, hcfg = {}, None
    for ci in configs:
        r, cfg = run_config(ci, args, torch, K, W, dev)
        per[r["key"]] = r
        if ci == headline:
            hcfg, h = cfg, r
        torch.cuda.empty_cache()
    res = {
        "metric": METRIC,
        "value": h["step_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": hcfg.name, "kv_layout": "K token-major, V channel-major, fp16 side data",
                   "decode_splits": h["decode_splits"], "copy_ring": h["copy_ring"],
                   "quantize_launches": h["quantize_launches"]},
        "roofline": h["roofline"],
        "detail": {"headline": h["key"], "step": "quantize K and V of the batch + one decode call",
                   "configs": {k: {kk: vv for kk, vv in v.items() if kk not in ("workload", "key")}
                               for k, v in per.items()}},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(hcfg, args.cpu_seqs)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
