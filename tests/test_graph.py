"""The hot path under HIP graph capture: quantizing K and V and the decode call are
recorded once into a graph (torch.cuda.CUDAGraph on the launch stream) and replayed
several times, with other device work between the replays; every replay must give the
same bits as the eager calls. The library issues kernel launches only (no memset, no
allocation, no copy), so the captured graph holds nothing else."""
import math
import sys

import numpy as np
import pytest
import torch

import kv_cache_quantization_04_amd as K
from harness import i32, kfmt, to_dev
from test_gpu_parity import small_paged

pytestmark = pytest.mark.gpu

CASES = [
    # 16-token pages, g = 8 (two pages per matrix-core pass), one quantize launch per cache
    dict(T=16, lens=(100, 37, 260), kbits=3, vbits=3, Hq=16, Hkv=2),
    # 128-token pages: K and V in one quantize launch, decode over whole-page images
    dict(T=128, lens=(300, 129), kbits=4, vbits=4, iters=4, Hq=8, Hkv=2, pair=True),
    # MLA latent + rope
    dict(mla=True, D=512, R=64, T=128, Hq=32, Hkv=1, lens=(300, 129), iters=4),
]


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("kw", CASES, ids=["paged16", "pair128", "mla"])
@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
def test_graph_replays_equal_eager(gpu, kw, noalloc):
    kw = dict(kw)
    pair = kw.pop("pair", False)
    w = small_paged(31 + len(kw), **kw)
    log("graph case", kw, "pair", pair, "noalloc", noalloc)
    f_k, f_v, dt = w["fk"], w["fv"], w["dtype"]
    ks = to_dev(w["ks"], dt)
    vs = to_dev(w["vs"], dt) if f_v is not None else None
    tst, tv, tp = i32(w["tst"]), i32(w["tv"]), i32(w["tp"])
    q, bt, sl = to_dev(w["q"], dt), i32(w["bt"]), i32(w["lens"])
    L = int(w["lens"].max())
    sm = 1.0 / math.sqrt(f_k.head_dim + f_k.rope_dim)
    dk = K.DeviceCache(kfmt(f_k), w["P"], w["Hkv"])
    dv = K.DeviceCache(kfmt(f_v), w["P"], w["Hkv"]) if f_v is not None else None
    splits = K.kv_decode_attn_default_splits(dk, dv, q.shape[0], q.shape[1], L)
    ws = torch.zeros(max(4, K.kv_decode_attn_workspace_bytes(q.shape[0], q.shape[1], (dv or dk).fmt.head_dim, splits)),
                     dtype=torch.uint8, device=gpu)
    out = torch.zeros((q.shape[0], q.shape[1], (dv or dk).fmt.head_dim), dtype=torch.float32, device=gpu)

    def step():
        if pair:
            K.kv_quantize_kv(dk, dv, ks, vs, tst, tv, tp)
        else:
            K.kv_quantize(dk, ks, tst, tv, tp)
            if dv is not None:
                K.kv_quantize(dv, vs, tst, tv, tp)
        if noalloc:
            K.kv_decode_attn_noalloc(q, dk, dv, bt, sl, L, sm, num_splits=splits, out=out)
        else:
            K.kv_decode_attn(q, dk, dv, bt, sl, L, sm, num_splits=splits, workspace=ws, out=out)

    def state():
        parts = [dk.codes, dk.sz, dk.cnorm, out]
        if dk.rope is not None:
            parts.append(dk.rope)
        if dv is not None:
            parts += [dv.codes, dv.sz, dv.cnorm]
        return [p.clone() for p in parts]

    def clear():  # fill kernels (no memset nodes anywhere)
        for t in [dk.codes, dk.sz, dk.cnorm, out] + ([dk.rope] if dk.rope is not None else []) + \
                 ([dv.codes, dv.sz, dv.cnorm] if dv is not None else []):
            t.zero_()

    step()
    torch.cuda.synchronize()
    ref = state()
    assert any(bool(p.any()) for p in ref)

    side = torch.cuda.Stream()
    with torch.cuda.stream(side):  # warm-up on the capture stream, as torch asks
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    clear()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    other = torch.randn(256, 256, device=gpu)
    for r in range(4):
        clear()
        other = other @ other.T / 256.0  # unrelated eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = state()
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {r}"
        log("  replay", r, "equal to eager")
