"""kv_decode_attn_noalloc (the split partials in the library's per-GPU scratch array)
against kv_decode_attn (a caller workspace): the same kernels and split rule, so the
outputs are equal bit for bit; two calls in a row, the second smaller, then a request
beyond the scratch size, which is refused before any launch."""
import math
import sys

import numpy as np
import pytest
import torch

import kv_cache_quantization_04_amd as K
from harness import i32, kfmt, to_dev, upload, orc_quantize
from test_gpu_parity import small_paged

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def caches(w):
    kc, _ = orc_quantize(w["fk"], w["ks"], w["dtype"], w["tst"], w["tv"], w["tp"], w["P"], with_quot=False)
    dk = K.DeviceCache(kfmt(w["fk"]), w["P"], w["Hkv"])
    upload(kc, dk)
    dv = None
    if w["fv"] is not None:
        vc, _ = orc_quantize(w["fv"], w["vs"], w["dtype"], w["tst"], w["tv"], w["tp"], w["P"], with_quot=False)
        dv = K.DeviceCache(kfmt(w["fv"]), w["P"], w["Hkv"])
        upload(vc, dv)
    return dk, dv


def test_noalloc_decode_equals_workspace_decode(gpu):
    cases = [
        dict(T=16, lens=(3000, 700, 17, 1), kbits=3, vbits=3, Hq=16, Hkv=2),           # staged 16-token pages
        dict(T=128, lens=(600, 131), kbits=4, vbits=2, iters=4),                         # smaller, second call
        dict(mla=True, D=512, R=64, T=128, Hq=16, Hkv=1, lens=(300, 5), iters=4),       # MLA kernel
    ]
    for n, kw in enumerate(cases):
        log("noalloc case", kw)
        w = small_paged(300 + n, **kw)
        dk, dv = caches(w)
        q = to_dev(w["q"], w["dtype"])
        bt, sl, L = i32(w["bt"]), i32(w["lens"]), int(w["lens"].max())
        sm = 1.0 / math.sqrt(w["fk"].head_dim + w["fk"].rope_dim)
        for splits in (0, 3):
            ref = K.kv_decode_attn(q, dk, dv, bt, sl, L, sm, num_splits=splits)
            got = K.kv_decode_attn_noalloc(q, dk, dv, bt, sl, L, sm, num_splits=splits)
            torch.cuda.synchronize()
            assert torch.equal(got, ref), f"{kw} splits {splits}"
            assert bool(torch.isfinite(got).all())


def test_noalloc_refuses_partials_beyond_the_scratch(gpu):
    w = small_paged(310, T=16, lens=(40, 20), kbits=3, vbits=3, Hq=16, Hkv=2)
    dk, dv = caches(w)
    q = to_dev(w["q"], w["dtype"])
    B, Hq = q.shape[0], q.shape[1]
    splits = 1024
    assert K.kv_decode_attn_workspace_bytes(B, Hq, 128, splits) <= K.KVQ_NOALLOC_SCRATCH_BYTES  # fits: runs
    out = K.kv_decode_attn_noalloc(q, dk, dv, i32(w["bt"]), i32(w["lens"]), 40, 0.1, num_splits=splits)
    ref = K.kv_decode_attn(q, dk, dv, i32(w["bt"]), i32(w["lens"]), 40, 0.1, num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    # 64 sequences x 64 heads x 1024 splits of 130 floats: far beyond the scratch
    qb = torch.zeros((64, 64, 128), dtype=torch.bfloat16, device=gpu)
    bt = i32(np.zeros((64, 8), np.int32))
    sl = i32(np.ones(64, np.int32))
    assert K.kv_decode_attn_workspace_bytes(64, 64, 128, 1024) > K.KVQ_NOALLOC_SCRATCH_BYTES
    sentinel = torch.full((64, 64, 128), 7.0, device=gpu)
    dk8 = K.DeviceCache(kfmt(w["fk"]), w["P"], 8)
    dv8 = K.DeviceCache(kfmt(w["fv"]), w["P"], 8)
    with pytest.raises(K.KvqError) as e:
        K.kv_decode_attn_noalloc(qb, dk8, dv8, bt, sl, 16, 0.1, num_splits=1024, out=sentinel)
    assert e.value.status == K.KVQ_EWORKSPACE
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all())
