"""Host logic of the parity harness: how side-data differences are classified."""
import numpy as np

import oracle as O
import workloads as W
from harness import SIDE_CASCADE_ULP, compare_blocks, tie_margin


def pair(seed=0):
    f = W.Fmt(64, 0, 16, 64, 32, 4, 2, 0)  # two scale groups per token
    rng = np.random.default_rng(seed)
    a, b = O.HostCache(f, 1, 1), O.HostCache(f, 1, 1)
    for x, y in ((a.codes, b.codes), (a.sz, b.sz), (a.cnorm, b.cnorm)):
        x[...] = rng.integers(0, 256 if x.dtype == np.uint8 else 0x3C00, size=x.shape).astype(x.dtype)
        y[...] = x
    return a, b


def test_identical_blocks():
    a, b = pair()
    st = compare_blocks(a, b, [0])
    assert st["flips"] == st["side_ulp1"] == st["side_bad"] == st["side_cascade"] == 0


def test_side_difference_after_a_normalizer_flip_is_a_cascade():
    a, b = pair()
    a.cnorm[0, 0, 5] += 1                 # channel 5 (group 0) one ulp off
    a.sz[0, 0, 3, 0, 1] += 2              # Z of token 3, group 0: two ulps
    a.sz[0, 0, 7, 0, 0] += SIDE_CASCADE_ULP
    st = compare_blocks(a, b, [0])
    assert st["side_ulp1"] == 1 and st["side_cascade"] == 2 and st["side_bad"] == 0


def test_side_difference_without_a_flip_in_its_group_is_bad():
    a, b = pair()
    a.cnorm[0, 0, 5] += 1                 # group 0
    a.sz[0, 0, 3, 1, 1] += 2              # group 1: not explained
    st = compare_blocks(a, b, [0])
    assert st["side_bad"] == 1 and st["side_cascade"] == 0


def test_large_side_difference_is_bad_even_after_a_flip():
    a, b = pair()
    a.cnorm[0, 0, 5] += 1
    a.sz[0, 0, 3, 0, 0] += SIDE_CASCADE_ULP + 1
    st = compare_blocks(a, b, [0])
    assert st["side_bad"] == 1


def test_normalizer_differences_are_never_cascades():
    a, b = pair()
    a.cnorm[0, 0, 5] += 2
    st = compare_blocks(a, b, [0])
    assert st["side_bad"] == 1 and st["side_cascade"] == 0


def with_quot(a, b, seed=1):
    """b (the oracle side) gets quotients consistent with its codes: code + u, |u| < 0.4."""
    f = b.f
    rng = np.random.default_rng(seed)
    b.quot = O.unpack(b.codes[0, 0], f).astype(np.float64)[None, None] + rng.uniform(-0.4, 0.4, (1, 1, 16, 64))
    return a, b


def set_code(c: O.HostCache, t, j, v):
    codes = O.unpack(c.codes[0, 0], c.f)
    codes[t, j] = v
    c.codes[0, 0] = O.pack(codes, c.f)


def test_flip_at_a_tie_is_explained():
    a, b = with_quot(*pair())
    co = int(O.unpack(b.codes[0, 0], b.f)[4, 9])
    up = co + 1 if co < 15 else co - 1
    b.quot[0, 0, 4, 9] = (co + up) / 2 + 0.3 * tie_margin(4) * (1 if up > co else -1)
    set_code(a, 4, 9, up)
    st = compare_blocks(a, b, [0])
    assert st["flips"] == 1 and st["flips_tie"] == 1 and st["flips_bad"] == 0


def test_flip_far_from_a_tie_is_unexplained():
    a, b = with_quot(*pair())
    co = int(O.unpack(b.codes[0, 0], b.f)[4, 9])
    b.quot[0, 0, 4, 9] = co + 0.1
    set_code(a, 4, 9, co + 1 if co < 15 else co - 1)
    st = compare_blocks(a, b, [0])
    assert st["flips_bad"] == 1 and st["flips_tie"] == 0


def test_flip_after_a_side_difference_is_explained_by_it():
    a, b = with_quot(*pair())
    co = int(O.unpack(b.codes[0, 0], b.f)[6, 40])
    b.quot[0, 0, 6, 40] = co + 0.1
    set_code(a, 6, 40, co + 1 if co < 15 else co - 1)
    a.sz[0, 0, 6, 1, 0] += 1              # S of token 6, group 1 (channels 32..63)
    st = compare_blocks(a, b, [0])
    assert st["flips_side"] == 1 and st["flips_bad"] == 0 and st["side_ulp1"] == 1
