"""Host logic of the parity harness: how side-data differences are classified."""
import numpy as np

import oracle as O
import workloads as W
from harness import SIDE_CASCADE_ULP, compare_blocks


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
