"""lrs_sort_digits_noalloc: the sort with the library's static per-GPU scratch
instead of caller temp storage (for callers that cannot allocate).

Each case makes two calls in a row, the second on a smaller input, and
compares each output, bit for bit, with lrs_sort_digits on the same input
with caller temp storage (itself parity-tested against the oracle).  Also:
in-place use, a sort too large for the scratch (rejected, nothing written),
and the call captured into a HIP graph and replayed on new input.
"""
from __future__ import annotations

import numpy as np
import pytest

import sorting_lsd_radix_sort_amd as lrs
from gpu_util import announce, to_dev, to_host
from sorting_lsd_radix_sort_amd import inputs

pytestmark = pytest.mark.gpu

KEY_BITS = {"u32": 32, "i32": 32, "f32": 32, "u64": 64, "i64": 64, "f64": 64}


def reference(key_type, digit_bits, keys, vals, begin_bit, end_bit):
    """lrs_sort_digits with caller temp storage."""
    import torch
    kin = to_dev(keys)
    kout = torch.empty_like(kin)
    vin = None if vals is None else to_dev(vals)
    vout = None if vals is None else torch.empty_like(vin)
    n = keys.size
    need = lrs.lrs_sort_digits(key_type, digit_bits, None, 0, kin, vin, kout, vout, n, begin_bit, end_bit)
    temp = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    lrs.lrs_sort_digits(key_type, digit_bits, temp, need, kin, vin, kout, vout, n, begin_bit, end_bit)
    torch.cuda.synchronize()
    return to_host(kout), None if vals is None else to_host(vout)


def noalloc(key_type, digit_bits, keys, vals, begin_bit, end_bit, in_place=False):
    import torch
    kin = to_dev(keys)
    kout = kin if in_place else torch.empty_like(kin)
    vin = None if vals is None else to_dev(vals)
    vout = None if vals is None else (vin if in_place else torch.empty_like(vin))
    torch.cuda.synchronize()
    lrs.lrs_sort_digits_noalloc(key_type, digit_bits, kin, vin, kout, vout, keys.size, begin_bit, end_bit)
    torch.cuda.synchronize()
    return to_host(kout), None if vals is None else to_host(vout)


def same(a, b):
    return a is None and b is None or np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("key_type,pairs,digit_bits,bits,sizes", [
    ("u32", False, 8, (0, 32), (3_000_017, 1_000_003)),     # multi-pass path, then a smaller one
    ("f32", True, 8, (0, 32), (1_500_007, 70_001)),
    ("u64", True, 8, (0, 64), (1_000_003, 30_011)),
    ("i32", False, 11, (0, 32), (2_000_003, 17_000)),       # 2048-digit passes
    ("u32", True, 8, (0, 20), (7_000_001, 16_384)),          # near the limit, then one launch per pass
    ("f64", False, 8, (3, 41), (2_500_001, 400_009)),
])
def test_noalloc_matches_sort_digits(key_type, pairs, digit_bits, bits, sizes):
    for rep, n in enumerate(sizes):
        announce("noalloc %s pairs=%s digits=%d bits=%s n=%d call %d" % (key_type, pairs, digit_bits, bits, n, rep))
        keys = inputs.random_keys(key_type, n, 500 + rep, "uniform" if rep == 0 else "dup")
        vals = np.arange(n, dtype=np.uint32) if pairs else None
        want_k, want_v = reference(key_type, digit_bits, keys, vals, *bits)
        got_k, got_v = noalloc(key_type, digit_bits, keys, vals, *bits)
        assert same(got_k, want_k), "keys differ (call %d)" % rep
        assert same(got_v, want_v), "values differ (call %d)" % rep


@pytest.mark.parametrize("key_type,pairs,passes_bits", [("u32", True, (0, 24)), ("u64", False, (0, 64))])
def test_noalloc_in_place(key_type, pairs, passes_bits):
    n = 1_234_567
    keys = inputs.random_keys(key_type, n, 77, "uniform")
    vals = np.arange(n, dtype=np.uint32) if pairs else None
    announce("noalloc in place %s n=%d bits=%s" % (key_type, n, passes_bits))
    want_k, want_v = reference(key_type, 8, keys, vals, *passes_bits)
    got_k, got_v = noalloc(key_type, 8, keys, vals, *passes_bits, in_place=True)
    assert same(got_k, want_k) and same(got_v, want_v)


def test_noalloc_too_large_is_rejected_and_writes_nothing():
    import torch
    n = lrs.NOALLOC_SCRATCH_BYTES // 4 + 1   # the alternate key buffer alone exceeds the scratch
    announce("noalloc too large n=%d" % n)
    kin = torch.zeros(n, dtype=torch.int32, device="cuda:0").view(torch.uint32)
    kout = torch.full((n,), 7, dtype=torch.int32, device="cuda:0")
    with pytest.raises(lrs.LrsError) as ei:
        lrs.lrs_sort_digits_noalloc("u32", 8, kin, None, kout, None, n, 0, 32)
    assert ei.value.status == lrs.LRS_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert int((kout != 7).sum().item()) == 0
    # and the call right below the limit works
    small = inputs.random_keys("u32", 2_000_000, 3, "uniform")
    got_k, _ = noalloc("u32", 8, small, None, 0, 32)
    want_k, _ = reference("u32", 8, small, None, 0, 32)
    assert same(got_k, want_k)


def test_noalloc_in_a_graph():
    """Captured into a HIP graph (torch.cuda.graph) and replayed on new input,
    with eager work between replays: every replay equals lrs_sort_digits on
    the same input."""
    import torch
    n = 1_000_003
    announce("noalloc graph replays n=%d" % n)
    kin = torch.empty(n, dtype=torch.int32, device="cuda:0").view(torch.uint32)
    vin = torch.empty(n, dtype=torch.int32, device="cuda:0").view(torch.uint32)
    kout = torch.empty_like(kin)
    vout = torch.empty_like(vin)
    first = inputs.random_keys("u32", n, 1, "uniform")
    kin.copy_(to_dev(first))
    vin.copy_(to_dev(np.arange(n, dtype=np.uint32)))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lrs.lrs_sort_digits_noalloc("u32", 8, kin, vin, kout, vout, n, 0, 32, s)  # first call: outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lrs.lrs_sort_digits_noalloc("u32", 8, kin, vin, kout, vout, n, 0, 32)
    for rep in range(4):
        keys = inputs.random_keys("u32", n, 40 + rep, "dup" if rep % 2 else "uniform")
        vals = np.random.default_rng(rep).permutation(n).astype(np.uint32)
        kin.copy_(to_dev(keys))
        vin.copy_(to_dev(vals))
        torch.cuda.synchronize()
        g.replay()
        (torch.arange(1 << 20, device="cuda:0") * 3).sum().item()  # eager work between replays
        torch.cuda.synchronize()
        want_k, want_v = reference("u32", 8, keys, vals, 0, 32)
        assert same(to_host(kout), want_k), "replay %d: keys" % rep
        assert same(to_host(vout), want_v), "replay %d: values" % rep
