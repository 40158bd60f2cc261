"""The sort captured into a HIP graph (torch.cuda.graph) and replayed.

The library enqueues only kernel launches on the caller's stream (no memset,
no host synchronization, no allocation), so a sort with its temp storage
allocated beforehand can be captured.  Each replay runs on new input written
between replays, with eager work in between, and its output is checked
against an eager sort of the same input (bit-exact), several times over.
"""
from __future__ import annotations

import numpy as np
import pytest

import sorting_lsd_radix_sort_amd as lrs
from gpu_util import announce, to_dev, to_host
from sorting_lsd_radix_sort_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("key_type,n,pairs,digit_bits", [("u32", 65_536, False, 8), ("f32", 300_007, True, 8),
                                                         ("u64", 100_003, True, 8), ("u32", 200_003, False, 11),
                                                         ("u32", 5_000, True, 8)])
def test_graph_replays_match_eager(key_type, n, pairs, digit_bits):
    import torch
    announce("graph capture %s n=%d pairs=%s digits=%d" % (key_type, n, pairs, digit_bits))
    first = inputs.random_keys(key_type, n, 90, "fmix" if key_type in ("f32",) else "uniform")
    kin = to_dev(first)
    kout = torch.empty_like(kin)
    vin = to_dev(np.arange(n, dtype=np.uint32)) if pairs else None
    vout = torch.empty_like(vin) if pairs else None
    need = lrs.lrs_sort_digits(key_type, digit_bits, None, 0, kin, vin, kout, vout, n, 0,
                               8 * first.dtype.itemsize)
    temp = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    bits = 8 * first.dtype.itemsize

    def sort_on_current_stream():
        lrs.lrs_sort_digits(key_type, digit_bits, temp, need, kin, vin, kout, vout, n, 0, bits,
                            torch.cuda.current_stream())

    # eager once (warms the library's per-device caches), then capture
    sort_on_current_stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sort_on_current_stream()
    torch.cuda.synchronize()

    for rep in range(4):
        data = inputs.random_keys(key_type, n, 100 + rep, "dup" if rep % 2 else "uniform")
        kin.copy_(to_dev(data))
        if pairs:
            vin.copy_(to_dev(np.random.default_rng(rep).permutation(n).astype(np.uint32)))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_k = to_host(kout).copy()
        got_v = to_host(vout).copy() if pairs else None
        # eager sort of the same input, with some unrelated eager work first
        (torch.arange(1 << 20, device="cuda:0") * 3).sum().item()
        sort_on_current_stream()
        torch.cuda.synchronize()
        assert np.array_equal(got_k.view(np.uint8), to_host(kout).view(np.uint8)), "replay %d: keys differ" % rep
        if pairs:
            assert np.array_equal(got_v, to_host(vout)), "replay %d: values differ" % rep


@pytest.mark.parametrize("profiling", [False, True])
def test_concurrent_calls_on_separate_streams(profiling):
    """Calls from several host threads at once, each on its own stream with its
    own temp storage (the library's per-device caches are shared), each
    bit-exact with the oracle's result for its input; also with per-launch
    profiling on (every thread's launches then reserve records under the
    library's lock, and every record reads back)."""
    import threading
    import torch
    import oracle
    announce("concurrent calls on separate streams, profiling %s" % profiling)
    if profiling:
        lrs.lrs_prof_start(64)  # fewer records than launches: the rest go unrecorded
    cases = [("u32", 300_001, 1), ("f32", 200_003, 2), ("u64", 150_001, 3), ("i32", 250_007, 4)]
    data = {c: inputs.random_keys(c[0], c[1], c[2], "uniform") for c in cases}
    results, errors = {}, []

    def work(case):
        try:
            keys = data[case]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                kin = to_dev(keys)
                for _ in range(3):
                    out = lrs.sort_keys(kin, stream=s)
            s.synchronize()
            results[case] = to_host(out)
        except Exception as e:  # reported below, in the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(c,)) for c in cases]
    try:
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        if profiling:
            lrs.lrs_prof_stop()
            count = lrs.lrs_prof_count()
            assert count == 64, count
            for i in range(count):
                kind, ms = lrs.lrs_prof_read(i)
                assert kind in lrs.KERNEL_NAMES and ms >= 0.0
    finally:
        if profiling:
            lrs.lrs_prof_release()
    assert not errors, errors
    for c in cases:
        want = oracle.sort_keys(data[c])
        assert np.array_equal(results[c].view(np.uint8), want.view(np.uint8)), c


def test_side_stream_outside_stream_context():
    """sort_keys / sort_pairs on a side stream, called outside any stream
    context: their temp storage and outputs come from torch's current stream,
    so they are recorded on the side stream; memory allocated and filled on the
    current stream right after the calls must not disturb the sorts still
    running there.  Both results bit-exact with the oracle."""
    import torch
    import oracle
    announce("side stream outside a stream context")
    keys = inputs.random_keys("u32", 3_000_017, 11, "uniform")
    vals = np.arange(keys.size, dtype=np.uint32)
    kin, vin = to_dev(keys), to_dev(vals)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    # a long queue on the side stream, so the sorts are still running when the
    # current stream reuses freed memory
    ko = lrs.sort_keys(kin, stream=s)
    for _ in range(4):
        ko2, vo2 = lrs.sort_pairs(kin, vin, stream=s)
    junk = [torch.full((keys.size * 2,), 0x5A5A5A5A, dtype=torch.int32, device="cuda:0") for _ in range(6)]
    s.synchronize()
    torch.cuda.synchronize()
    del junk
    want_k = oracle.sort_keys(keys)
    wk, wv = oracle.sort_pairs(keys, vals)
    assert np.array_equal(to_host(ko), want_k)
    assert np.array_equal(to_host(ko2), wk)
    assert np.array_equal(to_host(vo2), wv)
