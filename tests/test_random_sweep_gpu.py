"""A seeded random sweep over the sort's argument space, on cuda:0.

Each case draws every argument at once: key type, keys alone or pairs, n
(log-uniform up to 4M, or at or next to a size where the kernel shapes or the
path change), bit range, key distribution, digit width and in-place use of
keys and values.
The result is compared element by element with the oracle.  The cases come
from a fixed seed, so a failure names a case that can be run again by its
index.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import announce, gpu_sort
from sorting_lsd_radix_sort_amd import inputs

pytestmark = pytest.mark.gpu

KEY_TYPES = ["u32", "i32", "f32", "u64", "i64", "f64"]
# sizes where the path changes: the one-workgroup limits, the small-tile
# bound, the 16-wave shape's threshold, and tile multiples
EDGES = [1, 2, 3, 63, 64, 65, 1023, 1024, 1025, 4095, 4096, 6143, 6144, 6145, 8192, 8193, 16384, 16385,
         99_999, 100_000, 100_001, (1 << 17) - 1, 1 << 17, (1 << 17) + 1, 199_999, 200_000, 200_001,
         (1 << 21) - 1, 1 << 21, (1 << 21) + 1, 16384 * 130 + 5, 8192 * 300 - 1,
         # a block of 24 tiles split in 4 columns, plus one key; a ragged last column
         16384 * 24 * 3 + 1, 393216 * 4 - 7]
CASES = 300


def _case(i):
    rng = np.random.default_rng(7_000 + i)
    key_type = KEY_TYPES[rng.integers(len(KEY_TYPES))]
    bits = 64 if key_type.endswith("64") else 32
    pairs = bool(rng.integers(2))
    if rng.random() < 0.3:
        n = int(EDGES[rng.integers(len(EDGES))])
    else:
        n = int(np.exp(rng.uniform(0, np.log(4_000_000))))
    r = rng.random()
    if r < 0.4:
        b, e = 0, bits
    elif r < 0.45:
        b = e = int(rng.integers(bits + 1))
    else:
        b, e = sorted(int(x) for x in rng.integers(0, bits + 1, size=2))
    dists = ["uniform", "dup", "and3"] + (["fmix"] if key_type.startswith("f") else [])
    dist = dists[rng.integers(len(dists))]
    digit_bits = 11 if rng.random() < 0.25 else 8
    ipk = rng.random() < 0.25
    ipv = pairs and rng.random() < 0.25
    return key_type, pairs, n, b, e, dist, digit_bits, ipk, ipv


@pytest.mark.parametrize("block", range(6))
def test_random_sweep(block):
    per = CASES // 6
    for i in range(block * per, (block + 1) * per):
        key_type, pairs, n, b, e, dist, digit_bits, ipk, ipv = _case(i)
        keys = inputs.random_keys(key_type, n, 9_000 + i, dist)
        vals = np.random.default_rng(i).permutation(n).astype(np.uint32) if pairs else None
        announce("sweep case %d: %s pairs=%s n=%d bits=[%d,%d) %s digits=%d in-place keys=%s vals=%s"
                 % (i, key_type, pairs, n, b, e, dist, digit_bits, ipk, ipv))
        got_k, got_v = gpu_sort(keys, vals, b, e, in_place_keys=ipk, in_place_vals=ipv,
                                digit_bits=digit_bits if digit_bits != 8 or i % 2 else None)
        if pairs:
            want_k, want_v = oracle.sort_pairs(keys, vals, b, e)
            assert np.array_equal(got_v, want_v), "case %d: values differ" % i
        else:
            want_k = oracle.sort_keys(keys, b, e)
        assert np.array_equal(got_k.view(np.uint8), want_k.view(np.uint8)), "case %d: keys differ" % i
