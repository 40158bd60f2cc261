"""Invariant checkers for sort outputs, written independently of the oracle's
sorting loop and of the GPU path.

They check what the pages fix for a stable LSD radix sort: the output is
ordered by the key bits [begin_bit, end_bit), it is a permutation of the input
(keys carried with their payload), and equal digits keep their input order
(page "GPU radix sort: from the CUB implementation to performance tuning",
section 6, fifth pitfall; quant67.com survey, section 11.3, the (value,
original index) order that makes a sort stable).

For float and signed keys the ordering word of a key is the oracle's order
code (float sign-flip, signed sign-bit flip), which tests/test_oracle.py pins
against IEEE-754 ordering, numpy's signed comparisons and closed forms;
unsigned keys need no code.
"""
from __future__ import annotations

import numpy as np

import oracle

UINT_OF = {"u32": np.uint32, "i32": np.uint32, "f32": np.uint32,
           "u64": np.uint64, "i64": np.uint64, "f64": np.uint64}
_TYPE_OF = {np.dtype(np.uint32): "u32", np.dtype(np.int32): "i32", np.dtype(np.float32): "f32",
            np.dtype(np.uint64): "u64", np.dtype(np.int64): "i64", np.dtype(np.float64): "f64"}


def raw_bits(keys: np.ndarray) -> np.ndarray:
    """Keys as unsigned words of the same width (their bit patterns)."""
    return keys.view(UINT_OF[_TYPE_OF[keys.dtype]])


def key_type_of(keys: np.ndarray) -> str:
    return _TYPE_OF[keys.dtype]


def order_field(keys: np.ndarray, begin_bit: int, end_bit: int) -> np.ndarray:
    """F(k) = (T(k) >> begin_bit) mod 2^(end_bit - begin_bit) as uint64."""
    if keys.dtype in (np.uint32, np.uint64):
        words = keys.astype(np.uint64)
    else:
        words = oracle.order_codes(keys)
    width = end_bit - begin_bit
    if width == 0:
        return np.zeros(words.shape, dtype=np.uint64)
    mask = np.uint64((1 << width) - 1)
    return (words >> np.uint64(begin_bit)) & mask


def expected_permutation(keys: np.ndarray, begin_bit: int, end_bit: int) -> np.ndarray:
    """The unique stable permutation, from numpy's stable argsort."""
    return np.argsort(order_field(keys, begin_bit, end_bit), kind="stable")


def check_sorted(out_keys: np.ndarray, begin_bit: int, end_bit: int) -> None:
    f = order_field(out_keys, begin_bit, end_bit)
    bad = np.nonzero(f[1:] < f[:-1])[0]
    assert bad.size == 0, "output not ordered at position %d" % (bad[0] + 1)


def check_multiset(in_keys: np.ndarray, out_keys: np.ndarray) -> None:
    assert in_keys.shape == out_keys.shape
    assert np.array_equal(np.sort(raw_bits(in_keys)), np.sort(raw_bits(out_keys))), \
        "output keys are not a permutation of the input keys"


def check_pairs(in_keys: np.ndarray, out_keys: np.ndarray, out_vals: np.ndarray,
                begin_bit: int, end_bit: int) -> None:
    """Full invariant check for a pair sort whose input payload is 0..n-1."""
    n = in_keys.size
    assert out_keys.shape == in_keys.shape and out_vals.shape == in_keys.shape
    perm = out_vals.astype(np.int64)
    assert perm.size == 0 or (perm.min() >= 0 and perm.max() < n), "payload out of range"
    assert np.array_equal(np.bincount(perm, minlength=n), np.ones(n, dtype=np.int64)), \
        "payload is not a permutation of 0..n-1"
    assert np.array_equal(raw_bits(out_keys), raw_bits(in_keys)[perm]), \
        "an output key is not the input key its payload names"
    check_sorted(out_keys, begin_bit, end_bit)
    f = order_field(out_keys, begin_bit, end_bit)
    ties = f[1:] == f[:-1]
    bad = np.nonzero(ties & (perm[1:] <= perm[:-1]))[0]
    assert bad.size == 0, "equal keys out of input order at position %d" % (bad[0] + 1)


def first_mismatch(a: np.ndarray, b: np.ndarray) -> int:
    """Index of the first differing element of two equal-length arrays, or -1."""
    d = np.nonzero(raw_bits(a) != raw_bits(b))[0]
    return int(d[0]) if d.size else -1
