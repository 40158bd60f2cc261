"""Pins of the CPU oracle to facts the pages and mathematics fix (no GPU).

Each test checks the oracle against something other than itself: values the
pages print, IEEE-754 float ordering enumerated exhaustively, Python's stable
comparison sort on every short sequence over colliding alphabets, numpy's
stable argsort, and closed forms (constant keys, sorted inputs).
"""
from __future__ import annotations

import itertools
import math
import os
import subprocess

import numpy as np
import pytest

import checks
import oracle
from sorting_lsd_radix_sort_amd import inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


# ---------------------------------------------------------------- worked examples

def test_worked_example_keys():
    """kwkr.cn essay, section 2.2: [4,2,7,1,8,3,6,5] sorts to [1..8]."""
    lines = dict(ln.split(":", 1) for ln in _golden_lines("p1_s2_2_worked_example.txt"))
    src = np.array(lines["input"].split(), dtype=np.uint32)
    want = np.array(lines["output"].split(), dtype=np.uint32)
    assert np.array_equal(oracle.sort_keys(src), want)
    # Same keys as uint64 and as float32 values give the same order.
    assert np.array_equal(oracle.sort_keys(src.astype(np.uint64)), want.astype(np.uint64))
    assert np.array_equal(oracle.sort_keys(src.astype(np.float32)), want.astype(np.float32))


def test_worked_example_pairs():
    """With an original-index payload the output payload is where each printed
    output key stood in the printed input (the keys are distinct)."""
    lines = dict(ln.split(":", 1) for ln in _golden_lines("p1_s2_2_worked_example.txt"))
    src = [int(x) for x in lines["input"].split()]
    want = [int(x) for x in lines["output"].split()]
    want_payload = [src.index(k) for k in want]
    ko, vo = oracle.sort_pairs(np.array(src, dtype=np.uint32), np.arange(8, dtype=np.uint32))
    assert ko.tolist() == want and vo.tolist() == want_payload == [3, 1, 5, 0, 7, 6, 2, 4]


def test_bitonic_sequence_closed_form():
    """quant67.com survey, section 3.1 prints [1,3,5,7,6,4,2,0] as a bitonic
    sequence; its ascending sort is 0..7 (distinct values)."""
    got = oracle.sort_keys(np.array([1, 3, 5, 7, 6, 4, 2, 0], dtype=np.uint32))
    assert got.tolist() == list(range(8))


def test_float_patterns_from_page():
    """kwkr.cn essay, section 3.3: -1.0 is 0xBF800000 and 1.0 is 0x3F800000;
    as unsigned words they order wrongly, through the encoding they order right."""
    rows = [ln.split() for ln in _golden_lines("p1_s3_3_float_patterns.txt")]
    vals = np.array([float(r[0]) for r in rows], dtype=np.float32)
    pats = np.array([int(r[1], 16) for r in rows], dtype=np.uint32)
    assert np.array_equal(vals.view(np.uint32), pats)
    # Unsigned order of the raw patterns puts 1.0 first: the page's warning.
    assert oracle.sort_keys(pats).view(np.float32).tolist() == [1.0, -1.0]
    # The float sort puts -1.0 first; the encoded words are ordered.
    assert oracle.sort_keys(vals).tolist() == [-1.0, 1.0]
    enc = oracle.f2s(pats)
    assert enc[0] < enc[1]


def test_int32_endpoints_from_page():
    """Page "GPU radix sort ...", section 5.2: sign-flipped int32 endpoints map to
    0 and 0xFFFFFFFF; a uint32 sort of such words puts them in signed order."""
    rows = [ln.split() for ln in _golden_lines("p3_s5_2_int32_endpoints.txt")]
    ints = np.array([int(r[0]) for r in rows], dtype=np.int64)
    words = np.array([int(r[1], 16) for r in rows], dtype=np.uint32)
    # mapping check is on the page's own numbers
    assert np.array_equal(((ints + 2**31) & 0xFFFFFFFF).astype(np.uint32), words)
    order = oracle.sort_pairs(words[::-1].copy(), np.arange(2, dtype=np.uint32))[1]
    assert ints[::-1][order].tolist() == sorted(ints.tolist())


# ------------------------------------------------------- float transform, exhaustive

def test_float_transform_exhaustive(tmp_path):
    """Over all 2^32 bit patterns: f2s and s2f are inverse bijections, and the
    decoded floats of increasing encoded words increase under the FPU's own
    IEEE-754 comparison (-0.0 just before +0.0, NaNs only beyond -inf and
    +inf).  The loop is C (tests/native/float_order_check.c) for speed."""
    lib = oracle.build(force=False)
    exe = str(tmp_path / "float_order_check")
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "float_order_check.c")
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-o", exe, src, lib, "-lm",
                           "-Wl,-rpath," + os.path.dirname(lib)])
    parts = 8
    step = (1 << 32) // parts
    procs = [subprocess.Popen([exe, "%x" % (i * step), "%x" % ((i + 1) * step)],
                              stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
             for i in range(parts)]
    outs = [p.communicate(timeout=300)[0] for p in procs]
    assert all(p.returncode == 0 for p in procs), outs
    # exactly one -0.0 -> +0.0 step over the whole walk
    assert sum(int(o.split("zero_steps=")[1].split()[0]) for o in outs) == 1
    # the inf words are the closed-form images of the inf patterns
    assert all("neg_inf_word=007fffff pos_inf_word=ff800000" in o for o in outs)


def test_float_transform_specials():
    """Ordering of the special values the configs and the pages mention."""
    tiny = np.finfo(np.float32).tiny
    den = np.float32(1e-45)
    vals = np.array([np.inf, -0.0, 0.0, -np.inf, den, -den, tiny, -tiny,
                     np.finfo(np.float32).max, -np.finfo(np.float32).max, 1.0, -1.0],
                    dtype=np.float32)
    got = oracle.sort_keys(vals)
    want = sorted(vals.tolist(), key=lambda x: (x, math.copysign(1.0, x)))
    assert got.view(np.uint32).tolist() == np.array(want, dtype=np.float32).view(np.uint32).tolist()
    # -0.0 strictly before +0.0
    zs = [i for i, x in enumerate(got.tolist()) if x == 0.0]
    assert math.copysign(1, got[zs[0]]) < 0 and math.copysign(1, got[zs[1]]) > 0


def test_nan_reading():
    """NaNs are not filtered: positive NaNs sort after +inf and negative NaNs
    before -inf, and their bit patterns come back unchanged."""
    pats = np.array([0x7FC00000, 0x7F800000, 0xFFC00000, 0xFF800000, 0x00000000,
                     0x7F800001, 0xFFFFFFFF], dtype=np.uint32)
    out = oracle.sort_keys(pats.view(np.float32)).view(np.uint32)
    assert out.tolist() == [0xFFFFFFFF, 0xFFC00000, 0xFF800000, 0x00000000,
                            0x7F800000, 0x7F800001, 0x7FC00000]


# ----------------------------------------------------------------- brute force

def _stable_ref(keys, fkey):
    """Python's sorted() is a stable comparison sort."""
    return sorted(range(len(keys)), key=lambda i: fkey(keys[i]))


def _bitfield(b, e):
    width = e - b
    return lambda k: (k >> b) & ((1 << width) - 1)


ALPHA_U32 = [0x00000000, 0x00000100, 0x01000001, 0xFFFFFFFF]
ALPHA_U32_HIGH = [0x00000005, 0xFFF00005, 0x000FFFFF, 0x80000000]
RANGES_U32 = [(0, 32), (0, 20), (8, 16), (3, 17), (0, 0), (31, 32), (24, 32), (16, 20)]


def _brute(alphabet, dtype, ranges, max_len):
    for length in range(0, max_len + 1):
        for seq in itertools.product(alphabet, repeat=length):
            keys = np.array(seq, dtype=dtype)
            pay = np.arange(length, dtype=np.uint32)
            for b, e in ranges:
                want = _stable_ref(list(seq), _bitfield(b, e))
                ko, vo = oracle.sort_pairs(keys, pay, b, e)
                assert vo.tolist() == want, (seq, b, e)
                assert ko.tolist() == [seq[i] for i in want]
                assert oracle.sort_keys(keys, b, e).tolist() == [seq[i] for i in want]


def test_bruteforce_u32():
    _brute(ALPHA_U32, np.uint32, RANGES_U32, 6)
    _brute(ALPHA_U32_HIGH, np.uint32, RANGES_U32, 5)


def test_bruteforce_u64():
    alpha = [0, 1 << 32, 0xFFFFFFFFFFFFFFFF, 0x0100000000000001]
    _brute(alpha, np.uint64, [(0, 64), (0, 40), (32, 64), (5, 61), (63, 64), (56, 64)], 5)


def test_bruteforce_f32_full_range():
    """Full-range float sort equals Python's stable sort by (value, sign of zero)."""
    alpha = [-0.0, 0.0, math.inf, -1.0, 1e-45]
    for length in range(0, 6):
        for seq in itertools.product(alpha, repeat=length):
            keys = np.array(seq, dtype=np.float32)
            fl = keys.tolist()
            want = _stable_ref(fl, lambda x: (x, math.copysign(1.0, x)))
            ko, vo = oracle.sort_pairs(keys, np.arange(length, dtype=np.uint32))
            assert vo.tolist() == want, seq
            assert ko.view(np.uint32).tolist() == keys.view(np.uint32)[want].tolist()


def test_f32_partial_range_composes():
    """A float sort over [b,e) is the uint32 sort of the encoded words over [b,e),
    decoded -- both pieces pinned above."""
    rng = np.random.default_rng(11)
    x = inputs.random_keys("f32", 5000, 12, "f32mix")
    for b, e in [(0, 20), (8, 16), (3, 17), (31, 32), (16, 32)]:
        pay = rng.permutation(5000).astype(np.uint32)
        ko, vo = oracle.sort_pairs(x, pay, b, e)
        ku, vu = oracle.sort_pairs(oracle.f2s(x.view(np.uint32)), pay, b, e)
        assert np.array_equal(vo, vu)
        assert np.array_equal(ko.view(np.uint32), oracle.s2f(ku))


# ---------------------------------------------------- signed and float64 keys

def _signed_field(bits, b, e):
    """Order field of a two's-complement value v: its rank among all values of
    that width is v + 2^(bits-1) (an offset, not the oracle's bit flip)."""
    mask = (1 << (e - b)) - 1
    return lambda v: (((v + (1 << (bits - 1))) % (1 << bits)) >> b) & mask


def _brute_signed(alphabet, dtype, bits, ranges, max_len):
    for length in range(0, max_len + 1):
        for seq in itertools.product(alphabet, repeat=length):
            keys = np.array(seq, dtype=dtype)
            pay = np.arange(length, dtype=np.uint32)
            for b, e in ranges:
                want = _stable_ref(list(seq), _signed_field(bits, b, e))
                ko, vo = oracle.sort_pairs(keys, pay, b, e)
                assert vo.tolist() == want, (seq, b, e)
                assert ko.tolist() == [seq[i] for i in want]


def test_bruteforce_i32():
    _brute_signed([-2**31, -1, 0, 2**31 - 1], np.int32, 32, RANGES_U32, 5)
    _brute_signed([-256, 255, 1, -2], np.int32, 32, RANGES_U32, 5)


def test_bruteforce_i64():
    ranges = [(0, 64), (0, 40), (32, 64), (5, 61), (63, 64), (56, 64)]
    _brute_signed([-2**63, -1, 0, 2**63 - 1], np.int64, 64, ranges, 5)
    _brute_signed([-(1 << 40), (1 << 40) - 1, 7, -8], np.int64, 64, ranges, 4)


@pytest.mark.parametrize("key_type", ["i32", "i64"])
@pytest.mark.parametrize("dist", ["uniform", "dup", "and3"])
def test_numpy_stable_argsort_signed(key_type, dist):
    """Full-range signed sorts equal numpy's stable argsort of the values."""
    keys = inputs.random_keys(key_type, 200_003, 9, dist)
    ko, vo = oracle.sort_pairs(keys, np.arange(keys.size, dtype=np.uint32))
    want = np.argsort(keys, kind="stable")
    assert np.array_equal(vo, want.astype(np.uint32))
    assert np.array_equal(ko, keys[want])
    assert np.array_equal(oracle.sort_keys(keys), np.sort(keys))


def test_bruteforce_f64_full_range():
    """Full-range float64 sort equals Python's stable sort by (value, sign of zero)."""
    alpha = [-0.0, 0.0, math.inf, -1.0, 5e-324]
    for length in range(0, 6):
        for seq in itertools.product(alpha, repeat=length):
            keys = np.array(seq, dtype=np.float64)
            want = _stable_ref(keys.tolist(), lambda x: (x, math.copysign(1.0, x)))
            ko, vo = oracle.sort_pairs(keys, np.arange(length, dtype=np.uint32))
            assert vo.tolist() == want, seq
            assert ko.view(np.uint64).tolist() == keys.view(np.uint64)[want].tolist()


def test_numpy_lexsort_f64():
    """Full-range float64 pair sort equals numpy's stable lexsort by
    (value, then -0.0 before +0.0)."""
    x = inputs.random_keys("f64", 300_001, 6, "fmix")
    ko, vo = oracle.sort_pairs(x, np.arange(x.size, dtype=np.uint32))
    want = np.lexsort((~np.signbit(x), x))
    assert np.array_equal(vo, want.astype(np.uint32))
    assert np.array_equal(ko.view(np.uint64), x.view(np.uint64)[want])


def test_f64_code_order_and_round_trip():
    """On random non-NaN doubles of every scale, the float64 code orders as the
    FPU compares (with -0.0 below +0.0); on random bit patterns, NaNs included,
    the inverse restores every pattern."""
    rng = np.random.default_rng(17)
    pats = rng.integers(0, 2**64, size=4000, dtype=np.uint64)
    for p in pats.tolist():
        assert oracle.f64_uncode(oracle.order_code(p, oracle.KIND_F64)) == p
    vals = pats.view(np.float64)
    vals = vals[~np.isnan(vals)]
    specials = np.array([0.0, -0.0, np.inf, -np.inf, 5e-324, -5e-324, 2.2250738585072014e-308,
                         -1.7976931348623157e308, 1.0, -1.0], dtype=np.float64)
    vals = np.concatenate([vals, specials])
    codes = oracle.order_codes(vals)
    a, b = rng.integers(0, vals.size, size=(2, 20000))
    for i, j in zip(a.tolist(), b.tolist()):
        x, y = float(vals[i]), float(vals[j])
        kx, ky = (x, math.copysign(1.0, x)), (y, math.copysign(1.0, y))
        assert (kx < ky) == (int(codes[i]) < int(codes[j])), (x, y)


def test_f64_nan_reading():
    """As for float32: positive NaNs after +inf, negative NaNs before -inf."""
    pats = np.array([0x7FF8000000000000, 0x7FF0000000000000, 0xFFF8000000000000,
                     0xFFF0000000000000, 0x0, 0x7FF0000000000001, 0xFFFFFFFFFFFFFFFF],
                    dtype=np.uint64)
    out = oracle.sort_keys(pats.view(np.float64)).view(np.uint64)
    assert out.tolist() == [0xFFFFFFFFFFFFFFFF, 0xFFF8000000000000, 0xFFF0000000000000, 0x0,
                            0x7FF0000000000000, 0x7FF0000000000001, 0x7FF8000000000000]


@pytest.mark.parametrize("key_type", ["i32", "i64", "f64"])
def test_partial_range_composes(key_type):
    """A sort over [b,e) of signed or float64 keys is the unsigned sort of their
    order words over [b,e), mapped back: both pieces are pinned above."""
    dist = "fmix" if key_type == "f64" else "dup"
    x = inputs.random_keys(key_type, 4000, 21, dist)
    bits = 8 * x.dtype.itemsize
    rng = np.random.default_rng(3)
    words = oracle.order_codes(x)
    if bits == 32:
        words = words.astype(np.uint32)
    for b, e in [(0, 20), (8, 16), (3, 17), (bits - 1, bits), (bits - 16, bits)]:
        pay = rng.permutation(x.size).astype(np.uint32)
        ko, vo = oracle.sort_pairs(x, pay, b, e)
        ku, vu = oracle.sort_pairs(words, pay, b, e)
        assert np.array_equal(vo, vu)
        kind = {"i32": oracle.KIND_I32, "i64": oracle.KIND_I64, "f64": oracle.KIND_F64}[key_type]
        back = [oracle.f64_uncode(int(w)) if key_type == "f64" else oracle.order_code(int(w), kind)
                for w in ku.tolist()]
        assert ko.view(words.dtype).tolist() == back


@pytest.mark.parametrize("key_type,widths", [("u32", (11, 11, 10)), ("u32", (8, 8, 8, 8)), ("u32", (3, 16, 13)),
                                             ("f32", (11, 11, 10)), ("u64", (11,) * 5 + (9,)),
                                             ("i64", (16, 16, 16, 16)), ("u32", (32,))])
def test_digit_width_does_not_change_the_result(key_type, widths):
    """Stable sorts by consecutive bit fields, least significant first, give the
    stable sort by the whole field whatever the widths: the reading under the
    11-bit digit option (three passes of 11, 11 and 10 bits for 32-bit keys)."""
    x = inputs.random_keys(key_type, 3000, 31, "dup" if key_type in ("u32", "i64") else "fmix" if key_type == "f32" else "uniform")
    pay = np.random.default_rng(8).permutation(x.size).astype(np.uint32)
    bits = sum(widths)
    assert bits == 8 * x.dtype.itemsize
    ko, vo = x, pay
    b = 0
    for w in widths:
        ko, vo = oracle.sort_pairs(ko, vo, b, b + w)
        b += w
    want_k, want_v = oracle.sort_pairs(x, pay, 0, bits)
    assert np.array_equal(vo, want_v)
    assert np.array_equal(ko.view(np.uint8), want_k.view(np.uint8))


# ------------------------------------------------------- library cross-check

@pytest.mark.parametrize("key_type,dist", [("u32", "uniform"), ("u32", "dup"), ("u32", "and3"),
                                           ("u64", "uniform"), ("u64", "dup"), ("u64", "and3")])
def test_numpy_stable_argsort(key_type, dist):
    keys = inputs.random_keys(key_type, 200_003, 7, dist)
    bits = 32 if key_type == "u32" else 64
    for b, e in [(0, bits), (0, 20), (8, 16), (3, 17), (bits - 1, bits), (5, 5)]:
        ko, vo = oracle.sort_pairs(keys, np.arange(keys.size, dtype=np.uint32), b, e)
        want = np.argsort(checks.order_field(keys, b, e), kind="stable")
        assert np.array_equal(vo, want.astype(np.uint32)), (b, e)
        assert np.array_equal(ko, keys[want])
        assert np.array_equal(oracle.sort_keys(keys, b, e), keys[want])


def test_numpy_lexsort_f32():
    """Full-range float32 pair sort equals numpy's stable lexsort by
    (value, then -0.0 before +0.0) -- an ordering defined without the encoding."""
    x = inputs.random_keys("f32", 300_001, 5, "f32mix")
    ko, vo = oracle.sort_pairs(x, np.arange(x.size, dtype=np.uint32))
    want = np.lexsort((~np.signbit(x), x))
    assert np.array_equal(vo, want.astype(np.uint32))
    assert np.array_equal(ko.view(np.uint32), x.view(np.uint32)[want])


# ----------------------------------------------------------- invariants, closed forms

@pytest.mark.parametrize("name", ["c1_u32_keys_64k", "c3a_u32_pairs_and3", "c4_f32_pairs_normal",
                                  "c5a_u64_pairs", "c5b_u32_pairs_20bit", "c5b_u32_keys_20bit"])
def test_config_shaped_invariants(name):
    cfg = inputs.CONFIGS[name]
    n = min(cfg.n, 300_000)
    _, keys, vals = inputs.draw(name, n)
    if vals is None:
        out = oracle.sort_keys(keys, cfg.begin_bit, cfg.end_bit)
        checks.check_multiset(keys, out)
        checks.check_sorted(out, cfg.begin_bit, cfg.end_bit)
        want = checks.expected_permutation(keys, cfg.begin_bit, cfg.end_bit)
        assert np.array_equal(checks.raw_bits(out), checks.raw_bits(keys)[want])
    else:
        ko, vo = oracle.sort_pairs(keys, vals, cfg.begin_bit, cfg.end_bit)
        checks.check_pairs(keys, ko, vo, cfg.begin_bit, cfg.end_bit)


@pytest.mark.parametrize("const", [0xDEADBEEF, 0])
def test_all_equal_is_identity(const):
    keys = np.full(100_000, const, dtype=np.uint32)
    ko, vo = oracle.sort_pairs(keys, np.arange(keys.size, dtype=np.uint32))
    assert np.array_equal(ko, keys) and np.array_equal(vo, np.arange(keys.size, dtype=np.uint32))


def test_sorted_input_is_identity_and_reverse_reverses():
    keys = np.arange(50_000, dtype=np.uint32) * 977
    ko, vo = oracle.sort_pairs(keys, np.arange(keys.size, dtype=np.uint32))
    assert np.array_equal(vo, np.arange(keys.size))
    ko, vo = oracle.sort_pairs(keys[::-1].copy(), np.arange(keys.size, dtype=np.uint32))
    assert np.array_equal(vo, np.arange(keys.size)[::-1])


def test_empty_and_single():
    for dt in (np.uint32, np.uint64, np.float32):
        assert oracle.sort_keys(np.zeros(0, dtype=dt)).size == 0
        one = np.array([7], dtype=dt)
        assert np.array_equal(oracle.sort_keys(one), one)


def test_zero_width_range_copies():
    keys = inputs.random_keys("u32", 1000, 3)
    ko, vo = oracle.sort_pairs(keys, np.arange(1000, dtype=np.uint32), 9, 9)
    assert np.array_equal(ko, keys) and np.array_equal(vo, np.arange(1000))


def test_input_not_modified():
    keys = inputs.random_keys("u64", 10_000, 9)
    copy = keys.copy()
    oracle.sort_keys(keys)
    assert np.array_equal(keys, copy)


def test_oracle_argument_checks():
    k = np.zeros(4, dtype=np.uint32)
    assert oracle.raw_sort(oracle.KIND_U32, k, None, 0, 33) != 0
    assert oracle.raw_sort(oracle.KIND_U32, k, None, 10, 9) != 0
    assert oracle.raw_sort(oracle.KIND_U32, k, None, -1, 8) != 0
    assert oracle.raw_sort(oracle.KIND_U32, k, None, 0, 32) == 0
    assert oracle.raw_sort(oracle.KIND_U64, np.zeros(4, dtype=np.uint64), None, 0, 64) == 0


# ------------------------------------------------------------ checker sanity

def test_checkers_catch_planted_mistakes():
    """Plant mistakes in a correct oracle result and check the checkers see them:
    two equal keys swapped (stability), a dropped element (permutation) and two
    unequal keys swapped (order)."""
    keys = inputs.random_keys("u32", 5000, 4, "dup")
    ko, vo = oracle.sort_pairs(keys, np.arange(keys.size, dtype=np.uint32))
    checks.check_pairs(keys, ko, vo, 0, 32)
    i = int(np.nonzero(ko[1:] == ko[:-1])[0][0])
    v2 = vo.copy(); v2[[i, i + 1]] = v2[[i + 1, i]]
    with pytest.raises(AssertionError):
        checks.check_pairs(keys, ko, v2, 0, 32)
    v3 = vo.copy(); v3[0] = v3[1]
    with pytest.raises(AssertionError):
        checks.check_pairs(keys, ko, v3, 0, 32)
    j = int(np.nonzero(ko[1:] != ko[:-1])[0][0])
    k4 = ko.copy(); v4 = vo.copy()
    k4[[j, j + 1]] = k4[[j + 1, j]]; v4[[j, j + 1]] = v4[[j + 1, j]]
    with pytest.raises(AssertionError):
        checks.check_pairs(keys, k4, v4, 0, 32)
