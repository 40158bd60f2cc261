"""Host-only checks of the C ABI (no GPU): the library loads, exports every
function the headers declare, answers temp-size queries and rejects bad
arguments before touching a device."""
from __future__ import annotations

import ctypes
import glob
import os
import re

import pytest

import sorting_lsd_radix_sort_amd as lrs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# fake, well-aligned device addresses: queries and argument errors never dereference them
A, B, C, D, T = 1 << 40, 2 << 40, 3 << 40, 4 << 40, 5 << 40


def header_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(lrs_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_loads_and_exports_header_symbols():
    lib = lrs.load_library()
    declared = header_functions()
    assert "lrs_sort_pairs_f64" in declared and len(declared) >= 18
    for name in declared:
        assert hasattr(lib, name), "missing export " + name
    assert set(declared) == set(lrs.EXPORTED)


def test_status_strings():
    for st in (lrs.LRS_OK, lrs.LRS_ERR_INVALID_ARG, lrs.LRS_ERR_TEMP_TOO_SMALL, lrs.LRS_ERR_HIP):
        assert lrs.status_string(st).startswith("LRS_")
    assert "unknown" in lrs.status_string(99)


def q_keys(sfx, n, b, e, kin=A, kout=B):
    return getattr(lrs, "lrs_sort_keys_" + sfx)(None, 0, kin, kout, n, b, e)


def q_pairs(sfx, n, b, e, kin=A, vin=C, kout=B, vout=D):
    return getattr(lrs, "lrs_sort_pairs_" + sfx)(None, 0, kin, vin, kout, vout, n, b, e)


@pytest.mark.parametrize("sfx,ksz,bits", [("u32", 4, 32), ("i32", 4, 32), ("f32", 4, 32),
                                          ("u64", 8, 64), ("i64", 8, 64), ("f64", 8, 64)])
def test_temp_query_sizes(sfx, ksz, bits):
    n = 100_000_000
    # out-of-place, >= 2 passes: one alternate key buffer plus a small count matrix
    t = q_keys(sfx, n, 0, bits)
    assert ksz * n <= t <= ksz * n + 8 * 2**20
    # one pass out-of-place needs no alternate buffer
    assert q_keys(sfx, n, 0, 8) <= 8 * 2**20
    # in-place with an even pass count: still one alternate buffer
    assert q_keys(sfx, n, 0, 16, kin=A, kout=A) == q_keys(sfx, n, 0, 16)
    # in-place with an odd pass count (>= 3): two alternate buffers
    t3 = q_keys(sfx, n, 0, 24, kin=A, kout=A)
    assert 2 * ksz * n <= t3 <= 2 * ksz * n + 8 * 2**20
    # in-place single pass: one alternate buffer (result copied back)
    t1 = q_keys(sfx, n, 0, 8, kin=A, kout=A)
    assert ksz * n <= t1 <= ksz * n + 8 * 2**20
    # pairs add an alternate value buffer
    tp = q_pairs(sfx, n, 0, bits)
    assert (ksz + 4) * n <= tp <= (ksz + 4) * n + 8 * 2**20
    # the count matrix is bounded, so temp grows linearly with n
    assert q_keys(sfx, 2 * n, 0, bits) - 2 * t <= 8 * 2**20


def test_temp_query_small_and_empty():
    assert q_keys("u32", 0, 0, 32) > 0            # always a usable non-zero size
    assert q_keys("u32", 1, 0, 32) < 64 * 1024
    assert q_keys("u32", 5, 3, 3) < 64 * 1024     # empty bit range: plain copy


@pytest.mark.parametrize("sfx,bits", [("u32", 32), ("i32", 32), ("f32", 32), ("u64", 64), ("i64", 64),
                                      ("f64", 64)])
def test_invalid_bit_ranges(sfx, bits):
    for b, e in [(-1, 8), (9, 8), (0, bits + 1), (bits + 1, bits + 1)]:
        with pytest.raises(lrs.LrsError) as ei:
            q_keys(sfx, 10, b, e)
        assert ei.value.status == lrs.LRS_ERR_INVALID_ARG
    q_keys(sfx, 10, bits, bits)  # empty range at the top is valid


def test_invalid_sizes_and_pointers():
    for n in (-1, 2**32, 2**40):
        with pytest.raises(lrs.LrsError) as ei:
            q_keys("u32", n, 0, 32)
        assert ei.value.status == lrs.LRS_ERR_INVALID_ARG
    q_keys("u32", 2**32 - 1, 0, 32)  # the largest n is accepted
    bad = [dict(kin=0), dict(kout=0), dict(kin=A + 2), dict(kout=B + 4 * 3 + 1),
           dict(kin=A, kout=A + 4)]   # partial overlap of input and output
    for kw in bad:
        with pytest.raises(lrs.LrsError) as ei:
            q_keys("u32", 1000, 0, 32, **kw)
        assert ei.value.status == lrs.LRS_ERR_INVALID_ARG, kw
    with pytest.raises(lrs.LrsError):
        q_keys("u64", 10, 0, 64, kin=A + 4)  # uint64 keys need 8-byte alignment
    for kw in (dict(vin=0), dict(vout=0), dict(vin=C + 1), dict(vin=C, vout=C + 8)):
        with pytest.raises(lrs.LrsError) as ei:
            q_pairs("u32", 1000, 0, 32, **kw)
        assert ei.value.status == lrs.LRS_ERR_INVALID_ARG, kw
    # NULL pointers are fine when there is nothing to sort
    assert q_keys("u32", 0, 0, 32, kin=0, kout=0) > 0


def test_temp_too_small_and_empty_input_touch_nothing():
    need = q_keys("u32", 1_000_000, 0, 32)
    # the query covers up to 255 bytes of padding to the first 256-byte
    # boundary: an aligned temp needs 255 bytes less, a temp one byte past a
    # boundary needs all of it
    for t, size in [(T, need - 256), (T + 1, need - 1)]:
        with pytest.raises(lrs.LrsError) as ei:
            lrs.lrs_sort_keys_u32(t, size, A, B, 1_000_000, 0, 32, 0)
        assert ei.value.status == lrs.LRS_ERR_TEMP_TOO_SMALL
    with pytest.raises(lrs.LrsError) as ei:
        lrs.lrs_sort_pairs_f32(T, 16, A, C, B, D, 1_000_000, 0, 32, 0)
    assert ei.value.status == lrs.LRS_ERR_TEMP_TOO_SMALL
    # n == 0 returns before any device work
    need0 = q_keys("u32", 0, 0, 32)
    assert lrs.lrs_sort_keys_u32(T, need0, A, B, 0, 0, 32, 0) == need0


def test_null_temp_bytes_pointer():
    lib = lrs.load_library()
    assert lib.lrs_sort_keys_u32(None, None, A, B, 10, 0, 32, None) == lrs.LRS_ERR_INVALID_ARG


def test_device_copy_and_prof_argument_checks():
    lib = lrs.load_library()
    assert lib.lrs_device_copy(None, ctypes.c_void_p(A), 16, None) == lrs.LRS_ERR_INVALID_ARG
    assert lib.lrs_device_copy(None, None, 0, None) == lrs.LRS_OK
    assert lib.lrs_prof_start(0) == lrs.LRS_ERR_INVALID_ARG
    assert lib.lrs_prof_count() == 0
    k, ms = ctypes.c_int(), ctypes.c_float()
    assert lib.lrs_prof_read(0, ctypes.byref(k), ctypes.byref(ms)) == lrs.LRS_ERR_INVALID_ARG
    assert lib.lrs_prof_release() == lrs.LRS_OK


def q_digits(sfx, digit_bits, n, b, e, kin=A, vin=None, kout=B, vout=None):
    return lrs.lrs_sort_digits(sfx, digit_bits, None, 0, kin, vin, kout, vout, n, b, e)


@pytest.mark.parametrize("sfx,ksz,bits", [("u32", 4, 32), ("f32", 4, 32), ("u64", 8, 64), ("i64", 8, 64)])
def test_digit_width_temp_queries(sfx, ksz, bits):
    n = 100_000_000
    # 8-bit digits through the generic call ask what the typed call asks
    assert q_digits(sfx, 8, n, 0, bits) == q_keys(sfx, n, 0, bits)
    assert q_digits(sfx, 8, n, 0, bits, vin=C, vout=D) == q_pairs(sfx, n, 0, bits)
    # 11-bit digits: the same alternate buffers plus a count matrix 8 times
    # larger (2048 rows, at most 4096 columns of 4 bytes)
    t11 = q_digits(sfx, 11, n, 0, bits)
    assert ksz * n <= t11 <= ksz * n + 40 * 2**20
    assert t11 > q_keys(sfx, n, 0, bits)
    # one 11-bit pass covers [0, 11): no alternate buffer out of place
    assert q_digits(sfx, 11, n, 0, 11) <= 40 * 2**20
    # ... and in place it goes through one alternate and is copied back
    assert q_digits(sfx, 11, n, 0, 11, kin=A, kout=A) >= ksz * n
    # in place, 3 passes (33 bits or fewer in 11-bit digits) need two alternates
    t3 = q_digits(sfx, 11, n, 0, 32, kin=A, kout=A)
    assert 2 * ksz * n <= t3 <= 2 * ksz * n + 40 * 2**20
    # ... where 8-bit digits over 32 bits (4 passes) need one
    assert q_keys(sfx, n, 0, 32, kin=A, kout=A) <= ksz * n + 8 * 2**20


def test_digit_width_argument_checks():
    lib = lrs.load_library()
    tb = ctypes.c_size_t(0)
    for bits in (0, 4, 7, 9, 10, 12, 16, -8):
        st = lib.lrs_sort_digits(0, bits, None, ctypes.byref(tb), A, None, B, None, 100, 0, 32, None)
        assert st == lrs.LRS_ERR_INVALID_ARG, bits
    for key_type in (-1, 6, 99):
        st = lib.lrs_sort_digits(key_type, 11, None, ctypes.byref(tb), A, None, B, None, 100, 0, 32, None)
        assert st == lrs.LRS_ERR_INVALID_ARG, key_type
    # one value pointer without the other
    for vin, vout in ((C, None), (None, D)):
        st = lib.lrs_sort_digits(0, 11, None, ctypes.byref(tb), A, vin, B, vout, 100, 0, 32, None)
        assert st == lrs.LRS_ERR_INVALID_ARG
    # the usual checks apply: bit range, alignment, NULL temp_bytes
    assert lib.lrs_sort_digits(0, 11, None, ctypes.byref(tb), A, None, B, None, 100, 0, 33, None) == \
        lrs.LRS_ERR_INVALID_ARG
    assert lib.lrs_sort_digits(3, 11, None, ctypes.byref(tb), A + 4, None, B, None, 100, 0, 64, None) == \
        lrs.LRS_ERR_INVALID_ARG
    assert lib.lrs_sort_digits(0, 11, None, None, A, None, B, None, 100, 0, 32, None) == lrs.LRS_ERR_INVALID_ARG
    # a too-small temp is refused before any device work
    need = q_digits("u32", 11, 1_000_000, 0, 32)
    st = lib.lrs_sort_digits(0, 11, ctypes.c_void_p(T + 1), ctypes.byref(ctypes.c_size_t(need - 1)), A, None, B,
                             None, 1_000_000, 0, 32, None)
    assert st == lrs.LRS_ERR_TEMP_TOO_SMALL


def test_missing_library_fails_loudly(monkeypatch):
    """Without the built HIP library the binding raises; there is no other path."""
    monkeypatch.setattr(lrs, "_lib", None)
    monkeypatch.setattr(lrs, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "liblrsort.so"))
    with pytest.raises(RuntimeError, match="not built"):
        lrs.load_library()
    with pytest.raises(RuntimeError, match="not built"):
        lrs.lrs_sort_keys_u32(None, 0, A, B, 10, 0, 32)
    with pytest.raises(RuntimeError, match="not built"):
        lrs.lrs_sort_digits("u32", 11, None, 0, A, None, B, None, 10, 0, 32)


def test_pass_routing_exhaustive(tmp_path):
    """The route every kernel derives from the skipped passes (kernels.hpp:
    pass_route, final_buffer, skipped_passes), checked on the host for every
    pass count up to 12, every set of skipped passes, in place or not:
    each pass reads where the data is, never writes the input or a buffer the
    host did not reserve, and the data ends in the output (tests/native/
    route_check.hip; compiled with hipcc, run on the CPU)."""
    import shutil
    import subprocess
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "route_check.hip")
    exe = str(tmp_path / "route_check")
    subprocess.check_call([hipcc, "-std=c++17", "-O1", "-o", exe, src], cwd=str(tmp_path),
                          stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert " 0 failures" in res.stdout


def test_convenience_calls_check_sizes_before_any_work():
    """sort_keys / sort_pairs reject outputs or values whose size, dtype or
    layout does not match the keys with ValueError, before touching the
    library (checked with CPU tensors: no device is needed to reach the
    checks, and none of them may be reached past)."""
    import torch
    k = torch.zeros(10, dtype=torch.uint32)
    v = torch.zeros(10, dtype=torch.uint32)
    with pytest.raises(ValueError, match="elements"):
        lrs.sort_keys(k, out=torch.zeros(9, dtype=torch.uint32))
    with pytest.raises(ValueError, match="dtype"):
        lrs.sort_keys(k, out=torch.zeros(10, dtype=torch.int32))
    with pytest.raises(ValueError, match="contiguous"):
        lrs.sort_keys(k, out=torch.zeros(20, dtype=torch.uint32)[::2])
    with pytest.raises(ValueError, match="elements"):
        lrs.sort_pairs(k, torch.zeros(9, dtype=torch.uint32))
    with pytest.raises(ValueError, match="elements"):
        lrs.sort_pairs(k, v, values_out=torch.zeros(11, dtype=torch.uint32))
    with pytest.raises(ValueError, match="elements"):
        lrs.sort_pairs(k, v, keys_out=torch.zeros(3, dtype=torch.uint32))
    with pytest.raises(ValueError, match="contiguous"):
        lrs.sort_pairs(k, v, values_out=torch.zeros(20, dtype=torch.uint32)[::2])
    # well-formed CPU tensors reach the device check and are refused there
    with pytest.raises(ValueError, match="device tensors"):
        lrs.sort_pairs(k, v)


def test_noalloc_rejects_sizes_beyond_its_scratch_before_device_work():
    """lrs_sort_digits_noalloc checks arguments and its size limit on the host
    (no device is touched: this runs without a GPU).  Pointers are never
    dereferenced by these checks."""
    lib = lrs.load_library()
    # aligned, far apart (no overlap between the arrays), never dereferenced here
    fake, kout, vin_p, vout_p = (ctypes.c_void_p(i << 40) for i in (1, 2, 3, 4))
    nul = ctypes.c_void_p(None)
    cap = lrs.NOALLOC_SCRATCH_BYTES
    # 32-bit keys alone: the alternate buffer is 4n bytes; 2^24 keys need 64 MiB + the count matrix
    for code, ksz, pairs, n in [(0, 4, False, 1 << 24), (0, 4, True, 1 << 23), (3, 8, True, 6 << 20),
                                (2, 4, False, (cap // 4) + 1)]:
        st = lib.lrs_sort_digits_noalloc(code, 8, fake, vin_p if pairs else nul, kout, vout_p if pairs else nul,
                                         n, 0, 8 * ksz, None)
        assert st == lrs.LRS_ERR_TOO_LARGE, (code, pairs, n, st)
    assert "scratch" in lrs.status_string(lrs.LRS_ERR_TOO_LARGE)
    # argument errors come first
    assert lib.lrs_sort_digits_noalloc(0, 9, fake, nul, fake, nul, 10, 0, 32, None) == lrs.LRS_ERR_INVALID_ARG
    assert lib.lrs_sort_digits_noalloc(0, 8, fake, nul, fake, nul, 10, 0, 33, None) == lrs.LRS_ERR_INVALID_ARG
    assert lib.lrs_sort_digits_noalloc(0, 8, nul, nul, fake, nul, 10, 0, 32, None) == lrs.LRS_ERR_INVALID_ARG
    assert lib.lrs_sort_digits_noalloc(9, 8, fake, nul, fake, nul, 10, 0, 32, None) == lrs.LRS_ERR_INVALID_ARG
    # nothing to do: no device call either
    assert lib.lrs_sort_digits_noalloc(0, 8, nul, nul, nul, nul, 0, 0, 32, None) == lrs.LRS_OK
