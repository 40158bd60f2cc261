"""CPU oracle for the stable LSD radix sort -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library and its Python binding
never import it, and it imports nothing from them.

The arithmetic lives in ``lsd_oracle.c`` (plain C, one thread): the serial LSD
loop of the kwkr.cn essay on bitonic vs. LSD radix sort, section 3.1, with the
half-open bit range of the page "GPU radix sort: from the CUB implementation to
performance tuning", section 2, the float sign-flip encoding of the essay's
section 3.3 and the signed-integer sign flip of the page's section 5.2.  This module only builds that file with gcc and marshals numpy
arrays into it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lsd_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

KIND_U32, KIND_F32, KIND_U64, KIND_I32, KIND_I64, KIND_F64 = 0, 1, 2, 3, 4, 5
_KIND_OF_DTYPE = {np.dtype(np.uint32): KIND_U32, np.dtype(np.float32): KIND_F32,
                  np.dtype(np.uint64): KIND_U64, np.dtype(np.int32): KIND_I32,
                  np.dtype(np.int64): KIND_I64, np.dtype(np.float64): KIND_F64}
_KEY_BITS = {KIND_U32: 32, KIND_F32: 32, KIND_U64: 64, KIND_I32: 32, KIND_I64: 64, KIND_F64: 64}

_lib = None


def build(force: bool = True) -> str:
    """Compile lsd_oracle.c into liboracle.so with gcc (-O2, one thread)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-D_POSIX_C_SOURCE=199309L",
                               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.oracle_f2s.argtypes = [ctypes.c_uint32]
        lib.oracle_f2s.restype = ctypes.c_uint32
        lib.oracle_s2f.argtypes = [ctypes.c_uint32]
        lib.oracle_s2f.restype = ctypes.c_uint32
        for name, t in (("oracle_i32_code", ctypes.c_uint32), ("oracle_i64_code", ctypes.c_uint64),
                        ("oracle_f64_code", ctypes.c_uint64), ("oracle_f64_uncode", ctypes.c_uint64)):
            fn = getattr(lib, name)
            fn.argtypes = [t]
            fn.restype = t
        for name in ("oracle_f2s_array", "oracle_s2f_array"):
            fn = getattr(lib, name)
            fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
            fn.restype = None
        lib.oracle_code_array.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
        lib.oracle_code_array.restype = ctypes.c_int
        lib.oracle_sort.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                    ctypes.c_int, ctypes.c_int]
        lib.oracle_sort.restype = ctypes.c_int
        lib.oracle_time_sort.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p]
        lib.oracle_time_sort.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def f2s(bits) -> np.ndarray:
    """Float32 bit patterns (uint32 array) -> order-preserving uint32 words."""
    a = np.ascontiguousarray(bits, dtype=np.uint32)
    out = np.empty_like(a)
    _load().oracle_f2s_array(_ptr(a), _ptr(out), a.size)
    return out


def s2f(words) -> np.ndarray:
    """Inverse of :func:`f2s`: encoded uint32 words -> float32 bit patterns."""
    a = np.ascontiguousarray(words, dtype=np.uint32)
    out = np.empty_like(a)
    _load().oracle_s2f_array(_ptr(a), _ptr(out), a.size)
    return out


def order_code(bits, kind: int) -> int:
    """The oracle's order-preserving word of one key's bit pattern (an int)."""
    lib = _load()
    if kind == KIND_F32:
        return int(lib.oracle_f2s(int(bits)))
    if kind == KIND_I32:
        return int(lib.oracle_i32_code(int(bits)))
    if kind == KIND_I64:
        return int(lib.oracle_i64_code(int(bits)))
    if kind == KIND_F64:
        return int(lib.oracle_f64_code(int(bits)))
    return int(bits)


def order_codes(keys: np.ndarray) -> np.ndarray:
    """The oracle's order-preserving words of an array of keys, as uint64."""
    k = np.ascontiguousarray(keys).reshape(-1)
    kind = _KIND_OF_DTYPE.get(k.dtype)
    if kind is None:
        raise TypeError("no order code for %s" % k.dtype)
    out = np.empty(k.size, dtype=np.uint64)
    rc = _load().oracle_code_array(kind, _ptr(k), _ptr(out), k.size)
    if rc:
        raise ValueError("oracle_code_array failed with code %d" % rc)
    return out


def f64_uncode(word: int) -> int:
    """Inverse of the float64 order code (an int in, an int out)."""
    return int(_load().oracle_f64_uncode(int(word)))


def _prepare(keys, values, begin_bit, end_bit):
    keys = np.ascontiguousarray(keys)
    kind = _KIND_OF_DTYPE.get(keys.dtype)
    if kind is None:
        raise TypeError("oracle keys must be uint32, int32, float32, uint64, int64 or float64, "
                        "got %s" % keys.dtype)
    if end_bit is None:
        end_bit = _KEY_BITS[kind]
    if values is not None:
        values = np.ascontiguousarray(values, dtype=np.uint32)
        if values.shape != keys.shape:
            raise ValueError("values must have the same length as keys")
    return keys.reshape(-1), (None if values is None else values.reshape(-1)), kind, begin_bit, end_bit


def sort_keys(keys, begin_bit: int = 0, end_bit: int | None = None) -> np.ndarray:
    """Stable ascending sort of ``keys`` over bits [begin_bit, end_bit)."""
    k, _, kind, b, e = _prepare(keys, None, begin_bit, end_bit)
    out = np.empty_like(k)
    rc = _load().oracle_sort(kind, _ptr(k), None, _ptr(out), None, k.size, b, e)
    if rc:
        raise ValueError("oracle_sort failed with code %d" % rc)
    return out


def sort_pairs(keys, values, begin_bit: int = 0, end_bit: int | None = None):
    """Stable ascending sort of (key, value) pairs by key bits [begin_bit, end_bit)."""
    k, v, kind, b, e = _prepare(keys, values, begin_bit, end_bit)
    ko = np.empty_like(k)
    vo = np.empty_like(v)
    rc = _load().oracle_sort(kind, _ptr(k), _ptr(v), _ptr(ko), _ptr(vo), k.size, b, e)
    if rc:
        raise ValueError("oracle_sort failed with code %d" % rc)
    return ko, vo


def time_sort(keys, values=None, begin_bit: int = 0, end_bit: int | None = None,
              reps: int = 3) -> list[float]:
    """Wall time in seconds of each of ``reps`` oracle sorts (one host thread)."""
    k, v, kind, b, e = _prepare(keys, values, begin_bit, end_bit)
    ko = np.empty_like(k)
    vo = None if v is None else np.empty_like(v)
    times = np.zeros(reps, dtype=np.float64)
    rc = _load().oracle_time_sort(kind, _ptr(k), _ptr(v), _ptr(ko), _ptr(vo), k.size, b, e,
                                  reps, _ptr(times))
    if rc:
        raise ValueError("oracle_time_sort failed with code %d" % rc)
    return [float(t) for t in times]


def raw_sort(kind: int, keys, values, begin_bit: int, end_bit: int) -> int:
    """Calls the C entry point with caller-chosen arguments and returns its status
    code; used by tests of the oracle's own argument checks."""
    k = np.ascontiguousarray(keys)
    v = None if values is None else np.ascontiguousarray(values, dtype=np.uint32)
    ko = np.empty_like(k)
    vo = None if v is None else np.empty_like(v)
    return _load().oracle_sort(kind, _ptr(k), _ptr(v), _ptr(ko), _ptr(vo), k.size,
                               begin_bit, end_bit)
