"""lrsort: a stable LSD radix sort for AMD MI355X (gfx950).

Python binding of the C ABI in ``include/lrsort.h`` (ctypes).  Every function
named ``lrs_*`` here takes the same arguments as the C function of the same name
and only marshals them: device pointers may be given as ints or as torch device
tensors, the stream as an int handle, a ``torch.cuda.Stream`` or None (torch's
current stream).  All sorting work runs in the HIP kernels of ``liblrsort.so``;
there is no fallback, and a missing library raises.

``sort_keys`` / ``sort_pairs`` are conveniences over the same calls that
allocate outputs and temp storage as torch tensors.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "liblrsort.so")

LRS_OK = 0
LRS_ERR_INVALID_ARG = 1
LRS_ERR_TEMP_TOO_SMALL = 2
LRS_ERR_HIP = 3
LRS_ERR_TOO_LARGE = 4
NOALLOC_SCRATCH_BYTES = 64 << 20  # LRS_NOALLOC_SCRATCH_BYTES of include/lrsort.h

KERNEL_NAMES = {0: "upsweep", 1: "scan", 2: "downsweep", 3: "copy", 4: "finalize", 5: "tiny", 6: "small_pass"}

KEY_TYPES = ("u32", "i32", "f32", "u64", "i64", "f64")
SORT_FUNCTIONS = tuple("lrs_sort_keys_" + t for t in KEY_TYPES) + tuple("lrs_sort_pairs_" + t for t in KEY_TYPES)
# lrs_key_type codes of lrs_sort_digits
KEY_TYPE_CODES = {"u32": 0, "i32": 1, "f32": 2, "u64": 3, "i64": 4, "f64": 5}
DIGIT_BITS = (8, 11)
EXPORTED = SORT_FUNCTIONS + ("lrs_sort_digits", "lrs_status_string", "lrs_device_copy", "lrs_prof_start",
                             "lrs_prof_stop", "lrs_prof_count", "lrs_prof_read",
                             "lrs_prof_release", "lrs_bench_read", "lrs_sort_digits_noalloc")


class LrsError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s" % (where, status_string(status)))


_lib = None


def load_library() -> ctypes.CDLL:
    """Loads liblrsort.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("liblrsort.so is not built; run `python -m sorting_lsd_radix_sort_amd.build` "
                           "(or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i64, ci = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64, ctypes.c_int
    psz = ctypes.POINTER(ctypes.c_size_t)
    for name in SORT_FUNCTIONS:
        fn = getattr(lib, name)
        if "_pairs_" in name:
            fn.argtypes = [vp, psz, vp, vp, vp, vp, i64, ci, ci, vp]
        else:
            fn.argtypes = [vp, psz, vp, vp, i64, ci, ci, vp]
        fn.restype = ci
    lib.lrs_sort_digits.argtypes = [ci, ci, vp, psz, vp, vp, vp, vp, i64, ci, ci, vp]
    lib.lrs_sort_digits.restype = ci
    lib.lrs_sort_digits_noalloc.argtypes = [ci, ci, vp, vp, vp, vp, i64, ci, ci, vp]
    lib.lrs_sort_digits_noalloc.restype = ci
    lib.lrs_status_string.argtypes = [ci]
    lib.lrs_status_string.restype = ctypes.c_char_p
    lib.lrs_device_copy.argtypes = [vp, vp, sz, vp]
    lib.lrs_device_copy.restype = ci
    lib.lrs_prof_start.argtypes = [ci]
    lib.lrs_prof_start.restype = ci
    lib.lrs_prof_stop.argtypes = []
    lib.lrs_prof_stop.restype = ci
    lib.lrs_prof_count.argtypes = []
    lib.lrs_prof_count.restype = ci
    lib.lrs_prof_read.argtypes = [ci, ctypes.POINTER(ci), ctypes.POINTER(ctypes.c_float)]
    lib.lrs_prof_read.restype = ci
    lib.lrs_prof_release.argtypes = []
    lib.lrs_prof_release.restype = ci
    lib.lrs_bench_read.argtypes = [vp, sz, vp, vp]
    lib.lrs_bench_read.restype = ci
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().lrs_status_string(int(status)).decode()


def lrs_status_string(status: int) -> str:
    return status_string(status)


def _ptr(x) -> int | None:
    """Device pointer of an int, None, or a torch tensor (which must be on a GPU)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x or None
    if hasattr(x, "data_ptr"):
        if not x.is_cuda:
            raise ValueError("lrsort needs device tensors, got a tensor on %s" % x.device)
        return x.data_ptr()
    raise TypeError("cannot take a device pointer of %r" % type(x))


def _stream(s) -> int | None:
    if isinstance(s, int):
        return s or None
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream or None
    return s.cuda_stream or None


def _check(status: int, where: str) -> None:
    if status != LRS_OK:
        raise LrsError(status, where)


def _sort_call(name, d_temp, temp_bytes, arrays, n, begin_bit, end_bit, stream):
    lib = load_library()
    tb = ctypes.c_size_t(int(temp_bytes or 0))
    temp = _ptr(d_temp)
    st = None if temp is None else _stream(stream)
    status = getattr(lib, name)(temp, ctypes.byref(tb), *[_ptr(a) for a in arrays], int(n),
                                int(begin_bit), int(end_bit), st)
    _check(status, name)
    return tb.value


def _make_keys(name):
    def fn(d_temp, temp_bytes, d_keys_in, d_keys_out, n, begin_bit, end_bit, stream=None):
        """Calls the C function of the same name.  With d_temp None returns the
        temp bytes needed; otherwise enqueues the sort and returns temp_bytes.
        Raises LrsError on a non-OK status."""
        return _sort_call(name, d_temp, temp_bytes, (d_keys_in, d_keys_out), n, begin_bit, end_bit,
                          stream)
    fn.__name__ = name
    return fn


def _make_pairs(name):
    def fn(d_temp, temp_bytes, d_keys_in, d_values_in, d_keys_out, d_values_out, n, begin_bit,
           end_bit, stream=None):
        """Calls the C function of the same name (see the keys-only variants)."""
        return _sort_call(name, d_temp, temp_bytes, (d_keys_in, d_values_in, d_keys_out, d_values_out),
                          n, begin_bit, end_bit, stream)
    fn.__name__ = name
    return fn


lrs_sort_keys_u32 = _make_keys("lrs_sort_keys_u32")
lrs_sort_keys_i32 = _make_keys("lrs_sort_keys_i32")
lrs_sort_keys_f32 = _make_keys("lrs_sort_keys_f32")
lrs_sort_keys_u64 = _make_keys("lrs_sort_keys_u64")
lrs_sort_keys_i64 = _make_keys("lrs_sort_keys_i64")
lrs_sort_keys_f64 = _make_keys("lrs_sort_keys_f64")
lrs_sort_pairs_u32 = _make_pairs("lrs_sort_pairs_u32")
lrs_sort_pairs_i32 = _make_pairs("lrs_sort_pairs_i32")
lrs_sort_pairs_f32 = _make_pairs("lrs_sort_pairs_f32")
lrs_sort_pairs_u64 = _make_pairs("lrs_sort_pairs_u64")
lrs_sort_pairs_i64 = _make_pairs("lrs_sort_pairs_i64")
lrs_sort_pairs_f64 = _make_pairs("lrs_sort_pairs_f64")


def lrs_sort_digits(key_type, digit_bits, d_temp, temp_bytes, d_keys_in, d_values_in, d_keys_out,
                    d_values_out, n, begin_bit, end_bit, stream=None):
    """Calls the C function of the same name.  key_type is an lrs_key_type code
    or a suffix ("u32", ..., "f64"); the value arrays are both None for a
    keys-only sort.  With d_temp None returns the temp bytes needed."""
    lib = load_library()
    code = KEY_TYPE_CODES[key_type] if isinstance(key_type, str) else int(key_type)
    tb = ctypes.c_size_t(int(temp_bytes or 0))
    temp = _ptr(d_temp)
    st = None if temp is None else _stream(stream)
    status = lib.lrs_sort_digits(code, int(digit_bits), temp, ctypes.byref(tb), _ptr(d_keys_in),
                                 _ptr(d_values_in), _ptr(d_keys_out), _ptr(d_values_out), int(n),
                                 int(begin_bit), int(end_bit), st)
    _check(status, "lrs_sort_digits")
    return tb.value


def lrs_sort_digits_noalloc(key_type, digit_bits, d_keys_in, d_values_in, d_keys_out, d_values_out, n,
                            begin_bit, end_bit, stream=None) -> None:
    """Calls the C function of the same name: lrs_sort_digits with the
    library's static per-GPU scratch instead of temp storage (no allocation).
    Raises LrsError (status LRS_ERR_TOO_LARGE) for sorts beyond its size."""
    lib = load_library()
    code = KEY_TYPE_CODES[key_type] if isinstance(key_type, str) else int(key_type)
    status = lib.lrs_sort_digits_noalloc(code, int(digit_bits), _ptr(d_keys_in), _ptr(d_values_in),
                                         _ptr(d_keys_out), _ptr(d_values_out), int(n), int(begin_bit),
                                         int(end_bit), _stream(stream))
    _check(status, "lrs_sort_digits_noalloc")


def lrs_device_copy(d_dst, d_src, nbytes: int, stream=None) -> None:
    _check(load_library().lrs_device_copy(_ptr(d_dst), _ptr(d_src), int(nbytes), _stream(stream)),
           "lrs_device_copy")


# ---------------------------------------------------------------- profiling

def lrs_prof_start(capacity: int) -> None:
    _check(load_library().lrs_prof_start(int(capacity)), "lrs_prof_start")


def lrs_prof_stop() -> None:
    load_library().lrs_prof_stop()


def lrs_prof_count() -> int:
    return int(load_library().lrs_prof_count())


def lrs_prof_read(i: int) -> tuple[int, float]:
    kind = ctypes.c_int(0)
    ms = ctypes.c_float(0.0)
    _check(load_library().lrs_prof_read(int(i), ctypes.byref(kind), ctypes.byref(ms)), "lrs_prof_read")
    return kind.value, ms.value


def lrs_prof_release() -> None:
    load_library().lrs_prof_release()


def lrs_bench_read(d_src, nbytes: int, d_result, stream=None) -> None:
    _check(load_library().lrs_bench_read(_ptr(d_src), int(nbytes), _ptr(d_result), _stream(stream)),
           "lrs_bench_read")


# ------------------------------------------------------------- conveniences

_KEY_SUFFIX = {"torch.uint32": "u32", "torch.int32": "i32", "torch.float32": "f32",
               "torch.uint64": "u64", "torch.int64": "i64", "torch.float64": "f64"}
KEY_BITS = {"u32": 32, "i32": 32, "f32": 32, "u64": 64, "i64": 64, "f64": 64}


def key_suffix(dtype) -> str:
    try:
        return _KEY_SUFFIX[str(dtype)]
    except KeyError:
        raise TypeError("lrsort sorts keys of type uint32, int32, float32, uint64, int64 or "
                        "float64, not %s" % dtype) from None


def _temp_tensor(nbytes, device, temp):
    import torch
    if temp is not None and temp.numel() * temp.element_size() >= nbytes:
        return temp
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _side_stream(stream):
    """The torch stream a call is enqueued on when that is not torch's current
    stream (None otherwise): tensors the conveniences allocate, or copy into
    contiguous form, on the current stream are then recorded on it, so that
    the caching allocator does not hand their memory to other work while the
    sort still uses it."""
    import torch
    if stream is None:
        return None
    cur = torch.cuda.current_stream()
    handle = stream if isinstance(stream, int) else stream.cuda_stream
    if handle == cur.cuda_stream:
        return None
    return stream if not isinstance(stream, int) else torch.cuda.ExternalStream(handle)


def _keep_for(side, *tensors):
    if side is None:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(side)


def _check_out(name, t, n, dtype, device):
    """An output tensor must be contiguous with n elements of `dtype` on the
    input's device (checked before anything is enqueued)."""
    if t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if t.numel() != n:
        raise ValueError("%s holds %d elements, expected %d" % (name, t.numel(), n))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.device != device:
        raise ValueError("%s is on %s, the input on %s" % (name, t.device, device))


def sort_keys(keys, begin_bit: int = 0, end_bit: int | None = None, out=None, temp=None, stream=None,
              digit_bits: int = 8):
    """Stable ascending sort of a device tensor of keys (uint32, int32,
    float32, uint64, int64 or float64) over bits [begin_bit, end_bit) of their
    order code, in passes of `digit_bits` (8 or 11) bits; returns the output
    tensor.  A tensor of any shape is sorted as the flat array of its elements;
    `out`, when given, must be contiguous with as many elements, of the same
    dtype, on the same device (ValueError otherwise, before any work)."""
    import torch
    sfx = key_suffix(keys.dtype)
    end_bit = KEY_BITS[sfx] if end_bit is None else end_bit
    src = keys
    keys = keys.contiguous()
    n = keys.numel()
    if out is None:
        out = torch.empty_like(keys)
    else:
        _check_out("out", out, n, keys.dtype, keys.device)
    side = _side_stream(stream)
    if digit_bits != 8:
        need = lrs_sort_digits(sfx, digit_bits, None, 0, keys, None, out, None, n, begin_bit, end_bit)
        t = _temp_tensor(need, keys.device, temp)
        lrs_sort_digits(sfx, digit_bits, t, t.numel() * t.element_size(), keys, None, out, None, n,
                        begin_bit, end_bit, stream)
    else:
        fn = globals()["lrs_sort_keys_" + sfx]
        need = fn(None, 0, keys, out, n, begin_bit, end_bit)
        t = _temp_tensor(need, keys.device, temp)
        fn(t, t.numel() * t.element_size(), keys, out, n, begin_bit, end_bit, stream)
    _keep_for(side, t, out, keys if keys is not src else None)
    return out


def sort_pairs(keys, values, begin_bit: int = 0, end_bit: int | None = None, keys_out=None,
               values_out=None, temp=None, stream=None, digit_bits: int = 8):
    """Stable ascending pair sort (uint32 values) in passes of `digit_bits` (8
    or 11) bits; returns (keys_out, values_out).  `values` must hold as many
    elements as `keys`, and the outputs, when given, must be contiguous with
    that many elements of the inputs' dtypes on the same device (ValueError
    otherwise, before any work)."""
    import torch
    sfx = key_suffix(keys.dtype)
    if str(values.dtype) != "torch.uint32":
        raise TypeError("values must be uint32, not %s" % values.dtype)
    if values.numel() != keys.numel():
        raise ValueError("values hold %d elements, keys %d" % (values.numel(), keys.numel()))
    if values.device != keys.device:
        raise ValueError("values are on %s, keys on %s" % (values.device, keys.device))
    end_bit = KEY_BITS[sfx] if end_bit is None else end_bit
    ksrc, vsrc = keys, values
    keys = keys.contiguous()
    values = values.contiguous()
    n = keys.numel()
    if keys_out is None:
        keys_out = torch.empty_like(keys)
    else:
        _check_out("keys_out", keys_out, n, keys.dtype, keys.device)
    if values_out is None:
        values_out = torch.empty_like(values)
    else:
        _check_out("values_out", values_out, n, values.dtype, keys.device)
    side = _side_stream(stream)
    if digit_bits != 8:
        need = lrs_sort_digits(sfx, digit_bits, None, 0, keys, values, keys_out, values_out, n, begin_bit,
                               end_bit)
        t = _temp_tensor(need, keys.device, temp)
        lrs_sort_digits(sfx, digit_bits, t, t.numel() * t.element_size(), keys, values, keys_out,
                        values_out, n, begin_bit, end_bit, stream)
    else:
        fn = globals()["lrs_sort_pairs_" + sfx]
        need = fn(None, 0, keys, values, keys_out, values_out, n, begin_bit, end_bit)
        t = _temp_tensor(need, keys.device, temp)
        fn(t, t.numel() * t.element_size(), keys, values, keys_out, values_out, n, begin_bit, end_bit, stream)
    _keep_for(side, t, keys_out, values_out, keys if keys is not ksrc else None,
              values if values is not vsrc else None)
    return keys_out, values_out
