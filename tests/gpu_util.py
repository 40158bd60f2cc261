"""Helpers for GPU tests: move numpy arrays through the lrsort C ABI on cuda:0."""
from __future__ import annotations

import sys

import numpy as np

import sorting_lsd_radix_sort_amd as lrs

SFX = {np.dtype(np.uint32): "u32", np.dtype(np.int32): "i32", np.dtype(np.float32): "f32",
       np.dtype(np.uint64): "u64", np.dtype(np.int64): "i64", np.dtype(np.float64): "f64"}
BITS = {dt: 8 * dt.itemsize for dt in SFX}


def announce(msg: str) -> None:
    """Names the case on stderr before any GPU step, flushed, so a run that
    ends abruptly still shows what it was doing."""
    sys.stderr.write("[gpu case] %s\n" % msg)
    sys.stderr.flush()


def to_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def to_host(t) -> np.ndarray:
    return t.cpu().numpy()


def gpu_sort(keys: np.ndarray, vals: np.ndarray | None, begin_bit: int, end_bit: int,
             in_place_keys: bool = False, in_place_vals: bool = False, stream=None,
             digit_bits: int | None = None):
    """Sorts through the lrs_sort_* entry point for the key dtype (through
    lrs_sort_digits with that digit width when digit_bits is given); returns
    numpy (keys, values-or-None).  Allocates temp with the two-phase query."""
    import torch
    sfx = SFX[keys.dtype]
    n = keys.size
    kin = to_dev(keys)
    kout = kin if in_place_keys else torch.empty_like(kin)
    if digit_bits is not None:
        vin = None if vals is None else to_dev(vals)
        vout = None if vals is None else (vin if in_place_vals else torch.empty_like(vin))
        need = lrs.lrs_sort_digits(sfx, digit_bits, None, 0, kin, vin, kout, vout, n, begin_bit, end_bit)
        temp = torch.empty(need, dtype=torch.uint8, device="cuda:0")
        lrs.lrs_sort_digits(sfx, digit_bits, temp, need, kin, vin, kout, vout, n, begin_bit, end_bit, stream)
        torch.cuda.synchronize()
        return to_host(kout), None if vals is None else to_host(vout)
    if vals is None:
        fn = getattr(lrs, "lrs_sort_keys_" + sfx)
        need = fn(None, 0, kin, kout, n, begin_bit, end_bit)
        temp = torch.empty(need, dtype=torch.uint8, device="cuda:0")
        fn(temp, need, kin, kout, n, begin_bit, end_bit, stream)
        torch.cuda.synchronize()
        return to_host(kout), None
    vin = to_dev(vals)
    vout = vin if in_place_vals else torch.empty_like(vin)
    fn = getattr(lrs, "lrs_sort_pairs_" + sfx)
    need = fn(None, 0, kin, vin, kout, vout, n, begin_bit, end_bit)
    temp = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    fn(temp, need, kin, vin, kout, vout, n, begin_bit, end_bit, stream)
    torch.cuda.synchronize()
    return to_host(kout), to_host(vout)
