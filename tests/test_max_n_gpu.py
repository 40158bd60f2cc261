"""The largest n the boundary accepts: 2^32 - 1 uint32 keys (16 GiB), keys only,
in 8- and 11-bit digits.  Every 32-bit index of the path is at its limit
(output positions up to 2^32 - 2, digit totals up to n), and the outputs take
the plain-store form of the downsweeps.

The input is drawn on the device from a seeded generator (no oracle can hold
it), and the output is checked there, chunk by chunk: ordered, including across
chunk boundaries, and the same multiset as the input by its count per top
byte, its sum and the sum of a mixing hash of every key (a lost, duplicated or
altered key changes them).
"""
from __future__ import annotations

import pytest

import sorting_lsd_radix_sort_amd as lrs
from gpu_util import announce

pytestmark = pytest.mark.gpu

N = (1 << 32) - 1
CHUNK = 1 << 28


def _draw(n):
    import torch
    g = torch.Generator(device="cuda:0")
    g.manual_seed(20)
    x = torch.empty(n, dtype=torch.int32, device="cuda:0")
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        x[s:e] = torch.randint(0, 1 << 32, (e - s,), dtype=torch.int64, device="cuda:0", generator=g).to(torch.int32)
    return x


def _summary(x):
    """(count per top byte, sum, sum of a mixing hash) of the keys as uint32."""
    import torch
    cnt = torch.zeros(256, dtype=torch.int64, device=x.device)
    s1 = s2 = 0
    for s in range(0, x.numel(), CHUNK):
        v = x[s:s + CHUNK].to(torch.int64) & 0xFFFFFFFF
        cnt += torch.bincount(v >> 24, minlength=256)
        s1 += int(v.sum().item())
        h = ((v ^ (v >> 16)) * 0x45D9F3B) & 0xFFFFFFFF
        s2 += int(((h ^ (h >> 13)) & 0xFFFFFFFF).sum().item())
    return cnt.cpu(), s1, s2


def _ordered(x):
    import torch
    prev = None
    for s in range(0, x.numel(), CHUNK):
        v = x[s:s + CHUNK].to(torch.int64) & 0xFFFFFFFF
        if not bool((v[1:] >= v[:-1]).all().item()):
            return False
        if prev is not None and prev > int(v[0].item()):
            return False
        prev = int(v[-1].item())
    return True


@pytest.mark.parametrize("digit_bits", [8, 11])
def test_largest_n_uint32_keys(digit_bits):
    import torch
    announce("largest n: %d uint32 keys, %d-bit digits" % (N, digit_bits))
    try:
        kin = _draw(N)
        want = _summary(kin)
        kout = torch.empty_like(kin)
        need = lrs.lrs_sort_digits("u32", digit_bits, None, 0, kin, None, kout, None, N, 0, 32)
        temp = torch.empty(need, dtype=torch.uint8, device="cuda:0")
        lrs.lrs_sort_digits("u32", digit_bits, temp, need, kin, None, kout, None, N, 0, 32)
        torch.cuda.synchronize()
        del temp
        assert _ordered(kout), "output not ordered"
        got = _summary(kout)
        assert torch.equal(got[0], want[0]), "count per top byte differs"
        assert got[1] == want[1] and got[2] == want[2], "output keys are not a permutation of the input keys"
    finally:
        kin = kout = temp = None
        torch.cuda.empty_cache()  # 48 GB: not kept from the tests that follow


def test_uint64_keys_past_2gib():
    """64-bit keys alone, 2^28 + 5 of them (2 GiB + 40 bytes): the plain-store
    form of the register-carry downsweep without values, in 8- and 11-bit
    digits, checked on the device as above (ordered as unsigned words, same
    count per top byte, sum and hash sum)."""
    import torch
    n = (1 << 28) + 5
    sign = -(1 << 63)
    g = torch.Generator(device="cuda:0")
    g.manual_seed(21)
    hi = torch.randint(0, 1 << 32, (n,), dtype=torch.int64, device="cuda:0", generator=g)
    lo = torch.randint(0, 1 << 32, (n,), dtype=torch.int64, device="cuda:0", generator=g)
    kin = (hi << 32) | lo
    del hi, lo

    def summary(x):
        top = ((x >> 56) & 0xFF)
        mixed = (x ^ (x >> 29)) * 0x3C79AC492BA7B653  # wraps mod 2^64
        return torch.bincount(top, minlength=256).cpu(), int((x & 0xFFFFFFFF).sum().item()), \
            int(((x >> 32) & 0xFFFFFFFF).sum().item()), int((mixed >> 8).sum().item())

    want = summary(kin)
    for digit_bits in (8, 11):
        announce("uint64 keys past 2 GiB: n=%d, %d-bit digits" % (n, digit_bits))
        try:
            kout = torch.empty_like(kin)
            need = lrs.lrs_sort_digits("u64", digit_bits, None, 0, kin, None, kout, None, n, 0, 64)
            temp = torch.empty(need, dtype=torch.uint8, device="cuda:0")
            lrs.lrs_sort_digits("u64", digit_bits, temp, need, kin, None, kout, None, n, 0, 64)
            torch.cuda.synchronize()
            del temp
            signed = kout ^ sign  # unsigned order as signed order
            assert bool((signed[1:] >= signed[:-1]).all().item()), "output not ordered"
            del signed
            got = summary(kout)
            assert torch.equal(got[0], want[0]) and got[1:] == want[1:], \
                "output keys are not a permutation of the input keys"
        finally:
            kout = temp = None
            torch.cuda.empty_cache()
