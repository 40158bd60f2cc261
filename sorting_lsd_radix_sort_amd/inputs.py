"""Seeded synthetic inputs for the stable LSD radix sort.

This module only draws random numbers; it holds no sorting arithmetic, so both
the GPU path's tests and benchmark and the CPU oracle can be fed from it.

The workloads restate the pages' inputs -- "randomly generated uint32" in the
kwkr.cn essay's timing table (section 4) and "random 32-bit integers" in the
quant67.com survey's test setup (section 9.1) -- plus the skewed, float, 64-bit
and partial-bit-range variants the sort must handle.  No public dataset is used.
Every array comes from ``numpy.random.default_rng(seed)`` (PCG64) on the host.

Each config can also be drawn at a smaller ``n`` with the same seed and
distribution, for parity runs the oracle finishes in seconds.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Config:
    name: str
    key_type: str          # "u32", "f32" or "u64"
    n: int
    seed: int | None
    dist: str              # "uniform", "and3", "equal", "normal_zeros", "uniform20"
    pairs: bool
    begin_bit: int
    end_bit: int
    const_key: int = 0     # for dist == "equal"
    description: str = ""


CONFIGS: dict[str, Config] = {c.name: c for c in [
    Config("c1_u32_keys_64k", "u32", 65_536, 0, "uniform", False, 0, 32,
           description="65,536 uint32 keys uniform on [0, 2^32), seed 0, keys only, bits [0,32)"),
    Config("c2_u32_keys_1e8", "u32", 100_000_000, 1, "uniform", False, 0, 32,
           description="1e8 uint32 keys uniform on [0, 2^32), seed 1, keys only, bits [0,32)"),
    Config("c3a_u32_pairs_and3", "u32", 1 << 27, 2, "and3", True, 0, 32,
           description="2^27 uint32 keys, each the AND of three uniform words (seed 2), "
                       "uint32 index payload"),
    Config("c3b_u32_pairs_equal", "u32", 1 << 27, None, "equal", True, 0, 32, const_key=0xDEADBEEF,
           description="2^27 uint32 keys all equal to 0xDEADBEEF, uint32 index payload"),
    Config("c3b0_u32_pairs_zero", "u32", 1 << 27, None, "equal", True, 0, 32, const_key=0,
           description="2^27 uint32 keys all equal to 0, uint32 index payload"),
    Config("c4_f32_pairs_normal", "f32", 1 << 27, 3, "normal_zeros", True, 0, 32,
           description="2^27 float32 keys from N(0,1) (seed 3) with ~1% exact +-0.0, "
                       "uint32 index payload"),
    Config("c5a_u64_pairs", "u64", 1 << 26, 4, "uniform", True, 0, 64,
           description="2^26 uint64 keys uniform on [0, 2^64), seed 4, uint32 index payload"),
    Config("c5b_u32_pairs_20bit", "u32", 1 << 26, 5, "uniform20", True, 0, 20,
           description="2^26 uint32 keys uniform on [0, 2^20), seed 5, bits [0,20), "
                       "uint32 index payload"),
    Config("c5b_u32_keys_20bit", "u32", 1 << 26, 5, "uniform20", False, 0, 20,
           description="2^26 uint32 keys uniform on [0, 2^20), seed 5, bits [0,20), keys only"),
    # other key types through the same kernels (signed integers, float64)
    Config("f1_i32_keys_1e8", "i32", 100_000_000, 6, "uniform", False, 0, 32,
           description="1e8 int32 keys, uniform bit patterns (seed 6), keys only, bits [0,32)"),
    Config("f1_i64_pairs", "i64", 1 << 26, 8, "uniform", True, 0, 64,
           description="2^26 int64 keys, uniform bit patterns (seed 8), uint32 index payload"),
    Config("f1_f64_pairs_normal", "f64", 1 << 26, 7, "normal_zeros", True, 0, 64,
           description="2^26 float64 keys from N(0,1) (seed 7) with ~1% exact +-0.0, "
                       "uint32 index payload"),
]}

KEY_DTYPES = {"u32": np.uint32, "i32": np.int32, "f32": np.float32,
              "u64": np.uint64, "i64": np.int64, "f64": np.float64}
_BITS_DTYPE = {4: np.uint32, 8: np.uint64}


def draw_keys(cfg: Config, n: int | None = None) -> np.ndarray:
    """Keys of ``cfg`` (length ``n``, default the config's own size)."""
    n = cfg.n if n is None else int(n)
    if cfg.dist == "equal":
        return np.full(n, cfg.const_key, dtype=KEY_DTYPES[cfg.key_type])
    rng = np.random.default_rng(cfg.seed)
    if cfg.dist == "uniform":
        dt = np.dtype(KEY_DTYPES[cfg.key_type])
        return rng.integers(0, 2**(8 * dt.itemsize), size=n, dtype=_BITS_DTYPE[dt.itemsize]).view(dt)
    if cfg.dist == "uniform20":
        return rng.integers(0, 2**20, size=n, dtype=np.uint32)
    if cfg.dist == "and3":
        a = rng.integers(0, 2**32, size=n, dtype=np.uint32)
        a &= rng.integers(0, 2**32, size=n, dtype=np.uint32)
        a &= rng.integers(0, 2**32, size=n, dtype=np.uint32)
        return a
    if cfg.dist == "normal_zeros":
        dt = KEY_DTYPES[cfg.key_type]
        x = rng.standard_normal(n).astype(dt)
        zero = rng.random(n) < 0.01
        negative = rng.random(n) < 0.5
        x[zero & negative] = dt(-0.0)
        x[zero & ~negative] = dt(0.0)
        assert not np.isnan(x).any()
        return x
    raise ValueError("no generator for %s/%s" % (cfg.dist, cfg.key_type))


def draw_values(cfg: Config, n: int | None = None) -> np.ndarray | None:
    """The uint32 payload of ``cfg``: the original index 0..n-1 (None for keys only)."""
    n = cfg.n if n is None else int(n)
    return np.arange(n, dtype=np.uint32) if cfg.pairs else None


def draw(name: str, n: int | None = None):
    """(config, keys, values-or-None) for the named config."""
    cfg = CONFIGS[name]
    return cfg, draw_keys(cfg, n), draw_values(cfg, n)


def random_keys(key_type: str, n: int, seed: int, dist: str = "uniform") -> np.ndarray:
    """Ad-hoc seeded keys for edge-case tests, of any key type: "uniform"
    (uniform bit patterns), "dup" (few distinct values, heavy duplicates),
    "and3" (skewed bits: the AND of three uniform words) or "fmix" / "f32mix"
    (floats from N(0,1) with zeros of both signs, infinities, denormals and the
    extremes mixed in)."""
    rng = np.random.default_rng(seed)
    dt = np.dtype(KEY_DTYPES[key_type])
    udt = _BITS_DTYPE[dt.itemsize]
    bits = 8 * dt.itemsize
    if dist == "uniform":
        return rng.integers(0, 2**bits, size=n, dtype=udt).view(dt).copy()
    if dist == "dup":
        if dt.kind == "f":
            pool = np.concatenate([rng.standard_normal(5).astype(dt), np.array([0.0, -0.0], dtype=dt)])
        else:
            pool = rng.integers(0, 2**bits, size=7, dtype=udt).view(dt)
        return pool[rng.integers(0, len(pool), size=n)]
    if dist == "and3":
        a = rng.integers(0, 2**bits, size=n, dtype=udt)
        a &= rng.integers(0, 2**bits, size=n, dtype=udt)
        a &= rng.integers(0, 2**bits, size=n, dtype=udt)
        return a.view(dt).copy()
    if dist in ("fmix", "f32mix"):
        if dt.kind != "f":
            raise ValueError("fmix is for float keys")
        fi = np.finfo(dt)
        den = fi.smallest_subnormal
        specials = np.array([0.0, -0.0, np.inf, -np.inf, 1.0, -1.0, fi.tiny, -fi.tiny,
                             den, -den, fi.max, -fi.max], dtype=dt)
        x = rng.standard_normal(n).astype(dt)
        pick = rng.random(n) < 0.3
        x[pick] = specials[rng.integers(0, len(specials), size=int(pick.sum()))]
        return x
    raise ValueError(dist)
