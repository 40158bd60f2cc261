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
]}

KEY_DTYPES = {"u32": np.uint32, "f32": np.float32, "u64": np.uint64}


def draw_keys(cfg: Config, n: int | None = None) -> np.ndarray:
    """Keys of ``cfg`` (length ``n``, default the config's own size)."""
    n = cfg.n if n is None else int(n)
    if cfg.dist == "equal":
        return np.full(n, cfg.const_key, dtype=KEY_DTYPES[cfg.key_type])
    rng = np.random.default_rng(cfg.seed)
    if cfg.dist == "uniform" and cfg.key_type == "u32":
        return rng.integers(0, 2**32, size=n, dtype=np.uint32)
    if cfg.dist == "uniform" and cfg.key_type == "u64":
        return rng.integers(0, 2**64, size=n, dtype=np.uint64)
    if cfg.dist == "uniform20":
        return rng.integers(0, 2**20, size=n, dtype=np.uint32)
    if cfg.dist == "and3":
        a = rng.integers(0, 2**32, size=n, dtype=np.uint32)
        a &= rng.integers(0, 2**32, size=n, dtype=np.uint32)
        a &= rng.integers(0, 2**32, size=n, dtype=np.uint32)
        return a
    if cfg.dist == "normal_zeros":
        x = rng.standard_normal(n).astype(np.float32)
        zero = rng.random(n) < 0.01
        negative = rng.random(n) < 0.5
        x[zero & negative] = np.float32(-0.0)
        x[zero & ~negative] = np.float32(0.0)
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
    """Ad-hoc seeded keys for edge-case tests: "uniform", "dup" (few distinct
    values, heavy duplicates), "and3" (skewed bits) or "f32mix" (floats with
    zeros of both signs, infinities and denormals mixed in)."""
    rng = np.random.default_rng(seed)
    dt = KEY_DTYPES[key_type]
    if dist == "uniform":
        if key_type == "f32":
            return rng.integers(0, 2**32, size=n, dtype=np.uint32).view(np.float32).copy()
        return rng.integers(0, 2**(8 * np.dtype(dt).itemsize), size=n, dtype=dt)
    if dist == "dup":
        if key_type == "f32":
            pool = np.concatenate([rng.standard_normal(5).astype(np.float32),
                                   np.array([0.0, -0.0], dtype=np.float32)])
        else:
            pool = rng.integers(0, 2**(8 * np.dtype(dt).itemsize), size=7, dtype=dt)
        return pool[rng.integers(0, len(pool), size=n)]
    if dist == "and3":
        bits = 8 * np.dtype(dt).itemsize
        udt = np.uint64 if bits == 64 else np.uint32
        a = rng.integers(0, 2**bits, size=n, dtype=udt)
        a &= rng.integers(0, 2**bits, size=n, dtype=udt)
        a &= rng.integers(0, 2**bits, size=n, dtype=udt)
        return a.view(np.float32).copy() if key_type == "f32" else a
    if dist == "f32mix":
        specials = np.array([0.0, -0.0, np.inf, -np.inf, 1.0, -1.0,
                             np.finfo(np.float32).tiny, -np.finfo(np.float32).tiny,
                             np.float32(1e-45), np.float32(-1e-45),
                             np.finfo(np.float32).max, -np.finfo(np.float32).max],
                            dtype=np.float32)
        x = rng.standard_normal(n).astype(np.float32)
        pick = rng.random(n) < 0.3
        x[pick] = specials[rng.integers(0, len(specials), size=int(pick.sum()))]
        return x
    raise ValueError(dist)
