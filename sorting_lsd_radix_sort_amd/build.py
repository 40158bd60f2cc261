"""Builds the HIP library liblrsort.so in-tree for gfx950 with hipcc.

Run ``python -m sorting_lsd_radix_sort_amd.build``; ``__graft_entry__.build()``
calls :func:`build` too.  The library is one translation unit
(``csrc/lrsort.hip`` with the kernels of ``csrc/kernels.hpp``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "lrsort.hip")
DEPS = [SRC, os.path.join(PKG, "csrc", "kernels.hpp"),
        os.path.join(ROOT, "include", "lrsort.h"), os.path.join(ROOT, "include", "lrsort_prof.h")]
LIB = os.path.join(PKG, "liblrsort.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def command(out: str) -> list[str]:
    return [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
            "-fvisibility=hidden", "-Wall",
            # packed fp32 instructions stay off (the sort does no float math anyway)
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-o", out, SRC]


def build(verbose: bool = False) -> str:
    """Compiles liblrsort.so (always recompiles) and returns its path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(d) > t for d in DEPS)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
