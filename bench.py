#!/usr/bin/env python3
"""Benchmark of the stable LSD radix sort on one MI355X.

One step = one whole sort call (every pass: upsweep, scan, downsweep) of the
workload's input, already resident in HBM, into a preallocated output with
preallocated temp storage.  Default workload: 1e8 uint32 keys drawn uniformly
from [0, 2^32) with seed 1, keys only, bits [0, 32), 4 passes of 8-bit digits
(--digit-bits 11: the same sort in 3 passes of 11-bit digits).

Prints one JSON line with the throughput (Gkeys/s), the dominant kernel's
roofline figures (from HIP events around each launch, on the launch stream)
and the CPU oracle timed on a bounded sample of the same input.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published peak
PAGES_GPU_GKEYS = 6.25         # 1e8 32-bit ints in ~16 ms (quant67.com survey, sections 9.3-9.4)


def log(msg: str) -> None:
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def kernel_source_digest() -> str:
    """Digest of the library's source code with comments and blank space
    removed: a change to the kernels changes it, a change to their comments
    does not."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in ("sorting_lsd_radix_sort_amd/csrc/kernels.hpp", "sorting_lsd_radix_sort_amd/csrc/lrsort.hip"):
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, digit_bits: int, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary of this workload (profiles/<workload>[_d11]_traffic.txt), if it was
    taken with the current kernel source; None otherwise."""
    path = os.path.join(ROOT, "profiles", "%s%s_traffic.txt" % (workload, "_d11" if digit_bits == 11 else ""))
    try:
        fields = {}
        with open(path) as f:
            for ln in f:
                if ":" in ln and not ln.startswith("#"):
                    k, v = ln.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("kernel_source_digest") != kernel_source_digest():
            return None
        if fields.get("workload") != workload or int(fields.get("digit_bits", "0")) != digit_bits:
            return None
        return float(fields["traffic." + kernel])
    except (OSError, KeyError, ValueError):
        return None


def order_field(t, key_type: str, begin_bit: int, end_bit: int):
    """int64 tensor whose signed order is the order of the sort's field: bits
    [begin_bit, end_bit) of each key's order code (unsigned keys: the key;
    signed: sign bit flipped; floats: sign bit set when clear, every bit
    inverted when set).  Computed with torch on the device, independently of
    the library."""
    import torch
    width = 64 if key_type in ("u64", "i64", "f64") else 32
    if width == 32:
        b = t.view(torch.int32).to(torch.int64) & 0xFFFFFFFF
        if key_type == "i32":
            b = b ^ 0x80000000
        elif key_type == "f32":
            neg = (b >> 31) == 1
            b = torch.where(neg, b ^ 0xFFFFFFFF, b ^ 0x80000000)
        code_signed = b  # below 2^32: signed order is unsigned order
    else:
        b = t.view(torch.int64)
        sign = torch.iinfo(torch.int64).min  # bit 63
        if key_type == "u64":
            code = b
        elif key_type == "i64":
            code = b ^ sign
        else:
            code = torch.where(b < 0, ~b, b ^ sign)
        code_signed = code ^ sign  # unsigned order of the code as signed order
        if begin_bit == 0 and end_bit == 64:
            return code_signed
        b = code
    if begin_bit == 0 and end_bit == width:
        return code_signed
    field = (b >> begin_bit) if begin_bit < 64 else torch.zeros_like(b)
    if end_bit - begin_bit < 64:
        field = field & ((1 << (end_bit - begin_bit)) - 1)
    return field


def check_exact(kin, vin, kout, vout, key_type: str, begin_bit: int, end_bit: int) -> bool:
    """The output equals the unique stable sort of the input by its field,
    bit for bit, keys and values: torch's stable sort of the order field gives
    the permutation; the expected arrays are the inputs gathered by it."""
    import torch
    _, idx = torch.sort(order_field(kin, key_type, begin_bit, end_bit), stable=True)
    ok = bool(torch.equal(bits(kin)[idx], bits(kout)))
    if vin is not None:
        ok = ok and bool(torch.equal(bits(vin)[idx], bits(vout)))
    del idx
    return ok


def bits(t):
    """The tensor's bit patterns as signed integers of the same width (exact
    comparisons: float -0.0 and +0.0 differ, NaNs compare by pattern)."""
    import torch
    return t.view(torch.int64 if t.element_size() == 8 else torch.int32)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5,
                    help="untimed sorts before the timed ones, after the first sort and its output check")
    ap.add_argument("--config", default="c2_u32_keys_1e8")
    ap.add_argument("--cpu-sample", type=int, default=0,
                    help="keys of the input the CPU oracle sorts for the baseline (0: all of them)")
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ref-reps", type=int, default=400,
                    help="launches of each streaming reference (copy, read) timed before the warmup")
    ap.add_argument("--digit-bits", type=int, default=8, choices=(8, 11),
                    help="digit width of the passes (11: lrs_sort_digits with 2048-digit passes)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        log("bench.py measures one GPU only: this sort runs on a single MI355X and has no "
            "multi-GPU path (requested --gpus %d)." % args.gpus)
        return 2

    import numpy as np
    import torch

    import sorting_lsd_radix_sort_amd as lrs
    from sorting_lsd_radix_sort_amd import inputs

    cfg = inputs.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("[bench] drawing %s (n=%d)" % (cfg.name, cfg.n))
    keys_np = inputs.draw_keys(cfg)
    vals_np = inputs.draw_values(cfg)
    n = keys_np.size
    ksz = keys_np.dtype.itemsize
    vsz = 4 if vals_np is not None else 0
    db = args.digit_bits
    passes = (cfg.end_bit - cfg.begin_bit + db - 1) // db

    kin = torch.from_numpy(keys_np).to(dev)
    kout = torch.empty_like(kin)
    vin = torch.from_numpy(vals_np).to(dev) if vals_np is not None else None
    vout = torch.empty_like(vin) if vin is not None else None
    sfx = cfg.key_type
    if db != 8:
        def fn(d_temp, temp_bytes, *rest):
            ki, vi, ko, vo = rest[0], rest[1], rest[2], rest[3]
            return lrs.lrs_sort_digits(sfx, db, d_temp, temp_bytes, ki, vi, ko, vo, *rest[4:])
        arrays = (kin, vin, kout, vout)
    elif vin is None:
        fn = getattr(lrs, "lrs_sort_keys_" + sfx)
        arrays = (kin, kout)
    else:
        fn = getattr(lrs, "lrs_sort_pairs_" + sfx)
        arrays = (kin, vin, kout, vout)
    temp_bytes = fn(None, 0, *arrays, n, cfg.begin_bit, cfg.end_bit)
    temp = torch.empty(temp_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        fn(temp, temp_bytes, *arrays, n, cfg.begin_bit, cfg.end_bit, stream)

    # The first sort (its first call on the device also looks up the device's
    # properties) and an exact check of its output, before the warmup and the
    # timed region; the check's temporaries are released before timing.
    log("[bench] first sort and exact output check")
    step()
    torch.cuda.synchronize()
    exact = check_exact(kin, vin, kout, vout, cfg.key_type, cfg.begin_bit, cfg.end_bit)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log("[bench] output equals the stable sort of the input: %s" % exact)
    first_out_k = kout.clone()
    first_out_v = vout.clone() if vout is not None else None

    # ---- streaming references on the key array: the library's tuned device
    # copy (read + write) and read-only kernel, same stream, same size.  Taken
    # before the sorts' warmup: their ~100 ms of back-to-back kernels also bring
    # the GPU out of its idle clock state (kernels run ~10 % slower for the first
    # ~20 ms after an idle spell), so the warmup sorts start at working clocks.
    ref_reps = max(1, args.ref_reps)

    def time_ref(fn):
        ev2 = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for _ in range(2):
            fn()
        ev2[0].record(stream)
        for _ in range(ref_reps):
            fn()
        ev2[1].record(stream)
        torch.cuda.synchronize()
        return ev2[0].elapsed_time(ev2[1]) / ref_reps

    log("[bench] streaming references (%d copies, %d reads)" % (ref_reps, ref_reps))
    scratch = torch.empty_like(kin)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    copy_ms = time_ref(lambda: lrs.lrs_device_copy(scratch, kin, n * ksz, stream))
    copy_gbs = 2 * n * ksz / (copy_ms * 1e-3) / 1e9
    read_ms = time_ref(lambda: lrs.lrs_bench_read(kin, n * ksz, sink, stream))
    read_gbs = n * ksz / (read_ms * 1e-3) / 1e9
    del scratch


    log("[bench] warmup %d" % args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps back to back, one event on the launch
    # stream before and one after (no event between steps: on small sorts an
    # event between launches costs a noticeable part of a step)
    log("[bench] timing %d steps" % args.steps)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
    ev[1].record(stream)
    torch.cuda.synchronize()
    total_ms = ev[0].elapsed_time(ev[1])
    ms_per_step = total_ms / args.steps
    gkeys = n / (ms_per_step * 1e-3) / 1e9

    # ---- the spread of single steps: the same K steps again, an event after each
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]

    # ---- per-kernel durations: same K steps again with events around each launch.
    # Taken before the output check: the check's temporaries (several times the
    # input's size, kept in torch's allocator cache) measurably slow the sort's
    # kernels that run after them.
    log("[bench] per-kernel events over %d steps" % args.steps)
    lrs.lrs_prof_start(args.steps * (3 * passes + 1) + 16)  # (+ a copy launch for in-place sorts)
    try:
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        lrs.lrs_prof_stop()
        recs = [lrs.lrs_prof_read(i) for i in range(lrs.lrs_prof_count())]
    finally:
        lrs.lrs_prof_release()
    by_kind = {}
    for kind, ms in recs:
        by_kind.setdefault(lrs.KERNEL_NAMES[kind], []).append(ms)
    avg = {k: sum(v) / len(v) for k, v in by_kind.items()}
    launches = {k: len(v) for k, v in by_kind.items()}

    # the output of the last timed sort is the same as the first's
    same_again = bool(torch.equal(bits(kout), bits(first_out_k))) and (
        vout is None or bool(torch.equal(bits(vout), bits(first_out_v))))
    del first_out_k, first_out_v
    torch.cuda.empty_cache()
    log("[bench] output of the last sort equals the first's: %s" % same_again)

    # algorithmic bytes per launch: the upsweep reads K*n; the downsweep reads
    # and writes (K+V)*n; a small sort's one-launch pass does a whole pass,
    # (3K+2V)*n (its repeated counting reads hit L2, not HBM); the one-workgroup
    # sort reads and writes the data once, 2(K+V)*n.  The whole sort moves
    # P*(3K+2V)*n (strict reading P*(2K+2V)*n).
    per_launch = {"downsweep": 2 * (ksz + vsz) * n, "upsweep": ksz * n,
                  "small_pass": (3 * ksz + 2 * vsz) * n, "tiny": 2 * (ksz + vsz) * n}
    dominant = max((k for k in by_kind if k in per_launch), key=lambda k: sum(by_kind[k]))
    down_bytes = per_launch[dominant]
    achieved = down_bytes / (avg[dominant] * 1e-3) / 1e9
    sort_bytes = passes * (3 * ksz + 2 * vsz) * n
    strict_bytes = passes * (2 * ksz + 2 * vsz) * n

    workload = cfg.name

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        m = min(args.cpu_sample, n) if args.cpu_sample > 0 else n
        sample_k = np.ascontiguousarray(keys_np[:m])
        sample_v = None if vals_np is None else np.arange(m, dtype=np.uint32)
        log("[bench] CPU oracle on %d keys x %d runs" % (m, args.cpu_reps))
        times = oracle.time_sort(sample_k, sample_v, cfg.begin_bit, cfg.end_bit, reps=args.cpu_reps)
        t = statistics.median(times)
        cpu = {"value": m / t / 1e9, "unit": "Gkeys/s", "cores": 1, "kind": "oracle",
               "sample": "%s %d keys of the same input, %s, median of %d runs, one host thread "
                         "of %d (%s)" % ("all" if m == n else "first", m,
                                         "pairs" if vals_np is not None else "keys only",
                                         args.cpu_reps, os.cpu_count() or 0, cpu_model()),
               "seconds": t}

    result = {
        "metric": "Gkeys/s, uint32 LSD radix sort at 1e8 keys; % of HBM roofline",
        "value": gkeys,
        "unit": "Gkeys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (gkeys / PAGES_GPU_GKEYS) if cfg.name == "c2_u32_keys_1e8" else None,
        "dtype": cfg.key_type if vals_np is None else cfg.key_type + "+u32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "description": cfg.description, "n": n,
                   "key": cfg.key_type, "values": "u32" if vals_np is not None else None,
                   "begin_bit": cfg.begin_bit, "end_bit": cfg.end_bit, "passes": passes,
                   "digit_bits": db,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(workload, db, dominant),
                     "bytes_per_launch": down_bytes, "avg_launch_ms": avg[dominant]},
        "kernels_avg_ms": avg,
        "kernel_launches": launches,
        "upsweep_gbs": per_launch["upsweep"] / (avg["upsweep"] * 1e-3) / 1e9 if "upsweep" in avg else None,
        "sort_roofline": {"bytes": sort_bytes, "gbs": sort_bytes / (ms_per_step * 1e-3) / 1e9,
                          "frac": sort_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          "strict_bytes": strict_bytes,
                          "strict_frac": strict_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "step_ms_median": statistics.median(per_step),
        "step_ms_min": min(per_step),
        "copy_reference_gbs": copy_gbs,
        "read_reference_gbs": read_gbs,
        "output_checked": exact and same_again,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)
    return 0 if (exact and same_again) else 1


if __name__ == "__main__":
    sys.exit(main())
