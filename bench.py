#!/usr/bin/env python3
"""Decode-step throughput of the top-k sparse attention path on one MI355X.

Workload: the batched grouped-query exact variant at L = 128K, k = 4096
(B = 16 sequences, 64 query heads over 8 KV heads, d = 128, bf16 caches with
0.5% planted aligned keys), one fused topk_decode call per step: score every
cached key, exact top-k per (sequence, query head), softmax attention over
the kept K/V rows. Inputs are seeded synthetic caches resident in HBM before
timing starts (8 GiB of K and V, far above the 256 MB last-level cache).

Prints one JSON line: queries/s (value), the HBM GB/s over the counted bytes
(full K scan + k gathered K and V rows per query head) and its fraction of
8 TB/s, the roofline of the dominant kernel (the scoring scan, timed alone
with HIP events on the launch stream), and the fp64 CPU oracle's throughput
on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, AMD's published peak
METRIC = "decode queries/sec and HBM GB/s (% of roofline) at L=128K, k=4096, 1 MI355X"
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
CSRC = os.path.join(ROOT, "top_sparse_attention_topk_amd", "csrc")
COPY_BYTES = 1 << 30  # calibration kernel: torch.neg over 1 GiB of fp32 reads and writes this many bytes
COPY_KERNEL = "torch.neg (copy calibration)"
STEP_COUNTERS = os.path.join(ROOT, "profiles", "step_counters.json")
MFMA_COUNTERS = os.path.join(ROOT, "profiles", "mfma_counters.json")
PROBE_LIB = os.path.join(ROOT, "top_sparse_attention_topk_amd", "libtka_probe.so")
STREAM_BYTES = 4 << 30  # streaming-read probe: bytes read per launch


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def esize(w):
    import fixtures as fx
    return 4 if w.dtype == fx.F32 else 2


def counted_bytes(w) -> int:
    """Bytes a decode step must move: the full scan of the scored keys plus the
    kept K and V rows of every query head (shared kept sets: per KV head)."""
    import fixtures as fx
    es = esize(w)
    row = w.d * es
    if w.mode == fx.MODE_EXACT:
        kk = min(w.k, w.L)
        return w.B * w.Hkv * w.L * row + 2 * w.B * w.Hq * kk * row
    if w.mode == fx.MODE_BLOCK:
        m = w.m
        kk = min(w.k, m - 1)
        cur = w.L - (m - 1) * w.block
        return w.B * w.Hkv * m * w.d * 4 + 2 * w.B * w.Hq * (kk * w.block + cur) * row
    kk = min(w.k, w.L)
    return w.B * w.L * w.dI + 2 * w.B * w.Hkv * kk * row


def score_kernel_bytes(w) -> int:
    """Algorithmic bytes of one scoring launch: keys read once, q read, fp32 scores written."""
    import fixtures as fx
    es = esize(w)
    if w.mode == fx.MODE_EXACT:
        return w.B * w.Hkv * w.L * w.d * es + w.B * w.Hq * w.d * es + 4 * w.B * w.Hq * w.L
    if w.mode == fx.MODE_BLOCK:
        return w.B * w.Hkv * w.m * w.d * 4 + w.B * w.Hq * w.d * es + 4 * w.B * w.Hq * (w.m - 1)
    return w.B * w.L * w.dI + w.B * w.HI * (w.dI + 4) + 4 * w.B * w.L


def source_digest() -> str:
    """sha256 over every source of the decode path's kernels (csrc/, without the benchmark's own
    streaming probe in csrc/probe/): counters taken on other sources are stale."""
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(CSRC, "**", "*"), recursive=True)):
        if not os.path.isfile(path) or os.path.relpath(path, CSRC).startswith("probe"):
            continue
        with open(path, "rb") as f:
            h.update(os.path.relpath(path, CSRC).encode() + b"\0" + f.read())
    return h.hexdigest()


def traffic_from_profiles(kernel: str):
    """Measured HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated),
    if profiles/counters.json holds them for the current kernel sources."""
    try:
        with open(COUNTERS) as f:
            rec = json.load(f)
        if rec.get("source_sha256") != source_digest():
            return None
        ks = rec["kernels"]
        if kernel not in ks:  # a base name: the one instantiation that carries it
            hits = [n for n in ks if n.split("<")[0] == kernel]
            if len(hits) != 1:
                return None
            kernel = hits[0]
        k = ks[kernel]
        return int(k["fetch_bytes_per_launch"] + k["write_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def short_name(name: str) -> str:
    """Qualified kernel name with its template arguments (instantiations differ in work)."""
    name = name.strip()
    if name.startswith("void "):
        name = name[5:]
    return name.split("(")[0].strip()


def copy_calibration(launches: int = 3):
    """A plain elementwise kernel of known traffic (torch.neg over 1 GiB of
    fp32: 1 GiB read, 1 GiB written) to scale the HBM byte counters by."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(launches):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()


def summarize_trace(trace_dir: str, tail: int) -> None:
    """Per-kernel dispatch count and mean/min/max duration from a rocprofv3
    --kernel-trace csv, plus the mean of each kernel's last `tail` dispatches
    (the standalone timing loops run last)."""
    paths = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    per = {}
    for path in paths:
        with open(path) as f:
            for r in csv.DictReader(f):
                ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                per.setdefault(short_name(r["Kernel_Name"]), []).append((int(r["Start_Timestamp"]), ns))
    print(f"{'kernel':56s} {'calls':>6s} {'mean_us':>9s} {'min_us':>9s} {'max_us':>9s} {'last%d_us' % tail:>9s}")
    for name, v in sorted(per.items(), key=lambda kv: -sum(ns for _, ns in kv[1])):
        v.sort()
        ns = [d for _, d in v]
        last = ns[-tail:]
        print(f"{name[:56]:56s} {len(ns):6d} {sum(ns) / len(ns) / 1e3:9.1f} {min(ns) / 1e3:9.1f} "
              f"{max(ns) / 1e3:9.1f} {sum(last) / len(last) / 1e3:9.1f}")


def summarize_counters(fetch_dir: str, write_dir: str, tail: int) -> None:
    """HBM bytes per launch from a FETCH_SIZE run and a WRITE_SIZE run (KiB per
    dispatch), each divided by what the same counter reads for the copy
    calibration kernel over its known size; the mean over each kernel's last
    `tail` dispatches. Writes profiles/counters.json and prints a table."""
    vals = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    if r["Counter_Name"] != counter:
                        continue
                    name = COPY_KERNEL if "neg_kernel" in r["Kernel_Name"] else short_name(r["Kernel_Name"])
                    disp = vals.setdefault(name, {}).setdefault(counter, {})
                    key = int(r["Dispatch_Id"])
                    disp[key] = disp.get(key, 0.0) + float(r["Counter_Value"])

    def mean_tail(kernel, counter):
        d = vals[kernel][counter]
        v = [d[i] * 1024.0 for i in sorted(d)][-tail:]
        return sum(v) / len(v)

    if COPY_KERNEL not in vals:
        raise SystemExit(f"no copy calibration dispatches (torch.neg) among {sorted(vals)}")
    cf = mean_tail(COPY_KERNEL, "FETCH_SIZE") / COPY_BYTES
    cw = mean_tail(COPY_KERNEL, "WRITE_SIZE") / COPY_BYTES
    out = {"source_sha256": source_digest(),
           "calibration": {"kernel": COPY_KERNEL, "bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                           "fetch_factor": round(cf, 5), "write_factor": round(cw, 5)},
           "kernels": {}}
    print(f"calibration {COPY_KERNEL}: FETCH_SIZE/{COPY_BYTES} = {cf:.4f}, WRITE_SIZE/{COPY_BYTES} = {cw:.4f}")
    print(f"{'kernel':56s} {'fetch_raw_MB':>13s} {'write_raw_MB':>13s} {'fetch_MB':>10s} {'write_MB':>10s}")
    for name in sorted(vals):
        if name == COPY_KERNEL or "FETCH_SIZE" not in vals[name] or "WRITE_SIZE" not in vals[name]:
            continue
        f_raw, w_raw = mean_tail(name, "FETCH_SIZE"), mean_tail(name, "WRITE_SIZE")
        out["kernels"][name] = {"fetch_bytes_per_launch": round(f_raw / cf), "write_bytes_per_launch": round(w_raw / cw),
                                "fetch_raw_bytes": round(f_raw), "write_raw_bytes": round(w_raw)}
        print(f"{name[:56]:56s} {f_raw / 1e6:13.1f} {w_raw / 1e6:13.1f} {f_raw / cf / 1e6:10.1f} {w_raw / cw / 1e6:10.1f}")
    with open(COUNTERS, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


def fresh_record(path: str):
    """A profiles/*.json record if it was taken on the current kernel sources, else None."""
    try:
        with open(path) as f:
            rec = json.load(f)
        return rec if rec.get("source_sha256") == source_digest() else None
    except (OSError, ValueError):
        return None


def fused_step_bytes_needed(w) -> int:
    """Bytes the fused exact step cannot avoid: every K row scanned, q read, the kept V rows of every
    query head read (the logits come from the kept scores, so no K row is read twice), out written."""
    es = esize(w)
    kk = min(w.k, w.L)
    return (w.B * w.Hkv * w.L * w.d * es + w.B * w.Hq * w.d * es + w.B * w.Hq * kk * w.d * es
            + 4 * w.B * w.Hq * w.d)


def host_record() -> dict:
    """The host the CPU baseline ran on: CPU model, sockets, physical cores, logical CPUs, the CPUs this
    process may use and OMP_NUM_THREADS."""
    model, sockets, cores = None, set(), set()
    phys = core = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                k, _, v = line.partition(":")
                k, v = k.strip(), v.strip()
                if k == "model name" and model is None:
                    model = v
                elif k == "physical id":
                    phys = v
                    sockets.add(v)
                elif k == "core id":
                    core = v
                elif not k and phys is not None:
                    cores.add((phys, core))
                    phys = core = None
        if phys is not None:
            cores.add((phys, core))
    except OSError:
        pass
    return {"cpu_model": model, "sockets": len(sockets) or None, "physical_cores": len(cores) or None,
            "logical_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}


def stream_read_peak(torch, steps: int = 10) -> dict:
    """Measured HBM read ceiling: the committed streaming-read probe (csrc/probe/stream_read.hip) over
    4 GiB, read once per launch with 16-byte non-temporal loads, for 1, 2, 4 and 8 persistent
    workgroups of 256 threads per compute unit; HIP events on the launch stream. Beside it, the same
    stream with one byte written per 8 read (contiguous 1 KiB per 8 KiB tile: the ratio of a scan
    that writes an fp32 score per head for 8 heads of bf16 d = 128 rows), 1 and 2 workgroups per CU."""
    import ctypes
    lib = ctypes.CDLL(PROBE_LIB)
    lib.tka_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                          ctypes.c_void_p]
    lib.tka_probe_stream_read_write.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_int, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    buf = torch.empty(STREAM_BYTES, dtype=torch.uint8, device="cuda")
    sink = torch.empty(cus * 8 * 256, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    by = {}
    for wpc in (1, 2, 4, 8):
        grid = cus * wpc

        def run():
            if lib.tka_probe_stream_read(buf.data_ptr(), STREAM_BYTES, sink.data_ptr(), grid, st) != 0:
                raise RuntimeError("stream read probe launch failed")
        ms = time_loop(run, steps)
        by[str(wpc)] = round(STREAM_BYTES / (ms / 1e3) / 1e9, 1)
    dst = torch.empty(STREAM_BYTES // 8, dtype=torch.uint8, device="cuda")
    rw = {}
    for wpc in (1, 2):
        grid = cus * wpc

        def run_rw():
            if lib.tka_probe_stream_read_write(buf.data_ptr(), STREAM_BYTES, dst.data_ptr(), sink.data_ptr(), grid,
                                               st) != 0:
                raise RuntimeError("read-write probe launch failed")
        ms = time_loop(run_rw, steps)
        rw[str(wpc)] = {"ms": round(ms, 4), "gbps_read": round(STREAM_BYTES / (ms / 1e3) / 1e9, 1),
                        "gbps_read_plus_write": round(STREAM_BYTES * 9 / 8 / (ms / 1e3) / 1e9, 1)}
    del buf, sink, dst
    best = max(by.values())
    best_rw = max(v["gbps_read_plus_write"] for v in rw.values())
    return {"gbps": best, "frac_of_peak": round(best / PEAK_HBM_GBPS, 4), "bytes_per_launch": STREAM_BYTES,
            "gbps_by_workgroups_per_cu": by, "kernel": "tka_probe::stream_read_kernel (csrc/probe/stream_read.hip)",
            "with_writes": {"bytes_written_per_byte_read": 0.125, "gbps_read_plus_write": best_rw,
                            "frac_of_peak": round(best_rw / PEAK_HBM_GBPS, 4), "by_workgroups_per_cu": rw,
                            "kernel": "tka_probe::stream_read_write_kernel (csrc/probe/stream_read.hip)"}}


def _counter_rows(dirs):
    """(kernel short name, dispatch id, counter, value) of every counter_collection.csv under dirs."""
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    name = COPY_KERNEL if "neg_kernel" in r["Kernel_Name"] else short_name(r["Kernel_Name"])
                    yield name, int(r["Dispatch_Id"]), r["Counter_Name"], float(r["Counter_Value"])


def summarize_step_counters(fetch_dir: str, write_dir: str, steps: int) -> None:
    """HBM bytes per fused step from a --profile-step run under FETCH_SIZE and one under WRITE_SIZE: every
    dispatch of a libtka kernel summed, divided by the number of steps, each counter scaled by what it
    reads for the copy calibration kernel over its known size. Writes profiles/step_counters.json."""
    per = {}  # (kernel, counter) -> {dispatch: value}
    for name, disp, counter, val in _counter_rows([fetch_dir, write_dir]):
        if counter in ("FETCH_SIZE", "WRITE_SIZE"):
            d = per.setdefault((name, counter), {})
            d[disp] = d.get(disp, 0.0) + val * 1024.0  # KiB per dispatch
    cal = {c: sum(per.get((COPY_KERNEL, c), {}).values()) / max(len(per.get((COPY_KERNEL, c), {})), 1) / COPY_BYTES
           for c in ("FETCH_SIZE", "WRITE_SIZE")}
    if not all(cal.values()):
        raise SystemExit("no copy calibration dispatches in the step profile")
    kern = {}
    for (name, counter), d in per.items():
        if not name.startswith("tka::"):
            continue
        k = kern.setdefault(name, {"launches_per_step": len(d) / steps})
        k["fetch_bytes_per_step" if counter == "FETCH_SIZE" else "write_bytes_per_step"] = \
            round(sum(d.values()) / cal[counter] / steps)
    fetch = sum(k.get("fetch_bytes_per_step", 0) for k in kern.values())
    write = sum(k.get("write_bytes_per_step", 0) for k in kern.values())
    out = {"source_sha256": source_digest(), "workload": fx_workload_name(), "steps": steps,
           "bytes_per_step": fetch + write, "fetch_bytes_per_step": fetch, "write_bytes_per_step": write,
           "calibration": {"kernel": COPY_KERNEL, "fetch_factor": round(cal["FETCH_SIZE"], 5),
                           "write_factor": round(cal["WRITE_SIZE"], 5)},
           "kernels": kern}
    print(f"{'kernel':60s} {'launches':>8s} {'fetch_MB':>10s} {'write_MB':>10s}   (per step)")
    for name, k in sorted(kern.items(), key=lambda kv: -kv[1].get("fetch_bytes_per_step", 0)):
        print(f"{name[:60]:60s} {k['launches_per_step']:8.2f} {k.get('fetch_bytes_per_step', 0) / 1e6:10.1f} "
              f"{k.get('write_bytes_per_step', 0) / 1e6:10.1f}")
    print(f"{'step total':60s} {'':8s} {fetch / 1e6:10.1f} {write / 1e6:10.1f}  = {(fetch + write) / 1e6:.1f} MB")
    with open(STEP_COUNTERS, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


def fx_workload_name() -> str:
    import fixtures as fx
    return fx.WORKLOADS[os.environ.get("TKA_BENCH_WORKLOAD", "C3")].name


# MFMA kernels of the path, their MFMA instruction and the flops one instruction performs
MFMA_SHAPES = {"bf16_16x16x32": 2 * 16 * 16 * 32, "f8_32x32x64": 2 * 32 * 32 * 64}


def summarize_mfma(dirs, tail: int) -> None:
    """MFMA counters per kernel (mean per dispatch over each kernel's last `tail` dispatches) from
    --profile-mfma runs: rocprofv3's MfmaUtil (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs), in %),
    the raw counters, and the flops the MOPS counters imply (MOPS count operations in units of 512).
    Writes profiles/mfma_counters.json."""
    vals = {}
    for name, disp, counter, val in _counter_rows(dirs):
        d = vals.setdefault(name, {}).setdefault(counter, {})
        d[disp] = d.get(disp, 0.0) + val
    out = {"source_sha256": source_digest(), "kernels": {}}
    for name in sorted(vals):
        if not name.startswith("tka::"):
            continue
        rec = {}
        for counter, d in vals[name].items():
            v = [d[i] for i in sorted(d)][-tail:]
            rec[counter] = sum(v) / len(v)
        mops = sum(v for c, v in rec.items() if c.startswith("SQ_INSTS_VALU_MFMA_MOPS"))
        if mops:
            rec["mfma_flops_from_mops"] = mops * 512
        if "SQ_INSTS_VALU" in rec and rec.get("SQ_BUSY_CYCLES"):
            rec["valu_insts_per_busy_cycle"] = round(rec["SQ_INSTS_VALU"] / rec["SQ_BUSY_CYCLES"], 4)
        out["kernels"][name] = {k: (round(v, 3) if isinstance(v, float) else v) for k, v in rec.items()}
    cols = ["MfmaUtil", "SQ_INSTS_MFMA", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F8",
            "mfma_flops_from_mops", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU", "SQ_BUSY_CYCLES"]
    print("kernel | " + " | ".join(cols))
    for name, rec in out["kernels"].items():
        print(name[:70] + " | " + " | ".join(str(rec.get(c, "-")) for c in cols))
    with open(MFMA_COUNTERS, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


def profile_mfma(fx, tka, torch, np, steps: int) -> None:
    """Launch each MFMA kernel of the path a few times for the MFMA counters: the fused C3 step (sample
    scores, candidate scan), the full C3 scores, four queries per sequence (its sampled scan and its dense
    scores), the two-level step's group scores, and the C5 indexer scores."""
    w = fx.WORKLOADS["C3"]
    q, K, V = fx.make_attn(w)
    to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    qt, Kt, Vt = to(q), to(K), to(V)
    del K, V
    p = tka.problem(tka.EXACT, w.B, w.Hq, w.Hkv, w.d, w.L, w.k, tka.TKA_BF16)
    for _ in range(steps):
        tka.topk_decode(p, qt, Kt, Vt)
        tka.topk_attn_score(p, qt, Kt)
    M = 4
    qm = to(fx.encode(fx.normal(97, 0, w.B * M * w.Hq * w.d), fx.BF16).reshape(w.B, M, w.Hq, w.d))
    pm = tka.problem(tka.EXACT, w.B, w.Hq, w.Hkv, w.d, w.L, w.k, tka.TKA_BF16, n_queries=M)
    for _ in range(steps):
        tka.topk_decode(pm, qm, Kt, Vt)
        tka.topk_attn_score(pm, qm, Kt)
    ph = tka.problem(tka.HISA, w.B, w.Hq, w.Hkv, w.d, w.L, w.k, tka.TKA_BF16, 0.0, 64, top_blocks=128)
    means = tka.topk_block_mean_build(ph, Kt)
    for _ in range(steps):
        tka.topk_hisa_decode(ph, qt, Kt, Vt, means)
    torch.cuda.synchronize()
    del Kt, Vt, means
    torch.cuda.empty_cache()
    w5 = fx.WORKLOADS["C5"]
    qI, kI, wt = fx.make_indexer(w5)
    p5 = tka.problem(tka.INDEXER, w5.B, w5.Hq, w5.Hkv, w5.d, w5.L, w5.k, tka.TKA_BF16, 0.0, 0, w5.HI, w5.dI)
    qIt, kIt, wtt = torch.from_numpy(qI).cuda(), torch.from_numpy(kI).cuda(), torch.from_numpy(wt).cuda()
    for _ in range(steps):
        tka.topk_attn_score(p5, qIt, kIt, idx_w=wtt)
    torch.cuda.synchronize()
    log(f"[bench] profile-mfma: {steps} launches of each MFMA kernel done")


def time_windows(fn, steps: int, multiple: int = 1) -> float:
    """Median ms per call over five event-timed windows of back-to-back calls, each window at least
    100 ms (and `steps` calls), its length a whole multiple of `multiple` (replica passes)."""
    est = time_loop(fn, steps)
    n = max(steps, int(math.ceil(100.0 / max(est, 1e-4))))
    n = -(-n // multiple) * multiple
    return statistics.median([time_loop(fn, n) for _ in range(5)])


def time_loop(fn, steps: int) -> float:
    """Average ms per call from HIP events on the current stream (the launch stream)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def cpu_oracle_step(w, q, K, V, qI=None, kI=None, wt=None, repeats: int = 3) -> dict:
    """The fp64 oracle, as it stands, on one whole step of this workload (every row: score, full
    sort, attention) on all host threads, `repeats` times; the median with queries/s and GB/s over
    the same counted bytes as the GPU figures. An unoptimised reference, not a tuned CPU library."""
    import oracle as orc
    p = orc.problem_for(w)
    ts = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        orc.decode(p, q, K, V, qI=qI, kI=kI, w=wt)
        ts.append(time.perf_counter() - t0)
    t = statistics.median(ts)
    return {"kind": "oracle", "threads": orc.threads(), "repeats": repeats, "t_step_ms": round(t * 1e3, 3),
            "queries_per_s": round(w.B / t, 2), "gbps_counted": round(counted_bytes(w) / t / 1e9, 3)}


def proxy_variant(fx, tka, torch, np, w, steps: int, cpu: bool = False) -> dict:
    """Fused step and scoring launch of a proxy-score workload (block means or indexer), each timed
    alone on the launch stream; the scoring launch against the HBM roofline (its algorithmic bytes:
    proxy keys read once, q read, fp32 scores written).

    A step of these workloads touches 70-100 MB, which the 256 MB Infinity Cache (MALL) can hold
    across back-to-back steps. The reported times therefore rotate over R on-device replicas of
    every input (copies of the same bytes), R * counted bytes >= 1 GiB, so that each step reads
    HBM; the same loops on one replica are reported beside them as *_mall_warm (not HBM)."""
    q, K, V = fx.make_attn(w)
    to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    qt, Kt, Vt = to(q), to(K), to(V)
    res = {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "seq_len": w.L, "top_k": w.k}
    if cpu:  # the oracle on the same host bytes (one step of L = 1M takes seconds: one repeat there)
        oi = fx.make_indexer(w) if w.mode == fx.MODE_INDEXER else (None, None, None)
        res["cpu_oracle"] = cpu_oracle_step(w, q, K, V, *oi, repeats=1 if w.mode == fx.MODE_INDEXER else 3)
        del oi
    del K, V
    p = tka.problem(w.mode, w.B, w.Hq, w.Hkv, w.d, w.L, w.k, tka.TKA_BF16, 0.0, w.block, w.HI, w.dI)
    if w.mode == fx.MODE_BLOCK:
        means = tka.topk_block_mean_build(p, Kt)
        res["block_size"] = w.block
        res["mean_build_ms"] = round(time_loop(lambda: tka.topk_block_mean_build(p, Kt, means), steps), 4)
        ins = dict(q=qt, K=Kt, V=Vt, proxy_keys=means)
        idx = torch.empty((w.B, w.Hq, w.k), dtype=torch.int32, device="cuda")
    else:
        qI, kI, wt = fx.make_indexer(w)
        ins = dict(q=qt, K=Kt, V=Vt, proxy_keys=torch.from_numpy(kI).cuda(), q_idx=torch.from_numpy(qI).cuda(),
                   idx_w=torch.from_numpy(wt).cuda())
        res["indexer_heads"], res["indexer_dim"] = w.HI, w.dI
        idx = torch.empty((w.B, w.k), dtype=torch.int32, device="cuda")
    R = -(-(1 << 30) // counted_bytes(w))
    reps = [ins] + [{n: t.clone() for n, t in ins.items()} for _ in range(R - 1)]
    sc = torch.empty(tka.score_shape(p), dtype=torch.float32, device="cuda")
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    ws = torch.empty(tka.topk_decode_workspace_size(p), dtype=torch.uint8, device="cuda")

    def decode(r):
        kw = {n: t for n, t in r.items() if n not in ("q", "K", "V")}
        tka.topk_decode(p, r["q"], r["K"], r["V"], out=out, idx_out=idx, ws=ws, **kw)

    def score(r):
        if w.mode == fx.MODE_BLOCK:
            tka.topk_attn_score(p, r["q"], r["proxy_keys"], scores=sc)
        else:
            tka.topk_attn_score(p, r["q_idx"], r["proxy_keys"], idx_w=r["idx_w"], scores=sc)

    def rotated(fn):  # whole passes over the replicas; the median of five windows of >= 100 ms
        it = iter(range(1 << 62))
        return time_windows(lambda: fn(reps[next(it) % R]), -(-steps // R) * R, R)

    t_dec, t_sc = rotated(decode), rotated(score)
    t_dec_w, t_sc_w = time_loop(lambda: decode(ins), steps), time_loop(lambda: score(ins), steps)
    sb = score_kernel_bytes(w)
    res.update({"replicas": R, "decode_ms": round(t_dec, 4), "decode_queries_per_s": round(w.B / (t_dec / 1e3), 1),
                "score_ms": round(t_sc, 4), "score_algorithmic_bytes": sb,
                "score_gbps": round(sb / (t_sc / 1e3) / 1e9, 1),
                "score_frac": round(sb / (t_sc / 1e3) / 1e9 / PEAK_HBM_GBPS, 4),
                "decode_ms_mall_warm": round(t_dec_w, 4), "score_ms_mall_warm": round(t_sc_w, 4)})
    del reps, ins
    return res


def exact_variant(fx, tka, torch, np, w, steps: int, cpu: bool = False) -> dict:
    """The exact variant at another workload's size: the fused step and the three calls (score, select,
    gather) timed as one step, each on the launch stream. Footprints under 1 GiB rotate over R on-device
    replicas of q, K and V (R * counted bytes >= 1 GiB) so each step reads HBM rather than the 256 MB
    Infinity Cache; the single-replica loops are reported beside them as *_mall_warm. A step smaller
    than 1 MiB (C1) is latency-bound: its time is reported in microseconds, cache-resident."""
    q, K, V = fx.make_attn(w)
    if w.dtype == fx.BF16:
        to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        dt = tka.TKA_BF16
    else:
        to = lambda a: torch.from_numpy(a).cuda()
        dt = tka.TKA_F32
    ins = dict(q=to(q), K=to(K), V=to(V))
    cpu_rec = cpu_oracle_step(w, q, K, V) if cpu else None
    del K, V
    p = tka.problem(tka.EXACT, w.B, w.Hq, w.Hkv, w.d, w.L, w.k, dt)
    cb = counted_bytes(w)
    latency = cb < (1 << 20)
    R = 1 if latency else -(-(1 << 30) // cb)
    reps = [ins] + [{n: t.clone() for n, t in ins.items()} for _ in range(R - 1)]
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.B, w.Hq, w.k), dtype=torch.int32, device="cuda")
    ws = torch.empty(tka.topk_decode_workspace_size(p), dtype=torch.uint8, device="cuda")
    rows = w.B * w.Hq
    sc = torch.empty(tka.score_shape(p), dtype=torch.float32, device="cuda")
    sel_idx = torch.empty((rows, w.k), dtype=torch.int32, device="cuda")
    sel_val = torch.empty((rows, w.k), dtype=torch.float32, device="cuda")
    sws = torch.empty(max(tka.topk_select_workspace_size(rows, w.L, w.k), 1), dtype=torch.uint8, device="cuda")
    gws = torch.empty(max(tka.sparse_attn_gather_workspace_size(p, w.k), 1), dtype=torch.uint8, device="cuda")
    gout = torch.empty_like(out)

    def fused(r):
        tka.topk_decode(p, r["q"], r["K"], r["V"], out=out, idx_out=idx, ws=ws)

    # the candidate prefilter forced where the automatic choice takes the dense composition
    pp = tka.problem(tka.EXACT, w.B, w.Hq, w.Hkv, w.d, w.L, w.k, dt, decode_path=tka.TKA_PATH_PREFILTER)
    ws_p = torch.empty(tka.topk_decode_workspace_size(pp), dtype=torch.uint8, device="cuda")

    def fused_prefilter(r):
        tka.topk_decode(pp, r["q"], r["K"], r["V"], out=out, idx_out=idx, ws=ws_p)

    def three(r):
        tka.topk_attn_score(p, r["q"], r["K"], scores=sc)
        tka.topk_select(sc.reshape(rows, w.L), w.k, idx_out=sel_idx, sel_out=sel_val, ws=sws)
        tka.sparse_attn_gather(p, r["q"], r["K"], r["V"], sel_idx, sel_scores=sel_val, out=gout, ws=gws)

    def rotated(fn):  # whole passes over the replicas; the median of five windows of >= 100 ms
        it = iter(range(1 << 62))
        return time_windows(lambda: fn(reps[next(it) % R]), -(-steps // R) * R, R)

    t_f, t_3 = rotated(fused), rotated(three)
    res = {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d, "seq_len": w.L,
           "top_k": w.k, "dtype": "bf16" if w.dtype == fx.BF16 else "f32", "replicas": R,
           "counted_bytes_per_step": cb}
    if latency:
        res.update({"bound": "latency (the step's 0.3 MB stay in cache; no HBM roofline)",
                    "decode_us": round(t_f * 1e3, 2), "three_call_us": round(t_3 * 1e3, 2),
                    "decode_queries_per_s": round(w.B / (t_f / 1e3), 1)})
    else:
        gb = cb / (t_f / 1e3) / 1e9
        res.update({"decode_ms": round(t_f, 4), "decode_queries_per_s": round(w.B / (t_f / 1e3), 1),
                    "hbm_gbps_counted": round(gb, 1), "pct_of_hbm_peak": round(100 * gb / PEAK_HBM_GBPS, 2),
                    "three_call_ms": round(t_3, 4),
                    "three_call_queries_per_s": round(w.B / (t_3 / 1e3), 1),
                    "decode_prefilter_forced_ms": round(rotated(fused_prefilter), 4),
                    "decode_ms_mall_warm": round(time_loop(lambda: fused(ins), steps), 4),
                    "three_call_ms_mall_warm": round(time_loop(lambda: three(ins), steps), 4)})
    if cpu_rec is not None:
        res["cpu_oracle"] = cpu_rec
    del reps, ins
    return res


def _oracle_queries(orc, p, w, q, K, V, budget_s: float):
    done = 0
    t0 = time.perf_counter()
    while True:  # sequences in order, wrapping around, until the budget is spent
        b = done % w.B
        orc.decode(p, q, K, V, rows=list(range(b * w.Hq, (b + 1) * w.Hq)))
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    return done, time.perf_counter() - t0


def cpu_baseline(w, q, K, V, budget_s: float, single_budget_s: float):
    """The fp64 oracle, as it stands, on whole queries (all heads of one
    sequence) of the same workload until about budget_s seconds have passed,
    on all the threads OpenMP gives it; then the same on one thread."""
    import ctypes

    import oracle as orc
    p = orc.problem_for(w)
    threads = orc.threads()
    done, dt = _oracle_queries(orc, p, w, q, K, V, budget_s)
    res = {"value": done / dt, "unit": "queries/s", "cores": threads, "kind": "oracle",
           "sample": f"{done} whole queries ({done * w.Hq} query-head rows of L={w.L}) of the timed workload: "
                     f"fp64 scores, full sort, fp64 attention; {dt:.1f} s on {threads} threads",
           "host": host_record()}
    if single_budget_s > 0:
        gomp = ctypes.CDLL("libgomp.so.1")  # the OpenMP runtime the oracle's parallel loops use
        gomp.omp_set_num_threads(1)
        try:
            d1, t1 = _oracle_queries(orc, p, w, q, K, V, single_budget_s)
        finally:
            gomp.omp_set_num_threads(threads)
        res["single_core"] = {"value": d1 / t1, "unit": "queries/s", "cores": 1,
                              "sample": f"{d1} whole queries on one thread; {t1:.1f} s"}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="C3", help="fixtures.WORKLOADS key (C3 is the headline)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--cpu-single-budget", type=float, default=6.0,
                    help="seconds of oracle work on one thread (0: skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the adjacent paths (profiling runs: the roofline launches stay the last ones)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run the known-size copy kernel that HBM byte counters are scaled by")
    ap.add_argument("--summarize-trace", metavar="DIR", help="print kernel durations from a rocprofv3 trace; no GPU")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/counters.json from FETCH_SIZE / WRITE_SIZE runs; no GPU")
    ap.add_argument("--tail", type=int, default=3, help="summaries: mean over each kernel's last N dispatches")
    ap.add_argument("--profile-step", type=int, metavar="N",
                    help="run N fused steps of the workload and the copy calibration, nothing else (counters)")
    ap.add_argument("--summarize-step-counters", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "N"),
                    help="write profiles/step_counters.json from two --profile-step N runs; no GPU")
    ap.add_argument("--profile-mfma", type=int, metavar="N",
                    help="launch every MFMA kernel of the path N times (MFMA counters)")
    ap.add_argument("--summarize-mfma", nargs="+", metavar="DIR",
                    help="write profiles/mfma_counters.json from --profile-mfma counter runs; no GPU")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.tail)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.tail)
        return
    if args.summarize_step_counters:
        f_dir, w_dir, n = args.summarize_step_counters
        os.environ["TKA_BENCH_WORKLOAD"] = args.workload
        summarize_step_counters(f_dir, w_dir, int(n))
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma, args.tail)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the path has no multi-GPU mode.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fixtures as fx
    import top_sparse_attention_topk_amd as tka

    if args.profile_mfma:
        profile_mfma(fx, tka, torch, np, args.profile_mfma)
        return
    w = fx.WORKLOADS[args.workload]
    log(f"[bench] generating {w.name}")
    q, K, V = fx.make_attn(w)
    to = (lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()) if w.dtype == fx.BF16 else \
        (lambda a: torch.from_numpy(a).cuda())
    qt, Kt, Vt = to(q), to(K), to(V)
    dt = tka.TKA_BF16 if w.dtype == fx.BF16 else tka.TKA_F32
    p = tka.problem(w.mode, w.B, w.Hq, w.Hkv, w.d, w.L, w.k, dt, 0.0, w.block, w.HI, w.dI)
    kw = {}
    if w.mode == fx.MODE_BLOCK:
        kw["proxy_keys"] = tka.topk_block_mean_build(p, Kt)
    elif w.mode == fx.MODE_INDEXER:
        qI, kI, wt = fx.make_indexer(w)
        kw = dict(proxy_keys=torch.from_numpy(kI).cuda(), q_idx=torch.from_numpy(qI).cuda(),
                  idx_w=torch.from_numpy(wt).cuda())
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.B, w.k) if w.mode == fx.MODE_INDEXER else (w.B, w.Hq, w.k), dtype=torch.int32,
                      device="cuda")
    ws = torch.empty(tka.topk_decode_workspace_size(p), dtype=torch.uint8, device="cuda")
    step = lambda: tka.topk_decode(p, qt, Kt, Vt, out=out, idx_out=idx, ws=ws, **kw)
    if args.profile_step:
        for _ in range(args.profile_step):
            step()
        torch.cuda.synchronize()
        copy_calibration(launches=1)
        log(f"[bench] profile-step: {args.profile_step} steps and the copy calibration done")
        return

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    ev_ms = e0.elapsed_time(e1) / args.steps
    qps = w.B / (ms / 1e3)
    # beside the contract's one timed window: five event-timed windows of at least 100 ms each
    # (back-to-back steps), and their median
    # (left out of the short profiling runs, --no-extras)
    repeats = None
    if not args.no_extras:
        n_rep = max(args.steps, int(math.ceil(100.0 / max(ev_ms, 1e-3))))
        rep_ms = [round(time_loop(step, n_rep), 4) for _ in range(5)]
        repeats = {"steps_per_window": n_rep, "ms_per_step": rep_ms,
                   "median_ms_per_step": statistics.median(rep_ms),
                   "median_queries_per_s": round(w.B / (statistics.median(rep_ms) / 1e3), 1)}
    cb = counted_bytes(w)
    gbps = cb / (ms / 1e3) / 1e9

    # per-kernel split: each step of the path launched alone on the same stream
    log("[bench] per-kernel timing")
    if w.mode == fx.MODE_INDEXER:
        score_call = lambda: tka.topk_attn_score(p, kw["q_idx"], kw["proxy_keys"], idx_w=kw["idx_w"], scores=sc)
    elif w.mode == fx.MODE_BLOCK:
        score_call = lambda: tka.topk_attn_score(p, qt, kw["proxy_keys"], scores=sc)
    else:
        score_call = lambda: tka.topk_attn_score(p, qt, Kt, scores=sc)
    sc = torch.empty(tka.score_shape(p), dtype=torch.float32, device="cuda")
    t_score = time_loop(score_call, args.steps)
    rows = sc.numel() // sc.shape[-1]
    sel_idx = torch.empty((rows, w.k), dtype=torch.int32, device="cuda")
    sel_val = torch.empty((rows, w.k), dtype=torch.float32, device="cuda")
    nws = tka.topk_select_workspace_size(rows, sc.shape[-1], w.k)
    sws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    exact = w.mode == fx.MODE_EXACT
    t_select = time_loop(lambda: tka.topk_select(sc.reshape(rows, -1), w.k, idx_out=sel_idx,
                                                 sel_out=sel_val if exact else None, want_sel=exact, ws=sws),
                         args.steps)
    unit = w.block if w.mode == fx.MODE_BLOCK else 0
    shared = w.mode == fx.MODE_INDEXER
    gout = torch.empty_like(out)
    gws = torch.empty(max(tka.sparse_attn_gather_workspace_size(p, w.k, unit, shared), 1), dtype=torch.uint8,
                      device="cuda")
    gather_call = lambda: tka.sparse_attn_gather(p, qt, Kt, Vt, sel_idx, idx_unit=unit, shared=shared,
                                                 sel_scores=sel_val if exact else None, out=gout, ws=gws)
    t_gather = time_loop(gather_call, args.steps)
    select_call = lambda: tka.topk_select(sc.reshape(rows, -1), w.k, idx_out=sel_idx,
                                          sel_out=sel_val if exact else None, want_sel=exact, ws=sws)

    def three_call():
        score_call()
        select_call()
        gather_call()
    log("[bench] the three calls as one step")
    t_three = time_loop(three_call, args.steps)
    # dominant kernel of the timed step and its algorithmic bytes per launch
    t_thr = None
    if exact and dt == tka.TKA_BF16 and 2 <= w.G <= 16:
        # the fused step's scan: every key scored, pairs ranking at or above the
        # row's threshold kept. Timed alone with the row's k-th largest score
        # (the smallest selected one; selections come in index order) as threshold.
        thr = sel_val.min(dim=1).values.contiguous()
        cnt = torch.zeros(rows, dtype=torch.int32, device="cuda")
        cap = 3 * w.k
        cs = torch.empty((rows, cap), dtype=torch.float32, device="cuda")
        cpos = torch.empty((rows, cap), dtype=torch.int32, device="cuda")
        times = []
        for _ in range(args.steps):
            cnt.zero_()
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record()
            tka.topk_attn_score_threshold(p, qt, Kt, thr, cnt, cs, cpos)
            a1.record()
            times.append((a0, a1))
        torch.cuda.synchronize()
        t_thr = sum(a.elapsed_time(b) for a, b in times) / len(times)
        kept = int(cnt.sum().item())
        assert int(cnt.min().item()) >= w.k, "thresholded scan kept fewer than k pairs in a row"
        kname = f"tka::score_cand_persistent_kernel<{w.d}, false>"
        kbytes = (w.B * w.Hkv * w.L * w.d * 2 + w.B * w.Hq * w.d * 2 + 8 * rows + 8 * kept)
        kms = t_thr
    else:
        kname = {fx.MODE_EXACT: f"tka::score_exact_mfma_kernel<{w.d}, 0, 2>" if dt == tka.TKA_BF16 and 2 <= w.G <= 16
                 else "tka::score_vec_kernel", fx.MODE_BLOCK: "tka::score_vec_kernel",
                 fx.MODE_INDEXER: "tka::score_indexer_kernel"}[w.mode]
        kbytes = score_kernel_bytes(w)
        kms = t_score
    achieved = kbytes / (kms / 1e3) / 1e9
    traffic = traffic_from_profiles(kname)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic,
                "kernel": kname, "algorithmic_bytes": kbytes, "avg_launch_ms": round(kms, 4)}
    if t_thr is not None:
        roofline["kept_pairs"] = kept

    # the bytes the fused step moves: its unavoidable algorithmic bytes, and the HBM bytes its kernels'
    # counters read (FETCH_SIZE + WRITE_SIZE per step, copy-calibrated; null when taken on other sources)
    moved = None
    if exact:
        need = fused_step_bytes_needed(w)
        moved = {"bytes_needed": need, "gbps_needed": round(need / (ms / 1e3) / 1e9, 1),
                 "frac_needed": round(need / (ms / 1e3) / 1e9 / PEAK_HBM_GBPS, 4),
                 "what": "K scan + kept V rows + q + out (logits from the kept scores: no K row re-read)"}
        rec = fresh_record(STEP_COUNTERS)
        if rec and rec.get("workload") == w.name:
            mb = rec["bytes_per_step"]
            moved.update({"bytes_measured": mb, "gbps_measured": round(mb / (ms / 1e3) / 1e9, 1),
                          "frac_measured": round(mb / (ms / 1e3) / 1e9 / PEAK_HBM_GBPS, 4)})
        else:
            moved.update({"bytes_measured": None, "gbps_measured": None, "frac_measured": None})
    mrec = fresh_record(MFMA_COUNTERS)
    if mrec and kname in mrec.get("kernels", {}):
        roofline["mfma"] = mrec["kernels"][kname]
    log("[bench] streaming-read probe")
    read_peak = stream_read_peak(torch)

    result = {
        "metric": METRIC, "value": round(qps, 1), "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.dtype == fx.BF16 else "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d,
                   "seq_len": w.L, "top_k": w.k, "path": "fused topk_decode",
                   "gather_logits": "selected scores" if exact else "K rows"},
        "hbm_gbps_counted": round(gbps, 1), "pct_of_hbm_peak": round(100 * gbps / PEAK_HBM_GBPS, 2),
        "counted_bytes_per_step": cb,
        "counted_bytes_note": "headline byte count: full K scan + k gathered K and V rows per query head"
                              + (" (this path reads no gathered K row: see step_bytes)" if exact else ""),
        "step_bytes": moved, "event_ms_per_step": round(ev_ms, 4), "repeats": repeats,
        "three_call": {"ms_per_step": round(t_three, 4), "queries_per_s": round(w.B / (t_three / 1e3), 1),
                       "what": "topk_attn_score -> topk_select -> sparse_attn_gather, timed as one step"},
        "kernel_ms": {"score_full": round(t_score, 4), "select": round(t_select, 4), "gather": round(t_gather, 4),
                      "score_threshold": None if t_thr is None else round(t_thr, 4)},
        "roofline": roofline,
        "measured_read_peak": read_peak,
    }
    # adjacent paths on the same inputs (each timed alone on the launch stream)
    extras = {}
    if exact and not args.no_extras:
        log("[bench] certified adaptive k")
        eps = 0.9  # the synthetic caches spread their softmax mass widely: tau(k = 4096) is about 0.8
        ak_idx = torch.empty((rows, w.k), dtype=torch.int32, device="cuda")
        ak_k = torch.empty(rows, dtype=torch.int32, device="cuda")
        ak_tau = torch.empty(rows, dtype=torch.float32, device="cuda")
        ak_ws = torch.empty(max(tka.topk_select_adaptive_workspace_size(rows, sc.shape[-1], w.k), 1),
                            dtype=torch.uint8, device="cuda")
        t_ak = time_loop(lambda: tka.topk_select_adaptive(sc.reshape(rows, -1), eps, 1, w.k, idx_out=ak_idx,
                                                          k_out=ak_k, tau_out=ak_tau, ws=ak_ws), args.steps)
        del ak_ws
        torch.cuda.empty_cache()
        ad_out = torch.empty_like(out)
        ad_ws = torch.empty(tka.topk_decode_adaptive_workspace_size(p), dtype=torch.uint8, device="cuda")
        t_ad = time_loop(lambda: tka.topk_decode_adaptive(p, qt, Kt, Vt, eps, 1, out=ad_out, idx_out=ak_idx,
                                                          k_out=ak_k, tau_out=ak_tau, ws=ad_ws), args.steps)
        kf = ak_k.float()
        extras["adaptive"] = {"eps": eps, "k_max": w.k, "select_ms": round(t_ak, 4),
                              "select_score_gbps": round(4 * rows * sc.shape[-1] / (t_ak / 1e3) / 1e9, 1),
                              "decode_ms": round(t_ad, 4), "decode_queries_per_s": round(w.B / (t_ad / 1e3), 1),
                              "k_mean": round(float(kf.mean()), 1), "k_min": int(ak_k.min()),
                              "k_max_seen": int(ak_k.max()), "tau_max": round(float(ak_tau.max()), 5)}
        del ad_ws, ak_idx
        torch.cuda.empty_cache()
        # the two-level step on the same caches: 128 blocks of 64 kept, then the top k tokens
        log("[bench] two-level step")
        KB, bsz = 128, 64
        ph = tka.problem(tka.HISA, w.B, w.Hq, w.Hkv, w.d, w.L, w.k, dt, 0.0, bsz, top_blocks=KB)
        hmeans = tka.topk_block_mean_build(ph, Kt)
        h_out = torch.empty_like(out)
        h_idx = torch.empty((w.B, w.Hq, w.k), dtype=torch.int32, device="cuda")
        h_ws = torch.empty(tka.topk_hisa_decode_workspace_size(ph), dtype=torch.uint8, device="cuda")
        t_h = time_loop(lambda: tka.topk_hisa_decode(ph, qt, Kt, Vt, hmeans, out=h_out, idx_out=h_idx, ws=h_ws),
                        args.steps)
        m_blocks = (w.L + bsz - 1) // bsz
        h_bytes = (w.B * w.Hkv * m_blocks * w.d * 4 + rows * KB * bsz * w.d * 2 + rows * w.k * (w.d * 2 + 8))
        extras["hisa"] = {"block_size": bsz, "top_blocks": KB, "top_k": w.k, "decode_ms": round(t_h, 4),
                          "decode_queries_per_s": round(w.B / (t_h / 1e3), 1),
                          "algorithmic_bytes": h_bytes, "gbps": round(h_bytes / (t_h / 1e3) / 1e9, 1)}
        # the step's cache append on the same caches: row L-1 rewritten with its own values (no change),
        # alone and with the block-mean refresh of its block
        kn = Kt[:, :, w.L - 1].contiguous()
        vn = Vt[:, :, w.L - 1].contiguous()
        t_app = time_loop(lambda: tka.topk_cache_append(ph, kn, vn, Kt, Vt), args.steps)
        t_appm = time_loop(lambda: tka.topk_cache_append(ph, kn, vn, Kt, Vt, means=hmeans), args.steps)
        extras["append"] = {"kv_rows_us": round(t_app * 1e3, 2), "kv_rows_and_block_mean_us": round(t_appm * 1e3, 2)}
        del h_ws, hmeans
        torch.cuda.empty_cache()
        # several causal queries per sequence (speculative or chunked decoding) on the same caches
        if dt == tka.TKA_BF16 and 4 * w.G <= 64:
            log("[bench] four queries per sequence")
            M = 4
            qm_np = fx.encode(fx.normal(97, 0, w.B * M * w.Hq * w.d), fx.BF16).reshape(w.B, M, w.Hq, w.d)
            qm = torch.from_numpy(qm_np.view(np.int16)).view(torch.bfloat16).cuda()
            pm = tka.problem(tka.EXACT, w.B, w.Hq, w.Hkv, w.d, w.L, w.k, dt, n_queries=M)
            mq_out = torch.empty((w.B, M, w.Hq, w.d), dtype=torch.float32, device="cuda")
            mq_idx = torch.empty((w.B, M, w.Hq, w.k), dtype=torch.int32, device="cuda")
            mq_ws = torch.empty(tka.topk_decode_workspace_size(pm), dtype=torch.uint8, device="cuda")
            t_mq = time_loop(lambda: tka.topk_decode(pm, qm, Kt, Vt, out=mq_out, idx_out=mq_idx, ws=mq_ws),
                             args.steps)
            mq_sc = torch.empty(tka.score_shape(pm), dtype=torch.float32, device="cuda")
            t_mqs = time_loop(lambda: tka.topk_attn_score(pm, qm, Kt, scores=mq_sc), args.steps)
            flops = 2.0 * w.B * M * w.Hq * w.L * w.d
            sbytes = w.B * w.Hkv * w.L * w.d * 2 + w.B * M * w.Hq * w.L * 4
            extras["multi_query"] = {"queries_per_seq": M, "decode_ms": round(t_mq, 4),
                                     "query_tokens_per_s": round(w.B * M / (t_mq / 1e3), 1),
                                     "score_ms": round(t_mqs, 4),
                                     "score_tflops": round(flops / (t_mqs / 1e3) / 1e12, 2),
                                     "score_gbps": round(sbytes / (t_mqs / 1e3) / 1e9, 1)}
            del mq_ws, mq_sc
    del Kt, Vt, sc, ws
    torch.cuda.empty_cache()
    if exact and not args.no_extras and args.workload == "C3":
        # the exact variant at the other configurations' sizes: one fp32 query over 1024 keys (C1) and
        # one sequence of 32 query heads over 8 KV heads at L = 32K, k = 2048 (C2)
        for wname, key in (("C1", "exact_C1"), ("C2", "exact_C2")):
            log(f"[bench] {key}")
            extras[key] = exact_variant(fx, tka, torch, np, fx.WORKLOADS[wname], args.steps,
                                        cpu=not args.no_cpu_baseline)
            torch.cuda.empty_cache()
        # the proxy-score variants at their own workload sizes: block means (MoBA-style, top 16 blocks
        # of 64 at L = 128K) and the lightning indexer (E4M3 keys, top 2048 of L = 1M)
        for wname, key in (("C4", "block_mean_C4"), ("C5", "indexer_C5")):
            log(f"[bench] {key}")
            extras[key] = proxy_variant(fx, tka, torch, np, fx.WORKLOADS[wname], args.steps,
                                        cpu=not args.no_cpu_baseline)
            torch.cuda.empty_cache()
    result["extras"] = extras
    if args.copy_calibration:
        log("[bench] copy calibration kernel")
        copy_calibration()
    # SHA-256 of the seeded input bytes as uploaded (q, K, V in their storage dtype), hashed in place
    log("[bench] input digests")
    result["inputs_sha256"] = {n: hashlib.sha256(memoryview(np.ascontiguousarray(a)).cast("B")).hexdigest()
                               for n, a in (("q", q), ("K", K), ("V", V))}
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline (~{args.cpu_budget:.0f} s)")
        result["cpu_baseline"] = cpu_baseline(w, q, K, V, args.cpu_budget, args.cpu_single_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
