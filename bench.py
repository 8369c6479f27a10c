"""Throughput of the fused FP4 quantizer on one MI355X.

Headline step: one nvfp4_quantize call (per-token NVFP4 with Four-Over-Six
and the BF16 dequantized output) over the 8192 x 7168 BF16 MoE-activation
workload (Student-t(3) values with a log-normal per-token gain), inputs
resident in HBM.  value = algorithmic bytes per call / mean call time, in GB
(10^9 B) per second.  Buffers rotate over several input/output sets (more
than the 256 MB last-level cache) so repeated calls cannot be served from
cache.  Each measurement first spins the GPU up with 0.2 s of untimed
calls (after host-side work the clocks have dropped and the first tens of
milliseconds run several % slower), then runs the warm-up calls; the timed
calls run back to back between two HIP events on the stream the library
launches on (torch's current stream); a second pass with events around
every call gives the per-call spread.

Also reported on the same JSON line: the roofline of the dominant kernel,
a CPU baseline (the CPU oracle timed on this host), the other calls of the
path (standalone dequant, expert-weight quantize, ragged routed quantize,
MXFP4 Rollout-ResQ) and a device-copy ceiling.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import fp4_block_quantization_amd as fq  # noqa: E402
import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "quantize+dequant GB/s and % of HBM peak, 8192×7168 BF16 per-token 4/6"


def nvfp4_bytes(rows, hidden, dequant=True, groups=0):
    """Algorithmic HBM bytes of one nvfp4_quantize call: read the BF16
    input, write codes (1/2 B per element), E4M3 block scales (1/16 B per
    element), FP32 token scales, and optionally the BF16 dequant."""
    b = rows * hidden * 2 + rows * hidden // 2 + rows * hidden // 16 + rows * 4
    if dequant:
        b += rows * hidden * 2
    if groups:
        b += (groups + 1) * 8
    return b


def dequant_bytes(rows, hidden):
    return rows * hidden // 2 + rows * hidden // 16 + rows * 4 + rows * hidden * 2


def mx_bytes(rows, hidden):
    """Read BF16; write primary codes (1/2 B/el) + E8M0 (1/32), residual kept
    codes (1/4), 2:4 metadata (1/8) and residual E8M0 (1/32)."""
    n = rows * hidden
    return n * 2 + n // 2 + n // 32 + n // 4 + n // 8 + n // 32


SPINUP_S = 0.2  # untimed back-to-back calls before the warm-up


def rate(ms, nbytes):
    """Time per call (ms) and algorithmic bytes -> µs, GB/s and the fraction
    of the HBM peak."""
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"us": round(ms * 1e3, 2), "GBps": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def spin_up(fn, sets, seconds=SPINUP_S):
    """Back-to-back calls for `seconds` of wall time: after host-side work
    (workload generation, allocation) the GPU clocks have dropped, and the
    first tens of milliseconds of calls run several % slower."""
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            fn(sets[i % len(sets)])
            i += 1
        torch.cuda.synchronize()


def time_calls(fn, sets, steps, warmup, per_call=False):
    """Spin up, run `warmup` untimed calls, then time `steps` calls (fn(set)
    round-robin).  Returns (mean ms per call over the `steps` back-to-back
    calls bracketed by two HIP events on the current stream, per-call ms
    from a second pass with events around every call, or None)."""
    stream = torch.cuda.current_stream()
    spin_up(fn, sets)
    for i in range(warmup):
        fn(sets[i % len(sets)])
    torch.cuda.synchronize()
    wall0 = torch.cuda.Event(enable_timing=True)
    wall1 = torch.cuda.Event(enable_timing=True)
    wall0.record(stream)
    for i in range(steps):
        fn(sets[i % len(sets)])
    wall1.record(stream)
    torch.cuda.synchronize()
    mean = wall0.elapsed_time(wall1) / steps
    per = None
    if per_call:
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        for i in range(steps):
            starts[i].record(stream)
            fn(sets[i % len(sets)])
            ends[i].record(stream)
        torch.cuda.synchronize()
        per = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])
    return mean, per


def rotating_nvfp4_sets(x, n, dequant=True):
    rows, hidden = x.shape
    sets = []
    for i in range(n):
        xi = x if i == 0 else x.clone()
        out = (torch.empty((rows, hidden // 2), dtype=torch.uint8, device=x.device),
               torch.empty((rows, hidden // 16), dtype=torch.uint8, device=x.device),
               torch.empty((rows,), dtype=torch.float32, device=x.device),
               torch.empty_like(x) if dequant else None)
        sets.append((xi, out))
    return sets


def cpu_baseline(x_bits, rows_sample, repeats=7):
    """The CPU oracle as it stands (single-threaded C), over a bounded
    sample of the headline workload's rows; median of `repeats`."""
    import oracle
    xs = np.ascontiguousarray(x_bits[:rows_sample])
    oracle.nvfp4_quantize(xs[:8], True)  # load the library, warm caches
    times = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        oracle.nvfp4_quantize(xs, True, dequant=True)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    hidden = xs.shape[1]
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    # the same oracle function, rows split across host threads (ctypes
    # releases the GIL); reported beside the single-core figure
    from concurrent.futures import ThreadPoolExecutor
    nthr = min(16, os.cpu_count() or 1)
    bounds = [(i * len(xs) // nthr, (i + 1) * len(xs) // nthr) for i in range(nthr)]
    with ThreadPoolExecutor(nthr) as ex:
        mt = []
        for _ in range(repeats):
            t0 = time.perf_counter()
            list(ex.map(lambda ab: oracle.nvfp4_quantize(xs[ab[0]:ab[1]], True, dequant=True),
                        bounds))
            mt.append(time.perf_counter() - t0)
    tm = float(np.median(mt))
    return {"value": nvfp4_bytes(rows_sample, hidden) / t / 1e9, "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": "%d of 8192 rows x %d, per-token NVFP4 4/6 + BF16 dequant, median of %d "
                      "runs of %.2f s" % (rows_sample, hidden, repeats, t),
            "elements_per_s": rows_sample * hidden / t, "cpu_model": cpu,
            "host_threads_available": os.cpu_count(),
            "all_cores": {"value": nvfp4_bytes(rows_sample, hidden) / tm / 1e9, "unit": "GB/s",
                          "threads": nthr, "elements_per_s": rows_sample * hidden / tm}}


def _code_only(text):
    """C/C++ source without comments, blank lines or trailing blanks, so
    that an edit of comments alone leaves the digest unchanged."""
    out, i, n, quote = [], 0, len(text), None
    while i < n:
        ch = text[i]
        if quote:
            out.append(ch)
            if ch == "\\" and i + 1 < n:
                out.append(text[i + 1])
                i += 1
            elif ch == quote:
                quote = None
        elif ch in "\"'":
            quote = ch
            out.append(ch)
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
            continue
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
            continue
        else:
            out.append(ch)
        i += 1
    lines = (ln.rstrip() for ln in "".join(out).splitlines())
    return "\n".join(ln for ln in lines if ln)


def source_digest():
    """Digest of the kernel sources' code (comments excluded)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp4_block_quantization_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_record(kernel_key):
    """HBM traffic per launch from the committed rocprofv3 counter summary,
    valid only while the kernel sources are unchanged since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path)).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != source_digest():
        return None
    return rec.get("bytes_per_launch")


# Kernels of the bench run, named by what each dispatch computes.  The
# split kernel serves both full-width workloads; its smaller grid is the
# 8192-row headline call.
HEADLINE_KEY = "nvfp4_quantize_split<fos,dq> moe_act 8192x7168"


def _labels(rows):
    """Name each dispatch of a bench run by what it computes: the kernel,
    its total work-items (Grid_Size / Grid_Size_X) and, for the global-scale
    call, the reduction of the tensor-max partials that precedes its
    quantize pass."""
    out = []
    prev = ""
    for r in rows:
        name = r["Kernel_Name"]
        grid = int(r.get("Grid_Size") or r.get("Grid_Size_X"))
        lab = None
        if "nvfp4_quantize_split<1, true" in name:
            if grid == 8192 * 256:
                lab = ("nvfp4_quantize_global (quantize pass) moe_act 8192x7168"
                       if "global_amax_reduce" in prev else HEADLINE_KEY)
            elif grid == 65536 * 256:
                lab = "nvfp4_quantize_split<fos,dq> expert_weights 65536x7168"
        elif "nvfp4_quantize_split<1, false" in name and grid == 65536 // 4 * 256:
            lab = "nvfp4_quantize_split<fos> ragged_routed 65536x2048"
        elif "nvfp4_quantize_split<2, true" in name and grid == 8192 * 256:
            lab = "nvfp4_quantize_split<fp16-decision,dq> moe_act 8192x7168"
        elif "global_amax_pass" in name:
            lab = "nvfp4_quantize_global (amax pass) moe_act 8192x7168"
        elif "global_amax_reduce" in name:
            lab = "nvfp4_quantize_global (partials reduce) moe_act 8192x7168"
        elif "nvfp4_dequantize" in name:
            lab = "nvfp4_dequantize moe_act 8192x7168"
        elif "nvfp4_guided" in name:
            lab = "nvfp4_quantize_guided moe_act 8192x7168"
        elif "mxfp4_resq_units<false>" in name:
            lab = "mxfp4_resq_quantize resq_act 8192x7168"
        elif "mxfp4_resq_units<true>" in name:
            lab = "mxfp4_resq_dense_quantize resq_act 8192x7168"
        elif "mxfp4_reconstruct_units<1>" in name:
            lab = "mxfp4_resq_reconstruct (S2:4) resq_act 8192x7168"
        elif "copyBuffer" in name and grid == 131072:
            lab = "copyBuffer 256 MiB (device copy, counter calibration)"
        out.append(lab)
        prev = name
    return out


def _read_dispatches(path, counter=None):
    import csv
    rows = list(csv.DictReader(open(path)))
    if counter is not None:  # one row per dispatch and counter
        rows = [r for r in rows if r["Counter_Name"] == counter]
    rows.sort(key=lambda r: int(r.get("Dispatch_Id") or r.get("Correlation_Id") or 0))
    return rows, _labels(rows)


def summarize_profiles(trace_dir, fetch_dir, write_dir, out_dir):
    """Turn the rocprofv3 CSV output of the three profiling runs of this
    script (kernel trace, FETCH_SIZE, WRITE_SIZE) into the text summaries
    under profiles/ and the per-launch traffic table the bench reads."""
    import glob
    cmd_trace = ("rocprofv3 --kernel-trace --stats -f csv -d %s -o run -- python bench.py "
                 "--no-cpu" % trace_dir)
    cmd_pmc = ("rocprofv3 --pmc {c} -f csv -d {d} -o run -- python bench.py --steps 20 "
               "--warmup 2 --sets 2 --no-cpu")
    # kernel durations per (kernel, workload)
    trace = glob.glob(os.path.join(trace_dir, "*kernel_trace.csv"))[0]
    rows, labels = _read_dispatches(trace)
    dur = {}
    for r, lab in zip(rows, labels):
        if lab:
            dur.setdefault(lab, []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    stats = glob.glob(os.path.join(trace_dir, "*kernel_stats.csv"))[0]
    import csv
    srows = list(csv.DictReader(open(stats)))
    lines = ["# Kernel durations, bench.py default run (moe_act 8192x7168 headline + secondary "
             "calls)", "", "Command (repo root, MI355X):", "", "    " + cmd_trace, "",
             "Per kernel and workload, from the kernel trace (us):", "",
             "| kernel / workload | dispatches | mean | p10 | p50 | p90 | min | max |",
             "|---|---|---|---|---|---|---|---|"]
    for lab, d in sorted(dur.items()):
        a = np.array(d)
        lines.append("| %s | %d | %.2f | %.2f | %.2f | %.2f | %.2f | %.2f |" % (
            lab, a.size, a.mean(), np.percentile(a, 10), np.median(a), np.percentile(a, 90),
            a.min(), a.max()))
    lines += ["", "rocprofv3 --stats summary (all kernels of the run):", "",
              "| kernel | calls | total ns | average ns | % |", "|---|---|---|---|---|"]
    for r in srows[:12]:
        lines.append("| %s | %s | %s | %s | %s |" % (r["Name"][:90], r["Calls"],
                                                    r["TotalDurationNs"], r["AverageNs"],
                                                    r["Percentage"]))
    os.makedirs(out_dir, exist_ok=True)
    open(os.path.join(out_dir, "kernel_trace_bench_default.md"), "w").write("\n".join(lines) + "\n")

    # HBM bytes per dispatch, calibrated on the 256 MiB device copy
    def counter(dir_, cname):
        path = glob.glob(os.path.join(dir_, "*counter_collection.csv"))[0]
        rows, labels = _read_dispatches(path, cname)
        per = {}
        for r, lab in zip(rows, labels):
            if lab:
                per.setdefault(lab, []).append(float(r["Counter_Value"]))
        return {k: float(np.median(v)) for k, v in per.items()}
    fetch = counter(fetch_dir, "FETCH_SIZE")
    write = counter(write_dir, "WRITE_SIZE")
    copy_key = "copyBuffer 256 MiB (device copy, counter calibration)"
    copy_bytes = float(1 << 28)
    f_scale = copy_bytes / (fetch[copy_key] * 1024.0)
    w_scale = copy_bytes / (write[copy_key] * 1024.0)
    algo = {HEADLINE_KEY: (8192 * 7168 * 2, nvfp4_bytes(8192, 7168) - 8192 * 7168 * 2),
            "nvfp4_quantize_split<fos,dq> expert_weights 65536x7168":
                (65536 * 7168 * 2, nvfp4_bytes(65536, 7168) - 65536 * 7168 * 2),
            "nvfp4_quantize_split<fos> ragged_routed 65536x2048":
                (65536 * 2048 * 2 + 65 * 8, nvfp4_bytes(65536, 2048, dequant=False)
                 - 65536 * 2048 * 2),
            "nvfp4_dequantize moe_act 8192x7168":
                (8192 * 7168 // 2 + 8192 * 7168 // 16 + 8192 * 4, 8192 * 7168 * 2),
            "mxfp4_resq_quantize resq_act 8192x7168":
                (8192 * 7168 * 2, mx_bytes(8192, 7168) - 8192 * 7168 * 2),
            "mxfp4_resq_dense_quantize resq_act 8192x7168":
                (8192 * 7168 * 2, 8192 * 7168 // 2 * 2 + 8192 * 7168 // 32 * 2),
            "mxfp4_resq_reconstruct (S2:4) resq_act 8192x7168":
                (8192 * 7168 // 2 + 8192 * 7168 // 32 * 2 + 8192 * 7168 // 4 + 8192 * 7168 // 8,
                 8192 * 7168 * 4),
            "nvfp4_quantize_guided moe_act 8192x7168":
                (8192 * 7168 * 2 + 8192 * 7168 // 2 + 8192 * 7168 // 16 + 8192 * 4,
                 8192 * 7168 // 2),
            "nvfp4_quantize_split<fp16-decision,dq> moe_act 8192x7168":
                (8192 * 7168 * 2, nvfp4_bytes(8192, 7168) - 8192 * 7168 * 2),
            "nvfp4_quantize_global (amax pass) moe_act 8192x7168": (8192 * 7168 * 2, 4 * 512),
            "nvfp4_quantize_global (partials reduce) moe_act 8192x7168": (4 * 512, 4),
            "nvfp4_quantize_global (quantize pass) moe_act 8192x7168":
                (8192 * 7168 * 2 + 4, nvfp4_bytes(8192, 7168) - 8192 * 7168 * 2 - 8192 * 4),
            copy_key: (copy_bytes, copy_bytes)}
    digest = source_digest()
    table = {}
    lines = ["# HBM traffic per dispatch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
             "Commands (repo root, MI355X), one counter per run:", "",
             "    " + cmd_pmc.format(c="FETCH_SIZE", d=fetch_dir),
             "    " + cmd_pmc.format(c="WRITE_SIZE", d=write_dir), "",
             "Both counters are in KiB per dispatch.  Calibration on the runtime's device copy "
             "of 256 MiB (268435456 B read, 268435456 B written): FETCH_SIZE reads %.0f KiB "
             "(scale x%.4f), WRITE_SIZE reads %.0f KiB (scale x%.4f).  Median over dispatches; "
             "kernel sources digest %s." % (fetch[copy_key], f_scale, write[copy_key], w_scale,
                                            digest), "",
             "| kernel / workload | read B (scaled) | algorithmic read B | ratio | write B (scaled) "
             "| algorithmic write B | ratio |", "|---|---|---|---|---|---|---|"]
    for lab in sorted(fetch):
        if lab not in write or lab not in algo:
            continue
        rd, wr = fetch[lab] * 1024.0 * f_scale, write[lab] * 1024.0 * w_scale
        ar, aw = algo[lab]
        lines.append("| %s | %.0f | %.0f | %.3f | %.0f | %.0f | %.3f |" % (
            lab, rd, ar, rd / ar, wr, aw, wr / aw))
        table[lab] = {"bytes_per_launch": round(rd + wr), "read_bytes": round(rd),
                      "write_bytes": round(wr), "source_digest": digest,
                      "fetch_scale": f_scale, "write_scale": w_scale}
    open(os.path.join(out_dir, "hbm_traffic_bench.md"), "w").write("\n".join(lines) + "\n")
    json.dump(table, open(os.path.join(out_dir, "traffic.json"), "w"), indent=1, sort_keys=True)
    print("\n".join(lines))


SQ_COUNTERS = ("GRBM_GUI_ACTIVE SQ_WAVES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_INSTS_SALU "
               "SQ_INSTS_LDS SQ_WAVE_CYCLES SQ_BUSY_CYCLES")
N_SIMDS = 256 * 4  # MI355X: 256 compute units of 4 SIMDs
N_XCDS = 8
PEAK_CLOCK_HZ = 2.4e9


def summarize_sq(sq_dir, out_dir):
    """Instruction mix and VALU occupancy per kernel from one rocprofv3
    --pmc run of SQ_COUNTERS over this script: instructions per wave, issue
    cycles per VALU instruction (SQ_ACTIVE_INST_VALU counts in units of 4
    cycles), and the share of the SIMDs' cycles spent issuing VALU work --
    once against GRBM_GUI_ACTIVE (reported summed over the XCDs, so divided
    by their number) and once against the dispatch's own duration at the
    2.4 GHz peak clock."""
    import glob
    path = glob.glob(os.path.join(sq_dir, "*counter_collection.csv"))[0]
    per = {}
    for cname in SQ_COUNTERS.split():
        rows, labels = _read_dispatches(path, cname)
        for r, lab in zip(rows, labels):
            if lab:
                d = per.setdefault(lab, {}).setdefault(cname, [])
                d.append((float(r["Counter_Value"]),
                          (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9))
    cmd = ("rocprofv3 --pmc %s -f csv -d %s -o run -- python bench.py --steps 20 --warmup 2 "
           "--sets 2 --no-cpu" % (SQ_COUNTERS, sq_dir))
    lines = ["# SQ instruction counters per dispatch (rocprofv3 --pmc)", "",
             "Command (repo root, MI355X), one run:", "", "    " + cmd, "",
             "Medians over the dispatches of each kernel (the counter run serializes "
             "dispatches).  Cycles per VALU instruction = 4 SQ_ACTIVE_INST_VALU / "
             "SQ_INSTS_VALU.  VALU busy = 4 SQ_ACTIVE_INST_VALU / (%d SIMDs x cycles), with "
             "cycles = GRBM_GUI_ACTIVE / %d (the counter is summed over the XCDs), or = the "
             "dispatch time x 2.4 GHz." % (N_SIMDS, N_XCDS), "",
             "| kernel / workload | waves | VALU instr / wave | SALU / wave | LDS / wave | "
             "cycles / VALU instr | VALU busy (GRBM) | VALU busy (time x 2.4 GHz) |",
             "|---|---|---|---|---|---|---|---|"]
    for lab in sorted(per):
        c = {k: np.median([v for v, _ in per[lab][k]]) for k in per[lab]}
        t = np.median([d for _, d in per[lab]["SQ_INSTS_VALU"]])
        waves = c["SQ_WAVES"]
        valu_cycles = 4 * c["SQ_ACTIVE_INST_VALU"] / N_SIMDS
        lines.append("| %s | %.0f | %.1f | %.1f | %.1f | %.2f | %.1f%% | %.1f%% |" % (
            lab, waves, c["SQ_INSTS_VALU"] / waves, c["SQ_INSTS_SALU"] / waves,
            c["SQ_INSTS_LDS"] / waves, 4 * c["SQ_ACTIVE_INST_VALU"] / c["SQ_INSTS_VALU"],
            100 * valu_cycles / (c["GRBM_GUI_ACTIVE"] / N_XCDS),
            100 * valu_cycles / (t * PEAK_CLOCK_HZ)))
    os.makedirs(out_dir, exist_ok=True)
    open(os.path.join(out_dir, "sq_counters_bench.md"), "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def size_sweep(x, dev):
    """Time per call against the row count for the headline quantize
    (4/6 + dequant), the standalone dequant, MXFP4 Rollout-ResQ and a device
    copy of the input, on rows of moe_act (tiled past 8192 rows).  Every
    size rotates over enough buffer sets to span about 1 GiB, so that no
    size is served by the last-level cache and all see a similar footprint.
    A fit of time = fixed + rows * per_row separates the per-launch cost
    from the steady-state rate."""
    out = {}
    hidden = x.shape[1]
    for rows in (1024, 2048, 4096, 8192, 16384, 32768):
        reps = (rows + x.shape[0] - 1) // x.shape[0]
        xr = x.repeat(reps, 1)[:rows].contiguous()
        nsets = max(1, min(32, -(-(1 << 30) // nvfp4_bytes(rows, hidden))))
        sets = rotating_nvfp4_sets(xr, nsets)
        mx = [fq.mxfp4_resq_quantize(s[0]) for s in sets]
        steps = max(100, 400 * 8192 // rows)
        t = {}
        t["nvfp4_quantize"], _ = time_calls(
            lambda s: fq.nvfp4_quantize(s[0], True, out=s[1]), sets, steps, steps // 4)
        t["nvfp4_dequantize"], _ = time_calls(
            lambda s: fq.nvfp4_dequantize(s[1][0], s[1][1], s[1][2], out=s[1][3]), sets, steps,
            steps // 4)
        t["mxfp4_resq_quantize"], _ = time_calls(
            lambda i: fq.mxfp4_resq_quantize(sets[i][0], out=mx[i]), list(range(nsets)), steps,
            steps // 4)
        t["device_copy"], _ = time_calls(lambda s: s[1][3].copy_(s[0]), sets, steps, steps // 4)
        out[rows] = {k: round(v * 1e3, 3) for k, v in t.items()}
        out[rows]["sets"] = nsets
        print("[bench] sweep rows %d: %s" % (rows, json.dumps(out[rows])), file=sys.stderr,
              flush=True)
        del sets, mx, xr
        torch.cuda.empty_cache()
    fit = {}
    r = np.array(sorted(out), dtype=np.float64)
    for k in ("nvfp4_quantize", "nvfp4_dequantize", "mxfp4_resq_quantize", "device_copy"):
        us = np.array([out[int(v)][k] for v in r])
        big = r >= 4096  # the linear regime: several waves of workgroups per CU
        per_row, fixed = np.polyfit(r[big], us[big], 1)
        fit[k] = {"fixed_us": round(float(fixed), 2), "ns_per_row": round(float(per_row) * 1e3, 3)}
    return {"hidden": hidden, "us_per_call": out, "linear_fit_rows_ge_4096": fit}


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-sq":
        # python bench.py --summarize-sq SQ_DIR
        summarize_sq(sys.argv[2], os.path.join(ROOT, "profiles"))
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-profiles":
        # python bench.py --summarize-profiles TRACE_DIR FETCH_DIR WRITE_DIR
        summarize_profiles(*sys.argv[2:5], os.path.join(ROOT, "profiles"))
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--sets", type=int, default=6, help="rotating buffer sets")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--parts",
                    default="copy,dequant,resq,resq_dense,trace,global,ragged,weights,fp16",
                    help="secondary measurements to run (comma list)")
    ap.add_argument("--cpu-rows", type=int, default=8192)
    ap.add_argument("--sweep", action="store_true",
                    help="print only a row-count sweep (time per call vs rows) as JSON")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: the quantizer is row-local and needs no "
              "communication, so a multi-GPU figure is not produced (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    fq.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t0 = time.time()
    x_bits = workloads.rows("moe_act")
    rows, hidden = x_bits.shape
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    print("[bench] generated moe_act %dx%d in %.1f s" % (rows, hidden, time.time() - t0),
          file=sys.stderr, flush=True)

    if args.sweep:
        print(json.dumps(size_sweep(x, dev)), flush=True)
        return

    sets = rotating_nvfp4_sets(x, args.sets)
    ms, per = time_calls(lambda s: fq.nvfp4_quantize(s[0], True, out=s[1]), sets, args.steps,
                         args.warmup, per_call=True)
    nbytes = nvfp4_bytes(rows, hidden)
    gbs = nbytes / (ms * 1e-3) / 1e9
    print("[bench] nvfp4_quantize moe_act: %.2f us per call back to back, %.0f GB/s; per-call "
          "events p10 %.2f p50 %.2f p90 %.2f us" % (
              ms * 1e3, gbs, np.percentile(per, 10) * 1e3, np.median(per) * 1e3,
              np.percentile(per, 90) * 1e3), file=sys.stderr, flush=True)

    key = HEADLINE_KEY
    traffic = traffic_record(key)
    roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": nbytes,
                "kernel": key, "launch_us_mean": round(ms * 1e3, 3),
                "launch_us_p50_per_call_events": round(float(np.median(per)) * 1e3, 3)}
    del sets
    torch.cuda.empty_cache()

    secondary = {}
    parts = set() if args.no_secondary else set(args.parts.split(","))
    if "copy" in parts:
        # device copy ceiling (a plain copy kernel of 2 x 256 MiB traffic);
        # also the calibration kernel for the HBM byte counters
        src = torch.empty(1 << 28, dtype=torch.uint8, device=dev)
        dsts = [torch.empty_like(src) for _ in range(3)]
        p, _ = time_calls(lambda d: d.copy_(src), dsts, 100, 10)
        secondary["device_copy_GBps"] = round(2 * src.numel() / (p * 1e-3) / 1e9, 1)
        del src, dsts
    if "dequant" in parts:
        # standalone dequant on the headline shape
        c, s_, ts, _ = fq.nvfp4_quantize(x, True, dequant=False)
        dsets = [(c.clone(), s_.clone(), ts.clone(), torch.empty_like(x)) for _ in range(4)]
        p, _ = time_calls(lambda d: fq.nvfp4_dequantize(d[0], d[1], d[2], out=d[3]), dsets, 200, 20)
        b = dequant_bytes(rows, hidden)
        secondary["nvfp4_dequantize moe_act 8192x7168"] = {
            **rate(p, b)}
        del dsets, c, s_, ts
        torch.cuda.empty_cache()
    if "resq" in parts:
        # MXFP4 Rollout-ResQ
        xr = workloads.tensor("resq_act", dev)
        msets = [xr] + [xr.clone() for _ in range(3)]
        mouts = [fq.mxfp4_resq_quantize(m) for m in msets]
        p, _ = time_calls(lambda i: fq.mxfp4_resq_quantize(msets[i], out=mouts[i]),
                          list(range(4)), 200, 20)
        b = mx_bytes(*xr.shape)
        secondary["mxfp4_resq_quantize resq_act 8192x7168"] = {
            **rate(p, b)}
        del msets, mouts, xr
        torch.cuda.empty_cache()
    if "resq_dense" in parts:
        # Rollout-ResQ-Dense and the reconstruction error of the three
        # variants on the resq_act workload (MSE over all elements, FP64)
        xr = workloads.tensor("resq_act", dev)
        msets = [xr] + [xr.clone() for _ in range(3)]
        douts = [fq.mxfp4_resq_dense_quantize(m) for m in msets]
        p, _ = time_calls(lambda i: fq.mxfp4_resq_dense_quantize(msets[i], out=douts[i]),
                          list(range(4)), 200, 20)
        r_, h_ = xr.shape
        b = r_ * h_ * 2 + r_ * h_ // 2 * 2 + r_ * h_ // 32 * 2
        secondary["mxfp4_resq_dense_quantize resq_act 8192x7168"] = {
            **rate(p, b)}
        sp = fq.mxfp4_resq_quantize(xr)
        de = douts[0]
        xf = xr.float().double()
        mse = {}
        recon = {"primary only": (sp[0], sp[1], None, None, None, 0),
                 "primary + S2:4 residual": (sp[0], sp[1], sp[2], sp[3], sp[4], 1),
                 "primary + dense residual": (de[0], de[1], de[2], None, de[3], 2)}
        xh = torch.empty((r_, h_), dtype=torch.float32, device=dev)
        for name, a in recon.items():
            fq.mxfp4_resq_reconstruct(*a[:5], residual=a[5], out=xh)
            err = (xf - xh.double())
            mse[name] = {"mse": float((err * err).mean()),
                         "rel_mse": float((err * err).sum() / (xf * xf).sum())}
        p, _ = time_calls(lambda i: fq.mxfp4_resq_reconstruct(
            sp[0], sp[1], sp[2], sp[3], sp[4], residual=1, out=xh), [0], 200, 20)
        b = r_ * h_ // 2 + r_ * h_ // 32 * 2 + r_ * h_ // 4 + r_ * h_ // 8 + r_ * h_ * 4
        secondary["mxfp4_resq_reconstruct (S2:4) resq_act 8192x7168"] = {
            **rate(p, b)}
        secondary["Rollout-ResQ reconstruction error resq_act"] = mse
        del msets, douts, sp, de, xf, xh, xr
        torch.cuda.empty_cache()
    if "trace" in parts:
        # TRACE rollout-guided rounding: the rollout quantizes moe_act; the
        # training side holds the same values perturbed by ~1 BF16 step
        # (relative N(0, 2^-8)).  Elementwise code mismatches with the
        # rollout: the training side quantizing on its own (round to
        # nearest, its own scales), and guided by the rollout's codes under
        # the rollout's scales; plus the share of the independent mismatches
        # that land on adjacent codewords.
        xt = torch.from_numpy(workloads.perturbed(x_bits, seed=2).view(np.int16)).view(
            torch.bfloat16).to(dev)
        rc, rs, rt, _ = fq.nvfp4_quantize(x, True, dequant=False)
        gsets = [(xt, (torch.empty_like(rc), None)) for _ in range(2)]
        p, _ = time_calls(lambda s_: fq.nvfp4_quantize_guided(s_[0], rc, rs, rt, dequant=False,
                                                              out=s_[1]), gsets, 500, 50)
        b = rows * hidden * 2 + rows * hidden // 2 * 2 + rows * hidden // 16 + rows * 4
        secondary["nvfp4_quantize_guided moe_act 8192x7168 (no dequant)"] = {
            **rate(p, b)}

        def nib(c):
            return torch.stack([c & 15, c >> 4], -1).reshape(c.shape[0], -1)
        own = nib(fq.nvfp4_quantize(xt, True, dequant=False)[0])
        guided = nib(fq.nvfp4_quantize_guided(xt, rc, rs, rt, dequant=False)[0])
        ref = nib(rc)
        mis_own = own != ref
        mag_own, mag_ref = (own & 7).int(), (ref & 7).int()
        adjacent = mis_own & ((own >> 3) == (ref >> 3)) & ((mag_own - mag_ref).abs() == 1)
        n_el = ref.numel()
        secondary["TRACE guided rounding moe_act (training = rollout x (1 + 2^-8 N(0,1)))"] = {
            "elements": n_el,
            "mismatch_frac_independent_rne": round(float(mis_own.sum()) / n_el, 7),
            "mismatch_frac_guided": round(float((guided != ref).sum()) / n_el, 7),
            "adjacent_share_of_independent_mismatches":
                round(float(adjacent.sum()) / max(1, int(mis_own.sum())), 5)}
        del xt, rc, rs, rt, gsets, own, guided, ref, mis_own, adjacent
        torch.cuda.empty_cache()
    if "global" in parts:
        # the naive one-scale-per-tensor NVFP4: speed, and the batch
        # dependency -- the blocks of each 1024-row slice that change when
        # the slice is quantized on its own instead of in the full tensor
        gsets = rotating_nvfp4_sets(x, args.sets)
        outs = [(s_[1][0], s_[1][1], torch.empty(1, dtype=torch.float32, device=dev), s_[1][3])
                for s_ in gsets]
        p, _ = time_calls(lambda i: fq.nvfp4_quantize_global(gsets[i][0], True, out=outs[i]),
                          list(range(len(gsets))), 500, 50)
        secondary["nvfp4_quantize_global moe_act 8192x7168 (amax pass + quantize)"] = {
            **rate(p, nbytes)}
        del gsets, outs
        torch.cuda.empty_cache()
        full = fq.nvfp4_quantize_global(x, True, dequant=False)
        pt_full = fq.nvfp4_quantize(x, True, dequant=False)
        changed = pt_changed = 0
        for r0 in range(0, rows, 1024):
            part = fq.nvfp4_quantize_global(x[r0:r0 + 1024], True, dequant=False)
            same = (part[1] == full[1][r0:r0 + 1024]) & (
                part[0].view(-1, hidden // 16, 8) == full[0][r0:r0 + 1024].view(-1, hidden // 16, 8)).all(-1)
            changed += int((~same).sum())
            pp = fq.nvfp4_quantize(x[r0:r0 + 1024], True, dequant=False)
            pt_changed += int((pp[0] != pt_full[0][r0:r0 + 1024]).sum() + (pp[1] != pt_full[1][r0:r0 + 1024]).sum())
        secondary["batch dependency moe_act (8 slices of 1024 rows vs the whole tensor)"] = {
            "global_scale_blocks_changed_frac": round(changed / (rows * hidden // 16), 6),
            "per_token_bytes_changed": pt_changed}
        del full, pt_full
        torch.cuda.empty_cache()
    if "ragged" in parts:
        # ragged routed, quantize only
        xg = workloads.tensor("ragged_routed", dev)
        offs = torch.from_numpy(workloads.group_offsets()).to(dev)
        gsets = rotating_nvfp4_sets(xg, 2, dequant=False)
        p, _ = time_calls(lambda s: fq.nvfp4_quantize(s[0], True, offsets=offs, out=s[1]),
                          gsets, 200, 20)
        b = nvfp4_bytes(*xg.shape, dequant=False, groups=offs.numel() - 1)
        secondary["nvfp4_quantize ragged_routed 65536x2048 (64 groups, no dequant)"] = {
            **rate(p, b)}
        del gsets, xg
        torch.cuda.empty_cache()
    if "weights" in parts:
        # expert weights, 32 x 2048 x 7168
        xw = workloads.tensor("expert_weights", dev)
        wsets = rotating_nvfp4_sets(xw, 1)
        p, _ = time_calls(lambda s: fq.nvfp4_quantize(s[0], True, out=s[1]), wsets, 50, 5)
        b = nvfp4_bytes(*xw.shape)
        secondary["nvfp4_quantize expert_weights 65536x7168"] = {
            **rate(p, b)}
        del wsets, xw
        torch.cuda.empty_cache()
    if "fp16" in parts:
        # the FP16 fast path's 4/6 decision (four_over_six = 2): speed on the
        # headline shape, and how often its choice equals the FP32 one
        fsets = rotating_nvfp4_sets(x, args.sets)
        p, _ = time_calls(lambda s: fq.nvfp4_quantize(s[0], 2, out=s[1]), fsets, 1000, 100)
        secondary["nvfp4_quantize fp16-decision moe_act 8192x7168"] = {
            **rate(p, nbytes)}
        del fsets
        torch.cuda.empty_cache()
        agree = {}
        for name in ("tiny_ref", "moe_act", "expert_weights"):
            xa = x if name == "moe_act" else workloads.tensor(name, dev)
            c1, s1, _, _ = fq.nvfp4_quantize(xa, 1, dequant=False)
            c2, s2, _, _ = fq.nvfp4_quantize(xa, 2, dequant=False)
            r, h = xa.shape
            same = (s1 == s2) & (c1.view(r, h // 16, 8) == c2.view(r, h // 16, 8)).all(-1)
            agree[name] = {"blocks": same.numel(),
                           "same_choice_frac": round(float(same.float().mean()), 7)}
            del xa, c1, s1, c2, s2, same
            torch.cuda.empty_cache()
        secondary["fp16-decision agreement with the FP32 choice"] = agree
    if secondary:
        print("[bench] secondary: %s" % json.dumps(secondary), file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(x_bits, min(args.cpu_rows, rows))
        print("[bench] cpu oracle: %.3f GB/s (%s)" % (cpu["value"], cpu["sample"]),
              file=sys.stderr, flush=True)

    line = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "moe_act: 8192x7168 BF16 MoE expert input activations, "
                               "Student-t(3) x per-token LogNormal(0,0.5); per-token NVFP4 "
                               "Four-Over-Six + BF16 dequant", "rows": rows, "hidden": hidden,
                   "four_over_six": True, "dequant": True, "rotating_sets": args.sets,
                   "input_sha256": hashlib.sha256(x_bits.tobytes()).hexdigest()},
        "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
        "elements_per_s": rows * hidden / (ms * 1e-3),
        "roofline": roofline, "cpu_baseline": cpu, "secondary": secondary,
        "spinup_s_before_warmup": SPINUP_S,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
