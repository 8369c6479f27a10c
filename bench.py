"""Throughput of the fused FP4 quantizer on one MI355X.

Headline step: one nvfp4_quantize call (per-token NVFP4 with Four-Over-Six
and the BF16 dequantized output) over the 8192 x 7168 BF16 MoE-activation
workload (Student-t(3) values with a log-normal per-token gain), inputs
resident in HBM.  value = algorithmic bytes per call / mean call time, in GB
(10^9 B) per second.  Buffers rotate over several input/output sets (more
than the 256 MB last-level cache) so repeated calls cannot be served from
cache.  Each measurement first spins the GPU up with 0.2 s of untimed
calls (after host-side work the clocks have dropped and the first tens of
milliseconds run several % slower), then runs the warm-up calls, the last
three of them queued after a synchronize and ahead of the start event (so
that the event does not time the host's issue of the first timed call); the
timed calls run back to back between two HIP events on the stream the
library launches on (torch's current stream); a second pass with events
around every call gives the per-call spread.

Also reported on the same JSON line: the roofline of the dominant kernel,
a CPU baseline (the CPU oracle timed on this host), and under "secondary"
every other call of the path, each on at least four distinct rotating
input/output sets spanning at least 1 GiB (the sets and the working set are
listed with each figure), the K0 HBM probes (copy, read and write
ceilings in the quantizer's access pattern) and the memory-pattern
stand-ins of the NVFP4 and MXFP4-ResQ kernels (their loads and stores
without the per-block arithmetic).

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
       python bench.py --sweep       (time per call against the row count)
"""
import argparse
import ctypes
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
from fp4_block_quantization_amd import _build  # noqa: E402
import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "quantize+dequant GB/s and % of HBM peak, 8192×7168 BF16 per-token 4/6"
GIB = 1 << 30


# ------------------------------------------------------ algorithmic bytes --

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


def mx_dense_bytes(rows, hidden):
    n = rows * hidden
    return n * 2 + n // 2 * 2 + n // 32 * 2


def reconstruct_bytes(rows, hidden):
    """S2:4 reconstruction: read primary codes and scales, kept residual
    codes, metadata and residual scales; write FP32."""
    n = rows * hidden
    return n // 2 + n // 32 * 2 + n // 4 + n // 8 + n * 4


def guided_bytes(rows, hidden, guide=True, dequant=False):
    """Read x, the guide codes (if any), the rollout's block and token
    scales; write the codes (and the dequant)."""
    n = rows * hidden
    b = n * 2 + n // 16 + rows * 4 + n // 2
    if guide:
        b += n // 2
    if dequant:
        b += n * 2
    return b


# --------------------------------------------------------------- timing --

SPINUP_S = 0.2  # untimed back-to-back calls before the warm-up
QUEUED_WARMUP = 3  # warm-up calls queued ahead of the start event (time_calls)


def rate(ms, nbytes, elements=None):
    """Time per call (ms), algorithmic bytes and elements -> µs, GB/s,
    elements/s and the fraction of the HBM peak."""
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {"us": round(ms * 1e3, 2), "GBps": round(gbs, 1),
           "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    if elements is not None:
        out["elements_per_s"] = float("%.4g" % (elements / (ms * 1e-3)))
    return out


def spin_up(fn, sets, seconds=None):
    """Back-to-back calls for `seconds` of wall time: after host-side work
    (workload generation, allocation) the GPU clocks have dropped, and the
    first tens of milliseconds of calls run several % slower."""
    seconds = SPINUP_S if seconds is None else seconds
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            fn(sets[i % len(sets)])
            i += 1
        torch.cuda.synchronize()


def time_calls(fn, sets, steps, warmup, per_call=False):
    """Spin up, run `warmup` untimed calls, then time `steps` calls (fn(set)
    round-robin, continuing the warm-up's rotation).  Returns (mean ms per
    call over the `steps` back-to-back calls bracketed by two HIP events on
    the current stream, per-call ms from a second pass with events around
    every call, or None).

    The last QUEUED_WARMUP warm-up calls are queued after the synchronize,
    ahead of the start event: the GPU then reaches that event with the first
    timed call already queued behind it.  Recorded on an idle GPU, the start
    event would also time the host's latency of issuing the first call
    (about 6 us, +0.31 us per call over 20 calls)."""
    stream = torch.cuda.current_stream()
    spin_up(fn, sets)
    n = len(sets)
    queued = min(QUEUED_WARMUP, warmup)
    for i in range(warmup - queued):
        fn(sets[i % n])
    torch.cuda.synchronize()
    for i in range(warmup - queued, warmup):
        fn(sets[i % n])
    wall0 = torch.cuda.Event(enable_timing=True)
    wall1 = torch.cuda.Event(enable_timing=True)
    wall0.record(stream)
    for i in range(steps):
        fn(sets[(warmup + i) % n])
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


def n_sets(bytes_per_set, min_sets=4, min_total=GIB, cap=512):
    """Rotating sets: at least min_sets, and enough to span min_total bytes
    (four times the 256 MB last-level cache)."""
    return int(min(cap, max(min_sets, -(-min_total // max(1, bytes_per_set)))))


def tensors_of(obj):
    if isinstance(obj, torch.Tensor):
        return [obj]
    if isinstance(obj, (list, tuple)):
        return [t for o in obj for t in tensors_of(o)]
    if isinstance(obj, dict):
        return [t for o in obj.values() for t in tensors_of(o)]
    return []


def working_set(sets):
    """Bytes of the distinct tensors the rotating sets hold."""
    seen = {}
    for t in tensors_of(sets):
        seen[(t.data_ptr(), t.numel())] = t.numel() * t.element_size()
    return sum(seen.values())


def measure(fn, sets, nbytes, elements, steps, warmup=None):
    """One secondary figure: time per call over the rotating sets, with the
    set count and working set."""
    steps = max(steps, 2 * len(sets))
    ms, _ = time_calls(fn, sets, steps, steps // 10 if warmup is None else warmup)
    r = rate(ms, nbytes, elements)
    r.update({"sets": len(sets), "working_set_bytes": working_set(sets), "calls": steps})
    return r


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def stream_ptr():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def membench():
    """K0: libfp4q_membench.so (include/fp4q_membench.h)."""
    if not os.path.exists(_build.MEMBENCH_PATH):
        raise RuntimeError("libfp4q_membench.so is not built: run __graft_entry__.build()")
    M = ctypes.CDLL(_build.MEMBENCH_PATH)
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    M.fp4q_k0_copy.argtypes = [vp, vp, i64, ci, vp]
    M.fp4q_k0_read.argtypes = [vp, i64, ci, ci, vp, vp]
    M.fp4q_k0_write.argtypes = [vp, i64, ci, vp]
    M.fp4q_k0_mix.argtypes = [vp, vp, i64, ci, ci, vp]
    return M


def standin():
    """The memory-pattern stand-in build of the quantizer (same C ABI,
    per-block arithmetic compiled out; measurement only)."""
    if not os.path.exists(_build.STANDIN_PATH):
        raise RuntimeError("libfp4q_standin.so is not built: run __graft_entry__.build()")
    return fq.declare(ctypes.CDLL(_build.STANDIN_PATH))


def exactdecision():
    """The quantizer built to decide every 4/6 block from both exactly
    computed errors (no certified margin; same results; measurement only)."""
    if not os.path.exists(_build.EXACTDECISION_PATH):
        raise RuntimeError("libfp4q_exactdecision.so is not built: run __graft_entry__.build()")
    return fq.declare(ctypes.CDLL(_build.EXACTDECISION_PATH))


def _ok(status, what):
    if status != 0:
        raise RuntimeError("%s returned status %d" % (what, status))


def rotating_nvfp4_sets(x, n, dequant=True):
    """n input/output sets: x and n - 1 copies, each with its own outputs."""
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


def nvfp4_via(S, s, offs=None, fos=1):
    """nvfp4_quantize of another build of the library (stand-in or exact
    decision) on a rotating set (x, outputs)."""
    x, (c, sc, ts, dq) = s
    ng = 0 if offs is None else offs.numel() - 1
    _ok(S.nvfp4_quantize(ptr(x), x.shape[0], x.shape[1], ptr(offs), ng, fos, ptr(c), ptr(sc),
                         ptr(ts), ptr(dq), stream_ptr()), "nvfp4_quantize of a measurement build")


# ------------------------------------------------------------ CPU baseline --

def host_cpu():
    """CPU model, logical CPUs and physical cores the host reports, and the
    CPUs this process may run on.  A virtual machine may show a generic
    model name; the CPUID family/model/stepping and the widest vector
    extensions then still place the CPU's generation."""
    model, phys = "unknown", set()
    cpuid, vec = None, []
    cur = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" not in line:
                if cur:
                    phys.add((cur.get("physical id"), cur.get("core id")))
                cur = {}
                continue
            k, v = [t.strip() for t in line.split(":", 1)]
            cur[k] = v
            if k == "model name" and model == "unknown":
                model = v
            if k == "stepping" and cpuid is None:
                cpuid = "family %s model %s stepping %s" % (cur.get("cpu family"),
                                                              cur.get("model"), v)
            if k == "flags" and not vec:
                f = set(v.split())
                vec = [e for e in ("avx2", "avx512f", "avx512_bf16", "avx512_vnni") if e in f]
        if cur:
            phys.add((cur.get("physical id"), cur.get("core id")))
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu_model": model, "cpuid": cpuid, "vector_extensions": vec,
            "host_logical_cpus": os.cpu_count(),
            "host_physical_cores": len(phys) if phys and None not in next(iter(phys)) else None,
            "cpus_usable_by_this_process": usable}


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
    cpu = host_cpu()
    # the same oracle function, rows split across host threads (ctypes
    # releases the GIL); reported beside the single-core figure
    from concurrent.futures import ThreadPoolExecutor
    nthr = max(1, min(16, cpu["cpus_usable_by_this_process"] or 1))
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
            "elements_per_s": rows_sample * hidden / t, **cpu,
            "all_cores": {"value": nvfp4_bytes(rows_sample, hidden) / tm / 1e9, "unit": "GB/s",
                          "threads": nthr, "elements_per_s": rows_sample * hidden / tm}}


# ------------------------------------------------- profile summaries --

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


# Kernels of the bench run, named by what each dispatch computes.
HEADLINE_KEY = "nvfp4_quantize_split<fos,dq> moe_act 8192x7168"
DQ_KEY = "nvfp4_dequantize moe_act 8192x7168"
DQ_PACKED_KEY = "nvfp4_dequantize moe_act 8192x7168 (one allocation per kind)"
COPY_CAL_KEY = "K0 copy nt 256 MiB (counter calibration)"
R, H, RG, HG = 8192, 7168, 65536, 2048


def _label(name, grid):
    """Name one dispatch (kernel name, total work-items) of a bench run."""
    standin = "fp4q_standin" in name
    if "fp4q_exactdecision" in name:
        if "nvfp4_quantize_split<1, true, 2, false>" in name and grid == R * 256:
            return "exact-error decision nvfp4_quantize_split<fos,dq> moe_act 8192x7168"
        if "nvfp4_quantize_split<1, false, 2, false>" in name and grid == RG * 64:
            return "exact-error decision nvfp4_quantize_split<fos> ragged_routed 65536x2048"
        return None
    if "k0_copy<1>" in name:
        return COPY_CAL_KEY
    if "k0_copy<0>" in name:
        return "K0 copy 256 MiB"
    if "k0_copy<2>" in name:
        return "K0 copy nt sc1 256 MiB"
    if "k0_mix<" in name:
        import re
        m = re.search(r"k0_mix<(\d), (\d)>", name)
        return None if not m else "K0 mix read 4 KiB, write 4/%s KiB%s 256 MiB" % (
            m.group(1), ("", " nt", " nt sc1")[int(m.group(2))])
    if "k0_write<1>" in name:
        return "K0 write nt 256 MiB"
    if "k0_write<2>" in name:
        return "K0 write nt sc1 256 MiB"
    if "k0_read<" in name:
        import re
        m = re.search(r"k0_read<(.+?),\s*(true|false)>", name)
        if not m:
            return None
        t = m.group(1)
        w = 16 if "(4)" in t or "[4]" in t else 8 if "(2)" in t or "[2]" in t else \
            1 if "char" in t else 2 if "short" in t else 4
        return "K0 read %dB%s 256 MiB" % (w, " nt" if m.group(2) == "true" else "")
    if standin:
        if "nvfp4_quantize_split<1, true" in name and grid == R * 256:
            return "stand-in nvfp4_quantize_split<fos,dq> moe_act 8192x7168"
        if "nvfp4_quantize_split<1, false" in name and grid == RG * 64:
            return "stand-in nvfp4_quantize_split<fos> ragged_routed 65536x2048"
        if "mxfp4_resq_units<false>" in name:
            return "stand-in mxfp4_resq_quantize resq_act 8192x7168"
        return None
    if "nvfp4_quantize_split<1, true, 2, true>" in name and grid == R * 256:
        return "nvfp4_quantize_global (quantize pass) moe_act 8192x7168"
    if "nvfp4_quantize_split<1, true, 2, false>" in name:
        if grid == R * 256:
            return HEADLINE_KEY
        if grid == RG * 256:
            return "nvfp4_quantize_split<fos,dq> expert_weights 65536x7168"
        if grid == 256 * 64:
            return "nvfp4_quantize_split<fos,dq> tiny_ref 256x2048"
    if "nvfp4_quantize_split<0, true, 2, false>" in name and grid == 256 * 64:
        return "nvfp4_quantize_split<6-only,dq> tiny_ref 256x2048"
    if "nvfp4_quantize_split<1, false, 2, false>" in name and grid == RG * 64:
        return "nvfp4_quantize_split<fos> ragged_routed 65536x2048"
    if "nvfp4_quantize_split<2, true, 2, false>" in name and grid == R * 256:
        return "nvfp4_quantize_split<fp16-decision,dq> moe_act 8192x7168"
    if "nvfp4_quantize_split<2, false, 2, false>" in name and grid == RG * 64:
        return "nvfp4_quantize_split<fp16-decision> ragged_routed 65536x2048"
    if "global_amax_pass" in name:
        return "nvfp4_quantize_global (amax pass) moe_act 8192x7168"
    if "nvfp4_dequantize" in name:
        return DQ_KEY
    if "nvfp4_guided_units<false, false>" in name:
        return "nvfp4_quantize_guided moe_act 8192x7168"
    if "nvfp4_guided_units<true, false>" in name:
        return "nvfp4_quantize_guided (no guide: nearest) moe_act 8192x7168"
    if "mxfp4_resq_units<false>" in name:
        return "mxfp4_resq_quantize resq_act 8192x7168"
    if "mxfp4_resq_units<true>" in name:
        return "mxfp4_resq_dense_quantize resq_act 8192x7168"
    if "mxfp4_reconstruct_units<1>" in name:
        return "mxfp4_resq_reconstruct (S2:4) resq_act 8192x7168"
    return None


def _read_dispatches(path, counter=None):
    import csv
    rows = list(csv.DictReader(open(path)))
    if counter is not None:  # one row per dispatch and counter
        rows = [r for r in rows if r["Counter_Name"] == counter]
    rows.sort(key=lambda r: int(r.get("Dispatch_Id") or r.get("Correlation_Id") or 0))
    return rows, [_label(r["Kernel_Name"], int(r.get("Grid_Size") or r.get("Grid_Size_X")))
                  for r in rows]


def algorithmic_rw():
    """(read, write) algorithmic bytes per dispatch of every labelled kernel."""
    n, ng = R * H, RG * HG
    mib256 = float(1 << 28)
    rw = {HEADLINE_KEY: (n * 2, nvfp4_bytes(R, H) - n * 2),
          "nvfp4_quantize_split<fos,dq> expert_weights 65536x7168":
              (RG * H * 2, nvfp4_bytes(RG, H) - RG * H * 2),
          "nvfp4_quantize_split<fos,dq> tiny_ref 256x2048":
              (256 * 2048 * 2, nvfp4_bytes(256, 2048) - 256 * 2048 * 2),
          "nvfp4_quantize_split<6-only,dq> tiny_ref 256x2048":
              (256 * 2048 * 2, nvfp4_bytes(256, 2048) - 256 * 2048 * 2),
          "nvfp4_quantize_split<fos> ragged_routed 65536x2048":
              (ng * 2 + 65 * 8, nvfp4_bytes(RG, HG, dequant=False) - ng * 2),
          "nvfp4_quantize_split<fp16-decision,dq> moe_act 8192x7168":
              (n * 2, nvfp4_bytes(R, H) - n * 2),
          "nvfp4_quantize_split<fp16-decision> ragged_routed 65536x2048":
              (ng * 2 + 65 * 8, nvfp4_bytes(RG, HG, dequant=False) - ng * 2),
          DQ_KEY: (n // 2 + n // 16 + R * 4, n * 2),
          DQ_PACKED_KEY: (n // 2 + n // 16 + R * 4, n * 2),
          "nvfp4_quantize_guided moe_act 8192x7168":
              (n * 2 + n // 2 + n // 16 + R * 4, n // 2),
          "nvfp4_quantize_guided (no guide: nearest) moe_act 8192x7168":
              (n * 2 + n // 16 + R * 4, n // 2),
          "nvfp4_quantize_global (amax pass) moe_act 8192x7168": (n * 2, 2 * 512),
          "nvfp4_quantize_global (quantize pass) moe_act 8192x7168":
              (n * 2 + 2 * 512, nvfp4_bytes(R, H) - n * 2 - R * 4 + 4),
          "mxfp4_resq_quantize resq_act 8192x7168": (n * 2, mx_bytes(R, H) - n * 2),
          "mxfp4_resq_dense_quantize resq_act 8192x7168": (n * 2, mx_dense_bytes(R, H) - n * 2),
          "mxfp4_resq_reconstruct (S2:4) resq_act 8192x7168":
              (reconstruct_bytes(R, H) - n * 4, n * 4),
          "stand-in nvfp4_quantize_split<fos,dq> moe_act 8192x7168":
              (n * 2, nvfp4_bytes(R, H) - n * 2),
          "stand-in nvfp4_quantize_split<fos> ragged_routed 65536x2048":
              (ng * 2 + 65 * 8, nvfp4_bytes(RG, HG, dequant=False) - ng * 2),
          "stand-in mxfp4_resq_quantize resq_act 8192x7168": (n * 2, mx_bytes(R, H) - n * 2),
          "exact-error decision nvfp4_quantize_split<fos,dq> moe_act 8192x7168":
              (n * 2, nvfp4_bytes(R, H) - n * 2),
          "exact-error decision nvfp4_quantize_split<fos> ragged_routed 65536x2048":
              (ng * 2 + 65 * 8, nvfp4_bytes(RG, HG, dequant=False) - ng * 2),
          COPY_CAL_KEY: (mib256, mib256), "K0 copy 256 MiB": (mib256, mib256),
          "K0 copy nt sc1 256 MiB": (mib256, mib256),
          "K0 write nt 256 MiB": (0.0, mib256), "K0 write nt sc1 256 MiB": (0.0, mib256)}
    for d in (2, 4):
        for m in ("", " nt", " nt sc1"):
            rw["K0 mix read 4 KiB, write 4/%d KiB%s 256 MiB" % (d, m)] = (mib256, mib256 / d)
    for w in (1, 2, 4, 8, 16):
        rw["K0 read %dB 256 MiB" % w] = (mib256, 0.0)
    rw["K0 read 16B nt 256 MiB"] = (mib256, 0.0)
    return rw


PMC_CMD = ("rocprofv3 --pmc {c} -f csv -d {d} -o run -- python bench.py --no-cpu "
           "--secondary-steps 8 --steps 20 --warmup 2 --sets 2 --spinup 0")


def summarize_profiles(trace_dir, fetch_dir, write_dir, out_dir):
    """Turn the rocprofv3 CSV output of the three profiling runs of this
    script (kernel trace, FETCH_SIZE, WRITE_SIZE) into the text summaries
    under profiles/ and the per-launch traffic table the bench reads."""
    import csv
    import glob
    cmd_trace = ("rocprofv3 --kernel-trace --stats -f csv -d %s -o run -- python bench.py "
                 "--no-cpu" % trace_dir)
    trace = glob.glob(os.path.join(trace_dir, "*kernel_trace.csv"))[0]
    rows, labels = _read_dispatches(trace)
    dur = {}
    for r, lab in zip(rows, labels):
        if lab:
            dur.setdefault(lab, []).append(
                (int(r["Start_Timestamp"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    # the dequant is timed over two layouts of the same sets, one after the
    # other: its dispatches split at the longest pause between them
    if len(dur.get(DQ_KEY, ())) > 1:
        d = sorted(dur[DQ_KEY])
        gaps = [b[0] - a[0] for a, b in zip(d, d[1:])]
        k = int(np.argmax(gaps))
        if gaps[k] > 500_000:  # ns: the second layout's set-up, not a gap between calls
            dur[DQ_KEY], dur[DQ_PACKED_KEY] = d[:k + 1], d[k + 1:]
    dur = {lab: [t for _, t in v] for lab, v in dur.items()}
    stats = glob.glob(os.path.join(trace_dir, "*kernel_stats.csv"))[0]
    srows = list(csv.DictReader(open(stats)))
    algo = algorithmic_rw()
    lines = ["# Kernel durations, bench.py default run (moe_act 8192x7168 headline + secondary "
             "calls, K0 probes, stand-ins)", "", "Command (repo root, MI355X):", "",
             "    " + cmd_trace, "",
             "Per kernel and workload, from the kernel trace (us); GB/s and % of the 8 TB/s "
             "peak on the algorithmic bytes and the mean:", "",
             "| kernel / workload | dispatches | mean | p10 | p50 | p90 | min | max | GB/s | % peak |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for lab, d in sorted(dur.items()):
        a = np.array(d)
        rd, wr = algo.get(lab, (0.0, 0.0))
        gbs = (rd + wr) / (a.mean() * 1e-6) / 1e9 if rd + wr else float("nan")
        lines.append("| %s | %d | %.2f | %.2f | %.2f | %.2f | %.2f | %.2f | %.0f | %.1f |" % (
            lab, a.size, a.mean(), np.percentile(a, 10), np.median(a), np.percentile(a, 90),
            a.min(), a.max(), gbs, 100 * gbs / HBM_PEAK_GBS))
    lines += ["", "rocprofv3 --stats summary (the 16 kernels with most time):", "",
              "| kernel | calls | total ns | average ns | % |", "|---|---|---|---|---|"]
    for r in srows[:16]:
        lines.append("| %s | %s | %s | %s | %s |" % (r["Name"][:100], r["Calls"],
                                                    r["TotalDurationNs"], r["AverageNs"],
                                                    r["Percentage"]))
    os.makedirs(out_dir, exist_ok=True)
    open(os.path.join(out_dir, "kernel_trace_bench_default.md"), "w").write("\n".join(lines) + "\n")

    # HBM bytes per dispatch, calibrated on the K0 copy of 256 MiB
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
    f_scale = algo[COPY_CAL_KEY][0] / (fetch[COPY_CAL_KEY] * 1024.0)
    w_scale = algo[COPY_CAL_KEY][1] / (write[COPY_CAL_KEY] * 1024.0)
    digest = source_digest()
    table = {}
    lines = ["# HBM traffic per dispatch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
             "Commands (repo root, MI355X), one counter per run:", "",
             "    " + PMC_CMD.format(c="FETCH_SIZE", d=fetch_dir),
             "    " + PMC_CMD.format(c="WRITE_SIZE", d=write_dir), "",
             "Both counters are in KiB per dispatch.  Calibration on K0's non-temporal copy of "
             "256 MiB (268435456 B read with 16-byte loads, 268435456 B written): FETCH_SIZE "
             "reads %.0f KiB (scale x%.4f), WRITE_SIZE reads %.0f KiB (scale x%.4f).  The K0 "
             "read-only rows give FETCH_SIZE per load width (raw ratio = unscaled counter bytes "
             "/ bytes read).  Median over dispatches; kernel sources digest %s." % (
                 fetch[COPY_CAL_KEY], f_scale, write[COPY_CAL_KEY], w_scale, digest), "",
             "| kernel / workload | read B (scaled) | algorithmic read B | ratio | raw read ratio "
             "| write B (scaled) | algorithmic write B | ratio |",
             "|---|---|---|---|---|---|---|---|"]
    for lab in sorted(set(fetch) | set(write)):
        if lab not in algo:
            continue
        ar, aw = algo[lab]
        rd = fetch.get(lab, float("nan")) * 1024.0 * f_scale
        wr = write.get(lab, float("nan")) * 1024.0 * w_scale
        ratio = lambda a, b: "%.3f" % (a / b) if b else "-"
        lines.append("| %s | %.0f | %.0f | %s | %s | %.0f | %.0f | %s |" % (
            lab, rd, ar, ratio(rd, ar), ratio(fetch.get(lab, float("nan")) * 1024.0, ar), wr,
            aw, ratio(wr, aw)))
        if lab in fetch and lab in write:
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
    cmd = PMC_CMD.format(c=SQ_COUNTERS, d=sq_dir)
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
        if lab.startswith("K0"):
            continue
        c = {k: np.median([v for v, _ in per[lab][k]]) for k in per[lab]}
        t = np.median([d for _, d in per[lab]["SQ_INSTS_VALU"]])
        waves = c["SQ_WAVES"]
        valu_cycles = 4 * c["SQ_ACTIVE_INST_VALU"] / N_SIMDS
        lines.append("| %s | %.0f | %.1f | %.1f | %.1f | %.2f | %.1f%% | %.1f%% |" % (
            lab, waves, c["SQ_INSTS_VALU"] / waves, c["SQ_INSTS_SALU"] / waves,
            c["SQ_INSTS_LDS"] / waves, 4 * c["SQ_ACTIVE_INST_VALU"] / max(1, c["SQ_INSTS_VALU"]),
            100 * valu_cycles / (c["GRBM_GUI_ACTIVE"] / N_XCDS),
            100 * valu_cycles / (t * PEAK_CLOCK_HZ)))
    os.makedirs(out_dir, exist_ok=True)
    open(os.path.join(out_dir, "sq_counters_bench.md"), "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


# ------------------------------------------------------------- size sweep --

def size_sweep(x, dev):
    """Time per call against the row count for the headline quantize
    (4/6 + dequant), its memory-pattern stand-in, the standalone dequant,
    MXFP4 Rollout-ResQ and K0's copy of the same bytes as the quantize call
    moves, on rows of moe_act (tiled past 8192 rows).  Every size rotates
    over enough buffer sets to span about 1 GiB, so that no size is served
    by the last-level cache and all see a similar footprint.  A fit of time =
    fixed + rows * per_row separates the per-launch cost from the
    steady-state rate."""
    out = {}
    hidden = x.shape[1]
    S, M = standin(), membench()
    for rows in (1024, 2048, 4096, 8192, 16384, 32768):
        reps = (rows + x.shape[0] - 1) // x.shape[0]
        xr = x.repeat(reps, 1)[:rows].contiguous()
        nb = nvfp4_bytes(rows, hidden)
        nsets = n_sets(nb, min_sets=1, cap=32)
        sets = rotating_nvfp4_sets(xr, nsets)
        mx = [fq.mxfp4_resq_quantize(s[0]) for s in sets]
        # K0 copies of nb / 2 bytes each way (read + write = nb)
        half = (nb // 2) // 16 * 16
        cp = [(torch.empty(half, dtype=torch.uint8, device=dev),
               torch.empty(half, dtype=torch.uint8, device=dev)) for _ in range(nsets)]
        steps = max(100, 400 * 8192 // rows)
        t = {}
        t["nvfp4_quantize"], _ = time_calls(
            lambda s: fq.nvfp4_quantize(s[0], True, out=s[1]), sets, steps, steps // 4)
        t["stand-in nvfp4_quantize"], _ = time_calls(
            lambda s: nvfp4_via(S, s), sets, steps, steps // 4)
        t["nvfp4_dequantize"], _ = time_calls(
            lambda s: fq.nvfp4_dequantize(s[1][0], s[1][1], s[1][2], out=s[1][3]), sets, steps,
            steps // 4)
        t["mxfp4_resq_quantize"], _ = time_calls(
            lambda i: fq.mxfp4_resq_quantize(sets[i][0], out=mx[i]), list(range(nsets)), steps,
            steps // 4)
        t["K0 copy nt sc1 (same bytes)"], _ = time_calls(
            lambda c: M.fp4q_k0_copy(ptr(c[0]), ptr(c[1]), half, 2, stream_ptr()), cp, steps,
            steps // 4)
        out[rows] = {k: round(v * 1e3, 3) for k, v in t.items()}
        out[rows]["sets"] = nsets
        print("[bench] sweep rows %d: %s" % (rows, json.dumps(out[rows])), file=sys.stderr,
              flush=True)
        del sets, mx, xr, cp
        torch.cuda.empty_cache()
    fit = {}
    r = np.array(sorted(out), dtype=np.float64)
    for k in out[int(r[0])]:
        if k == "sets":
            continue
        us = np.array([out[int(v)][k] for v in r])
        big = r >= 4096  # the linear regime: several waves of workgroups per CU
        per_row, fixed = np.polyfit(r[big], us[big], 1)
        fit[k] = {"fixed_us": round(float(fixed), 2), "ns_per_row": round(float(per_row) * 1e3, 3),
                  "steady_state_GBps": round(nvfp4_bytes(1, hidden) / (per_row * 1e-6) / 1e9, 0)
                  if "dequantize" not in k and "mxfp4" not in k else None}
    return {"hidden": hidden, "us_per_call": out, "linear_fit_rows_ge_4096": fit}


def write_sweep_summary(sw, path, cmd):
    ks = [k for k in sw["us_per_call"][min(sw["us_per_call"])] if k != "sets"]
    rows = sorted(sw["us_per_call"])
    lines = ["# Time per call against row count (hidden %d, moe_act rows)" % sw["hidden"], "",
             "Command (repo root, MI355X): `%s` (HIP events over back-to-back calls, every "
             "size rotating over about 1 GiB of buffer sets)." % cmd, "",
             "| call | " + " | ".join("%d rows" % r for r in rows) +
             " | fixed us (fit, rows >= 4096) | ns per row | steady-state GB/s |",
             "|---|" + "---|" * len(rows) + "---|---|---|"]
    for k in ks:
        f = sw["linear_fit_rows_ge_4096"][k]
        lines.append("| %s | %s | %.2f | %.3f | %s |" % (
            k, " | ".join("%.2f" % sw["us_per_call"][r][k] for r in rows), f["fixed_us"],
            f["ns_per_row"], f["steady_state_GBps"] if f["steady_state_GBps"] else "-"))
    lines += ["", "The stand-in is the quantize kernel built with its per-block arithmetic "
              "compiled out (-DFP4Q_STANDIN=1): the same loads, row amax, row constants, "
              "reciprocal tables and stores.  The K0 copy moves the same number of bytes "
              "(half read, half written) in 4 KiB per wavefront with non-temporal loads and "
              "non-temporal sc1 stores (the quantizer's dequant stream); its steady-state "
              "column counts the quantize call's bytes per row."]
    open(path, "w").write("\n".join(lines) + "\n")


# ------------------------------------------------------------------ main --

def main():
    global SPINUP_S
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
    ap.add_argument("--sets", type=int, default=6, help="rotating buffer sets of the headline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--secondary-steps", type=int, default=None,
                    help="timed calls of every secondary figure (default: per figure)")
    ap.add_argument("--parts",
                    default="k0,standin,exact,tiny,dequant,resq,resq_dense,trace,global,"
                            "ragged,weights,fp16",
                    help="secondary measurements to run (comma list)")
    ap.add_argument("--cpu-rows", type=int, default=8192)
    ap.add_argument("--sweep", action="store_true",
                    help="print only a row-count sweep (time per call vs rows) as JSON")
    ap.add_argument("--sweep-summary", default=None,
                    help="with --sweep: also write a markdown summary to this path")
    ap.add_argument("--spinup", type=float, default=SPINUP_S,
                    help="seconds of untimed calls before each measurement's warm-up")
    args = ap.parse_args()
    SPINUP_S = args.spinup

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
        sw = size_sweep(x, dev)
        if args.sweep_summary:
            write_sweep_summary(sw, args.sweep_summary, "python bench.py --sweep")
        print(json.dumps(sw), flush=True)
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
                "launch_us_p50_per_call_events": round(float(np.median(per)) * 1e3, 3),
                "headline_working_set_bytes": working_set(sets)}
    del sets
    torch.cuda.empty_cache()

    secondary = {}
    parts = set() if args.no_secondary else set(args.parts.split(","))
    ss = args.secondary_steps

    def steps(default):
        return default if ss is None else ss

    def log(name):
        print("[bench] %s: %s" % (name, json.dumps(secondary[name])), file=sys.stderr,
              flush=True)

    n_el = rows * hidden
    if "k0" in parts:
        # K0: the copy ceiling in the quantizer's access pattern (4 KiB per
        # wavefront, 1 KiB per instruction) -- non-temporal with sc1 stores
        # (the quantizer's dequant stream), non-temporal and plain -- on
        # 256 MiB per call rotating over 4 x 512 MiB; then reads at every
        # load width (the counter calibration) and the two non-temporal
        # writes
        M = membench()
        sz = 1 << 28
        bufs = [(torch.empty(sz, dtype=torch.uint8, device=dev),
                 torch.empty(sz, dtype=torch.uint8, device=dev)) for _ in range(4)]
        for b in bufs:
            b[0].fill_(0x5A)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        for nt in (2, 1, 0):
            name = "K0 copy%s 256 MiB" % ("", " nt", " nt sc1")[nt]
            secondary[name] = measure(
                lambda b: _ok(M.fp4q_k0_copy(ptr(b[0]), ptr(b[1]), sz, nt, stream_ptr()), name),
                bufs, 2 * sz, None, steps(100))
            log(name)
        for w, nt in ((1, 0), (2, 0), (4, 0), (8, 0), (16, 0), (16, 1)):
            name = "K0 read %dB%s 256 MiB" % (w, " nt" if nt else "")
            secondary[name] = measure(
                lambda b: _ok(M.fp4q_k0_read(ptr(b[0]), sz, w, nt, ptr(sink), stream_ptr()),
                              name), bufs, sz, None, steps(50))
            log(name)
        for nt in (1, 2):
            name = "K0 write%s 256 MiB" % ("", " nt", " nt sc1")[nt]
            secondary[name] = measure(
                lambda b: _ok(M.fp4q_k0_write(ptr(b[1]), sz, nt, stream_ptr()), name), bufs, sz,
                None, steps(100))
            log(name)
        # the read/write mixes: 4 KiB read and 2 or 1 KiB written per
        # wavefront (the routed-token call's mix is about 1 KiB)
        for d, nt in ((4, 1), (4, 2), (2, 1)):
            name = "K0 mix read 4 KiB, write 4/%d KiB%s 256 MiB" % (d, ("", " nt", " nt sc1")[nt])
            secondary[name] = measure(
                lambda b: _ok(M.fp4q_k0_mix(ptr(b[0]), ptr(b[1]), sz, d, nt, stream_ptr()), name),
                bufs, sz + sz // d, None, steps(100))
            log(name)
        # the copy ceiling: the faster of the K0 copies
        secondary["device_copy_GBps"] = max(secondary["K0 copy%s 256 MiB" % m]["GBps"]
                                            for m in ("", " nt", " nt sc1"))
        del bufs, sink
        torch.cuda.empty_cache()
    if "standin" in parts:
        # the memory-pattern stand-ins: the headline kernel and the ragged
        # call with their per-block arithmetic compiled out, and K3 likewise
        S = standin()
        ssets = rotating_nvfp4_sets(x, args.sets)
        name = "stand-in nvfp4_quantize moe_act 8192x7168 (4/6 + dequant pattern)"
        secondary[name] = measure(lambda s: nvfp4_via(S, s), ssets, nbytes, n_el,
                                  steps(1000))
        log(name)
        del ssets
        xg = workloads.tensor("ragged_routed", dev)
        offs = torch.from_numpy(workloads.group_offsets()).to(dev)
        bg = nvfp4_bytes(*xg.shape, dequant=False, groups=offs.numel() - 1)
        gsets = rotating_nvfp4_sets(xg, n_sets(bg), dequant=False)
        name = "stand-in nvfp4_quantize ragged_routed 65536x2048 (no dequant pattern)"
        secondary[name] = measure(lambda s: nvfp4_via(S, s, offs), gsets, bg, xg.numel(),
                                  steps(500))
        log(name)
        del gsets, xg
        xr = workloads.tensor("resq_act", dev)
        bm = mx_bytes(*xr.shape)
        msets = []
        for i in range(n_sets(bm)):
            xi = xr if i == 0 else xr.clone()
            msets.append((xi, fq.mxfp4_resq_quantize(xi)))
        name = "stand-in mxfp4_resq_quantize resq_act 8192x7168"
        secondary[name] = measure(
            lambda m: _ok(S.mxfp4_resq_quantize(ptr(m[0]), m[0].shape[0], m[0].shape[1],
                                                *[ptr(t) for t in m[1]], stream_ptr()), name),
            msets, bm, xr.numel(), steps(500))
        log(name)
        del msets, xr
        torch.cuda.empty_cache()
    if "exact" in parts:
        # the straightforward FP32 4/6 decision (both errors by the
        # definition for every block), against which the pages measure
        # their FP16 shortcut: the headline and the ragged call
        E = exactdecision()
        esets = rotating_nvfp4_sets(x, args.sets)
        name = "exact-error decision nvfp4_quantize moe_act 8192x7168 (4/6 + dequant)"
        secondary[name] = measure(lambda s: nvfp4_via(E, s), esets, nbytes, n_el,
                                  steps(1000))
        log(name)
        del esets
        xg = workloads.tensor("ragged_routed", dev)
        offs = torch.from_numpy(workloads.group_offsets()).to(dev)
        bg = nvfp4_bytes(*xg.shape, dequant=False, groups=offs.numel() - 1)
        gsets = rotating_nvfp4_sets(xg, n_sets(bg), dequant=False)
        name = "exact-error decision nvfp4_quantize ragged_routed 65536x2048 (no dequant)"
        secondary[name] = measure(lambda s: nvfp4_via(E, s, offs), gsets, bg, xg.numel(),
                                  steps(500))
        log(name)
        del gsets, xg
        torch.cuda.empty_cache()
    if "tiny" in parts:
        # C1, launch-bound by construction (2.4 MB a call): reported, not
        # graded; 448 rotating sets span 1 GiB
        xt = workloads.tensor("tiny_ref", dev)
        bt = nvfp4_bytes(*xt.shape)
        tsets = rotating_nvfp4_sets(xt, n_sets(bt))
        for fos, mode in ((1, "4/6"), (0, "6-only")):
            name = "nvfp4_quantize tiny_ref 256x2048 %s + dequant" % mode
            secondary[name] = measure(lambda s: fq.nvfp4_quantize(s[0], fos, out=s[1]), tsets,
                                      bt, xt.numel(), steps(2000))
            log(name)
        del tsets, xt
        torch.cuda.empty_cache()
    if "dequant" in parts:
        # standalone dequant on the headline shape: distinct codes, scales
        # and outputs per set
        c, s_, ts, _ = fq.nvfp4_quantize(x, True, dequant=False)
        b = dequant_bytes(rows, hidden)
        nd = n_sets(b)
        dsets = [(c.clone(), s_.clone(), ts.clone(), torch.empty_like(x)) for _ in range(nd)]
        name = "nvfp4_dequantize moe_act 8192x7168"
        secondary[name] = measure(lambda d: fq.nvfp4_dequantize(d[0], d[1], d[2], out=d[3]),
                                  dsets, b, n_el, steps(400))
        del dsets
        torch.cuda.empty_cache()
        # the same sets with each kind held in one allocation (every set's
        # codes together, and so on): the same bytes and rotation, but this
        # call's time depends on where its inputs lie (the other calls'
        # do not), so both figures are reported
        C = c.repeat(nd, 1).view(nd, rows, hidden // 2)
        S = s_.repeat(nd, 1).view(nd, rows, hidden // 16)
        T = ts.repeat(nd).view(nd, rows)
        D = torch.empty((nd, rows, hidden), dtype=torch.bfloat16, device=dev)
        psets = [(C[i], S[i], T[i], D[i]) for i in range(nd)]
        secondary[name]["one_allocation_per_kind"] = measure(
            lambda d: fq.nvfp4_dequantize(d[0], d[1], d[2], out=d[3]), psets, b, n_el, steps(400))
        log(name)
        del psets, C, S, T, D, c, s_, ts
        torch.cuda.empty_cache()
    if "resq" in parts or "resq_dense" in parts:
        xr = workloads.tensor("resq_act", dev)
        r_, h_ = xr.shape
    if "resq" in parts:
        # MXFP4 Rollout-ResQ
        b = mx_bytes(r_, h_)
        msets = []
        for i in range(n_sets(b)):
            xi = xr if i == 0 else xr.clone()
            msets.append((xi, fq.mxfp4_resq_quantize(xi)))
        name = "mxfp4_resq_quantize resq_act 8192x7168"
        secondary[name] = measure(lambda m: fq.mxfp4_resq_quantize(m[0], out=m[1]), msets, b,
                                  xr.numel(), steps(400))
        log(name)
        del msets
        torch.cuda.empty_cache()
    if "resq_dense" in parts:
        # Rollout-ResQ-Dense, the S2:4 reconstruction, and the reconstruction
        # error of the three variants (MSE over all elements, FP64)
        b = mx_dense_bytes(r_, h_)
        msets = []
        for i in range(n_sets(b)):
            xi = xr if i == 0 else xr.clone()
            msets.append((xi, fq.mxfp4_resq_dense_quantize(xi)))
        name = "mxfp4_resq_dense_quantize resq_act 8192x7168"
        secondary[name] = measure(lambda m: fq.mxfp4_resq_dense_quantize(m[0], out=m[1]), msets,
                                  b, xr.numel(), steps(400))
        log(name)
        de = msets[0][1]
        del msets
        sp = fq.mxfp4_resq_quantize(xr)
        xf = xr.float().double()
        mse = {}
        recon = {"primary only": (sp[0], sp[1], None, None, None, 0),
                 "primary + S2:4 residual": (sp[0], sp[1], sp[2], sp[3], sp[4], 1),
                 "primary + dense residual": (de[0], de[1], de[2], None, de[3], 2)}
        xh = torch.empty((r_, h_), dtype=torch.float32, device=dev)
        for nm, a in recon.items():
            fq.mxfp4_resq_reconstruct(*a[:5], residual=a[5], out=xh)
            err = (xf - xh.double())
            mse[nm] = {"mse": float((err * err).mean()),
                       "rel_mse": float((err * err).sum() / (xf * xf).sum())}
        del xf, xh, err
        torch.cuda.empty_cache()
        b = reconstruct_bytes(r_, h_)
        rsets = [(tuple(t.clone() for t in sp), torch.empty((r_, h_), dtype=torch.float32,
                                                              device=dev))
                 for _ in range(n_sets(b))]
        name = "mxfp4_resq_reconstruct (S2:4) resq_act 8192x7168"
        secondary[name] = measure(lambda q: fq.mxfp4_resq_reconstruct(*q[0], residual=1,
                                                                      out=q[1]),
                                  rsets, b, xr.numel(), steps(400))
        log(name)
        secondary["Rollout-ResQ reconstruction error resq_act"] = mse
        del rsets, sp, de
        torch.cuda.empty_cache()
    if "resq" in parts or "resq_dense" in parts:
        del xr
    if "trace" in parts:
        # TRACE rollout-guided rounding: the rollout quantizes moe_act; the
        # training side holds the same values perturbed by ~1 BF16 step
        # (relative N(0, 2^-8)).  Timed: guided rounding and round to nearest
        # under the rollout's scales, each set with its own training tensor,
        # rollout codes and scales and outputs.
        def training_copy(seed):
            return torch.from_numpy(workloads.perturbed(x_bits, seed=seed).view(np.int16)).view(
                torch.bfloat16).to(dev)
        bgd = guided_bytes(rows, hidden, guide=True)
        gsets = []
        for i in range(n_sets(bgd)):
            xt = training_copy(2 + i)
            roll = fq.nvfp4_quantize(x if i == 0 else x.clone(), True, dequant=False)[:3]
            gsets.append((xt, roll, torch.empty_like(roll[0])))
        name = "nvfp4_quantize_guided moe_act 8192x7168 (no dequant)"
        secondary[name] = measure(
            lambda g: fq.nvfp4_quantize_guided(g[0], *g[1], dequant=False, out=(g[2], None)),
            gsets, bgd, n_el, steps(400))
        log(name)
        bnn = guided_bytes(rows, hidden, guide=False)
        name = "nvfp4_quantize_guided, no guide (nearest) moe_act 8192x7168 (no dequant)"
        secondary[name] = measure(
            lambda g: fq.nvfp4_quantize_guided(g[0], None, g[1][1], g[1][2], dequant=False,
                                               out=(g[2], None)),
            gsets, bnn, n_el, steps(400))
        log(name)
        xt, (rc, rs, rt) = gsets[0][0], gsets[0][1]
        del gsets
        torch.cuda.empty_cache()

        def signed_index(c):
            """Codeword position on the signed grid -7..7 (+0 and -0 are the
            same codeword)."""
            n = torch.stack([c & 15, c >> 4], -1).reshape(c.shape[0], -1).int()
            mag = n & 7
            return torch.where((n & 8) != 0, -mag, mag)

        ref = signed_index(rc)

        def agreement(codes):
            got = signed_index(codes)
            mis = got != ref
            adj = mis & ((got - ref).abs() == 1)
            return {"mismatch_frac": round(float(mis.sum()) / ref.numel(), 7),
                    "adjacent_share_of_mismatches":
                        round(float(adj.sum()) / max(1, int(mis.sum())), 5)}
        own = fq.nvfp4_quantize(xt, True, dequant=False)[0]  # its own scales
        nearest = fq.nvfp4_quantize_guided(xt, None, rs, rt, dequant=False)[0]
        guided = fq.nvfp4_quantize_guided(xt, rc, rs, rt, dequant=False)[0]
        secondary["TRACE codeword agreement with the rollout, moe_act (training = rollout x "
                  "(1 + 2^-8 N(0,1)))"] = {
            "elements": ref.numel(),
            "nearest_under_rollout_scales": agreement(nearest),
            "nearest_under_own_scales": agreement(own),
            "guided_under_rollout_scales": agreement(guided)}
        log("TRACE codeword agreement with the rollout, moe_act (training = rollout x "
            "(1 + 2^-8 N(0,1)))")
        del xt, rc, rs, rt, own, nearest, guided, ref
        torch.cuda.empty_cache()
    if "global" in parts:
        # the naive one-scale-per-tensor NVFP4: speed (two kernels: the
        # tensor-max pass and the quantize pass), and the batch dependency
        gsets = rotating_nvfp4_sets(x, args.sets)
        outs = [((s_[1][0], s_[1][1], torch.empty(1, dtype=torch.float32, device=dev), s_[1][3]),
                 torch.empty(fq.GLOBAL_WORKSPACE_BYTES, dtype=torch.uint8, device=dev))
                for s_ in gsets]
        gl = [(g[0], o) for g, o in zip(gsets, outs)]
        name = "nvfp4_quantize_global moe_act 8192x7168 (tensor-max pass + quantize)"
        secondary[name] = measure(
            lambda g: fq.nvfp4_quantize_global(g[0], True, out=g[1][0], workspace=g[1][1]), gl,
            nbytes, n_el, steps(1000))
        secondary[name]["GBps_on_own_bytes"] = round(
            (nbytes + n_el * 2) / (secondary[name]["us"] * 1e-6) / 1e9, 1)
        log(name)
        del gsets, outs, gl
        torch.cuda.empty_cache()
        full = fq.nvfp4_quantize_global(x, True, dequant=False)
        pt_full = fq.nvfp4_quantize(x, True, dequant=False)
        changed = pt_changed = 0
        for r0 in range(0, rows, 1024):
            part = fq.nvfp4_quantize_global(x[r0:r0 + 1024], True, dequant=False)
            same = (part[1] == full[1][r0:r0 + 1024]) & (
                part[0].view(-1, hidden // 16, 8) == full[0][r0:r0 + 1024].view(
                    -1, hidden // 16, 8)).all(-1)
            changed += int((~same).sum())
            pp = fq.nvfp4_quantize(x[r0:r0 + 1024], True, dequant=False)
            pt_changed += int((pp[0] != pt_full[0][r0:r0 + 1024]).sum() +
                              (pp[1] != pt_full[1][r0:r0 + 1024]).sum())
        secondary["batch dependency moe_act (8 slices of 1024 rows vs the whole tensor)"] = {
            "global_scale_blocks_changed_frac": round(changed / (rows * hidden // 16), 6),
            "per_token_bytes_changed": pt_changed}
        del full, pt_full
        torch.cuda.empty_cache()
    if "ragged" in parts:
        # ragged routed, quantize only
        xg = workloads.tensor("ragged_routed", dev)
        offs = torch.from_numpy(workloads.group_offsets()).to(dev)
        b = nvfp4_bytes(*xg.shape, dequant=False, groups=offs.numel() - 1)
        gsets = rotating_nvfp4_sets(xg, n_sets(b), dequant=False)
        name = "nvfp4_quantize ragged_routed 65536x2048 (64 groups, no dequant)"
        secondary[name] = measure(lambda s: fq.nvfp4_quantize(s[0], True, offsets=offs, out=s[1]),
                                  gsets, b, xg.numel(), steps(1000))
        log(name)
        del gsets, xg
        torch.cuda.empty_cache()
    if "weights" in parts:
        # expert weights, 32 x 2048 x 7168: one set of 4.3 GB (two sets
        # measure slower, which points at address-translation reach)
        xw = workloads.tensor("expert_weights", dev)
        wsets = rotating_nvfp4_sets(xw, 1)
        b = nvfp4_bytes(*xw.shape)
        name = "nvfp4_quantize expert_weights 65536x7168"
        secondary[name] = measure(lambda s: fq.nvfp4_quantize(s[0], True, out=s[1]), wsets, b,
                                  xw.numel(), steps(50), warmup=5)
        log(name)
        del wsets, xw
        torch.cuda.empty_cache()
    if "fp16" in parts:
        # the FP16 fast path's 4/6 decision (four_over_six = 2): speed on the
        # headline shape, and how often its choice equals the FP32 one
        fsets = rotating_nvfp4_sets(x, args.sets)
        name = "nvfp4_quantize fp16-decision moe_act 8192x7168"
        secondary[name] = measure(lambda s: fq.nvfp4_quantize(s[0], 2, out=s[1]), fsets, nbytes,
                                  n_el, steps(1000))
        log(name)
        del fsets
        # and on the VALU-bound routed-token call
        xg = workloads.tensor("ragged_routed", dev)
        offs = torch.from_numpy(workloads.group_offsets()).to(dev)
        b = nvfp4_bytes(*xg.shape, dequant=False, groups=offs.numel() - 1)
        gsets = rotating_nvfp4_sets(xg, n_sets(b), dequant=False)
        name = "nvfp4_quantize fp16-decision ragged_routed 65536x2048 (no dequant)"
        secondary[name] = measure(lambda s: fq.nvfp4_quantize(s[0], 2, offsets=offs, out=s[1]),
                                  gsets, b, xg.numel(), steps(1000))
        log(name)
        del gsets, xg
        torch.cuda.empty_cache()
        agree = {}
        for wname in ("tiny_ref", "moe_act", "expert_weights"):
            xa = x if wname == "moe_act" else workloads.tensor(wname, dev)
            c1, s1, _, _ = fq.nvfp4_quantize(xa, 1, dequant=False)
            c2, s2, _, _ = fq.nvfp4_quantize(xa, 2, dequant=False)
            r, h = xa.shape
            same = (s1 == s2) & (c1.view(r, h // 16, 8) == c2.view(r, h // 16, 8)).all(-1)
            agree[wname] = {"blocks": same.numel(),
                            "same_choice_frac": round(float(same.float().mean()), 7)}
            del xa, c1, s1, c2, s2, same
            torch.cuda.empty_cache()
        secondary["fp16-decision agreement with the FP32 choice"] = agree

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
