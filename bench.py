"""Benchmark: Engram prefill forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = one engram_forward over the DeepSeek-V4.1-shaped prefill: B=1,
T=4096, dim=5120, hc=4, 24 hash columns of head_dim 64 (wkv 1536 -> 25600),
a 25,160,950-row fp8 table, seeded synthetic inputs already resident in HBM.
The forward runs fully fused: hash -> the fp8 row gather fused into the wkv
bf16 MFMA projection, whose epilogue reduces the key columns into the gate's
partial sums (engram_wkv_gate_partials) -> the gate from those partials.
Prints one JSON line: whole-job tokens/s, the roofline of the dominant call,
engram_wkv_gate_partials (projection flops per call over its average call
time, measured here with HIP events on the stream it runs on; the call is
the offset/scale prep kernel plus the two projection kernels), the gate's
HBM rate, and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Engram prefill tokens/s @dim5120 hc4 (1 GPU); % MFMA peak (wkv), % HBM BW (gate)"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "wkv_gate_partials_prefill_traffic.json")
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "wkv_gathered_decode_traffic.json")
DECODE_KERNELS = ("prep_kernel", "wkv_gathered_64")  # one engram_wkv_gathered call at M = 64


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample", type=int, default=2048, help="tokens the oracle runs")
    p.add_argument("--cpu-threads", type=int, default=0,
                   help="threads for the oracle timing (default: all the host offers)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run 3 plain device copies of exactly 1 GiB (a known-size kernel "
                        "against which HBM byte counters are scaled)")
    p.add_argument("--workload", choices=("prefill", "decode", "long_mixed", "hash_layers",
                                          "gate_stress"),
                   default="prefill",
                   help="prefill (the default and the headline line); decode: 128 steps "
                        "of 64 sequences after a 512-token prefill, replayed as one graph; "
                        "long_mixed: T=32768 with Zipf(1.1) ids and 30%% of positions masked "
                        "in spans; hash_layers: 8 Engram layers' hashes of the T=4096 prefill "
                        "in one launch; gate_stress: the gate and add alone over 65,536 tokens "
                        "of given kv")
    p.add_argument("--summarize", nargs=3, metavar=("STATS_DIR", "FETCH_DIR", "WRITE_DIR"),
                   help="no GPU work: turn the CSV output of three rocprofv3 runs of this "
                        "script (--kernel-trace --stats; --pmc FETCH_SIZE; --pmc WRITE_SIZE, "
                        "the last two with --copy-calibration) into the summaries under "
                        "profiles/")
    p.add_argument("--summarize-decode-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="no GPU work: turn FETCH_SIZE and WRITE_SIZE runs of `--workload decode "
                        "--copy-calibration` into the decode projection's traffic summary "
                        "under profiles/")
    p.add_argument("--summarize-counters", nargs=3, metavar=("PMC_DIR", "NAME", "ROCPROF_ARGS"),
                   help="no GPU work: turn one rocprofv3 --pmc run of the prefill bench into "
                        "profiles/NAME.txt")
    p.add_argument("--summarize-stats", nargs=3, metavar=("STATS_DIR", "NAME", "BENCH_ARGS"),
                   help="no GPU work: turn one rocprofv3 --kernel-trace --stats run of "
                        "`bench.py BENCH_ARGS` into profiles/NAME.txt")
    return p.parse_args()


def summarize_stats(stats_dir, name, bench_args):
    """Kernel table (calls, average, min, max, share) plus median durations
    of the library's kernels, for any bench workload."""
    rows = _csv(stats_dir, "kernel_stats.csv")
    lines = ["# rocprofv3 kernel-trace statistics: python3 bench.py %s" % bench_args,
             "# command (repository root = <repo>):",
             "#   cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format "
             "csv -d <out> -o <name> -- python3 <repo>/bench.py %s" % bench_args,
             "# averages include every call (set-up and warm-up calls too).",
             "",
             "%-40s %7s %12s %12s %12s %7s" % ("kernel", "calls", "avg_ns", "min_ns", "max_ns", "pct")]
    for r in rows:
        lines.append("%-40s %7s %12.0f %12s %12s %7s" % (
            short_name(r["Name"]), r["Calls"], float(r["AverageNs"]), r["MinNs"], r["MaxNs"],
            r["Percentage"]))
    durs = {}
    for r in _csv(stats_dir, "kernel_trace.csv"):
        if "engram::" in r["Kernel_Name"]:
            durs.setdefault(short_name(r["Kernel_Name"]), []).append(
                int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines.append("")
    lines.append("# median ns per library kernel (kernel trace):")
    for k, v in sorted(durs.items()):
        lines.append("#   %-40s %10d  (%d calls)" % (k, sorted(v)[len(v) // 2], len(v)))
    out = os.path.join(ROOT, "profiles", name + ".txt")
    open(out, "w").write("\n".join(lines) + "\n")
    print("wrote", os.path.relpath(out, ROOT))


def summarize_counters(pmc_dir, name, rocprof_args):
    """Mean of each collected counter per library kernel, from one rocprofv3
    --pmc run of the prefill bench, with the derived clock and matrix-core
    busy share where GRBM_GUI_ACTIVE and SQ_VALU_MFMA_BUSY_CYCLES are present
    (GUI_ACTIVE is summed over the 8 XCDs; the busy cycles over the 1024
    SIMDs).  GUI_ACTIVE also counts a fixed number of cycles per dispatch
    beyond the kernel's own run; that part is fitted over the run's short
    dispatches (every kernel under 120 us: cycles per XCD = rate * duration
    + fixed) and taken off before the clock is derived."""
    import numpy as np
    per = {}
    fit_x, fit_y = [], []
    for r in _csv(pmc_dir, "counter_collection.csv"):
        dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        if r["Counter_Name"] == "GRBM_GUI_ACTIVE" and dur < 120e3:
            fit_x.append(dur / 1e3)
            fit_y.append(float(r["Counter_Value"]) / N_XCD_COUNT)
        if "engram::" not in r["Kernel_Name"]:
            continue
        k = short_name(r["Kernel_Name"])
        d = per.setdefault(k, {"_dur": {}})
        d.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        d["_dur"][r["Dispatch_Id"]] = dur
    fixed = 0.0
    if len(fit_x) >= 2:
        A = np.vstack([np.array(fit_x), np.ones(len(fit_x))]).T
        rate, fixed = np.linalg.lstsq(A, np.array(fit_y), rcond=None)[0]
    lines = ["# rocprofv3 counters per dispatch (mean over dispatches): Engram prefill bench",
             "# command (repository root = <repo>):",
             "#   cd /tmp && export TMPDIR=/tmp && rocprofv3 %s --output-format csv -d <out> "
             "-o <name> -- python3 <repo>/bench.py --no-cpu-baseline --steps 5 --warmup 3"
             % rocprof_args]
    if fixed:
        lines.append("# GRBM_GUI_ACTIVE per XCD over the %d dispatches under 120 us fits %.0f "
                     "cycles per us + %.0f per dispatch;" % (len(fit_x), rate, fixed))
        lines.append("#   the clock below is (GUI_ACTIVE per XCD - %.0f) / median time, and the "
                     "matrix-core busy share is over those cycles" % fixed)
    lines.append("")
    for k in sorted(per):
        d = per[k]
        durs = sorted(d.pop("_dur").values())
        med = durs[len(durs) // 2]
        lines.append("%s  (%d dispatches, median %.1f us)" % (k, len(durs), med / 1e3))
        for c in sorted(d):
            lines.append("    %-28s %14.4g" % (c, sum(d[c]) / len(d[c])))
        # with the fixed part taken off, a clock derived from GUI_ACTIVE means
        # something only for kernels that run much longer than that part
        # (50 us and up)
        if "GRBM_GUI_ACTIVE" in d and med >= 50e3:
            gui = sum(d["GRBM_GUI_ACTIVE"]) / len(d["GRBM_GUI_ACTIVE"]) / N_XCD_COUNT - fixed
            lines.append("    clock (GUI_ACTIVE per XCD less fixed / median time)  %.2f GHz"
                         % (gui / med))
            if "SQ_VALU_MFMA_BUSY_CYCLES" in d:
                busy = sum(d["SQ_VALU_MFMA_BUSY_CYCLES"]) / len(d["SQ_VALU_MFMA_BUSY_CYCLES"])
                lines.append("    matrix cores busy (busy / SIMDs / cycles)  %.1f %%"
                             % (100.0 * busy / SIMD_COUNT / gui))
    out = os.path.join(ROOT, "profiles", name + ".txt")
    open(out, "w").write("\n".join(lines) + "\n")
    print("wrote", os.path.relpath(out, ROOT))


N_XCD_COUNT = 8       # MI355X XCDs
SIMD_COUNT = 1024     # 256 CUs x 4 SIMDs


def kernel_source_digest() -> str:
    """Digest of the fused projection's sources with comments and blank
    lines dropped: the counted traffic stays valid across comment edits."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gram_memory_layer_amd", "csrc")
    for f in ("wkv_gathered.hip", "tiles.h", "internal.h"):
        src = open(os.path.join(csrc, f)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        src = "\n".join(l.rstrip() for l in src.splitlines() if l.strip())
        h.update(src.encode())
    return h.hexdigest()[:16]


def traffic_record(launch_flops_tokens: int, path: str = TRAFFIC_FILE):
    """HBM bytes per call of the roofline's kernels (engram_wkv_gate_partials,
    or engram_wkv_gathered at decode size) from the committed rocprofv3
    counter summary, or None if it was taken on a different kernel source or
    workload."""
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != kernel_source_digest() or rec.get("tokens") != launch_flops_tokens:
        return None
    return rec.get("hbm_bytes_per_launch")


def mfma_ceiling(dev, stream, w) -> dict:
    """The part's matrix-core ceiling on this machine: the projection's MFMA back
    to back from registers (libengram_probe.so), 8 waves per CU, once with
    operands whose bits change every step (as in a GEMM) and once with zero
    operands; then the same MFMA fed from LDS with the projection's own W
    values and its per-k-step fragment reads, but no global traffic
    (`lds_fed`).  TFLOP/s over event time, and the shader clock the loop ran
    at (shader-clock ticks over constant-rate wall-clock ticks, median over
    workgroups)."""
    import ctypes as C
    import torch
    path = os.path.join(ROOT, "bench_probe", "libengram_probe.so")
    if not os.path.exists(path):
        raise SystemExit("libengram_probe.so is not built; run `python -m bench_probe.build`")
    L = C.CDLL(path)
    L.engram_probe_mfma_flops.restype = C.c_double
    L.engram_probe_mfma_flops.argtypes = [C.c_int, C.c_int]
    L.engram_probe_mfma.restype = C.c_int
    L.engram_probe_mfma.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int,
                                    C.c_void_p]
    L.engram_probe_mfma_lds_flops.restype = C.c_double
    L.engram_probe_mfma_lds_flops.argtypes = [C.c_int, C.c_int]
    L.engram_probe_mfma_lds.restype = C.c_int
    L.engram_probe_mfma_lds.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_void_p, C.c_int,
                                        C.c_int, C.c_void_p]
    L.engram_probe_wall_clock_hz.restype = C.c_int
    L.engram_probe_wall_clock_hz.argtypes = [C.POINTER(C.c_int64)]
    hz = C.c_int64(0)
    if L.engram_probe_wall_clock_hz(C.byref(hz)) != 0 or hz.value <= 0:
        raise SystemExit("no wall-clock rate for the MFMA probe")
    blocks = torch.cuda.get_device_properties(dev).multi_processor_count
    threads = blocks * 512
    gen = torch.Generator(device=dev)
    gen.manual_seed(20262)
    seed = torch.randint(-2**31, 2**31 - 1, (threads * 8,), dtype=torch.int32, device=dev,
                         generator=gen)
    sums = torch.empty(threads, dtype=torch.float32, device=dev)
    clocks = torch.empty(blocks * 2, dtype=torch.int64, device=dev)
    iters = 40000
    res = {}
    for mode, zero in (("changing_operands", 0), ("zero_operands", 1), ("lds_fed", -1)):
        def once():
            if zero < 0:
                r = L.engram_probe_mfma_lds(w.data_ptr(), w.numel() * w.element_size(),
                                            sums.data_ptr(), clocks.data_ptr(), blocks, iters,
                                            stream.cuda_stream)
            else:
                r = L.engram_probe_mfma(seed.data_ptr(), sums.data_ptr(), clocks.data_ptr(),
                                        blocks, iters, zero, stream.cuda_stream)
            if r != 0:
                raise SystemExit("MFMA probe launch failed: %d" % r)
        once()
        times = []
        ratios = []
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            once()
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1) / 1e3)
            c = clocks.cpu().view(-1, 2).double()
            ratios.append(float((c[:, 0] / c[:, 1]).median()) * hz.value / 1e9)
        t = sorted(times)[1]
        flops = (L.engram_probe_mfma_lds_flops(blocks, iters) if zero < 0
                 else L.engram_probe_mfma_flops(blocks, iters))
        res[mode] = {"tflops": round(flops / t / 1e12, 1), "clock_ghz": round(sorted(ratios)[1], 3)}
    return res


def time_launches(fn, n, stream):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(n):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / n * 1e-3  # seconds per launch


def time_gpu(fn, n, stream):
    """Seconds per call of fn on the GPU alone, for the stage and kernel
    figures (the headline steps keep time_launches): the n calls are captured
    once in a HIP graph and the graph is replayed, so they run back to back
    with no host launch gaps between them (a call shorter than its host-side
    launch cost would otherwise be timed at the host's pace).  fn must be
    capture-safe: the library calls allocate nothing and never synchronise."""
    import torch
    graph = torch.cuda.CUDAGraph()
    fn()  # anything lazily set up happens outside the capture
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for _ in range(n):
            fn()
    graph.replay()  # warm
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    graph.replay()
    end.record(stream)
    end.synchronize()
    del graph
    return start.elapsed_time(end) / n * 1e-3


# ------------------------------------------------------------------ profile summaries
COPY_BYTES = 1 << 30
FUSED_KERNELS = ("prep_kernel", "wkv_gathered_256<3, true, true>", "wkv_gathered_128")


def is_fused(k: str) -> bool:
    """The kernels of one engram_wkv_gate_partials call."""
    return k in FUSED_KERNELS or k.split("<")[0] in ("prep_kernel", "wkv_gathered_128")


def short_name(name: str) -> str:
    import re
    m = re.search(r"engram::(?:\(anonymous namespace\)::)?(\w+)(<[^>]*>)?\(", name)
    if m:
        return m.group(1) + (m.group(2) or "")
    return name[:40]


def _csv(d, suffix):
    import csv
    files = [f for f in os.listdir(d) if f.endswith(suffix)]
    if len(files) != 1:
        raise SystemExit("%s: expected one *%s, found %r" % (d, suffix, files))
    return list(csv.DictReader(open(os.path.join(d, files[0]))))


def _counter_means(d, counter):
    """Mean counter value (KiB per dispatch) per engram kernel, and the value
    for the 1 GiB calibration copy (the copy dispatch with the largest value)."""
    per, copy = {}, 0.0
    for r in _csv(d, "counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        v = float(r["Counter_Value"])
        n = r["Kernel_Name"]
        if "engram::" in n:
            per.setdefault(short_name(n), []).append(v)
        elif "copy" in n.lower():
            copy = max(copy, v)
    if copy <= 0:
        raise SystemExit("%s: no calibration copy dispatch (run with --copy-calibration)" % d)
    return {k: sum(v) / len(v) for k, v in per.items()}, copy


def summarize(stats_dir, fetch_dir, write_dir):
    tokens = 4096
    cmd_base = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 %s --output-format csv -d <out> -o <name> "
                "-- python3 <repo>/bench.py --no-cpu-baseline %s")
    # kernel-trace statistics
    rows = _csv(stats_dir, "kernel_stats.csv")
    lines = ["# rocprofv3 kernel-trace statistics: Engram prefill forward, T=4096, dim 5120, hc 4",
             "# command (repository root = <repo>):",
             "#   " + cmd_base % ("--kernel-trace --stats", ""),
             "# engram_wkv_gate_partials = prep_kernel + wkv_gathered_256<3, true, true> + wkv_gathered_128<L>",
             "# (prep_kernel and wkv_gathered_128 also run in the engram_wkv_gathered calls bench times);",
             "# averages include every call (warm-up and cold-clock launches too);",
             "# mfma_loop and mfma_lds_loop are the bench's matrix-core ceiling probes (libengram_probe.so).",
             "",
             "%-34s %7s %12s %12s %12s %7s" % ("kernel", "calls", "avg_ns", "min_ns", "max_ns", "pct")]
    for r in rows:
        lines.append("%-34s %7s %12.0f %12s %12s %7s" % (
            short_name(r["Name"]), r["Calls"], float(r["AverageNs"]), r["MinNs"], r["MaxNs"],
            r["Percentage"]))
    fused_avg = sum(float(r["AverageNs"]) for r in rows if is_fused(short_name(r["Name"])))
    # medians from the trace: robust to the few cold-clock launches
    durs = {}
    for r in _csv(stats_dir, "kernel_trace.csv"):
        k = short_name(r["Kernel_Name"])
        if is_fused(k) or k.startswith(("gate_kernel", "hash_kernel")):
            durs.setdefault(k, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    med = {k: sorted(v)[len(v) // 2] for k, v in durs.items()}
    lines.append("")
    lines.append("# median ns per kernel (kernel trace): " +
                 ", ".join("%s %d" % (k, v) for k, v in sorted(med.items())))
    lines.append("# engram_wkv_gate_partials per call: sum of averages %.1f us, sum of medians %.1f us"
                 % (fused_avg / 1e3,
                    sum(v for k, v in med.items() if is_fused(k)) / 1e3))
    open(os.path.join(ROOT, "profiles", "engram_prefill_T4096_kernel_stats.txt"), "w").write(
        "\n".join(lines) + "\n")

    # HBM bytes from FETCH_SIZE / WRITE_SIZE, scaled by the calibration copy
    fetch, copy_f = _counter_means(fetch_dir, "FETCH_SIZE")
    write, copy_w = _counter_means(write_dir, "WRITE_SIZE")
    fs = COPY_BYTES / (copy_f * 1024.0)
    ws = COPY_BYTES / (copy_w * 1024.0)
    lines = ["# HBM traffic per dispatch from rocprofv3 counters, Engram prefill T=4096, dim 5120, hc 4",
             "# commands (two runs, one counter each; repository root = <repo>):",
             "#   " + cmd_base % ("--pmc FETCH_SIZE --kernel-trace", "--steps 5 --warmup 3 --copy-calibration"),
             "#   " + cmd_base % ("--pmc WRITE_SIZE --kernel-trace", "--steps 5 --warmup 3 --copy-calibration"),
             "# calibration: a device copy of exactly 1 GiB reads FETCH_SIZE = %.1f KiB (scale %.4f)"
             % (copy_f, fs),
             "#   and WRITE_SIZE = %.1f KiB (scale %.4f)" % (copy_w, ws),
             "# source digest of the fused projection (bench.kernel_source_digest): %s"
             % kernel_source_digest(),
             "",
             "%-26s %14s %14s %12s %12s" % ("kernel", "FETCH_KiB", "WRITE_KiB", "fetch_MB*", "write_MB*")]
    total = {"fetch": 0.0, "write": 0.0}
    for k in sorted(set(fetch) | set(write)):
        f, w_ = fetch.get(k, 0.0), write.get(k, 0.0)
        lines.append("%-26s %14.1f %14.1f %12.1f %12.1f" % (k, f, w_, f * 1024 * fs / 1e6,
                                                            w_ * 1024 * ws / 1e6))
        if is_fused(k):
            total["fetch"] += f * 1024 * fs
            total["write"] += w_ * 1024 * ws
    lines.append("# * scaled by the calibration copy; MB = 1e6 bytes.")
    lines.append("# engram_wkv_gate_partials per call: fetch %.1f MB + write %.1f MB" %
                 (total["fetch"] / 1e6, total["write"] / 1e6))
    open(os.path.join(ROOT, "profiles", "engram_prefill_T4096_traffic.txt"), "w").write(
        "\n".join(lines) + "\n")
    rec = {"kernel": "engram_wkv_gate_partials (" + " + ".join(FUSED_KERNELS) + ")",
           "workload": "prefill T=4096 dim 5120 hc 4", "tokens": tokens,
           "summary": "engram_prefill_T4096_traffic.txt (the rocprofv3 commands in its header)",
           "source_digest": kernel_source_digest(),
           "fetch_bytes_per_launch": int(total["fetch"]),
           "write_bytes_per_launch": int(total["write"]),
           "fetch_scale": fs, "write_scale": ws,
           "hbm_bytes_per_launch": int(total["fetch"] + total["write"])}
    json.dump(rec, open(TRAFFIC_FILE, "w"), indent=1)
    print("wrote profiles/engram_prefill_T4096_kernel_stats.txt, "
          "profiles/engram_prefill_T4096_traffic.txt, %s" % os.path.relpath(TRAFFIC_FILE, ROOT))


def summarize_decode_traffic(fetch_dir, write_dir):
    """HBM bytes per engram_wkv_gathered call at M = 64 (prep_kernel +
    wkv_gathered_64, the decode roofline's kernels) from one FETCH_SIZE and one
    WRITE_SIZE run of the decode bench, scaled by its 1 GiB calibration copy."""
    cmd = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc %s --kernel-trace --output-format csv "
           "-d <out> -o <name> -- python3 <repo>/bench.py --workload decode --copy-calibration")
    fetch, copy_f = _counter_means(fetch_dir, "FETCH_SIZE")
    write, copy_w = _counter_means(write_dir, "WRITE_SIZE")
    fs = COPY_BYTES / (copy_f * 1024.0)
    ws = COPY_BYTES / (copy_w * 1024.0)
    lines = ["# HBM traffic per dispatch from rocprofv3 counters, Engram decode B=64 (one token "
             "per sequence), dim 5120, hc 4",
             "# commands (two runs, one counter each; repository root = <repo>):",
             "#   " + cmd % "FETCH_SIZE", "#   " + cmd % "WRITE_SIZE",
             "# calibration: a device copy of exactly 1 GiB reads FETCH_SIZE = %.1f KiB (scale %.4f)"
             % (copy_f, fs),
             "#   and WRITE_SIZE = %.1f KiB (scale %.4f)" % (copy_w, ws),
             "# source digest of the gathered projection (bench.kernel_source_digest): %s"
             % kernel_source_digest(),
             "",
             "%-34s %14s %14s %12s %12s" % ("kernel", "FETCH_KiB", "WRITE_KiB", "fetch_MB*", "write_MB*")]
    total = {"fetch": 0.0, "write": 0.0}
    for k in sorted(set(fetch) | set(write)):
        f, w_ = fetch.get(k, 0.0), write.get(k, 0.0)
        lines.append("%-34s %14.1f %14.1f %12.2f %12.2f" % (k, f, w_, f * 1024 * fs / 1e6,
                                                            w_ * 1024 * ws / 1e6))
        if k.split("<")[0] in DECODE_KERNELS:
            total["fetch"] += f * 1024 * fs
            total["write"] += w_ * 1024 * ws
    lines.append("# * scaled by the calibration copy; MB = 1e6 bytes.")
    lines.append("# engram_wkv_gathered at M = 64 per call: fetch %.2f MB + write %.2f MB "
                 "(algorithmic: W 78.64 + fp8 rows and scales 0.10 + kv 3.28 = 82.02 MB)"
                 % (total["fetch"] / 1e6, total["write"] / 1e6))
    open(os.path.join(ROOT, "profiles", "engram_decode_B64_traffic.txt"), "w").write(
        "\n".join(lines) + "\n")
    rec = {"kernel": "engram_wkv_gathered at M = 64 (" + " + ".join(DECODE_KERNELS) + ")",
           "workload": "decode B=64 dim 5120 hc 4", "tokens": 64,
           "summary": "engram_decode_B64_traffic.txt (the rocprofv3 commands in its header)",
           "source_digest": kernel_source_digest(),
           "fetch_bytes_per_launch": int(total["fetch"]),
           "write_bytes_per_launch": int(total["write"]),
           "fetch_scale": fs, "write_scale": ws,
           "hbm_bytes_per_launch": int(total["fetch"] + total["write"])}
    json.dump(rec, open(DECODE_TRAFFIC_FILE, "w"), indent=1)
    print("wrote profiles/engram_decode_B64_traffic.txt, %s" % os.path.relpath(DECODE_TRAFFIC_FILE, ROOT))


def main():
    args = parse()
    if args.summarize:
        summarize(*args.summarize)
        return
    if args.summarize_stats:
        summarize_stats(*args.summarize_stats)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.summarize_decode_traffic:
        summarize_decode_traffic(*args.summarize_decode_traffic)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the Engram path is built and timed per GPU "
              "(split across GPUs it would take whole sequences, or token ranges plus a "
              "look-back halo of raw ids, per GPU, with no activation exchange).",
              file=sys.stderr)
        sys.exit(2)
    if args.workload == "decode":
        decode(args)
        return
    if args.workload == "long_mixed":
        long_mixed(args)
        return
    if args.workload == "hash_layers":
        hash_layers(args)
        return
    if args.workload == "gate_stress":
        gate_stress(args)
        return
    import numpy as np
    import torch

    import gram_memory_layer_amd as ge
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.config("prefill")
    t = synth.hash_tables(cfg)
    g = ge.Geometry.make(cfg.dim, cfg.hc_mult, cfg.max_ngram_size, cfg.n_heads, cfg.head_dim,
                         t["num_embeddings"], cfg.vocab, cfg.pad_id, cfg.norm_eps)
    tables = {k: torch.from_numpy(t[k]).to(dev) for k in ("token_map", "mult", "prime", "offset")}
    table, scales = synth.embedding_table(cfg, t["num_embeddings"], dev)
    w = synth.wkv_weight(cfg, dev)
    q, k = synth.qk_weights(cfg, dev)
    B, T = cfg.B, cfg.T
    n_tok = B * T
    ids_np = synth.token_ids(cfg, B, T)
    ids = torch.from_numpy(ids_np).to(dev)
    x = synth.activations(cfg, n_tok, dev).reshape(B, T, cfg.hc_mult, cfg.dim)
    mask = torch.from_numpy(synth.token_mask(cfg, B, T)).to(dev)
    out = torch.empty_like(x)
    layer = ge.EngramLayer(g, tables, table, scales, w, q, k)
    ws = layer.workspace(n_tok)
    stream = torch.cuda.current_stream(dev)

    def step():
        ge.engram_forward(g, tables, table, scales, w, q, k, x, ids, mask=mask, out=out,
                          workspace=ws)

    # The cold-cache forwards and then the stage timings run before the
    # forward's warm-up and timed steps: the timed forwards then run at the
    # clocks the part holds under load (after an idle phase a few warm-up
    # forwards leave it in its clock ramp, 3-4% slower at 20 warm-up forwards
    # than at 200), and after stage work that leaves no flushed lines behind.

    # the same forward with the caches cold: a 512 MiB write (past the 256 MB
    # MALL and the 8 x 4 MB L2) between forwards, each forward timed alone
    flush = torch.empty(1 << 29, dtype=torch.uint8, device=dev)
    cold = []
    for _ in range(10):
        flush.fill_(1)
        s0 = torch.cuda.Event(enable_timing=True)
        s1 = torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        step()
        s1.record(stream)
        s1.synchronize()
        cold.append(s0.elapsed_time(s1))
    del flush
    cold_ms = sorted(cold)[len(cold) // 2]

    # ---- per-stage launch times (each stage alone, same inputs, same stream).
    # The forward runs hash_prep_kernel (the hash written straight as the
    # projection's row offsets and scales, with q*k) -> the projection's
    # persistent and tail kernels -> gate_from_partials; the stage calls below
    # are the public entry points (engram_hash writes hash ids, and the
    # projection call starts with its own prep kernel), plus the less fused
    # alternatives, timed for comparison
    if not ge.engram_gate_partials_supported(g, n_tok):
        raise SystemExit("the fully fused prefill path does not apply to this workload")
    hid = ge.engram_hash(g, tables, ids)
    rows = ge.engram_gather(g, table, scales, hid)
    kv = ge.engram_wkv(g, rows, w)
    scratch = torch.empty(ge.engram_wkv_gathered_scratch_size(g, n_tok), dtype=torch.uint8,
                          device=dev)
    xf = x.reshape(n_tok, cfg.hc_mult, cfg.dim)
    v, part = ge.engram_wkv_gate_partials(g, table, scales, hid, w, xf, q, k, scratch=scratch)
    outf = out.reshape(n_tok, cfg.hc_mult, cfg.dim)
    ge.engram_gate_from_partials(g, xf, v, part, mask=mask, out=outf)
    ge.engram_wkv_gathered(g, table, scales, hid, w, kv=kv, scratch=scratch)
    ge.engram_gate_add(g, x, kv, q, k, mask=mask, out=out)
    torch.cuda.synchronize()
    reps = max(args.steps, 50)
    st_gather = time_gpu(lambda: ge.engram_gather(g, table, scales, hid, rows=rows), reps, stream)
    st_wkv = time_gpu(lambda: ge.engram_wkv(g, rows, w, kv=kv), reps, stream)
    st_fused = time_gpu(
        lambda: ge.engram_wkv_gathered(g, table, scales, hid, w, kv=kv, scratch=scratch), reps,
        stream)
    st_gate = time_gpu(lambda: ge.engram_gate_add(g, x, kv, q, k, mask=mask, out=out), reps,
                            stream)
    st_hash = time_gpu(lambda: ge.engram_hash(g, tables, ids, hash_ids=hid), reps, stream)
    st_proj = time_gpu(
        lambda: ge.engram_wkv_gate_partials(g, table, scales, hid, w, xf, q, k, v=v, part=part,
                                            scratch=scratch), reps, stream)
    st_pgate = time_gpu(
        lambda: ge.engram_gate_from_partials(g, xf, v, part, mask=mask, out=outf), reps, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    sec = time_launches(step, args.steps, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tokens_per_s = n_tok / sec

    flops_per_token = 2 * g.K * g.N
    wkv_flops = flops_per_token * n_tok
    achieved = wkv_flops / st_proj / 1e12
    traffic = traffic_record(n_tok)
    # the gate from partials: x and v read, out written, partial pairs read
    gate_bytes = n_tok * (2 * g.hc_mult * g.dim * 2 + g.dim * 2 +
                          g.hc_mult * (g.dim // 128) * 8)
    rec = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Engram prefill forward, B=1 T=4096, dim=5120 hc=4, 24 hash cols x "
                               "head_dim 64 (wkv 1536->25600), 25,160,950-row fp8 e4m3 table",
                   "global_batch": B, "seq_len": T, "parallelism": "single GPU"},
        "roofline": {"kernel": "engram_wkv_gate_partials", "bound": "mfma",
                     "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
        "stages_us": {"hash": round(st_hash * 1e6, 2),
                      "wkv_gate_partials": round(st_proj * 1e6, 2),
                      "gate_from_partials": round(st_pgate * 1e6, 2),
                      "alt_wkv_gathered": round(st_fused * 1e6, 2),
                      "alt_gate_add": round(st_gate * 1e6, 2),
                      "alt_gather": round(st_gather * 1e6, 2),
                      "alt_wkv": round(st_wkv * 1e6, 2)},
        "gate_hbm": {"kernel": "engram_gate_from_partials",
                     "achieved": round(gate_bytes / st_pgate / 1e9, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gate_bytes / st_pgate / 1e9 / PEAK_HBM_GBS, 4)},
        "ms_per_step_cold_caches": round(cold_ms, 4),
        "wall_s": round(wall, 3),
    }

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        rec["copy_calibration_bytes"] = 1 << 30
        del src, dst

    # the same projection against the part's measured matrix-core ceiling
    ceil = mfma_ceiling(dev, stream, w)
    ceil["projection_frac_of_changing_operand_ceiling"] = round(
        achieved / ceil["changing_operands"]["tflops"], 4)
    ceil["projection_frac_of_lds_fed_ceiling"] = round(achieved / ceil["lds_fed"]["tflops"], 4)
    rec["mfma_ceiling"] = ceil

    if not args.no_cpu_baseline:
        if args.cpu_threads > 0:
            import oracle
            oracle.set_num_threads(args.cpu_threads)
        rec["cpu_baseline"] = cpu_baseline(cfg, t, table, scales, w, q, k, x, ids_np, mask,
                                           args.cpu_sample)
    print(json.dumps(rec), flush=True)


def decode(args):
    """Decode: B=64 sequences, 128 steps of one token after a 512-token
    prefill of the hash state.  The 128 forwards are captured once in a graph
    (the library allocates nothing and needs no host synchronisation) and the
    graph is replayed; one step = one forward of 64 tokens.  The roofline is
    the projection's weight stream: W (78.6 MB) + the fp8 rows + kv per step
    over the event-timed engram_wkv_gathered call at M = 64."""
    import torch

    import gram_memory_layer_amd as ge
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.config("decode")
    t = synth.hash_tables(cfg)
    g = ge.Geometry.make(cfg.dim, cfg.hc_mult, cfg.max_ngram_size, cfg.n_heads, cfg.head_dim,
                         t["num_embeddings"], cfg.vocab, cfg.pad_id, cfg.norm_eps)
    tables = {k: torch.from_numpy(t[k]).to(dev) for k in ("token_map", "mult", "prime", "offset")}
    table, scales = synth.embedding_table(cfg, t["num_embeddings"], dev)
    w = synth.wkv_weight(cfg, dev)
    q, k = synth.qk_weights(cfg, dev)
    B, S = cfg.B, cfg.steps
    state0 = torch.full((B, cfg.max_ngram_size - 1), cfg.pad_id, dtype=torch.int32, device=dev)
    ge.engram_hash(g, tables, torch.from_numpy(synth.token_ids(cfg, B, cfg.prefill,
                                                               name="prefill_ids")).to(dev),
                   state=state0)
    step_ids = synth.token_ids(cfg, B, S, name="step_ids")
    ids = [torch.from_numpy(step_ids[:, s:s + 1].copy()).to(dev) for s in range(S)]
    # fresh activations for every step (2.6 MB each, 128 steps)
    xs = [synth.activations(cfg, B, dev, name="x_step%d" % s).reshape(B, 1, cfg.hc_mult, cfg.dim)
          for s in range(S)]
    out = torch.empty_like(xs[0])
    ws = torch.empty(ge.engram_forward_workspace_size(g, B), dtype=torch.uint8, device=dev)
    state = state0.clone()

    def steps():
        for s in range(S):
            ge.engram_forward(g, tables, table, scales, w, q, k, xs[s], ids[s], state=state,
                              out=out, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        steps()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        steps()
    stream = torch.cuda.current_stream(dev)
    for _ in range(max(args.warmup // 10, 2)):
        graph.replay()
    torch.cuda.synchronize()
    reps = max(args.steps // 10, 3)
    t0 = time.perf_counter()
    sec = time_launches(graph.replay, reps, stream) / S  # per step
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    eager = time_launches(steps, 2, stream) / S

    # the block's own forward takes hash ids (one engram_hash_layers launch
    # serves every layer of a step): the same 128 steps from their hash ids
    hstate = state0.clone()
    hids = [ge.engram_hash(g, tables, ids[s], state=hstate) for s in range(S)]

    def steps_hashed():
        for s in range(S):
            ge.engram_forward_hashed(g, table, scales, w, q, k, xs[s], hids[s], out=out,
                                     workspace=ws)

    with torch.cuda.stream(side):
        steps_hashed()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph_h = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph_h):
        steps_hashed()
    for _ in range(2):
        graph_h.replay()
    sec_hashed = time_launches(graph_h.replay, reps, stream) / S
    del graph_h

    hid = ge.engram_hash(g, tables, ids[0])
    kv = torch.empty((B, g.N), dtype=torch.bfloat16, device=dev)
    scratch = torch.empty(ge.engram_wkv_gathered_scratch_size(g, B), dtype=torch.uint8, device=dev)
    ge.engram_wkv_gathered(g, table, scales, hid, w, kv=kv, scratch=scratch)
    st_proj = time_gpu(lambda: ge.engram_wkv_gathered(g, table, scales, hid, w, kv=kv,
                                                      scratch=scratch), 200, stream)
    proj_bytes = g.N * g.K * 2 + B * g.n_hash_cols * (64 + 2) + B * g.N * 2
    if args.copy_calibration:  # a 1 GiB copy for the counter runs to scale by
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    rec = {
        "metric": "Engram decode tokens/s @dim5120 hc4 (1 GPU), B=64, 128 steps after 512",
        "value": round(B / sec, 1), "unit": "tokens/s", "n_gpus": 1, "steps": S * reps,
        "warmup": max(args.warmup // 10, 2) * S, "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Engram decode, B=64 x 1 token per step, 128 steps replayed as "
                               "one graph, dim=5120 hc=4, 24 hash cols x head_dim 64",
                   "global_batch": B, "seq_len": 1, "parallelism": "single GPU"},
        "roofline": {"kernel": "engram_wkv_gathered (M=64)", "bound": "hbm",
                     "achieved": round(proj_bytes / st_proj / 1e9, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(proj_bytes / st_proj / 1e9 / PEAK_HBM_GBS, 4),
                     "traffic": traffic_record(B, DECODE_TRAFFIC_FILE)},
        "eager_ms_per_step": round(eager * 1e3, 4),
        "from_hash_ids_ms_per_step": round(sec_hashed * 1e3, 4),
        "projection_us": round(st_proj * 1e6, 2),
        "wall_s": round(wall, 3),
    }
    print(json.dumps(rec), flush=True)


def long_mixed(args):
    """Long mixed prefill: B=1, T=32768, Zipf(1.1) token ids, 30% of the
    positions masked in spans of 256..1024.  The forward projects only the
    live positions (packed in order).  Also timed: the same work through the
    dense stage calls (every position projected, then the masked gate), and
    engram_wkv_gate_partials on the live positions alone, whose flops over
    its call time give the roofline line."""
    import numpy as np
    import torch

    import gram_memory_layer_amd as ge
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.config("long_mixed")
    t = synth.hash_tables(cfg)
    g = ge.Geometry.make(cfg.dim, cfg.hc_mult, cfg.max_ngram_size, cfg.n_heads, cfg.head_dim,
                         t["num_embeddings"], cfg.vocab, cfg.pad_id, cfg.norm_eps)
    tables = {k: torch.from_numpy(t[k]).to(dev) for k in ("token_map", "mult", "prime", "offset")}
    table, scales = synth.embedding_table(cfg, t["num_embeddings"], dev)
    w = synth.wkv_weight(cfg, dev)
    q, k = synth.qk_weights(cfg, dev)
    B, T = cfg.B, cfg.T
    n_tok = B * T
    ids = torch.from_numpy(synth.token_ids(cfg, B, T)).to(dev)
    x = synth.activations(cfg, n_tok, dev).reshape(B, T, cfg.hc_mult, cfg.dim)
    mask_np = synth.token_mask(cfg, B, T)
    mask = torch.from_numpy(mask_np).to(dev)
    out = torch.empty_like(x)
    layer = ge.EngramLayer(g, tables, table, scales, w, q, k)
    ws = layer.workspace(n_tok)
    stream = torch.cuda.current_stream(dev)
    steps = max(args.steps // 5, 5)
    warm = max(args.warmup // 5, 3)

    def step():
        ge.engram_forward(g, tables, table, scales, w, q, k, x, ids, mask=mask, out=out,
                          workspace=ws)

    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    sec = time_launches(step, steps, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # the dense stage calls over the same inputs
    xf = x.reshape(n_tok, cfg.hc_mult, cfg.dim)
    outf = out.reshape(n_tok, cfg.hc_mult, cfg.dim)
    hid = ge.engram_hash(g, tables, ids).reshape(n_tok, -1)
    v, part = ge.engram_wkv_gate_partials(g, table, scales, hid, w, xf, q, k)
    scratch = torch.empty(ge.engram_wkv_gathered_scratch_size(g, n_tok), dtype=torch.uint8,
                          device=dev)

    def dense():
        ge.engram_hash(g, tables, ids, hash_ids=hid.reshape(B, T, -1))
        ge.engram_wkv_gate_partials(g, table, scales, hid, w, xf, q, k, v=v, part=part,
                                    scratch=scratch)
        ge.engram_gate_from_partials(g, xf, v, part, mask=mask.reshape(-1), out=outf)

    dense()
    sec_dense = time_gpu(dense, steps, stream)
    # the projection over the live positions alone
    live = torch.from_numpy(np.nonzero(mask_np.reshape(-1))[0]).to(dev)
    n_live = int(live.numel())
    hid_l = hid.index_select(0, live).contiguous()
    x_l = xf.index_select(0, live).contiguous()
    v_l, part_l = ge.engram_wkv_gate_partials(g, table, scales, hid_l, w, x_l, q, k)
    sec_proj = time_gpu(
        lambda: ge.engram_wkv_gate_partials(g, table, scales, hid_l, w, x_l, q, k, v=v_l,
                                            part=part_l), steps, stream)
    achieved = 2 * g.K * g.N * n_live / sec_proj / 1e12
    # the row gather on its own over every position (Zipf ids: rows repeat)
    rows = ge.engram_gather(g, table, scales, hid)
    sec_gather = time_gpu(lambda: ge.engram_gather(g, table, scales, hid, rows=rows), steps,
                          stream)
    gather_read = n_tok * g.n_hash_cols * (g.head_dim + g.head_dim // 32)
    gather_write = n_tok * g.K * 2
    # the forward with out aliasing x (a masked position is then not touched);
    # on a copy of x, which it overwrites
    xi = x.clone()

    def step_in_place():
        ge.engram_forward(g, tables, table, scales, w, q, k, xi, ids, mask=mask, out=xi,
                          workspace=ws)

    step_in_place()
    sec_inplace = time_launches(step_in_place, steps, stream)
    rec = {
        "metric": "Engram long mixed prefill tokens/s @dim5120 hc4 (1 GPU), T=32768, 30% masked",
        "value": round(n_tok / sec, 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warm, "ms_per_step": round(sec * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "Engram long mixed prefill, B=1 T=32768, Zipf(1.1) ids, 30% "
                               "masked in spans of 256..1024, dim=5120 hc=4",
                   "global_batch": B, "seq_len": T, "parallelism": "single GPU"},
        "roofline": {"kernel": "engram_wkv_gate_partials (live positions)", "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None},
        "live_positions": n_live,
        "dense_stage_calls_ms": round(sec_dense * 1e3, 4),
        "out_aliasing_x_ms": round(sec_inplace * 1e3, 4),
        "gather_hbm": {"kernel": "engram_gather (every position)",
                       "achieved": round((gather_read + gather_write) / sec_gather / 1e9, 1),
                       "peak": PEAK_HBM_GBS, "unit": "GB/s",
                       "frac": round((gather_read + gather_write) / sec_gather / 1e9 /
                                     PEAK_HBM_GBS, 4),
                       "read_bytes": gather_read, "write_bytes": gather_write,
                       "us": round(sec_gather * 1e6, 2)},
        "live_projection_ms": round(sec_proj * 1e3, 4),
        "wall_s": round(wall, 3),
    }
    print(json.dumps(rec), flush=True)


def hash_layers(args):
    """Eight Engram layers' hashes of the T=4096 prefill: one engram_hash_layers
    launch against eight engram_hash calls (each layer with its own tables and
    table size, drawn like the prefill's with a seed of its own).  Bytes per
    call: ids once, token ids and table reads from L2, 96 B of hash ids per
    position and layer written."""
    import dataclasses

    import torch

    import gram_memory_layer_amd as ge
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    base = synth.config("prefill")
    n_layers = 8
    geoms, tabs = [], []
    for l in range(n_layers):
        cfg = dataclasses.replace(base, index=200 + l)
        t = synth.hash_tables(cfg)
        geoms.append(ge.Geometry.make(cfg.dim, cfg.hc_mult, cfg.max_ngram_size, cfg.n_heads,
                                      cfg.head_dim, t["num_embeddings"], cfg.vocab, cfg.pad_id,
                                      cfg.norm_eps))
        tabs.append({k: torch.from_numpy(t[k]).to(dev)
                     for k in ("token_map", "mult", "prime", "offset")})
    B, T = base.B, base.T
    ids = torch.from_numpy(synth.token_ids(base, B, T)).to(dev)
    out = torch.empty((n_layers, B, T, geoms[0].n_hash_cols), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def one():
        ge.engram_hash_layers(geoms, tabs, ids, hash_ids=out)

    def separate():
        for l in range(n_layers):
            ge.engram_hash(geoms[l], tabs[l], ids, hash_ids=out[l])

    # both captured in HIP graphs and replayed, so that the times are the
    # GPU's (a launch from Python costs more than these kernels take)
    one()
    separate()
    torch.cuda.synchronize()
    graphs = []
    for fn in (one, separate):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for _ in range(10):
                fn()
        graphs.append(gr)
    for gr in graphs:
        gr.replay()
    torch.cuda.synchronize()
    steps = max(args.steps // 10, 5)
    sec = time_launches(graphs[0].replay, steps, stream) / 10
    sec_sep = time_launches(graphs[1].replay, steps, stream) / 10
    steps *= 10
    rec = {
        "metric": "Engram hash of 8 layers, positions/s (1 GPU), T=4096",
        "value": round(B * T / sec, 1), "unit": "positions/s", "n_gpus": 1, "steps": steps,
        "warmup": 1, "ms_per_step": round(sec * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int64", "data": "synthetic",
        "config": {"workload": "hash ids of 8 Engram layers (own tables each), B=1 T=4096, "
                               "24 hash columns", "global_batch": B, "seq_len": T,
                   "parallelism": "single GPU"},
        "separate_calls_ms": round(sec_sep * 1e3, 4),
    }
    print(json.dumps(rec), flush=True)


def gate_stress(args):
    """The gate and add alone (engram_gate_add) over B=8 x T=8192 tokens whose
    kv is given: keys built from the stream (25% exactly orthogonal under the
    weights, 15% near-zero dot products, the rest c*x + noise), value N(0,1).
    Algorithmic bytes: x and kv read, out written = 133,120 B per token
    (8.72 GB)."""
    import torch

    import gram_memory_layer_amd as ge
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.config("gate_stress")
    t = synth.hash_tables(cfg)
    g = ge.Geometry.make(cfg.dim, cfg.hc_mult, cfg.max_ngram_size, cfg.n_heads, cfg.head_dim,
                         t["num_embeddings"], cfg.vocab, cfg.pad_id, cfg.norm_eps)
    n = cfg.n_tokens
    x = synth.activations(cfg, n, dev)
    q, k = synth.qk_weights(cfg, dev)
    kv, _ = synth.gate_stress_kv(cfg, x, q, k)
    out = torch.empty_like(x)
    stream = torch.cuda.current_stream(dev)

    def step():
        ge.engram_gate_add(g, x, kv, q, k, out=out)

    # warm-up as long as the other workloads' (a few calls leave the part
    # below its steady clocks: 3 calls measured 8% slower than 20)
    warm = max(args.warmup, 3)
    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    steps = max(args.steps // 5, 10)
    sec = time_launches(step, steps, stream)
    nbytes = n * (2 * cfg.hc_mult * cfg.dim * 2 + g.N * 2)
    gbs = nbytes / sec / 1e9
    rec = {
        "metric": "Engram gate and add GB/s @dim5120 hc4 (1 GPU), 65,536 tokens",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": round(sec * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "Engram gate and add alone, B=8 T=8192, dim=5120 hc=4, given kv "
                               "(orthogonal, near-zero and scaled keys)",
                   "global_batch": cfg.B, "seq_len": cfg.T, "parallelism": "single GPU"},
        "roofline": {"kernel": "engram_gate_add", "bound": "hbm", "achieved": round(gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": None},
    }
    print(json.dumps(rec), flush=True)


def cpu_baseline(cfg, t, table, scales, w, q, k, x, ids_np, mask, n_sample):
    """The oracle on the first `n_sample` positions of the same workload:
    hash (whole prefix it needs), row gather, fp64 projection, gate."""
    import numpy as np
    import torch

    import oracle
    b = lambda z: z.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    S = n_sample
    hid = None
    geom = {"max_ngram_size": cfg.max_ngram_size, "n_heads": cfg.n_heads, "vocab": cfg.vocab,
            "pad_id": cfg.pad_id, "hc_mult": cfg.hc_mult, "dim": cfg.dim,
            "norm_eps": cfg.norm_eps}
    # the rows the sample touches, copied out of the device table (input bytes)
    st = oracle.HashState(1, S + 8)
    hid = oracle.hash_ids(t, geom, st, ids_np[:, :S])
    uniq, inv = np.unique(hid.reshape(-1), return_inverse=True)
    idx = torch.from_numpy(uniq.astype(np.int64)).to(table.device)
    tab = table.index_select(0, idx).cpu().numpy()
    sc = scales.index_select(0, idx).cpu().numpy()
    wb, qb, kb = b(w), b(q), b(k)
    xb = b(x.reshape(-1, cfg.hc_mult, cfg.dim)[:S])
    mk = mask.reshape(-1)[:S].cpu().numpy()
    t0 = time.perf_counter()
    st = oracle.HashState(1, S + 8)
    h = oracle.hash_ids(t, geom, st, ids_np[:, :S])
    _, inv = np.unique(h.reshape(-1), return_inverse=True)
    rows = oracle.embed_rows(tab, sc, inv.astype(np.int32)).reshape(S, -1)
    kv = oracle.linear(rows, wb)
    oracle.gate_and_add(xb, kv, qb, kb, cfg.norm_eps, mk)
    el = time.perf_counter() - t0
    return {"value": round(S / el, 3), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": "first %d positions of the T=4096 prefill (all four "
                                        "stages, fp64), %.1f s" % (S, el),
            "nproc": len(os.sched_getaffinity(0)), "host_cpus": os.cpu_count(),
            "cpu_model": cpu_model()}


def cpu_model() -> str:
    """The host CPU's model name (what lscpu reports), from /proc/cpuinfo."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
