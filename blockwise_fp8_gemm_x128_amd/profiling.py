"""Text summaries of rocprofv3 output from bench.py runs, per kernel function of the library.

    python -m blockwise_fp8_gemm_x128_amd.profiling time STATS_CSV BENCH_LOG [--title T]
        kernel time per function (rocprofv3 --kernel-trace --stats) beside the algorithmic
        work per launch and the HIP-event durations that the same profiled bench run printed
    python -m blockwise_fp8_gemm_x128_amd.profiling traffic FETCH_CSV WRITE_CSV CFETCH_CSV CWRITE_CSV
        HBM bytes per launch per function from two counter passes (FETCH_SIZE, then
        WRITE_SIZE, KiB per dispatch), each scaled by the same counter's reading for a plain
        copy of known size (bench.py --copy-calibration), with one `traffic-record:` line per
        function that bench.py reads back while the function's sources are unchanged
    python -m blockwise_fp8_gemm_x128_amd.profiling ceiling TRACE_CSV BENCH_LOG
        the matrix-core microbenchmark (bench.py --ceiling) under the kernel trace: rocprof
        duration and rate of each timed probe launch beside the bench's own figures
    python -m blockwise_fp8_gemm_x128_amd.profiling sq CSV [CSV ...]
        ratios of shader-sequencer counters (instruction mix, matrix-core and LDS activity,
        waits) per GEMM function, from one or more counter passes

Kernel names are reduced to the names bench.py accounts launches under (the function name,
with "(columns only)" for the transposed quantiser's instance of the two-orientation kernel and
"[pow2]" for power-of-two-scale instances of templated kernels).
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def function_of(kernel_name: str) -> str:
    """Library function name of a rocprofv3 kernel name ('' for kernels of other libraries)."""
    m = re.search(r"puro::\(anonymous namespace\)::([A-Za-z0-9_]+)(<([^>]*)>)?\(", kernel_name)
    if not m:
        return ""
    name, targs = m.group(1), (m.group(3) or "")
    args = [a.strip() for a in targs.split(",")] if targs else []
    if name.startswith("quant_") and args:
        pow2 = args[0] == "true"
        if name == "quant_dual_1x128_kernel" and len(args) > 1 and args[1] == "false":
            name += "(columns only)"
        return name + ("[pow2]" if pow2 else "")
    if args:
        return f"{name}<{', '.join(args)}>"
    return name


def _rows(path):
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def bench_json(log_path: str):
    """The JSON line bench.py printed (last line of the log that parses as a JSON object)."""
    out = None
    with open(log_path) as fh:
        for line in fh:
            line = line.strip()
            if line.startswith("{") and line.endswith("}"):
                try:
                    out = json.loads(line)
                except ValueError:
                    pass
    return out


def time_summary(stats_csv: str, log_path: str, title: str) -> str:
    rows = _rows(stats_csv)
    b = bench_json(log_path) or {}
    fns = b.get("kernels_by_function", {})
    total_ns = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = [title, "",
             "rocprofv3 --stats, this library's kernels (the run's other kernels are torch's input",
             "generation and the copy/calibration helpers):",
             f"  {'function':38s} {'calls':>6s} {'total ms':>9s} {'avg us':>8s} {'min us':>8s} "
             f"{'max us':>8s} {'% time':>7s} {'events us':>9s} {'rate (rocprof avg)':>20s}"]
    per = []
    for r in rows:
        fn = function_of(r["Name"])
        if not fn:
            continue
        avg_us = float(r["AverageNs"]) / 1e3
        ent = fns.get(fn, {})
        work = ent.get("work_per_launch")
        rate = ""
        if work:
            if fn.startswith("gemm"):
                rate = f"{work / (avg_us * 1e-6) / 1e12:9.1f} TFLOP/s ({work / (avg_us * 1e-6) / 5e15:.3f})"
            else:
                rate = f"{work / (avg_us * 1e-6) / 1e9:9.1f} GB/s ({work / (avg_us * 1e-6) / 8e12:.3f})"
        ev = ent.get("avg_launch_us")
        per.append(float(r["TotalDurationNs"]))
        lines.append(f"  {fn:38s} {int(r['Calls']):6d} {float(r['TotalDurationNs']) / 1e6:9.3f} "
                     f"{avg_us:8.2f} {float(r['MinNs']) / 1e3:8.2f} {float(r['MaxNs']) / 1e3:8.2f} "
                     f"{100.0 * float(r['TotalDurationNs']) / total_ns:7.2f} "
                     f"{(f'{ev:9.2f}' if ev else ' ' * 9)} {rate:>20s}")
    lines += ["",
              "'events us' is the same function's average HIP-event duration in the bench's",
              "kernel timing pass of this run; the rate is the algorithmic work per launch",
              "(flops or bytes, averaged over the function's launches in the step) over the",
              "rocprof average, with its fraction of 5.0 PFLOP/s or 8 TB/s in parentheses."]
    if b:
        lines += ["", f"bench line of the profiled run: {b.get('ms_per_step', 0):.2f} ms per step, "
                      f"{b.get('value', 0):.0f} tokens/s (dominant function "
                      f"{b.get('roofline', {}).get('kernel')}, frac "
                      f"{b.get('roofline', {}).get('frac', 0):.3f} by events)"]
    return "\n".join(lines) + "\n"


def _counter_per_fn(path: str):
    acc = {}
    for r in _rows(path):
        fn = function_of(r["Kernel_Name"])
        if not fn:
            continue
        d = acc.setdefault(fn, [0.0, 0])
        d[0] += float(r["Counter_Value"])
        d[1] += 1
    return {fn: v / n for fn, (v, n) in acc.items()}


def _copy_kib(path: str) -> float:
    """Counter reading of the calibration copy (the largest neg kernel dispatch)."""
    best = 0.0
    for r in _rows(path):
        if "neg_kernel" in r["Kernel_Name"]:
            best = max(best, float(r["Counter_Value"]))
    if best <= 0:
        raise SystemExit(f"{path}: no calibration copy dispatch found")
    return best


def traffic_summary(fetch_csv, write_csv, cfetch_csv, cwrite_csv, title: str,
                    algorithmic=None) -> str:
    sys.path.insert(0, ROOT)
    import bench  # the source digests bench.py checks the records against

    copy_bytes = 1 << 30  # bench.py --copy-calibration: 2^28 fp32 read and written once
    ff = copy_bytes / (_copy_kib(cfetch_csv) * 1024.0)
    wf = copy_bytes / (_copy_kib(cwrite_csv) * 1024.0)
    fetch, write = _counter_per_fn(fetch_csv), _counter_per_fn(write_csv)
    lines = [title, "",
             f"Calibration (plain copy, 1 GiB read and 1 GiB written): fetch factor {ff:.5f}, "
             f"write factor {wf:.5f}",
             "(HBM bytes = FETCH_SIZE KiB x 1024 x fetch factor + WRITE_SIZE KiB x 1024 x write "
             "factor)", "",
             f"  {'function':38s} {'read MB':>9s} {'write MB':>9s} {'total MB':>9s} "
             f"{'algorithmic':>11s} {'ratio':>6s}"]
    recs = []
    for fn in sorted(set(fetch) & set(write)):
        rd = fetch[fn] * 1024.0 * ff / 1e6
        wr = write[fn] * 1024.0 * wf / 1e6
        alg = (algorithmic or {}).get(fn)
        lines.append(f"  {fn:38s} {rd:9.2f} {wr:9.2f} {rd + wr:9.2f} "
                     f"{(f'{alg / 1e6:11.2f}' if alg else ' ' * 11)} "
                     f"{(f'{(rd + wr) * 1e6 / alg:6.2f}' if alg else '')}")
        if fn.startswith(("gemm", "quant")):
            recs.append({"function": fn, "fetch_kib_per_launch": fetch[fn],
                         "write_kib_per_launch": write[fn], "fetch_factor": ff,
                         "write_factor": wf, "source_digest": bench.source_digest(fn)})
    lines += ["", "Records read by bench.py (counters averaged over the function's launches; "
                  "valid while its sources hash to source_digest):"]
    lines += ["traffic-record: " + json.dumps(r) for r in recs]
    return "\n".join(lines) + "\n"


def _per_dispatch(path: str):
    """{dispatch id: {'fn': function, counter: value, ...}} of a counter CSV (this library's
    kernels only)."""
    out = {}
    for r in _rows(path):
        fn = function_of(r["Kernel_Name"])
        if not fn:
            continue
        d = out.setdefault(r["Dispatch_Id"], {"fn": fn})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def sq_summary(csvs, title: str) -> str:
    """Ratios of shader-sequencer counters per GEMM function, each summed over the function's
    dispatches in every counter pass given."""
    agg = {}
    for path in csvs:
        for d in _per_dispatch(path).values():
            a = agg.setdefault(d["fn"], {"n": {}})
            a["n"][path] = a["n"].get(path, 0) + 1
            for k, v in d.items():
                if k != "fn":
                    a[k] = a.get(k, 0.0) + v

    def ratio(a, num, den):
        return a[num] / a[den] if num in a and a.get(den) else float("nan")

    lines = [title, "",
             "Ratios (instruction counts or cycles, summed over the function's dispatches):",
             "  VALU/MFMA   SQ_INSTS_VALU / SQ_INSTS_MFMA (the promotion alone: 4 FMAs and 1/4",
             "              multiply per MFMA for fwd/dgrad, 4 multiplies + 4 FMAs for wgrad)",
             "  LDS/MFMA    SQ_INSTS_LDS / SQ_INSTS_MFMA",
             "  SALU/MFMA   SQ_INSTS_SALU / SQ_INSTS_MFMA",
             "  confl/LDS   SQ_LDS_BANK_CONFLICT cycles per LDS instruction",
             "  MFMA busy   SQ_VALU_MFMA_BUSY_CYCLES / (4 x SQ_BUSY_CU_CYCLES): share of SIMD",
             "              cycles the matrix core is busy while the CUs are busy",
             "  LDS active  SQ_LDS_IDX_ACTIVE / SQ_BUSY_CU_CYCLES",
             "  wait        SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (share of wave cycles waiting on a",
             "              memory counter)",
             "  waitLDS     SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES", "",
             f"  {'function':28s} {'n':>3s} {'VALU/MFMA':>9s} {'LDS/MFMA':>8s} {'SALU/MFMA':>9s} "
             f"{'confl/LDS':>9s} "
             f"{'MFMA busy':>9s} {'LDS active':>10s} {'wait':>6s} {'waitLDS':>7s}"]
    for fn in sorted(agg):
        if not fn.startswith("gemm"):
            continue
        a = agg[fn]
        busy = a.get("SQ_BUSY_CU_CYCLES")
        lines.append(
            f"  {fn:28s} {max(a['n'].values()):3d} {ratio(a, 'SQ_INSTS_VALU', 'SQ_INSTS_MFMA'):9.2f} "
            f"{ratio(a, 'SQ_INSTS_LDS', 'SQ_INSTS_MFMA'):8.2f} "
            f"{ratio(a, 'SQ_INSTS_SALU', 'SQ_INSTS_MFMA'):9.2f} "
            f"{ratio(a, 'SQ_LDS_BANK_CONFLICT', 'SQ_INSTS_LDS'):9.3f} "
            f"{(a['SQ_VALU_MFMA_BUSY_CYCLES'] / (4 * busy) if busy else float('nan')):9.3f} "
            f"{(a['SQ_LDS_IDX_ACTIVE'] / busy if busy and 'SQ_LDS_IDX_ACTIVE' in a else float('nan')):10.3f} "
            f"{ratio(a, 'SQ_WAIT_INST_ANY', 'SQ_WAVE_CYCLES'):6.3f} "
            f"{ratio(a, 'SQ_WAIT_INST_LDS', 'SQ_WAVE_CYCLES'):7.3f}")
    return "\n".join(lines) + "\n"


def ceiling_summary(trace_csv: str, log_path: str, title: str) -> str:
    """The matrix-core microbenchmark (bench.py --ceiling) under the kernel trace: each timed
    probe launch's rocprof duration beside the bench's own figures for it. The probe launches
    come in the bench's order, a short warm-up launch before each timed one."""
    b = bench_json(log_path) or {}
    rows = b.get("mfma_ceiling", {})
    iters = b.get("iters", 0)
    launches = [r for r in _rows(trace_csv) if "mfma_probe_kernel" in r["Kernel_Name"]]
    launches.sort(key=lambda r: int(r["Dispatch_Id"]))
    timed = launches[1::2]
    lines = [title, "",
             f"  {'operands | waves per SIMD | loop':66s} {'rocprof ms':>10s} {'PF':>6s} "
             f"{'of 5 PF':>7s} {'events PF':>9s} {'clock GHz':>9s}"]
    for (name, v), r in zip(rows.items(), timed):
        ms = (float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) / 1e6
        waves = int(r["Grid_Size_X"]) // 64
        pf = waves * iters * 8 * 2.0 * 16 * 16 * 128 / (ms * 1e-3) / 1e15
        clk = v["clock_ghz"] * 100.0 / v["ticks_mhz"] if v.get("ticks_mhz") else float("nan")
        lines.append(f"  {name:66s} {ms:10.2f} {pf:6.2f} {pf / 5.0:7.3f} {v['pflops']:9.2f} "
                     f"{clk:9.2f}")
    lines += ["",
              "PF: flops of the timed launch over its rocprof duration ('events PF': over the HIP-event",
              "duration of the bench's own run). clock: the median wave's shader-clock cycles",
              "(s_memtime) over its constant-rate ticks (s_memrealtime, 100 MHz) across the loop."]
    return "\n".join(lines) + "\n"


def main(argv=None):
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("time")
    t.add_argument("stats_csv")
    t.add_argument("bench_log")
    t.add_argument("--title", default="Kernel time per function")
    r = sub.add_parser("traffic")
    r.add_argument("fetch_csv")
    r.add_argument("write_csv")
    r.add_argument("cfetch_csv")
    r.add_argument("cwrite_csv")
    r.add_argument("--bench-log", default=None,
                   help="bench.py output of the counter run, for the algorithmic bytes")
    r.add_argument("--title", default="HBM traffic per launch per function")
    c = sub.add_parser("ceiling")
    c.add_argument("trace_csv")
    c.add_argument("log")
    c.add_argument("--title", default="Matrix-core microbenchmark")
    q = sub.add_parser("sq")
    q.add_argument("csvs", nargs="+")
    q.add_argument("--title", default="Shader-sequencer counters per GEMM function")
    a = p.parse_args(argv)
    if a.cmd == "ceiling":
        sys.stdout.write(ceiling_summary(a.trace_csv, a.log, a.title))
    elif a.cmd == "sq":
        sys.stdout.write(sq_summary(a.csvs, a.title))
    elif a.cmd == "time":
        sys.stdout.write(time_summary(a.stats_csv, a.bench_log, a.title))
    else:
        alg = None
        if a.bench_log:
            b = bench_json(a.bench_log) or {}
            alg = {fn: e.get("traffic_bytes_per_launch")
                   for fn, e in b.get("kernels_by_function", {}).items()}
        sys.stdout.write(traffic_summary(a.fetch_csv, a.write_csv, a.cfetch_csv, a.cwrite_csv,
                                         a.title, alg))


if __name__ == "__main__":
    main()
