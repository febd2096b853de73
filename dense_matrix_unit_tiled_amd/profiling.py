"""Summaries of rocprofv3 output for the benchmark (host-side tooling, no GPU work).

``bench.py --summarize DIR`` reads the CSV files that these rocprofv3 runs of
``bench.py`` wrote under DIR and writes short text summaries into ``profiles/``:

  kernel trace   rocprofv3 --kernel-trace --stats --output-format csv -d DIR/trace -o run
                     -- python3 bench.py --workload W --steps 200 --warmup 1000 --no-cpu-baseline
  HBM traffic    rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/fetch -o run
                     -- python3 bench.py --workload W --steps 100 --warmup 1000 --no-cpu-baseline
                        --copy-calibration 256
                 (the same with WRITE_SIZE into DIR/write)
  matrix cores   rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_LDS_BANK_CONFLICT
                     SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS SQ_INSTS_MFMA GRBM_GUI_ACTIVE
                     --output-format csv -d DIR/sq -o run -- python3 bench.py ... (as above)

FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what the same
counter reads for a plain device-to-device copy of 256 MiB (the
``--copy-calibration`` leg): factor = copied bytes / counter bytes.

The GPU raises its shader clock only after a few hundred back-to-back
launches, so the figures that depend on time or clock (the kernel's average
duration, the matrix-core busy fraction) are taken over the last dispatches
of each run -- the ones the benchmark times -- not over the warm-up.
"""
from __future__ import annotations

import csv
import glob
import json
import os
import statistics
from collections import defaultdict

COPY_MIB = 256
# A shader clock is derived from GRBM_GUI_ACTIVE only over dispatches at least this long, and only
# when it does not exceed the chip's peak shader clock.
MIN_CLOCK_DISPATCH_US = 50.0
MAX_SCLK_GHZ = 2.4


def _rows(pattern: str):
    out = []
    for f in glob.glob(pattern, recursive=True):
        with open(f) as fh:
            out.extend(csv.DictReader(fh))
    return out


def _counter_means(rows, last: int = 0):
    """{(kernel name, counter): mean value per dispatch} (over the last `last` dispatches if > 0)"""
    acc = defaultdict(list)
    for r in rows:
        acc[(r["Kernel_Name"], r["Counter_Name"])].append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    out = {}
    for k, v in acc.items():
        vals = [x for _, x in sorted(v)]
        if last:
            vals = vals[-last:]
        out[k] = sum(vals) / len(vals)
    return out


def _timed_average_us(rows, timed: int):
    """Average duration (us) of the last `timed` GEMM dispatches of a per-dispatch kernel trace."""
    d = sorted((int(r["Dispatch_Id"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
               for r in rows if is_gemm(r["Kernel_Name"]))
    d = [x for _, x in d][-timed:]
    return (sum(d) / len(d), len(d)) if d else (None, 0)


def _pick(means, counter, pred):
    vals = [v for (k, c), v in means.items() if c == counter and pred(k)]
    return vals[0] if vals else None


def is_gemm(name: str) -> bool:
    """A kernel of this library (GEMM kernels and the fused attention kernel)."""
    return "dmu::gemm_" in name or "attn_fwd" in name


def is_copy(name: str) -> bool:
    return "copyBuffer" in name


def summarize(d: str, profiles: str, workload_name: str, kernel_label: str, source_digest: str,
              commands: dict, timed: int = 200, counted: int = 100, bench_line: dict | None = None) -> dict:
    """Write profiles/<label>_<workload>_*.md and traffic_<workload>.json; return the figures.
    ``bench_line``: the JSON line of a plain bench.py run of the same workload in the same session
    (same GPU, just before the profiled runs), kept beside the figures it is compared with."""
    os.makedirs(profiles, exist_ok=True)
    result = {"workload": workload_name, "kernel": kernel_label, "source_digest": source_digest}
    if bench_line is not None:
        result["bench_same_session"] = {k: bench_line.get(k) for k in ("value", "unit", "ms_per_step", "steps",
                                                                         "warmup")}
        result["bench_same_session"]["kernel"] = bench_line.get("config", {}).get("kernel")

    # kernel trace statistics
    stats = _rows(os.path.join(d, "trace", "**", "*kernel_stats.csv"))
    if stats:
        lines = [f"# Kernel trace: {workload_name}", "",
                 "Command (from the repository root on the GPU host):", "",
                 "```", commands["trace"], "```", "",
                 "| kernel | calls | average (us) | min (us) | max (us) | share |",
                 "|---|---|---|---|---|---|"]
        for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
            name = r["Name"]
            if len(name) > 90:
                name = name[:87] + "..."
            lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                         f"{float(r['Percentage']):.1f}% |")
            if is_gemm(r["Name"]):
                result["avg_us_all_dispatches"] = float(r["AverageNs"]) / 1e3
        avg, n = _timed_average_us(_rows(os.path.join(d, "trace", "**", "*kernel_trace.csv")), timed)
        if avg is not None:
            result["avg_us"] = avg
            lines += ["", f"Library-kernel dispatches timed by the benchmark (the last {n}, after the warm-up that "
                          f"raises the clock): average {avg:.2f} us."]
            if bench_line is not None:
                lines += ["", f"A plain `python3 bench.py --workload ...` run in the same session, just before: "
                              f"{bench_line['ms_per_step'] * 1e3:.2f} us per step (HIP events over "
                              f"{bench_line['steps']} back-to-back launches, after {bench_line['warmup']} "
                              f"warm-up launches), {bench_line['value']} {bench_line['unit']}."]
        open(os.path.join(profiles, f"{kernel_label}_{workload_name}_kernel_trace.md"), "w").write(
            "\n".join(lines) + "\n")

    # HBM traffic, calibrated with the plain copy
    fetch = _counter_means(_rows(os.path.join(d, "fetch", "**", "*counter_collection.csv")), counted)
    write = _counter_means(_rows(os.path.join(d, "write", "**", "*counter_collection.csv")), counted)
    if fetch and write:
        copy_bytes = COPY_MIB * (1 << 20)
        f_copy = _pick(fetch, "FETCH_SIZE", is_copy)
        w_copy = _pick(write, "WRITE_SIZE", is_copy)
        f_gemm = _pick(fetch, "FETCH_SIZE", is_gemm)
        w_gemm = _pick(write, "WRITE_SIZE", is_gemm)
        f_factor = copy_bytes / (f_copy * 1024)
        w_factor = copy_bytes / (w_copy * 1024)
        fetch_b = f_gemm * 1024 * f_factor
        write_b = w_gemm * 1024 * w_factor
        result.update({"fetch_kib_per_dispatch": f_gemm, "write_kib_per_dispatch": w_gemm,
                       "copy_fetch_kib": f_copy, "copy_write_kib": w_copy,
                       "fetch_factor": f_factor, "write_factor": w_factor,
                       "traffic_bytes_per_launch": fetch_b + write_b,
                       "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b})
        md = [f"# HBM traffic: {workload_name}", "",
              "Commands (from the repository root on the GPU host):", "", "```",
              commands["fetch"], commands["write"], "```", "",
              f"Calibration: a plain device copy of {COPY_MIB} MiB reads FETCH_SIZE = {f_copy:.0f} KiB "
              f"and WRITE_SIZE = {w_copy:.0f} KiB, so the factors are {f_factor:.3f} (fetch) and "
              f"{w_factor:.3f} (write).", "",
              "| per kernel launch | counter (KiB) | calibrated bytes |", "|---|---|---|",
              f"| FETCH_SIZE | {f_gemm:.0f} | {fetch_b / 1e6:.1f} MB |",
              f"| WRITE_SIZE | {w_gemm:.0f} | {write_b / 1e6:.1f} MB |",
              f"| total | | {(fetch_b + write_b) / 1e6:.1f} MB |", "",
              f"Kernel source digest: `{source_digest}`."]
        open(os.path.join(profiles, f"traffic_{workload_name}.md"), "w").write("\n".join(md) + "\n")

    # matrix-core and LDS counters
    sq_rows = _rows(os.path.join(d, "sq", "**", "*counter_collection.csv"))
    sq = _counter_means(sq_rows, counted)
    if sq:
        get = lambda c: _pick(sq, c, is_gemm)
        busy = get("SQ_VALU_MFMA_BUSY_CYCLES")
        grbm = get("GRBM_GUI_ACTIVE")
        conflict, active = get("SQ_LDS_BANK_CONFLICT"), get("SQ_LDS_IDX_ACTIVE")
        md = [f"# Matrix-core and LDS counters: {workload_name}", "",
              "Command (from the repository root on the GPU host):", "", "```", commands["sq"], "```", "",
              "| counter (per kernel dispatch, summed over the chip) | value |", "|---|---|"]
        for c in ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_LDS",
                  "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE"):
            v = get(c)
            if v is not None:
                md.append(f"| {c} | {v:.4g} |")
        if busy and grbm:
            # GRBM_GUI_ACTIVE is summed over the 8 XCDs; 1024 SIMDs
            util = busy / (grbm / 8 * 1024)
            md += ["", f"MFMA busy fraction = MFMA_BUSY / (GUI_ACTIVE / 8 XCDs x 1024 SIMDs) = {util:.3f}."]
            result["mfma_busy_fraction"] = util
            dur, _ = _timed_average_us([r for r in sq_rows if r["Counter_Name"] == "GRBM_GUI_ACTIVE"], counted)
            if dur:
                result["counter_dispatch_us"] = dur
                clk = grbm / 8 / (dur * 1e-6) / 1e9
                if dur >= MIN_CLOCK_DISPATCH_US and clk <= MAX_SCLK_GHZ:
                    md += [f"Dispatch duration under counter collection {dur:.2f} us; GUI_ACTIVE / 8 / duration = "
                           f"{clk:.2f} GHz (GUI_ACTIVE cycles per second of dispatch; the busy fraction above "
                           f"uses the same cycles)."]
                    result["gui_active_ghz"] = clk
                else:
                    # GUI_ACTIVE also counts the cycles the command processor spends setting up and
                    # draining the dispatch, outside the dispatch's own start and end timestamps;
                    # over a dispatch of a few microseconds they dominate, and the quotient is no clock
                    md += [f"Dispatch duration under counter collection {dur:.2f} us: too short for a clock "
                           f"from GUI_ACTIVE / 8 / duration ({clk:.2f} GHz would exceed the "
                           f"{MAX_SCLK_GHZ} GHz peak or rest on set-up and drain cycles outside the "
                           f"dispatch); no clock is reported, and the busy fraction above is a lower bound."]
        if conflict is not None and active:
            md += [f"LDS bank-conflict cycles / LDS active cycles = {conflict / active:.3f}."]
            result["lds_conflict_fraction"] = conflict / active
            result["lds_bank_conflict_cycles"] = conflict
        open(os.path.join(profiles, f"{kernel_label}_{workload_name}_counters.md"), "w").write("\n".join(md) + "\n")
    if "traffic_bytes_per_launch" in result:
        json.dump(result, open(os.path.join(profiles, f"traffic_{workload_name}.json"), "w"), indent=1)
    return result


# ---------------------------------------------------------------------------
# Phase log: per-workgroup timestamps that the kernels write while a log is set
# (dmu_phase_log).  One record of 8 64-bit words per workgroup (per tile for the
# persistent kernel, per worker for stream-K):
#   0 start, 1 end of the main loop, 2 end of the partial-sum additions (stream-K
#   finisher; persistent kernel: the next tile's first loads issued; = 1 elsewhere),
#   3 end of the epilogue or of the partial store
#   -- the chip's 100 MHz constant clock (s_memrealtime), as wavefront 0 sees them;
#   4 start, 5 end -- the shader clock counter (s_memtime);
#   6 HW_ID (low word) and XCC_ID (high word) of wavefront 0;
#   7 workgroup id (low word) and K-tiles of the record (high word).
# ---------------------------------------------------------------------------
REALTIME_HZ = 100e6
PHASE_KINDS = {1: "one workgroup per tile", 2: "persistent (one record per tile)",
               3: "stream-K (one record per worker)", 4: "attention (one record per workgroup)"}


def median_launch(raw: dict) -> dict:
    """The launch of a --phases file whose span (first start to last end) is the median one: the
    only launch whose records the file keeps."""
    return raw["launches"][raw["median_launch"]]


def mfma_busy_at_clock(flops: float, flop_per_clock_per_cu: float, compute_units: int, span_us: float,
                       clock_ghz: float) -> float:
    """Matrix-core busy fraction over a launch's span at a given shader clock: the clocks the
    dense matrix cores need for `flops` (flops / (units x dense FLOP per clock and unit)) over the
    clocks in the span."""
    return flops / (compute_units * flop_per_clock_per_cu) / (span_us * 1e-6 * clock_ghz * 1e9)


def phase_summary(log, kind: int, compute_units: int, launch_us: float | None = None) -> dict:
    """Figures of one launch's phase log (`log`: n records of 8 unsigned 64-bit words, as
    written by the kernel): span from the first start to the last end, start skew, per-record
    main loop / partial-sum / epilogue durations (min, median, max), the compute-unit time the
    records cover against compute units x span, the shader clock over each record (s_memtime
    ticks over s_memrealtime time), and the records per XCD.  Pure host arithmetic."""
    recs = [[int(x) for x in r] for r in log]
    if not recs:
        raise ValueError("empty phase log")
    t0 = min(r[0] for r in recs)
    us = lambda ticks: ticks / REALTIME_HZ * 1e6
    start = [us(r[0] - t0) for r in recs]
    loop = [us(r[1] - r[0]) for r in recs]
    fix = [us(r[2] - r[1]) for r in recs]
    epi = [us(r[3] - r[2]) for r in recs]
    end = [us(r[3] - t0) for r in recs]
    dur = [e - s for s, e in zip(start, end)]
    span = max(end)
    clk = [(r[5] - r[4]) / (us(r[3] - r[0]) * 1e3) for r in recs if r[3] > r[0]]
    xcd = defaultdict(list)
    for k, r in enumerate(recs):
        xcd[(r[6] >> 32) & 0xF].append(k)
    stat = lambda v: {"min": round(min(v), 3), "median": round(statistics.median(v), 3), "max": round(max(v), 3)}
    # when the records run in one wave of at most one per compute unit, the compute-unit time
    # they leave unused is compute units x span minus the time they cover
    covered = sum(dur)
    out = {
        "records": len(recs),
        "kind": PHASE_KINDS.get(kind, str(kind)),
        "span_us": round(span, 3),
        "start_skew_us": round(max(start), 3),
        "duration_us": stat(dur),
        "main_loop_us": stat(loop),
        "partial_sums_us": stat(fix),
        "epilogue_us": stat(epi),
        "tail_us": round(span - statistics.median(end), 3),
        "cu_time_covered": round(covered / (compute_units * span), 4),
        "shader_clock_ghz": stat(clk) if clk else None,
        "records_per_xcd": {x: len(v) for x, v in sorted(xcd.items())},
        "per_xcd": {x: {"main_loop_median_us": round(statistics.median(loop[k] for k in v), 3),
                        "end_max_us": round(max(end[k] for k in v), 3),
                        "shader_clock_ghz_median": round(statistics.median(
                            (recs[k][5] - recs[k][4]) / (us(recs[k][3] - recs[k][0]) * 1e3) for k in v), 3)
                        if all(recs[k][3] > recs[k][0] for k in v) else None}
                    for x, v in sorted(xcd.items())},
    }
    if launch_us is not None:
        out["launch_us"] = round(launch_us, 3)
        out["outside_span_us"] = round(launch_us - span, 3)
    return out


def phase_markdown(workload_name: str, kernel: str, command: str, s: dict) -> str:
    """The committed summary of a phase breakdown."""
    f = lambda d: f"{d['min']:.2f} / {d['median']:.2f} / {d['max']:.2f}"
    lines = [f"# Phase breakdown: {workload_name}", "",
             f"Kernel `{kernel}`, {s['records']} records ({s['kind']}), one launch at steady clock "
             "(the median-span launch of those timed).", "",
             "Command (from the repository root on the GPU host):", "", "```", command, "```", "",
             "| phase | µs (min / median / max over records) |", "|---|---|",
             f"| whole record (start to end) | {f(s['duration_us'])} |",
             f"| main loop (prologue loads and every K-tile) | {f(s['main_loop_us'])} |",
             f"| partial sums (stream-K finisher; persistent: next tile's loads issued) | {f(s['partial_sums_us'])} |",
             f"| epilogue (or partial store) | {f(s['epilogue_us'])} |", "",
             "| launch-wide | value |", "|---|---|",
             f"| span, first start to last end | {s['span_us']:.2f} µs |",
             f"| start skew (last start after first) | {s['start_skew_us']:.2f} µs |",
             f"| tail (last end after the median end) | {s['tail_us']:.2f} µs |",
             f"| compute-unit time covered / (units x span) | {s['cu_time_covered']:.3f} |"]
    if "launch_us" in s:
        lines.append(f"| event-timed launch | {s['launch_us']:.2f} µs |")
        lines.append(f"| launch time outside the span | {s['outside_span_us']:.2f} µs |")
    if s.get("shader_clock_ghz"):
        lines.append(f"| shader clock over a record (min / median / max) | {f(s['shader_clock_ghz'])} GHz |")
    if s.get("mfma_busy_at_shader_clock") is not None:
        lines.append(f"| matrix-core busy over the span at the median shader clock | "
                     f"{s['mfma_busy_at_shader_clock']:.3f} |")
    lines.append(f"| records per XCD | {s['records_per_xcd']} |")
    lines += ["", "| XCD | main loop median (µs) | last end (µs) | shader clock median (GHz) |", "|---|---|---|---|"]
    for x, v in s["per_xcd"].items():
        clk = "—" if v["shader_clock_ghz_median"] is None else f"{v['shader_clock_ghz_median']:.3f}"
        lines.append(f"| {x} | {v['main_loop_median_us']:.2f} | {v['end_max_us']:.2f} | {clk} |")
    lines += ["", "Timestamps: the 100 MHz constant clock (10 ns steps) read by wavefront 0 of each "
              "workgroup at its start, after its main loop, after the stream-K partial sums and after "
              "its epilogue; the shader clock counter at start and end.", ""]
    return "\n".join(lines)
