"""Benchmark of the gfx950 GEMM: 4096^3 bf16, A and B row-major, fp32 accumulate,
bf16 output (the 4096^3 example of "Tensor Cores, CUTLASS and CuTe", sections
opening and 4.1, here in its NN form).

One step = one D = A*B launch through the C ABI over inputs already resident
in HBM.  W untimed warm-up steps, then exactly K steps timed with HIP events
on the launch stream, bracketed by device synchronisation.  The default W is
large on purpose: after start-up or idle the GPU needs a few hundred launches
(some tens of ms) to raise its shader clock, and timing from a cold start
measures that ramp instead of the kernel.  Prints one JSON
line with the throughput, the MFMA roofline of the kernel and the CPU oracle's
rate on a bounded row slice of the same product (and its per-core rate), plus
medians of individually timed launches, warm and cold (a 1 GiB buffer written
before each), and the dense peak re-derived from this machine's compute units
and clock.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2|c1|c3|c4s|c4o|c5|c5nn|c5dq|c6|lk|lksk|c4fa]
                  [--no-cpu-baseline] [--copy-calibration MiB]
  python bench.py --summarize DIR [--workload W] [--bench-line FILE]   (rocprofv3 output -> profiles/)
"""
from __future__ import annotations

import argparse
import hashlib
import glob
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published dense peaks (matrix cores), TFLOP/s or TOP/s, and HBM3E bandwidth.
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "i8": 5000.0, "e4m3": 5000.0}
# dense matrix-core FLOP (OP) per clock and compute unit of gfx950, by input type
DENSE_FLOP_PER_CLOCK_PER_CU = {"bf16": 4096, "f16": 4096, "i8": 8192, "e4m3": 8192}
PEAK_HBM_GBS = 8000.0

WORKLOAD_NAMES = {
    "c1": "gemm_256x256x256_f16_nn_f32acc_f32out",
    "c2": "gemm_4096x4096x4096_bf16_nn_f32acc_bf16out",
    "c3": "gemm_5000x3000x2050_f16_tn_f16out",
    "c4s": "batched32_gemm_4096x4096x128_f16_tn_f32out",
    "c4o": "batched32_gemm_4096x128x4096_f16_nn_f32out",
    "c5": "gemm_8192x8192x8192_i8_tn_i32out",
    "c5nn": "gemm_8192x8192x8192_i8_nn_i32out",
    "c6": "gemm_8192x8192x8192_e4m3_tn_f32acc_bf16out",
    "lk": "gemm_1024x1024x16384_bf16_nn_f32acc_bf16out",
    "lksk": "gemm_1024x1024x16384_bf16_nn_f32acc_bf16out_streamk",
    "c5dq": "gemm_8192x8192x8192_i8_tn_dequant_rowcol_scale_bias_gelu_bf16out",
}

# Fused attention (dmu_attention): batch, seq_q, seq_k, head_dim, in type, out type.
ATTENTION_WORKLOADS = {"c4fa": (32, 4096, 4096, 128, "f16", "f32")}
# the matrix-core-bound products whose bench line also measures the matrix-core ceiling
CEILING_WORKLOADS = {"c2", "c3", "c5", "c5nn", "c5dq"}
WORKLOAD_NAMES["c4fa"] = "batched32_attention_4096x4096x128_f16_f32out_fused"

# Workloads that run the persistent stream-K schedule (dmu_gemm_streamk): base problem.
STREAMK_WORKLOADS = {"lksk": "lk"}

# Workloads that run with the fused epilogue (dmu_gemm_ex): base problem, output type, activation.
EPILOGUE_WORKLOADS = {"c5dq": ("c5", "bf16", "gelu_tanh")}


# Host-only sources: argument checks, kernel selection, launch plumbing.  They do not change
# a kernel's memory traffic, and a change of the kernel they select shows in its name, which
# a stored reading is also checked against.
HOST_SOURCES = {"dmu_host.hip", "dmu_host.hpp"}


def source_digest(workload: str = "c2") -> str:
    """Digest of the device code a workload's kernel is built from (a stored counter reading is
    valid only for it): every kernel source except the layout probes and the host-only files,
    and the attention source only for the attention workloads."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "dense_matrix_unit_tiled_amd", "csrc", "*"))):
        name = os.path.basename(f)
        if name == "dmu_probe.hip" or name in HOST_SOURCES or \
                (name == "dmu_attention.hip" and workload not in ATTENTION_WORKLOADS):
            continue
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def stored_record(workload: str, kernel: str):
    """The committed rocprofv3 counter record of a workload (profiles/traffic_<workload>.json), or
    None when there is none or it was taken on other device code or another kernel."""
    path = os.path.join(ROOT, "profiles", f"traffic_{WORKLOAD_NAMES[workload]}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_digest") != source_digest(workload) or rec.get("kernel") != kernel:
        return None
    return rec


def stored_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None."""
    rec = stored_record(workload, kernel)
    return None if rec is None else rec.get("traffic_bytes_per_launch")


def stored_phases(workload: str, kernel: str):
    """The committed phase breakdown of a workload (profiles/phases_<workload>.json) in brief --
    span, median shader clock over the workgroups (s_memtime), the matrix-core busy fraction at
    that clock -- or None when there is none or it was logged on other device code or another
    kernel."""
    path = os.path.join(ROOT, "profiles", f"phases_{WORKLOAD_NAMES[workload]}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_digest") != source_digest(workload) or rec.get("kernel") != kernel:
        return None
    clk = rec.get("shader_clock_ghz") or {}
    return {"span_us": rec["span_us"], "main_loop_median_us": rec["main_loop_us"]["median"],
            "epilogue_median_us": rec["epilogue_us"]["median"], "shader_clock_ghz": clk.get("median"),
            "mfma_busy_at_shader_clock": rec.get("mfma_busy_at_shader_clock"),
            "source": f"profiles/phases_{WORKLOAD_NAMES[workload]}.json (dmu_phase_log, device-code digest "
                      f"{rec['source_digest']})"}


def stored_counters(workload: str, kernel: str):
    """The matrix-core and LDS counter figures of the committed record (the same counter runs as
    the traffic), or None: MFMA busy fraction, LDS bank-conflict cycles and their share of the LDS
    active cycles, the shader clock over the dispatch, and the record they come from."""
    rec = stored_record(workload, kernel)
    if rec is None or "mfma_busy_fraction" not in rec:
        return None
    out = {"mfma_busy": round(rec["mfma_busy_fraction"], 4),
           "lds_bank_conflict_cycles": rec.get("lds_bank_conflict_cycles"),
           "lds_bank_conflict_frac": None if rec.get("lds_conflict_fraction") is None
           else round(rec["lds_conflict_fraction"], 5),
           "sclk_ghz": None if rec.get("gui_active_ghz") is None else round(rec["gui_active_ghz"], 3),
           "dispatch_us": None if rec.get("counter_dispatch_us") is None else round(rec["counter_dispatch_us"], 2),
           "source": f"profiles/traffic_{WORKLOAD_NAMES[workload]}.json (rocprofv3 --pmc, "
                     f"device-code digest {rec['source_digest']})"}
    return out


# The pages' own figures for the 4096^3 bf16 product, on the A100 they were written for: context
# for the MI355X numbers, not a target ("Tensor Cores, CUTLASS and CuTe", opening section: the
# BF16 tensor-core and FP32 peaks; section 4.1: the work, the minimum traffic and the time at the
# tensor-core peak).
CONTEXT_A100 = {
    "gpu": "A100 (the page's own machine)",
    "bf16_tensor_core_peak_tflops": 312.0,
    "fp32_peak_tflops": 19.5,
    "gemm_4096_gflop": 137.4,
    "gemm_4096_min_traffic_mb": 100.7,
    "gemm_4096_time_at_peak_ms": 0.44,
    "source": "Tensor Cores, CUTLASS and CuTe: opening section (peaks) and section 4.1 (the 4096^3 "
              "problem: work, minimum traffic, time at the tensor-core peak)",
}


def profile_commands(workload: str, d: str) -> dict:
    """The rocprofv3 runs whose output --summarize reads (run from the repository root)."""
    bench = f"python3 bench.py --workload {workload}"
    small = f"{bench} --steps 100 --warmup 1000 --no-cpu-baseline --copy-calibration 256"
    sq = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE "
          "SQ_INSTS_LDS SQ_INSTS_MFMA GRBM_GUI_ACTIVE")
    return {
        "trace": f"rocprofv3 --kernel-trace --stats --output-format csv -d {d}/trace -o run -- "
                 f"{bench} --steps 200 --warmup 1000 --no-cpu-baseline",
        "fetch": f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/fetch -o run -- {small}",
        "write": f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/write -o run -- {small}",
        "sq": f"rocprofv3 --pmc {sq} --output-format csv -d {d}/sq -o run -- {small}",
    }


def algorithmic_bytes(p, ep_bytes: int = 0) -> int:
    """Bytes one launch must move at least: A, B and D once (C once more when present), plus
    the epilogue vectors."""
    esz = {"f16": 2, "bf16": 2, "i8": 1, "e4m3": 1}[p.in_type]
    osz = {"f32": 4, "i32": 4, "f16": 2, "bf16": 2}[p.out_type]
    mn = p.batch * p.M * p.N
    return (p.batch * (p.M + p.N) * p.K * esz + mn * osz * (2 if p.C is not None else 1) + ep_bytes)


def roofline(flops: float, nbytes: float, seconds: float, peak_tflops: float, traffic, counters=None) -> dict:
    """The bound of the launch by its algorithmic intensity against the chip's ridge: the
    matrix cores (TFLOP/s against the dtype's dense peak) or HBM (GB/s against 8 TB/s), with the
    committed counter figures of the same kernel (MFMA busy, LDS bank conflicts, clock) when
    they describe the current device code."""
    ridge = peak_tflops * 1e12 / (PEAK_HBM_GBS * 1e9)  # FLOP per byte
    if flops / nbytes >= ridge:
        a = flops / seconds / 1e12
        r = {"bound": "mfma", "achieved": round(a, 3), "peak": peak_tflops, "unit": "TFLOP/s",
             "frac": round(a / peak_tflops, 4), "traffic": traffic}
    else:
        a = nbytes / seconds / 1e9
        r = {"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(a / PEAK_HBM_GBS, 4), "traffic": traffic}
    r["counters"] = counters
    return r


def kernel_for(workload: str) -> str:
    """Name of the kernel variant the workload's call selects (host-side query, no GPU)."""
    import dense_matrix_unit_tiled_amd as dmu
    import workloads

    if workload in ATTENTION_WORKLOADS:
        *_, in_t, out_t = ATTENTION_WORKLOADS[workload]
        return f"attn_fwd_{in_t}_{out_t}"

    base, out_override = (EPILOGUE_WORKLOADS[workload][:2] if workload in EPILOGUE_WORKLOADS else
                          (STREAMK_WORKLOADS.get(workload, workload), None))
    M, N, K, batch, in_t, out_t, acc_t, la, lb = workloads.FULL[base]
    out_t = out_override or out_t
    lda, ldb, sa, sb = workloads._layout_params(M, N, K, la, lb)
    base = 1 << 40  # aligned stand-in addresses: only validation and selection run
    a = dmu.gemm_args(M, N, K, base, lda, base + (1 << 36), ldb, base + (2 << 36), N, in_type=in_t,
                      out_type=out_t, acc_type=acc_t, layout_a=la, layout_b=lb, batch=batch,
                      stride_a=sa if batch > 1 else 0, stride_b=sb if batch > 1 else 0,
                      stride_d=M * N if batch > 1 else 0,
                      C=(base + (3 << 36)) if workload == "c1" else None, ldc=N if workload == "c1" else 0)
    name = dmu.dmu_gemm_kernel_name(a)
    if workload in STREAMK_WORKLOADS and "generic" not in name:
        # the stream-K kernel runs 256 x 128 tiles where the data-parallel plan has 256 x 256,
        # and 128 x 128 where it has 64 x 128
        name = "streamk_" + name.replace("mfma_256x256w4", "mfma_256x128").replace("mfma_256x256", "mfma_256x128") \
            .replace("mfma_64x128", "mfma_128x128")
    return name


def cpu_baseline(p, budget_s: float = 15.0):
    """The oracle, as it stands, on the host cores over a bounded row slice of the product."""
    import numpy as np

    import oracle

    threads = oracle.default_threads()

    def run(rows, nthreads=threads):
        A = p.A[: rows * p.lda] if p.layout_a == "row" else p.A
        t0 = time.perf_counter()
        oracle.gemm(rows, p.N, p.K, A, p.lda, p.B, p.ldb, in_type=p.in_type, out_type=p.out_type,
                    layout_a=p.layout_a, layout_b=p.layout_b, ldd=p.N, nthreads=nthreads)
        return time.perf_counter() - t0

    rows = threads
    t = run(rows)
    rows2 = int(min(p.M, max(rows, rows * budget_s / max(t, 1e-3))))
    rows2 = max(threads, (rows2 // threads) * threads)
    t2 = run(rows2)
    flops = 2.0 * rows2 * p.N * p.K
    # one thread on a few rows: the per-core rate
    r1 = min(p.M, 8)
    t1 = run(r1, 1)
    return {"value": round(flops / t2 / 1e12, 6), "unit": "TFLOPS", "cores": threads, "kind": "oracle",
            "sample": f"rows 0..{rows2 - 1} of the {p.M}x{p.N}x{p.K} product "
                      f"({rows2}x{p.N}x{p.K} MACs, {t2:.1f} s, fp64 sums, {threads} threads)",
            "per_core_value": round(2.0 * r1 * p.N * p.K / t1 / 1e12, 6),
            "per_core_sample": f"rows 0..{r1 - 1}, one thread, {t1:.2f} s"}


def attention_cpu_baseline(batch, sq, sk, hd, Q, K, V, in_t, out_t, scale, budget_s: float = 15.0):
    """The oracle, as it stands, on the host cores over a bounded sample of query rows."""
    import numpy as np

    import oracle

    threads = oracle.default_threads()

    def run(n):
        rows = np.stack([np.arange(n) % batch, (np.arange(n) * 997) % sq], axis=1)
        t0 = time.perf_counter()
        oracle.attention_rows(batch, sq, sk, hd, hd, Q, hd, sq * hd, K, hd, sk * hd, V, hd, sk * hd, rows,
                              in_type=in_t, out_type=out_t, scale=scale, nthreads=threads)
        return time.perf_counter() - t0

    n = threads
    t = run(n)
    n2 = int(min(batch * sq, max(n, n * budget_s / max(t, 1e-3))))
    n2 = max(threads, (n2 // threads) * threads)
    t2 = run(n2)
    flops = 4.0 * n2 * sk * hd
    return {"value": round(flops / t2 / 1e12, 6), "unit": "TFLOPS", "cores": threads, "kind": "oracle",
            "sample": f"{n2} query rows spread over the {batch} slices of the {batch}x{sq}x{sk}x{hd} "
                      f"attention ({t2:.1f} s, fp64, {threads} threads)"}


def run_attention(args, dmu, workloads, torch, np, to_dev) -> int:
    """Time the fused attention forward over inputs resident in HBM (same protocol as the GEMM)."""
    batch, sq, sk, hd, in_t, out_t = ATTENTION_WORKLOADS[args.workload]
    rng = np.random.default_rng([41, 0])
    # Q, K, V uniform in [-1, 1] (the recipe of the batched attention-shaped pair), scale 1/sqrt(d)
    Q = workloads.to_bits(rng.uniform(-1, 1, batch * sq * hd), in_t)
    K = workloads.to_bits(rng.uniform(-1, 1, batch * sk * hd), in_t)
    V = workloads.to_bits(rng.uniform(-1, 1, batch * sk * hd), in_t)
    dQ, dK, dV = to_dev(Q), to_dev(K), to_dev(V)
    dO = torch.zeros(batch * sq * hd, dtype=torch.float32 if out_t == "f32" else torch.int16, device="cuda:0")
    scale = 1.0 / hd ** 0.5
    a = dmu.attention_args(batch, sq, sk, hd, dQ, hd, dK, hd, dV, hd, dO, hd, in_type=in_t, out_type=out_t,
                           scale=scale, stride_q=sq * hd, stride_k=sk * hd, stride_v=sk * hd,
                           stride_o=sq * hd)
    stream = torch.cuda.current_stream()
    kernel = kernel_for(args.workload)
    print(f"# workload {WORKLOAD_NAMES[args.workload]} kernel {kernel}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        dmu.dmu_attention(a, stream)
    torch.cuda.synchronize()
    if args.phases:
        return run_phases(args, lambda: dmu.dmu_attention(a, stream), stream, dmu, torch, np, kernel)
    lt = launch_times(lambda: dmu.dmu_attention(a, stream), stream, torch)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        dmu.dmu_attention(a, stream)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    print(f"# timed {args.steps} launches: {ms * 1e3:.2f} us each", file=sys.stderr, flush=True)
    copy_calibration(args, torch)
    flops = 4.0 * batch * sq * sk * hd  # the two products, 2 flops per multiply-add
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[in_t]
    result = {
        "metric": "achieved TFLOPS (fused attention forward, both products)", "value": round(tflops, 3),
        "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": in_t, "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.workload], "batch": batch, "seq_q": sq, "seq_k": sk,
                   "head_dim": hd, "in_type": in_t, "out_type": out_t, "kernel": kernel,
                   "pct_of_peak": round(100 * tflops / peak, 2)},
        "roofline": dict(roofline(flops, batch * (sq + 2 * sk) * hd * 2 + batch * sq * hd * (4 if out_t == "f32" else 2),
                                  ms * 1e-3, peak, stored_traffic(args.workload, kernel),
                                  stored_counters(args.workload, kernel)),
                         phase_log=stored_phases(args.workload, kernel)),
        "launch_times": lt,
        "peak_derived": peak_derived(dmu, in_t),
        "cpu_baseline": None if args.no_cpu_baseline else
        attention_cpu_baseline(batch, sq, sk, hd, Q, K, V, in_t, out_t, scale),
    }
    print(json.dumps(result), flush=True)
    return 0


# Back-to-back launches before the individually timed ones, whatever --warmup is: the shader
# clock settles only after a few hundred launches (about 300 for the 4096^3 product).
LAUNCH_TIMES_RAMP = 400


def launch_times(launch, stream, torch, n_warm: int = 50, n_cold: int = 20, rewarm: int = 300,
                 ramp: int = LAUNCH_TIMES_RAMP) -> dict:
    """Medians of individually timed launches: warm (back to back, after `ramp` untimed launches
    that bring the clock up), and cold (a 1 GiB buffer written on the same stream before each
    launch, which evicts the inputs from the L2 caches and the 256 MB last-level cache).  Run
    before the timed region, then warmed up again, so that the timed launches stay the last ones
    a trace records."""
    def per_launch(n, flush=None):
        evs = []
        for i in range(n):
            if flush is not None:
                flush.fill_(float(i))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch()
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        ts = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
        return ts[len(ts) // 2]

    for _ in range(ramp):
        launch()
    torch.cuda.synchronize()
    warm = per_launch(n_warm)
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0")
    cold = per_launch(n_cold, flush)
    del flush
    for _ in range(rewarm):
        launch()
    torch.cuda.synchronize()
    return {"warm_median_us": round(warm, 2), "warm_launches": n_warm, "ramp_launches": ramp,
            "cold_median_us": round(cold, 2), "cold_launches": n_cold,
            "cold_flush": "1 GiB written before each launch"}


# Dense multiply-accumulate rate per compute unit and clock of the matrix cores, in flops
# (16 x 16 x 32 bf16/fp16: 8192 multiply-adds per 16 cycles on each of 4 SIMDs; 8-bit
# inputs twice that).
FLOP_PER_CLOCK_PER_CU = {"bf16": 4096, "f16": 4096, "i8": 8192, "e4m3": 8192}


CEILING_ROUNDS, CEILING_WORKGROUPS = 128, 256


def mfma_ceiling(dmu, torch, in_type: str, stream, n_ramp: int = 400, n_timed: int = 200):
    """The matrix-core rate this machine sustains with nothing else running (dmu_mfma_ceiling: the
    tiled kernels' instruction on register operands, a grid shaped like the 4096^3 launch), timed
    like the product itself, with the median shader clock of its workgroups; None for types that
    have no ceiling kernel."""
    if in_type not in ("bf16", "f16", "i8"):
        return None
    stamps = torch.zeros(CEILING_WORKGROUPS * 4, dtype=torch.int64, device="cuda:0")
    launch = lambda st=None: dmu.dmu_mfma_ceiling(in_type, CEILING_ROUNDS, CEILING_WORKGROUPS, st, stream)
    for _ in range(n_ramp):
        launch()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(n_timed):
        launch()
    e1.record(stream)
    launch(stamps)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n_timed
    r = stamps.view(-1, 4).cpu().numpy().astype("float64")
    clk = sorted((r[:, 3] - r[:, 1]) / ((r[:, 2] - r[:, 0]) * 10.0))  # s_memtime ticks per ns
    flop_per_instr = 16 * 16 * (64 if in_type == "i8" else 32) * 2
    flops = CEILING_WORKGROUPS * 8 * CEILING_ROUNDS * 32 * flop_per_instr
    tf = flops / (us * 1e-6) / 1e12
    return {"tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_TFLOPS[in_type], 4), "us": round(us, 3),
            "shader_clock_ghz": round(clk[len(clk) // 2], 3),
            "grid": f"{CEILING_WORKGROUPS} workgroups x 8 wavefronts, {CEILING_ROUNDS} rounds of 32 "
                    f"instructions each ({flops / 1e9:.1f} G{'OP' if in_type == 'i8' else 'FLOP'})",
            "source": "dmu_mfma_ceiling (register operands, no memory traffic)"}


def peak_derived(dmu, dtype: str) -> dict:
    """The dense peak re-derived on this machine: compute units x peak clock x flops per clock."""
    cus, khz = dmu.dmu_device_info(0)
    per = FLOP_PER_CLOCK_PER_CU[dtype]
    return {"tflops": round(cus * khz * 1e3 * per / 1e12, 1), "compute_units": cus,
            "max_sclk_mhz": round(khz / 1e3), "flop_per_clock_per_cu": per,
            "source": "dmu_device_info (HIP device attributes)"}


def copy_calibration(args, torch):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()


PHASE_LOG_RECORDS = 1 << 16


def run_phases(args, launch, stream, dmu, torch, np, kernel) -> int:
    """Log `args.phases` back-to-back launches (after the warm-up), each into its own phase log,
    with HIP events around each on the launch stream, and write each launch's event time and span
    and the raw records of the median-span launch to `args.phases_file`."""
    logs = [torch.zeros(PHASE_LOG_RECORDS * 8, dtype=torch.int64, device="cuda:0") for _ in range(args.phases)]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in logs]
    counts = []
    torch.cuda.synchronize()
    try:
        for log, (e0, e1) in zip(logs, ev):
            dmu.dmu_phase_log(log, PHASE_LOG_RECORDS)
            e0.record(stream)
            launch()
            e1.record(stream)
            counts.append(dmu.dmu_phase_log_last())
    finally:
        dmu.dmu_phase_log(None, 0)
    torch.cuda.synchronize()
    cus, _ = dmu.dmu_device_info(0)
    out = {"workload": WORKLOAD_NAMES[args.workload], "kernel": kernel, "source_digest": source_digest(args.workload),
           "compute_units": cus, "warmup": args.warmup, "launches": []}
    for log, (e0, e1), (n, kind) in zip(logs, ev, counts):
        recs = log.view(-1, 8)[:n].cpu().numpy().view(np.uint64)
        span = int(recs[:, 3].max()) - int(recs[:, 0].min()) if n else 0
        out["launches"].append({"event_us": e0.elapsed_time(e1) * 1e3, "kind": kind, "n": int(n),
                                "span_ticks": span, "recs": recs})
    # only the median-span launch keeps its records (the others: event time and span)
    order = sorted(range(len(out["launches"])), key=lambda i: out["launches"][i]["span_ticks"])
    out["median_launch"] = order[len(order) // 2]
    for i, L in enumerate(out["launches"]):
        recs = L.pop("recs")
        if i == out["median_launch"]:
            L["records"] = [[int(x) for x in r] for r in recs]
    path = args.phases_file
    if os.path.dirname(path):
        os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as fh:
        json.dump(out, fh)
    from dense_matrix_unit_tiled_amd import profiling
    best = profiling.median_launch(out)
    print(json.dumps(profiling.phase_summary(best["records"], best["kind"], cus, best["event_us"])), flush=True)
    return 0


def summarize_phases(path: str, workload: str) -> int:
    """profiles/phases_<workload name>.{json,md} from a --phases output file."""
    from dense_matrix_unit_tiled_amd import profiling
    raw = json.load(open(path))
    if raw["workload"] != WORKLOAD_NAMES[workload]:
        print(f"bench.py: {path} holds {raw['workload']}, not {WORKLOAD_NAMES[workload]}", file=sys.stderr)
        return 2
    best = profiling.median_launch(raw)
    summ = profiling.phase_summary(best["records"], best["kind"], raw["compute_units"], best["event_us"])
    summ.update(workload=raw["workload"], kernel=raw["kernel"], source_digest=raw["source_digest"],
                launches_logged=len(raw["launches"]))
    import workloads
    if workload in ATTENTION_WORKLOADS:
        batch, sq, sk, hd, in_t, _ = ATTENTION_WORKLOADS[workload]
        flops = 4.0 * batch * sq * sk * hd
    else:
        base = EPILOGUE_WORKLOADS.get(workload, (STREAMK_WORKLOADS.get(workload, workload),))[0]
        M, N, K, batch, in_t = workloads.FULL[base][:5]
        flops = 2.0 * M * N * K * batch
    if summ.get("shader_clock_ghz"):
        summ["mfma_busy_at_shader_clock"] = round(profiling.mfma_busy_at_clock(
            flops, DENSE_FLOP_PER_CLOCK_PER_CU[in_t], raw["compute_units"], summ["span_us"],
            summ["shader_clock_ghz"]["median"]), 4)
    base = os.path.join(ROOT, "profiles", f"phases_{raw['workload']}")
    with open(base + ".json", "w") as fh:
        json.dump(summ, fh, indent=1)
    cmd = (f"python3 bench.py --workload {workload} --phases {len(raw['launches'])} --warmup {raw['warmup']} "
           f"--phases-file {path}")
    with open(base + ".md", "w") as fh:
        fh.write(profiling.phase_markdown(raw["workload"], raw["kernel"], cmd, summ))
    print(json.dumps(summ))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default="c2", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--summarize", metavar="DIR", default=None,
                    help="summarize rocprofv3 output under DIR into profiles/ and exit")
    ap.add_argument("--phases", type=int, default=0, metavar="N",
                    help="after the warm-up, log N back-to-back launches' per-workgroup phase "
                         "timestamps into --phases-file and exit")
    ap.add_argument("--phases-file", metavar="FILE", default="phases.json",
                    help="output of --phases (raw records of the median-span launch)")
    ap.add_argument("--summarize-phases", metavar="FILE", default=None,
                    help="summarize a --phases output file into profiles/ and exit")
    ap.add_argument("--bench-line", metavar="FILE", default=None,
                    help="with --summarize: the output of a plain bench.py run of the workload in the same "
                         "session, kept beside the summaries")
    args = ap.parse_args()
    if args.summarize:
        from dense_matrix_unit_tiled_amd import profiling

        kernel = kernel_for(args.workload)
        line = None
        if args.bench_line:
            rows = [json.loads(x) for x in open(args.bench_line) if x.startswith("{")]
            line = rows[-1] if rows else None
            if line is None or line.get("config", {}).get("workload") != WORKLOAD_NAMES[args.workload]:
                print(f"bench.py: {args.bench_line} holds no bench line of {args.workload}", file=sys.stderr)
                return 2
        res = profiling.summarize(args.summarize, os.path.join(ROOT, "profiles"), WORKLOAD_NAMES[args.workload],
                                  kernel, source_digest(args.workload),
                                  profile_commands(args.workload, "gpurun_out/prof_" + args.workload),
                                  timed=200, bench_line=line)
        print(json.dumps(res))
        return 0
    if args.summarize_phases:
        return summarize_phases(args.summarize_phases, args.workload)
    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU; --gpus {args.gpus} is not supported",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import dense_matrix_unit_tiled_amd as dmu
    import workloads

    def to_dev(x):  # raw element bits on the GPU (uint16 patterns travel as int16)
        x = np.ascontiguousarray(x)
        return torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).to("cuda:0")

    if args.workload in ATTENTION_WORKLOADS:
        return run_attention(args, dmu, workloads, torch, np, to_dev)

    ep = None
    ep_bytes = 0
    if args.workload in EPILOGUE_WORKLOADS:
        base, out_t, act = EPILOGUE_WORKLOADS[args.workload]
        p = workloads.with_output(workloads.make(base, "random", 0), out_t)
        e = workloads.make_epilogue(p, 0, act=act)
        ep_vecs = [to_dev(v) for v in (e.row_scale, e.col_scale, e.bias)]  # kept alive for the launches
        ep_bytes = sum(v.size * 4 for v in (e.row_scale, e.col_scale, e.bias))
        ep = dmu.epilogue_args(row_scale=ep_vecs[0], stride_row_scale=e.stride_rs, col_scale=ep_vecs[1],
                               stride_col_scale=e.stride_cs, bias=ep_vecs[2], stride_bias=e.stride_bias,
                               act=e.act)
    else:
        p = workloads.make(STREAMK_WORKLOADS.get(args.workload, args.workload), "random", 0)
    dA, dB = to_dev(p.A), to_dev(p.B)
    dC = to_dev(p.C) if p.C is not None else None
    out_dt = {"f32": torch.float32, "f16": torch.int16, "bf16": torch.int16, "i32": torch.int32}
    dD = torch.zeros(p.batch * p.stride_d, dtype=out_dt[p.out_type], device="cuda:0")
    a = dmu.gemm_args(p.M, p.N, p.K, dA, p.lda, dB, p.ldb, dD, p.ldd, in_type=p.in_type,
                      out_type=p.out_type, acc_type=p.acc_type, layout_a=p.layout_a,
                      layout_b=p.layout_b, batch=p.batch, stride_a=p.stride_a, stride_b=p.stride_b,
                      C=dC, ldc=p.ldc, stride_c=p.stride_c, stride_d=p.stride_d)
    kernel = kernel_for(args.workload)
    stream = torch.cuda.current_stream()
    print(f"# workload {WORKLOAD_NAMES[args.workload]} kernel {kernel}", file=sys.stderr, flush=True)

    launch = (lambda: dmu.dmu_gemm(a, stream)) if ep is None else (lambda: dmu.dmu_gemm_ex(a, ep, stream))
    ws_bytes = 0
    if args.workload in STREAMK_WORKLOADS:
        ws_bytes = dmu.dmu_gemm_streamk_workspace_size(a)
        ws = torch.zeros(max(ws_bytes, 4) // 4 + 1, dtype=torch.int32, device="cuda:0")  # zero-filled once
        launch = lambda: dmu.dmu_gemm_streamk(a, None, ws, 4 * ws.numel(), stream)
    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    if args.phases:
        return run_phases(args, launch, stream, dmu, torch, np, kernel)
    lt = launch_times(launch, stream, torch)

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        launch()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    print(f"# timed {args.steps} launches: {ms * 1e3:.2f} us each", file=sys.stderr, flush=True)

    ceiling = None
    if not args.copy_calibration and args.workload in CEILING_WORKLOADS:
        ceiling = mfma_ceiling(dmu, torch, p.in_type, stream)
    copy_calibration(args, torch)
    sk_failed = None
    if args.workload in STREAMK_WORKLOADS and ws_bytes:
        sk_failed = dmu.dmu_gemm_streamk_error(ws, stream, check=False)

    flops = float(p.flops)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[p.in_type]
    traffic = stored_traffic(args.workload, kernel)
    result = {
        "metric": "achieved TFLOPS (% of MFMA peak) for 4096³ bf16 GEMM, fp32 accumulate"
        if args.workload == "c2" else f"achieved {'TOPS' if p.in_type == 'i8' else 'TFLOPS'}",
        "value": round(tflops, 3),
        "unit": "TOPS" if p.in_type == "i8" else "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.in_type,
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.workload], "M": p.M, "N": p.N, "K": p.K,
                   "batch": p.batch, "layout_a": p.layout_a, "layout_b": p.layout_b,
                   "in_type": p.in_type, "acc_type": p.acc_type, "out_type": p.out_type,
                   "kernel": kernel, "pct_of_peak": round(100 * tflops / peak, 2)},
        "roofline": dict(roofline(flops, algorithmic_bytes(p, ep_bytes), ms * 1e-3, peak, traffic,
                                  stored_counters(args.workload, kernel)),
                         phase_log=stored_phases(args.workload, kernel)),
        "launch_times": lt,
        "peak_derived": peak_derived(dmu, p.in_type),
    }
    if ceiling is not None:
        result["roofline"]["mfma_ceiling"] = ceiling
        result["roofline"]["frac_of_ceiling"] = round(tflops / ceiling["tflops"], 4)
    if sk_failed is not None:
        result["streamk_wait_failed"] = sk_failed  # a wait that gave up leaves a wrong D (never expected)
    if args.workload == "c2":
        result["context_a100"] = dict(CONTEXT_A100, this_run_ms=round(ms, 6),
                                      this_run_vs_a100_time_at_peak=round(CONTEXT_A100["gemm_4096_time_at_peak_ms"] / ms, 3))
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(p)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 1 if sk_failed else 0


if __name__ == "__main__":
    sys.exit(main())
