"""bench.py's host logic (CPU only): the roofline bound of each workload and the one-GPU rule."""
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import pytest

import bench
import workloads


def full(cfg):
    M, N, K, b, it, ot, at, la, lb = workloads.FULL[cfg]
    return SimpleNamespace(M=M, N=N, K=K, batch=b, in_type=it, out_type=ot, C=None)


@pytest.mark.parametrize("cfg,bound", [("c2", "mfma"), ("c5", "mfma"), ("c6", "mfma"), ("c3", "mfma"),
                                       ("c4s", "hbm"), ("c4o", "hbm")])
def test_roofline_bound_by_intensity(cfg, bound):
    p = full(cfg)
    r = bench.roofline(2.0 * p.M * p.N * p.K * p.batch, bench.algorithmic_bytes(p), 1e-4,
                       bench.PEAK_TFLOPS[p.in_type], None)
    assert r["bound"] == bound
    assert r["unit"] == ("TFLOP/s" if bound == "mfma" else "GB/s")
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-3)


def test_algorithmic_bytes_of_the_4096_cube():
    # A and B bf16 (2 x 32 MiB) + D bf16 (32 MiB)
    assert bench.algorithmic_bytes(full("c2")) == 3 * 4096 * 4096 * 2


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True, text=True,
                       cwd=bench.ROOT, timeout=60)
    assert r.returncode != 0 and "one GPU" in r.stderr


@pytest.mark.parametrize("cfg", sorted(bench.WORKLOAD_NAMES))
def test_committed_traffic_matches_current_kernels(cfg):
    """A stored HBM-traffic reading describes the device code it was taken on: every committed
    counter record carries the digest of the current kernel sources (a kernel change without
    new counter runs fails here), and its text summary names the same digest and kernel."""
    base = os.path.join(bench.ROOT, "profiles", f"traffic_{bench.WORKLOAD_NAMES[cfg]}")
    if not os.path.exists(base + ".json"):
        pytest.skip(f"no counter record for {cfg}")
    rec = json.load(open(base + ".json"))
    assert rec["source_digest"] == bench.source_digest(cfg)
    assert rec["traffic_bytes_per_launch"] == pytest.approx(
        rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"], rel=1e-9)
    text = open(base + ".md").read()
    assert f"`{rec['source_digest']}`" in text
    assert bench.stored_traffic(cfg, rec["kernel"]) == rec["traffic_bytes_per_launch"]


@pytest.mark.parametrize("cfg", sorted(set(workloads.FULL) & set(bench.WORKLOAD_NAMES)))
def test_committed_profiles_name_the_selected_kernel(cfg):
    """The committed rocprofv3 summaries of a workload describe the kernel that the library's
    selection picks for its full-size problem today (no GPU needed: device-looking addresses are
    never dereferenced by the selection)."""
    import dense_matrix_unit_tiled_amd as dmu
    M, N, K, b, it, ot, at, la, lb = workloads.FULL[cfg]
    fake = 1 << 40
    a = dmu.gemm_args(M, N, K, fake, K if la == "row" else M, fake + (1 << 36), N if lb == "row" else K,
                      fake + (2 << 36), N, in_type=it, out_type=ot, acc_type=at, layout_a=la, layout_b=lb,
                      batch=b, stride_a=M * K, stride_b=K * N, stride_d=M * N)
    kernel = dmu.dmu_gemm_kernel_name(a)
    name = bench.WORKLOAD_NAMES[cfg]
    assert os.path.exists(os.path.join(bench.ROOT, "profiles", f"{kernel}_{name}_kernel_trace.md"))
    rec = json.load(open(os.path.join(bench.ROOT, "profiles", f"traffic_{name}.json")))
    assert rec["kernel"] == kernel
