"""Build ``libdmu.so`` (the gfx950 GEMM library) in-tree with hipcc.

Every ``csrc/*.hip`` unit is compiled for gfx950 in parallel into ``_build/``
and linked into ``dense_matrix_unit_tiled_amd/libdmu.so``.  The LDS-poisoning
debug build of the same sources (``-DDMU_LDS_POISON=1``, see dmu_tiled.hpp) goes
to ``_build_poison/`` and ``libdmu_poison.so``; only its test loads it.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libdmu.so")
POISON_LIB_PATH = os.path.join(HERE, "libdmu_poison.so")
VARIANTS = {None: (BUILD, LIB_PATH, []),
            "poison": (os.path.join(ROOT, "_build_poison"), POISON_LIB_PATH, ["-DDMU_LDS_POISON=1"])}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Multiply-adds are fused freely except where a `#pragma clang fp contract(off)`
# says otherwise (the fused epilogue, whose every operation rounds on its own so
# that every kernel computes it to the same bits): plain "fast" would ignore the
# pragma and fuse differently in different kernels.
#
# Packed fp32 VALU instructions are disabled for all device code: this library
# does not use them, and hipcc -O3 would otherwise form them from plain float
# code.  The host pass warns that it does not know the feature.
#
# The kernels index register arrays only with indices that are constant after
# full unrolling; a loop the compiler declines to unroll would turn such an
# array into scratch memory.  The unroll threshold is therefore raised, a loop
# that stays rolled is an error, and the per-kernel resource report is checked:
# a kernel with scratch memory or VGPR spills fails the build (SGPR spills go
# to VGPR lanes, not to memory; they are listed in _build/resource_usage.txt).
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-munsafe-fp-atomics", "-ffp-contract=fast-honor-pragmas",
                "-mllvm", "-pragma-unroll-threshold=1000000", "-Werror=pass-failed",
                "-Rpass-analysis=kernel-resource-usage"]

_REMARK = re.compile(r"remark:\s+(Function Name|ScratchSize \[bytes/lane\]|VGPRs Spill|SGPRs Spill|VGPRs|AGPRs|"
                     r"Occupancy \[waves/SIMD\]):\s*(\S+)")


def resource_usage(text: str) -> list:
    """[{kernel, VGPRs, AGPRs, ScratchSize, ...}] from the compiler's resource remarks."""
    out = []
    for key, val in _REMARK.findall(text):
        if key == "Function Name":
            out.append({"kernel": val})
        elif out:
            out[-1][key.split(" [")[0]] = int(val)
    return out


def _compile(job) -> tuple:
    src, build_dir, defines = job
    obj = os.path.join(build_dir, os.path.basename(src).replace(".hip", ".o"))
    cmd = [HIPCC, *DEVICE_FLAGS, *defines, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed for {src}")
    usage = resource_usage(r.stderr)
    bad = [u for u in usage if u.get("ScratchSize", 0) or u.get("VGPRs Spill", 0)]
    if bad:
        raise RuntimeError(f"{src}: kernels with scratch memory or spills: {bad}")
    return obj, usage


def build(jobs: int | None = None, variants=(None, "poison")) -> str:
    """Compile every unit of each variant (the product library, then the debug build) in one
    pool and link each; returns the product library's path."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    work = []
    for v in variants:
        build_dir, _, defines = VARIANTS[v]
        os.makedirs(build_dir, exist_ok=True)
        work += [(src, build_dir, defines) for src in srcs]
    jobs = jobs or min(len(work), max(1, len(os.sched_getaffinity(0))), 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, work))
    for v in variants:
        build_dir, lib_path, _ = VARIANTS[v]
        mine = [r for r, w in zip(results, work) if w[1] == build_dir]
        with open(os.path.join(build_dir, "resource_usage.txt"), "w") as fh:
            for _, usage in mine:
                for u in usage:
                    fh.write(" ".join(f"{k}={v}" for k, v in u.items()) + "\n")
        tmp = lib_path + ".tmp"
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in mine]],
                       check=True)
        os.replace(tmp, lib_path)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
