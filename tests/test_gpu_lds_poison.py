"""The LDS-poisoning debug build (libdmu_poison.so, the same sources compiled with
DMU_LDS_POISON=1) against the product library, through the C ABI.

In the debug build every wavefront overwrites its staging slots of a stage with all-ones
bytes -- NaN in fp16, bf16 and e4m3, -1 in int8 -- right after the barrier that retires
the stage, long before the next K-tile's data lands there.  The stage ring's argument
("Tensor Cores, CUTLASS and CuTe" section 4.3: a stage is overwritten only after the
barrier that follows its last reads) is then checked by the data: any fragment read that
strays past its barrier feeds poison into D.  Every tiled form (eight and four wavefronts,
the 16-bit and 8-bit transposed LDS layouts, masked K tails, int8, e4m3, the persistent and
the stream-K schedules) must give the product build's bits exactly, and meet the oracle's bar."""
import os

import numpy as np
import pytest

import dense_matrix_unit_tiled_amd as dmu
from dense_matrix_unit_tiled_amd.build import POISON_LIB_PATH
import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = [
    ("c2", dict(M=520, N=264, K=1000), "256x256"),    # bf16, B row-major (transposed tiles), K tail
    ("c2", dict(M=520, N=264, K=1000), "256x256w4"),
    ("c2", dict(M=520, N=264, K=1000), "128x128"),
    ("c2", dict(M=520, N=264, K=1000), "64x128"),
    ("c3", dict(M=300, N=270, K=1030), "256x256"),    # fp16 -> fp16, 4-byte rows, masked K tail
    ("c3", dict(M=300, N=270, K=1030), "256x128"),
    ("c3", dict(M=300, N=270, K=1030), "64x128"),
    ("c5", dict(M=300, N=260, K=1024), "256x256"),    # int8
    ("c5nn", dict(M=300, N=272, K=1024), "256x256"),  # int8, B row-major: the 8-bit transposed layout
    ("c5nn", dict(M=300, N=272, K=1024), "128x128"),
    ("c6", dict(M=300, N=260, K=1024), "256x128"),    # e4m3
    ("c6", dict(M=300, N=260, K=1024), "128x128"),
    ("c6", dict(M=300, N=260, K=1024), "64x128"),
    ("c5nn", dict(M=300, N=272, K=1024), "64x128"),
    ("c4o", dict(M=300, N=128, K=1024, batch=2), None),
]


def both(p, force=None, env=None):
    """D from the product library and from the debug build, same call."""
    old = {k: os.environ.get(k) for k in (env or {})}
    os.environ.update(env or {})
    try:
        ref = gu.run_dmu(p, force=force)
        with dmu.library_override(POISON_LIB_PATH):
            got = gu.run_dmu(p, force=force)
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    return ref, got


def test_debug_build_is_present():
    assert os.path.exists(POISON_LIB_PATH), "libdmu_poison.so is built by dense_matrix_unit_tiled_amd.build.build()"


@pytest.mark.parametrize("cfg,sizes,kernel", CASES)
def test_poisoned_stages_leave_results_unchanged(cfg, sizes, kernel):
    p = workloads.make(cfg, "random", 41, **sizes)
    ref, got = both(p, force=kernel)
    gu.assert_bits_equal(got, ref, where=gu.valid_mask(p))
    gu.assert_close(got, gu.run_oracle(p), p, where=gu.valid_mask(p))


def test_poisoned_persistent_form():
    """Short K loops over many tiles on the persistent grid (the next tile's first K-tile is
    loaded before the current epilogue)."""
    p = workloads.make("c4s", "random", 42, M=1000, N=520, K=256, batch=4)
    ref, got = both(p, force="256x128", env={"DMU_PERSIST": "always"})
    gu.assert_bits_equal(got, ref, where=gu.valid_mask(p))


def test_poisoned_streamk_schedule():
    p = workloads.make("c1", "random", 43, M=256, N=256, K=8192)  # 4 tiles, each split over 64 workers
    p.C = None
    ref, _, _ = gu.run_streamk(p)
    with dmu.library_override(POISON_LIB_PATH):
        got, name, ws = gu.run_streamk(p)
    assert "generic" not in name
    gu.assert_bits_equal(got, ref, where=gu.valid_mask(p))
