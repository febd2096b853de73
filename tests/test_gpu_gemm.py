"""Parity of the HIP GEMM (through the C ABI) with the CPU oracle.

* reduced sizes of every problem (several tiles, ragged tails), each kernel
  family, element by element against the full oracle product;
* full-size problems: the structured (integer-valued) inputs bit for bit
  against their closed forms, and random inputs on sampled outputs against
  the oracle's one-by-one evaluation;
* invariants: tiled kernel == fallback kernel bit for bit, storage-order
  identity, batch == loop of single products, C linearity, identity A,
  launch-to-launch reproducibility;
* edge cases: tiny and ragged shapes, K = 0, empty problems, misaligned
  pointers and padded leading dimensions, rounding ties and subnormal outputs.
"""
import numpy as np
import pytest

import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

REDUCED = {
    "c1": dict(),
    "c2": dict(M=520, N=264, K=200),
    "c3": dict(M=300, N=270, K=130),
    "c4s": dict(M=300, N=260, K=128, batch=3),
    "c4o": dict(M=300, N=128, K=520, batch=2),
    "c5": dict(M=300, N=260, K=384),
    "c5nn": dict(M=300, N=272, K=384),   # int8 with a row-major B: the 8-bit transposed layout
}
KERNELS = [None, "256x256", "256x256w4", "128x128", "256x128", "64x128", "generic"]


@pytest.mark.parametrize("cfg", list(REDUCED))
@pytest.mark.parametrize("kernel", KERNELS)
def test_reduced_random_parity(cfg, kernel):
    p = workloads.make(cfg, "random", 1, **REDUCED[cfg])
    got, name = gu.run_dmu(p, force=kernel, return_name=True)
    if kernel == "generic":
        assert "generic" in name
    elif kernel == "256x256w4" and p.in_type == "i8":
        assert "mfma_256x256_" in name, name  # the four-wavefront tile is built for 16-bit inputs
    elif kernel is not None and cfg != "c3":
        assert kernel in name, name
    if cfg == "c5nn" and kernel != "generic":
        assert "_t8_" in name, name
    want = gu.run_oracle(p)
    gu.assert_close(got, want, p, where=gu.valid_mask(p))


@pytest.mark.parametrize("cfg", list(REDUCED))
def test_reduced_with_c_and_padding(cfg):
    p = workloads.make(cfg, "random", 2, pad=8, with_c=True, **REDUCED[cfg])
    got = gu.run_dmu(p)
    want = gu.run_oracle(p)
    gu.assert_close(got, want, p, where=gu.valid_mask(p))


def closed_form(p) -> np.ndarray:
    """Expected D of the structured workloads, as fp64 values [batch, M, N]."""
    i = np.arange(p.M)[None, :, None]
    j = np.arange(p.N)[None, None, :]
    b = np.arange(p.batch)[:, None, None]
    if p.name in ("c1", "c2", "c5", "c5nn"):
        return p.K * (i % 16) * (j % 8) + 0 * b
    if p.name == "c3":
        n_i = (p.K // 16) + ((i % 16) < (p.K % 16))
        return n_i * (j % 8) + 0 * b
    if p.name == "c4s":
        return 128.0 * ((i + b) % 16) * (j % 8)
    if p.name == "c4o":
        return (((i + b) % p.K + 3 * b + j) % 64) - 32.0
    raise ValueError(p.name)


def as_values(p, flat):
    v = gu.values(flat, p.out_type) if p.out_type != "i32" else flat.astype(np.float64)
    out = np.empty((p.batch, p.M, p.N))
    for b in range(p.batch):
        out[b] = v[b * p.stride_d: b * p.stride_d + p.M * p.ldd].reshape(p.M, p.ldd)[:, : p.N]
    return out


@pytest.mark.parametrize("cfg", ["c1", "c2", "c3", "c4s", "c4o", "c5", "c5nn"])
def test_full_size_structured_exact(cfg):
    p = workloads.make(cfg, "structured")
    got = as_values(p, gu.run_dmu(p))
    want = closed_form(p)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"


@pytest.mark.parametrize("cfg", ["c1", "c2", "c3", "c4s", "c4o", "c5", "c5nn"])
def test_full_size_random_sampled(cfg):
    p = workloads.make(cfg, "random", 0)
    got = gu.run_dmu(p)
    bij = gu.sample_bij(p, n=384)
    want = gu.oracle_at(p, bij)
    gu.assert_close(got[gu.flat_index(p, bij)], want, p)


@pytest.mark.parametrize("kernel", [None, "256x256w4"])
def test_tiled_equals_fallback_bitwise(kernel):
    """Every output element goes through the same K-step sequence of the same matrix
    instruction in each tiled form and in the fallback: bit-identical results."""
    for cfg in ("c2", "c3", "c4s", "c5", "c5nn"):
        if kernel == "256x256w4" and cfg.startswith("c5"):
            continue  # 16-bit inputs only
        p = workloads.make(cfg, "random", 3, **REDUCED[cfg])
        a = gu.run_dmu(p, force=kernel)
        b = gu.run_dmu(p, force="generic")
        gu.assert_bits_equal(a, b, where=gu.valid_mask(p))


@pytest.mark.parametrize("cfg", ["c2", "c3"])
def test_four_wavefront_tile_full_size(cfg):
    """The four-wavefront 256 x 256 tile (accumulators in AGPRs) on the full problems: structured
    inputs bit for bit against their closed forms, random inputs on sampled outputs."""
    s = workloads.make(cfg, "structured")
    got, name = gu.run_dmu(s, force="256x256w4", return_name=True)
    assert "256x256w4" in name, name
    bad = np.argwhere(as_values(s, got) != closed_form(s))
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"
    p = workloads.make(cfg, "random", 0)
    got = gu.run_dmu(p, force="256x256w4")
    bij = gu.sample_bij(p, n=384)
    gu.assert_close(got[gu.flat_index(p, bij)], gu.oracle_at(p, bij), p)


@pytest.mark.parametrize("in_t,out_t", [("f16", "f32"), ("bf16", "bf16"), ("f16", "f16"), ("i8", "i32")])
def test_storage_order_identity(in_t, out_t):
    """Same values stored row- or column-major give bit-identical results."""
    rng = np.random.default_rng(9)
    M, N, K = 136, 200, 144
    if in_t == "i8":
        a = rng.integers(-128, 128, (1, M, K))
        b = rng.integers(-128, 128, (1, K, N))
    else:
        a = rng.uniform(-1, 1, (1, M, K))
        b = rng.uniform(-1, 1, (1, K, N))
    results = []
    for la in ("row", "col"):
        for lb in ("row", "col"):
            p = workloads.make("c5" if in_t == "i8" else "c1", "random", 0, M=M, N=N, K=K)
            p.in_type, p.out_type = in_t, out_t
            p.acc_type = "i32" if in_t == "i8" else "f32"
            p.layout_a, p.layout_b = la, lb
            p.A, p.lda = workloads.store(a, in_t, la)
            p.B, p.ldb = workloads.store(b, in_t, lb)
            p.C = None
            results.append(gu.run_dmu(p))
    for r in results[1:]:
        gu.assert_bits_equal(r, results[0])


def test_batch_equals_loop_of_single_products():
    p = workloads.make("c4s", "random", 4, M=200, N=136, K=128, batch=4)
    full = gu.run_dmu(p)
    for b in range(p.batch):
        q = workloads.make("c4s", "random", 4, M=200, N=136, K=128, batch=1)
        q.A = p.A[b * p.stride_a: (b + 1) * p.stride_a]
        q.B = p.B[b * p.stride_b: (b + 1) * p.stride_b]
        one = gu.run_dmu(q)
        gu.assert_bits_equal(full[b * p.stride_d: (b + 1) * p.stride_d], one)


def test_broadcast_stride_zero():
    p = workloads.make("c4s", "random", 5, M=64, N=96, K=128, batch=3)
    p.stride_b = 0
    p.B = p.B[: 96 * 128]
    got = gu.run_dmu(p)
    gu.assert_close(got, gu.run_oracle(p), p)


def test_c_linearity_integer_data():
    """Integer-valued data: gemm(C = X) == gemm(C = 0) + X exactly (fp32 output)."""
    p = workloads.make("c2", "structured", M=300, N=260, K=256)
    p.out_type = "f32"
    rng = np.random.default_rng(13)
    c = np.round(rng.uniform(-8, 8, p.M * p.ldd)).astype(np.float32)
    no_c = gu.run_dmu(p)
    p.C, p.ldc = c, p.ldd
    with_c = gu.run_dmu(p)
    gu.assert_bits_equal(with_c, no_c + c)


def test_identity_a_gives_b_plus_c():
    M = K = 160
    N = 96
    eye = np.eye(M)[None]
    rng = np.random.default_rng(8)
    b = rng.uniform(-1, 1, (1, K, N))
    p = workloads.make("c1", "random", 0, M=M, N=N, K=K, with_c=True)
    p.A, p.lda = workloads.store(eye, "f16", "row")
    p.B, p.ldb = workloads.store(b, "f16", "row")
    got = gu.run_dmu(p)
    want = gu.run_oracle(p)
    gu.assert_bits_equal(got, want)


def test_reproducible_across_launches():
    p = workloads.make("c2", "random", 6, M=1000, N=1000, K=512)
    first = gu.run_dmu(p)
    for _ in range(4):
        gu.assert_bits_equal(gu.run_dmu(p), first)


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (1, 7, 3), (33, 1, 65), (65, 33, 17), (127, 129, 255),
                                   (256, 257, 257), (255, 130, 8), (8, 8, 4096)])
@pytest.mark.parametrize("cfg", ["c1", "c3", "c5", "c2"])
def test_ragged_shapes(M, N, K, cfg):
    p = workloads.make(cfg, "random", 7, M=M, N=N, K=K, with_c=True)
    got = gu.run_dmu(p)
    gu.assert_close(got, gu.run_oracle(p), p, where=gu.valid_mask(p))


def test_k_zero_gives_c():
    p = workloads.make("c3", "random", 0, M=70, N=50, K=0, with_c=True)
    p.lda = p.ldb = 1
    got = gu.run_dmu(p)
    gu.assert_bits_equal(got, p.C)
    p.C = None
    gu.assert_bits_equal(gu.run_dmu(p, fill=0x1234), np.zeros(p.M * p.ldd, np.uint16))


def test_empty_problem_leaves_d_untouched():
    import torch

    import dense_matrix_unit_tiled_amd as dmu

    p = workloads.make("c1", "random", 0, M=8, N=8, K=8)
    dA, dB = gu.to_dev(p.A), gu.to_dev(p.B)
    dD = torch.full((64,), 7.0, dtype=torch.float32, device="cuda:0")
    for kw in (dict(M=0), dict(N=0), dict(batch=0)):
        args = gu.make_args(p, dA, dB, dD)
        for k, v in kw.items():
            setattr(args, k, v)
        assert dmu.dmu_gemm_kernel_name(args) is None
        dmu.dmu_gemm(args)
    torch.cuda.synchronize()
    assert torch.all(dD == 7.0)


@pytest.mark.parametrize("offset", [1, 2, 3])
def test_misaligned_pointers(offset):
    """Operands starting 1-3 elements past an aligned address (generic or 4-byte paths)."""
    base = workloads.make("c3", "random", 11, M=150, N=90, K=66)
    p = workloads.make("c3", "random", 11, M=150, N=90, K=66)
    p.A = np.concatenate([np.zeros(offset, np.uint16), base.A])
    p.B = np.concatenate([np.zeros(offset, np.uint16), base.B])
    import torch
    dA = gu.to_dev(p.A)[offset:]
    dB = gu.to_dev(p.B)[offset:]
    dD = torch.zeros(p.M * p.ldd + offset, dtype=torch.int16, device="cuda:0")[offset:]
    args = gu.make_args(base, dA, dB, dD)
    import dense_matrix_unit_tiled_amd as dmu
    dmu.dmu_gemm(args)
    torch.cuda.synchronize()
    got = dD.cpu().numpy().view(np.uint16)
    gu.assert_close(got, gu.run_oracle(base), base)


def test_output_rounding_ties_exact():
    """Integer sums that sit exactly halfway between fp16 / bf16 neighbours."""
    K = 64
    targets = np.array([257, 259, 261, 513, 515, 2049, 2051, 4097, 4099, 1025, 1027, 511])
    M, N = len(targets), 8
    a = np.zeros((1, M, K))
    # row i sums to targets[i] * (j + 1) when B[k][j] = j + 1 ... keep j = 0 column exact
    for r, t in enumerate(targets):
        q, rem = divmod(int(t), K)
        a[0, r, :] = q
        a[0, r, :rem] += 1
    b = np.ones((1, K, N))
    for out_t, in_t in (("bf16", "bf16"), ("f16", "f16")):
        p = workloads.make("c2" if in_t == "bf16" else "c3", "random", 0, M=M, N=N, K=K)
        p.layout_a, p.layout_b = "row", "row"
        p.A, p.lda = workloads.store(a, in_t, "row")
        p.B, p.ldb = workloads.store(b, in_t, "row")
        p.C = None
        gu.assert_bits_equal(gu.run_dmu(p), gu.run_oracle(p))


def test_fp16_subnormal_outputs_exact():
    """Products landing in the fp16 subnormal range are rounded, not flushed."""
    M, N, K = 64, 64, 32
    rng = np.random.default_rng(12)
    a = rng.integers(1, 8, (1, M, K)) * 2.0 ** -12
    b = rng.integers(0, 4, (1, K, N)) * 2.0 ** -14
    p = workloads.make("c3", "random", 0, M=M, N=N, K=K)
    p.layout_b = "row"
    p.A, p.lda = workloads.store(a, "f16", "row")
    p.B, p.ldb = workloads.store(b, "f16", "row")
    p.C = None
    got = gu.run_dmu(p)
    gu.assert_bits_equal(got, gu.run_oracle(p))
    assert np.any((got & 0x7C00) == 0) and np.any(got != 0)


@pytest.mark.parametrize("cfg,K,pad", [("c3", 2049, 3), ("c3", 2050, 0), ("c3", 131, 1), ("c5", 65, 3),
                                       ("c5", 130, 2), ("c5", 4097, 3), ("c3", 65, 3)])
def test_dword_aligned_rows_masked_k_tail(cfg, K, pad):
    """Rows only 4-byte aligned and K not a multiple of 16 bytes: the tiled kernel's
    16-byte loads straddle row ends and must clear the next row's bytes."""
    p = workloads.make(cfg, "random", 13, M=300, N=200, K=K, pad=pad)
    got, name = gu.run_dmu(p, return_name=True)
    assert "_kd_" in name, name
    gu.assert_close(got, gu.run_oracle(p), p, where=gu.valid_mask(p))
    gu.assert_bits_equal(got, gu.run_dmu(p, force="generic"), where=gu.valid_mask(p))


def test_device_info_matches_the_runtime():
    """The compute units and peak clock the bench derives its on-machine peak from."""
    import dense_matrix_unit_tiled_amd as dmu

    torch = gu._torch()
    cus, khz = dmu.dmu_device_info(0)
    assert cus == torch.cuda.get_device_properties(0).multi_processor_count
    assert 500_000 <= khz <= 5_000_000


# more tiles than one workgroup per compute unit, so that workers loop over several tiles
PERSIST_CASES = [
    ("c2", "128x128", dict(M=2000, N=4100, K=72)),            # 16 x 33 tiles, ragged edges
    ("c2", "256x256", dict(M=2000, N=8200, K=72)),            # 8 x 33 tiles
    ("c5", "256x128", dict(M=2000, N=4100, K=128)),           # int8, 8 x 33 tiles
    ("c3", None, dict(M=2000, N=4100, K=130)),                # rows 4-byte aligned, K tail
    ("c4s", None, dict(M=300, N=260, K=128, batch=40)),       # 3 x 3 tiles x 40 batches
    ("c1", "128x128", dict(M=2000, N=4000, K=64)),            # with C
    ("c6", None, dict(M=2000, N=4100, K=256)),                # e4m3, two K-tiles (main loop: no short-K form)
    ("c5", "128x128", dict(M=2000, N=4100, K=256)),           # int8, two K-tiles: the short-K loop
    ("c3", "256x128", dict(M=2000, N=4100, K=100)),           # 4-byte rows, two K-tiles, masked tail: short
]


@pytest.mark.parametrize("cfg,kernel,shape", PERSIST_CASES, ids=[f"{c}-{k}" for c, k, _ in PERSIST_CASES])
def test_persistent_form_matches(cfg, kernel, shape, monkeypatch):
    """The persistent form (a fixed set of workgroups looping over the tiles, the next tile's first
    K-tile -- or, when K spans at most the staging sets, its whole K range -- loaded before the
    current tile's epilogue), forced on problems with more tiles than
    workers, ragged edges and batches: against the oracle, and bit-identical to the
    one-workgroup-per-tile launch."""
    p = workloads.make(cfg, "random", 5, **shape)
    monkeypatch.setenv("DMU_PERSIST", "never")
    ref = gu.run_dmu(p, force=kernel)
    monkeypatch.setenv("DMU_PERSIST", "always")
    got = gu.run_dmu(p, force=kernel)
    assert np.array_equal(got, ref)
    want = gu.run_oracle(p)
    gu.assert_close(got, want, p, where=gu.valid_mask(p))


# long K loops under the forced persistent form (the default keeps it for four K-tiles or fewer)
PERSIST_LONG_K = [
    ("c2", "256x256", dict(M=2000, N=8200, K=1000)),          # bf16, 8 x 33 tiles, 16 K-tiles, K tail
    ("c6", "256x128", dict(M=2000, N=4200, K=1024)),          # e4m3, 8 x 33 tiles, 8 K-tiles
    ("c5", "256x256", dict(M=2100, N=8200, K=640)),           # int8, 9 x 33 tiles, 5 K-tiles
]


@pytest.mark.parametrize("cfg,kernel,shape", PERSIST_LONG_K, ids=[f"{c}-{k}" for c, k, _ in PERSIST_LONG_K])
def test_persistent_form_long_k(cfg, kernel, shape, monkeypatch):
    """The persistent form forced on K loops longer than its default's limit: bit-identical to the
    one-workgroup-per-tile launch, and on sampled outputs against the oracle."""
    p = workloads.make(cfg, "random", 7, **shape)
    monkeypatch.setenv("DMU_PERSIST", "never")
    ref = gu.run_dmu(p, force=kernel)
    monkeypatch.setenv("DMU_PERSIST", "always")
    got = gu.run_dmu(p, force=kernel)
    assert np.array_equal(got, ref)
    bij = gu.sample_bij(p, n=256, seed=3)
    gu.assert_close(got[gu.flat_index(p, bij)], gu.oracle_at(p, bij), p)


def int8_layouts(la, lb, seed, M, N, K):
    """An int8 problem with the same logical A and B values stored in the given layouts."""
    p = workloads.make("c5nn", "random", seed, M=M, N=N, K=K)
    a = np.asarray(p.A).reshape(1, M, p.lda)[:, :, :K].astype(np.float64)
    b = np.asarray(p.B).reshape(1, K, p.ldb)[:, :, :N].astype(np.float64)
    p.A, p.lda = workloads.store(a, "i8", la)
    p.B, p.ldb = workloads.store(b, "i8", lb)
    p.layout_a, p.layout_b = la, lb
    return p


@pytest.mark.parametrize("kernel", ["256x256", "256x128", "128x128"])
@pytest.mark.parametrize("lb", ["row", "col"])
def test_int8_column_major_a_tiled(kernel, lb):
    """A column-major int8 A (M a multiple of 16) takes the tiled kernel's 8-bit transposed LDS
    layout, with either B: exact against the oracle, and bit for bit against the fallback."""
    p = int8_layouts("col", lb, 41, M=272, N=304, K=448)
    got, name = gu.run_dmu(p, force=kernel, return_name=True)
    assert f"mfma_{kernel}_t8_{'t8' if lb == 'row' else 'k16'}_i8" in name, name
    gu.assert_close(got, gu.run_oracle(p), p, where=gu.valid_mask(p))
    gu.assert_bits_equal(got, gu.run_dmu(p, force="generic"), where=gu.valid_mask(p))
