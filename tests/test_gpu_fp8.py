"""Parity of the FP8 e4m3 GEMM with the oracle.

e4m3 inputs, fp32 accumulation, fp32/fp16/bf16 output ("Tensor Cores, CUTLASS
and CuTe", sections 2.1 and 6.5), through the C ABI against the oracle: element
by element at reduced sizes (several tiles, ragged M/N/K, each kernel family,
K-contiguous and other layouts), bit for bit where every step is exact
(integer-valued data, the largest and subnormal e4m3 values), the tiled kernel
against the fallback bit for bit, batches with strides, the fused epilogue, and
sampled outputs of the full 8192^3 problem.

The bar is that of the 16-bit inputs: |D - ref| <= 1e-3 sqrt(K) max|A| max|B|
[+ 2e-2 |ref| for 16-bit outputs] -- e4m3 products are exact in fp32, so the
accumulation is the only source of error, as for fp16/bf16 inputs.
"""
import numpy as np
import pytest

import dense_matrix_unit_tiled_amd as dmu
import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

KERNELS = [None, "256x128", "128x128", "64x128", "generic"]


def problem(out_t, seed, M=300, N=270, K=384, la="row", lb="col", batch=1, pad=0, with_c=False,
            kind="random"):
    p = workloads.make("c6", kind, seed, M=M, N=N, K=K, batch=batch, pad=pad, with_c=with_c)
    if (la, lb) != ("row", "col"):
        # same logical values stored in the requested layouts
        vals_a = gu.values(p.A, "e4m3").reshape(batch, M, p.lda)[:, :, :K]
        vals_b = gu.values(p.B, "e4m3").reshape(batch, N, p.ldb)[:, :, :K].transpose(0, 2, 1)
        p.A, p.lda = workloads.store(vals_a, "e4m3", la, pad)
        p.B, p.ldb = workloads.store(vals_b, "e4m3", lb, pad)
        p.layout_a, p.layout_b = la, lb
        if batch > 1:
            p.stride_a = (M if la == "row" else K) * p.lda
            p.stride_b = (K if lb == "row" else N) * p.ldb
    if out_t != p.out_type:
        p = workloads.with_output(p, out_t, seed)
    return p


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("out_t", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("K", [384, 200, 130])
def test_reduced_parity(out_t, kernel, K):
    """K = 384: 16-byte rows; 200: 4-byte rows with a masked K tail; 130: the fallback."""
    p = problem(out_t, 1, K=K, with_c=out_t != "f32")
    got = gu.run_dmu(p, force=kernel)
    gu.assert_close(got, gu.run_oracle(p), p, where=gu.valid_mask(p))


@pytest.mark.parametrize("la,lb", [("row", "row"), ("col", "col"), ("col", "row")])
def test_other_layouts(la, lb):
    """An M-contiguous A whose M, or an N-contiguous B whose N, is not a multiple of 16 goes
    through the fallback kernel."""
    p = problem("bf16", 2, M=150, N=140, K=260, la=la, lb=lb)
    got, name = gu.run_dmu(p, return_name=True)
    assert "generic" in name, name
    gu.assert_close(got, gu.run_oracle(p), p, where=gu.valid_mask(p))


@pytest.mark.parametrize("kernel", ["256x128", "128x128"])
@pytest.mark.parametrize("out_t", ["f32", "bf16"])
@pytest.mark.parametrize("K", [384, 200])
@pytest.mark.parametrize("la,lb", [("row", "row"), ("col", "col"), ("col", "row")])
def test_transposed_8bit_tiled(kernel, out_t, K, la, lb):
    """A row-major B (N-contiguous, N a multiple of 16) or a column-major A (M-contiguous, M a
    multiple of 16) takes the tiled kernel's 8-bit transposed LDS layout (ds_read_b64_tr_b8
    fragments): against the oracle, and bit for bit against the fallback, which issues the same
    instructions on the same fragments."""
    p = problem(out_t, 4, M=304, N=272, K=K, la=la, lb=lb, with_c=out_t != "f32")
    got, name = gu.run_dmu(p, force=kernel, return_name=True)
    assert "_t8_" in name and kernel in name, name
    gu.assert_close(got, gu.run_oracle(p), p, where=gu.valid_mask(p))
    gu.assert_bits_equal(got, gu.run_dmu(p, force="generic"), where=gu.valid_mask(p))


@pytest.mark.parametrize("kernel", ["256x128", "128x128"])
def test_tiled_equals_fallback_bit_for_bit(kernel):
    p = problem("f32", 3, M=520, N=264, K=640)
    a = gu.run_dmu(p, force=kernel)
    b = gu.run_dmu(p, force="generic")
    gu.assert_bits_equal(a, b, where=gu.valid_mask(p))


@pytest.mark.parametrize("out_t", ["f32", "bf16"])
def test_structured_exact(out_t):
    """A = i mod 16, B = j mod 8 (exact in e4m3): every sum is exact, D matches bit for bit."""
    p = problem(out_t, 0, M=300, N=260, K=1024, kind="structured")
    got = gu.run_dmu(p)
    gu.assert_bits_equal(got, gu.run_oracle(p), where=gu.valid_mask(p))


def test_largest_values_exact():
    """448 * -448 summed over K = 1024: -2^22 * 49 * ... exact in fp32."""
    p = problem("f32", 0, M=128, N=136, K=1024)
    p.A = np.full_like(p.A, 0x7E)   # 448
    p.B = np.full_like(p.B, 0xFE)   # -448
    got = gu.run_dmu(p)
    mask = gu.valid_mask(p)
    assert np.all(got[mask] == np.float32(-1024 * 448.0 * 448.0))


def test_subnormal_inputs_kept():
    """e4m3 subnormals m 2^-9 times 1 reach the fp32 accumulator unflushed."""
    M, N, K = 64, 64, 128
    p = problem("f32", 0, M=M, N=N, K=K)
    A = np.zeros((M, K), dtype=np.uint8)
    A[:, 5] = (np.arange(M) % 7) + 1            # subnormal codes 1..7
    p.A = A.ravel()
    p.B = np.full((N, K), 0x38, dtype=np.uint8).ravel()  # 1.0
    got = gu.run_dmu(p).reshape(M, p.ldd)[:, :N]
    want = ((np.arange(M) % 7) + 1) * 2.0 ** -9
    assert np.array_equal(got, np.repeat(want[:, None], N, axis=1).astype(np.float32))


def test_batched_with_strides():
    p = problem("bf16", 4, M=200, N=136, K=256, batch=3, pad=16, with_c=True)
    got = gu.run_dmu(p)
    gu.assert_close(got, gu.run_oracle(p), p, where=gu.valid_mask(p))


@pytest.mark.parametrize("act", ["none", "gelu_tanh"])
def test_fused_epilogue(act):
    """Per-row and per-column scales (FP8 dequantisation), bias and an activation."""
    p = problem("bf16", 5, M=300, N=260, K=512)
    ep = workloads.make_epilogue(p, 3, act=act)
    got = gu.run_dmu(p, ep=ep)
    want = gu.run_oracle(p, ep=ep)
    bij = gu.all_bij(p)
    idx = gu.flat_index(p, bij)
    gu.assert_close_epilogue(got[idx], want[idx], p, ep, bij)


def test_full_size_sampled():
    """The full 8192^3 e4m3 problem (bf16 output) on sampled outputs evaluated one by one."""
    p = workloads.make("c6", "random", 0)
    got = gu.run_dmu(p)
    bij = gu.sample_bij(p, n=384)
    want = gu.oracle_at(p, bij)
    idx = gu.flat_index(p, bij)
    gu.assert_close(got[idx], want, p)
