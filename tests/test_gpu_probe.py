"""Single-wavefront layout probes on the GPU (the gfx950 counterpart of the
layout experiment, KingOfEgg sections 6-7): every (lane, register) of each
MFMA variant, the LDS fragment reads and the epilogue conversion.

A failure prints each wrong (lane, register) with the (row, col) the value
actually belongs to, so a wrong mapping is located at once.
"""
import numpy as np
import pytest

import dense_matrix_unit_tiled_amd as dmu
import oracle
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

MFMA = [dmu.DMU_PROBE_MFMA_32x32x16_BF16, dmu.DMU_PROBE_MFMA_32x32x16_F16,
        dmu.DMU_PROBE_MFMA_16x16x32_BF16, dmu.DMU_PROBE_MFMA_16x16x32_F16,
        dmu.DMU_PROBE_MFMA_32x32x32_I8, dmu.DMU_PROBE_MFMA_16x16x64_I8,
        dmu.DMU_PROBE_MFMA_16x16x128_E4M3]
TNAME = {dmu.DMU_BF16: "bf16", dmu.DMU_F16: "f16", dmu.DMU_I8: "i8", dmu.DMU_E4M3: "e4m3"}


def acc_owner(m: int, lane: int, r: int):
    """(row, col) of accumulator register r of lane `lane` (hypothesis under test)."""
    if m == 32:
        return 8 * (r // 4) + 4 * (lane // 32) + r % 4, lane % 32
    return 4 * (lane // 16) + r, lane % 16


def run_mfma_probe(variant, A, B):
    import torch

    m, n, k, t, regs = dmu.dmu_probe_info(variant)
    tn = TNAME[t]
    a_bits = np.ascontiguousarray(gu.workloads_to_bits(A, tn))
    bt_bits = np.ascontiguousarray(gu.workloads_to_bits(B.T.copy(), tn))
    out = torch.zeros(64 * regs, dtype=torch.int32, device="cuda:0")
    dmu.dmu_probe(variant, gu.to_dev(a_bits), gu.to_dev(bt_bits), out)
    torch.cuda.synchronize()
    raw = out.cpu().numpy().reshape(64, regs)
    return raw.view(np.float32) if tn != "i8" else raw


def check_mfma(variant, A, B):
    m, n, k, t, regs = dmu.dmu_probe_info(variant)
    got = run_mfma_probe(variant, A, B)
    D = A.astype(np.int64) @ B.astype(np.int64)
    bad = []
    for lane in range(64):
        for r in range(regs):
            i, j = acc_owner(m, lane, r)
            if got[lane, r] != D[i, j]:
                owners = list(zip(*np.nonzero(D == got[lane, r])))[:3]
                bad.append((lane, r, (i, j), got[lane, r], D[i, j], owners))
    assert not bad, "wrong (lane, reg): " + "; ".join(
        f"lane {l} reg {r} expected D{ij}={w} got {g} (found at {o})" for l, r, ij, g, w, o in bad[:12])


@pytest.mark.parametrize("variant", MFMA)
def test_mfma_layout_experiment_pattern(variant):
    """A[i][k] = i, B[k][j] = j  =>  D[i][j] = k * i * j, checked per lane and register."""
    m, n, k, t, regs = dmu.dmu_probe_info(variant)
    A = np.repeat(np.arange(m)[:, None], k, axis=1)
    B = np.repeat(np.arange(n)[None, :], k, axis=0)
    check_mfma(variant, A, B)


@pytest.mark.parametrize("variant", MFMA)
def test_mfma_k_pairing(variant):
    """A[i][k] = k, B[k][j] = k: any mismatch between how A and B pair their k
    slots lowers sum(k^2) (rearrangement inequality), which the i*j pattern cannot see."""
    m, n, k, t, regs = dmu.dmu_probe_info(variant)
    # values exact in the input type (e4m3 holds the integers up to 16; a mispairing
    # by a multiple of 16 is left to the random-integer probe)
    kk = np.arange(k) % {dmu.DMU_I8: 64, dmu.DMU_E4M3: 16}.get(t, 256)
    A = np.repeat(kk[None, :], m, axis=0)
    B = np.repeat(kk[:, None], n, axis=1)
    if t == dmu.DMU_I8:
        A, B = A - 32, B - 32
    check_mfma(variant, A, B)


@pytest.mark.parametrize("variant", MFMA)
def test_mfma_random_integers(variant):
    m, n, k, t, regs = dmu.dmu_probe_info(variant)
    rng = np.random.default_rng(variant)
    lo, hi = (-128, 128) if t == dmu.DMU_I8 else (-8, 9)
    check_mfma(variant, rng.integers(lo, hi, (m, k)), rng.integers(lo, hi, (k, n)))


@pytest.mark.parametrize("variant", [dmu.DMU_PROBE_MFMA_32x32x16_F16, dmu.DMU_PROBE_MFMA_32x32x16_BF16])
def test_mfma_keeps_subnormal_inputs(variant):
    """Subnormal fp16/bf16 inputs times 1 reach the fp32 accumulator unflushed."""
    import torch

    m, n, k, t, regs = dmu.dmu_probe_info(variant)
    tn = TNAME[t]
    a_bits = np.zeros((m, k), dtype=np.uint16)
    a_bits[:, 0] = np.arange(1, m + 1)  # the m smallest positive subnormals
    one = 0x3C00 if tn == "f16" else 0x3F80
    bt_bits = np.zeros((n, k), dtype=np.uint16)
    bt_bits[:, 0] = one
    out = torch.zeros(64 * regs, dtype=torch.int32, device="cuda:0")
    dmu.dmu_probe(variant, gu.to_dev(a_bits), gu.to_dev(bt_bits), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(64, regs).view(np.float32)
    vals = oracle.decode(tn, a_bits[:, 0])
    for lane in range(64):
        for r in range(regs):
            i, j = acc_owner(m, lane, r)
            assert got[lane, r] == np.float32(vals[i]), (lane, r, got[lane, r], vals[i])


def test_lds_read_b128():
    import torch

    img = np.arange(2048, dtype=np.uint16)
    addr = ((np.arange(64) * 37) % 256 * 16).astype(np.int32)
    out = torch.zeros(64 * 4, dtype=torch.int32, device="cuda:0")
    dmu.dmu_probe(dmu.DMU_PROBE_LDS_READ_B128, gu.to_dev(img), gu.to_dev(addr), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16).reshape(64, 8)
    want = np.stack([img[a // 2: a // 2 + 8] for a in addr])
    assert np.array_equal(got, want)


def test_lds_read_tr16_mapping():
    """ds_read_b64_tr_b16: within each group of 16 lanes, the 16 addressed 4-element
    rows R[j] (j = source lane in the group) are read transposed: output lane i gets
    element i % 4 of rows i / 4, i / 4 + 4, i / 4 + 8, i / 4 + 12.  So if lane j
    addresses X[k0 + j / 4][n0 + 4 * (j % 4)], output lane i holds X[k0 .. k0+3][n0 + i]:
    four consecutive k of one column, the operand layout of a K x N row-major tile."""
    import torch

    img = np.arange(2048, dtype=np.uint16)
    out = torch.zeros(64 * 2, dtype=torch.int32, device="cuda:0")
    # (a) lane j addresses its own 4 elements: the raw permutation
    addr = (np.arange(64) * 8).astype(np.int32)
    dmu.dmu_probe(dmu.DMU_PROBE_LDS_READ_TR16, gu.to_dev(img), gu.to_dev(addr), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16).reshape(64, 4)
    src = [[(int(v) // 4, int(v) % 4) for v in row] for row in got]
    want = [[(16 * (l // 16) + l % 16 // 4 + 4 * e, l % 4) for e in range(4)] for l in range(64)]
    table = "\n".join(f"lane {l:2d}: {src[l]}" for l in range(64))
    assert src == want, "observed (src lane, src elem) per output slot:\n" + table
    # (b) the operand use: a k x n row-major tile of 16-bit words (32 x 64 = the 4 KiB image)
    X = np.arange(32 * 64, dtype=np.uint16).reshape(32, 64)
    g = np.arange(64) // 16
    j = np.arange(64) % 16
    k0, n0 = 4 * g, 0
    addr = (((k0 + j // 4) * 64 + n0 + 4 * (j % 4)) * 2).astype(np.int32)
    dmu.dmu_probe(dmu.DMU_PROBE_LDS_READ_TR16, gu.to_dev(X.reshape(-1)), gu.to_dev(addr), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16).reshape(64, 4)
    for lane in range(64):
        kk = 4 * (lane // 16)
        assert np.array_equal(got[lane], X[kk:kk + 4, lane % 16]), lane


def test_lds_read_tr8_mapping():
    """ds_read_b64_tr_b8: within each group of 16 lanes, the 16 addressed 8-byte rows are read
    transposed byte-wise: if lane j addresses X[k0 + j / 2][n0 + 8 (j % 2) .. +7] of a K x N
    row-major byte tile, output lane i holds X[k0 .. k0+7][n0 + i] -- eight consecutive k of one
    column, half of an int8 / e4m3 operand fragment of the 16 x 16 x 64 instruction."""
    import torch

    out = torch.zeros(64 * 2, dtype=torch.int32, device="cuda:0")
    # (a) lane j addresses its own 8 bytes: the raw permutation.  Within group g the addressed
    # bytes lie in [128 g, 128 g + 128), so a byte's value (its position mod 256) names it.
    img = (np.arange(4096) % 256).astype(np.uint8)
    addr = (np.arange(64) * 8).astype(np.int32)
    dmu.dmu_probe(dmu.DMU_PROBE_LDS_READ_TR8, gu.to_dev(img), gu.to_dev(addr), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint8).reshape(64, 8)
    src = []
    for l in range(64):
        g = l // 16
        pos = [128 * g + ((int(v) - 128 * g) % 256) for v in got[l]]
        src.append([(p // 8, p % 8) for p in pos])
    want = [[(16 * (l // 16) + 2 * e + (l % 16) // 8, l % 8) for e in range(8)] for l in range(64)]
    table = "\n".join(f"lane {l:2d}: {src[l]}" for l in range(64))
    assert src == want, "observed (src lane, src byte) per output byte:\n" + table
    # (b) the operand use: a 32 x 128 row-major byte tile
    X = (np.arange(32 * 128) * 7 % 251).astype(np.uint8).reshape(32, 128)
    g = np.arange(64) // 16
    j = np.arange(64) % 16
    k0, n0 = 8 * g, 16 * g
    addr = ((k0 + j // 2) * 128 + n0 + 8 * (j % 2)).astype(np.int32)
    dmu.dmu_probe(dmu.DMU_PROBE_LDS_READ_TR8, gu.to_dev(X.reshape(-1)), gu.to_dev(addr), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint8).reshape(64, 8)
    for lane in range(64):
        kk, nn = 8 * (lane // 16), 16 * (lane // 16) + lane % 16
        assert np.array_equal(got[lane], X[kk:kk + 8, nn]), lane


def test_lds_fragment_format():
    """The tiled kernel's staging writes + fragment reads of a K-contiguous tile return,
    for lane l, row block rb and K-step ks, bytes 64*ks + 16*(l/16) .. +15 of logical
    row 16*rb + l % 16."""
    import torch

    words = np.arange(32 * 64, dtype=np.uint16)  # 32 rows x 64 16-bit words = 128 bytes/row
    out = torch.zeros(64 * 16, dtype=torch.int32, device="cuda:0")
    dmu.dmu_probe(dmu.DMU_PROBE_LDS_FRAG, gu.to_dev(words), None, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16).reshape(64, 2, 2, 8)
    for lane in range(64):
        for rb in range(2):
            for ks in range(2):
                w0 = (16 * rb + lane % 16) * 64 + (64 * ks + 16 * (lane // 16)) // 2
                assert np.array_equal(got[lane, rb, ks], words[w0: w0 + 8]), (lane, rb, ks)


def test_lds_fragment_format_transposed():
    """The tiled kernel's staging writes + transposing fragment reads of an M/N-contiguous
    tile (64 K-rows x 128 values) return, for lane l, column block cb and K-step ks, the
    values X[32*ks + 8*(l/16) + 0..7][16*cb + l % 16]: the operand layout of the 16 x 16
    instruction."""
    import torch

    X = np.arange(64 * 128, dtype=np.uint16).reshape(64, 128)
    out = torch.zeros(64 * 64, dtype=torch.int32, device="cuda:0")
    dmu.dmu_probe(dmu.DMU_PROBE_LDS_FRAG_T, gu.to_dev(X.reshape(-1)), None, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16).reshape(64, 8, 2, 8)
    for lane in range(64):
        for cb in range(8):
            for ks in range(2):
                k0 = 32 * ks + 8 * (lane // 16)
                want = X[k0: k0 + 8, 16 * cb + lane % 16]
                assert np.array_equal(got[lane, cb, ks], want), (lane, cb, ks, got[lane, cb, ks], want)


@pytest.mark.parametrize("t,variant", [("bf16", dmu.DMU_PROBE_CVT_BF16), ("f16", dmu.DMU_PROBE_CVT_F16)])
def test_epilogue_conversion_rounds_to_nearest_even(t, variant):
    import torch

    rng = np.random.default_rng(5)
    special = [1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -11, 1 + 3 * 2 ** -11, -(1 + 2 ** -8),
               2.0 ** -24, 1.5 * 2 ** -24, 2.5 * 2 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
               2.0 ** -130, 1.5 * 2 ** -133, 65504.0, 65519.0, 65520.0, 1e30, -1e30,
               np.inf, -np.inf, 0.0, -0.0, 3.0e38]
    x = np.concatenate([np.array(special), rng.standard_normal(256 - len(special) - 32) *
                        2.0 ** rng.integers(-30, 20, 256 - len(special) - 32),
                        rng.uniform(-1, 1, 32) * 2.0 ** -20]).astype(np.float32)
    out = torch.zeros(256, dtype=torch.int16, device="cuda:0")
    dmu.dmu_probe(variant, gu.to_dev(x), None, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    want = oracle.encode(t, x.astype(np.float64))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


def test_lane_swap_pairs():
    """v_permlane16_swap / v_permlane32_swap with equal operands give each lane the values of
    lanes l and l^16 (l^32), in some order: the attention kernel's row max over 4 lanes."""
    import torch

    vals = (np.arange(64, dtype=np.uint32) * 7919 + 13).astype(np.uint32)
    out = torch.zeros(64 * 4, dtype=torch.int32, device="cuda:0")
    dmu.dmu_probe(dmu.DMU_PROBE_LANE_SWAP, gu.to_dev(vals.view(np.int32)), None, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32).reshape(64, 4)
    for lane in range(64):
        assert sorted(got[lane, :2]) == sorted([vals[lane], vals[lane ^ 16]]), lane
        assert sorted(got[lane, 2:]) == sorted([vals[lane], vals[lane ^ 32]]), lane


@pytest.mark.parametrize("in_type,peak", [("bf16", 2500.0), ("i8", 5000.0)])
def test_mfma_ceiling_rate_and_stamps(in_type, peak):
    """The ceiling microbenchmark runs at a plausible fraction of the published dense peak (never
    above it) and stamps every workgroup with a consistent start and end."""
    import torch

    wgs, rounds = 256, 64
    stamps = torch.zeros(wgs * 4, dtype=torch.int64, device="cuda:0")
    for _ in range(50):
        dmu.dmu_mfma_ceiling(in_type, rounds, wgs)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(20):
        dmu.dmu_mfma_ceiling(in_type, rounds, wgs)
    e1.record()
    dmu.dmu_mfma_ceiling(in_type, rounds, wgs, stamps)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / 20
    flop = wgs * 8 * rounds * 32 * 16 * 16 * (64 if in_type == "i8" else 32) * 2
    tflops = flop / (us * 1e-6) / 1e12
    assert 0.2 * peak < tflops <= 1.02 * peak, tflops
    r = stamps.view(-1, 4).cpu().numpy()
    assert np.all(r[:, 0] > 0) and np.all(r[:, 2] >= r[:, 0]) and np.all(r[:, 3] > r[:, 1])
