"""The C-ABI library on the CPU: it loads, exports every function include/dmu.h
declares, and rejects bad arguments before any HIP call (no GPU is touched:
only validation, kernel selection and static strings are exercised)."""
import ctypes
import os
import re

import pytest

import dense_matrix_unit_tiled_amd as dmu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "dmu.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dmu_\w+)\s*\(", text)))


def test_exports_every_declared_function():
    lib = ctypes.CDLL(dmu.LIB_PATH)
    names = declared_functions()
    assert {"dmu_gemm", "dmu_gemm_check", "dmu_gemm_kernel_name", "dmu_status_string",
            "dmu_last_error", "dmu_probe", "dmu_probe_info"} <= set(names)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_device_info_argument_errors():
    """NULL outputs and negative devices are rejected before any HIP call."""
    lib = dmu.library()
    c = ctypes.c_int()
    assert lib.dmu_device_info(0, None, ctypes.byref(c)) == dmu.DMU_ERR_INVALID_ARG
    assert lib.dmu_device_info(0, ctypes.byref(c), None) == dmu.DMU_ERR_INVALID_ARG
    assert lib.dmu_device_info(-1, ctypes.byref(c), ctypes.byref(c)) == dmu.DMU_ERR_INVALID_ARG
    assert "negative device" in dmu.dmu_last_error()


def test_struct_layout_matches_header():
    # 4 int64 + 5 int32 (+4 pad) + 4 x (pointer + 2 int64)
    assert ctypes.sizeof(dmu.dmu_gemm_args) == 32 + 24 + 4 * 24
    assert dmu.dmu_gemm_args.A.offset == 56
    # 3 x (pointer + int64) + int32 (+4 pad)
    assert ctypes.sizeof(dmu.dmu_epilogue) == 3 * 16 + 8
    assert dmu.dmu_epilogue.act.offset == 48


FAKE = 1 << 40  # device-looking addresses; never dereferenced by validation


def args(**kw):
    base = dict(M=256, N=256, K=256, A=FAKE, lda=256, B=FAKE + (1 << 30), ldb=256,
                D=FAKE + (2 << 30), ldd=256, in_type="f16", out_type="f32")
    base.update(kw)
    return dmu.gemm_args(**base)


def test_valid_arguments_pass():
    assert dmu.dmu_gemm_check(args()) == dmu.DMU_OK
    assert dmu.dmu_last_error() == ""


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), dmu.DMU_ERR_INVALID_ARG),
    (dict(K=-5), dmu.DMU_ERR_INVALID_ARG),
    (dict(lda=255), dmu.DMU_ERR_INVALID_ARG),
    (dict(ldb=100), dmu.DMU_ERR_INVALID_ARG),
    (dict(ldd=10), dmu.DMU_ERR_INVALID_ARG),
    (dict(A=None), dmu.DMU_ERR_INVALID_ARG),
    (dict(D=None), dmu.DMU_ERR_INVALID_ARG),
    (dict(out_type="i32"), dmu.DMU_ERR_UNSUPPORTED),
    (dict(in_type="i8", out_type="f32", acc_type="f32"), dmu.DMU_ERR_UNSUPPORTED),
    (dict(in_type="i8", out_type="i32", acc_type="f32"), dmu.DMU_ERR_UNSUPPORTED),
    (dict(in_type="f32", out_type="f32"), dmu.DMU_ERR_UNSUPPORTED),
    (dict(in_type="bf16", out_type="f16"), dmu.DMU_ERR_UNSUPPORTED),
    (dict(D=FAKE + 100), dmu.DMU_ERR_INVALID_ARG),                 # D overlaps A
    (dict(batch=2, stride_d=100), dmu.DMU_ERR_INVALID_ARG),        # batches of D overlap
    (dict(stride_a=-1, batch=2, stride_d=65536), dmu.DMU_ERR_INVALID_ARG),
    (dict(C=FAKE + (2 << 30) + 4, ldc=256), dmu.DMU_ERR_INVALID_ARG),  # C partially overlaps D
    (dict(M=1 << 31), dmu.DMU_ERR_UNSUPPORTED),
    (dict(D=FAKE + (2 << 30) + 1), dmu.DMU_ERR_INVALID_ARG),      # not element aligned
    (dict(layout_a="row", lda=0, K=0), dmu.DMU_ERR_INVALID_ARG),
])
def test_rejections(kw, status):
    a = args(**kw)
    assert dmu.dmu_gemm_check(a) == status
    assert dmu.dmu_last_error() != ""
    with pytest.raises(dmu.DmuError) as e:
        dmu.dmu_gemm(a, stream=0)  # rejected before any HIP call
    assert e.value.status == status


def test_in_place_c_equal_d_allowed():
    d = FAKE + (2 << 30)
    assert dmu.dmu_gemm_check(args(C=d, ldc=256)) == dmu.DMU_OK


def test_bad_layout_code():
    a = args()
    a.layout_a = 7
    assert dmu.dmu_gemm_check(a) == dmu.DMU_ERR_INVALID_ARG


def test_empty_problems_launch_nothing():
    for kw in (dict(M=0), dict(N=0), dict(batch=0)):
        a = args(**kw)
        assert dmu.dmu_gemm_check(a) == dmu.DMU_OK
        assert dmu.dmu_gemm_kernel_name(a) is None
        assert dmu.dmu_gemm(a, stream=0) == dmu.DMU_OK  # returns before any HIP call


@pytest.mark.parametrize("kw,expect", [
    (dict(M=4096, N=4096, K=4096, lda=4096, ldb=4096, ldd=4096, in_type="bf16", out_type="bf16"),
     "mfma_256x256_k16_t16_bf16_bf16"),
    (dict(M=4096, N=4096, K=4096, lda=4096, layout_b="col", ldb=4096, ldd=4096, in_type="bf16",
          out_type="bf16"), "mfma_256x256_k16_k16_bf16_bf16"),
    (dict(in_type="f16", out_type="f32"), "mfma_64x128_k16_t16_f16_f32"),   # few tiles: 64 x 128
    (dict(M=1024, N=1024, K=16384, lda=16384, ldb=1024, ldd=1024, in_type="bf16", out_type="bf16"),
     "mfma_64x128_k16_t16_bf16_bf16"),                                          # 64 tiles of 128 x 128
    (dict(M=1408, N=1408, K=512, lda=512, ldb=1408, ldd=1408, in_type="bf16", out_type="bf16"),
     "mfma_64x128_k16_t16_bf16_bf16"),                                          # 121 tiles of 128 x 128
    (dict(M=1536, N=1536, K=512, lda=512, ldb=1536, ldd=1536, in_type="bf16", out_type="bf16"),
     "mfma_128x128_k16_t16_bf16_bf16"),                                         # 144: no longer few
    (dict(layout_a="col", in_type="f16", out_type="f32"), "mfma_128x128_t16_t16_f16_f32"),  # A M-contiguous
    (dict(M=5000, N=3000, K=2050, lda=2050, layout_b="col", ldb=2050, ldd=3000, in_type="f16",
          out_type="f16", acc_type="f16"), "mfma_256x256_kd_kd_f16_f16"),
    (dict(M=8192, N=8192, K=8192, lda=8192, layout_b="col", ldb=8192, ldd=8192, in_type="i8",
          out_type="i32"), "mfma_256x256_k16_k16_i8_i32"),
    # 8-bit row-major B: the 8-bit transposed LDS layout when N is a multiple of 16, else the fallback
    (dict(M=8192, N=8192, K=8192, lda=8192, ldb=8192, ldd=8192, in_type="i8", out_type="i32"),
     "mfma_256x256_k16_t8_i8_i32"),
    (dict(M=8192, N=8184, K=8192, lda=8192, ldb=8184, ldd=8184, in_type="i8", out_type="i32"),
     "mfma_generic64_any_any_i8_i32"),
    (dict(M=4096, N=4096, K=4096, lda=4096, ldb=4096, ldd=4096, in_type="e4m3", out_type="bf16",
          acc_type="f32"), "mfma_256x128_k16_t8_e4m3_bf16"),
    (dict(M=4096, N=4096, K=4096, lda=4096, layout_a="col", ldb=4096, ldd=4096, in_type="i8",
          out_type="i32"), "mfma_256x256_t8_t8_i8_i32"),   # 8-bit column-major A and row-major B
    (dict(M=4096, N=4096, K=4096, lda=4096, layout_a="col", ldb=4096, layout_b="col", ldd=4096,
          in_type="i8", out_type="i32"), "mfma_256x256_t8_k16_i8_i32"),
    (dict(M=4088, N=4096, K=4096, lda=4088, layout_a="col", ldb=4096, ldd=4096, in_type="i8",
          out_type="i32"), "mfma_generic64_any_any_i8_i32"),   # M not a multiple of 16
    (dict(M=4096, N=128, K=4096, lda=4096, ldb=128, ldd=128, batch=32, stride_a=4096 * 4096,
          stride_b=4096 * 128, stride_d=4096 * 128), "mfma_256x128_k16_t16_f16_f32"),
    # two K-tiles or fewer: 256 x 128 even with enough tiles for 256 x 256; four: 256 x 256
    (dict(M=4096, N=4096, K=128, lda=128, layout_b="col", ldb=128, ldd=4096, batch=32,
          stride_a=4096 * 128, stride_b=4096 * 128, stride_d=4096 * 4096), "mfma_256x128_k16_k16_f16_f32"),
    (dict(M=4096, N=4096, K=256, lda=256, layout_b="col", ldb=256, ldd=4096, batch=32,
          stride_a=4096 * 256, stride_b=4096 * 256, stride_d=4096 * 4096), "mfma_256x256_k16_k16_f16_f32"),
    (dict(A=FAKE + 2), "mfma_generic64_any_any_f16_f32"),       # 2-byte aligned A
    (dict(K=255, lda=255, ldb=256), "mfma_generic64_any_any_f16_f32"),  # odd K row-major A
    (dict(K=0, lda=1), "mfma_generic64_any_any_f16_f32"),
])
def test_kernel_selection(kw, expect):
    assert dmu.dmu_gemm_kernel_name(args(**kw)) == expect


def test_force_generic_env(monkeypatch):
    monkeypatch.setenv("DMU_FORCE_KERNEL", "generic")
    assert dmu.dmu_gemm_kernel_name(args()) == "mfma_generic64_any_any_f16_f32"


def test_status_strings():
    for s in (dmu.DMU_OK, dmu.DMU_ERR_INVALID_ARG, dmu.DMU_ERR_UNSUPPORTED, dmu.DMU_ERR_HIP):
        assert dmu.dmu_status_string(s).startswith("DMU_")
    assert "unknown" in dmu.dmu_status_string(42)


def test_probe_info():
    assert dmu.dmu_probe_info(dmu.DMU_PROBE_MFMA_32x32x16_BF16) == (32, 32, 16, dmu.DMU_BF16, 16)
    assert dmu.dmu_probe_info(dmu.DMU_PROBE_MFMA_16x16x64_I8) == (16, 16, 64, dmu.DMU_I8, 4)
    with pytest.raises(dmu.DmuError):
        dmu.dmu_probe_info(999)
    with pytest.raises(dmu.DmuError):
        dmu.dmu_probe(dmu.DMU_PROBE_MFMA_32x32x16_BF16, None, None, None, stream=0)


def ep(**kw):
    base = dict(row_scale=FAKE + (3 << 30), col_scale=FAKE + (3 << 30) + 4096, bias=FAKE + (3 << 30) + 8192,
                act="gelu_tanh")
    base.update(kw)
    return dmu.epilogue_args(**base)


@pytest.mark.parametrize("in_t,out_t", [("f16", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("bf16", "f32"),
                                        ("i8", "f32"), ("i8", "f16"), ("i8", "bf16")])
def test_epilogue_valid(in_t, out_t):
    a = args(in_type=in_t, out_type=out_t)
    assert dmu.dmu_gemm_ex_check(a, ep()) == dmu.DMU_OK
    assert dmu.dmu_gemm_ex_check(a, None) == dmu.DMU_OK
    assert dmu.dmu_gemm_ex_check(a, ep(row_scale=None, col_scale=None, bias=None, act="relu")) == dmu.DMU_OK
    # batched, broadcast (stride 0) and strided vectors
    b = args(in_type=in_t, out_type=out_t, batch=3, stride_d=256 * 256, stride_a=0, stride_b=0)
    assert dmu.dmu_gemm_ex_check(b, ep(stride_row_scale=300, stride_col_scale=0, stride_bias=260)) == dmu.DMU_OK


@pytest.mark.parametrize("kw,akw,status", [
    (dict(act=3), {}, dmu.DMU_ERR_INVALID_ARG),
    (dict(act=-1), {}, dmu.DMU_ERR_INVALID_ARG),
    (dict(stride_bias=-1), {}, dmu.DMU_ERR_INVALID_ARG),
    (dict(col_scale=FAKE + (3 << 30) + 2), {}, dmu.DMU_ERR_INVALID_ARG),          # misaligned
    (dict(bias=FAKE + (2 << 30) + 64), {}, dmu.DMU_ERR_INVALID_ARG),               # bias inside D
    (dict(), dict(in_type="i8", out_type="i32"), dmu.DMU_ERR_UNSUPPORTED),        # int32 takes no epilogue
    (dict(row_scale=None, col_scale=None, bias=None, act="relu"), dict(in_type="i8", out_type="i32"),
     dmu.DMU_ERR_UNSUPPORTED),
])
def test_epilogue_rejections(kw, akw, status):
    a = args(**akw)
    e = ep(**kw)
    assert dmu.dmu_gemm_ex_check(a, e) == status
    assert dmu.dmu_last_error() != ""
    with pytest.raises(dmu.DmuError) as err:
        dmu.dmu_gemm_ex(a, e, stream=0)  # rejected before any HIP call
    assert err.value.status == status


def test_int32_output_takes_empty_epilogue():
    a = args(in_type="i8", out_type="i32")
    assert dmu.dmu_gemm_ex_check(a, dmu.epilogue_args()) == dmu.DMU_OK


@pytest.mark.parametrize("out_t", ["f32", "f16", "bf16"])
def test_dequantising_kernel_names(out_t):
    a = args(in_type="i8", out_type=out_t, K=512, lda=512, ldb=512, layout_b="col")
    assert dmu.dmu_gemm_kernel_name(a).endswith(f"i8_{out_t}")


def att(**kw):
    base = dict(batch=2, seq_q=300, seq_k=200, head_dim=128, Q=FAKE, ldq=128, K=FAKE + (1 << 30), ldk=128,
                V=FAKE + (2 << 30), ldv=128, O=FAKE + (3 << 30), ldo=128, in_type="f16", out_type="f32",
                scale=0.088, stride_q=300 * 128, stride_k=200 * 128, stride_v=200 * 128, stride_o=300 * 128)
    base.update(kw)
    return dmu.attention_args(**base)


def test_attention_struct_layout():
    # 4 int64 + 2 int32 + float (+4 pad) + 4 x (pointer + 2 int64)
    assert ctypes.sizeof(dmu.dmu_attention_args) == 32 + 16 + 4 * 24
    assert dmu.dmu_attention_args.Q.offset == 48


@pytest.mark.parametrize("kw", [dict(), dict(in_type="bf16", out_type="bf16"), dict(out_type="f16"),
                                dict(batch=0), dict(seq_q=0), dict(seq_q=1, seq_k=1, batch=1)])
def test_attention_valid(kw):
    assert dmu.dmu_attention_check(att(**kw)) == dmu.DMU_OK


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), dmu.DMU_ERR_UNSUPPORTED),
    (dict(in_type="f32"), dmu.DMU_ERR_UNSUPPORTED),
    (dict(out_type="i32"), dmu.DMU_ERR_UNSUPPORTED),
    (dict(seq_k=0), dmu.DMU_ERR_INVALID_ARG),
    (dict(seq_q=-1), dmu.DMU_ERR_INVALID_ARG),
    (dict(ldk=100), dmu.DMU_ERR_INVALID_ARG),
    (dict(ldq=130), dmu.DMU_ERR_UNSUPPORTED),                    # rows not 16-byte aligned
    (dict(V=FAKE + (2 << 30) + 2), dmu.DMU_ERR_UNSUPPORTED),      # misaligned pointer
    (dict(stride_o=100), dmu.DMU_ERR_INVALID_ARG),               # batches of O overlap
    (dict(O=FAKE + 4096), dmu.DMU_ERR_INVALID_ARG),              # O overlaps Q
    (dict(K=None), dmu.DMU_ERR_INVALID_ARG),
    (dict(stride_k=-1), dmu.DMU_ERR_INVALID_ARG),
])
def test_attention_rejections(kw, status):
    a = att(**kw)
    assert dmu.dmu_attention_check(a) == status
    assert dmu.dmu_last_error() != ""
    with pytest.raises(dmu.DmuError) as e:
        dmu.dmu_attention(a, stream=0)  # rejected before any HIP call
    assert e.value.status == status


TN8 = dict(layout_b="col", in_type="e4m3")


@pytest.mark.parametrize("kw,expect", [
    (dict(M=8192, N=8192, K=8192, lda=8192, ldb=8192, ldd=8192, out_type="bf16", **TN8),
     "mfma_256x128_k16_k16_e4m3_bf16"),
    (dict(out_type="f32", **TN8), "mfma_64x128_k16_k16_e4m3_f32"),
    (dict(K=200, lda=200, ldb=200, out_type="f16", **TN8), "mfma_64x128_kd_kd_e4m3_f16"),
    (dict(K=130, lda=130, ldb=130, out_type="f32", **TN8), "mfma_generic64_any_any_e4m3_f32"),
    (dict(in_type="e4m3", out_type="f32"), "mfma_64x128_k16_t8_e4m3_f32"),  # B row-major: 8-bit transposed
    (dict(in_type="e4m3", out_type="f32", N=250, ldb=250, ldd=250), "mfma_generic64_any_any_e4m3_f32"),
    (dict(M=4096, N=128, K=4096, lda=4096, ldb=4096, ldd=128, out_type="f32", **TN8),
     "mfma_256x128_k16_k16_e4m3_f32"),
])
def test_e4m3_kernel_selection(kw, expect):
    assert dmu.dmu_gemm_kernel_name(args(**kw)) == expect


def test_e4m3_never_takes_the_256x256_tile(monkeypatch):
    """e4m3 fragments need the registers of a 64 x 64 wavefront tile: a forced 256x256 runs 256x128."""
    monkeypatch.setenv("DMU_FORCE_KERNEL", "256x256")
    a = args(M=4096, N=4096, K=4096, lda=4096, ldb=4096, ldd=4096, out_type="bf16", **TN8)
    assert dmu.dmu_gemm_kernel_name(a) == "mfma_256x128_k16_k16_e4m3_bf16"


@pytest.mark.parametrize("kw", [dict(out_type="i32"), dict(out_type="f32", acc_type="i32"),
                                dict(out_type="f16", acc_type="f16")])
def test_e4m3_rejections(kw):
    assert dmu.dmu_gemm_check(args(in_type="e4m3", **kw)) == dmu.DMU_ERR_UNSUPPORTED


@pytest.mark.parametrize("out_t", ["f32", "f16", "bf16"])
def test_e4m3_epilogue_valid(out_t):
    assert dmu.dmu_gemm_ex_check(args(out_type=out_t, **TN8), ep()) == dmu.DMU_OK


def test_e4m3_probe_info():
    assert dmu.dmu_probe_info(dmu.DMU_PROBE_MFMA_16x16x128_E4M3) == (16, 16, 128, dmu.DMU_E4M3, 4)


def test_streamk_argument_errors_before_any_hip_call():
    lib = ctypes.CDLL(dmu.LIB_PATH)
    lib.dmu_gemm_streamk_workspace_size.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    assert lib.dmu_gemm_streamk_workspace_size(ctypes.addressof(args()), None) == dmu.DMU_ERR_INVALID_ARG
    assert dmu.dmu_gemm_streamk(args(M=-1), None, None, 0, stream=0, check=False) == dmu.DMU_ERR_INVALID_ARG
    assert dmu.dmu_gemm_streamk(args(out_type="i32"), None, None, 0, stream=0, check=False) == \
        dmu.DMU_ERR_UNSUPPORTED
    assert dmu.dmu_gemm_streamk(args(M=0), None, None, 0, stream=0) == dmu.DMU_OK  # empty: nothing launched


def test_streamk_error_query_argument_errors_before_any_hip_call():
    """A NULL result pointer or a misaligned workspace is rejected before the query touches the
    GPU (a NULL workspace names the library's own scratch, a GPU-side path)."""
    lib = dmu.library()
    failed = ctypes.c_int(7)
    assert lib.dmu_gemm_streamk_error(FAKE, None, None) == dmu.DMU_ERR_INVALID_ARG
    assert lib.dmu_gemm_streamk_error(FAKE + 4, None, ctypes.byref(failed)) == dmu.DMU_ERR_INVALID_ARG
    assert "aligned" in dmu.dmu_last_error()
    assert failed.value == 0
    with pytest.raises(dmu.DmuError):
        dmu.dmu_gemm_streamk_error(FAKE + 4, stream=0)


def test_phase_log_argument_errors():
    """The phase log takes a buffer with a count, or NULL with 0; checked before any HIP call."""
    lib = dmu.library()
    assert lib.dmu_phase_log(None, 4) == dmu.DMU_ERR_INVALID_ARG
    assert "record count" in dmu.dmu_last_error()
    assert lib.dmu_phase_log(ctypes.c_void_p(1 << 40), 0) == dmu.DMU_ERR_INVALID_ARG
    assert lib.dmu_phase_log(ctypes.c_void_p((1 << 40) + 4), 4) == dmu.DMU_ERR_INVALID_ARG
    assert "aligned" in dmu.dmu_last_error()
    assert lib.dmu_phase_log(None, 0) == dmu.DMU_OK
    n, k = ctypes.c_size_t(7), ctypes.c_int(7)
    assert lib.dmu_phase_log_last(None, ctypes.byref(k)) == dmu.DMU_ERR_INVALID_ARG
    assert lib.dmu_phase_log_last(ctypes.byref(n), None) == dmu.DMU_ERR_INVALID_ARG
    assert dmu.dmu_phase_log_last() == (0, 0)


def test_phase_log_capacity_checked_before_launch(monkeypatch):
    """A launch that would write more records than the log holds fails before any HIP call
    (the log is never dereferenced on the host; the problem's 128 tiles need 128 records)."""
    monkeypatch.setenv("DMU_PERSIST", "never")  # no device query for the persistent choice
    fake = 1 << 40
    a = dmu.gemm_args(1024, 1024, 256, fake, 256, fake + (1 << 36), 256, fake + (2 << 36), 1024,
                      in_type="bf16", out_type="bf16", layout_a="row", layout_b="col")
    assert dmu.dmu_gemm_kernel_name(a).startswith("mfma_64x128")
    dmu.dmu_phase_log(fake + (3 << 36), 127)
    try:
        assert dmu.library().dmu_gemm(ctypes.byref(a), None) == dmu.DMU_ERR_INVALID_ARG
        assert "128 phase records" in dmu.dmu_last_error()
    finally:
        dmu.dmu_phase_log(None, 0)


def test_mfma_ceiling_argument_errors():
    """The ceiling microbenchmark rejects bad counts, misaligned stamps and types without a kernel,
    before any HIP call."""
    lib = dmu.library()
    assert lib.dmu_mfma_ceiling(dmu.DMU_BF16, 0, 256, None, None) == dmu.DMU_ERR_INVALID_ARG
    assert lib.dmu_mfma_ceiling(dmu.DMU_BF16, 128, 0, None, None) == dmu.DMU_ERR_INVALID_ARG
    assert lib.dmu_mfma_ceiling(dmu.DMU_BF16, 128, 256, ctypes.c_void_p((1 << 40) + 4), None) == \
        dmu.DMU_ERR_INVALID_ARG
    assert lib.dmu_mfma_ceiling(dmu.DMU_F32, 128, 256, None, None) == dmu.DMU_ERR_UNSUPPORTED
    assert "no ceiling kernel" in dmu.dmu_last_error()
