"""Host-side checks of the C ABI (CPU only: no kernel is launched).

The library must load, export every function include/qmm.h declares, report
the block geometry, and reject bad arguments with the documented status codes
before touching a device.
"""
import ctypes
import os
import re

import pytest

import gguf_block_quant_qmm_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qmm_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(q.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(q.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), f"libqmm.so does not export {name}"


def test_geometry():
    assert [q.block_elems(d) for d in (2, 3, 8, 12, 13, 14)] == [32, 32, 32, 256, 256, 256]
    assert [q.block_bytes(d) for d in (2, 3, 8, 12, 13, 14)] == [18, 20, 34, 144, 176, 210]
    assert q.block_elems(4) == 0 and q.block_bytes(99) == 0
    assert q.blob_bytes(q.QMM_Q4_1, 4096, 4096) == 4096 * 128 * 20
    # the tied Q6_K head of the 1B model on the pages: 2048 x 128256, ~205 MiB
    assert q.blob_bytes(q.QMM_Q6_K, 128256, 2048) == 215_470_080
    assert q.blob_bytes(q.QMM_Q4_0, 4096, 4096) == 4096 * 128 * 18
    assert q.blob_bytes(q.QMM_Q4_0, 4096, 4100) == 0     # K % 32
    assert q.blob_bytes(7, 4, 32) == 0                    # dtype


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define\s+(QMM_[A-Z0-9_]+)\s+\(?(-?\d+)\)?", text))
    for name, val in consts.items():
        assert getattr(q, name) == int(val), name


def test_strerror_is_total():
    for code in range(-8, 2):
        assert isinstance(q.strerror(code), str) and q.strerror(code)


A16 = 0x7F0000000000  # a 16-byte aligned fake device address: never dereferenced


@pytest.mark.parametrize("args,code", [
    ((A16, 5, 8, 32, A16, A16), q.QMM_ERR_DTYPE),
    ((A16, 2, 0, 32, A16, A16), q.QMM_ERR_SHAPE),
    ((A16, 2, 8, 0, A16, A16), q.QMM_ERR_SHAPE),
    ((A16, 2, 8, 48, A16, A16), q.QMM_ERR_SHAPE),
    ((A16, 12, 8, 128, A16, A16), q.QMM_ERR_SHAPE),
    ((0, 2, 8, 64, A16, A16), q.QMM_ERR_NULL),
    ((A16, 2, 8, 64, 0, A16), q.QMM_ERR_NULL),
    ((A16, 2, 8, 64, A16, 0), q.QMM_ERR_NULL),
    ((A16 + 2, 2, 8, 64, A16, A16), q.QMM_ERR_ALIGN),
    ((A16, 2, 8, 64, A16 + 4, A16), q.QMM_ERR_ALIGN),
    ((A16, 2, 8, 64, A16, A16 + 2), q.QMM_ERR_ALIGN),
])
def test_gemv_rejects(args, code):
    assert q.lib().qmm_gemv(*args, None) == code


@pytest.mark.parametrize("args,code", [
    ((A16, 2, 8, 64, 0, A16, A16), q.QMM_ERR_SHAPE),
    ((A16, 2, 8, 64, -3, A16, A16), q.QMM_ERR_SHAPE),
    ((A16, 14, 8, 300, 4, A16, A16), q.QMM_ERR_SHAPE),
    ((A16, 1, 8, 64, 4, A16, A16), q.QMM_ERR_DTYPE),
    ((A16, 8, 8, 64, 4, 0, A16), q.QMM_ERR_NULL),
    ((A16, 8, 8, 64, 4, A16 + 8, A16), q.QMM_ERR_ALIGN),
])
def test_gemm_rejects(args, code):
    assert q.lib().qmm_gemm(*args, None) == code


def test_gemm_path_selection():
    # below the crossover every token gets the GEMV's f32 arithmetic
    assert q.gemm_path(q.QMM_Q4_K, 14336, 4096, 1) == 0
    # K <= 4096: several tokens per weight read, crossover 5 (Q4_0, Q8_0, Q6_K) or 3 (Q4_K)
    # on tall matrices, later on short ones (few matrix-core tiles)
    assert q.gemm_path(q.QMM_Q4_K, 14336, 4096, 2) == 0
    assert q.gemm_path(q.QMM_Q4_K, 14336, 4096, 3) == 1
    assert q.gemm_path(q.QMM_Q4_K, 4096, 4096, 4) == 0
    assert q.gemm_path(q.QMM_Q4_K, 4096, 4096, 5) == 1
    for dt in (q.QMM_Q4_0, q.QMM_Q8_0, q.QMM_Q6_K):
        assert q.gemm_path(dt, 14336, 4096, 4) == 0
        assert q.gemm_path(dt, 14336, 4096, 5) == 1
    for dt in (q.QMM_Q4_0, q.QMM_Q8_0):
        assert q.gemm_path(dt, 4096, 4096, 4) == 0
        assert q.gemm_path(dt, 4096, 4096, 5) == 1
    assert q.gemm_path(q.QMM_Q6_K, 4096, 4096, 7) == 0
    assert q.gemm_path(q.QMM_Q6_K, 4096, 4096, 8) == 1
    assert q.gemm_path(q.QMM_Q4_0, 2048, 4096, 6) == 0
    assert q.gemm_path(q.QMM_Q4_0, 2048, 4096, 7) == 1
    assert q.gemm_path(q.QMM_Q8_0, 2048, 4096, 7) == 0
    assert q.gemm_path(q.QMM_Q8_0, 2048, 4096, 8) == 1
    assert q.gemm_path(q.QMM_Q6_K, 128256, 4096, 4) == 0
    # K > 4096: one GEMV launch per token, crossover 3 (Q4_0, Q6_K) or 2 (Q8_0, Q4_K)
    assert q.gemm_path(q.QMM_Q4_0, 4096, 14336, 2) == 0
    assert q.gemm_path(q.QMM_Q4_0, 4096, 14336, 3) == 1
    assert q.gemm_path(q.QMM_Q8_0, 4096, 8192, 2) == 1
    assert q.gemm_path(q.QMM_Q6_K, 4096, 8192, 2) == 0
    assert q.gemm_path(q.QMM_Q4_1, 4096, 4096, 4) == 0
    assert q.gemm_path(q.QMM_Q4_1, 14336, 4096, 3) == 0   # tall Q4_1: matrix cores from N = 4
    assert q.gemm_path(q.QMM_Q4_1, 14336, 4096, 4) == 1
    assert q.gemm_path(q.QMM_Q4_1, 4096, 4096, 5) == 1
    assert q.gemm_path(q.QMM_Q4_1, 4096, 8192, 2) == 1
    assert q.gemm_path(q.QMM_Q5_K, 4096, 4096, 2) == 0
    assert q.gemm_path(q.QMM_Q5_K, 4096, 4096, 3) == 1
    assert q.gemm_path(q.QMM_Q4_K, 14336, 4096, 512) == 1
    assert q.gemm_path(q.QMM_Q4_K, 14336, 100, 512) == q.QMM_ERR_SHAPE
    assert q.tolerance(q.QMM_Q4_0, 4096, 4096, 1) == 1e-5


def test_valid_call_without_gpu_reports_device(monkeypatch):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    assert q.lib().qmm_gemv(A16, 2, 8, 64, A16, A16, None) == q.QMM_ERR_DEVICE


def _concat(n, blobs, Ms, dtype, K, x, ys):
    def arr(ct, v):
        return (ct * len(v))(*v) if v is not None else None
    return q.lib().qmm_gemv_concat(n, arr(ctypes.c_void_p, blobs), arr(ctypes.c_int64, Ms), dtype, K, x,
                                   arr(ctypes.c_void_p, ys), None)


@pytest.mark.parametrize("n,blobs,Ms,dtype,K,x,ys,code", [
    (0, [A16], [8], 2, 64, A16, [A16], q.QMM_ERR_SHAPE),
    (5, [A16] * 5, [8] * 5, 2, 64, A16, [A16] * 5, q.QMM_ERR_SHAPE),
    (2, [A16, A16], [8, 0], 2, 64, A16, [A16, A16], q.QMM_ERR_SHAPE),
    (2, [A16, A16], [8, 8], 2, 48, A16, [A16, A16], q.QMM_ERR_SHAPE),
    (2, [A16, A16], [8, 8], 4, 64, A16, [A16, A16], q.QMM_ERR_DTYPE),
    (2, None, [8, 8], 2, 64, A16, [A16, A16], q.QMM_ERR_NULL),
    (2, [A16, A16], None, 2, 64, A16, [A16, A16], q.QMM_ERR_NULL),
    (2, [A16, A16], [8, 8], 2, 64, A16, None, q.QMM_ERR_NULL),
    (2, [A16, 0], [8, 8], 2, 64, A16, [A16, A16], q.QMM_ERR_NULL),
    (2, [A16, A16], [8, 8], 2, 64, 0, [A16, A16], q.QMM_ERR_NULL),
    (2, [A16, A16], [8, 8], 2, 64, A16, [A16, 0], q.QMM_ERR_NULL),
    (2, [A16, A16 + 8], [8, 8], 2, 64, A16, [A16, A16], q.QMM_ERR_ALIGN),
    (2, [A16, A16], [8, 8], 2, 64, A16 + 4, [A16, A16], q.QMM_ERR_ALIGN),
    (2, [A16, A16], [8, 8], 2, 64, A16, [A16, A16 + 1], q.QMM_ERR_ALIGN),
])
def test_gemv_concat_rejects(n, blobs, Ms, dtype, K, x, ys, code):
    assert _concat(n, blobs, Ms, dtype, K, x, ys) == code


@pytest.mark.parametrize("args,code", [
    ((A16, A16, 5, 8, 64, A16, A16), q.QMM_ERR_DTYPE),
    ((A16, A16, 2, 0, 64, A16, A16), q.QMM_ERR_SHAPE),
    ((A16, A16, 2, 8, 96, A16, A16), q.QMM_ERR_SHAPE),       # odd number of Q4_0 blocks
    ((A16, A16, 14, 8, 256, A16, A16), q.QMM_ERR_SHAPE),     # odd number of Q6_K super-blocks
    ((A16, A16, 12, 8, 16640, A16, A16), q.QMM_ERR_SHAPE),   # K > 16384
    ((0, A16, 2, 8, 64, A16, A16), q.QMM_ERR_NULL),
    ((A16, 0, 2, 8, 64, A16, A16), q.QMM_ERR_NULL),
    ((A16, A16, 2, 8, 64, 0, A16), q.QMM_ERR_NULL),
    ((A16, A16, 2, 8, 64, A16, 0), q.QMM_ERR_NULL),
    ((A16, A16 + 2, 2, 8, 64, A16, A16), q.QMM_ERR_ALIGN),
    ((A16, A16, 2, 8, 64, A16 + 8, A16), q.QMM_ERR_ALIGN),
    ((A16, A16, 2, 8, 64, A16, A16 + 2), q.QMM_ERR_ALIGN),
])
def test_gemv_swiglu_rejects(args, code):
    assert q.lib().qmm_gemv_swiglu(*args, None) == code


def test_fused_calls_without_gpu_report_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    assert _concat(2, [A16, A16], [8, 8], 2, 64, A16, [A16, A16]) == q.QMM_ERR_DEVICE
    assert q.lib().qmm_gemv_swiglu(A16, A16, 2, 8, 64, A16, A16, None) == q.QMM_ERR_DEVICE


@pytest.mark.parametrize("args,code", [
    ((A16, 5, 8, 64, A16, A16, A16, A16), q.QMM_ERR_DTYPE),
    ((A16, 2, 0, 64, A16, A16, A16, A16), q.QMM_ERR_SHAPE),
    ((A16, 2, 8, 96, A16, A16, A16, A16), q.QMM_ERR_SHAPE),        # odd number of Q4_0 blocks
    ((A16, 12, 8, 16640, A16, A16, A16, A16), q.QMM_ERR_SHAPE),    # K > 16384
    ((A16, 2, 1 << 31, 64, A16, A16, A16, A16), q.QMM_ERR_SHAPE),  # M beyond int32
    ((0, 2, 8, 64, A16, A16, A16, A16), q.QMM_ERR_NULL),
    ((A16, 2, 8, 64, 0, A16, A16, A16), q.QMM_ERR_NULL),
    ((A16, 2, 8, 64, A16, 0, A16, A16), q.QMM_ERR_NULL),
    ((A16, 2, 8, 64, A16, A16, 0, A16), q.QMM_ERR_NULL),
    ((A16, 2, 8, 64, A16, A16 + 8, A16, A16), q.QMM_ERR_ALIGN),
    ((A16, 2, 8, 64, A16, A16, A16 + 4, A16), q.QMM_ERR_ALIGN),
    ((A16, 2, 8, 64, A16, A16, A16, A16 + 2), q.QMM_ERR_ALIGN),
])
def test_gemv_argmax_rejects(args, code):
    assert q.lib().qmm_gemv_argmax(*args, None) == code


def test_argmax_without_value_and_gpu_reports_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    assert q.lib().qmm_gemv_argmax(A16, 2, 8, 64, A16, A16, A16, None, None) == q.QMM_ERR_DEVICE


@pytest.mark.parametrize("args,code", [
    ((A16, A16, 5, 8, 1024, 4, A16, A16), q.QMM_ERR_DTYPE),
    ((A16, A16, 2, 8, 1024, 0, A16, A16), q.QMM_ERR_SHAPE),
    ((A16, A16, 12, 8, 16640, 1, A16, A16), q.QMM_ERR_SHAPE),   # f32 path: K > 16384
    ((A16, A16, 2, 8, 96, 2, A16, A16), q.QMM_ERR_SHAPE),       # f32 path: odd Q4_0 block count
    ((A16, A16, 2, 8, 1088, 64, A16, A16), q.QMM_ERR_SHAPE),    # matrix cores: K not a multiple of 256
    ((A16, A16, 14, 8, 768, 64, A16, A16), q.QMM_ERR_SHAPE),    # Q6_K: odd super-block count
    ((0, A16, 2, 8, 1024, 64, A16, A16), q.QMM_ERR_NULL),
    ((A16, 0, 2, 8, 1024, 64, A16, A16), q.QMM_ERR_NULL),
    ((A16, A16, 2, 8, 1024, 64, 0, A16), q.QMM_ERR_NULL),
    ((A16, A16, 2, 8, 1024, 64, A16, 0), q.QMM_ERR_NULL),
    ((A16, A16 + 4, 2, 8, 1024, 64, A16, A16), q.QMM_ERR_ALIGN),
    ((A16, A16, 2, 8, 1024, 64, A16 + 8, A16), q.QMM_ERR_ALIGN),
    ((A16, A16, 2, 8, 1024, 64, A16, A16 + 1), q.QMM_ERR_ALIGN),
])
def test_gemm_swiglu_rejects(args, code):
    assert q.lib().qmm_gemm_swiglu(*args, None) == code


def test_gemm_swiglu_without_gpu_reports_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    assert q.lib().qmm_gemm_swiglu(A16, A16, 12, 8, 1024, 64, A16, A16, None) == q.QMM_ERR_DEVICE
    assert q.lib().qmm_gemm_swiglu(A16, A16, 2, 8, 1024, 2, A16, A16, None) == q.QMM_ERR_DEVICE


@pytest.mark.parametrize("args,code", [
    ((A16, 0, 64, A16, A16), q.QMM_ERR_SHAPE),
    ((A16, 2, 0, A16, A16), q.QMM_ERR_SHAPE),
    ((A16, 2, 48, A16, A16), q.QMM_ERR_SHAPE),          # K % 32
    ((0, 2, 64, A16, A16), q.QMM_ERR_NULL),
    ((A16, 2, 64, 0, A16), q.QMM_ERR_NULL),
    ((A16, 2, 64, A16, 0), q.QMM_ERR_NULL),
    ((A16 + 4, 2, 64, A16, A16), q.QMM_ERR_ALIGN),
    ((A16, 2, 64, A16 + 8, A16), q.QMM_ERR_ALIGN),
    ((A16, 2, 64, A16, A16 + 4), q.QMM_ERR_ALIGN),
])
def test_quantize_q8_0_rejects(args, code):
    assert q.lib().qmm_quantize_q8_0(*args, None) == code


@pytest.mark.parametrize("args,code", [
    ((A16, 5, 8, 64, 1, A16, A16, A16), q.QMM_ERR_DTYPE),
    ((A16, 2, 8, 64, 0, A16, A16, A16), q.QMM_ERR_SHAPE),
    ((A16, 12, 8, 128, 1, A16, A16, A16), q.QMM_ERR_SHAPE),
    ((A16, 2, 0, 64, 1, A16, A16, A16), q.QMM_ERR_SHAPE),
    ((0, 2, 8, 64, 1, A16, A16, A16), q.QMM_ERR_NULL),
    ((A16, 2, 8, 64, 1, 0, A16, A16), q.QMM_ERR_NULL),
    ((A16, 2, 8, 64, 1, A16, 0, A16), q.QMM_ERR_NULL),
    ((A16, 2, 8, 64, 1, A16, A16, 0), q.QMM_ERR_NULL),
    ((A16 + 2, 2, 8, 64, 1, A16, A16, A16), q.QMM_ERR_ALIGN),
    ((A16, 2, 8, 64, 1, A16 + 8, A16, A16), q.QMM_ERR_ALIGN),
    ((A16, 2, 8, 64, 1, A16, A16 + 4, A16), q.QMM_ERR_ALIGN),
    ((A16, 2, 8, 64, 1, A16, A16, A16 + 2), q.QMM_ERR_ALIGN),
])
def test_gemm_q8act_rejects(args, code):
    assert q.lib().qmm_gemm_q8act(*args, None) == code


def test_q8act_calls_without_gpu_report_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    assert q.lib().qmm_quantize_q8_0(A16, 2, 64, A16, A16, None) == q.QMM_ERR_DEVICE
    assert q.lib().qmm_gemm_q8act(A16, 14, 8, 256, 3, A16, A16, A16, None) == q.QMM_ERR_DEVICE


@pytest.mark.parametrize("args,code", [
    ((A16, 5, 8, 64, A16, A16), q.QMM_ERR_DTYPE),
    ((A16, 2, 8, 96, A16, A16), q.QMM_ERR_SHAPE),      # odd Q4_0 block count: no one-launch kernel
    ((A16, 12, 8, 16640, A16, A16), q.QMM_ERR_SHAPE),  # K > 16384
    ((A16, 2, 0, 64, A16, A16), q.QMM_ERR_SHAPE),
    ((0, 2, 8, 64, A16, A16), q.QMM_ERR_NULL),
    ((A16, 2, 8, 64, 0, A16), q.QMM_ERR_NULL),
    ((A16 + 2, 2, 8, 64, A16, A16), q.QMM_ERR_ALIGN),
    ((A16, 2, 8, 64, A16 + 4, A16), q.QMM_ERR_ALIGN),
    ((A16, 2, 8, 64, A16, A16 + 2), q.QMM_ERR_ALIGN),
])
def test_gemv_q8act_rejects(args, code):
    assert q.lib().qmm_gemv_q8act(*args, None) == code
    # the SwiGLU form takes the same checks with the blob given twice
    a = (args[0], args[0]) + args[1:]
    assert q.lib().qmm_gemv_swiglu_q8act(*a, None) == code


def test_gemv_concat_q8act_rejects():
    arr = lambda ct, v: (ct * len(v))(*v)
    L = q.lib()
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    assert L.qmm_gemv_concat_q8act(0, arr(vp, [A16]), arr(i64, [8]), 2, 64, A16, arr(vp, [A16]), None) == q.QMM_ERR_SHAPE
    assert L.qmm_gemv_concat_q8act(5, arr(vp, [A16] * 5), arr(i64, [8] * 5), 2, 64, A16, arr(vp, [A16] * 5),
                                   None) == q.QMM_ERR_SHAPE
    assert L.qmm_gemv_concat_q8act(2, arr(vp, [A16, 0]), arr(i64, [8, 8]), 2, 64, A16, arr(vp, [A16, A16]),
                                   None) == q.QMM_ERR_NULL
    assert L.qmm_gemv_concat_q8act(2, arr(vp, [A16, A16]), arr(i64, [8, 8]), 2, 96, A16, arr(vp, [A16, A16]),
                                   None) == q.QMM_ERR_SHAPE
    assert L.qmm_gemv_concat_q8act(1, arr(vp, [A16]), arr(i64, [8]), 2, 64, A16 + 4, arr(vp, [A16]),
                                   None) == q.QMM_ERR_ALIGN


def test_one_launch_q8act_without_gpu_reports_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    arr = lambda ct, v: (ct * len(v))(*v)
    L = q.lib()
    assert L.qmm_gemv_q8act(A16, 14, 8, 4096, A16, A16, None) == q.QMM_ERR_DEVICE
    assert L.qmm_gemv_swiglu_q8act(A16, A16, 2, 8, 4096, A16, A16, None) == q.QMM_ERR_DEVICE
    assert L.qmm_gemv_concat_q8act(2, arr(ctypes.c_void_p, [A16, A16]), arr(ctypes.c_int64, [8, 9]), 2, 4096, A16,
                                   arr(ctypes.c_void_p, [A16, A16]), None) == q.QMM_ERR_DEVICE


def test_oversized_products_are_rejected():
    # each size within 2^40, but a product of two beyond 2^56: no launch, no wrap-around
    big = 1 << 39
    assert q.lib().qmm_gemm(A16, 2, big, big, 1, A16, A16, None) == q.QMM_ERR_SHAPE
    assert q.lib().qmm_gemm(A16, 2, 8, big, big, A16, A16, None) == q.QMM_ERR_SHAPE
    assert q.lib().qmm_gemm(A16, 2, big, 64, big, A16, A16, None) == q.QMM_ERR_SHAPE
    assert q.lib().qmm_gemm_q8act(A16, 2, 8, big, big, A16, A16, A16, None) == q.QMM_ERR_SHAPE
    assert q.lib().qmm_quantize_q8_0(A16, big, big, A16, A16, None) == q.QMM_ERR_SHAPE
    assert q.blob_bytes(q.QMM_Q4_0, big, big) == 0


@pytest.mark.parametrize("args,code", [
    ((A16, 5, 8, 64, A16, A16, A16, 0), q.QMM_ERR_DTYPE),
    ((A16, 2, 8, 96, A16, A16, A16, 0), q.QMM_ERR_SHAPE),
    ((A16, 2, 1 << 31, 64, A16, A16, A16, 0), q.QMM_ERR_SHAPE),   # rows beyond int32
    ((A16, 2, 8, 64, A16, 0, A16, 0), q.QMM_ERR_NULL),
    ((A16, 2, 8, 64, A16, A16, 0, 0), q.QMM_ERR_NULL),
    ((A16, 2, 8, 64, A16 + 4, A16, A16, 0), q.QMM_ERR_ALIGN),
    ((A16, 2, 8, 64, A16, A16 + 8, A16, 0), q.QMM_ERR_ALIGN),
    ((A16, 2, 8, 64, A16, A16, A16 + 4, 0), q.QMM_ERR_ALIGN),
    ((A16, 2, 8, 64, A16, A16, A16, A16 + 2), q.QMM_ERR_ALIGN),
])
def test_gemv_argmax_q8act_rejects(args, code):
    assert q.lib().qmm_gemv_argmax_q8act(*args, None) == code


def test_argmax_q8act_without_gpu_reports_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    assert q.lib().qmm_gemv_argmax_q8act(A16, 14, 8, 4096, A16, A16, A16, None, None) == q.QMM_ERR_DEVICE


def test_library_reads_no_tuning_environment():
    """The shipped library takes no lever from the environment: a caller's
    environment cannot move a call to another kernel or tolerance class."""
    import subprocess
    import sys
    code = ("import gguf_block_quant_qmm_amd as q; "
            "print(q.gemm_path(12, 14336, 4096, 1), q.gemm_path(12, 14336, 4096, 512), "
            "q.gemm_kernel(12, 14336, 4096, 512), q.gemm_kernel(2, 300, 96, 40), "
            "q.q8act_kernel(12, 14336, 4096, 512), q.q8act_kernel(12, 4096, 4096, 40))")
    env = dict(os.environ, PYTHONPATH=ROOT)
    base = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, check=True).stdout
    env.update(QMM_GEMM_MFMA_FROM_N="1", QMM_GEMM_KERNEL="0", QMM_SWIGLU_KERNEL="2", QMM_GEMV_WAVES_PER_CU="3",
               QMM_Q8_MFMA_FROM_N="1000")
    lev = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, check=True).stdout
    assert base == lev and base.split()[:2] == ["0", "1"] and base.split()[4:] == ["1", "0"]


def test_q8act_path_reports_each_path():
    """The int8 matrix cores take large grids from N = 32; few tokens, small grids, Q6_K and
    the dtypes or K the int8 kernel does not take stay on the token groups."""
    assert q.q8act_kernel(q.QMM_Q4_K, 14336, 4096, 512) == 1
    assert q.q8act_kernel(q.QMM_Q8_0, 14336, 4096, 32) == 1
    assert q.q8act_kernel(q.QMM_Q4_0, 14336, 4096, 16) == 0
    assert q.q8act_kernel(q.QMM_Q4_0, 4096, 4096, 40) == 0
    assert q.q8act_kernel(q.QMM_Q6_K, 14336, 4096, 512) == 0
    assert q.q8act_kernel(q.QMM_Q4_1, 14336, 4096, 512) == 0
    assert q.q8act_kernel(q.QMM_Q8_0, 14336, 16416, 512) == 0  # K above 16384
    assert q.q8act_kernel(q.QMM_Q4_K, 14336, 4096, 0) == q.QMM_ERR_SHAPE


def test_gemm_kernel_reports_each_path():
    assert q.gemm_kernel(q.QMM_Q4_K, 14336, 4096, 1) == q.QMM_KERNEL_GEMV
    assert q.gemm_kernel(q.QMM_Q4_0, 4096, 4096, 3) == q.QMM_KERNEL_GEMV_TOKENS
    assert 0 <= q.gemm_kernel(q.QMM_Q4_K, 14336, 4096, 512) < 100
    assert q.gemm_kernel(q.QMM_Q4_K, 14336, 100, 512) == q.QMM_ERR_SHAPE
    assert q.gemm_kernel(5, 14336, 4096, 512) == q.QMM_ERR_DTYPE


def test_repack_sizes_and_argument_checks():
    """qmm_repack / qmm_gemm_repacked: Q6_K only, 320 bytes per super-block; the
    checks that come before any device call."""
    L = q.lib()
    assert q.repack_bytes(q.QMM_Q6_K, 3, 512) == 3 * 2 * 320
    assert q.repack_bytes(q.QMM_Q6_K, 14336, 4096) == 14336 * 16 * 320
    assert q.repack_bytes(q.QMM_Q8_0, 3, 512) == 3 * 8 * 72
    assert q.repack_bytes(q.QMM_Q8_0, 3, 96) == 0  # K not a multiple of 256
    assert L.qmm_repack(A16, q.QMM_Q8_0, 3, 96, A16, None) == q.QMM_ERR_SHAPE
    for dt in (q.QMM_Q4_0, q.QMM_Q4_K, q.QMM_Q4_1, q.QMM_Q5_K, 5):
        assert q.repack_bytes(dt, 3, 512) == 0
        assert L.qmm_repack(A16, dt, 3, 512, A16, None) in (q.QMM_ERR_DTYPE,)
    assert q.repack_bytes(q.QMM_Q6_K, 3, 500) == 0
    assert L.qmm_repack(A16, q.QMM_Q6_K, 3, 500, A16, None) == q.QMM_ERR_SHAPE
    assert L.qmm_repack(None, q.QMM_Q6_K, 3, 512, A16, None) == q.QMM_ERR_NULL
    assert L.qmm_repack(A16, q.QMM_Q6_K, 3, 512, A16 + 4, None) == q.QMM_ERR_ALIGN
    assert L.qmm_gemm_repacked(A16, q.QMM_Q4_K, 3, 512, 4, A16, A16, None) == q.QMM_ERR_DTYPE
    assert L.qmm_gemm_repacked(A16, q.QMM_Q6_K, 3, 1 << 22, 4, A16, A16, None) == q.QMM_ERR_SHAPE
    assert L.qmm_gemm_repacked(A16, q.QMM_Q6_K, 3, 512, 4, A16 + 8, A16, None) == q.QMM_ERR_ALIGN
    assert L.qmm_gemm_repacked(A16, q.QMM_Q6_K, 3, 512, 4, A16, None, None) == q.QMM_ERR_NULL


def test_repacked_kernel_choice_matches_the_gguf_form():
    """With an even number of super-blocks per row the repacked GEMM runs the
    kernel qmm_gemm runs on the GGUF bytes (so the two give the same bits);
    with an odd number it still runs a register-B kernel."""
    for M, K, N in [(14336, 4096, 512), (4096, 4096, 512), (4096, 4096, 32), (14336, 4096, 32),
                    (4096, 4096, 128), (4096, 4096, 256), (128256, 4096, 9), (1000, 1536, 20)]:
        for dt in (q.QMM_Q6_K, q.QMM_Q8_0):
            assert q.gemm_repacked_kernel(dt, M, K, N) == q.gemm_kernel(dt, M, K, N)
    assert q.gemm_kernel(q.QMM_Q6_K, 300, 768, 40) == 0  # the LDS-tile kernel for odd block counts
    assert 0 < q.gemm_repacked_kernel(q.QMM_Q6_K, 300, 768, 40) < 100


def test_swiglu_kernel_reports_each_form():
    """The SwiGLU forms qmm_gemm_swiglu picks (tile ids of qmm_gemm.hip)."""
    dt = q.QMM_Q4_K
    assert q.swiglu_kernel(dt, 14336, 4096, 2) == q.QMM_KERNEL_GEMV
    assert q.swiglu_kernel(dt, 14336, 4096, 40) == 1
    assert q.swiglu_kernel(dt, 14336, 4096, 128) == 2
    assert q.swiglu_kernel(dt, 14336, 4096, 200) == 5   # the wavefront pair form, one round
    assert q.swiglu_kernel(dt, 14336, 4096, 384) == 2
    assert q.swiglu_kernel(dt, 14336, 4096, 512) == 5
    assert q.swiglu_kernel(dt, 4096, 4096, 512) == 2
    assert q.swiglu_kernel(dt, 14336, 100, 512) == q.QMM_ERR_SHAPE
    assert q.swiglu_kernel(5, 14336, 4096, 512) == q.QMM_ERR_DTYPE
