"""Python binding of libqmm, the GGUF block-quantized matmul for MI355X.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of include/qmm.h.  Tensors are PyTorch device
tensors (PyTorch supplies device memory and streams); the functions also
accept raw device addresses as ints.  If libqmm.so is missing the calls raise;
there is no CPU fallback.

    qmm_gemv(w, dtype, M, K, x, y, stream=None)      y[M] = W x
    qmm_gemm(w, dtype, M, K, N, X, Y, stream=None)   Y[N][M] = X W^T
    qmm_gemv_concat(ws, dtype, Ms, K, x, ys, stream=None)
                                                     ys[i] = W_i x, one launch
    qmm_gemv_swiglu(gate, up, dtype, M, K, x, out, stream=None)
                                                     out = silu(W_gate x) * (W_up x)
    qmm_gemv_argmax(w, dtype, M, K, x, work, index, value=None, stream=None)
                                                     index = argmax_m (W x)[m]
    qmm_gemv_argmax_noalloc(w, dtype, M, K, x, index, value=None, stream=None)
                                                     the same, scratch in a static
                                                     device array (no work buffer)
    qmm_gemm_swiglu(gate, up, dtype, M, K, N, X, out, stream=None)
                                                     out = silu(X Wg^T) * (X Wu^T)
    qmm_quantize_q8_0(X, N, K, scales, quants, stream=None)
                                                     X -> Q8_0 activation blocks
    qmm_gemm_q8act(w, dtype, M, K, N, scales, quants, Y, stream=None)
                                                     Y = Xq W^T (int8 activations)
    qmm_repack(w, dtype, M, K, packed, stream=None)  Q6_K / Q8_0 -> the GEMM's repacked layout
    qmm_gemm_repacked(packed, dtype, M, K, N, X, Y, stream=None)
                                                     Y[N][M] = X W^T from the repacked copy
    qmm_gemv_q8act / qmm_gemv_concat_q8act / qmm_gemv_swiglu_q8act /
    qmm_gemv_argmax_q8act                            the decode calls above with x
                                                     quantized inside the launch
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmm.so")

# dtype tags (GGUF type ids) and status codes, as in include/qmm.h
QMM_Q4_0, QMM_Q4_1, QMM_Q8_0, QMM_Q4_K, QMM_Q5_K, QMM_Q6_K = 2, 3, 8, 12, 13, 14
DTYPES = {"Q4_0": QMM_Q4_0, "Q4_1": QMM_Q4_1, "Q8_0": QMM_Q8_0, "Q4_K": QMM_Q4_K, "Q5_K": QMM_Q5_K,
          "Q6_K": QMM_Q6_K}
QMM_OK, QMM_ERR_NULL, QMM_ERR_DTYPE, QMM_ERR_SHAPE = 0, -1, -2, -3
QMM_ERR_ALIGN, QMM_ERR_DEVICE, QMM_ERR_LAUNCH, QMM_ERR_SCRATCH = -4, -5, -6, -7

QMM_GEMV_MAX_MATS = 4
QMM_ARGMAX_WORK_BYTES = 32768
QMM_NOALLOC_SCRATCH_BYTES = 32768
QMM_READ_PROBE_OUT_FLOATS = 4096

EXPORTS = ("qmm_gemv", "qmm_gemv_concat", "qmm_gemv_swiglu", "qmm_gemv_argmax", "qmm_gemv_argmax_noalloc", "qmm_gemm", "qmm_gemm_swiglu",
           "qmm_quantize_q8_0", "qmm_gemm_q8act", "qmm_gemv_q8act", "qmm_gemv_concat_q8act",
           "qmm_gemv_swiglu_q8act", "qmm_gemv_argmax_q8act", "qmm_repack_bytes", "qmm_repack", "qmm_gemm_repacked", "qmm_gemm_repacked_kernel",
           "qmm_gemm_path", "qmm_gemm_q8act_path", "qmm_gemm_kernel", "qmm_gemm_swiglu_kernel", "qmm_read_probe", "qmm_blob_bytes", "qmm_block_elems",
           "qmm_block_bytes", "qmm_strerror")

_lib = None


class QmmError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {strerror(code)} (status {code})")
        self.code = code


def lib():
    """The loaded libqmm.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m gguf_block_quant_qmm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.qmm_gemv.argtypes = [vp, ci, i64, i64, vp, vp, vp]
        L.qmm_gemv.restype = ci
        L.qmm_gemv_concat.argtypes = [ci, vp, vp, ci, i64, vp, vp, vp]
        L.qmm_gemv_concat.restype = ci
        L.qmm_gemv_swiglu.argtypes = [vp, vp, ci, i64, i64, vp, vp, vp]
        L.qmm_gemv_swiglu.restype = ci
        L.qmm_gemv_argmax.argtypes = [vp, ci, i64, i64, vp, vp, vp, vp, vp]
        L.qmm_gemv_argmax.restype = ci
        L.qmm_gemv_argmax_noalloc.argtypes = [vp, ci, i64, i64, vp, vp, vp, vp]
        L.qmm_gemv_argmax_noalloc.restype = ci
        L.qmm_gemm_swiglu.argtypes = [vp, vp, ci, i64, i64, i64, vp, vp, vp]
        L.qmm_gemm_swiglu.restype = ci
        L.qmm_gemm.argtypes = [vp, ci, i64, i64, i64, vp, vp, vp]
        L.qmm_gemm.restype = ci
        L.qmm_quantize_q8_0.argtypes = [vp, i64, i64, vp, vp, vp]
        L.qmm_quantize_q8_0.restype = ci
        L.qmm_gemm_q8act.argtypes = [vp, ci, i64, i64, i64, vp, vp, vp, vp]
        L.qmm_gemm_q8act.restype = ci
        L.qmm_gemv_q8act.argtypes = [vp, ci, i64, i64, vp, vp, vp]
        L.qmm_gemv_q8act.restype = ci
        L.qmm_gemv_concat_q8act.argtypes = [ci, vp, vp, ci, i64, vp, vp, vp]
        L.qmm_gemv_concat_q8act.restype = ci
        L.qmm_gemv_swiglu_q8act.argtypes = [vp, vp, ci, i64, i64, vp, vp, vp]
        L.qmm_gemv_swiglu_q8act.restype = ci
        L.qmm_gemv_argmax_q8act.argtypes = [vp, ci, i64, i64, vp, vp, vp, vp, vp]
        L.qmm_gemv_argmax_q8act.restype = ci
        L.qmm_repack_bytes.argtypes = [ci, i64, i64]
        L.qmm_repack_bytes.restype = i64
        L.qmm_repack.argtypes = [vp, ci, i64, i64, vp, vp]
        L.qmm_repack.restype = ci
        L.qmm_gemm_repacked.argtypes = [vp, ci, i64, i64, i64, vp, vp, vp]
        L.qmm_gemm_repacked.restype = ci
        L.qmm_gemm_repacked_kernel.argtypes = [ci, i64, i64, i64]
        L.qmm_gemm_repacked_kernel.restype = ci
        L.qmm_gemm_path.argtypes = [ci, i64, i64, i64]
        L.qmm_gemm_path.restype = ci
        L.qmm_gemm_q8act_path.argtypes = [ci, i64, i64, i64]
        L.qmm_gemm_q8act_path.restype = ci
        L.qmm_gemm_swiglu_kernel.argtypes = [ci, i64, i64, i64]
        L.qmm_gemm_swiglu_kernel.restype = ci
        L.qmm_gemm_kernel.argtypes = [ci, i64, i64, i64]
        L.qmm_gemm_kernel.restype = ci
        L.qmm_read_probe.argtypes = [vp, i64, vp, vp]
        L.qmm_read_probe.restype = ci
        L.qmm_blob_bytes.argtypes = [ci, i64, i64]
        L.qmm_blob_bytes.restype = i64
        L.qmm_block_elems.argtypes = [ci]
        L.qmm_block_bytes.argtypes = [ci]
        L.qmm_strerror.argtypes = [ci]
        L.qmm_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().qmm_strerror(code).decode()


def block_elems(dtype: int) -> int:
    return lib().qmm_block_elems(dtype)


def block_bytes(dtype: int) -> int:
    return lib().qmm_block_bytes(dtype)


def blob_bytes(dtype: int, M: int, K: int) -> int:
    return lib().qmm_blob_bytes(dtype, M, K)


def gemm_path(dtype: int, M: int, K: int, N: int) -> int:
    return lib().qmm_gemm_path(dtype, M, K, N)


QMM_KERNEL_GEMV, QMM_KERNEL_GEMV_TOKENS = 100, 101


def q8act_kernel(dtype: int, M: int, K: int, N: int) -> int:
    """0: qmm_gemm_q8act runs token groups (single-token bits); 1: the int8 matrix cores."""
    return lib().qmm_gemm_q8act_path(dtype, M, K, N)


def swiglu_kernel(dtype: int, M: int, K: int, N: int) -> int:
    """Form qmm_gemm_swiglu runs for these sizes (see include/qmm.h)."""
    return lib().qmm_gemm_swiglu_kernel(dtype, M, K, N)


def gemm_kernel(dtype: int, M: int, K: int, N: int) -> int:
    """Id of the kernel qmm_gemm runs for these sizes (see include/qmm.h)."""
    return lib().qmm_gemm_kernel(dtype, M, K, N)


def qmm_read_probe(buf, nbytes: int, out, stream=None) -> None:
    """A plain streaming read of nbytes of buf (diagnostic read ceiling)."""
    import torch
    rc = lib().qmm_read_probe(_addr(buf, nbytes, "buf"), nbytes,
                              _addr(out, 4 * QMM_READ_PROBE_OUT_FLOATS, "out", torch.float32), _stream(stream))
    if rc != QMM_OK:
        raise QmmError(rc, "qmm_read_probe")


def tolerance(dtype: int, M: int, K: int, N: int) -> float:
    """Relative tolerance (of sum |w x|) that the chosen path guarantees."""
    return 2e-3 if gemm_path(dtype, M, K, N) == 1 else 1e-5


def _addr(t, nbytes: int | None, what: str, torch_dtype=None) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if torch_dtype is not None and t.dtype != torch_dtype:
        raise ValueError(f"{what} must be {torch_dtype}, got {t.dtype}")
    if nbytes is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{what} holds {t.numel() * t.element_size()} bytes, needs {nbytes}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def qmm_gemv(w, dtype: int, M: int, K: int, x, y, stream=None) -> None:
    import torch
    nb = blob_bytes(dtype, M, K)
    rc = lib().qmm_gemv(_addr(w, nb or None, "w_blob"), dtype, M, K,
                        _addr(x, 4 * K, "x", torch.float32), _addr(y, 4 * M, "y", torch.float32),
                        _stream(stream))
    if rc != QMM_OK:
        raise QmmError(rc, "qmm_gemv")


def qmm_gemm(w, dtype: int, M: int, K: int, N: int, X, Y, stream=None) -> None:
    import torch
    nb = blob_bytes(dtype, M, K)
    rc = lib().qmm_gemm(_addr(w, nb or None, "w_blob"), dtype, M, K, N,
                        _addr(X, 4 * N * K, "X", torch.float32), _addr(Y, 4 * N * M, "Y", torch.float32),
                        _stream(stream))
    if rc != QMM_OK:
        raise QmmError(rc, "qmm_gemm")


def repack_bytes(dtype: int, M: int, K: int) -> int:
    return lib().qmm_repack_bytes(dtype, M, K)


def gemm_repacked_kernel(dtype: int, M: int, K: int, N: int) -> int:
    return lib().qmm_gemm_repacked_kernel(dtype, M, K, N)


def qmm_repack(w, dtype: int, M: int, K: int, packed, stream=None) -> None:
    rc = lib().qmm_repack(_addr(w, blob_bytes(dtype, M, K) or None, "w_blob"), dtype, M, K,
                          _addr(packed, repack_bytes(dtype, M, K) or None, "packed"), _stream(stream))
    if rc != QMM_OK:
        raise QmmError(rc, "qmm_repack")


def qmm_gemm_repacked(packed, dtype: int, M: int, K: int, N: int, X, Y, stream=None) -> None:
    import torch
    rc = lib().qmm_gemm_repacked(_addr(packed, repack_bytes(dtype, M, K) or None, "packed"), dtype, M, K, N,
                                 _addr(X, 4 * N * K, "X", torch.float32), _addr(Y, 4 * N * M, "Y", torch.float32),
                                 _stream(stream))
    if rc != QMM_OK:
        raise QmmError(rc, "qmm_gemm_repacked")


def qmm_gemv_concat(ws, dtype: int, Ms, K: int, x, ys, stream=None) -> None:
    import torch
    n = len(ws)
    if not (len(Ms) == n == len(ys)):
        raise ValueError("ws, Ms and ys need one entry per matrix")
    blobs = (ctypes.c_void_p * max(n, 1))(*[_addr(w, blob_bytes(dtype, M, K) or None, f"ws[{i}]")
                                            for i, (w, M) in enumerate(zip(ws, Ms))])
    rows = (ctypes.c_int64 * max(n, 1))(*[int(M) for M in Ms])
    outs = (ctypes.c_void_p * max(n, 1))(*[_addr(y, 4 * M, f"ys[{i}]", torch.float32)
                                           for i, (y, M) in enumerate(zip(ys, Ms))])
    rc = lib().qmm_gemv_concat(n, blobs, rows, dtype, K, _addr(x, 4 * K, "x", torch.float32), outs,
                               _stream(stream))
    if rc != QMM_OK:
        raise QmmError(rc, "qmm_gemv_concat")


def qmm_gemv_swiglu(gate, up, dtype: int, M: int, K: int, x, out, stream=None) -> None:
    import torch
    nb = blob_bytes(dtype, M, K) or None
    rc = lib().qmm_gemv_swiglu(_addr(gate, nb, "gate"), _addr(up, nb, "up"), dtype, M, K,
                               _addr(x, 4 * K, "x", torch.float32), _addr(out, 4 * M, "out", torch.float32),
                               _stream(stream))
    if rc != QMM_OK:
        raise QmmError(rc, "qmm_gemv_swiglu")


def qmm_gemv_argmax(w, dtype: int, M: int, K: int, x, work, index, value=None, stream=None) -> None:
    import torch
    rc = lib().qmm_gemv_argmax(_addr(w, blob_bytes(dtype, M, K) or None, "w_blob"), dtype, M, K,
                               _addr(x, 4 * K, "x", torch.float32), _addr(work, QMM_ARGMAX_WORK_BYTES, "work"),
                               _addr(index, 8, "index", torch.int64), _addr(value, 4, "value", torch.float32),
                               _stream(stream))
    if rc != QMM_OK:
        raise QmmError(rc, "qmm_gemv_argmax")


def qmm_gemv_argmax_noalloc(w, dtype: int, M: int, K: int, x, index, value=None, stream=None) -> None:
    import torch
    rc = lib().qmm_gemv_argmax_noalloc(_addr(w, blob_bytes(dtype, M, K) or None, "w_blob"), dtype, M, K,
                                       _addr(x, 4 * K, "x", torch.float32), _addr(index, 8, "index", torch.int64),
                                       _addr(value, 4, "value", torch.float32), _stream(stream))
    if rc != QMM_OK:
        raise QmmError(rc, "qmm_gemv_argmax_noalloc")


def qmm_gemm_swiglu(gate, up, dtype: int, M: int, K: int, N: int, X, out, stream=None) -> None:
    import torch
    nb = blob_bytes(dtype, M, K) or None
    rc = lib().qmm_gemm_swiglu(_addr(gate, nb, "gate"), _addr(up, nb, "up"), dtype, M, K, N,
                               _addr(X, 4 * N * K, "X", torch.float32), _addr(out, 4 * N * M, "out", torch.float32),
                               _stream(stream))
    if rc != QMM_OK:
        raise QmmError(rc, "qmm_gemm_swiglu")


def qmm_quantize_q8_0(X, N: int, K: int, scales, quants, stream=None) -> None:
    import torch
    nb = K // 32 if K > 0 else 0
    rc = lib().qmm_quantize_q8_0(_addr(X, 4 * N * K, "X", torch.float32), N, K,
                                 _addr(scales, 4 * N * nb, "scales", torch.float32),
                                 _addr(quants, N * K, "quants", torch.int8), _stream(stream))
    if rc != QMM_OK:
        raise QmmError(rc, "qmm_quantize_q8_0")


def qmm_gemm_q8act(w, dtype: int, M: int, K: int, N: int, scales, quants, Y, stream=None) -> None:
    import torch
    nb = blob_bytes(dtype, M, K)
    rc = lib().qmm_gemm_q8act(_addr(w, nb or None, "w_blob"), dtype, M, K, N,
                              _addr(scales, 4 * N * (K // 32), "scales", torch.float32),
                              _addr(quants, N * K, "quants", torch.int8), _addr(Y, 4 * N * M, "Y", torch.float32),
                              _stream(stream))
    if rc != QMM_OK:
        raise QmmError(rc, "qmm_gemm_q8act")


def qmm_gemv_q8act(w, dtype: int, M: int, K: int, x, y, stream=None) -> None:
    import torch
    nb = blob_bytes(dtype, M, K)
    rc = lib().qmm_gemv_q8act(_addr(w, nb or None, "w_blob"), dtype, M, K,
                              _addr(x, 4 * K, "x", torch.float32), _addr(y, 4 * M, "y", torch.float32),
                              _stream(stream))
    if rc != QMM_OK:
        raise QmmError(rc, "qmm_gemv_q8act")


def qmm_gemv_concat_q8act(ws, dtype: int, Ms, K: int, x, ys, stream=None) -> None:
    import torch
    n = len(ws)
    if not (len(Ms) == n == len(ys)):
        raise ValueError("ws, Ms and ys need one entry per matrix")
    blobs = (ctypes.c_void_p * max(n, 1))(*[_addr(w, blob_bytes(dtype, M, K) or None, f"ws[{i}]")
                                            for i, (w, M) in enumerate(zip(ws, Ms))])
    rows = (ctypes.c_int64 * max(n, 1))(*[int(M) for M in Ms])
    outs = (ctypes.c_void_p * max(n, 1))(*[_addr(y, 4 * M, f"ys[{i}]", torch.float32)
                                           for i, (y, M) in enumerate(zip(ys, Ms))])
    rc = lib().qmm_gemv_concat_q8act(n, blobs, rows, dtype, K, _addr(x, 4 * K, "x", torch.float32), outs,
                                     _stream(stream))
    if rc != QMM_OK:
        raise QmmError(rc, "qmm_gemv_concat_q8act")


def qmm_gemv_swiglu_q8act(gate, up, dtype: int, M: int, K: int, x, out, stream=None) -> None:
    import torch
    nb = blob_bytes(dtype, M, K) or None
    rc = lib().qmm_gemv_swiglu_q8act(_addr(gate, nb, "gate"), _addr(up, nb, "up"), dtype, M, K,
                                     _addr(x, 4 * K, "x", torch.float32), _addr(out, 4 * M, "out", torch.float32),
                                     _stream(stream))
    if rc != QMM_OK:
        raise QmmError(rc, "qmm_gemv_swiglu_q8act")


def qmm_gemv_argmax_q8act(w, dtype: int, M: int, K: int, x, work, index, value=None, stream=None) -> None:
    import torch
    rc = lib().qmm_gemv_argmax_q8act(_addr(w, blob_bytes(dtype, M, K) or None, "w_blob"), dtype, M, K,
                                     _addr(x, 4 * K, "x", torch.float32), _addr(work, QMM_ARGMAX_WORK_BYTES, "work"),
                                     _addr(index, 8, "index", torch.int64), _addr(value, 4, "value", torch.float32),
                                     _stream(stream))
    if rc != QMM_OK:
        raise QmmError(rc, "qmm_gemv_argmax_q8act")
