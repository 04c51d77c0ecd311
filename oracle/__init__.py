"""CPU oracle for the GGUF block-quantized matmul -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library in
``gguf_block_quant_qmm_amd`` and its binding) never imports, links or runs it,
and the oracle shares no code with that path.

The arithmetic lives in ``oracle.c`` (plain C, f64 accumulation); this module
only compiles it with gcc and marshals numpy arrays through ctypes.  See the
header of ``oracle.c`` for what is computed and which page passage each part
follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# GGUF type ids, as the oracle's C source numbers them.
Q4_0, Q4_1, Q8_0, Q4_K, Q5_K, Q6_K = 2, 3, 8, 12, 13, 14
NAMES = {Q4_0: "Q4_0", Q4_1: "Q4_1", Q8_0: "Q8_0", Q4_K: "Q4_K", Q5_K: "Q5_K", Q6_K: "Q6_K"}
BY_NAME = {v: k for k, v in NAMES.items()}

_lib = None


def build(force: bool = True, extra_flags: list[str] | None = None, out: str | None = None) -> str:
    """Compile oracle.c into a shared library with gcc (-O2, no fast-math)."""
    out = out or _LIB
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(_SRC):
        return out
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", _SRC, "-o", out + ".tmp", "-lm"]
    if extra_flags:
        cmd[1:1] = list(extra_flags)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _bind(lib):
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_block_elems.argtypes = [ctypes.c_int]
    lib.oracle_block_bytes.argtypes = [ctypes.c_int]
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_double.restype = ctypes.c_double
    lib.oracle_dequant.argtypes = [ctypes.c_int, vp, i64, i64, vp]
    lib.oracle_matmul_rows.argtypes = [ctypes.c_int, vp, i64, i64, i64, vp, i64, vp, vp, vp, vp]
    lib.oracle_matmul.argtypes = [ctypes.c_int, vp, i64, i64, i64, vp, vp, vp, vp]
    lib.oracle_silu.argtypes = [ctypes.c_double]
    lib.oracle_silu.restype = ctypes.c_double
    lib.oracle_swiglu_rows.argtypes = [ctypes.c_int, vp, vp, i64, i64, i64, vp, i64, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_argmax.argtypes = [ctypes.c_int, vp, i64, i64, vp, vp, vp, vp]
    lib.oracle_float_to_half.argtypes = [ctypes.c_float]
    lib.oracle_float_to_half.restype = ctypes.c_uint16
    lib.oracle_quantize_q8_0.argtypes = [vp, i64, i64, vp, vp]
    lib.oracle_matmul_q8act_rows.argtypes = [ctypes.c_int, vp, i64, i64, i64, vp, vp, i64, vp, vp, vp, vp, vp]
    return lib


def load_variant(path: str):
    """Load a separately compiled build of oracle.c (used by the mutation test)."""
    return _bind(ctypes.CDLL(path))


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def block_elems(dtype: int, L=None) -> int:
    return (L or lib()).oracle_block_elems(dtype)


def block_bytes(dtype: int, L=None) -> int:
    return (L or lib()).oracle_block_bytes(dtype)


def blob_bytes(dtype: int, M: int, K: int, L=None) -> int:
    bs = block_elems(dtype, L)
    if bs == 0:
        raise ValueError(f"unknown dtype {dtype}")
    return M * (K // bs) * block_bytes(dtype, L)


def half_to_double(h: int, L=None) -> float:
    return (L or lib()).oracle_half_to_double(h)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def dequant(dtype: int, blob: np.ndarray, M: int, K: int, L=None) -> np.ndarray:
    """W[M][K] in f64."""
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    if blob.size < blob_bytes(dtype, M, K, L):
        raise ValueError("blob too small")
    W = np.empty((M, K), dtype=np.float64)
    _check((L or lib()).oracle_dequant(dtype, _ptr(blob), M, K, _ptr(W)), "dequant")
    return W


def matmul(dtype: int, blob: np.ndarray, M: int, K: int, X: np.ndarray, rows=None, L=None):
    """Y[N][R] f32, Y64[N][R] f64 and S[N][R] f64 for rows R (default: all M).

    X is f32 [N][K] (a 1-D x is treated as N=1).
    """
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    X = np.ascontiguousarray(X, dtype=np.float32)
    if X.ndim == 1:
        X = X[None, :]
    N = X.shape[0]
    if X.shape[1] != K:
        raise ValueError("X has the wrong K")
    if blob.size < blob_bytes(dtype, M, K, L):
        raise ValueError("blob too small")
    if rows is None:
        nrows, rows_p, rows_arr = M, None, None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        nrows, rows_p = rows_arr.size, _ptr(rows_arr)
    Y = np.empty((N, nrows), dtype=np.float32)
    Y64 = np.empty((N, nrows), dtype=np.float64)
    S = np.empty((N, nrows), dtype=np.float64)
    rc = (L or lib()).oracle_matmul_rows(dtype, _ptr(blob), M, K, N, _ptr(X), nrows, rows_p,
                                         _ptr(Y), _ptr(Y64), _ptr(S))
    _check(rc, "matmul")
    return Y, Y64, S


def silu(v: float, L=None) -> float:
    """v / (1 + e^-v) in f64 (oracle.c, oracle_silu)."""
    return (L or lib()).oracle_silu(float(v))


def swiglu(dtype: int, gate: np.ndarray, up: np.ndarray, M: int, K: int, X: np.ndarray, rows=None, L=None):
    """The gate/up projection with SwiGLU: out = silu(W_gate x) * (W_up x).

    Returns a dict of [N][R] arrays: ``out`` (f32), ``out64`` (f64), ``g`` and
    ``u`` (the f64 projections) and ``sg``, ``su`` (their sums of |w x|).
    """
    gate = np.ascontiguousarray(gate, dtype=np.uint8)
    up = np.ascontiguousarray(up, dtype=np.uint8)
    X = np.ascontiguousarray(X, dtype=np.float32)
    if X.ndim == 1:
        X = X[None, :]
    N = X.shape[0]
    if X.shape[1] != K:
        raise ValueError("X has the wrong K")
    nb = blob_bytes(dtype, M, K, L)
    if gate.size < nb or up.size < nb:
        raise ValueError("blob too small")
    if rows is None:
        nrows, rows_p = M, None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        nrows, rows_p = rows_arr.size, _ptr(rows_arr)
    r = {"out": np.empty((N, nrows), np.float32)}
    for k in ("out64", "g", "u", "sg", "su"):
        r[k] = np.empty((N, nrows), np.float64)
    rc = (L or lib()).oracle_swiglu_rows(dtype, _ptr(gate), _ptr(up), M, K, N, _ptr(X), nrows, rows_p,
                                         *(_ptr(r[k]) for k in ("out", "out64", "g", "u", "sg", "su")))
    _check(rc, "swiglu")
    return r


def argmax(dtype: int, blob: np.ndarray, M: int, K: int, x: np.ndarray, L=None):
    """(index, f64 maximum, its S) of the greedy argmax over y = W x (smallest index on ties)."""
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    if x.size != K:
        raise ValueError("x has the wrong K")
    if blob.size < blob_bytes(dtype, M, K, L):
        raise ValueError("blob too small")
    idx = np.zeros(1, np.int64)
    best = np.zeros(1, np.float64)
    bs = np.zeros(1, np.float64)
    _check((L or lib()).oracle_argmax(dtype, _ptr(blob), M, K, _ptr(x), _ptr(idx), _ptr(best), _ptr(bs)), "argmax")
    return int(idx[0]), float(best[0]), float(bs[0])


def num_threads() -> int:
    return lib().oracle_num_threads()


def float_to_half(v: float, L=None) -> int:
    """The binary16 bits of f32 v, rounded to nearest even."""
    return (L or lib()).oracle_float_to_half(float(np.float32(v)))


def quantize_q8_0(X: np.ndarray, L=None):
    """X f32 [N][K] (K % 32 == 0) -> (scales f32 [N][K/32], quants int8 [N][K])."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    if X.ndim == 1:
        X = X[None, :]
    N, K = X.shape
    scales = np.empty((N, K // 32), dtype=np.float32)
    quants = np.empty((N, K), dtype=np.int8)
    _check((L or lib()).oracle_quantize_q8_0(_ptr(X), N, K, _ptr(scales), _ptr(quants)), "quantize_q8_0")
    return scales, quants


def dequant_q8_0_act(scales: np.ndarray, quants: np.ndarray) -> np.ndarray:
    """Xq[n][k] = scales[n][k/32] * quants[n][k], exact in f64."""
    q = np.asarray(quants, dtype=np.float64)
    return q * np.repeat(np.asarray(scales, dtype=np.float64), 32, axis=-1)


def matmul_q8act(dtype: int, blob: np.ndarray, M: int, K: int, scales: np.ndarray, quants: np.ndarray,
                 rows=None, L=None):
    """Y[N][R] f32, Y64, S and Splus [N][R] f64 with Q8_0-quantized activations.

    scales f32 [N][K/32] and quants int8 [N][K] as quantize_q8_0 returns them;
    Splus is the rounding scale of the int8 kernels (S plus the weights'
    offset terms taken separately).
    """
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    quants = np.ascontiguousarray(quants, dtype=np.int8)
    if quants.ndim == 1:
        quants, scales = quants[None, :], scales[None, :]
    N = quants.shape[0]
    if quants.shape[1] != K or scales.shape != (N, K // 32):
        raise ValueError("activation codes or scales have the wrong shape")
    if blob.size < blob_bytes(dtype, M, K, L):
        raise ValueError("blob too small")
    if rows is None:
        nrows, rows_p = M, None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        nrows, rows_p = rows_arr.size, _ptr(rows_arr)
    Y = np.empty((N, nrows), dtype=np.float32)
    Y64, S, Sp = (np.empty((N, nrows), dtype=np.float64) for _ in range(3))
    rc = (L or lib()).oracle_matmul_q8act_rows(dtype, _ptr(blob), M, K, N, _ptr(scales), _ptr(quants), nrows,
                                               rows_p, _ptr(Y), _ptr(Y64), _ptr(S), _ptr(Sp))
    _check(rc, "matmul_q8act")
    return Y, Y64, S, Sp
