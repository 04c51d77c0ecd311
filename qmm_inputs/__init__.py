"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and
the bench.

This module only draws random numbers and lays them out as block bytes; it
holds none of the matmul's arithmetic (no dequantization, no dot products) and
imports neither the oracle nor the HIP library.

Distributions (the workload table the inputs stand in for):
  Q8_0: d ~ U[0.002, 0.02], q ~ U{-127..127}
  Q4_0: d ~ U[0.005, 0.05], 16 uniform nibble bytes
  Q4_1: d ~ U[0.005, 0.05], m = -d * U[6, 9] (a block minimum below zero, so
        the weights straddle zero as a quantized zero-mean row does), 16
        uniform nibble bytes
  Q4_K: d, dmin ~ U[5e-4, 2e-3], 12 uniform scale bytes (so every 6-bit
        sc/m is uniform on 0..63), 128 uniform nibble bytes
  Q5_K: as Q4_K, plus 32 uniform fifth-bit bytes (so q is uniform on 0..31)
  Q6_K: d ~ U[2e-4, 1e-3], uniform ql/qh bytes (so q is uniform on 0..63),
        int8 sub-scales ~ U{-64..63}
  activations: f32 ~ N(0, 1)
Every f16 scale is drawn in f32 and rounded to nearest-even f16; the stored
f16 is the truth.  No generator emits a subnormal, infinite or NaN scale.

Seeds: numpy PCG64 seeded with ``[0, workload_id, tensor_id]`` so that every
(workload, tensor) pair gets its own stream.
"""
from __future__ import annotations

import numpy as np

Q4_0, Q4_1, Q8_0, Q4_K, Q5_K, Q6_K = 2, 3, 8, 12, 13, 14
NAMES = {Q4_0: "Q4_0", Q4_1: "Q4_1", Q8_0: "Q8_0", Q4_K: "Q4_K", Q5_K: "Q5_K", Q6_K: "Q6_K"}
BY_NAME = {v: k for k, v in NAMES.items()}
# (weights per block, bytes per block) -- the GGUF block geometry.
GEOMETRY = {Q4_0: (32, 18), Q4_1: (32, 20), Q8_0: (32, 34), Q4_K: (256, 144), Q5_K: (256, 176),
            Q6_K: (256, 210)}


def rng_for(workload_id: int, tensor_id: int = 0) -> np.random.Generator:
    return np.random.default_rng([0, int(workload_id), int(tensor_id)])


def blob_bytes(dtype: int, M: int, K: int) -> int:
    bs, bb = GEOMETRY[dtype]
    return M * (K // bs) * bb


def _f16_bytes(vals_f32: np.ndarray) -> np.ndarray:
    """[n] f32 -> [n, 2] little-endian f16 bytes (round to nearest even)."""
    h = vals_f32.astype(np.float32).astype("<f2")
    return h.view(np.uint8).reshape(-1, 2)


def make_blob(dtype: int, M: int, K: int, rng: np.random.Generator, q8_full_range: bool = False) -> np.ndarray:
    """Random row-major blob of M rows x K weights, as a flat uint8 array.

    q8_full_range: Q8_0 codes drawn from the whole int8 range [-128, 127]
    (the format allows -128; the workload distribution stops at -127)."""
    bs, bb = GEOMETRY[dtype]
    if K % bs:
        raise ValueError(f"K={K} is not a multiple of {bs}")
    nblk = M * (K // bs)
    blk = np.empty((nblk, bb), dtype=np.uint8)
    if dtype == Q8_0:
        blk[:, 0:2] = _f16_bytes(rng.uniform(0.002, 0.02, nblk).astype(np.float32))
        lo = -128 if q8_full_range else -127
        blk[:, 2:34] = rng.integers(lo, 128, size=(nblk, 32), dtype=np.int8).view(np.uint8)
    elif dtype == Q4_0:
        blk[:, 0:2] = _f16_bytes(rng.uniform(0.005, 0.05, nblk).astype(np.float32))
        blk[:, 2:18] = rng.integers(0, 256, size=(nblk, 16), dtype=np.uint8)
    elif dtype == Q4_1:
        d = rng.uniform(0.005, 0.05, nblk).astype(np.float32)
        blk[:, 0:2] = _f16_bytes(d)
        blk[:, 2:4] = _f16_bytes((-d * rng.uniform(6.0, 9.0, nblk)).astype(np.float32))
        blk[:, 4:20] = rng.integers(0, 256, size=(nblk, 16), dtype=np.uint8)
    elif dtype == Q4_K:
        blk[:, 0:2] = _f16_bytes(rng.uniform(5e-4, 2e-3, nblk).astype(np.float32))
        blk[:, 2:4] = _f16_bytes(rng.uniform(5e-4, 2e-3, nblk).astype(np.float32))
        blk[:, 4:144] = rng.integers(0, 256, size=(nblk, 140), dtype=np.uint8)
    elif dtype == Q5_K:
        blk[:, 0:2] = _f16_bytes(rng.uniform(5e-4, 2e-3, nblk).astype(np.float32))
        blk[:, 2:4] = _f16_bytes(rng.uniform(5e-4, 2e-3, nblk).astype(np.float32))
        blk[:, 4:176] = rng.integers(0, 256, size=(nblk, 172), dtype=np.uint8)
    elif dtype == Q6_K:
        blk[:, 0:192] = rng.integers(0, 256, size=(nblk, 192), dtype=np.uint8)
        blk[:, 192:208] = rng.integers(-64, 64, size=(nblk, 16), dtype=np.int8).view(np.uint8)
        blk[:, 208:210] = _f16_bytes(rng.uniform(2e-4, 1e-3, nblk).astype(np.float32))
    else:
        raise ValueError(f"unknown dtype {dtype}")
    return blk.reshape(-1)


def make_x(N: int, K: int, rng: np.random.Generator) -> np.ndarray:
    """Activations X[N][K], f32 ~ N(0, 1)."""
    return rng.standard_normal((N, K), dtype=np.float32)


# The workloads: every configuration the parity tests and the bench use.
# id -> (label, dtype, M, K, N-list)
WORKLOADS = {
    1: ("q8_0 gemv 1024x1024", Q8_0, 1024, 1024, [1]),
    2: ("q4_0 gemv llama8b q_proj 4096x4096", Q4_0, 4096, 4096, [1]),
    3: ("q4_0 gemv llama8b gate/up 14336x4096", Q4_0, 14336, 4096, [1]),
    4: ("q4_0 gemv llama8b down 4096x14336", Q4_0, 4096, 14336, [1]),
    5: ("q6_k lm-head gemv 128256x4096", Q6_K, 128256, 4096, [1]),
    6: ("q4_k prefill gemm 14336x4096", Q4_K, 14336, 4096, [32, 512]),
    7: ("sweep q8_0 4096x4096", Q8_0, 4096, 4096, [1, 2, 4, 8, 16, 32, 64, 128, 256, 512]),
    8: ("sweep q4_0 4096x4096", Q4_0, 4096, 4096, [1, 2, 4, 8, 16, 32, 64, 128, 256, 512]),
    9: ("sweep q4_k 4096x4096", Q4_K, 4096, 4096, [1, 2, 4, 8, 16, 32, 64, 128, 256, 512]),
    10: ("sweep q6_k 4096x4096", Q6_K, 4096, 4096, [1, 2, 4, 8, 16, 32, 64, 128, 256, 512]),
    # not workloads of the pages' tables: the added dtypes, same sweep
    11: ("sweep q4_1 4096x4096", Q4_1, 4096, 4096, [1, 2, 4, 8, 16, 32, 64, 128, 256, 512]),
    12: ("sweep q5_k 4096x4096", Q5_K, 4096, 4096, [1, 2, 4, 8, 16, 32, 64, 128, 256, 512]),
}


def workload(wid: int, N: int | None = None):
    """(dtype, M, K, blob, X) for a workload; X has N rows (default: first N)."""
    label, dtype, M, K, ns = WORKLOADS[wid]
    N = ns[0] if N is None else N
    blob = make_blob(dtype, M, K, rng_for(wid, 0))
    X = make_x(N, K, rng_for(wid, 1000 + N))
    return dtype, M, K, blob, X
