"""The load-time Q6_K / Q8_0 repack and the GEMM on the repacked copy.

The pages repack prefill weights once at load into a second, kernel-friendly
copy kept beside the GGUF bytes (page "cera 0.5.2 src/backend/cpu.rs", the
Q4_0 / Q4_K weight repacking).  Here Q6_K and Q8_0 are repacked for the
matrix-core GEMM (qmm_repack) and qmm_gemm_repacked runs on that copy.

  * the repacked bytes, bit for bit, against a re-layout written here from the
    GGUF readings (Q6_K ql / qh / sc / d and Q8_0 d / q, the oracle's
    readings) and the layouts qmm.h documents: one code byte per weight at
    its lane position, then the scales as f32 (exact products);
  * qmm_gemm_repacked against the oracle on the ORIGINAL blob at the
    matrix-core tolerance (2e-3 of sum |w x|), N = 1 .. 513, ragged M;
  * bit for bit against qmm_gemm on the original blob wherever qmm_gemm runs
    the matrix cores with an even number of super-blocks per row (the same
    f16 weights and the same matrix-core steps), over every kernel id;
  * the hand-built edge blocks (negative and subnormal d, Q6_K sub-scales of
    both signs, Q8_0 codes of -128) with unit-vector and N(0, 1) activations;
  * the full 14336 x 4096 N = 512 shape on sampled rows.
"""
import numpy as np
import pytest
import torch

import gguf_block_quant_qmm_amd as q
import oracle
from qmm_inputs import make_blob, make_x, rng_for
from test_gpu_edge_blocks import golden_blob, unit_and_normal

pytestmark = pytest.mark.gpu

Q6, Q8 = q.QMM_Q6_K, q.QMM_Q8_0
DTS = [Q6, Q8]
NAME = {Q6: "Q6_K", Q8: "Q8_0"}
TAU = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def relayout_q6_k(blob, M, K):
    """The repacked Q6_K bytes, from the GGUF Q6_K layout: element j of a super-block
    (h = j / 128, g = (j % 128) / 32, l = j % 32) has the low (g < 2) or high
    nibble of ql[64h + 32(g & 1) + l] and bits 2g, 2g+1 of qh[32h + l] as
    bits 4, 5; its scale is sc[j / 16] (int8) times d (f16).  Repacked:
    weight k = 64c + 16s + 8kh + i at byte 64c + 32kh + 8s + i, then f32
    d * sc[0..15]."""
    nsb = M * (K // 256)
    b = blob.reshape(nsb, 210)
    j = np.arange(256)
    h, g, l = j // 128, (j % 128) // 32, j % 32
    qlb = b[:, 64 * h + 32 * (g & 1) + l]
    lo = np.where(g < 2, qlb & 15, qlb >> 4)
    hi = (b[:, 128 + 32 * h + l] >> (2 * g)) & 3
    codes = (lo | (hi << 4)).astype(np.uint8)
    c, s, kh, i = j // 64, (j % 64) // 16, (j % 16) // 8, j % 8
    pos = 64 * c + 32 * kh + 8 * s + i
    out = np.zeros((nsb, 320), np.uint8)
    out[:, pos] = codes
    d = b[:, 208:210].copy().view("<f2").astype(np.float32)  # [nsb, 1]
    sc = b[:, 192:208].view(np.int8).astype(np.float32)
    out[:, 256:320] = (d * sc).astype("<f4").view(np.uint8)
    return out.reshape(-1)


def relayout_q8_0(blob, M, K):
    """The repacked Q8_0 bytes, from the GGUF Q8_0 layout (f16 d, then int8
    q[32]): per pair of blocks, the 64 codes q + 128 in order, then both d as
    f32."""
    npair = M * (K // 64)
    b = blob.reshape(npair, 2, 34)
    out = np.zeros((npair, 72), np.uint8)
    out[:, :64] = (b[:, :, 2:].reshape(npair, 64).view(np.int8).astype(np.int16) + 128).astype(np.uint8)
    d = b[:, :, 0:2].copy().reshape(npair, 4).view("<f2").astype(np.float32)  # [npair, 2]
    out[:, 64:] = d.astype("<f4").view(np.uint8)
    return out.reshape(-1)


def relayout(dt, blob, M, K):
    return relayout_q6_k(blob, M, K) if dt == Q6 else relayout_q8_0(blob, M, K)


def gpu_repack(dt, blob, M, K):
    packed = torch.full((q.repack_bytes(dt, M, K),), 0xA5, dtype=torch.uint8, device="cuda")
    q.qmm_repack(to_dev(blob), dt, M, K, packed)
    torch.cuda.synchronize()
    return packed


def gpu_gemm_repacked(dt, packed, M, K, X):
    N = X.shape[0]
    Y = torch.full((N, M), float("nan"), device="cuda")
    q.qmm_gemm_repacked(packed, dt, M, K, N, to_dev(X), Y)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


def gpu_gemm(dt, bd, M, K, X):
    N = X.shape[0]
    Y = torch.full((N, M), float("nan"), device="cuda")
    q.qmm_gemm(bd, dt, M, K, N, to_dev(X), Y)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


def check(Yg, Y64, S, label):
    assert Yg.shape == Y64.shape, label
    assert np.all(np.isfinite(Yg)), f"{label}: non-finite output"
    err = np.abs(Yg.astype(np.float64) - Y64)
    zero = S == 0
    assert np.all(Yg[zero] == 0), f"{label}: S = 0 but output is not exactly 0"
    if (~zero).any():
        ratio = err[~zero] / S[~zero]
        worst = int(np.argmax(ratio))
        assert ratio[worst] <= TAU, f"{label}: |err|/S = {ratio[worst]:.3g} > {TAU} at flat index {worst}"


@pytest.mark.parametrize("dt", DTS, ids=NAME.get)
@pytest.mark.parametrize("M,K", [(1, 256), (37, 512), (300, 1280), (129, 4096)])
def test_repack_bytes(dt, M, K):
    for blob in (make_blob(dt, M, K, rng_for(1400, M), q8_full_range=True), golden_blob(dt, M, K)):
        got = gpu_repack(dt, blob, M, K).cpu().numpy()
        want = relayout(dt, blob, M, K)
        assert got.size == want.size == q.repack_bytes(dt, M, K)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, f"{NAME[dt]} M={M} K={K}: {bad.size} bytes differ, first at {bad[:5]}"


@pytest.mark.parametrize("dt", DTS, ids=NAME.get)
def test_repack_ragged_last_workgroup(dt):
    M, K = 1001, 768  # Q6_K: 48048 sub-blocks, Q8_0: 24024 blocks -- a partial last workgroup
    blob = make_blob(dt, M, K, rng_for(1401, 0))
    got = gpu_repack(dt, blob, M, K).cpu().numpy()
    assert np.array_equal(got, relayout(dt, blob, M, K))


@pytest.mark.parametrize("dt", DTS, ids=NAME.get)
@pytest.mark.parametrize("N", [1, 2, 5, 17, 32, 33, 64, 65, 130, 513])
def test_gemm_repacked_matches_oracle(dt, N):
    for i, (M, K) in enumerate([(70, 512), (129, 768), (300, 1024), (97, 2304)]):
        blob = make_blob(dt, M, K, rng_for(1410, i), q8_full_range=True)
        X = make_x(N, K, rng_for(1410, 1000 * N + i))
        _, Y64, S = oracle.matmul(dt, blob, M, K, X)
        Yg = gpu_gemm_repacked(dt, gpu_repack(dt, blob, M, K), M, K, X)
        check(Yg, Y64, S, f"repacked {NAME[dt]} M={M} K={K} N={N}")


# (M, K, N) chosen to reach every matrix-core kernel the repacked GEMM can run
BITWISE = [(14336, 1024, 512), (4096, 1024, 512), (1000, 1536, 20), (4096, 1024, 32), (14336, 1024, 32),
           (4096, 1024, 128), (4096, 1024, 256), (777, 2048, 77), (333, 512, 9)]


@pytest.mark.parametrize("dt", DTS, ids=NAME.get)
def test_gemm_repacked_reaches_every_kernel(dt):
    ids = {q.gemm_repacked_kernel(dt, M, K, N) for M, K, N in BITWISE}
    assert ids == set(range(1, 8)), ids


@pytest.mark.parametrize("dt", DTS, ids=NAME.get)
@pytest.mark.parametrize("M,K,N", BITWISE)
def test_gemm_repacked_bitwise_equals_qmm_gemm(dt, M, K, N):
    assert q.gemm_path(dt, M, K, N) == 1
    assert q.gemm_repacked_kernel(dt, M, K, N) == q.gemm_kernel(dt, M, K, N)
    blob = make_blob(dt, M, K, rng_for(1420, M + N), q8_full_range=True)
    X = make_x(N, K, rng_for(1420, 7 * N + K))
    Yr = gpu_gemm_repacked(dt, gpu_repack(dt, blob, M, K), M, K, X)
    Yo = gpu_gemm(dt, to_dev(blob), M, K, X)
    assert np.array_equal(Yr.view(np.uint32), Yo.view(np.uint32)), f"{NAME[dt]} M={M} K={K} N={N}: bits differ"
    rows = np.unique(np.concatenate([np.random.default_rng(M).choice(M, min(M, 40), replace=False), [0, M - 1]]))
    _, Y64, S = oracle.matmul(dt, blob, M, K, X, rows=rows)
    check(Yr[:, rows], Y64, S, f"repacked {NAME[dt]} M={M} K={K} N={N}")


@pytest.mark.parametrize("dt", DTS, ids=NAME.get)
@pytest.mark.parametrize("N", [1, 7, 40, 300])
def test_gemm_repacked_edge_blocks(dt, N):
    M, K = 97, 2048
    for shift in (0, 5):
        blob = golden_blob(dt, M, K, shift)
        X = unit_and_normal(K, max(2, N - 2), 1430 + N + shift)[:N] if N > 2 else make_x(N, K, rng_for(1430, N))
        _, Y64, S = oracle.matmul(dt, blob, M, K, X)
        Yr = gpu_gemm_repacked(dt, gpu_repack(dt, blob, M, K), M, K, X)
        check(Yr, Y64, S, f"repacked {NAME[dt]} edge blocks N={N} shift={shift}")
        if q.gemm_path(dt, M, K, N) == 1:
            assert np.array_equal(Yr.view(np.uint32), gpu_gemm(dt, to_dev(blob), M, K, X).view(np.uint32))


@pytest.mark.parametrize("dt", DTS, ids=NAME.get)
def test_gemm_repacked_full_size(dt):
    M, K, N = 14336, 4096, 512
    blob = make_blob(dt, M, K, rng_for(1440, 0))
    X = make_x(N, K, rng_for(1440, 1))
    packed = gpu_repack(dt, blob, M, K)
    Yr = gpu_gemm_repacked(dt, packed, M, K, X)
    assert np.array_equal(Yr.view(np.uint32), gpu_gemm(dt, to_dev(blob), M, K, X).view(np.uint32))
    rows = np.unique(np.concatenate([np.random.default_rng(3).choice(M, 48, replace=False), [0, M - 1]]))
    _, Y64, S = oracle.matmul(dt, blob, M, K, X, rows=rows)
    check(Yr[:, rows], Y64, S, f"repacked {NAME[dt]} 14336x4096 N=512")


def test_repack_argument_errors():
    blob = to_dev(make_blob(Q6, 8, 512, rng_for(1450, 0)))
    packed = torch.empty(q.repack_bytes(Q6, 8, 512) + 16, dtype=torch.uint8, device="cuda")
    X = torch.zeros((4, 512), device="cuda")
    Y = torch.empty((4, 8), device="cuda")
    L = q.lib()
    s = torch.cuda.current_stream().cuda_stream
    assert L.qmm_repack(blob.data_ptr(), q.QMM_Q4_K, 8, 512, packed.data_ptr(), s) == q.QMM_ERR_DTYPE
    assert L.qmm_repack(blob.data_ptr(), Q8, 8, 64, packed.data_ptr(), s) == q.QMM_ERR_SHAPE
    assert L.qmm_repack(blob.data_ptr(), Q6, 8, 500, packed.data_ptr(), s) == q.QMM_ERR_SHAPE
    assert L.qmm_repack(blob.data_ptr(), Q6, 8, 512, packed.data_ptr() + 8, s) == q.QMM_ERR_ALIGN
    assert L.qmm_repack(None, Q6, 8, 512, packed.data_ptr(), s) == q.QMM_ERR_NULL
    assert L.qmm_gemm_repacked(packed.data_ptr(), q.QMM_Q4_0, 8, 512, 4, X.data_ptr(), Y.data_ptr(), s) == \
        q.QMM_ERR_DTYPE
    assert L.qmm_gemm_repacked(packed.data_ptr() + 4, Q6, 8, 512, 4, X.data_ptr(), Y.data_ptr(), s) == \
        q.QMM_ERR_ALIGN
    assert L.qmm_gemm_repacked(packed.data_ptr(), Q6, 8, 512, 0, X.data_ptr(), Y.data_ptr(), s) == q.QMM_ERR_SHAPE
    torch.cuda.synchronize()
