"""Seeded random shapes through every entry point, against the oracle.

For each dtype, random M (1..3000), K (block multiples with even and odd
block counts, up to 20480), N (1..600, weighted towards the small values
where the paths switch), and random matrix counts for the fused calls.  The
bar is the same as the fixed-shape tests: 1e-5 * S on the f32 paths, 2e-3 * S
on the matrix-core path (whichever qmm_gemm_path reports), the GEMV's bits for
qmm_gemv_concat and for qmm_gemm below the crossover, and a valid maximum for
qmm_gemv_argmax; for the int8-activation calls the oracle's quantizer bits and
1e-5 * Splus.
"""
import numpy as np
import pytest
import torch

import gguf_block_quant_qmm_amd as q
import oracle
from qmm_inputs import make_blob, make_x, rng_for

pytestmark = pytest.mark.gpu

DTYPES = [q.QMM_Q4_0, q.QMM_Q8_0, q.QMM_Q4_K, q.QMM_Q6_K, q.QMM_Q4_1, q.QMM_Q5_K]
NAME = {2: "Q4_0", 3: "Q4_1", 8: "Q8_0", 12: "Q4_K", 13: "Q5_K", 14: "Q6_K"}
BS = {2: 32, 3: 32, 8: 32, 12: 256, 13: 256, 14: 256}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def within(Yg, Y64, S, tau, label):
    Yg = Yg.astype(np.float64)
    assert np.all(np.isfinite(Yg)), f"{label}: non-finite"
    zero = S == 0
    assert np.all(Yg[zero] == 0), f"{label}: S = 0 but output not 0"
    if (~zero).any():
        r = np.abs(Yg - Y64)[~zero] / S[~zero]
        assert r.max() <= tau, f"{label}: |err|/S = {r.max():.3g} > {tau}"


def fused_ok(dt, K):
    """The shapes qmm_gemv_swiglu / qmm_gemv_argmax accept."""
    return K % 64 == 0 and K <= 16384 and (dt in (q.QMM_Q4_K, q.QMM_Q5_K) or (K // BS[dt]) % 2 == 0)


def random_shape(rng, dt):
    bs = BS[dt]
    nb = int(rng.integers(1, (20480 // bs) + 1)) if rng.random() < 0.3 else int(rng.integers(1, (4096 // bs) + 1))
    M = int(rng.integers(1, 3001))
    N = int(rng.choice([1, 2, 3, 4, 5, 7, 9, 16, 33, 64, 129, 257, 600]))
    while M * nb * bs * N > 60_000_000:   # keep the oracle at a second or so
        M = max(1, M // 2)
        if M == 1:
            N = max(1, N // 2)
    return M, nb * bs, N


@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
def test_random_gemm(dt):
    rng = np.random.default_rng(4242 + dt)
    for case in range(12):
        M, K, N = random_shape(rng, dt)
        blob = make_blob(dt, M, K, rng_for(4300 + dt, case))
        X = make_x(N, K, rng_for(4400 + dt, case))
        bd = dev(blob)
        Y = torch.full((N, M), float("nan"), device="cuda")
        q.qmm_gemm(bd, dt, M, K, N, dev(X), Y)
        torch.cuda.synchronize()
        Yg = Y.cpu().numpy()
        _, Y64, S = oracle.matmul(dt, blob, M, K, X)
        label = f"{NAME[dt]} case {case} M={M} K={K} N={N}"
        within(Yg, Y64, S, q.tolerance(dt, M, K, N), label)
        if q.gemm_path(dt, M, K, N) == 0:
            y = torch.empty(M, device="cuda")
            for n in range(min(N, 3)):
                q.qmm_gemv(bd, dt, M, K, dev(X[n]), y)
                torch.cuda.synchronize()
                assert np.array_equal(y.cpu().numpy().view(np.uint32), Yg[n].view(np.uint32)), \
                    f"{label}: token {n} differs from qmm_gemv"


@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
def test_random_fused(dt):
    rng = np.random.default_rng(4500 + dt)
    for case in range(6):
        n = int(rng.integers(1, 5))
        bs = BS[dt]
        K = bs * int(rng.integers(1, (8192 // bs) + 1))
        Ms = [int(rng.integers(1, 2000)) for _ in range(n)]
        blobs = [make_blob(dt, M, K, rng_for(4600 + dt, 10 * case + i)) for i, M in enumerate(Ms)]
        x = make_x(1, K, rng_for(4700 + dt, case))
        bds, xd = [dev(b) for b in blobs], dev(x.reshape(-1))
        ys = [torch.full((M,), float("nan"), device="cuda") for M in Ms]
        q.qmm_gemv_concat(bds, dt, Ms, K, xd, ys)
        for i, (M, b) in enumerate(zip(Ms, blobs)):
            ref = torch.empty(M, device="cuda")
            q.qmm_gemv(bds[i], dt, M, K, xd, ref)
            torch.cuda.synchronize()
            assert torch.equal(ys[i], ref), f"{NAME[dt]} concat case {case} matrix {i}: bits differ"
        # argmax over the first matrix, where the call takes the shape
        M0 = Ms[0]
        if fused_ok(dt, K):
            work = torch.empty(q.QMM_ARGMAX_WORK_BYTES, dtype=torch.uint8, device="cuda")
            idx = torch.empty(1, dtype=torch.int64, device="cuda")
            q.qmm_gemv_argmax(bds[0], dt, M0, K, xd, work, idx)
            torch.cuda.synchronize()
            y0 = ys[0].cpu().numpy()
            assert int(idx.item()) == int(np.flatnonzero(y0 == y0.max())[0]), f"{NAME[dt]} argmax case {case}"
            oi, obest, os_ = oracle.argmax(dt, blobs[0], M0, K, x)
            _, Y64, S = oracle.matmul(dt, blobs[0], M0, K, x, rows=[int(idx.item())])
            assert Y64[0, 0] >= obest - 1e-5 * (S[0, 0] + os_)
        else:
            with pytest.raises(q.QmmError):
                q.qmm_gemv_argmax(bds[0], dt, M0, K, xd, torch.empty(q.QMM_ARGMAX_WORK_BYTES, dtype=torch.uint8,
                                                                     device="cuda"),
                                  torch.empty(1, dtype=torch.int64, device="cuda"))


@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
def test_random_pair(dt):
    """Two matrices of one shape through qmm_gemv_concat (the paired form):
    random M and K, each output the bits of its own qmm_gemv."""
    rng = np.random.default_rng(4550 + dt)
    bs = BS[dt]
    for case in range(6):
        K = bs * int(rng.integers(1, (16384 // bs) + 1))
        M = int(rng.integers(1, 3000))
        blobs = [make_blob(dt, M, K, rng_for(4650 + dt, 10 * case + i)) for i in range(2)]
        x = make_x(1, K, rng_for(4750 + dt, case))
        bds, xd = [dev(b) for b in blobs], dev(x.reshape(-1))
        ys = [torch.full((M,), float("nan"), device="cuda") for _ in range(2)]
        q.qmm_gemv_concat(bds, dt, [M, M], K, xd, ys)
        for i in range(2):
            ref = torch.empty(M, device="cuda")
            q.qmm_gemv(bds[i], dt, M, K, xd, ref)
            torch.cuda.synchronize()
            assert torch.equal(ys[i], ref), f"{NAME[dt]} pair case {case} M={M} K={K} matrix {i}: bits differ"


@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
def test_random_q8act(dt):
    """Random shapes through the int8-activation entry points: the quantizer
    bit-exact with the oracle's, qmm_gemm_q8act within 1e-5 of Splus, and the
    one-launch calls bit-identical to quantize + qmm_gemm_q8act where they take
    the shape (QMM_ERR_SHAPE otherwise)."""
    rng = np.random.default_rng(4800 + dt)
    for case in range(8):
        M, K, N = random_shape(rng, dt)
        N = min(N, 40)
        blob = make_blob(dt, M, K, rng_for(4900 + dt, case))
        X = make_x(N, K, rng_for(5000 + dt, case))
        bd, Xd = dev(blob), dev(X)
        sc = torch.empty((N, K // 32), device="cuda")
        qq = torch.empty((N, K), dtype=torch.int8, device="cuda")
        Y = torch.full((N, M), float("nan"), device="cuda")
        q.qmm_quantize_q8_0(Xd, N, K, sc, qq)
        q.qmm_gemm_q8act(bd, dt, M, K, N, sc, qq, Y)
        torch.cuda.synchronize()
        label = f"{NAME[dt]} q8act case {case} M={M} K={K} N={N}"
        so, qo = oracle.quantize_q8_0(X)
        assert np.array_equal(sc.cpu().numpy().view(np.uint32), so.view(np.uint32)), f"{label}: scales"
        assert np.array_equal(qq.cpu().numpy(), qo), f"{label}: codes"
        _, Y64, _, Sp = oracle.matmul_q8act(dt, blob, M, K, so, qo)
        Yg = Y.cpu().numpy()
        within(Yg, Y64, Sp, 1e-5, label)
        y = torch.full((M,), float("nan"), device="cuda")
        if fused_ok(dt, K):
            # against the two-step form for that one token (N = 1: the
            # few-token arithmetic; an N-token call from N = 16 may run on the
            # int8 matrix cores, whose bits differ)
            y1 = torch.full((1, M), float("nan"), device="cuda")
            q.qmm_gemm_q8act(bd, dt, M, K, 1, sc[0:1], qq[0:1], y1)
            q.qmm_gemv_q8act(bd, dt, M, K, Xd[0], y)
            torch.cuda.synchronize()
            assert np.array_equal(y.cpu().numpy().view(np.uint32), y1.cpu().numpy()[0].view(np.uint32)), \
                f"{label}: one-launch call differs from quantize + q8act"
        else:
            with pytest.raises(q.QmmError):
                q.qmm_gemv_q8act(bd, dt, M, K, Xd[0], y)
