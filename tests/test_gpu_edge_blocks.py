"""The hand-built edge blocks through every HIP entry point, against the oracle.

The 21 records of tests/golden/*_blocks.txt hold the values the random
generator never draws: Q8_0 codes of -128 (a legal stored code: page "cera
0.5.2 src/backend/cpu.rs", the portable Q8_0 quantizer clamps to [-128, 127]),
negative and f16-subnormal scales d, a subnormal and a negative Q4_1 minimum,
K-quant scales and minimums that use the high 2 bits of the 6-bit packing,
Q5_K fifth bits and Q6_K sub-scales of both signs.  Blobs are made of these
blocks in rotated order (every record at every block position, and rows made
of one record only), so every kernel decodes every record at every place it
can sit in a row.

Activations: unit vectors e_k (y = column k of W, exact on every path: a
single product, no rounding on the f32 paths and one exact f16 weight on the
matrix cores, since every golden weight is an f16 value) and N(0, 1).

Bar: |Y - Y_exact| <= tau * S per output with the path's tau (1e-5 on the
f32 path, 2e-3 on the matrix cores), Splus for the int8 activations, the
SwiGLU bound for the gated calls; fused calls and several-token calls also
bit for bit against their one-matrix, one-token forms.  Every kernel id that
qmm_gemm can choose for a dtype is reached (qmm_gemm_kernel reports it).
"""
import numpy as np
import pytest
import torch

import gguf_block_quant_qmm_amd as q
import oracle
from pins import load_golden
from qmm_inputs import make_blob, make_x, rng_for
from test_gpu_fused import check_argmax, check_swiglu, check_swiglu_tau

pytestmark = pytest.mark.gpu

DTYPES = [q.QMM_Q4_0, q.QMM_Q8_0, q.QMM_Q4_K, q.QMM_Q6_K, q.QMM_Q4_1, q.QMM_Q5_K]
NAME = {2: "Q4_0", 3: "Q4_1", 8: "Q8_0", 12: "Q4_K", 13: "Q5_K", 14: "Q6_K"}
TAU = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bs_of(dt):
    return 256 if dt in (q.QMM_Q4_K, q.QMM_Q5_K, q.QMM_Q6_K) else 32


def golden_blob(dt, M, K, shift=0):
    """M x K blob of golden blocks: block b of row m is record (3m + b + shift) mod n;
    rows m = 1 (mod 7) repeat one record across the whole row."""
    recs = load_golden(NAME[dt])
    n = len(recs)
    nb = K // bs_of(dt)
    rows = []
    for m in range(M):
        if m % 7 == 1:
            idx = [(m // 7 + shift) % n] * nb
        else:
            idx = [(3 * m + b + shift) % n for b in range(nb)]
        rows.append(b"".join(recs[i][1] for i in idx))
    return np.frombuffer(b"".join(rows), np.uint8).copy()


def unit_and_normal(K, n_unit, seed):
    """X: n_unit unit vectors (positions spread over the row, both ends
    included) followed by two N(0, 1) rows."""
    ks = np.unique(np.concatenate([[0, K - 1], np.random.default_rng(seed).choice(K, n_unit - 2, replace=False)]))
    X = np.zeros((len(ks) + 2, K), np.float32)
    X[np.arange(len(ks)), ks] = 1.0
    X[len(ks):] = make_x(2, K, rng_for(1300, seed))
    return X


def check(Yg, Y64, S, tau, label):
    assert Yg.shape == Y64.shape, label
    assert np.all(np.isfinite(Yg)), f"{label}: non-finite output"
    err = np.abs(Yg.astype(np.float64) - Y64)
    zero = S == 0
    assert np.all(Yg[zero] == 0), f"{label}: S = 0 but output is not exactly 0"
    if (~zero).any():
        ratio = err[~zero] / S[~zero]
        worst = int(np.argmax(ratio))
        assert ratio[worst] <= tau, f"{label}: |err|/S = {ratio[worst]:.3g} > {tau} at flat index {worst}"


def sample_rows(M, n, seed):
    if M <= 3 * n:
        return np.arange(M)
    r = np.random.default_rng(seed).choice(M, n, replace=False)
    return np.unique(np.concatenate([r, np.arange(8), M - 1 - np.arange(40)]))


# ------------------------------------------------------------------- GEMV

def gemv_shapes(dt):
    # whole-row wavefronts, a workgroup splitting K, and (32-weight blocks:
    # an odd block count) the byte-load kernel
    s = [(77, 4096), (33, 8192), (5, 16384)]
    if bs_of(dt) == 32:
        s.append((21, 96))
    elif dt == q.QMM_Q6_K:
        s.append((21, 768))
    return s


@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
def test_gemv_edge_blocks(dt):
    for i, (M, K) in enumerate(gemv_shapes(dt)):
        blob = golden_blob(dt, M, K, shift=i)
        bd = to_dev(blob)
        X = unit_and_normal(K, 6, 10 * dt + i)
        _, Y64, S = oracle.matmul(dt, blob, M, K, X)
        for n in range(X.shape[0]):
            y = torch.full((M,), float("nan"), device="cuda")
            q.qmm_gemv(bd, dt, M, K, to_dev(X[n]), y)
            torch.cuda.synchronize()
            check(y.cpu().numpy()[None], Y64[n:n + 1], S[n:n + 1], TAU, f"{NAME[dt]} gemv M={M} K={K} x#{n}")


def test_q8_0_full_code_range_gemv_and_gemm():
    """Random Q8_0 blobs whose codes include -128 (the generator's full-range
    mode), through the GEMV, the several-token path and the matrix cores."""
    dt, M, K = q.QMM_Q8_0, 300, 4096
    blob = make_blob(dt, M, K, rng_for(1310, 0), q8_full_range=True)
    assert np.any(blob.reshape(-1, 34)[:, 2:].view(np.int8) == -128)
    bd = to_dev(blob)
    for N in (1, 3, 40):
        X = make_x(N, K, rng_for(1310, N))
        _, Y64, S = oracle.matmul(dt, blob, M, K, X)
        Y = torch.full((N, M), float("nan"), device="cuda")
        q.qmm_gemm(bd, dt, M, K, N, to_dev(X), Y)
        torch.cuda.synchronize()
        check(Y.cpu().numpy(), Y64, S, q.tolerance(dt, M, K, N), f"Q8_0 full range N={N}")


# ------------------------------------------------------------------- GEMM

# (M, K, N) candidates; each dtype's shapes must reach every kernel id the
# library can choose for it (asserted below)
GEMM_CANDIDATES = [
    (77, 1024, 1),      # one f32 GEMV
    (77, 1024, 2),      # several-token f32 GEMV (or the matrix cores from N = 2)
    (77, 1024, 4),
    (70, 96, 40),       # 32-weight blocks, odd count: LDS-staged kernel
    (21, 768, 40),      # Q6_K with an odd super-block count: LDS-staged kernel
    (300, 512, 17),     # register-B kernel, 32-token tiles
    (300, 512, 65),     # register-B kernel, 64-token tiles
    (7200, 512, 1000),  # register-B kernel, 8 wavefronts x 128 tokens
    (33000, 1024, 17),  # register-B kernel, 32-token tiles, tall
    (300, 1024, 17),    # split-K kernel
    (12300, 1024, 20),  # split-K kernel, two row fragments
    (2100, 1024, 100),  # split-K kernel, 64 tokens
    (3200, 1024, 150),  # split-K kernel, 64 tokens, two row fragments
]


def gemm_cases(dt):
    bs = bs_of(dt)
    return [(M, K, N) for (M, K, N) in GEMM_CANDIDATES
            if K % bs == 0 and not (dt == q.QMM_Q6_K and K == 96) and not (bs == 32 and K == 768)]


def reachable_ids(dt):
    """Every id qmm_gemm_kernel reports over a wide grid of shapes."""
    ids = set()
    bs = bs_of(dt)
    for K in (96, 512, 768, 1024, 4096, 8192):
        if K % bs:
            continue
        for M in (1, 70, 300, 2100, 3200, 7200, 12300, 33000, 128256):
            for N in (1, 2, 3, 4, 5, 17, 20, 32, 33, 64, 65, 100, 128, 150, 256, 512, 1000):
                ids.add(q.gemm_kernel(dt, M, K, N))
    return ids


@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
def test_gemm_edge_blocks_every_kernel(dt):
    seen = set()
    for i, (M, K, N) in enumerate(gemm_cases(dt)):
        kid = q.gemm_kernel(dt, M, K, N)
        seen.add(kid)
        blob = golden_blob(dt, M, K, shift=i)
        bd = to_dev(blob)
        X = unit_and_normal(K, min(N, 6), 100 * dt + i) if N >= 4 else make_x(N, K, rng_for(1320 + dt, i))
        if X.shape[0] < N:
            X = np.concatenate([X, make_x(N - X.shape[0], K, rng_for(1330 + dt, i))])
        X = X[:N]
        rows = sample_rows(M, 120, 1340 + i) if M * N > 400000 else None
        _, Y64, S = oracle.matmul(dt, blob, M, K, X, rows=rows)
        Y = torch.full((N, M), float("nan"), device="cuda")
        q.qmm_gemm(bd, dt, M, K, N, to_dev(X), Y)
        torch.cuda.synchronize()
        Yg = Y.cpu().numpy()
        assert np.all(np.isfinite(Yg)), f"{NAME[dt]} kernel {kid}: non-finite output"
        if rows is not None:
            Yg = Yg[:, rows]
        check(Yg, Y64, S, q.tolerance(dt, M, K, N), f"{NAME[dt]} gemm kernel {kid} M={M} K={K} N={N}")
        if kid == q.QMM_KERNEL_GEMV_TOKENS:
            # each token has the bits of its own GEMV
            for n in range(N):
                y = torch.empty(M, device="cuda")
                q.qmm_gemv(bd, dt, M, K, to_dev(X[n]), y)
                torch.cuda.synchronize()
                assert torch.equal(y, Y[n]), f"{NAME[dt]} M={M} K={K} N={N}: token {n} differs from qmm_gemv"
    missing = reachable_ids(dt) - seen
    assert not missing, f"{NAME[dt]}: kernels {sorted(missing)} not reached by the edge-block shapes"


# ------------------------------------------------------------ fused calls

@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
def test_fused_calls_edge_blocks(dt):
    for i, (Ms, K) in enumerate((([77, 40], 4096), ([33, 5, 9], 8192))):
        blobs = [golden_blob(dt, M, K, shift=j) for j, M in enumerate(Ms)]
        bds = [to_dev(b) for b in blobs]
        X = unit_and_normal(K, 4, 200 * dt + i)
        for n in range(X.shape[0]):
            x = X[n]
            xd = to_dev(x)
            label = f"{NAME[dt]} K={K} x#{n}"
            # several matrices in one launch: each its own GEMV's bits
            ys = [torch.full((M,), float("nan"), device="cuda") for M in Ms]
            q.qmm_gemv_concat(bds, dt, Ms, K, xd, ys)
            for b, bd, M, y in zip(blobs, bds, Ms, ys):
                ref = torch.empty(M, device="cuda")
                q.qmm_gemv(bd, dt, M, K, xd, ref)
                torch.cuda.synchronize()
                assert torch.equal(y, ref), f"{label}: concat differs from qmm_gemv"
                _, Y64, S = oracle.matmul(dt, b, M, K, x)
                check(y.cpu().numpy()[None], Y64, S, TAU, f"{label} concat")
            # gate/up with SwiGLU (rows of the first two shapes' first matrix)
            M = Ms[0]
            gate, up = blobs[0], golden_blob(dt, M, K, shift=5)
            gd, ud = bds[0], to_dev(up)
            out = torch.full((M,), float("nan"), device="cuda")
            q.qmm_gemv_swiglu(gd, ud, dt, M, K, xd, out)
            g_gpu, u_gpu = torch.empty(M, device="cuda"), torch.empty(M, device="cuda")
            q.qmm_gemv(gd, dt, M, K, xd, g_gpu)
            q.qmm_gemv(ud, dt, M, K, xd, u_gpu)
            torch.cuda.synchronize()
            r = oracle.swiglu(dt, gate, up, M, K, x)
            check_swiglu(out.cpu().numpy(), r, g_gpu.cpu().numpy(), u_gpu.cpu().numpy(), f"{label} swiglu")
            # greedy argmax over the GEMV's outputs
            check_argmax(dt, gate, M, K, x, f"{label} argmax")


@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
def test_gemm_swiglu_edge_blocks(dt):
    M, K = 129, 4096
    gate, up = golden_blob(dt, M, K, shift=1), golden_blob(dt, M, K, shift=4)
    gd, ud = to_dev(gate), to_dev(up)
    for N in (3, 40):
        X = unit_and_normal(K, min(N, 6), 300 * dt + N)[:N]
        if X.shape[0] < N:
            X = np.concatenate([X, make_x(N - X.shape[0], K, rng_for(1350 + dt, N))])
        out = torch.full((N, M), float("nan"), device="cuda")
        q.qmm_gemm_swiglu(gd, ud, dt, M, K, N, to_dev(X), out)
        torch.cuda.synchronize()
        r = oracle.swiglu(dt, gate, up, M, K, X)
        check_swiglu_tau(out.cpu().numpy(), r, q.tolerance(dt, M, K, N), f"{NAME[dt]} gemm swiglu N={N}")


# ------------------------------------------------------- int8 activations

def check_splus(Yg, Y64, Sp, label):
    check(Yg, Y64, Sp, TAU, label)


@pytest.mark.parametrize("dt", [q.QMM_Q8_0, q.QMM_Q4_0, q.QMM_Q4_K], ids=NAME.get)
def test_q8act_matrix_cores_edge_blocks(dt):
    """The golden blocks through the int8 matrix cores."""
    M, K, N = 14000, 1024, 40
    blob = golden_blob(dt, M, K, shift=3)
    X = unit_and_normal(K, 12, 500 * dt)
    X = np.concatenate([X, make_x(N - X.shape[0], K, rng_for(1360 + dt, 0))])[:N]
    assert q.q8act_kernel(dt, M, K, N) == 1
    so, qo = oracle.quantize_q8_0(X)
    rows = sample_rows(M, 200, 1370 + dt)
    _, Y64, _, Sp = oracle.matmul_q8act(dt, blob, M, K, so, qo, rows=rows)
    Y = torch.full((N, M), float("nan"), device="cuda")
    q.qmm_gemm_q8act(to_dev(blob), dt, M, K, N, to_dev(so), to_dev(qo), Y)
    torch.cuda.synchronize()
    check_splus(Y.cpu().numpy()[:, rows], Y64, Sp, f"{NAME[dt]} int8 matrix cores, golden blocks")


@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
def test_q8act_edge_blocks(dt):
    for i, (M, K) in enumerate(((77, 4096), (33, 8192))):
        blob = golden_blob(dt, M, K, shift=i + 2)
        bd = to_dev(blob)
        X = unit_and_normal(K, 5, 400 * dt + i)
        N = X.shape[0]
        sc = torch.empty((N, K // 32), device="cuda")
        qq = torch.empty((N, K), dtype=torch.int8, device="cuda")
        q.qmm_quantize_q8_0(to_dev(X), N, K, sc, qq)
        torch.cuda.synchronize()
        so, qo = oracle.quantize_q8_0(X)
        assert np.array_equal(sc.cpu().numpy().view(np.uint32), so.view(np.uint32)), "quantizer scales"
        assert np.array_equal(qq.cpu().numpy(), qo), "quantizer codes"
        _, Y64, _, Sp = oracle.matmul_q8act(dt, blob, M, K, so, qo)
        Y = torch.full((N, M), float("nan"), device="cuda")
        q.qmm_gemm_q8act(bd, dt, M, K, N, sc, qq, Y)
        torch.cuda.synchronize()
        check_splus(Y.cpu().numpy(), Y64, Sp, f"{NAME[dt]} q8act M={M} K={K} N={N}")
        # one-launch decode calls: the bits of quantize + qmm_gemm_q8act
        up = golden_blob(dt, M, K, shift=i + 5)
        udv = to_dev(up)
        for n in range(N):
            xd = to_dev(X[n])
            y = torch.full((M,), float("nan"), device="cuda")
            q.qmm_gemv_q8act(bd, dt, M, K, xd, y)
            ys = [torch.full((M,), float("nan"), device="cuda") for _ in range(2)]
            q.qmm_gemv_concat_q8act([bd, udv], dt, [M, M], K, xd, ys)
            Yu = torch.full((1, M), float("nan"), device="cuda")
            q.qmm_gemm_q8act(udv, dt, M, K, 1, sc[n:n + 1], qq[n:n + 1], Yu)
            torch.cuda.synchronize()
            assert torch.equal(y, Y[n]), f"{NAME[dt]} x#{n}: qmm_gemv_q8act differs from the two-step form"
            assert torch.equal(ys[0], Y[n]) and torch.equal(ys[1], Yu[0]), f"{NAME[dt]} x#{n}: concat q8act"
            # gate/up with SwiGLU on the int8 projections: silu(g) * u of the
            # projections' own bits, to f32 rounding
            out = torch.full((M,), float("nan"), device="cuda")
            q.qmm_gemv_swiglu_q8act(bd, udv, dt, M, K, xd, out)
            torch.cuda.synchronize()
            g2, u2 = Y[n].cpu().numpy().astype(np.float64), Yu[0].cpu().numpy().astype(np.float64)
            with np.errstate(over="ignore"):
                mine = g2 / (1.0 + np.exp(-g2)) * u2
            lim = 4 * 2.0 ** -24 * np.abs(mine) + 2.0 ** -119 * np.abs(u2)
            assert np.all(np.abs(out.cpu().numpy() - mine) <= lim), f"{NAME[dt]} x#{n}: swiglu q8act"
            work = torch.empty(q.QMM_ARGMAX_WORK_BYTES, dtype=torch.uint8, device="cuda")
            idx = torch.full((1,), -7, dtype=torch.int64, device="cuda")
            val = torch.full((1,), float("nan"), device="cuda")
            q.qmm_gemv_argmax_q8act(bd, dt, M, K, xd, work, idx, val)
            torch.cuda.synchronize()
            yy = y.cpu().numpy()
            want = int(np.flatnonzero(yy == yy.max())[0])
            assert int(idx.item()) == want, f"{NAME[dt]} x#{n}: argmax q8act {int(idx.item())}, want {want}"
            assert val.cpu().numpy()[0] == yy[want]
