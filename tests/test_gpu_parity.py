"""HIP path against the CPU oracle, element by element, through the C ABI.

Bar: |Y_gpu - Y_exact| <= tau * S per output, with S = sum_k |W x| and
Y_exact the oracle's f64 sum (within 1e-12 S of exact); tau = 1e-5 on the
f32 path (qmm_gemv, qmm_gemm at N = 1) and 2e-3 on the f16 matrix-core path;
S = 0 demands an exact 0.

  * small shapes, full output: several tiles, ragged M/N/K tails, odd block
    counts (the byte-load kernels), N beyond 512;
  * every workload at its full size in the launch configuration the bench
    times, compared on sampled rows (all N columns of each sampled row);
  * bitwise: qmm_gemm at N = 1 equals qmm_gemv; two runs give equal bits.
"""
import numpy as np
import pytest
import torch

import gguf_block_quant_qmm_amd as q
import oracle
from qmm_inputs import WORKLOADS, make_blob, make_x, rng_for

pytestmark = pytest.mark.gpu

DTYPES = [q.QMM_Q4_0, q.QMM_Q8_0, q.QMM_Q4_K, q.QMM_Q6_K, q.QMM_Q4_1, q.QMM_Q5_K]
NAME = {2: "Q4_0", 3: "Q4_1", 8: "Q8_0", 12: "Q4_K", 13: "Q5_K", 14: "Q6_K"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_gemv(dt, blob_d, M, K, x):
    y = torch.full((M,), float("nan"), device="cuda")
    q.qmm_gemv(blob_d, dt, M, K, to_dev(x.reshape(-1)), y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def gpu_gemm(dt, blob_d, M, K, X):
    N = X.shape[0]
    Y = torch.full((N, M), float("nan"), device="cuda")
    q.qmm_gemm(blob_d, dt, M, K, N, to_dev(X), Y)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


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


def bs_of(dt):
    return 256 if dt in (q.QMM_Q4_K, q.QMM_Q5_K, q.QMM_Q6_K) else 32


# ----------------------------------------------------------------- GEMV ----

def gemv_shapes(dt):
    if bs_of(dt) == 32:
        # nb odd -> byte-load kernel; K = 65600 -> more units than threads
        return [(1, 32), (1, 64), (3, 96), (67, 256), (300, 1024), (129, 4160), (50, 14336), (33, 16416),
                (5, 65600)]
    return [(1, 256), (3, 512), (67, 768), (300, 2048), (50, 4096), (9, 16640)]


@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
def test_gemv_small(dt):
    for i, (M, K) in enumerate(gemv_shapes(dt)):
        blob = make_blob(dt, M, K, rng_for(500 + dt, i))
        x = make_x(1, K, rng_for(500 + dt, 100 + i))
        _, Y64, S = oracle.matmul(dt, blob, M, K, x)
        yg = gpu_gemv(dt, to_dev(blob), M, K, x)
        check(yg[None, :], Y64, S, 1e-5, f"{NAME[dt]} gemv M={M} K={K}")


@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
def test_gemv_long_rows(dt):
    # K = 14336 split over 4 wavefronts on 2048+ rows: one row per group and a
    # short ring for Q4_0 / Q4_1 / Q4_K; uneven row ranges per workgroup
    K = 14336
    for i, M in enumerate((2048, 4099, 8193)):
        blob = make_blob(dt, M, K, rng_for(530 + dt, i))
        x = make_x(1, K, rng_for(530 + dt, 100 + i))
        _, Y64, S = oracle.matmul(dt, blob, M, K, x)
        yg = gpu_gemv(dt, to_dev(blob), M, K, x)
        check(yg[None, :], Y64, S, 1e-5, f"{NAME[dt]} gemv M={M} K={K}")


@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
def test_gemv_row_phases(dt):
    # rows of two wavefronts (4097 <= K <= 8192): two row phases share each
    # workgroup's staging of x; few rows leave phases with one group fewer
    # than others, or none (they decode zeros and store nothing)
    for K in (6144, 8192):
        for i, M in enumerate((1, 5, 130, 4099)):
            blob = make_blob(dt, M, K, rng_for(540 + dt, 10 * i + K // 2048))
            x = make_x(1, K, rng_for(540 + dt, 100 + 10 * i + K // 2048))
            _, Y64, S = oracle.matmul(dt, blob, M, K, x)
            yg = gpu_gemv(dt, to_dev(blob), M, K, x)
            check(yg[None, :], Y64, S, 1e-5, f"{NAME[dt]} gemv M={M} K={K}")


@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
def test_gemv_rows_per_wavefront(dt):
    # M spans the launch variants: 1..4 row groups per wavefront fetched up
    # front, and the prefetch ring beyond; K = 4096 (independent wavefronts)
    # and K = 8192 (a workgroup splits K), each with a ragged last group.
    for K in (4096, 8192):
        for i, M in enumerate((1001, 8193, 12003, 17001, 40001)):
            blob = make_blob(dt, M, K, rng_for(520 + dt, 10 * i + K // 4096))
            x = make_x(1, K, rng_for(520 + dt, 100 + 10 * i + K // 4096))
            _, Y64, S = oracle.matmul(dt, blob, M, K, x)
            yg = gpu_gemv(dt, to_dev(blob), M, K, x)
            check(yg[None, :], Y64, S, 1e-5, f"{NAME[dt]} gemv M={M} K={K}")


# ----------------------------------------------------------------- GEMM ----

def gemm_shapes(dt):
    if bs_of(dt) == 32:
        return [(70, 96), (300, 1024), (129, 2080)]
    return [(70, 512), (129, 768), (300, 1024)]


@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
@pytest.mark.parametrize("N", [2, 3, 17, 32, 33, 64, 65, 130, 513])
def test_gemm_small(dt, N):
    for i, (M, K) in enumerate(gemm_shapes(dt)):
        blob = make_blob(dt, M, K, rng_for(600 + dt, i))
        X = make_x(N, K, rng_for(600 + dt, 1000 * N + i))
        _, Y64, S = oracle.matmul(dt, blob, M, K, X)
        Yg = gpu_gemm(dt, to_dev(blob), M, K, X)
        check(Yg, Y64, S, q.tolerance(dt, M, K, N), f"{NAME[dt]} gemm M={M} K={K} N={N}")


@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
def test_gemm_register_b_kernel_ragged(dt):
    # M/256 x N/128 >= 200 workgroups selects the register-B kernel with 8
    # wavefronts x 128 tokens for every dtype (K = 512 keeps the Q6_K block
    # count even); M and N both end in partial tiles.  Sampled rows include
    # the last (partial) row tile.
    M, K, N = 7200, 512, 1000
    assert q.gemm_kernel(dt, M, K, N) == 1
    blob = make_blob(dt, M, K, rng_for(650 + dt, 0))
    X = make_x(N, K, rng_for(650 + dt, 1))
    rows = np.unique(np.concatenate([sample_rows(M, 40, 650 + dt), np.arange(M - 40, M)]))
    _, Y64, S = oracle.matmul(dt, blob, M, K, X, rows=rows)
    Yg = gpu_gemm(dt, to_dev(blob), M, K, X)
    assert np.all(np.isfinite(Yg))
    check(Yg[:, rows], Y64, S, q.tolerance(dt, M, K, N), f"{NAME[dt]} register-B gemm M={M} K={K} N={N}")


# ------------------------------------------------------------ properties ----

@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
def test_gemm_n1_is_gemv_bitwise_and_deterministic(dt):
    for i, (M, K) in enumerate([(300, 4 * bs_of(dt) * 4), (77, 3 * bs_of(dt))]):
        blob_d = to_dev(make_blob(dt, M, K, rng_for(700 + dt, i)))
        x = make_x(1, K, rng_for(700 + dt, 10 + i))
        a = gpu_gemv(dt, blob_d, M, K, x)
        b = gpu_gemm(dt, blob_d, M, K, x)[0]
        c = gpu_gemv(dt, blob_d, M, K, x)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "qmm_gemm(N=1) != qmm_gemv"
        assert np.array_equal(a.view(np.uint32), c.view(np.uint32)), "gemv not deterministic"
        X = make_x(40, K, rng_for(700 + dt, 20 + i))
        assert np.array_equal(gpu_gemm(dt, blob_d, M, K, X), gpu_gemm(dt, blob_d, M, K, X)), "gemm not deterministic"
        # below the crossover qmm_gemm runs the GEMV per token: its bits
        X2 = make_x(2, K, rng_for(700 + dt, 30 + i))
        if q.gemm_path(dt, M, K, 2) == 0:
            G = gpu_gemm(dt, blob_d, M, K, X2)
            for n in range(2):
                assert np.array_equal(G[n].view(np.uint32), gpu_gemv(dt, blob_d, M, K, X2[n]).view(np.uint32))


@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
def test_zero_scales_give_exact_zero(dt):
    M, K = 45, 8 * bs_of(dt)
    blob = make_blob(dt, M, K, rng_for(800 + dt, 0)).reshape(M * (K // bs_of(dt)), -1)
    offs = {2: [0], 3: [0, 2], 8: [0], 12: [0, 2], 13: [0, 2], 14: [208]}[dt]
    for o in offs:
        blob[:, o:o + 2] = 0
    blob = blob.reshape(-1)
    x = make_x(3, K, rng_for(800 + dt, 1))
    _, Y64, S = oracle.matmul(dt, blob, M, K, x)
    assert np.all(S == 0)
    bd = to_dev(blob)
    assert np.all(gpu_gemv(dt, bd, M, K, x[0]) == 0)
    assert np.all(gpu_gemm(dt, bd, M, K, x) == 0)


def test_sparse_rows_keep_f32_bound():
    # Q4_0 rows whose weights are all zero (nibble 8) but one: S is tiny, the
    # f32 GEMV must still be within 1e-5 of it (no cancellation shortcuts).
    M, K = 64, 1024
    blob = make_blob(q.QMM_Q4_0, M, K, rng_for(810, 0)).reshape(M, K // 32, 18)
    blob[:, :, 2:] = 0x88
    blob[:, 3, 2] = 0x8F
    blob = blob.reshape(-1)
    x = make_x(1, K, rng_for(810, 1)) * np.float32(1e3)
    _, Y64, S = oracle.matmul(q.QMM_Q4_0, blob, M, K, x)
    check(gpu_gemv(q.QMM_Q4_0, to_dev(blob), M, K, x)[None, :], Y64, S, 1e-5, "sparse q4_0 rows")


def test_sparse_q4_1_rows_keep_f32_bound():
    # Q4_1 rows whose weights d*q + m are all exactly zero (m = -8d, nibble 8)
    # but one per block: the kernel must form each weight before it meets x
    M, K = 64, 4096
    blob = make_blob(q.QMM_Q4_1, M, K, rng_for(811, 0)).reshape(M, K // 32, 20)
    blob[:, :, 0:2] = np.frombuffer(np.float16(2.0 ** -6).tobytes(), np.uint8)
    blob[:, :, 2:4] = np.frombuffer(np.float16(-(2.0 ** -3)).tobytes(), np.uint8)
    blob[:, :, 4:20] = 0x88
    blob[:, :, 4 + 3] = 0x8F          # element 3 of every block: q = 15 -> 7d
    blob = blob.reshape(-1)
    x = make_x(1, K, rng_for(811, 1)) * np.float32(1000.0)
    _, Y64, S = oracle.matmul(q.QMM_Q4_1, blob, M, K, x)
    check(gpu_gemv(q.QMM_Q4_1, to_dev(blob), M, K, x)[None, :], Y64, S, 1e-5, "sparse q4_1 rows")


def test_streams_and_errors_on_device():
    M, K = 64, 256
    blob_d = to_dev(make_blob(q.QMM_Q4_K, M, K, rng_for(820, 0)))
    x = to_dev(make_x(1, K, rng_for(820, 1)).reshape(-1))
    y = torch.empty(M, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        q.qmm_gemv(blob_d, q.QMM_Q4_K, M, K, x, y, stream=s)
    s.synchronize()
    ref = torch.empty(M, device="cuda")
    q.qmm_gemv(blob_d, q.QMM_Q4_K, M, K, x, ref)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)
    # misaligned device pointers are refused before any launch
    with pytest.raises(q.QmmError) as e:
        q.qmm_gemv(blob_d.data_ptr() + 2, q.QMM_Q4_K, M, K, x, y)
    assert e.value.code == q.QMM_ERR_ALIGN


# ------------------------------------------------- full-size workloads ----

def sample_rows(M, n, seed):
    r = np.random.default_rng(seed).choice(M, size=min(n, M), replace=False)
    return np.unique(np.concatenate([r, [0, M - 1]]))


@pytest.mark.parametrize("wid", sorted(WORKLOADS))
def test_workload_full_size(wid):
    label, dt, M, K, ns = WORKLOADS[wid]
    blob = make_blob(dt, M, K, rng_for(wid, 0))
    blob_d = to_dev(blob)
    for N in ns:
        X = make_x(N, K, rng_for(wid, 1000 + N))
        # one token: every row (the C oracle takes about a second even for the
        # 128256-row head); several tokens: sampled rows
        rows = np.arange(M) if N == 1 else sample_rows(M, 96 if N <= 64 else 48, wid * 7919 + N)
        _, Y64, S = oracle.matmul(dt, blob, M, K, X, rows=rows)
        Yg = gpu_gemv(dt, blob_d, M, K, X)[None, :] if N == 1 else gpu_gemm(dt, blob_d, M, K, X)
        assert np.all(np.isfinite(Yg)), f"{label} N={N}: non-finite output"
        check(Yg[:, rows], Y64, S, q.tolerance(dt, M, K, N), f"{label} N={N}")
    del blob_d
    torch.cuda.empty_cache()


# ------------------------------------------------- few tokens, f32 path ----
#
# Below the crossover qmm_gemm gives every token the GEMV's f32 arithmetic:
# Y[n] must equal qmm_gemv(X[n]) bit for bit (several tokens share one weight
# read where K <= 4096), and lie within 1e-5 * S of the oracle.

def few_token_shapes(dt):
    if bs_of(dt) == 32:
        return [(1, 64), (67, 256), (1001, 1024), (300, 4096), (129, 8192)]
    return [(1, 256), (67, 512), (1001, 1024), (300, 4096), (129, 8192)]


@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
def test_gemm_few_tokens_match_gemv_bitwise(dt):
    for i, (M, K) in enumerate(few_token_shapes(dt)):
        blob = make_blob(dt, M, K, rng_for(640 + dt, i))
        bd = to_dev(blob)
        for N in range(2, 9):
            if q.gemm_path(dt, M, K, N) != 0:
                break
            X = make_x(N, K, rng_for(640 + dt, 100 * N + i))
            Yg = gpu_gemm(dt, bd, M, K, X)
            for n in range(N):
                yn = gpu_gemv(dt, bd, M, K, X[n])
                assert np.array_equal(Yg[n].view(np.uint32), yn.view(np.uint32)), \
                    f"{NAME[dt]} M={M} K={K} N={N}: token {n} differs from qmm_gemv"
            _, Y64, S = oracle.matmul(dt, blob, M, K, X)
            check(Yg, Y64, S, 1e-5, f"{NAME[dt]} few tokens M={M} K={K} N={N}")


def test_lm_head_verify_batch_matches_decode():
    """Verifying 4 drafted positions on the Q6_K LM head (128256 x 4096) gives
    each position exactly the logits greedy decoding computed."""
    dt, M, K, N = q.QMM_Q6_K, 128256, 4096, 4
    assert q.gemm_path(dt, M, K, N) == 0
    blob = make_blob(dt, M, K, rng_for(5, 0))
    bd = to_dev(blob)
    X = make_x(N, K, rng_for(5, 40))
    Yg = gpu_gemm(dt, bd, M, K, X)
    for n in range(N):
        assert np.array_equal(Yg[n].view(np.uint32), gpu_gemv(dt, bd, M, K, X[n]).view(np.uint32))
    rows = sample_rows(M, 256, 41)
    _, Y64, S = oracle.matmul(dt, blob, M, K, X, rows=rows)
    check(Yg[:, rows], Y64, S, 1e-5, "Q6_K LM head N=4")


@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
def test_gemm_skinny_two_fragments_ragged(dt):
    # N <= 32 on >= 192 two-fragment row tiles selects the split-K kernel with
    # two 32-row fragments per wavefront; M ends in a partial 64-row tile (and
    # a partial 32-row fragment), N in a partial token tile
    M, K, N = 12350, 1024, 17
    blob = make_blob(dt, M, K, rng_for(660 + dt, 0))
    X = make_x(N, K, rng_for(660 + dt, 1))
    rows = np.unique(np.concatenate([sample_rows(M, 40, 660 + dt), np.arange(M - 70, M)]))
    _, Y64, S = oracle.matmul(dt, blob, M, K, X, rows=rows)
    Yg = gpu_gemm(dt, to_dev(blob), M, K, X)
    assert np.all(np.isfinite(Yg))
    check(Yg[:, rows], Y64, S, q.tolerance(dt, M, K, N), f"{NAME[dt]} two-fragment skinny gemm M={M} K={K} N={N}")


@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
@pytest.mark.parametrize("N", [100, 130])
def test_gemm_skinny_64_token_tiles_ragged(dt, N):
    # 4000 rows: N = 100 selects split-K tiles of 32 rows x 64 tokens, N = 130
    # tiles of 64 rows x 64 tokens (one round of <= 256 workgroups each); M
    # and N end in partial tiles
    M, K = 4000, 1024
    blob = make_blob(dt, M, K, rng_for(670 + dt, N))
    X = make_x(N, K, rng_for(670 + dt, 1000 + N))
    rows = np.unique(np.concatenate([sample_rows(M, 40, 670 + dt + N), np.arange(M - 70, M)]))
    _, Y64, S = oracle.matmul(dt, blob, M, K, X, rows=rows)
    Yg = gpu_gemm(dt, to_dev(blob), M, K, X)
    assert np.all(np.isfinite(Yg))
    check(Yg[:, rows], Y64, S, q.tolerance(dt, M, K, N), f"{NAME[dt]} 64-token skinny gemm M={M} K={K} N={N}")


# --------------------------------------------------------- read ceiling ----

@pytest.mark.parametrize("nbytes", [16, 4096, 33030144, (1 << 31) + 4096])
def test_read_probe_reads_every_dword(nbytes):
    """qmm_read_probe (the bench's read ceiling) reads every dword once: the
    XOR of its per-workgroup folds is the XOR of the buffer's dwords."""
    rng = np.random.default_rng(nbytes % 1000)
    if nbytes > (1 << 30):
        buf = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda")
        host = buf.cpu().numpy().view(np.uint32)
        want = int(np.bitwise_xor.reduce(host))
    else:
        host = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint32)
        buf = torch.from_numpy(host.view(np.int32)).cuda()
        want = int(np.bitwise_xor.reduce(host))
    out = torch.zeros(q.QMM_READ_PROBE_OUT_FLOATS, device="cuda")
    q.qmm_read_probe(buf, nbytes, out)
    torch.cuda.synchronize()
    got = int(np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32)))
    assert got == want
