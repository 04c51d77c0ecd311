"""The int8-activation variant on the GPU against the CPU oracle, through the C ABI.

  * qmm_quantize_q8_0: scales and codes bit-identical to the oracle's
    quantizer (a floating-point decision that yields integers, taken in f32 on
    both sides): hand-derived blocks, special values (zeros, NaN, +-Inf,
    overflowing and subnormal scales, ties), random rows up to 512 x 14336.
  * qmm_gemm_q8act: |Y_gpu - Y_exact| <= 1e-5 * Splus per output, Y_exact the
    oracle's f64 sum over the dequantized codes and Splus = sum_k
    (|w - o| + |o|) |xq| (o the weight's offset part; Splus = S for Q8_0, Q4_0
    and Q6_K); the codes the GPU reads are the oracle's.  Small shapes with
    ragged M, odd block counts (the byte-load kernel), K beyond 4096 (the
    K-split workgroups), N from 1 to 9; full-size workloads on sampled rows.
  * Bitwise: a token of an N-token call equals the single-token call; two
    runs give equal bits.
  * The one-launch decode calls (qmm_gemv_q8act, qmm_gemv_concat_q8act,
    qmm_gemv_swiglu_q8act), which quantize x inside the launch: bit-identical
    to qmm_quantize_q8_0 + qmm_gemm_q8act (concat: to one call per matrix),
    and against the oracle within 1e-5 of Splus; the SwiGLU form within the
    SwiGLU bound carried from the int8 projections' bound.
"""
import numpy as np
import pytest
import torch

import gguf_block_quant_qmm_amd as q
import oracle
from qmm_inputs import WORKLOADS, make_blob, make_x, rng_for
from pins import load_q8_act_golden

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


def gpu_quantize(X):
    N, K = X.shape
    sc = torch.full((N, K // 32), float("nan"), device="cuda")
    qq = torch.full((N, K), 99, dtype=torch.int8, device="cuda")
    q.qmm_quantize_q8_0(to_dev(X), N, K, sc, qq)
    torch.cuda.synchronize()
    return sc.cpu().numpy(), qq.cpu().numpy()


def gpu_q8act(dt, blob_d, M, K, sc, qq):
    N = qq.shape[0]
    Y = torch.full((N, M), float("nan"), device="cuda")
    q.qmm_gemm_q8act(blob_d, dt, M, K, N, to_dev(sc), to_dev(qq), Y)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


def same_bits(a, b):
    return np.array_equal(np.asarray(a).view(np.uint32), np.asarray(b).view(np.uint32))


def check(Yg, Y64, Sp, label):
    assert Yg.shape == Y64.shape, label
    assert np.all(np.isfinite(Yg)), f"{label}: non-finite output"
    err = np.abs(Yg.astype(np.float64) - Y64)
    zero = Sp == 0
    assert np.all(Yg[zero] == 0), f"{label}: Splus = 0 but output is not exactly 0"
    if (~zero).any():
        ratio = err[~zero] / Sp[~zero]
        worst = int(np.argmax(ratio))
        assert ratio[worst] <= TAU, f"{label}: |err|/Splus = {ratio[worst]:.3g} > {TAU} at flat index {worst}"


# ------------------------------------------------------------ quantizer ----

def check_quantizer(X, label):
    s_o, q_o = oracle.quantize_q8_0(X)
    s_g, q_g = gpu_quantize(X)
    assert same_bits(s_g, s_o), f"{label}: scales differ at {np.argwhere(s_g.view(np.uint32) != s_o.view(np.uint32))[:4].tolist()}"
    bad = np.argwhere(q_g != q_o)
    assert bad.size == 0, f"{label}: codes differ at {bad[:4].tolist()}"


def test_quantizer_hand_derived_blocks():
    recs = load_q8_act_golden()
    X = np.stack([r[1] for r in recs])
    s_g, q_g = gpu_quantize(X)
    for i, (name, _, scale, codes) in enumerate(recs):
        assert s_g[i, 0] == scale or (scale != scale and s_g[i, 0] != s_g[i, 0]), name
        assert np.array_equal(q_g[i], codes), name
    check_quantizer(X, "golden blocks")


def test_quantizer_special_values():
    rng = rng_for(900, 0)
    rows = []
    base = rng.standard_normal(64).astype(np.float32)
    rows.append(np.zeros(64, np.float32))                               # d = 0: id = 0, all codes 0
    r = base.copy(); r[3] = np.nan; rows.append(r)                      # NaN skipped by amax, code 0
    r = base.copy(); r[40] = np.inf; rows.append(r)                     # amax = Inf: scale Inf, codes 0
    r = base.copy(); r[5] = -np.inf; r[6] = np.nan; rows.append(r)
    rows.append(base * np.float32(1e7))                                 # d > 65504: f16 scale Inf
    rows.append(base * np.float32(1e-39))                               # subnormal d: 1/d overflows, id = 0
    rows.append(base * np.float32(1e-30))                               # small normal d, f16 scale 0 or subnormal
    r = (np.arange(64, dtype=np.float32) - 31.5)                        # ties: k + 0.5 with d = 1
    r[0] = 127.0; r[32] = -127.0; rows.append(r.astype(np.float32))
    rows.append(np.full(64, -3.0e-5, np.float32))                       # f16-subnormal scale
    rows.append(np.float32(3.4e38) * np.sign(base).astype(np.float32))  # amax near f32 max
    check_quantizer(np.stack(rows).astype(np.float32), "special rows")


@pytest.mark.parametrize("N,K", [(1, 32), (3, 96), (7, 4096), (5, 14336), (512, 4096), (2, 65600)])
def test_quantizer_random(N, K):
    X = make_x(N, K, rng_for(901, N * 100000 + K))
    X[0, :32] *= np.float32(1e3)
    check_quantizer(X, f"N={N} K={K}")


# ------------------------------------------------------- int8 matmul ----

def shapes(dt):
    if bs_of(dt) == 32:
        # odd block count -> byte-load kernel; K > 4096 -> K-split workgroups;
        # K > 16384 -> byte-load kernel
        return [(1, 64), (3, 96), (67, 256), (300, 1024), (129, 4160), (50, 14336), (33, 16416)]
    return [(1, 256), (3, 512), (67, 768), (300, 2048), (50, 4096), (9, 16640)]


@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 9])
def test_q8act_small(dt, N):
    for i, (M, K) in enumerate(shapes(dt)):
        blob = make_blob(dt, M, K, rng_for(910 + dt, i))
        sc, qq = oracle.quantize_q8_0(make_x(N, K, rng_for(910 + dt, 100 * N + i)))
        _, Y64, _, Sp = oracle.matmul_q8act(dt, blob, M, K, sc, qq)
        Yg = gpu_q8act(dt, to_dev(blob), M, K, sc, qq)
        check(Yg, Y64, Sp, f"{NAME[dt]} q8act M={M} K={K} N={N}")


@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
def test_q8act_tokens_match_single_token_bitwise(dt):
    for i, (M, K) in enumerate([(301, 4 * bs_of(dt) * 4), (97, 8192 if bs_of(dt) == 256 else 4160)]):
        blob_d = to_dev(make_blob(dt, M, K, rng_for(920 + dt, i)))
        sc, qq = oracle.quantize_q8_0(make_x(7, K, rng_for(920 + dt, 10 + i)))
        Y = gpu_q8act(dt, blob_d, M, K, sc, qq)
        assert same_bits(Y, gpu_q8act(dt, blob_d, M, K, sc, qq)), f"{NAME[dt]}: two runs differ"
        for n in range(7):
            y1 = gpu_q8act(dt, blob_d, M, K, sc[n:n + 1], qq[n:n + 1])
            assert same_bits(Y[n:n + 1], y1), f"{NAME[dt]} M={M} K={K}: token {n} of 7 differs from its own call"


def test_q8act_planted_cancellation():
    # Q4_K rows whose weights are mostly the minimum term: the offset part is
    # taken through the code sums, so the bound is relative to Splus, and the
    # result must still meet it where S alone is much smaller
    dt, M, K = q.QMM_Q4_K, 64, 2048
    blob = make_blob(dt, M, K, rng_for(930, 0)).reshape(M, K // 256, 144)
    blob[:, :, 16:] = 0x11                     # every code 1: w = d*sc - dmin*m
    blob = blob.reshape(-1)
    sc, qq = oracle.quantize_q8_0(make_x(2, K, rng_for(930, 1)))
    _, Y64, S, Sp = oracle.matmul_q8act(dt, blob, M, K, sc, qq)
    Yg = gpu_q8act(dt, to_dev(blob), M, K, sc, qq)
    check(Yg, Y64, Sp, "Q4_K planted offsets")


def sample_rows(M, n, seed):
    rows = rng_for(940, seed).choice(M, size=min(n, M), replace=False)
    return np.unique(np.concatenate([rows, [0, M - 1]]))


@pytest.mark.parametrize("wid,N", [(1, 1), (2, 1), (3, 1), (4, 1), (5, 1), (5, 4), (6, 32), (8, 8), (10, 3)])
def test_q8act_full_size_workloads(wid, N):
    label, dt, M, K, _ = WORKLOADS[wid]
    blob = make_blob(dt, M, K, rng_for(wid, 0))
    X = make_x(N, K, rng_for(wid, 1000 + N))
    # the quantizer at full size, then the matmul on the oracle's codes
    check_quantizer(X, label)
    sc, qq = oracle.quantize_q8_0(X)
    rows = sample_rows(M, 96, wid * 10 + N)
    _, Y64, _, Sp = oracle.matmul_q8act(dt, blob, M, K, sc, qq, rows=rows)
    Yg = gpu_q8act(dt, to_dev(blob), M, K, sc, qq)
    assert np.all(np.isfinite(Yg)), label
    check(Yg[:, rows], Y64, Sp, f"{label} q8act N={N}")


def test_quantize_then_matmul_on_device():
    # the two entry points chained on device buffers, against the oracle's
    # quantizer and matmul end to end
    dt, M, K, N = q.QMM_Q6_K, 513, 4096, 3
    blob = make_blob(dt, M, K, rng_for(950, 0))
    X = make_x(N, K, rng_for(950, 1))
    sc_d = torch.empty((N, K // 32), device="cuda")
    qq_d = torch.empty((N, K), dtype=torch.int8, device="cuda")
    Y = torch.empty((N, M), device="cuda")
    q.qmm_quantize_q8_0(to_dev(X), N, K, sc_d, qq_d)
    q.qmm_gemm_q8act(to_dev(blob), dt, M, K, N, sc_d, qq_d, Y)
    torch.cuda.synchronize()
    sc, qq = oracle.quantize_q8_0(X)
    _, Y64, _, Sp = oracle.matmul_q8act(dt, blob, M, K, sc, qq)
    check(Y.cpu().numpy(), Y64, Sp, "quantize + q8act on device")


# ------------------------------------- one-launch decode (quantize inside) ----

def fused_shapes(dt):
    # K <= 4096: whole-row wavefronts; beyond: K-split workgroups (max 16384).
    # 1000 rows at K = 12288 or 14336 give the K-split workgroups several row
    # groups each (a ring), with x quantized once per workgroup; 2051 rows take
    # one-row groups (Q4_1)
    if bs_of(dt) == 32:
        return [(1, 64), (5, 128), (67, 1024), (300, 4096), (50, 4160), (33, 14336), (9, 16384), (1000, 14336),
                (2051, 14336)]
    # Q6_K needs an even super-block count per row
    return [(1, 512 if dt == q.QMM_Q6_K else 256), (3, 512), (67, 1024), (300, 4096), (50, 8192), (9, 16384),
            (1000, 12288 if dt == q.QMM_Q6_K else 14336)]


def test_gemv_q8act_rejects_odd_q6_k_blocks():
    blob_d = to_dev(make_blob(q.QMM_Q6_K, 4, 768, rng_for(965, 0)))
    x_d = to_dev(make_x(1, 768, rng_for(965, 1)).reshape(-1))
    with pytest.raises(q.QmmError) as e:
        one_launch(q.QMM_Q6_K, blob_d, 4, 768, x_d)
    assert e.value.code == q.QMM_ERR_SHAPE


def two_step(dt, blob_d, M, K, x_d):
    sc = torch.empty((1, K // 32), device="cuda")
    qq = torch.empty((1, K), dtype=torch.int8, device="cuda")
    y = torch.full((1, M), float("nan"), device="cuda")
    q.qmm_quantize_q8_0(x_d, 1, K, sc, qq)
    q.qmm_gemm_q8act(blob_d, dt, M, K, 1, sc, qq, y)
    torch.cuda.synchronize()
    return y.cpu().numpy()[0]


def one_launch(dt, blob_d, M, K, x_d):
    y = torch.full((M,), float("nan"), device="cuda")
    q.qmm_gemv_q8act(blob_d, dt, M, K, x_d, y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
def test_gemv_q8act_is_quantize_then_q8act(dt):
    for i, (M, K) in enumerate(fused_shapes(dt)):
        blob = make_blob(dt, M, K, rng_for(960 + dt, i))
        x = make_x(1, K, rng_for(960 + dt, 100 + i))
        x[0, :7] *= np.float32(50.0)  # a block with a larger maximum
        blob_d, x_d = to_dev(blob), to_dev(x.reshape(-1))
        y = one_launch(dt, blob_d, M, K, x_d)
        assert same_bits(y, two_step(dt, blob_d, M, K, x_d)), f"{NAME[dt]} M={M} K={K}: not the two-step bits"
        sc, qq = oracle.quantize_q8_0(x)
        _, Y64, _, Sp = oracle.matmul_q8act(dt, blob, M, K, sc, qq)
        check(y[None, :], Y64, Sp, f"{NAME[dt]} gemv_q8act M={M} K={K}")


def special_blocks(rng):
    # 32-activation blocks whose scales stay finite in f16: all zeros, a NaN
    # element (skipped by the maximum, code 0), a subnormal scale (1/d
    # overflows: codes 0), a tiny normal scale, rounding ties, an
    # f16-subnormal scale
    base = rng.standard_normal(32).astype(np.float32)
    out = [np.zeros(32, np.float32)]
    r = base.copy(); r[3] = np.nan; out.append(r)
    r = base.copy(); r[0] = np.nan; r[31] = np.nan; out.append(r)
    out.append(base * np.float32(1e-39))
    out.append(base * np.float32(1e-30))
    r = np.arange(32, dtype=np.float32) - np.float32(15.5); r[0] = 127.0; out.append(r)
    out.append(np.full(32, -3.0e-5, np.float32))
    return out


@pytest.mark.parametrize("dt", [q.QMM_Q4_0, q.QMM_Q8_0, q.QMM_Q4_K, q.QMM_Q6_K], ids=NAME.get)
def test_gemv_q8act_special_activations(dt):
    # special blocks spread over x so that they land in every lane of an
    # 8-lane block group and in every quantization round of a thread, for
    # whole-row wavefronts (K = 4096) and K-split workgroups (K = 16384): the
    # in-launch quantizer must give the standalone quantizer's bits
    for i, K in enumerate((4096, 16384)):
        M = 67
        rng = rng_for(990 + dt, i)
        blob = make_blob(dt, M, K, rng)
        x = make_x(1, K, rng_for(990 + dt, 10 + i)).reshape(-1)
        specials = special_blocks(rng)
        for j, b in enumerate(range(1, K // 32, 3)):
            x[32 * b:32 * b + 32] = specials[j % len(specials)]
        blob_d, x_d = to_dev(blob), to_dev(x)
        y = one_launch(dt, blob_d, M, K, x_d)
        assert np.all(np.isfinite(y)), f"{NAME[dt]} K={K}: non-finite output"
        assert same_bits(y, two_step(dt, blob_d, M, K, x_d)), f"{NAME[dt]} K={K}: not the two-step bits"
        sc, qq = oracle.quantize_q8_0(x.reshape(1, K))
        _, Y64, _, Sp = oracle.matmul_q8act(dt, blob, M, K, sc, qq)
        check(y[None, :], Y64, Sp, f"{NAME[dt]} gemv_q8act special K={K}")


@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
def test_gemv_concat_q8act(dt):
    K = 4 * bs_of(dt) * (4 if bs_of(dt) == 32 else 1)
    for K, Ms in ((K, [300, 77, 1]), (8192, [300, 77, 1]), (K, [300, 300]), (8192, [129, 129])):
        blobs = [to_dev(make_blob(dt, M, K, rng_for(970 + dt, j))) for j, M in enumerate(Ms)]
        x_d = to_dev(make_x(1, K, rng_for(970 + dt, 9)).reshape(-1))
        ys = [torch.full((M,), float("nan"), device="cuda") for M in Ms]
        q.qmm_gemv_concat_q8act(blobs, dt, Ms, K, x_d, ys)
        torch.cuda.synchronize()
        for j, (b, M, y) in enumerate(zip(blobs, Ms, ys)):
            assert same_bits(y.cpu().numpy(), one_launch(dt, b, M, K, x_d)), f"{NAME[dt]} K={K}: matrix {j}"


def check_swiglu_q8(out, g64, u64, sg, su, g_gpu, u_gpu, label):
    out = out.astype(np.float64)
    silu = np.vectorize(oracle.silu)
    exact = silu(g64) * u64
    with np.errstate(over="ignore"):
        silu_g = g64 / (1.0 + np.exp(-g64))
    bound = TAU * (1.1 * sg * (np.abs(u64) + TAU * su) + np.abs(silu_g) * su) + 4 * 2.0 ** -24 * np.abs(exact)
    assert np.all(np.isfinite(out)), f"{label}: non-finite output"
    zero = (sg == 0) | (su == 0)
    assert np.all(out[zero] == 0), f"{label}: a zero projection must give exactly 0"
    bad = np.abs(out - exact) > bound
    assert not bad.any(), f"{label}: {int(bad.sum())} outputs outside the bound"
    g2, u2 = g_gpu.astype(np.float64), u_gpu.astype(np.float64)
    with np.errstate(over="ignore"):
        mine = g2 / (1.0 + np.exp(-g2)) * u2
    lim = 4 * 2.0 ** -24 * np.abs(mine) + 2.0 ** -119 * np.abs(u2)
    assert np.all(np.abs(out - mine) <= lim), f"{label}: not silu(g) * u of the int8 projections"


@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
def test_gemv_swiglu_q8act(dt):
    for i, (M, K) in enumerate([(300, 1024 if bs_of(dt) == 32 else 2048), (67, 8192)]):
        gate = make_blob(dt, M, K, rng_for(980 + dt, i))
        up = make_blob(dt, M, K, rng_for(980 + dt, 10 + i))
        x = make_x(1, K, rng_for(980 + dt, 20 + i)) * np.float32(2.0)
        g_d, u_d, x_d = to_dev(gate), to_dev(up), to_dev(x.reshape(-1))
        out = torch.full((M,), float("nan"), device="cuda")
        q.qmm_gemv_swiglu_q8act(g_d, u_d, dt, M, K, x_d, out)
        torch.cuda.synchronize()
        sc, qq = oracle.quantize_q8_0(x)
        _, G64, _, SG = oracle.matmul_q8act(dt, gate, M, K, sc, qq)
        _, U64, _, SU = oracle.matmul_q8act(dt, up, M, K, sc, qq)
        check_swiglu_q8(out.cpu().numpy(), G64[0], U64[0], SG[0], SU[0], one_launch(dt, g_d, M, K, x_d),
                        one_launch(dt, u_d, M, K, x_d), f"{NAME[dt]} swiglu_q8act M={M} K={K}")


def test_one_launch_decode_layer_full_size():
    # the llama8b Q4_0 decode layer as the bench runs it, and the Q6_K head
    for wid, sub in ((2, None), (3, None), (4, None), (5, None)):
        label, dt, M, K, _ = WORKLOADS[wid]
        blob = make_blob(dt, M, K, rng_for(wid, 0))
        x = make_x(1, K, rng_for(wid, 1001))
        blob_d, x_d = to_dev(blob), to_dev(x.reshape(-1))
        y = one_launch(dt, blob_d, M, K, x_d)
        assert same_bits(y, two_step(dt, blob_d, M, K, x_d)), f"{label}: not the two-step bits"
        sc, qq = oracle.quantize_q8_0(x)
        rows = sample_rows(M, 64, wid)
        _, Y64, _, Sp = oracle.matmul_q8act(dt, blob, M, K, sc, qq, rows=rows)
        check(y[None, rows], Y64, Sp, f"{label} gemv_q8act")
    # gate + up in one launch
    _, dt, M, K, _ = WORKLOADS[3]
    blobs = [to_dev(make_blob(dt, M, K, rng_for(3, j))) for j in range(2)]
    x_d = to_dev(make_x(1, K, rng_for(3, 1001)).reshape(-1))
    ys = [torch.empty(M, device="cuda") for _ in range(2)]
    q.qmm_gemv_concat_q8act(blobs, dt, [M, M], K, x_d, ys)
    torch.cuda.synchronize()
    for b, y in zip(blobs, ys):
        assert same_bits(y.cpu().numpy(), one_launch(dt, b, M, K, x_d)), "gate+up concat q8act"


def run_argmax_q8(dt, blob_d, M, K, x_d):
    work = torch.empty(q.QMM_ARGMAX_WORK_BYTES, dtype=torch.uint8, device="cuda")
    idx = torch.full((1,), -7, dtype=torch.int64, device="cuda")
    val = torch.full((1,), float("nan"), device="cuda")
    q.qmm_gemv_argmax_q8act(blob_d, dt, M, K, x_d, work, idx, val)
    torch.cuda.synchronize()
    return int(idx.item()), float(val.item())


@pytest.mark.parametrize("dt", DTYPES, ids=NAME.get)
def test_gemv_argmax_q8act(dt):
    for i, (M, K) in enumerate([(1, 512), (777, 1024), (300, 8192), (5000, 4096)]):
        blob = make_blob(dt, M, K, rng_for(990 + dt, i))
        x = make_x(1, K, rng_for(990 + dt, 10 + i))
        blob_d, x_d = to_dev(blob), to_dev(x.reshape(-1))
        y = one_launch(dt, blob_d, M, K, x_d)
        idx, val = run_argmax_q8(dt, blob_d, M, K, x_d)
        first = int(np.flatnonzero(y == y.max())[0])
        assert idx == first and val == y[first], f"{NAME[dt]} M={M} K={K}: argmax {idx} vs {first}"
        # against the exact int8 logits: the pick is a maximum within the bound
        sc, qq = oracle.quantize_q8_0(x)
        _, Y64, _, Sp = oracle.matmul_q8act(dt, blob, M, K, sc, qq)
        best = int(np.argmax(Y64[0]))
        assert Y64[0, idx] >= Y64[0, best] - TAU * (Sp[0, idx] + Sp[0, best]), f"{NAME[dt]}: not a maximum"
        if M > 1 and first > 0:
            # plant a tie: an earlier row becomes a copy of the winner
            rb = blob.size // M
            tied = blob.copy()
            tied[(first - 1) * rb:first * rb] = blob[first * rb:(first + 1) * rb]
            idx2, _ = run_argmax_q8(dt, to_dev(tied), M, K, x_d)
            assert idx2 == first - 1, f"{NAME[dt]}: a tie must go to the smaller row"


def test_gemv_argmax_q8act_lm_head():
    label, dt, M, K, _ = WORKLOADS[5]
    blob = make_blob(dt, M, K, rng_for(5, 0))
    x = make_x(1, K, rng_for(5, 1001))
    blob_d, x_d = to_dev(blob), to_dev(x.reshape(-1))
    y = one_launch(dt, blob_d, M, K, x_d)
    idx, val = run_argmax_q8(dt, blob_d, M, K, x_d)
    first = int(np.flatnonzero(y == y.max())[0])
    assert idx == first and val == y[first], f"{label}: argmax {idx} vs {first}"


@pytest.mark.parametrize("dt", [q.QMM_Q4_0, q.QMM_Q6_K, q.QMM_Q4_K], ids=NAME.get)
def test_q8act_many_tokens(dt):
    # 600 tokens = 150 token groups of 4 on the fast kernel (the last group
    # full), and 600 grid rows on the byte-load kernel (odd block count)
    for i, (M, K) in enumerate([(130, 4 * bs_of(dt) * (4 if bs_of(dt) == 32 else 1)),
                                (70, 3 * bs_of(dt))]):
        N = 600
        blob = make_blob(dt, M, K, rng_for(995 + dt, i))
        sc, qq = oracle.quantize_q8_0(make_x(N, K, rng_for(995 + dt, 10 + i)))
        _, Y64, _, Sp = oracle.matmul_q8act(dt, blob, M, K, sc, qq)
        Yg = gpu_q8act(dt, to_dev(blob), M, K, sc, qq)
        check(Yg, Y64, Sp, f"{NAME[dt]} q8act M={M} K={K} N={N}")


# ------------------------------------------------- int8 matrix cores ----
#
# From N = 32 tokens (large enough grids), Q8_0, Q4_0 and Q4_K run on the int8 matrix cores: one
# 32-deep integer step per activation block, the block sums scaled once in f32
# and summed in two levels (bound 1e-5 * Splus, as the few-token kernels).

MFMA_I8 = [q.QMM_Q8_0, q.QMM_Q4_0, q.QMM_Q4_K]


def i8_shapes(dt):
    # ragged M (partial 32-row fragments and 256-row workgroups) tall enough
    # for the matrix cores, K from one k-tile up to 16384 (the longest
    # two-level sum)
    if bs_of(dt) == 32:
        return [(14337, 64), (14401, 1024), (14433, 4160), (14339, 16384)]
    return [(14337, 256), (14401, 1024), (14433, 4352), (14339, 16384)]


@pytest.mark.parametrize("dt", MFMA_I8, ids=NAME.get)
@pytest.mark.parametrize("N", [40, 65, 130])
def test_q8act_matrix_cores(dt, N):
    for i, (M, K) in enumerate(i8_shapes(dt)):
        blob = make_blob(dt, M, K, rng_for(1500 + dt, i), q8_full_range=True)
        sc, qq = oracle.quantize_q8_0(make_x(N, K, rng_for(1500 + dt, 100 * N + i)))
        assert q.q8act_kernel(dt, M, K, N) == 1, "shape not on the matrix cores"
        rows = np.unique(np.concatenate([sample_rows(M, 60, 1501 + i), M - 1 - np.arange(33)]))
        _, Y64, _, Sp = oracle.matmul_q8act(dt, blob, M, K, sc, qq, rows=rows)
        Yg = gpu_q8act(dt, to_dev(blob), M, K, sc, qq)
        assert np.all(np.isfinite(Yg))
        check(Yg[:, rows], Y64, Sp, f"{NAME[dt]} int8 matrix cores M={M} K={K} N={N}")


@pytest.mark.parametrize("dt", MFMA_I8, ids=NAME.get)
def test_q8act_matrix_cores_deterministic_and_cancelling(dt):
    M, K, N = 16129, 2048, 40
    assert q.q8act_kernel(dt, M, K, N) == 1
    blob = make_blob(dt, M, K, rng_for(1510 + dt, 0))
    if dt == q.QMM_Q4_K:
        b = blob.reshape(M, K // 256, 144)
        b[::3, :, 16:] = 0x11          # rows whose weights are mostly the minimum term
        blob = b.reshape(-1)
    elif dt == q.QMM_Q4_0:
        b = blob.reshape(M, K // 32, 18)
        b[::3, :, 2:] = 0x88           # every code 8: w = 0, S = 0, exact zeros required
        blob = b.reshape(-1)
    sc, qq = oracle.quantize_q8_0(make_x(N, K, rng_for(1510 + dt, 1)))
    rows = np.unique(np.concatenate([np.arange(0, 600), M - 1 - np.arange(40)]))
    _, Y64, _, Sp = oracle.matmul_q8act(dt, blob, M, K, sc, qq, rows=rows)
    bd = to_dev(blob)
    Y1 = gpu_q8act(dt, bd, M, K, sc, qq)
    Y2 = gpu_q8act(dt, bd, M, K, sc, qq)
    assert same_bits(Y1, Y2), f"{NAME[dt]}: two runs differ"
    check(Y1[:, rows], Y64, Sp, f"{NAME[dt]} int8 matrix cores, planted rows")


def test_q8act_matrix_cores_full_size_n512():
    """The Q4_K 14336 x 4096 prefill shape at N = 512, sampled rows."""
    dt, M, K, N = q.QMM_Q4_K, 14336, 4096, 512
    blob = make_blob(dt, M, K, rng_for(6, 0))
    sc, qq = oracle.quantize_q8_0(make_x(N, K, rng_for(6, 1512)))
    rows = sample_rows(M, 48, 1520)
    _, Y64, _, Sp = oracle.matmul_q8act(dt, blob, M, K, sc, qq, rows=rows)
    Yg = gpu_q8act(dt, to_dev(blob), M, K, sc, qq)
    assert np.all(np.isfinite(Yg))
    check(Yg[:, rows], Y64, Sp, "Q4_K 14336x4096 N=512 int8 matrix cores")
