"""Checks that pin the CPU oracle to something other than itself.

Each ``pin_*`` function takes an oracle library handle (``None`` = the normal
build) and raises AssertionError on a mismatch, so that the same checks can
run against deliberately broken builds of the oracle (test_oracle_mutants).

  pin_golden          hand-built blocks with design values (tests/golden/)
  pin_unit_vectors    x = e_k on small blobs made of those blocks: y = W[:, k]
  pin_closed_form     x = all ones: y = dequantized row sums, computed from
                      the block fields with integer sums (no element placement)
  pin_bruteforce      tiny random shapes against an exact rational result
                      from a separately written decoder (fractions.Fraction)
  pin_invariants      GEMM column == GEMV, 2x scales -> 2x output, row
                      permutation, power-of-two scaling of x, additivity
  pin_half            f16 decoding against Python's own binary16 unpacking
  pin_sizes           block sizes and the page's ~205 MiB Q6_K head
  pin_silu            SiLU at closed-form points (sigmoid(ln 3) = 3/4, the
                      minimum -W(1/e)), the odd-part identity and its limits
  pin_swiglu          gate/up SwiGLU on fixture blocks with unit vectors:
                      g and u are the fixtures' design values, out = silu(g) u
  pin_argmax          greedy argmax on fixture blocks with unit vectors (the
                      design values pick the winner), planted ties and a
                      planted maximum in the last row
  pin_q8_act_golden   the Q8_0 activation quantizer on hand-derived blocks
                      (tests/golden/q8_0_act.txt): ties to even, the f16
                      scale, the zero / NaN / Inf / subnormal guards
  pin_float_to_half   f32 -> f16 rounding against numpy's conversion
  pin_q8_act_bound    quantizer closed-form error bound, block maximum -> 127,
                      sign and power-of-two symmetry
  pin_q8_matmul       weights x quantized activations: exact rational brute
                      force (with the offset-term scale), all-ones closed
                      form, one scaled block, token and row placement
"""
from __future__ import annotations

import math
import os
import struct
from fractions import Fraction

import numpy as np

import oracle
from qmm_inputs import make_blob, make_x, rng_for

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
DTYPES = (oracle.Q4_0, oracle.Q8_0, oracle.Q4_K, oracle.Q6_K, oracle.Q4_1, oracle.Q5_K)


# ----------------------------------------------------------------- fixtures

def _expand(tokens, conv):
    out = []
    for t in tokens:
        if "*" in t:
            v, n = t.split("*")
            out += [conv(v)] * int(n)
        else:
            out.append(conv(t))
    return out


def _num(s: str) -> float:
    s = s.strip()
    if s.lstrip("-").startswith("0x"):
        return float.fromhex(s)
    return float(s)


def load_golden(dtype_name: str):
    """[(record name, block bytes, expected weights)] from tests/golden/<dtype>_blocks.txt."""
    path = os.path.join(GOLDEN, f"{dtype_name.lower()}_blocks.txt")
    recs, cur, key = [], None, None
    with open(path) as f:
        for raw in f:
            line = raw.rstrip("\n")
            if not line.strip() or line.lstrip().startswith("#"):
                continue
            if line.startswith("["):
                cur = {"name": line.strip("[] "), "block": [], "expect": []}
                recs.append(cur)
                continue
            if line.startswith("block:"):
                key, line = "block", line[len("block:"):]
            elif line.startswith("expect:"):
                key, line = "expect", line[len("expect:"):]
            cur[key] += line.split()
    out = []
    for r in recs:
        blk = bytes(_expand(r["block"], lambda s: int(s, 16)))
        exp = np.array(_expand(r["expect"], _num), dtype=np.float64)
        out.append((r["name"], blk, exp))
    return out


def pin_golden(L=None):
    for dt in DTYPES:
        name = oracle.NAMES[dt]
        recs = load_golden(name)
        assert recs, f"no fixtures for {name}"
        for rname, blk, exp in recs:
            bs, bb = oracle.block_elems(dt, L), oracle.block_bytes(dt, L)
            assert len(blk) == bb, f"{rname}: fixture block is {len(blk)} bytes, format says {bb}"
            assert exp.size == bs, f"{rname}: {exp.size} expected values for a {bs}-weight block"
            W = oracle.dequant(dt, np.frombuffer(blk, np.uint8), 1, bs, L=L)[0]
            bad = np.nonzero(W != exp)[0]
            assert bad.size == 0, f"{rname}: weight {bad[0]} decodes to {W[bad[0]]}, design value {exp[bad[0]]}"


def pin_unit_vectors(L=None):
    """Blobs of 3 rows made of the fixture blocks in rotated order; X = I_K."""
    for dt in DTYPES:
        recs = load_golden(oracle.NAMES[dt])
        bs = oracle.block_elems(dt, L)
        nblk = 2 if bs == 256 else 4                       # K = 512 or 128
        K, M = nblk * bs, 3
        rows_b, rows_w = [], []
        for m in range(M):
            pick = [recs[(m + b) % len(recs)] for b in range(nblk)]
            rows_b.append(b"".join(p[1] for p in pick))
            rows_w.append(np.concatenate([p[2] for p in pick]))
        blob = np.frombuffer(b"".join(rows_b), np.uint8)
        W = np.stack(rows_w)
        Y, _, _ = oracle.matmul(dt, blob, M, K, np.eye(K, dtype=np.float32), L=L)
        assert Y.shape == (K, M)
        bad = np.argwhere(Y.T != W.astype(np.float32))
        assert bad.size == 0, f"{oracle.NAMES[dt]}: y[{bad[0][0]}] for x = e_{bad[0][1]} is wrong"


# --------------------------------------------------------------- closed form

def _f16(a: np.ndarray) -> np.ndarray:
    return a.copy().view("<f2").astype(np.float64).reshape(-1)


def closed_form_row_sums(dt: int, blob: np.ndarray, M: int, K: int) -> np.ndarray:
    """y = W . ones, from the block fields: scale x (sum of integer codes)."""
    bs, bb = {oracle.Q4_0: (32, 18), oracle.Q4_1: (32, 20), oracle.Q8_0: (32, 34),
              oracle.Q4_K: (256, 144), oracle.Q5_K: (256, 176), oracle.Q6_K: (256, 210)}[dt]
    nb = K // bs
    B = blob[: M * nb * bb].reshape(M, nb, bb)
    if dt == oracle.Q8_0:
        d = _f16(np.ascontiguousarray(B[:, :, 0:2])).reshape(M, nb)
        qsum = B[:, :, 2:34].view(np.int8).astype(np.int64).sum(axis=2)
        per_block = d * qsum
    elif dt == oracle.Q4_0:
        d = _f16(np.ascontiguousarray(B[:, :, 0:2])).reshape(M, nb)
        qs = B[:, :, 2:18].astype(np.int64)
        qsum = (qs & 15).sum(axis=2) + (qs >> 4).sum(axis=2)
        per_block = d * (qsum - 8 * 32)
    elif dt == oracle.Q4_1:
        d = _f16(np.ascontiguousarray(B[:, :, 0:2])).reshape(M, nb)
        m = _f16(np.ascontiguousarray(B[:, :, 2:4])).reshape(M, nb)
        qs = B[:, :, 4:20].astype(np.int64)
        qsum = (qs & 15).sum(axis=2) + (qs >> 4).sum(axis=2)
        per_block = d * qsum + 32 * m
    elif dt == oracle.Q4_K:
        d = _f16(np.ascontiguousarray(B[:, :, 0:2])).reshape(M, nb)
        dmin = _f16(np.ascontiguousarray(B[:, :, 2:4])).reshape(M, nb)
        s = B[:, :, 4:16].astype(np.int64)
        sc = np.empty((M, nb, 8), np.int64)
        mn = np.empty((M, nb, 8), np.int64)
        sc[:, :, 0:4] = s[:, :, 0:4] & 63
        mn[:, :, 0:4] = s[:, :, 4:8] & 63
        sc[:, :, 4:8] = (s[:, :, 8:12] & 15) | ((s[:, :, 0:4] >> 6) << 4)
        mn[:, :, 4:8] = (s[:, :, 8:12] >> 4) | ((s[:, :, 4:8] >> 6) << 4)
        chunks = B[:, :, 16:144].astype(np.int64).reshape(M, nb, 4, 32)
        qsum = np.empty((M, nb, 8), np.int64)
        qsum[:, :, 0::2] = (chunks & 15).sum(axis=3)       # even sub-blocks: low nibbles
        qsum[:, :, 1::2] = (chunks >> 4).sum(axis=3)       # odd sub-blocks: high nibbles
        per_block = (d[:, :, None] * sc * qsum - 32 * dmin[:, :, None] * mn).sum(axis=2)
    elif dt == oracle.Q5_K:
        d = _f16(np.ascontiguousarray(B[:, :, 0:2])).reshape(M, nb)
        dmin = _f16(np.ascontiguousarray(B[:, :, 2:4])).reshape(M, nb)
        s = B[:, :, 4:16].astype(np.int64)
        sc = np.empty((M, nb, 8), np.int64)
        mn = np.empty((M, nb, 8), np.int64)
        sc[:, :, 0:4] = s[:, :, 0:4] & 63
        mn[:, :, 0:4] = s[:, :, 4:8] & 63
        sc[:, :, 4:8] = (s[:, :, 8:12] & 15) | ((s[:, :, 0:4] >> 6) << 4)
        mn[:, :, 4:8] = (s[:, :, 8:12] >> 4) | ((s[:, :, 4:8] >> 6) << 4)
        qh = B[:, :, 16:48].astype(np.int64)                       # [e]
        chunks = B[:, :, 48:176].astype(np.int64).reshape(M, nb, 4, 32)
        qsum = np.empty((M, nb, 8), np.int64)
        for i in range(8):
            nib = (chunks[:, :, i // 2] & 15) if i % 2 == 0 else (chunks[:, :, i // 2] >> 4)
            qsum[:, :, i] = nib.sum(axis=2) + 16 * ((qh >> i) & 1).sum(axis=2)
        per_block = (d[:, :, None] * sc * qsum - 32 * dmin[:, :, None] * mn).sum(axis=2)
    elif dt == oracle.Q6_K:
        ql = B[:, :, 0:128].astype(np.int64).reshape(M, nb, 2, 2, 32)     # [h][c][l]
        qh = B[:, :, 128:192].astype(np.int64).reshape(M, nb, 2, 32)      # [h][l]
        sc = B[:, :, 192:208].view(np.int8).astype(np.int64).reshape(M, nb, 2, 4, 2)  # [h][g][l/16]
        d = _f16(np.ascontiguousarray(B[:, :, 208:210])).reshape(M, nb)
        lo = np.stack([ql[:, :, :, 0] & 15, ql[:, :, :, 1] & 15,
                       ql[:, :, :, 0] >> 4, ql[:, :, :, 1] >> 4], axis=3)  # [h][g][l]
        hi = np.stack([(qh >> (2 * g)) & 3 for g in range(4)], axis=3)   # [h][g][l]
        q = (lo + 16 * hi).reshape(M, nb, 2, 4, 2, 16).sum(axis=5)        # per 16-group
        per_block = d * (sc * (q - 32 * 16)).sum(axis=(2, 3, 4))
    else:
        raise ValueError(dt)
    out = np.zeros(M, np.float64)
    for b in range(nb):            # block terms are exact multiples of 2^-24: any order is exact
        out += per_block[:, b]
    return out


def pin_closed_form(L=None):
    for i, dt in enumerate(DTYPES):
        bs = oracle.block_elems(dt, L)
        M, K = 37, 8 * bs
        blob = make_blob(dt, M, K, rng_for(900 + i, 0))
        _, Y64, _ = oracle.matmul(dt, blob, M, K, np.ones((1, K), np.float32), L=L)
        ref = closed_form_row_sums(dt, blob, M, K)
        bad = np.nonzero(Y64[0] != ref)[0]
        assert bad.size == 0, (f"{oracle.NAMES[dt]}: row {bad[0]} sum {Y64[0][bad[0]]!r} != "
                               f"closed form {ref[bad[0]]!r}")


# ---------------------------------------------------------------- brute force

def _h(b: bytes, off: int) -> Fraction:
    return Fraction(struct.unpack("<e", b[off:off + 2])[0])


def exact_weights(dt: int, blk: bytes) -> list:
    """One block -> its weights as exact rationals; written independently of oracle.c."""
    if dt == oracle.Q8_0:
        d = _h(blk, 0)
        return [d * v for v in struct.unpack("<32b", blk[2:34])]
    if dt == oracle.Q4_0:
        d = _h(blk, 0)
        lows = [(c & 0x0F) - 8 for c in blk[2:18]]
        highs = [(c >> 4) - 8 for c in blk[2:18]]
        return [d * v for v in lows + highs]
    if dt == oracle.Q4_1:
        d, m = _h(blk, 0), _h(blk, 2)
        return [d * (c & 0x0F) + m for c in blk[4:20]] + [d * (c >> 4) + m for c in blk[4:20]]
    if dt == oracle.Q4_K:
        d, dmin = _h(blk, 0), _h(blk, 2)
        s = blk[4:16]
        sc, mn = [], []
        for i in range(8):
            if i < 4:
                sc.append(s[i] % 64)
                mn.append(s[i + 4] % 64)
            else:
                sc.append(s[i + 4] % 16 + 16 * (s[i - 4] // 64))
                mn.append(s[i + 4] // 16 + 16 * (s[i] // 64))
        w = []
        for i in range(8):
            chunk = blk[16 + 32 * (i // 2): 16 + 32 * (i // 2) + 32]
            for c in chunk:
                q = c % 16 if i % 2 == 0 else c // 16
                w.append(d * sc[i] * q - dmin * mn[i])
        return w
    if dt == oracle.Q5_K:
        d, dmin = _h(blk, 0), _h(blk, 2)
        s, qh, qs = blk[4:16], blk[16:48], blk[48:176]
        w = []
        for i in range(8):
            if i < 4:
                sc, mn = s[i] % 64, s[i + 4] % 64
            else:
                sc = s[i + 4] % 16 + 16 * (s[i - 4] // 64)
                mn = s[i + 4] // 16 + 16 * (s[i] // 64)
            for e in range(32):
                byte = qs[32 * (i // 2) + e]
                q = (byte % 16 if i % 2 == 0 else byte // 16) + 16 * ((qh[e] >> i) & 1)
                w.append(d * sc * q - dmin * mn)
        return w
    if dt == oracle.Q6_K:
        ql, qh = blk[0:128], blk[128:192]
        sc = struct.unpack("<16b", blk[192:208])
        d = _h(blk, 208)
        w = [None] * 256
        for h in range(2):
            for g in range(4):
                for l in range(32):
                    byte = ql[64 * h + 32 * (g % 2) + l]
                    lo = byte % 16 if g < 2 else byte // 16
                    hi = (qh[32 * h + l] // (4 ** g)) % 4
                    j = 128 * h + 32 * g + l
                    w[j] = d * sc[j // 16] * (lo + 16 * hi - 32)
        return w
    raise ValueError(dt)


def round_f32(v: Fraction) -> np.float32:
    """Correctly rounded (nearest, ties to even) f32 of an exact rational."""
    f = np.float32(float(v))
    cands = {f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))}
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - v),
                                     int(np.array(c, np.float32).view(np.uint32)) & 1))
    return np.float32(best)


def pin_bruteforce(L=None):
    shapes = [(1, 1), (3, 2), (5, 4), (8, 3)]
    for i, dt in enumerate(DTYPES):
        bs, bb = oracle.block_elems(dt, L), oracle.block_bytes(dt, L)
        for j, (M, N) in enumerate(shapes):
            K = 2 * bs if bs == 256 else 8 * bs
            blob = make_blob(dt, M, K, rng_for(950 + i, j))
            X = make_x(N, K, rng_for(950 + i, 100 + j))
            Y, Y64, S = oracle.matmul(dt, blob, M, K, X, L=L)
            raw = blob.tobytes()
            nb = K // bs
            for m in range(M):
                w = []
                for b in range(nb):
                    off = (m * nb + b) * bb
                    w += exact_weights(dt, raw[off:off + bb])
                for n in range(N):
                    xs = [Fraction(float(v)) for v in X[n]]
                    exact = sum((wk * xk for wk, xk in zip(w, xs)), Fraction(0))
                    mag = sum((abs(wk * xk) for wk, xk in zip(w, xs)), Fraction(0))
                    bound = Fraction(K) * Fraction(2) ** -53 * mag
                    err = abs(Fraction(float(Y64[n, m])) - exact)
                    assert err <= bound, (f"{oracle.NAMES[dt]} M={M} N={N}: y[{n},{m}] f64 off by "
                                          f"{float(err):.3g} > {float(bound):.3g}")
                    assert abs(Fraction(float(S[n, m])) - mag) <= bound, "S is not sum |w x|"
                    want = round_f32(exact)
                    if Y[n, m] != want:
                        # allowed only when the exact value sits within the f64 bound of a tie
                        lo = min(Y[n, m], want)
                        mid = (Fraction(float(lo)) + Fraction(float(max(Y[n, m], want)))) / 2
                        assert abs(mid - exact) <= bound, (f"{oracle.NAMES[dt]}: y[{n},{m}] = {Y[n, m]!r}, "
                                                           f"correctly rounded {want!r}")


# ---------------------------------------------------------------- invariants

def _double_scales(dt: int, blob: np.ndarray, M: int, K: int) -> np.ndarray:
    """Blob with every f16 scale (d, and dmin for Q4_K) multiplied by 2."""
    bs, bb = {oracle.Q4_0: (32, 18), oracle.Q4_1: (32, 20), oracle.Q8_0: (32, 34),
              oracle.Q4_K: (256, 144), oracle.Q5_K: (256, 176), oracle.Q6_K: (256, 210)}[dt]
    B = blob.copy().reshape(-1, bb)
    offs = {oracle.Q4_0: [0], oracle.Q4_1: [0, 2], oracle.Q8_0: [0], oracle.Q4_K: [0, 2], oracle.Q5_K: [0, 2],
            oracle.Q6_K: [208]}[dt]
    for o in offs:
        h = np.ascontiguousarray(B[:, o:o + 2]).view("<f2").reshape(-1)
        h2 = (h.astype(np.float32) * 2).astype("<f2")
        assert np.all(h2.astype(np.float64) == 2 * h.astype(np.float64)), "doubling must stay exact"
        B[:, o:o + 2] = h2.view(np.uint8).reshape(-1, 2)
    return B.reshape(-1)


def pin_invariants(L=None):
    for i, dt in enumerate(DTYPES):
        bs = oracle.block_elems(dt, L)
        M, K, N = 11, 4 * bs, 5
        blob = make_blob(dt, M, K, rng_for(970 + i, 0))
        X = make_x(N, K, rng_for(970 + i, 1))
        Y, Y64, S = oracle.matmul(dt, blob, M, K, X, L=L)
        name = oracle.NAMES[dt]
        # GEMM column n is the GEMV on X[n]
        for n in range(N):
            y1, y164, _ = oracle.matmul(dt, blob, M, K, X[n], L=L)
            assert np.array_equal(y164[0], Y64[n]), f"{name}: GEMM column {n} != GEMV"
        # doubling every scale doubles y exactly
        _, Yd, _ = oracle.matmul(dt, _double_scales(dt, blob, M, K), M, K, X, L=L)
        assert np.array_equal(Yd, 2 * Y64), f"{name}: 2x scales did not give 2x output"
        # power-of-two scaling of x is exact
        _, Yx, _ = oracle.matmul(dt, blob, M, K, X * np.float32(0.25), L=L)
        assert np.array_equal(Yx, 0.25 * Y64), f"{name}: y(x/4) != y(x)/4"
        # additivity within the f64 bound
        X2 = make_x(N, K, rng_for(970 + i, 2))
        _, Ya, Sa = oracle.matmul(dt, blob, M, K, X2, L=L)
        _, Ys, _ = oracle.matmul(dt, blob, M, K, (X.astype(np.float64) + X2).astype(np.float32), L=L)
        Xs = (X.astype(np.float64) + X2).astype(np.float32)
        rnd = Xs.astype(np.float64) - (X.astype(np.float64) + X2)       # rounding of the sum
        assert np.all(np.abs(rnd) <= np.abs(Xs) * 2.0 ** -24)
        # |y(X1+X2) - y(X1) - y(X2)| <= |W| |rnd| + f64 error
        Wabs = np.abs(oracle.dequant(dt, blob, M, K, L=L))
        lim = (np.abs(rnd) @ Wabs.T) + 4 * K * 2.0 ** -53 * (S + Sa + (np.abs(Xs) @ Wabs.T))
        assert np.all(np.abs(Ys - Y64 - Ya) <= lim), f"{name}: not additive in x"
        # permuting rows of the blob permutes y
        bb = oracle.block_bytes(dt, L)
        perm = np.random.default_rng(7).permutation(M)
        pblob = blob.reshape(M, -1)[perm].reshape(-1)
        assert pblob.size == M * (K // bs) * bb
        _, Yp, _ = oracle.matmul(dt, pblob, M, K, X, L=L)
        assert np.array_equal(Yp, Y64[:, perm]), f"{name}: row permutation not followed"
        # row subsets give the same numbers as the full call
        rows = [M - 1, 0, 5]
        _, Yr, _ = oracle.matmul(dt, blob, M, K, X, rows=rows, L=L)
        assert np.array_equal(Yr, Y64[:, rows]), f"{name}: row-subset call differs"


def pin_half(L=None):
    for h in list(range(0, 0x10000, 97)) + [0x0000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF,
                                              0x8000, 0x8001, 0xC000, 0xFBFF, 0x7C00, 0xFC00]:
        want = struct.unpack("<e", struct.pack("<H", h))[0]
        got = oracle.half_to_double(h, L)
        if want != want:
            assert got != got, f"f16 {h:#06x} should be NaN"
        else:
            assert got == want and np.signbit(got) == np.signbit(want), f"f16 {h:#06x}: {got!r} != {want!r}"


def pin_sizes(L=None):
    assert [oracle.block_bytes(d, L) for d in DTYPES] == [18, 34, 144, 210, 20, 176]
    assert [oracle.block_elems(d, L) for d in DTYPES] == [32, 32, 256, 256, 32, 256]
    # tied Q6_K head, hidden size 2048 x vocab 128256, "~205 MiB" on the page
    head = oracle.blob_bytes(oracle.Q6_K, 128256, 2048, L)
    assert head == 215_470_080 and round(head / 2**20) == 205


# ------------------------------------------------------------------- SwiGLU

def pin_silu(L=None):
    ln3 = math.log(3.0)
    assert oracle.silu(0.0, L) == 0.0, "silu(0) must be 0"
    # sigmoid(ln 3) = 1 / (1 + 1/3) = 3/4 and sigmoid(-ln 3) = 1/4
    assert abs(oracle.silu(ln3, L) - 0.75 * ln3) <= 4e-16 * ln3, "silu(ln 3) != 3/4 ln 3"
    assert abs(oracle.silu(-ln3, L) + 0.25 * ln3) <= 4e-16 * ln3, "silu(-ln 3) != -1/4 ln 3"
    # the minimum: at v* = -1 - W(1/e) the value is -W(1/e), W = Lambert's W
    w = 0.5
    for _ in range(60):                       # Newton on w e^w = 1/e
        w -= (w * math.exp(w) - math.exp(-1.0)) / (math.exp(w) * (1.0 + w))
    assert abs(w - 0.2784645427610738) < 1e-15
    assert abs(oracle.silu(-1.0 - w, L) + w) <= 1e-15, "silu minimum is not -W(1/e)"
    # sigmoid(v) + sigmoid(-v) = 1, so silu(v) - silu(-v) = v
    for v in (1e-3, 0.5, 1.0, 2.5, 10.0, 30.0):
        assert abs(oracle.silu(v, L) - oracle.silu(-v, L) - v) <= 2e-16 * v, f"odd-part identity fails at {v}"
    # limits: e^-v overflow gives -0, large v gives v
    lo = oracle.silu(-1000.0, L)
    assert lo == 0.0 and math.copysign(1.0, lo) < 0, "silu(-1000) should be -0"
    assert oracle.silu(1000.0, L) == 1000.0 and oracle.silu(40.0, L) == 40.0


def pin_swiglu(L=None):
    """Gate and up blobs from the fixture blocks (up rotated against gate);
    x = e_k picks column k, so g and u are design values."""
    for dt in DTYPES:
        recs = load_golden(oracle.NAMES[dt])
        bs = oracle.block_elems(dt, L)
        nblk = 2 if bs == 256 else 4
        K, M = nblk * bs, 3

        def make(shift):
            rb, rw = [], []
            for m in range(M):
                pick = [recs[(m + b + shift) % len(recs)] for b in range(nblk)]
                rb.append(b"".join(p[1] for p in pick))
                rw.append(np.concatenate([p[2] for p in pick]))
            return np.frombuffer(b"".join(rb), np.uint8), np.stack(rw)

        gate, Wg = make(0)
        up, Wu = make(1)
        ks = list(range(0, K, 7)) + [K - 1]
        X = np.eye(K, dtype=np.float32)[ks] * np.float32(8.0)
        r = oracle.swiglu(dt, gate, up, M, K, X, L=L)
        name = oracle.NAMES[dt]
        assert np.array_equal(r["g"], 8.0 * Wg[:, ks].T), f"{name}: g is not the gate projection"
        assert np.array_equal(r["u"], 8.0 * Wu[:, ks].T), f"{name}: u is not the up projection"
        assert np.array_equal(r["sg"], np.abs(r["g"])) and np.array_equal(r["su"], np.abs(r["u"]))
        for n in range(len(ks)):
            for m in range(M):
                g, u = 8.0 * Wg[m, ks[n]], 8.0 * Wu[m, ks[n]]
                want = oracle.silu(g, L) * u
                assert r["out64"][n, m] == want, f"{name}: out[{n},{m}] != silu(g) u"
                assert r["out"][n, m] == np.float32(want)
        # the order of the operands matters wherever g != u
        swapped = np.array([[oracle.silu(8.0 * Wu[m, k], L) * 8.0 * Wg[m, k] for m in range(M)] for k in ks])
        assert not np.array_equal(swapped, r["out64"]), f"{name}: fixtures cannot tell gate from up"
        # a row subset gives the same numbers
        rs = oracle.swiglu(dt, gate, up, M, K, X, rows=[2, 0], L=L)
        assert np.array_equal(rs["out64"], r["out64"][:, [2, 0]])


# ------------------------------------------------------------------- argmax

def pin_argmax(L=None):
    for dt in DTYPES:
        recs = load_golden(oracle.NAMES[dt])
        bs = oracle.block_elems(dt, L)
        nblk = 2 if bs == 256 else 4
        K, M = nblk * bs, 5
        rb, rw = [], []
        for m in range(M):
            pick = [recs[(m + b) % len(recs)] for b in range(nblk)]
            rb.append(b"".join(p[1] for p in pick))
            rw.append(np.concatenate([p[2] for p in pick]))
        blob, W = np.frombuffer(b"".join(rb), np.uint8), np.stack(rw)
        name = oracle.NAMES[dt]
        for k in list(range(0, K, 5)) + [K - 1]:
            col = W[:, k]
            want = int(np.flatnonzero(col == col.max())[0])      # first of the design maxima
            for sgn in (1.0, -1.0):
                x = np.zeros(K, np.float32)
                x[k] = sgn
                c = sgn * col
                want = int(np.flatnonzero(c == c.max())[0])
                idx, best, _ = oracle.argmax(dt, blob, M, K, x, L=L)
                assert idx == want and best == c.max(), f"{name}: x = {sgn:+} e_{k}: argmax {idx}, design {want}"
        # a planted maximum in the last row, and ties resolved to the smallest index
        assert not np.array_equal(W[0], W[1]), f"{name}: fixture rows 0 and 1 must differ"
        dup = np.frombuffer(b"".join([rb[1], rb[0], rb[1], rb[1]]), np.uint8)
        x = np.zeros(K, np.float32)
        k = int(np.argmax(np.abs(W[1] - W[0])))
        x[k] = 1.0 if W[1, k] > W[0, k] else -1.0
        idx, _, _ = oracle.argmax(dt, dup, 4, K, x, L=L)
        assert idx == 0, f"{name}: three equal maxima at rows 0, 2, 3 should give 0, got {idx}"
        last = np.frombuffer(b"".join([rb[0], rb[0], rb[1]]), np.uint8)
        idx, _, _ = oracle.argmax(dt, last, 3, K, x, L=L)
        assert idx == 2, f"{name}: the maximum sits in the last row, got {idx}"


# ------------------------------------------------- Q8_0-quantized activations

def _f32(s: str) -> np.float32:
    s = s.strip().lower()
    if s in ("nan", "inf", "-inf"):
        return np.float32(float(s))
    return np.float32(_num(s))


def load_q8_act_golden():
    """[(record name, x f32[32], scale, codes int8[32])] from tests/golden/q8_0_act.txt."""
    recs, cur, key = [], None, None
    with open(os.path.join(GOLDEN, "q8_0_act.txt")) as f:
        for raw in f:
            line = raw.rstrip("\n")
            if not line.strip() or line.lstrip().startswith("#"):
                continue
            if line.startswith("["):
                cur = {"name": line.strip("[] "), "x": [], "scale": [], "q": []}
                recs.append(cur)
                continue
            for k in ("x", "scale", "q"):
                if line.startswith(k + ":"):
                    key, line = k, line[len(k) + 1:]
            cur[key] += line.split()
    out = []
    for r in recs:
        x = np.array(_expand(r["x"], _f32), dtype=np.float32)
        q = np.array(_expand(r["q"], int), dtype=np.int8)
        out.append((r["name"], x, _f32(r["scale"][0]), q))
    return out


def pin_q8_act_golden(L=None):
    recs = load_q8_act_golden()
    assert len(recs) >= 8
    for name, x, scale, q in recs:
        assert x.size == 32 and q.size == 32, f"{name}: a record is one block of 32"
        sc, qq = oracle.quantize_q8_0(x[None, :], L=L)
        assert (sc[0, 0] == scale) or (scale != scale and sc[0, 0] != sc[0, 0]), \
            f"{name}: scale {float(sc[0, 0])!r}, hand-derived {float(scale)!r}"
        bad = np.nonzero(qq[0] != q)[0]
        assert bad.size == 0, f"{name}: code {bad[0]} is {qq[0][bad[0]]}, hand-derived {q[bad[0]]}"
    # blocks are independent and tokens are rows: the records stacked as one
    # token of 32*R values and as R tokens give the same scales and codes
    X = np.stack([r[1] for r in recs])
    s2, q2 = oracle.quantize_q8_0(X, L=L)
    s1, q1 = oracle.quantize_q8_0(X.reshape(1, -1), L=L)
    assert np.array_equal(q2.reshape(-1), q1.reshape(-1))
    assert np.array_equal(s2.reshape(-1), s1.reshape(-1), equal_nan=True)


def pin_float_to_half(L=None):
    """f32 -> binary16 rounding against numpy's conversion (nearest, ties to even)."""
    rng = np.random.default_rng(7)
    vals = [np.float32(v) for v in (0.0, -0.0, 1.0, 65504.0, 65519.99, 65520.0, -65520.0, 1e6, 2.0 ** -24,
                                    2.0 ** -25, 2.0 ** -25 * 1.0001, 3 * 2.0 ** -26, 2.0 ** -14, 6.1e-5,
                                    np.inf, -np.inf)]
    # every half-way point between adjacent finite halves (exact in f32)
    h = np.arange(0, 0x7C00, 37, dtype=np.uint16)
    a = h.view(np.float16).astype(np.float32)
    b = (h + 1).view(np.float16).astype(np.float32)
    vals += list((a + b) / np.float32(2))
    vals += list(rng.standard_normal(2000).astype(np.float32) * np.float32(2.0) ** rng.integers(-30, 17, 2000))
    for v in vals:
        for sv in (v, -v):
            with np.errstate(over="ignore"):
                want = int(np.array(sv, np.float32).astype(np.float16).view(np.uint16))
            got = oracle.float_to_half(sv, L)
            assert got == want, f"f16({float(sv)!r}) = {got:#06x}, numpy gives {want:#06x}"
    assert oracle.float_to_half(np.float32(np.nan), L) & 0x7C00 == 0x7C00
    assert oracle.float_to_half(np.float32(np.nan), L) & 0x03FF != 0


def pin_q8_act_bound(L=None):
    """Codes and scales of random activations against the quantizer's closed-form bound.

    With d = amax/127 and codes rounded from v/d, |q d - v| <= d/2 (up to the
    f32 rounding of v/d), and the stored scale differs from d by at most half
    an f16 ulp, so |q scale - v| <= d (1/2 + 2^-16) + 127 |scale - d|.  The
    element of largest |v| gets |q| = 127; negating x negates the codes;
    scaling x by 2^j scales the scales and keeps the codes.
    """
    rng = rng_for(990, 0)
    for mag in (1e-3, 1.0, 37.0, 3e4):
        X = (rng.standard_normal((3, 256)) * mag).astype(np.float32)
        X[1, 32:96] = 0.0                      # blocks 1 and 2 of token 1: all zero
        sc, q = oracle.quantize_q8_0(X, L=L)
        blocks = X.reshape(3, 8, 32).astype(np.float64)
        amax = np.abs(blocks).max(axis=2)
        d = amax / 127.0
        assert np.all(np.abs(q.astype(np.int32)) <= 127)
        err = np.abs(q.reshape(3, 8, 32) * sc[..., None].astype(np.float64) - blocks)
        bound = d * (0.5 + 2.0 ** -16) + 127 * np.abs(sc.astype(np.float64) - d)
        assert np.all(err <= bound[..., None] * (1 + 1e-6)), f"mag {mag}: |q scale - x| above the bound"
        assert np.all(np.abs(sc.astype(np.float64) - d) <= d * 2.0 ** -11 + 2.0 ** -25), "scale is not f16(d)"
        top = np.abs(blocks).argmax(axis=2)
        qb = q.reshape(3, 8, 32)
        for n in range(3):
            for b in range(8):
                if amax[n, b] > 0:
                    assert abs(int(qb[n, b, top[n, b]])) == 127, f"mag {mag}: block max does not get 127"
        assert np.all(sc[1, 1:3] == 0) and np.all(qb[1, 1:3] == 0), "a zero block needs scale 0, codes 0"
        sn, qn = oracle.quantize_q8_0(-X, L=L)
        assert np.array_equal(sn, sc) and np.array_equal(qn, -q), "negating x must negate the codes"
        if mag <= 37.0:
            s4, q4 = oracle.quantize_q8_0(X * np.float32(4.0), L=L)
            assert np.array_equal(q4, q), "x * 4 changed the codes"
            normal = sc >= 2.0 ** -14                  # on the subnormal f16 grid the scale rounds differently
            assert np.array_equal(s4[normal], sc[normal] * np.float32(4.0)), "x * 4 did not scale the scales"


def exact_offsets(dt: int, blk: bytes) -> list:
    """The code-independent term of every weight of one block (0 for formats without one)."""
    bs = 256 if dt in (oracle.Q4_K, oracle.Q5_K, oracle.Q6_K) else 32
    if dt == oracle.Q4_1:
        return [_h(blk, 2)] * 32
    if dt in (oracle.Q4_K, oracle.Q5_K):
        dmin, s = _h(blk, 2), blk[4:16]
        out = []
        for i in range(8):
            mn = s[i + 4] % 64 if i < 4 else s[i + 4] // 16 + 16 * (s[i] // 64)
            out += [-dmin * mn] * 32
        return out
    return [Fraction(0)] * bs


def pin_q8_matmul(L=None):
    """Weights x Q8_0 activations: exact rational brute force, the closed form, tokens and rows."""
    shapes = [(1, 1), (3, 2), (4, 3)]
    for i, dt in enumerate(DTYPES):
        name = oracle.NAMES[dt]
        bs, bb = oracle.block_elems(dt, L), oracle.block_bytes(dt, L)
        for j, (M, N) in enumerate(shapes):
            K = 2 * bs if bs == 256 else 8 * bs
            blob = make_blob(dt, M, K, rng_for(960 + i, j))
            sc, q = oracle.quantize_q8_0(make_x(N, K, rng_for(960 + i, 100 + j)), L=L)
            Y, Y64, S, Sp = oracle.matmul_q8act(dt, blob, M, K, sc, q, L=L)
            raw, nb = blob.tobytes(), K // bs
            for m in range(M):
                w, o = [], []
                for b in range(nb):
                    blk = raw[(m * nb + b) * bb:(m * nb + b + 1) * bb]
                    w += exact_weights(dt, blk)
                    o += exact_offsets(dt, blk)
                for n in range(N):
                    xs = [Fraction(float(sc[n, k // 32])) * int(q[n, k]) for k in range(K)]
                    exact = sum((wk * xk for wk, xk in zip(w, xs)), Fraction(0))
                    mag = sum((abs(wk * xk) for wk, xk in zip(w, xs)), Fraction(0))
                    magp = sum(((abs(wk - ok) + abs(ok)) * abs(xk) for wk, ok, xk in zip(w, o, xs)), Fraction(0))
                    bound = Fraction(K) * Fraction(2) ** -50 * magp
                    assert abs(Fraction(float(Y64[n, m])) - exact) <= bound, f"{name}: y[{n},{m}] f64 is off"
                    assert abs(Fraction(float(S[n, m])) - mag) <= bound, f"{name}: S is not sum |w xq|"
                    assert abs(Fraction(float(Sp[n, m])) - magp) <= bound, f"{name}: Splus misses an offset term"
                    want = round_f32(exact)
                    if Y[n, m] != want:
                        mid = (Fraction(float(min(Y[n, m], want))) + Fraction(float(max(Y[n, m], want)))) / 2
                        assert abs(mid - exact) <= bound, f"{name}: y[{n},{m}] not correctly rounded"
        # closed form: every code 1 with scale 1 is x = all ones
        M, K = 5, 2 * bs if bs == 256 else 8 * bs
        blob = make_blob(dt, M, K, rng_for(970 + i, 0))
        _, Y64, _, _ = oracle.matmul_q8act(dt, blob, M, K, np.ones((1, K // 32), np.float32),
                                           np.ones((1, K), np.int8), L=L)
        assert np.array_equal(Y64[0], closed_form_row_sums(dt, blob, M, K)), f"{name}: all-ones codes"
        # scale 2^-3 on one block only: y = 2^-3 * that block's columns summed
        scl = np.zeros((1, K // 32), np.float32)
        scl[0, 1] = 0.125
        _, Y64, _, _ = oracle.matmul_q8act(dt, blob, M, K, scl, np.ones((1, K), np.int8), L=L)
        W = np.array([[float(v) for b in range(K // bs)
                       for v in exact_weights(dt, blob.tobytes()[(m * (K // bs) + b) * bb:(m * (K // bs) + b + 1) * bb])]
                      for m in range(M)])
        assert np.array_equal(Y64[0], W[:, 32:64].sum(axis=1) * 0.125), f"{name}: block scale misplaced"
        # the second token's codes are its own; a row subset is the same numbers
        q2 = np.zeros((2, K), np.int8)
        q2[1, 3] = -7
        _, Y64, _, _ = oracle.matmul_q8act(dt, blob, M, K, np.ones((2, K // 32), np.float32), q2, rows=[4, 0], L=L)
        assert np.array_equal(Y64[0], [0.0, 0.0]) and np.array_equal(Y64[1], -7.0 * W[[4, 0], 3]), \
            f"{name}: token or row mix-up"


ALL_PINS = [pin_golden, pin_unit_vectors, pin_closed_form, pin_bruteforce, pin_invariants,
            pin_half, pin_sizes, pin_silu, pin_swiglu, pin_argmax, pin_q8_act_golden, pin_float_to_half,
            pin_q8_act_bound, pin_q8_matmul]
