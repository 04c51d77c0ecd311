/*
 * oracle.c -- plain, slow CPU oracle for the GGUF block-quantized matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
 * its Python binding) may link, load or call this file.  Only tests/, the
 * smoke check in __graft_entry__.py and the cpu_baseline leg of bench.py use
 * it.  It shares no code, header, table or constant with the HIP path.
 *
 * What it computes (the plain definition the method reaches):
 *
 *   W[m,k]  = dequant_t(blob, m, k)                       (exact in f64)
 *   Y[n,m]  = sum_k W[m,k] * X[n,k]   accumulated in f64, sequential k,
 *             then rounded once to f32 (round-to-nearest-even)
 *   S[n,m]  = sum_k |W[m,k] * X[n,k]| in f64               (tolerance scale)
 *
 * and, for the gate/up projection with SwiGLU (two matrices of one shape),
 *
 *   out[n,m] = silu(G[n,m]) * U[n,m],  silu(v) = v / (1 + e^-v)  in f64,
 *   G, U the f64 sums above for the gate and the up matrix;
 *
 * and, for greedy decoding, the argmax over m of the f64 sums of one token
 * (the smallest index among equal maxima);
 *
 * and, for the int8-activation variant, the page's Q8_0 quantization of the
 * activations (scale = f16(amax/127), codes = RNE(v / d), see
 * oracle_quantize_q8_0) and the same f64 sum with X replaced by the
 * dequantized codes, Xq[n,k] = scale[n][k/32] * q[n,k] (exact in f64).
 *
 * Source of the definition: page "cera 0.5.2 src/backend/cpu.rs", section
 * "Matrix multiplication" -- the scalar reference matmuls matmul_f32,
 * matmul_q4_0_f32, matmul_q8_0_f32 and matmul_q4km_f32 define
 * C = dequant(A) . B with A row-major in blocks, one block dot per step and
 * the output overwritten (not accumulated).  Here the activation operand is
 * stored token-major, X[N][K], and the output token-major, Y[N][M]; that is
 * the same contraction with the operand transposed (page "cera 0.3.1
 * src/model/gpu_lfm2.rs", batched-prefill scratch: contiguous token rows).
 *
 * Block formats (all little-endian; f16 is IEEE binary16, decoded exactly,
 * subnormals included, Inf/NaN propagate):
 *   Q8_0 (type 8,  32 weights, 34 B): d f16 @0, q int8[32] @2;   w = d*q
 *   Q4_1 (type 3,  32 weights, 20 B): d f16 @0, m f16 @2, qs u8[16] @4;
 *        nibbles placed as in Q4_0;  w = d*q + m
 *        (the pages name the format and its GEMV -- page "cera 0.5.2
 *         src/backend/cpu.rs", gemv_q4_1_f32 -- but print no layout;
 *         READING: the standard GGUF Q4_1 block, "parity unpinned" against
 *         the pages, pinned to hand-built fixtures written from the reading)
 *   Q4_0 (type 2,  32 weights, 18 B): d f16 @0, qs u8[16] @2;
 *        element e<16 is the low nibble of qs[e], e>=16 the high nibble of
 *        qs[e-16];  w = d*(q-8)
 *        (page "cera 0.5.2 src/backend/cpu.rs", Q4_0 weight repacking:
 *         the nibble() helper of repack_q4_0_8x8 and the little-endian scale
 *         read at the block start)
 *   Q4_K (type 12, 256 weights, 144 B): d f16 @0, dmin f16 @2,
 *        scales u8[12] @4, qs u8[128] @16.  Sub-block i = j/32, e = j%32;
 *        q = low nibble of qs[(i/2)*32+e] if i even, high nibble if odd;
 *        w = d*sc_i*q - dmin*m_i
 *        (same page, repack_q4_k_8x8: nibble placement and the baked
 *         products d*sc and dmin*mn).  The 6-bit (sc_i, m_i) packing of the
 *        12 scale bytes is not printed on the pages (decode_q4km_scales is
 *        only called); READING (standard GGUF k-quant packing):
 *          i<4 : sc = s[i]&63,               m = s[i+4]&63
 *          i>=4: sc = (s[i+4]&15)|((s[i-4]>>6)<<4),
 *                m  = (s[i+4]>>4)|((s[i]>>6)<<4)
 *   Q5_K (type 13, 256 weights, 176 B): d f16 @0, dmin f16 @2,
 *        scales u8[12] @4 (packed as Q4_K), qh u8[32] @16, qs u8[128] @48.
 *        Sub-block i = j/32, e = j%32: low 4 bits as Q4_K's nibble, fifth
 *        bit = bit i of qh[e];  q = lo | hi<<4;  w = d*sc_i*q - dmin*m_i
 *        (the pages name Q5_K and its GEMV -- page "cera 0.5.2
 *         src/backend/cpu.rs", gemv_q5km_f32 -- but print no layout;
 *         READING: the standard GGUF Q5_K block, "parity unpinned" against
 *         the pages, pinned to hand-built fixtures written from the reading)
 *   Q6_K (type 14, 256 weights, 210 B): ql u8[128] @0, qh u8[64] @128,
 *        sc int8[16] @192, d f16 @208.  Only the 210-byte size is on the
 *        pages (page "cera 0.3.1 src/model/gpu_lfm2.rs", upload_weight);
 *        READING (standard GGUF layout): for element j,
 *          h=j/128, r=j%128, g=r/32, l=r%32
 *          lo4 = ql[64h+32(g&1)+l] low nibble if g<2 else high nibble
 *          hi2 = (qh[32h+l] >> 2g) & 3
 *          q   = lo4 | hi2<<4;       w = d*sc[j/16]*(q-32)
 *
 * Parity pins: hand-built blocks, the all-ones closed form, unit vectors and
 * exact rational brute force; the f16 rounding against numpy's binary16
 * conversion; the Q8_0 activation quantizer against hand-derived blocks
 * (tests/golden/q8_0_act.txt) and its closed-form error bound; and
 * (tests/test_oracle_pins.py); SiLU at closed-form
 * points (sigmoid(ln 3) = 3/4, the minimum -W(1/e)) and SwiGLU on fixture
 * blocks with unit vectors.  The Q4_K scale
 * packing and the Q6_K bit layout are a reading of the GGUF convention that
 * no page value can confirm: for those two, "parity unpinned" against the
 * pages; they are pinned only against the hand-built fixtures written from
 * the same reading.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_Q4_0 2
#define OR_Q4_1 3
#define OR_Q8_0 8
#define OR_Q4_K 12
#define OR_Q5_K 13
#define OR_Q6_K 14

/* ---- format geometry --------------------------------------------------- */

int oracle_block_elems(int dtype) {
    switch (dtype) {
    case OR_Q4_0: return 32;
    case OR_Q4_1: return 32;
    case OR_Q8_0: return 32;
    case OR_Q4_K: return 256;
    case OR_Q5_K: return 256;
    case OR_Q6_K: return 256;
    default: return 0;
    }
}

int oracle_block_bytes(int dtype) {
    switch (dtype) {
    case OR_Q4_0: return 18;
    case OR_Q4_1: return 20;
    case OR_Q8_0: return 34;
    case OR_Q4_K: return 144;
    case OR_Q5_K: return 176;
    case OR_Q6_K: return 210;
    default: return 0;
    }
}

/* ---- IEEE binary16 -> double, exact ----------------------------------- */

double oracle_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 31;
    int frac = h & 1023;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);               /* subnormal: frac * 2^-24 */
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25); /* (1 + frac/1024) * 2^(e-15) */
    return sign ? -v : v;
}

static double half_at(const uint8_t *p) {
    return oracle_half_to_double((uint16_t)(p[0] | (p[1] << 8)));
}

/* ---- one block -> its weights, in f64 ---------------------------------- */

static void dequant_q8_0(const uint8_t *b, double *w) {
    double d = half_at(b);
    for (int j = 0; j < 32; j++)
        w[j] = d * (double)(int8_t)b[2 + j];
}

static void dequant_q4_0(const uint8_t *b, double *w) {
    double d = half_at(b);
    const uint8_t *qs = b + 2;
    for (int j = 0; j < 32; j++) {
        int q = (j < 16) ? (qs[j] & 15) : (qs[j - 16] >> 4);
        w[j] = d * (double)(q - 8);
    }
}

static void q4k_scale_min(const uint8_t *s, int i, int *sc, int *mn) {
    if (i < 4) {
        *sc = s[i] & 63;
        *mn = s[i + 4] & 63;
    } else {
        *sc = (s[i + 4] & 15) | ((s[i - 4] >> 6) << 4);
        *mn = (s[i + 4] >> 4) | ((s[i] >> 6) << 4);
    }
}

static void dequant_q4_k(const uint8_t *b, double *w) {
    double d = half_at(b);
    double dmin = half_at(b + 2);
    const uint8_t *s = b + 4;
    const uint8_t *qs = b + 16;
    for (int j = 0; j < 256; j++) {
        int i = j / 32, e = j % 32;
        int sc, mn;
        q4k_scale_min(s, i, &sc, &mn);
        uint8_t byte = qs[(i / 2) * 32 + e];
        int q = (i % 2 == 0) ? (byte & 15) : (byte >> 4);
        w[j] = d * (double)sc * (double)q - dmin * (double)mn;
    }
}

static void dequant_q5_k(const uint8_t *b, double *w) {
    double d = half_at(b), dmin = half_at(b + 2);
    const uint8_t *s = b + 4, *qh = b + 16, *qs = b + 48;
    for (int i = 0; i < 8; i++) {
        int sc, mn;
        q4k_scale_min(s, i, &sc, &mn);
        for (int e = 0; e < 32; e++) {
            uint8_t byte = qs[(i / 2) * 32 + e];
            int lo = (i % 2 == 0) ? (byte & 15) : (byte >> 4);
            int hi = (qh[e] >> i) & 1;
            w[32 * i + e] = d * (double)sc * (double)(lo | (hi << 4)) - dmin * (double)mn;
        }
    }
}

static void dequant_q6_k(const uint8_t *b, double *w) {
    const uint8_t *ql = b;
    const uint8_t *qh = b + 128;
    const int8_t *sc = (const int8_t *)(b + 192);
    double d = half_at(b + 208);
    for (int j = 0; j < 256; j++) {
        int h = j / 128, r = j % 128, g = r / 32, l = r % 32;
        uint8_t lob = ql[64 * h + 32 * (g & 1) + l];
        int lo4 = (g < 2) ? (lob & 15) : (lob >> 4);
        int hi2 = (qh[32 * h + l] >> (2 * g)) & 3;
        int q = lo4 | (hi2 << 4);
        w[j] = d * (double)sc[j / 16] * (double)(q - 32);
    }
}

static void dequant_q4_1(const uint8_t *b, double *w) {
    double d = half_at(b), m = half_at(b + 2);
    const uint8_t *qs = b + 4;
    for (int j = 0; j < 32; j++) {
        int q = (j < 16) ? (qs[j] & 15) : (qs[j - 16] >> 4);
        w[j] = d * (double)q + m;
    }
}

static int dequant_block(int dtype, const uint8_t *b, double *w) {
    switch (dtype) {
    case OR_Q8_0: dequant_q8_0(b, w); return 0;
    case OR_Q4_0: dequant_q4_0(b, w); return 0;
    case OR_Q4_1: dequant_q4_1(b, w); return 0;
    case OR_Q4_K: dequant_q4_k(b, w); return 0;
    case OR_Q5_K: dequant_q5_k(b, w); return 0;
    case OR_Q6_K: dequant_q6_k(b, w); return 0;
    default: return -2;
    }
}

static int check_shape(int dtype, int64_t M, int64_t K) {
    int bs = oracle_block_elems(dtype);
    if (bs == 0) return -2;
    if (M < 1 || K < bs || K % bs != 0) return -3;
    return 0;
}

/* Row m of W: row m starts at byte m*row_bytes, row_bytes = (K/bs)*BB, and
 * its blocks follow one another (page "cera 0.5.2 src/backend/cpu.rs",
 * matmul_q4_0_f32: row_start = i*bytes_per_row, block_offset = row_start +
 * bi*size_of block). */
static int dequant_row(int dtype, const uint8_t *blob, int64_t K, int64_t m, double *out) {
    int bs = oracle_block_elems(dtype), bb = oracle_block_bytes(dtype);
    int64_t nb = K / bs;
    const uint8_t *row = blob + m * nb * bb;
    for (int64_t b = 0; b < nb; b++) {
        int rc = dequant_block(dtype, row + b * bb, out + b * bs);
        if (rc) return rc;
    }
    return 0;
}

/* ---- public entry points ----------------------------------------------- */

/* W as f64 [M][K]. */
int oracle_dequant(int dtype, const uint8_t *blob, int64_t M, int64_t K, double *W) {
    int rc = check_shape(dtype, M, K);
    if (rc) return rc;
    for (int64_t m = 0; m < M; m++) {
        rc = dequant_row(dtype, blob, K, m, W + m * K);
        if (rc) return rc;
    }
    return 0;
}

/* Outputs for the listed rows only: for r in [0,nrows), m = rows[r],
 * Y[n*nrows + r] = f32(sum_k W[m,k] X[n,k]), Y64 the f64 sum, S the f64
 * sum of |W X|.  rows == NULL means all M rows in order (nrows == M).
 * Y64 and S may be NULL.  Threads split the row list (OpenMP, if built
 * with it); each output is still one sequential f64 sum over k. */
int oracle_matmul_rows(int dtype, const uint8_t *blob, int64_t M, int64_t K, int64_t N,
                       const float *X, int64_t nrows, const int64_t *rows,
                       float *Y, double *Y64, double *S) {
    int rc = check_shape(dtype, M, K);
    if (rc) return rc;
    if (N < 1 || nrows < 1) return -3;
    if (rows) {
        for (int64_t r = 0; r < nrows; r++)
            if (rows[r] < 0 || rows[r] >= M) return -3;
    } else if (nrows != M) {
        return -3;
    }
    int err = 0;
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)K);
        if (!w) {
#pragma omp atomic write
            err = -7;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < nrows; r++) {
            if (!w) continue;
            int64_t m = rows ? rows[r] : r;
            if (dequant_row(dtype, blob, K, m, w)) continue;
            for (int64_t n = 0; n < N; n++) {
                const float *x = X + n * K;
                double acc = 0.0, mag = 0.0;
                for (int64_t k = 0; k < K; k++) {
                    double p = w[k] * (double)x[k];
                    acc += p;
                    mag += fabs(p);
                }
                Y[n * nrows + r] = (float)acc;
                if (Y64) Y64[n * nrows + r] = acc;
                if (S) S[n * nrows + r] = mag;
            }
        }
        free(w);
    }
    return err;
}

/* Full output Y[N][M] (token-major), with optional Y64 and S of the same shape. */
int oracle_matmul(int dtype, const uint8_t *blob, int64_t M, int64_t K, int64_t N,
                  const float *X, float *Y, double *Y64, double *S) {
    return oracle_matmul_rows(dtype, blob, M, K, N, X, M, NULL, Y, Y64, S);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- fused gate/up projection with SwiGLU ------------------------------ */

/* SiLU (page "cera 0.5.2 src/backend/cpu.rs", activation functions: the
 * input times its logistic sigmoid), evaluated as v / (1 + e^-v) in f64.
 * Below v ~ -709, e^-v overflows to +Inf and the quotient is -0, the
 * function's limit. */
double oracle_silu(double v) { return v / (1.0 + exp(-v)); }

/* The gate/up projection with SwiGLU (same page, the fused gate + up GEMV
 * with in-register SwiGLU, and silu_mul_inplace: gate = silu(gate) * up):
 *     out[n][r] = silu(g) * u,   g = sum_k Wg[m,k] X[n,k],  u = sum_k Wu[m,k] X[n,k]
 * for m = rows[r] (all rows when rows == NULL), g and u the f64 sums of
 * oracle_matmul_rows.  out is the f32 rounding of the f64 product out64.
 * G, U, SG, SU receive g, u and their sums of |w x| (for the tolerance);
 * every output pointer but out may be NULL. */
int oracle_swiglu_rows(int dtype, const uint8_t *gate, const uint8_t *up, int64_t M, int64_t K, int64_t N,
                       const float *X, int64_t nrows, const int64_t *rows, float *out, double *out64,
                       double *G, double *U, double *SG, double *SU) {
    int rc = check_shape(dtype, M, K);
    if (rc) return rc;
    if (N < 1 || nrows < 1) return -3;
    size_t cnt = (size_t)N * (size_t)nrows;
    float *tmp = (float *)malloc(sizeof(float) * cnt);
    double *g = (double *)malloc(sizeof(double) * cnt), *u = (double *)malloc(sizeof(double) * cnt);
    double *sg = (double *)malloc(sizeof(double) * cnt), *su = (double *)malloc(sizeof(double) * cnt);
    if (!tmp || !g || !u || !sg || !su) {
        rc = -7;
    } else {
        rc = oracle_matmul_rows(dtype, gate, M, K, N, X, nrows, rows, tmp, g, sg);
        if (!rc) rc = oracle_matmul_rows(dtype, up, M, K, N, X, nrows, rows, tmp, u, su);
    }
    if (!rc) {
        for (size_t i = 0; i < cnt; i++) {
            double o = oracle_silu(g[i]) * u[i];
            out[i] = (float)o;
            if (out64) out64[i] = o;
            if (G) G[i] = g[i];
            if (U) U[i] = u[i];
            if (SG) SG[i] = sg[i];
            if (SU) SU[i] = su[i];
        }
    }
    free(tmp); free(g); free(u); free(sg); free(su);
    return rc;
}

/* ---- greedy argmax over the logits of one token ------------------------ */

/* The greedy argmax GEMV (page "cera 0.5.2 src/backend/cpu.rs", the argmax
 * GEMV that returns the index of the largest output without storing the
 * outputs): the row m with the largest exact f64 sum y[m] = sum_k W[m,k] x[k].
 * The pages give no rule for equal maxima; READING: the smallest index wins.
 * NaN sums never win.  Writes the index, the f64 maximum and the S of that
 * row; returns -3 when no row has a non-NaN sum. */
int oracle_argmax(int dtype, const uint8_t *blob, int64_t M, int64_t K, const float *x,
                  int64_t *index, double *best, double *best_s) {
    int rc = check_shape(dtype, M, K);
    if (rc) return rc;
    float *y = (float *)malloc(sizeof(float) * (size_t)M);
    double *y64 = (double *)malloc(sizeof(double) * (size_t)M), *s = (double *)malloc(sizeof(double) * (size_t)M);
    if (!y || !y64 || !s) {
        rc = -7;
    } else {
        rc = oracle_matmul_rows(dtype, blob, M, K, 1, x, M, NULL, y, y64, s);
    }
    if (!rc) {
        int64_t bi = -1;
        for (int64_t m = 0; m < M; m++) {
            if (y64[m] != y64[m]) continue;
            if (bi < 0 || y64[m] > y64[bi]) bi = m;
        }
        if (bi < 0) {
            rc = -3;
        } else {
            *index = bi;
            if (best) *best = y64[bi];
            if (best_s) *best_s = s[bi];
        }
    }
    free(y); free(y64); free(s);
    return rc;
}

/* ---- activations quantized to Q8_0 (the int8-activation variant) ------ */

/* f32 -> IEEE binary16, round to nearest, ties to even, from the format's
 * definition: the value is placed on the half grid of its binade (2^-24 for
 * the subnormals), rounded with rint() in the default rounding mode; values
 * at or beyond 65520 (half an ulp above the largest finite half, 65504)
 * become Inf; NaN stays NaN. */
uint16_t oracle_float_to_half(float f) {
    double v = (double)f, a = fabs(v);
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    if (isnan(v)) return (uint16_t)(sign | 0x7E00);
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00);
    if (a < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)rint(ldexp(a, 24)));
    int E;
    frexp(a, &E);                          /* a in [2^(E-1), 2^E) */
    double m = rint(ldexp(a, 11 - E));     /* 1024 <= m <= 2048 */
    int e = E - 1 + 15;
    if (m == 2048.0) {
        m = 1024.0;
        e++;
    }
    if (e >= 31) return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | (e << 10) | ((int)m - 1024));
}

/* X f32 [N][K] -> Q8_0 activation blocks: scales f32 [N][K/32] and quants
 * int8 [N][K] (page "cera 0.5.2 src/backend/cpu.rs", the portable Q8_0
 * quantizer quantize_f32_to_q8_0_scalar and its caller-owned scale / quant
 * buffers).  Per block of 32, all in f32:
 *   amax  = the largest |v| (a NaN element is skipped, as a max that ignores
 *           NaN does);
 *   d     = amax / 127;
 *   id    = 1 / d when d != 0 and 1/d is finite, else 0 (the page's guard for
 *           zero, subnormal and non-finite blocks);
 *   scale = d rounded to f16 and back (stored as f32);
 *   q     = v * id rounded to nearest, ties to even, clamped to [-128, 127];
 *           a NaN product gives 0 (a saturating float -> int8 conversion).
 * The codes use the unrounded 1/d, the stored scale the f16-rounded d, as on
 * the page.  Returns -3 unless N >= 1 and K is a positive multiple of 32. */
int oracle_quantize_q8_0(const float *X, int64_t N, int64_t K, float *scales, int8_t *quants) {
    if (N < 1 || K < 32 || K % 32 != 0) return -3;
    const int64_t nb = K / 32;
    for (int64_t n = 0; n < N; n++) {
        for (int64_t b = 0; b < nb; b++) {
            const float *v = X + n * K + 32 * b;
            float amax = 0.0f;
            for (int t = 0; t < 32; t++) {
                float a = fabsf(v[t]);
                if (a > amax) amax = a;
            }
            float d = amax / 127.0f;
            float r = 1.0f / d;
            float id = (d != 0.0f && isfinite(r)) ? r : 0.0f;
            scales[n * nb + b] = (float)oracle_half_to_double(oracle_float_to_half(d));
            for (int t = 0; t < 32; t++) {
                float q = rintf(v[t] * id);
                int8_t c;
                if (isnan(q)) c = 0;
                else if (q < -128.0f) c = -128;
                else if (q > 127.0f) c = 127;
                else c = (int8_t)q;
                quants[n * K + 32 * b + t] = c;
            }
        }
    }
    return 0;
}

/* The part of each weight that does not scale with its code: m for Q4_1,
 * -dmin*m_i for Q4_K and Q5_K, nothing for the others.  The int8 kernels take
 * that term through per-block sums of the activation codes (page "cera 0.5.2
 * src/backend/cpu.rs", the Q4_1 and K-quant int8 GEMMs, whose min term goes
 * through the activation column sums), so it sets their rounding scale. */
static void offset_block(int dtype, const uint8_t *b, double *o) {
    int bs = oracle_block_elems(dtype);
    for (int j = 0; j < bs; j++) o[j] = 0.0;
    if (dtype == OR_Q4_1) {
        double m = half_at(b + 2);
        for (int j = 0; j < 32; j++) o[j] = m;
    } else if (dtype == OR_Q4_K || dtype == OR_Q5_K) {
        double dmin = half_at(b + 2);
        for (int i = 0; i < 8; i++) {
            int sc, mn;
            q4k_scale_min(b + 4, i, &sc, &mn);
            for (int e = 0; e < 32; e++) o[32 * i + e] = -(dmin * (double)mn);
        }
    }
}

/* Y[n,m] = sum_k W[m,k] * Xq[n,k] with Xq[n,k] = scales[n][k/32] * quants[n][k]
 * (exact in f64), accumulated in f64 over sequential k and rounded once to
 * f32; S[n,m] = sum_k |W Xq|; Splus[n,m] = sum_k (|W - O| + |O|) |Xq| with O
 * the offset part above (Splus == S when O == 0).  Rows as in
 * oracle_matmul_rows; Y64, S and Splus may be NULL. */
int oracle_matmul_q8act_rows(int dtype, const uint8_t *blob, int64_t M, int64_t K, int64_t N,
                             const float *scales, const int8_t *quants, int64_t nrows, const int64_t *rows,
                             float *Y, double *Y64, double *S, double *Splus) {
    int rc = check_shape(dtype, M, K);
    if (rc) return rc;
    if (K % 32 != 0 || N < 1 || nrows < 1) return -3;
    if (rows) {
        for (int64_t r = 0; r < nrows; r++)
            if (rows[r] < 0 || rows[r] >= M) return -3;
    } else if (nrows != M) {
        return -3;
    }
    const int bs = oracle_block_elems(dtype), bb = oracle_block_bytes(dtype);
    const int64_t nb = K / bs, nb32 = K / 32;
    int err = 0;
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)K);
        double *o = (double *)malloc(sizeof(double) * (size_t)K);
        if (!w || !o) {
#pragma omp atomic write
            err = -7;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < nrows; r++) {
            if (!w || !o) continue;
            int64_t m = rows ? rows[r] : r;
            if (dequant_row(dtype, blob, K, m, w)) continue;
            const uint8_t *row = blob + (m * nb) * bb;
            for (int64_t b = 0; b < nb; b++) offset_block(dtype, row + b * bb, o + b * bs);
            for (int64_t n = 0; n < N; n++) {
                double sum = 0.0, sum_abs = 0.0, magp = 0.0;
                for (int64_t j = 0; j < K; j++) {
                    double xq = (double)scales[n * nb32 + j / 32] * (double)quants[n * K + j];
                    double p = w[j] * xq;
                    sum += p;
                    sum_abs += fabs(p);
                    magp += (fabs(w[j] - o[j]) + fabs(o[j])) * fabs(xq);
                }
                Y[n * nrows + r] = (float)sum;
                if (Y64) Y64[n * nrows + r] = sum;
                if (S) S[n * nrows + r] = sum_abs;
                if (Splus) Splus[n * nrows + r] = magp;
            }
        }
        free(w);
        free(o);
    }
    return err;
}
