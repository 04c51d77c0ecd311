/*
 * qmm.h -- C ABI of the GGUF block-quantized matmul library for AMD MI355X
 * (gfx950).  Library: gguf_block_quant_qmm_amd/libqmm.so.
 *
 * The operation (page "cera 0.5.2 src/backend/cpu.rs", section "Matrix
 * multiplication": matmul_q4_0_f32 / matmul_q8_0_f32 / matmul_q4km_f32 define
 * C = dequant(A) . B over a row-major blob of quantized blocks, overwriting C):
 *
 *     Y[n][m] = sum_k W[m][k] * X[n][k],   0 <= m < M, 0 <= n < N, 0 <= k < K
 *
 * where W[m][k] is weight k of row m decoded from the blob.  Activations and
 * outputs are f32 and token-major (page "cera 0.3.1 src/model/gpu_lfm2.rs",
 * batched prefill: contiguous token rows; at most 512 tokens per dispatch
 * there, any N >= 1 here).
 *
 * Weight blob layout (page "cera 0.5.2 src/backend/cpu.rs", matmul_q4_0_f32:
 * row i starts at i*bytes_per_row, its K/bs blocks follow back to back):
 *     row_bytes = (K / block_elems) * block_bytes,  blob = M * row_bytes bytes
 * Block formats (little-endian, f16 = IEEE binary16):
 *     Q8_0 (32 weights, 34 B): f16 d, int8 q[32];            w = d*q
 *     Q4_0 (32 weights, 18 B): f16 d, 16 nibble bytes;       w = d*(q-8)
 *          weight e<16 = low nibble of byte e, e>=16 = high nibble of byte e-16
 *          (same page, repack_q4_0_8x8)
 *     Q4_1 (32 weights, 20 B): f16 d, f16 m, 16 nibble bytes; w = d*q + m
 *          (nibbles as Q4_0; the pages name the format, gemv_q4_1_f32, but
 *          not its bytes: standard GGUF layout)
 *     Q4_K (256 weights, 144 B): f16 d, f16 dmin, 12 bytes of packed 6-bit
 *          (scale, min) for 8 sub-blocks of 32, 128 nibble bytes;
 *          w = d*sc*q - dmin*m  (same page, repack_q4_k_8x8; the 6-bit
 *          packing follows the standard GGUF k-quant layout)
 *     Q5_K (256 weights, 176 B): as Q4_K with 32 bytes qh after the scales:
 *          the fifth bit of element e of sub-block i is bit i of qh[e] (the
 *          pages name the format, gemv_q5km_f32, but not its bytes: standard
 *          GGUF layout)
 *     Q6_K (256 weights, 210 B): ql[128] low 4 bits, qh[64] high 2 bits,
 *          int8 sub-scales[16], f16 d;  w = d*sc*(q-32)  (210-byte size:
 *          page "cera 0.3.1 src/model/gpu_lfm2.rs", upload_weight; bit
 *          placement: standard GGUF layout)
 *
 * Arguments and ownership.  Every buffer is caller-owned device memory on the
 * current HIP device; the library never allocates, frees or keeps a pointer
 * after a call returns.  Calls are asynchronous on `stream` (a hipStream_t;
 * NULL = the null stream) and do not synchronise the host.  A call is
 * stateless: concurrent calls on different streams are safe.
 *
 * Errors.  Every argument is checked before any launch (the pages use release
 * asserts on the same conditions, cpu.rs gemm_preq_dispatch); a failed check
 * returns a negative code and launches nothing.  The blob's length cannot be
 * checked: the caller guarantees qmm_blob_bytes(dtype, M, K) readable bytes.
 * A fault inside a kernel surfaces at the caller's next synchronisation.
 * There is no silent fallback to another algorithm.
 *
 * Determinism.  Results are bitwise reproducible run to run (fixed reduction
 * order, no float atomics), and qmm_gemm with N == 1 returns exactly the bits
 * of qmm_gemv (page "cera 0.5.2 src/backend/cpu.rs", gemv_q4_1_f32: decode
 * and prefill must agree bit for bit).
 */
#ifndef QMM_H
#define QMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dtype tags: the GGUF tensor type ids */
#define QMM_Q4_0 2
#define QMM_Q4_1 3
#define QMM_Q8_0 8
#define QMM_Q4_K 12
#define QMM_Q5_K 13
#define QMM_Q6_K 14

/* status codes */
#define QMM_OK 0
#define QMM_ERR_NULL (-1)    /* a required pointer is NULL                          */
#define QMM_ERR_DTYPE (-2)   /* dtype is not one of the six tags above              */
#define QMM_ERR_SHAPE (-3)   /* M < 1, N < 1, K < block_elems or K % block_elems,
                                a size above 2^40 or a product of two above 2^56   */
#define QMM_ERR_ALIGN (-4)   /* blob not 16-B aligned, x/X not 16-B, y/Y not 4-B    */
#define QMM_ERR_DEVICE (-5)  /* no current HIP device, or it is not gfx950          */
#define QMM_ERR_LAUNCH (-6)  /* the kernel launch itself failed                     */
#define QMM_ERR_SCRATCH (-7) /* needs more than the static scratch (no-alloc calls) */

/* Decode GEMV (one token), page "cera 0.5.2 src/backend/cpu.rs", section
 * "GEMV (matrix-vector multiply)": y[m] = sum_k W[m][k] * x[k].
 *   w_blob  device, M*row_bytes bytes, 16-B aligned, row-major blocks
 *   dtype   QMM_Q4_0 | QMM_Q4_1 | QMM_Q8_0 | QMM_Q4_K | QMM_Q5_K | QMM_Q6_K
 *   M, K    rows and weights per row; K a multiple of the block size
 *   x       device f32 [K], 16-B aligned
 *   y       device f32 [M], 4-B aligned; overwritten
 * All f32 arithmetic: |y - exact| <= 1e-5 * sum_k |W[m][k] x[k]|. */
int qmm_gemv(const void *w_blob, int dtype, int64_t M, int64_t K,
             const float *x, float *y, void *stream);

/* Up to QMM_GEMV_MAX_MATS projections of one token in one launch, reading x
 * once (page "cera 0.5.2 src/backend/cpu.rs", the fused dual GEMV and the
 * concatenated three-matrix GEMV for the Q, K and V projections):
 *     ys[i][m] = sum_k W_i[m][k] * x[k],   0 <= m < Ms[i],  0 <= i < n.
 *   n       1 .. QMM_GEMV_MAX_MATS, else QMM_ERR_SHAPE
 *   w_blobs host array of n device pointers (each as w_blob of qmm_gemv)
 *   Ms      host array of n row counts
 *   dtype,K shared by all matrices
 *   x       device f32 [K], 16-B aligned
 *   ys      host array of n device pointers, f32 [Ms[i]], 4-B aligned;
 *           overwritten; the outputs must not overlap the blobs or x
 * Each ys[i] holds exactly the bits qmm_gemv returns for matrix i.  The
 * host arrays are read before the call returns and not kept.  Layouts that
 * the one-launch kernel does not take (K not a multiple of 64, an odd number
 * of blocks per row for Q4_0/Q4_1/Q8_0/Q6_K, K > 16384) run one launch per matrix
 * with the same results. */
#define QMM_GEMV_MAX_MATS 4
int qmm_gemv_concat(int n, const void *const *w_blobs, const int64_t *Ms, int dtype, int64_t K,
                    const float *x, float *const *ys, void *stream);

/* The gate/up projection of a gated feed-forward block with SwiGLU, one
 * token, one launch (page "cera 0.5.2 src/backend/cpu.rs", the fused gate +
 * up GEMV with in-register SwiGLU):
 *     out[m] = silu(g[m]) * u[m],  g = W_gate x,  u = W_up x,
 *     silu(v) = v / (1 + e^-v)   (same page, activation functions)
 *   gate_blob, up_blob  device blobs of one dtype and shape M x K
 *   x                   device f32 [K], 16-B aligned
 *   out                 device f32 [M], 4-B aligned; overwritten
 * g and u are the f32 GEMV sums (bits of qmm_gemv); with S_g, S_u their
 * sums of |w x| and tau = 1e-5:
 *   |out - exact| <= tau*(1.1*S_g*(|u| + tau*S_u) + |silu(g)|*S_u) + 4*2^-24*|out|.
 * Needs K a multiple of 64, at most 16384, and an even number of blocks per
 * row for Q4_0, Q4_1, Q8_0 and Q6_K; otherwise QMM_ERR_SHAPE. */
int qmm_gemv_swiglu(const void *gate_blob, const void *up_blob, int dtype, int64_t M, int64_t K,
                    const float *x, float *out, void *stream);

/* Greedy decoding: the argmax over the GEMV's outputs, without storing them
 * (page "cera 0.5.2 src/backend/cpu.rs", the greedy argmax GEMV):
 *     *index = the smallest m with y[m] = max_m' y[m'],  *value = y[*index]
 * where y is exactly the f32 output qmm_gemv returns (so the choice matches
 * argmax over qmm_gemv's bits).  NaN outputs never win; if every output is
 * NaN, *index = -1 and *value = NaN.  Ties: the smallest index (the pages
 * do not say; this is a reading).
 *   w_blob, dtype, M, K, x  as for qmm_gemv; M <= 2^31 - 1
 *   work    device scratch of QMM_ARGMAX_WORK_BYTES bytes, 16-B aligned,
 *           caller-owned; needs no initial value; clobbered
 *   index   device int64, 8-B aligned
 *   value   device f32 or NULL
 * An embedding table used as a tied LM head may carry padding rows past the
 * vocabulary (page "cera 0.5.0 src/model/llama.rs", project_logits_batched):
 * pass M = the vocabulary size; rows past M are never read.
 * Two launches on `stream` (the rows, then the winner).  Needs K a multiple
 * of 64, at most 16384, and an even number of blocks per row for Q4_0, Q4_1,
 * Q8_0 and Q6_K; otherwise QMM_ERR_SHAPE.  Concurrent calls need separate work
 * buffers. */
#define QMM_ARGMAX_WORK_BYTES 32768
int qmm_gemv_argmax(const void *w_blob, int dtype, int64_t M, int64_t K, const float *x,
                    void *work, int64_t *index, float *value, void *stream);

/* qmm_gemv_argmax without the work argument, for callers that cannot
 * allocate device memory (code under graph capture, serving loops that may
 * not call hipMalloc, harnesses that forbid it).  The workgroup candidates go
 * to a static device array of QMM_NOALLOC_SCRATCH_BYTES that the library holds
 * on every GPU it runs on until the process ends; nothing is allocated or
 * freed by the call.  Results, arguments and errors are those of
 * qmm_gemv_argmax (same kernels, bit-identical index and value); every valid
 * shape fits the array, and a launch that would need more returns
 * QMM_ERR_SCRATCH without launching.  All calls on one GPU share that GPU's
 * array: calls that overlap in time on one GPU (two streams, two threads)
 * race and must be serialised by the caller.  The array needs no initial
 * value (each call writes every slot it reads). */
#define QMM_NOALLOC_SCRATCH_BYTES 32768
int qmm_gemv_argmax_noalloc(const void *w_blob, int dtype, int64_t M, int64_t K, const float *x,
                            int64_t *index, float *value, void *stream);

/* Prefill / verify GEMM over N tokens (page "cera 0.3.1 src/model/gpu_lfm2.rs",
 * mul_mat_reg_tile: weights decoded once per k-tile and reused across all
 * token columns):  Y[n][m] = sum_k W[m][k] * X[n][k].
 *   X       device f32 [N][K] row-major, 16-B aligned
 *   Y       device f32 [N][M] row-major, 4-B aligned; overwritten
 * Below a measured crossover N it computes every token with the GEMV's f32
 * arithmetic, so Y[n] has exactly the bits qmm_gemv returns for X[n] (page
 * "cera 0.5.0 src/model/llama.rs", project_logits_batched: verifying drafted
 * tokens in one pass over the LM head; page "cera 0.5.2
 * src/backend/cpu.rs": decode and prefill must agree bit for bit).  With K a
 * multiple of 64 up to 4096 and an even number of blocks per row (Q4_0, Q4_1,
 * Q8_0, Q6_K) up to 4 tokens share one read of the weights and the crossover
 * is N = 5 (Q4_0, Q4_1, Q8_0, Q6_K; 4 for Q4_1 with M >= 12225) or 3 (Q4_K,
 * Q5_K); otherwise each token is
 * one GEMV launch and the crossover is 3 (Q4_0, Q6_K) or 2 (Q4_1, Q8_0, Q4_K,
 * Q5_K).  The path
 * qmm_gemm_path names: 0 = all-f32 arithmetic (tolerance 1e-5 of
 * sum |w x|), 1 = weights and activations rounded to f16 and multiplied on
 * the matrix cores with f32 accumulation (tolerance 2e-3 of sum |w x|; needs
 * |w|, |x| < 65504). */
int qmm_gemm(const void *w_blob, int dtype, int64_t M, int64_t K, int64_t N,
             const float *X, float *Y, void *stream);

/* The gate/up projection with SwiGLU for N tokens, one launch on the matrix
 * cores (page "cera 0.5.2 src/backend/cpu.rs", the fused gate + up + SiLU
 * GEMM dispatch; cpu.rs silu_mul_inplace for the activation):
 *     out[n][m] = silu(G[n][m]) * U[n][m],  G = X W_gate^T,  U = X W_up^T
 * Below the crossover that qmm_gemm_path reports as 0, each token runs
 * qmm_gemv_swiglu (same bits, same bound); on path 1 G and U are the f16
 * matrix-core sums (tolerance 2e-3 of their sum |w x|) carried into the
 * SwiGLU bound of qmm_gemv_swiglu with tau = 2e-3.  Neither projection is
 * stored.  Path 0 needs the shapes qmm_gemv_swiglu takes; path 1 needs K a
 * multiple of 256 (512 for Q6_K); otherwise QMM_ERR_SHAPE.
 *   gate_blob, up_blob  device blobs of one dtype and shape M x K
 *   X                   device f32 [N][K], 16-B aligned
 *   out                 device f32 [N][M], 4-B aligned; overwritten */
int qmm_gemm_swiglu(const void *gate_blob, const void *up_blob, int dtype, int64_t M, int64_t K,
                    int64_t N, const float *X, float *out, void *stream);

/* Q8_0 quantization of activations, the int8-activation variant's first step
 * (page "cera 0.5.2 src/backend/cpu.rs", the portable Q8_0 quantizer and its
 * caller-owned scale / quant buffers).  For each row n and each block b of 32
 * consecutive values v = X[n][32b .. 32b+32), in f32:
 *     amax = max |v| (NaN elements are skipped), d = amax / 127,
 *     id = 1/d when d != 0 and 1/d is finite, else 0,
 *     quants[n][32b+j] = round-half-even(v[j] * id) clamped to [-128, 127]
 *                        (a NaN product gives 0),
 *     scales[n][b] = d rounded to binary16 (round-half-even), stored as f32.
 * The codes use the unrounded 1/d, the scale the rounded d, as the page does.
 * Every output is the unique value this definition gives (correctly rounded
 * division and reciprocal), so results are bit-exact and deterministic.
 *   X       device f32 [N][K] row-major, 16-B aligned
 *   scales  device f32 [N][K/32], 16-B aligned; overwritten
 *   quants  device int8 [N][K], 16-B aligned; overwritten
 * N >= 1 and K a positive multiple of 32, else QMM_ERR_SHAPE. */
int qmm_quantize_q8_0(const float *X, int64_t N, int64_t K, float *scales, int8_t *quants,
                      void *stream);

/* The matmul on Q8_0-quantized activations (page "cera 0.5.2
 * src/backend/cpu.rs": the int8 GEMV/GEMM paths that take the activations as
 * Q8_0 blocks; the weights' offsets go through per-block sums of the
 * activation codes):
 *     Y[n][m] = sum_k W[m][k] * scales[n][k/32] * quants[n][k]
 * Each weight block meets the codes in exact integer dot products (one per
 * activation block of 32, one per 16-weight sub-scale group for Q6_K) that
 * are scaled once in f32: Q8_0 and Q4_0 by d*xs, Q6_K by d*xs*sc, Q4_K and
 * Q5_K by d*xs*sc with the minimum term dmin*xs*m times the block's code sum,
 * Q4_1 by d*xs with m*xs times the code sum.  Error bound: 1e-5 of
 * sum_k (|w - o| + |o|) |xq| per output, o the weight's offset part (m for
 * Q4_1, -dmin*m for Q4_K and Q5_K, none for the others), xq the dequantized
 * activation.  Up to 4 tokens share one read of the weights (K a multiple of
 * 64 up to 16384, even block count per row for Q4_0, Q4_1, Q8_0, Q6_K; other
 * shapes run one weight block per thread), and each token then has the bits
 * of its own single-token call.  From N = 32 tokens, where the grid is large
 * enough to pay (a measured cost model: e.g. 14336 x 4096 from N = 32, 4096 x
 * 4096 from N ~ 80), Q8_0, Q4_0 (K a multiple of 64) and Q4_K (K a multiple
 * of 256), K at most 16384, run on the int8 matrix cores: one 32-deep integer
 * step per activation block, each block sum scaled once in f32 (the same
 * bound; the bits differ from the single-token call).
 *   w_blob  device blob as for qmm_gemm, 16-B aligned
 *   scales  device f32 [N][K/32] as qmm_quantize_q8_0 writes them, 16-B aligned
 *   quants  device int8 [N][K], 16-B aligned
 *   Y       device f32 [N][M] row-major, 4-B aligned; overwritten
 * Errors as qmm_gemm. */
int qmm_gemm_q8act(const void *w_blob, int dtype, int64_t M, int64_t K, int64_t N,
                   const float *scales, const int8_t *quants, float *Y, void *stream);

/* Decode with int8 activations in one launch (page "cera 0.5.2
 * src/backend/cpu.rs": the decode GEMVs quantize the token's activations to
 * Q8_0 once and run integer block dots against every projection).  Each
 * workgroup quantizes x itself, with exactly the arithmetic of
 * qmm_quantize_q8_0, so the results are bit-identical to qmm_quantize_q8_0
 * followed by qmm_gemm_q8act with N = 1 (and so is the error bound).
 *   qmm_gemv_q8act         y[M] = W xq
 *   qmm_gemv_concat_q8act  ys[i] = W_i xq for n <= QMM_GEMV_MAX_MATS matrices
 *                          sharing dtype and K, one launch
 *   qmm_gemv_swiglu_q8act  out = silu(W_gate xq) * (W_up xq) (silu as
 *                          qmm_gemv_swiglu), neither projection stored
 *   x       device f32 [K], 16-B aligned (not modified)
 *   y, ys[i], out  device f32, 4-B aligned; overwritten
 * Shapes: K a multiple of 64 up to 16384 with an even block count per row
 * for Q4_0, Q4_1, Q8_0 and Q6_K (the one-launch kernel); others return
 * QMM_ERR_SHAPE (use qmm_quantize_q8_0 + qmm_gemm_q8act).  Other errors as
 * qmm_gemv. */
int qmm_gemv_q8act(const void *w_blob, int dtype, int64_t M, int64_t K, const float *x, float *y,
                   void *stream);
int qmm_gemv_concat_q8act(int n, const void *const *w_blobs, const int64_t *Ms, int dtype, int64_t K,
                          const float *x, float *const *ys, void *stream);
int qmm_gemv_swiglu_q8act(const void *gate_blob, const void *up_blob, int dtype, int64_t M, int64_t K,
                          const float *x, float *out, void *stream);

/* Greedy argmax with int8 activations (page "cera 0.5.2 src/backend/cpu.rs":
 * the greedy argmax GEMV runs on the Q8_0-quantized token): index = the
 * smallest row with the largest output of qmm_gemv_q8act (its bits, compared
 * in f32), value = that output.  Arguments, work buffer, shapes and errors as
 * qmm_gemv_argmax. */
int qmm_gemv_argmax_q8act(const void *w_blob, int dtype, int64_t M, int64_t K, const float *x,
                          void *work, int64_t *index, float *value, void *stream);

/* Which kernel qmm_gemm_q8act uses for these sizes: 0 = token groups (each
 * token's result has the bits of its single-token call), 1 = the int8 matrix
 * cores; a negative status for invalid arguments.  The bound is the same. */
int qmm_gemm_q8act_path(int dtype, int64_t M, int64_t K, int64_t N);

/* Load-time repack for the prefill GEMM (page "cera 0.5.2 src/backend/cpu.rs",
 * the Q4_0 / Q4_K weight repacking: a second copy of a prefill weight,
 * built once at load and kept beside the GGUF bytes, laid out for the GEMM
 * with the per-block scale products baked in; decode keeps the original).
 * Q6_K and Q8_0, whose GGUF blocks are 2 bytes off a dword on every other
 * block.  Every offset of a repacked copy is 16-byte aligned and a weight's
 * code is one byte, in the order the matrix-core lanes read them:
 *   Q6_K  320 bytes per 256 weights (GGUF: 210): 256 code bytes q (0..63),
 *         then the 16 sub-block scales d * sc[i] as f32 (GGUF splits each
 *         code over a nibble and two bits elsewhere);
 *   Q8_0  72 bytes per 64 weights (GGUF: 68): 64 code bytes q + 128, then the
 *         two block scales d as f32.
 *
 * qmm_repack_bytes: bytes of the repacked copy of M x K weights (Q6_K 1.52 x,
 *   Q8_0 1.06 x qmm_blob_bytes); 0 if dtype has no repacked form or the shape
 *   is invalid (K must be a multiple of 256).
 * qmm_repack: fills `packed` from the GGUF blob (one launch on `stream`).
 *   w_blob  device, 16-B aligned, qmm_blob_bytes(dtype, M, K) bytes
 *   packed  device, 16-B aligned, qmm_repack_bytes(dtype, M, K) bytes;
 *           overwritten; caller-owned, like w_blob
 *   dtype   QMM_Q6_K or QMM_Q8_0 (any other valid dtype: QMM_ERR_DTYPE)
 * qmm_gemm_repacked: Y[n][m] = sum_k W[m][k] * X[n][k] from the repacked
 *   copy, on the matrix cores for every N (the f16 class of qmm_gemm: 2e-3 of
 *   sum |w x|).  Where qmm_gemm runs the matrix cores too (qmm_gemm_path 1)
 *   and the row has an even number of blocks, Y has exactly qmm_gemm's bits:
 *   each weight is the same single rounding of its exact value to f16 and
 *   every matrix-core step sees the same operands.  K must be a multiple of
 *   256 below 2^22 (QMM_ERR_SHAPE otherwise); X, Y, N as for qmm_gemm.
 * qmm_gemm_repacked_kernel: which matrix-core kernel it runs (the ids of
 *   qmm_gemm_kernel), or a negative status. */
int64_t qmm_repack_bytes(int dtype, int64_t M, int64_t K);
int qmm_repack(const void *w_blob, int dtype, int64_t M, int64_t K, void *packed, void *stream);
int qmm_gemm_repacked(const void *packed, int dtype, int64_t M, int64_t K, int64_t N, const float *X,
                      float *Y, void *stream);
int qmm_gemm_repacked_kernel(int dtype, int64_t M, int64_t K, int64_t N);

/* Which arithmetic qmm_gemm uses for these sizes: 0 = f32 (GEMV family),
 * 1 = f16 matrix-core GEMM, or a negative status for invalid arguments. */
int qmm_gemm_path(int dtype, int64_t M, int64_t K, int64_t N);

/* Which kernel qmm_gemm launches for these sizes (a diagnostic: the tests use
 * it to show that their shapes reach every kernel):
 *   QMM_KERNEL_GEMV         the f32 GEMV, one launch per token
 *   QMM_KERNEL_GEMV_TOKENS  the f32 GEMV arithmetic, up to 4 tokens per read
 *                           of the weights
 *   0 .. 99                 a matrix-core kernel (the id names the kernel and
 *                           tile shape inside this library build)
 *   < 0                     a status code for invalid arguments */
#define QMM_KERNEL_GEMV 100
#define QMM_KERNEL_GEMV_TOKENS 101
int qmm_gemm_kernel(int dtype, int64_t M, int64_t K, int64_t N);

/* Which form qmm_gemm_swiglu launches for these sizes (a diagnostic, like
 * qmm_gemm_kernel): QMM_KERNEL_GEMV for the per-token f32 path, 1 .. 99 a
 * matrix-core tile (id inside this library build), < 0 a status code. */
int qmm_gemm_swiglu_kernel(int dtype, int64_t M, int64_t K, int64_t N);

/* A plain streaming read of `bytes` bytes of buf (a diagnostic: the ceiling
 * that any launch reading the same bytes can reach, which the bench puts each
 * GEMV launch against).  Non-temporal 16-byte loads, each wavefront
 * instruction reading 1 KB in a row, eight per thread in flight, no
 * arithmetic beyond a fold; one float per wavefront (at most
 * QMM_READ_PROBE_OUT_FLOATS) is written to out, and the XOR of those folds is
 * the XOR of the buffer's dwords.
 *   buf     device, 16-B aligned, `bytes` readable bytes (1 .. 2^40)
 *   out     device f32 [QMM_READ_PROBE_OUT_FLOATS], 4-B aligned; clobbered */
#define QMM_READ_PROBE_OUT_FLOATS 4096
int qmm_read_probe(const void *buf, int64_t bytes, float *out, void *stream);

/* Bytes of a blob of M rows x K weights; 0 if dtype or shape is invalid. */
int64_t qmm_blob_bytes(int dtype, int64_t M, int64_t K);

/* Weights and bytes per block; 0 for an unknown dtype. */
int qmm_block_elems(int dtype);
int qmm_block_bytes(int dtype);

/* Static text for a status code (never NULL). */
const char *qmm_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H */
