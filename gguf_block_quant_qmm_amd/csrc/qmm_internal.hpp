// qmm_internal.hpp -- launchers shared between the HIP sources of libqmm.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

namespace qmm {

// Tuning levers.  A measurement build (compiled with -DQMM_TUNING) reads
// them from the environment, once per process; the shipped library reads no
// environment at all and always takes the measured default, so a caller's
// environment can never move a call to another kernel or another tolerance.
inline int tuning_lever(const char *name, int dflt) {
#ifdef QMM_TUNING
    const char *e = getenv(name);
    return e ? atoi(e) : dflt;
#else
    (void)name;
    return dflt;
#endif
}

// y[M] = W x, f32 arithmetic.  `cus` = compute units of the current device.
hipError_t launch_gemv(int dtype, const void *blob, int64_t M, int64_t K, const float *x, float *y,
                       hipStream_t st, int cus);

// y_i = W_i x for n <= 4 matrices sharing K, in one launch where the layout
// allows (else one launch per matrix); bits equal launch_gemv's.
hipError_t launch_gemv_concat(int n, const void *const *blobs, const int64_t *Ms, int dtype, int64_t K,
                              const float *x, float *const *ys, hipStream_t st, int cus);

// out = silu(W_gate x) * (W_up x), one launch.  Needs gemv_fused_ok(dtype, K).
hipError_t launch_gemv_swiglu(int dtype, const void *gate, const void *up, int64_t M, int64_t K, const float *x,
                              float *out, hipStream_t st, int cus);
bool gemv_fused_ok(int dtype, int64_t K);

// index = the smallest row with the largest f32 GEMV output (bits of
// launch_gemv), value = that output; two launches (rows, then the winner
// among QMM_ARGMAX_WORK_BYTES / 8 workgroup candidates in `work`).  q8: the
// outputs of the int8 GEMV with x quantized in the launch instead.
hipError_t launch_gemv_argmax(int dtype, const void *blob, int64_t M, int64_t K, const float *x, void *work,
                              int64_t *index, float *value, hipStream_t st, int cus, bool q8 = false);

// Y[N][M] for a few tokens with the GEMV's f32 arithmetic, the weights read
// once per 4 tokens; each Y[n] has the bits launch_gemv gives for X[n].
// Needs gemv_tokens_ok(dtype, K) (whole-row wavefronts: K <= 4096).
bool gemv_tokens_ok(int dtype, int64_t K);
hipError_t launch_gemv_tokens(int dtype, const void *blob, int64_t M, int64_t K, int64_t N, const float *X,
                              float *Y, hipStream_t st, int cus);

// Y[N][M] = silu(X Wg^T) * (X Wu^T) on the matrix cores (one launch).
bool gemm_swiglu_ok(int dtype, int64_t K);
// Which SwiGLU tile launch_gemm_swiglu runs for these sizes (1..5, see
// qmm_gemm.hip).
int swiglu_tile(int64_t M, int64_t N);
hipError_t launch_gemm_swiglu(int dtype, const void *gate, const void *up, int64_t M, int64_t K, int64_t N,
                              const float *X, float *Y, hipStream_t st);

// Which matrix-core kernel launch_gemm_mfma runs for these sizes (one of the
// GEMM_K_* ids in qmm_gemm.hip), or -1 if dtype is unknown.
int gemm_kernel_choice(int dtype, int64_t M, int64_t K, int64_t N);

// Y[N][M] = X W^T on the matrix cores (f16 operands, f32 accumulation).
hipError_t launch_gemm_mfma(int dtype, const void *blob, int64_t M, int64_t K, int64_t N, const float *X,
                            float *Y, hipStream_t st);

// Q6_K / Q8_0 repacked for the GEMM: M rows of K weights from the GGUF blob
// into the QMM_Q6_K_R / QMM_Q8_0_R layout (K % 256 == 0); and the matrix-core
// GEMM on it, with the kernel choice of gemm_kernel_choice(dtype, ...)
// (gemm_repacked_ok: a repacked dtype whose K the register-B kernels take).
hipError_t launch_repack(int dtype, const void *src, int64_t M, int64_t K, void *dst, hipStream_t st);
bool gemm_repacked_ok(int dtype, int64_t K);
int gemm_repacked_kernel_choice(int dtype, int64_t M, int64_t K, int64_t N);
hipError_t launch_gemm_repacked(int dtype, const void *packed, int64_t M, int64_t K, int64_t N, const float *X,
                                float *Y, hipStream_t st);

// A plain streaming read of `bytes` bytes of buf (at most cus * 4 workgroups,
// one float per workgroup written to out).
hipError_t launch_read_probe(const void *buf, int64_t bytes, float *out, hipStream_t st, int cus);

// Q8_0 quantization of N activation rows of K (K % 32 == 0): scales f32
// [N][K/32], codes int8 [N][K].
hipError_t launch_quantize_q8_0(const float *X, int64_t N, int64_t K, float *scales, int8_t *quants,
                                hipStream_t st);

// Y[N][M] = W Xq^T with Q8_0-quantized activations (integer block dots, f32
// scaling); up to 4 tokens per weight read.
hipError_t launch_gemm_q8act(int dtype, const void *blob, int64_t M, int64_t K, int64_t N, const float *xsc,
                             const int8_t *xq, float *Y, hipStream_t st, int cus);

// The int8-activation matmul on the matrix cores (Q8_0, Q4_0, Q4_K; see
// gemm_i8_ok for the shapes): one int8 matrix step per activation block, each
// block sum scaled once in f32.
bool gemm_i8_ok(int dtype, int64_t M, int64_t K, int64_t N);
// Whether launch_gemm_q8act runs these sizes on the int8 matrix cores.
bool q8_use_mfma(int dtype, int64_t M, int64_t K, int64_t N);
hipError_t launch_gemm_q8act_mfma(int dtype, const void *blob, int64_t M, int64_t K, int64_t N, const float *xsc,
                                  const int8_t *xq, float *Y, hipStream_t st);

// One token of f32 activations quantized to Q8_0 inside the launch, then the
// int8 dots (codes and results bit-identical to launch_quantize_q8_0 followed
// by launch_gemm_q8act with N = 1).  mode 0: one matrix, 1: n <= 4 matrices
// sharing K and x, 2: gate/up with SwiGLU (blobs = {gate, up}, one output).
// Needs gemv_fused_ok(dtype, K).
hipError_t launch_gemv_q8in(int mode, int n, const void *const *blobs, const int64_t *Ms, int dtype, int64_t K,
                            const float *x, float *const *ys, hipStream_t st, int cus);

}  // namespace qmm
