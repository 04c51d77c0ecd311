// qmm_api.hip -- the C ABI declared in include/qmm.h: argument checks, device
// check, path selection, launch.  No allocation, no host synchronisation.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "qmm.h"
#include "qmm_internal.hpp"

namespace {

struct DeviceInfo {
    std::atomic<int> state{0};  // 0 unknown, 1 gfx950, 2 other
    int cus = 0;
};
constexpr int kMaxDevices = 64;
DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

int block_elems(int dtype) {
    switch (dtype) {
    case QMM_Q4_0:
    case QMM_Q4_1:
    case QMM_Q8_0: return 32;
    case QMM_Q4_K:
    case QMM_Q5_K:
    case QMM_Q6_K: return 256;
    default: return 0;
    }
}

int block_bytes(int dtype) {
    switch (dtype) {
    case QMM_Q4_0: return 18;
    case QMM_Q4_1: return 20;
    case QMM_Q8_0: return 34;
    case QMM_Q4_K: return 144;
    case QMM_Q5_K: return 176;
    case QMM_Q6_K: return 210;
    default: return 0;
    }
}

int check_shape(int dtype, int64_t M, int64_t K, int64_t N) {
    const int bs = block_elems(dtype);
    if (bs == 0) return QMM_ERR_DTYPE;
    if (M < 1 || N < 1 || K < bs || K % bs != 0) return QMM_ERR_SHAPE;
    // keep every byte offset and grid size inside 63 bits / the launch limits:
    // each size and each product of two of them
    constexpr int64_t kMax = int64_t(1) << 40, kMaxProd = int64_t(1) << 56;
    if (M > kMax || K > kMax || N > kMax) return QMM_ERR_SHAPE;
    if (M > kMaxProd / K || N > kMaxProd / K || N > kMaxProd / M) return QMM_ERR_SHAPE;
    return QMM_OK;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Current device must be gfx950; returns its compute-unit count through *cus
// (and its index through *dev_out).
int current_device(int *cus, int *dev_out = nullptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QMM_ERR_DEVICE;
    DeviceInfo &d = g_dev[dev];
    int st = d.state.load(std::memory_order_acquire);
    if (st == 0) {
        std::lock_guard<std::mutex> lk(g_dev_mu);
        st = d.state.load(std::memory_order_relaxed);
        if (st == 0) {
            hipDeviceProp_t prop;
            if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return QMM_ERR_DEVICE;
            const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
            d.cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
            st = ok ? 1 : 2;
            d.state.store(st, std::memory_order_release);
        }
    }
    if (st != 1) return QMM_ERR_DEVICE;
    *cus = d.cus;
    if (dev_out) *dev_out = dev;
    return QMM_OK;
}

// The scratch of the entry points that take no workspace (for callers that
// cannot allocate): one array per GPU, held until the process ends.  Host code
// never uses the array's name as an address (on the host it is only a
// stand-in): the device address of each GPU's copy is looked up once, with
// that GPU current, and kept in g_scratch.
__device__ __attribute__((aligned(256))) unsigned char scratch[QMM_NOALLOC_SCRATCH_BYTES];
std::atomic<void *> g_scratch[kMaxDevices];

// The device address of the current GPU's scratch (dev = its index).
int scratch_of(int dev, void **p) {
    void *v = g_scratch[dev].load(std::memory_order_acquire);
    if (!v) {
        std::lock_guard<std::mutex> lk(g_dev_mu);
        v = g_scratch[dev].load(std::memory_order_relaxed);
        if (!v) {
            if (hipGetSymbolAddress(&v, HIP_SYMBOL(scratch)) != hipSuccess || !v) return QMM_ERR_DEVICE;
            g_scratch[dev].store(v, std::memory_order_release);
        }
    }
    *p = v;
    return QMM_OK;
}

// N at and above which the f16 matrix-core GEMM runs; below it the f32 GEMV
// arithmetic runs for every token.  Measured on 4096-, 14336- and
// 128256-row weights:
//   * where the several-token GEMV applies (K <= 4096): up to 4 tokens share
//     one weight read and beat the matrix cores for Q4_0, Q8_0 and Q6_K
//     (e.g. the 128256 x 4096 Q6_K head at N = 4: 194 vs 241 us; 14336 x 4096
//     Q8_0: 26 vs 29 us) and Q4_1 (14336 x 4096 at N = 4: 22.6 vs 24.4 us), up
//     to 2 for Q4_K (17 vs 21 us at N = 2, 21 vs 20 us at N = 3);
//   * elsewhere one GEMV launch per token: two tie with the GEMM at N = 2
//     for Q4_0 and beat it for Q6_K; for Q8_0 and Q4_K the GEMM already wins.
// A measurement build (QMM_TUNING) takes QMM_GEMM_MFMA_FROM_N = n to move it;
// the shipped library reads no environment.
int64_t mfma_from_n(int dtype, int64_t M, int64_t K) {
    static const int64_t lever = [] {
        const int v = qmm::tuning_lever("QMM_GEMM_MFMA_FROM_N", 0);
        return (int64_t)(v >= 1 && v <= 1024 ? v : 0);
    }();
    if (lever) return lever;
    if (qmm::gemv_tokens_ok(dtype, K)) {
        // Up to 4096 rows the matrix-core kernels have few tiles and the GEMV
        // arithmetic (4 tokens per weight read, one launch per 4 tokens) stays
        // ahead longer (K = 4096, f32 against matrix cores): Q4_K 4096 rows N =
        // 3 / 4 8.2 / 9.6 against 10.0 us, 2048 rows 6.1 / 6.8 against 9.8;
        // Q6_K 4096 rows N = 5 / 7 14.8 / 17.9 against 18.7, 2048 rows N = 5 /
        // 7 10.8 / 12.9 against 18.1; Q4_0 2048 rows N = 5 / 6 9.2 / 9.9
        // against 10.8; Q8_0 2048 rows N = 7 12.4 against 12.8.
        const bool small = M <= 4096, tiny = M <= 2048;
        if (dtype == QMM_Q4_K) return small ? 5 : 3;
        if (dtype == QMM_Q5_K) return 3;
        if (dtype == QMM_Q6_K) return small ? 8 : 5;
        if (tiny && dtype == QMM_Q4_0) return 7;
        if (tiny && dtype == QMM_Q8_0) return 8;
        // tall Q4_1 (>= 192 two-fragment row tiles, where the small-N GEMM
        // halves its activation traffic): the matrix cores win from N = 4
        // (14336 x 4096: 21.2 vs 22.9-23.1 us)
        if (dtype == QMM_Q4_1 && (M + 63) / 64 >= 192) return 4;
        return 5;
    }
    return (dtype == QMM_Q4_0 || dtype == QMM_Q6_K) ? 3 : 2;
}

}  // namespace

extern "C" {

int qmm_block_elems(int dtype) { return block_elems(dtype); }
int qmm_block_bytes(int dtype) { return block_bytes(dtype); }

int64_t qmm_blob_bytes(int dtype, int64_t M, int64_t K) {
    if (check_shape(dtype, M, K, 1) != QMM_OK) return 0;
    return M * (K / block_elems(dtype)) * block_bytes(dtype);
}

const char *qmm_strerror(int code) {
    switch (code) {
    case QMM_OK: return "ok";
    case QMM_ERR_NULL: return "a required pointer is NULL";
    case QMM_ERR_DTYPE: return "unsupported dtype (expected Q4_0=2, Q4_1=3, Q8_0=8, Q4_K=12, Q5_K=13 or Q6_K=14)";
    case QMM_ERR_SHAPE: return "bad shape (need M >= 1, N >= 1, K a positive multiple of the block size)";
    case QMM_ERR_ALIGN: return "misaligned pointer (blob and x/X need 16-byte, y/Y 4-byte alignment)";
    case QMM_ERR_DEVICE: return "no current HIP device, or it is not gfx950";
    case QMM_ERR_LAUNCH: return "kernel launch failed";
    case QMM_ERR_SCRATCH: return "the call needs more scratch than the library's static buffer holds";
    default: return "unknown status code";
    }
}

int qmm_gemm_path(int dtype, int64_t M, int64_t K, int64_t N) {
    const int rc = check_shape(dtype, M, K, N);
    if (rc != QMM_OK) return rc;
    return N >= mfma_from_n(dtype, M, K) ? 1 : 0;
}

int qmm_gemm_kernel(int dtype, int64_t M, int64_t K, int64_t N) {
    const int rc = check_shape(dtype, M, K, N);
    if (rc != QMM_OK) return rc;
    if (N < mfma_from_n(dtype, M, K))
        return (N > 1 && qmm::gemv_tokens_ok(dtype, K)) ? QMM_KERNEL_GEMV_TOKENS : QMM_KERNEL_GEMV;
    return qmm::gemm_kernel_choice(dtype, M, K, N);
}

int qmm_gemm_swiglu_kernel(int dtype, int64_t M, int64_t K, int64_t N) {
    const int rc = check_shape(dtype, M, K, N);
    if (rc != QMM_OK) return rc;
    if (N < mfma_from_n(dtype, M, K)) return qmm::gemv_fused_ok(dtype, K) ? QMM_KERNEL_GEMV : QMM_ERR_SHAPE;
    if (!qmm::gemm_swiglu_ok(dtype, K)) return QMM_ERR_SHAPE;
    return qmm::swiglu_tile(M, N);
}

int qmm_gemm_q8act_path(int dtype, int64_t M, int64_t K, int64_t N) {
    const int rc = check_shape(dtype, M, K, N);
    if (rc != QMM_OK) return rc;
    return qmm::q8_use_mfma(dtype, M, K, N) ? 1 : 0;
}

// The repacked forms: Q6_K 320 bytes per 256 weights, Q8_0 72 bytes per 64
// (K a multiple of 256 for both, as the GEMM on them needs).
int64_t qmm_repack_bytes(int dtype, int64_t M, int64_t K) {
    if ((dtype != QMM_Q6_K && dtype != QMM_Q8_0) || check_shape(dtype, M, K, 1) != QMM_OK || K % 256 != 0) return 0;
    return dtype == QMM_Q6_K ? M * (K / 256) * 320 : M * (K / 64) * 72;
}

int qmm_repack(const void *w_blob, int dtype, int64_t M, int64_t K, void *packed, void *stream) {
    int rc = check_shape(dtype, M, K, 1);
    if (rc != QMM_OK) return rc;
    if (dtype != QMM_Q6_K && dtype != QMM_Q8_0) return QMM_ERR_DTYPE;
    if (K % 256 != 0) return QMM_ERR_SHAPE;
    if (!w_blob || !packed) return QMM_ERR_NULL;
    if (!aligned(w_blob, 16) || !aligned(packed, 16)) return QMM_ERR_ALIGN;
    int cus = 0;
    rc = current_device(&cus);
    if (rc != QMM_OK) return rc;
    const hipError_t e = qmm::launch_repack(dtype, w_blob, M, K, packed, (hipStream_t)stream);
    return e == hipSuccess ? QMM_OK : QMM_ERR_LAUNCH;
}

int qmm_gemm_repacked(const void *packed, int dtype, int64_t M, int64_t K, int64_t N, const float *X, float *Y,
                      void *stream) {
    int rc = check_shape(dtype, M, K, N);
    if (rc != QMM_OK) return rc;
    if (dtype != QMM_Q6_K && dtype != QMM_Q8_0) return QMM_ERR_DTYPE;
    if (!qmm::gemm_repacked_ok(dtype, K)) return QMM_ERR_SHAPE;
    if (!packed || !X || !Y) return QMM_ERR_NULL;
    if (!aligned(packed, 16) || !aligned(X, 16) || !aligned(Y, 4)) return QMM_ERR_ALIGN;
    int cus = 0;
    rc = current_device(&cus);
    if (rc != QMM_OK) return rc;
    const hipError_t e = qmm::launch_gemm_repacked(dtype, packed, M, K, N, X, Y, (hipStream_t)stream);
    return e == hipSuccess ? QMM_OK : QMM_ERR_LAUNCH;
}

int qmm_gemm_repacked_kernel(int dtype, int64_t M, int64_t K, int64_t N) {
    const int rc = check_shape(dtype, M, K, N);
    if (rc != QMM_OK) return rc;
    if (dtype != QMM_Q6_K && dtype != QMM_Q8_0) return QMM_ERR_DTYPE;
    if (!qmm::gemm_repacked_ok(dtype, K)) return QMM_ERR_SHAPE;
    return qmm::gemm_repacked_kernel_choice(dtype, M, K, N);
}

int qmm_read_probe(const void *buf, int64_t bytes, float *out, void *stream) {
    if (bytes < 1 || bytes > (int64_t(1) << 40)) return QMM_ERR_SHAPE;
    if (!buf || !out) return QMM_ERR_NULL;
    if (!aligned(buf, 16) || !aligned(out, 4)) return QMM_ERR_ALIGN;
    int cus = 0;
    const int rc = current_device(&cus);
    if (rc != QMM_OK) return rc;
    const hipError_t e = qmm::launch_read_probe(buf, bytes, out, (hipStream_t)stream, cus);
    return e == hipSuccess ? QMM_OK : QMM_ERR_LAUNCH;
}

int qmm_gemv(const void *w_blob, int dtype, int64_t M, int64_t K, const float *x, float *y, void *stream) {
    int rc = check_shape(dtype, M, K, 1);
    if (rc != QMM_OK) return rc;
    if (!w_blob || !x || !y) return QMM_ERR_NULL;
    if (!aligned(w_blob, 16) || !aligned(x, 16) || !aligned(y, 4)) return QMM_ERR_ALIGN;
    int cus = 0;
    rc = current_device(&cus);
    if (rc != QMM_OK) return rc;
    const hipError_t e = qmm::launch_gemv(dtype, w_blob, M, K, x, y, (hipStream_t)stream, cus);
    return e == hipSuccess ? QMM_OK : QMM_ERR_LAUNCH;
}

int qmm_gemv_concat(int n, const void *const *w_blobs, const int64_t *Ms, int dtype, int64_t K, const float *x,
                    float *const *ys, void *stream) {
    if (n < 1 || n > QMM_GEMV_MAX_MATS) return QMM_ERR_SHAPE;
    if (!w_blobs || !Ms || !ys || !x) return QMM_ERR_NULL;
    for (int i = 0; i < n; i++) {
        const int rc = check_shape(dtype, Ms[i], K, 1);
        if (rc != QMM_OK) return rc;
        if (!w_blobs[i] || !ys[i]) return QMM_ERR_NULL;
        if (!aligned(w_blobs[i], 16) || !aligned(ys[i], 4)) return QMM_ERR_ALIGN;
    }
    if (!aligned(x, 16)) return QMM_ERR_ALIGN;
    int cus = 0;
    const int rc = current_device(&cus);
    if (rc != QMM_OK) return rc;
    const hipError_t e = qmm::launch_gemv_concat(n, w_blobs, Ms, dtype, K, x, ys, (hipStream_t)stream, cus);
    return e == hipSuccess ? QMM_OK : QMM_ERR_LAUNCH;
}

int qmm_gemv_swiglu(const void *gate_blob, const void *up_blob, int dtype, int64_t M, int64_t K, const float *x,
                    float *out, void *stream) {
    int rc = check_shape(dtype, M, K, 1);
    if (rc != QMM_OK) return rc;
    if (!qmm::gemv_fused_ok(dtype, K)) return QMM_ERR_SHAPE;
    if (!gate_blob || !up_blob || !x || !out) return QMM_ERR_NULL;
    if (!aligned(gate_blob, 16) || !aligned(up_blob, 16) || !aligned(x, 16) || !aligned(out, 4)) return QMM_ERR_ALIGN;
    int cus = 0;
    rc = current_device(&cus);
    if (rc != QMM_OK) return rc;
    const hipError_t e = qmm::launch_gemv_swiglu(dtype, gate_blob, up_blob, M, K, x, out, (hipStream_t)stream, cus);
    return e == hipSuccess ? QMM_OK : QMM_ERR_LAUNCH;
}

int qmm_gemv_argmax(const void *w_blob, int dtype, int64_t M, int64_t K, const float *x, void *work,
                    int64_t *index, float *value, void *stream) {
    int rc = check_shape(dtype, M, K, 1);
    if (rc != QMM_OK) return rc;
    if (M > INT32_MAX || !qmm::gemv_fused_ok(dtype, K)) return QMM_ERR_SHAPE;
    if (!w_blob || !x || !work || !index) return QMM_ERR_NULL;
    if (!aligned(w_blob, 16) || !aligned(x, 16) || !aligned(work, 16) || !aligned(index, 8) ||
        (value && !aligned(value, 4)))
        return QMM_ERR_ALIGN;
    int cus = 0;
    rc = current_device(&cus);
    if (rc != QMM_OK) return rc;
    const hipError_t e = qmm::launch_gemv_argmax(dtype, w_blob, M, K, x, work, index, value, (hipStream_t)stream, cus);
    return e == hipSuccess ? QMM_OK : QMM_ERR_LAUNCH;
}

int qmm_gemv_argmax_noalloc(const void *w_blob, int dtype, int64_t M, int64_t K, const float *x, int64_t *index,
                            float *value, void *stream) {
    int rc = check_shape(dtype, M, K, 1);
    if (rc != QMM_OK) return rc;
    if (M > INT32_MAX || !qmm::gemv_fused_ok(dtype, K)) return QMM_ERR_SHAPE;
    if (!w_blob || !x || !index) return QMM_ERR_NULL;
    if (!aligned(w_blob, 16) || !aligned(x, 16) || !aligned(index, 8) || (value && !aligned(value, 4)))
        return QMM_ERR_ALIGN;
    int cus = 0, dev = -1;
    rc = current_device(&cus, &dev);
    if (rc != QMM_OK) return rc;
    void *work = nullptr;
    rc = scratch_of(dev, &work);
    if (rc != QMM_OK) return rc;
    // the candidates of every valid shape fit (at most QMM_NOALLOC_SCRATCH_BYTES / 8
    // workgroups); a launch that would need more is refused before it starts
    const hipError_t e = qmm::launch_gemv_argmax(dtype, w_blob, M, K, x, work, index, value, (hipStream_t)stream, cus);
    if (e == hipErrorInvalidConfiguration) return QMM_ERR_SCRATCH;
    return e == hipSuccess ? QMM_OK : QMM_ERR_LAUNCH;
}

int qmm_gemv_argmax_q8act(const void *w_blob, int dtype, int64_t M, int64_t K, const float *x, void *work,
                          int64_t *index, float *value, void *stream) {
    int rc = check_shape(dtype, M, K, 1);
    if (rc != QMM_OK) return rc;
    if (M > INT32_MAX || !qmm::gemv_fused_ok(dtype, K)) return QMM_ERR_SHAPE;
    if (!w_blob || !x || !work || !index) return QMM_ERR_NULL;
    if (!aligned(w_blob, 16) || !aligned(x, 16) || !aligned(work, 16) || !aligned(index, 8) ||
        (value && !aligned(value, 4)))
        return QMM_ERR_ALIGN;
    int cus = 0;
    rc = current_device(&cus);
    if (rc != QMM_OK) return rc;
    const hipError_t e =
        qmm::launch_gemv_argmax(dtype, w_blob, M, K, x, work, index, value, (hipStream_t)stream, cus, true);
    return e == hipSuccess ? QMM_OK : QMM_ERR_LAUNCH;
}

int qmm_gemm_swiglu(const void *gate_blob, const void *up_blob, int dtype, int64_t M, int64_t K, int64_t N,
                    const float *X, float *out, void *stream) {
    int rc = check_shape(dtype, M, K, N);
    if (rc != QMM_OK) return rc;
    const bool f32 = N < mfma_from_n(dtype, M, K);
    if (f32 ? !qmm::gemv_fused_ok(dtype, K) : !qmm::gemm_swiglu_ok(dtype, K)) return QMM_ERR_SHAPE;
    if (!gate_blob || !up_blob || !X || !out) return QMM_ERR_NULL;
    if (!aligned(gate_blob, 16) || !aligned(up_blob, 16) || !aligned(X, 16) || !aligned(out, 4)) return QMM_ERR_ALIGN;
    int cus = 0;
    rc = current_device(&cus);
    if (rc != QMM_OK) return rc;
    hipError_t e = hipSuccess;
    if (f32) {
        // the decode form per token: its bits, token by token
        for (int64_t n = 0; n < N && e == hipSuccess; n++)
            e = qmm::launch_gemv_swiglu(dtype, gate_blob, up_blob, M, K, X + n * K, out + n * M, (hipStream_t)stream,
                                        cus);
    } else {
        e = qmm::launch_gemm_swiglu(dtype, gate_blob, up_blob, M, K, N, X, out, (hipStream_t)stream);
    }
    return e == hipSuccess ? QMM_OK : QMM_ERR_LAUNCH;
}

int qmm_quantize_q8_0(const float *X, int64_t N, int64_t K, float *scales, int8_t *quants, void *stream) {
    if (N < 1 || K < 32 || K % 32 != 0 || N > (int64_t(1) << 40) || K > (int64_t(1) << 40) ||
        N > (int64_t(1) << 56) / K)
        return QMM_ERR_SHAPE;
    if (!X || !scales || !quants) return QMM_ERR_NULL;
    if (!aligned(X, 16) || !aligned(scales, 16) || !aligned(quants, 16)) return QMM_ERR_ALIGN;
    int cus = 0;
    const int rc = current_device(&cus);
    if (rc != QMM_OK) return rc;
    const hipError_t e = qmm::launch_quantize_q8_0(X, N, K, scales, quants, (hipStream_t)stream);
    return e == hipSuccess ? QMM_OK : QMM_ERR_LAUNCH;
}

int qmm_gemm_q8act(const void *w_blob, int dtype, int64_t M, int64_t K, int64_t N, const float *scales,
                   const int8_t *quants, float *Y, void *stream) {
    int rc = check_shape(dtype, M, K, N);
    if (rc != QMM_OK) return rc;
    if (!w_blob || !scales || !quants || !Y) return QMM_ERR_NULL;
    if (!aligned(w_blob, 16) || !aligned(scales, 16) || !aligned(quants, 16) || !aligned(Y, 4)) return QMM_ERR_ALIGN;
    int cus = 0;
    rc = current_device(&cus);
    if (rc != QMM_OK) return rc;
    const hipError_t e = qmm::launch_gemm_q8act(dtype, w_blob, M, K, N, scales, quants, Y, (hipStream_t)stream, cus);
    return e == hipSuccess ? QMM_OK : QMM_ERR_LAUNCH;
}

int qmm_gemv_q8act(const void *w_blob, int dtype, int64_t M, int64_t K, const float *x, float *y, void *stream) {
    int rc = check_shape(dtype, M, K, 1);
    if (rc != QMM_OK) return rc;
    if (!qmm::gemv_fused_ok(dtype, K)) return QMM_ERR_SHAPE;
    if (!w_blob || !x || !y) return QMM_ERR_NULL;
    if (!aligned(w_blob, 16) || !aligned(x, 16) || !aligned(y, 4)) return QMM_ERR_ALIGN;
    int cus = 0;
    rc = current_device(&cus);
    if (rc != QMM_OK) return rc;
    const void *blobs[1] = {w_blob};
    const int64_t Ms[1] = {M};
    float *ys[1] = {y};
    const hipError_t e = qmm::launch_gemv_q8in(0, 1, blobs, Ms, dtype, K, x, ys, (hipStream_t)stream, cus);
    return e == hipSuccess ? QMM_OK : QMM_ERR_LAUNCH;
}

int qmm_gemv_concat_q8act(int n, const void *const *w_blobs, const int64_t *Ms, int dtype, int64_t K,
                          const float *x, float *const *ys, void *stream) {
    if (n < 1 || n > QMM_GEMV_MAX_MATS) return QMM_ERR_SHAPE;
    if (!w_blobs || !Ms || !ys || !x) return QMM_ERR_NULL;
    for (int i = 0; i < n; i++) {
        const int rc = check_shape(dtype, Ms[i], K, 1);
        if (rc != QMM_OK) return rc;
        if (!w_blobs[i] || !ys[i]) return QMM_ERR_NULL;
        if (!aligned(w_blobs[i], 16) || !aligned(ys[i], 4)) return QMM_ERR_ALIGN;
    }
    if (!qmm::gemv_fused_ok(dtype, K)) return QMM_ERR_SHAPE;
    if (!aligned(x, 16)) return QMM_ERR_ALIGN;
    int cus = 0;
    const int rc = current_device(&cus);
    if (rc != QMM_OK) return rc;
    const hipError_t e = qmm::launch_gemv_q8in(1, n, w_blobs, Ms, dtype, K, x, ys, (hipStream_t)stream, cus);
    return e == hipSuccess ? QMM_OK : QMM_ERR_LAUNCH;
}

int qmm_gemv_swiglu_q8act(const void *gate_blob, const void *up_blob, int dtype, int64_t M, int64_t K,
                          const float *x, float *out, void *stream) {
    int rc = check_shape(dtype, M, K, 1);
    if (rc != QMM_OK) return rc;
    if (!qmm::gemv_fused_ok(dtype, K)) return QMM_ERR_SHAPE;
    if (!gate_blob || !up_blob || !x || !out) return QMM_ERR_NULL;
    if (!aligned(gate_blob, 16) || !aligned(up_blob, 16) || !aligned(x, 16) || !aligned(out, 4)) return QMM_ERR_ALIGN;
    int cus = 0;
    rc = current_device(&cus);
    if (rc != QMM_OK) return rc;
    const void *blobs[2] = {gate_blob, up_blob};
    const int64_t Ms[2] = {M, M};
    float *ys[2] = {out, out};
    const hipError_t e = qmm::launch_gemv_q8in(2, 2, blobs, Ms, dtype, K, x, ys, (hipStream_t)stream, cus);
    return e == hipSuccess ? QMM_OK : QMM_ERR_LAUNCH;
}

int qmm_gemm(const void *w_blob, int dtype, int64_t M, int64_t K, int64_t N, const float *X, float *Y,
             void *stream) {
    int rc = check_shape(dtype, M, K, N);
    if (rc != QMM_OK) return rc;
    if (!w_blob || !X || !Y) return QMM_ERR_NULL;
    if (!aligned(w_blob, 16) || !aligned(X, 16) || !aligned(Y, 4)) return QMM_ERR_ALIGN;
    int cus = 0;
    rc = current_device(&cus);
    if (rc != QMM_OK) return rc;
    hipError_t e = hipSuccess;
    if (N < mfma_from_n(dtype, M, K)) {
        // the GEMV's bits, token by token: several tokens per weight read where
        // the layout allows, else one GEMV launch per token
        if (N > 1 && qmm::gemv_tokens_ok(dtype, K)) {
            e = qmm::launch_gemv_tokens(dtype, w_blob, M, K, N, X, Y, (hipStream_t)stream, cus);
        } else {
            for (int64_t n = 0; n < N && e == hipSuccess; n++)
                e = qmm::launch_gemv(dtype, w_blob, M, K, X + n * K, Y + n * M, (hipStream_t)stream, cus);
        }
    } else {
        e = qmm::launch_gemm_mfma(dtype, w_blob, M, K, N, X, Y, (hipStream_t)stream);
    }
    return e == hipSuccess ? QMM_OK : QMM_ERR_LAUNCH;
}

}  // extern "C"
