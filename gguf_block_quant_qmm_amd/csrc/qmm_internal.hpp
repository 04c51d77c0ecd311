// qmm_internal.hpp -- launchers shared between the HIP sources of libqmm.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

// y[M] = W x, f32 arithmetic.  `cus` = compute units of the current device.
hipError_t launch_gemv(int dtype, const void *blob, int64_t M, int64_t K, const float *x, float *y,
                       hipStream_t st, int cus);

// Y[N][M] = X W^T on the matrix cores (f16 operands, f32 accumulation).
hipError_t launch_gemm_mfma(int dtype, const void *blob, int64_t M, int64_t K, int64_t N, const float *X,
                            float *Y, hipStream_t st);

}  // namespace qmm
