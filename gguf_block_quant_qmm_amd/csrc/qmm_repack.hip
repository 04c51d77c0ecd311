// qmm_repack.hip -- load-time repacking of Q6_K and Q8_0 weights for the
// matrix-core GEMM (page "cera 0.5.2 src/backend/cpu.rs", the Q4_0 / Q4_K weight
// repacking: a second copy of a prefill weight, built once at load and kept
// beside the GGUF bytes, laid out for the GEMM's lanes with the per-block
// scale products baked in; decode keeps reading the original).
//
// The GGUF Q6_K super-block (256 weights, 210 bytes: ql[128], qh[64], int8
// sc[16], f16 d) is 2 bytes off a dword on every other block, and a weight's
// 6-bit code sits in two places (a nibble of ql, two bits of qh).  The
// repacked super-block is 320 bytes, 16-byte aligned:
//   [0, 256)   one byte per weight, q in 0..63 (the weight is d sc (q - 32));
//              weight k at byte 64c + 32kh + 8s + j for k = 64c + 16s + 8kh + j
//              (c, s < 4; kh, j: kh < 2, j < 8), so a GEMM lane reads its
//              k-tile's codes with two 16-byte loads;
//   [256, 320) the 16 sub-block scales d * sc[i] as f32 (exact: an 11-bit
//              times an 8-bit integer significand).
// 1.52 x the source bytes.
//
// One thread per 16-weight sub-block: it reads its 16 low nibbles (ql), 16
// high-bit pairs (qh), sc[i] and d, and writes 2 x 8 code bytes and 1 scale.
//
// Q8_0 (32 weights, 34 bytes: f16 d, int8 q[32]; 2 bytes off a dword on every
// other block) is repacked per pair of blocks into 72 bytes:
//   [0, 64)    the 64 codes as q + 128 (unsigned bytes), in order;
//   [64, 72)   d of both blocks as f32.
// 1.06 x the source bytes.  One thread per block.
#include "qmm_device.hpp"
#include "qmm_internal.hpp"

namespace qmm {

namespace {

__global__ void __launch_bounds__(256) repack_q6_k_kernel(const uint8_t *__restrict__ src, int64_t nsub,
                                                          uint8_t *__restrict__ dst) {
    const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gt >= nsub) return;
    const int64_t sb = gt >> 4;
    const int i = (int)(gt & 15);  // sub-block: weights 16i .. 16i + 15 of the super-block
    const uint8_t *b = src + 210 * sb;
    // GGUF element j = 128h + 32g + l: low nibble (g < 2) or high nibble of
    // ql[64h + 32(g & 1) + l], plus bits 2g, 2g+1 of qh[32h + l] as bits 4, 5
    const int h = i >> 3, g = (i & 7) >> 1, l0 = 16 * (i & 1);
    const uint8_t *ql = b + 64 * h + 32 * (g & 1) + l0;
    const uint8_t *qh = b + 128 + 32 * h + l0;
    uint8_t q[16];
#pragma unroll
    for (int t = 0; t < 16; t++) {
        const int lo = g < 2 ? (ql[t] & 15) : (ql[t] >> 4);
        q[t] = (uint8_t)(lo | (((qh[t] >> (2 * g)) & 3) << 4));
    }
    const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)(b[208] | (b[209] << 8)));
    const float dsc = d * (float)(int8_t)b[192 + i];
    uint8_t *o = dst + 320 * sb;
    const int c = i >> 2, s = i & 3;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; k++)
        w[k] = (uint32_t)q[4 * k] | ((uint32_t)q[4 * k + 1] << 8) | ((uint32_t)q[4 * k + 2] << 16) |
               ((uint32_t)q[4 * k + 3] << 24);
    // weights 16i + t: t < 8 to lane half 0, t >= 8 to lane half 1
    *reinterpret_cast<uint2 *>(o + 64 * c + 8 * s) = uint2{w[0], w[1]};
    *reinterpret_cast<uint2 *>(o + 64 * c + 32 + 8 * s) = uint2{w[2], w[3]};
    *reinterpret_cast<float *>(o + 256 + 4 * i) = dsc;
}

__global__ void __launch_bounds__(256) repack_q8_0_kernel(const uint8_t *__restrict__ src, int64_t nblk,
                                                          uint8_t *__restrict__ dst) {
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblk) return;
    const uint8_t *p = src + 34 * b;
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; k++)
        w[k] = ((uint32_t)p[2 + 4 * k] | ((uint32_t)p[3 + 4 * k] << 8) | ((uint32_t)p[4 + 4 * k] << 16) |
                ((uint32_t)p[5 + 4 * k] << 24)) ^ 0x80808080u;  // q + 128 in each byte
    const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)(p[0] | (p[1] << 8)));
    uint8_t *o = dst + 72 * (b >> 1);
    const int h = (int)(b & 1);
    *reinterpret_cast<uint4 *>(o + 32 * h) = uint4{w[0], w[1], w[2], w[3]};
    *reinterpret_cast<uint4 *>(o + 32 * h + 16) = uint4{w[4], w[5], w[6], w[7]};
    *reinterpret_cast<float *>(o + 64 + 4 * h) = d;
}

hipError_t launch_repack_q6_k(const void *src, int64_t M, int64_t K, void *dst, hipStream_t st) {
    const int64_t nsub = M * (K / 256) * 16;
    // a dispatch counts its work-items in 32 bits: at most 2^26 sub-blocks
    // (2^22 super-blocks) per launch
    const int64_t max_sub = (int64_t)1 << 26;
    for (int64_t s0 = 0; s0 < nsub; s0 += max_sub) {
        const int64_t n = nsub - s0 < max_sub ? nsub - s0 : max_sub;
        hipLaunchKernelGGL(repack_q6_k_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                           static_cast<const uint8_t *>(src) + (s0 / 16) * 210, n,
                           static_cast<uint8_t *>(dst) + (s0 / 16) * 320);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_repack_q8_0(const void *src, int64_t M, int64_t K, void *dst, hipStream_t st) {
    const int64_t nblk = M * (K / 32);
    const int64_t max_blk = (int64_t)1 << 26;  // even: chunks start on a block pair
    for (int64_t b0 = 0; b0 < nblk; b0 += max_blk) {
        const int64_t n = nblk - b0 < max_blk ? nblk - b0 : max_blk;
        hipLaunchKernelGGL(repack_q8_0_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                           static_cast<const uint8_t *>(src) + b0 * 34, n,
                           static_cast<uint8_t *>(dst) + (b0 / 2) * 72);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_repack(int dtype, const void *src, int64_t M, int64_t K, void *dst, hipStream_t st) {
    switch (dtype) {
    case QMM_Q6_K: return launch_repack_q6_k(src, M, K, dst, st);
    case QMM_Q8_0: return launch_repack_q8_0(src, M, K, dst, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qmm
