// qmm_device.hpp -- device helpers for the gfx950 kernels: raw block fetches
// and the block geometry.  Included only by the HIP sources of libqmm.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmm.h"

namespace qmm {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// Block geometry (weights, bytes) per GGUF type id.
template <int DT> struct Geo;
template <> struct Geo<QMM_Q4_0> { static constexpr int BS = 32, BB = 18; };
template <> struct Geo<QMM_Q4_1> { static constexpr int BS = 32, BB = 20; };
template <> struct Geo<QMM_Q5_K> { static constexpr int BS = 256, BB = 176; };
template <> struct Geo<QMM_Q8_0> { static constexpr int BS = 32, BB = 34; };
template <> struct Geo<QMM_Q4_K> { static constexpr int BS = 256, BB = 144; };
template <> struct Geo<QMM_Q6_K> { static constexpr int BS = 256, BB = 210; };
// Q6_K repacked for the matrix-core GEMM (qmm_repack): per super-block of 256
// weights, 256 code bytes (q in 0..63, one per weight, in the order the GEMM's
// lanes read them) and the 16 sub-block scales d * sc as f32.  An internal
// type id: the C ABI names it by its source type and the repack entry points.
constexpr int QMM_Q6_K_R = 114;
template <> struct Geo<QMM_Q6_K_R> { static constexpr int BS = 256, BB = 320; };
// Q8_0 repacked the same way: per 64 weights (two GGUF blocks), 64 code bytes
// q + 128 (unsigned) in order, then the two block scales d as f32.
constexpr int QMM_Q8_0_R = 108;
template <> struct Geo<QMM_Q8_0_R> { static constexpr int BS = 64, BB = 72; };

__device__ __forceinline__ float h2f(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits16 & 0xFFFFu));
}

// Bytes [p, p+4N) of memory whose start is 4-byte aligned, as N dwords.
// NT: non-temporal loads (data streamed once, kept out of the caches).
template <int N, bool NT = false>
__device__ __forceinline__ void fetch_al(const uint8_t *p, uint32_t (&out)[N]) {
    const uint32_t *q = reinterpret_cast<const uint32_t *>(p);
#pragma unroll
    for (int i = 0; i < N; i++) out[i] = NT ? __builtin_nontemporal_load(q + i) : q[i];
}

// Bytes [p, p+4N) for a 2-byte aligned p: loads the N+1 aligned dwords that
// cover them and funnel-shifts.  The caller guarantees that the dword holding
// byte p+4N-1+(p&3) is inside the buffer.
template <int N, bool NT = false>
__device__ __forceinline__ void fetch_un(const uint8_t *p, uint32_t (&out)[N]) {
    const uint32_t sh = (uint32_t)((uintptr_t)p & 3u);
    // aligned down by pointer arithmetic, so the global address space is kept
    const uint32_t *q = reinterpret_cast<const uint32_t *>(p - sh);
    uint32_t w[N + 1];
#pragma unroll
    for (int i = 0; i < N + 1; i++) w[i] = NT ? __builtin_nontemporal_load(q + i) : q[i];
#pragma unroll
    for (int i = 0; i < N; i++) out[i] = __builtin_amdgcn_alignbyte(w[i + 1], w[i], sh);
}

// Bytes [p, p+nbytes) by single-byte loads, any alignment; the rest of the
// N dwords is zero.  Reads nothing outside [p, p+nbytes).
template <int N>
__device__ __forceinline__ void fetch_bytes(const uint8_t *p, int nbytes, uint32_t (&out)[N]) {
#pragma unroll
    for (int i = 0; i < N; i++) {
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const int o = 4 * i + b;
            if (o < nbytes) v |= (uint32_t)p[o] << (8 * b);
        }
        out[i] = v;
    }
}

// The dword holding byte p (aligned down, global address space kept).
__device__ __forceinline__ const uint32_t *dword_at(const uint8_t *p) {
    return reinterpret_cast<const uint32_t *>(p - ((uintptr_t)p & 3u));
}

__device__ __forceinline__ uint32_t byte_of(uint32_t v, int i) { return (v >> (8 * i)) & 0xFFu; }

// Q4_K sub-block i (0..7): 6-bit scale and min from the 12 packed bytes held
// in dwords s0 (bytes 0-3), s1 (4-7), s2 (8-11).  Standard GGUF k-quant
// packing: i<4 low 6 bits of byte i / i+4; i>=4 low/high nibble of byte i+4
// plus the top 2 bits of byte i-4 / i.
__device__ __forceinline__ void q4k_scale_min(uint32_t s0, uint32_t s1, uint32_t s2, int i,
                                              int &sc, int &mn) {
    if (i < 4) {
        sc = (int)(byte_of(s0, i) & 63u);
        mn = (int)(byte_of(s1, i) & 63u);
    } else {
        const int j = i - 4;
        sc = (int)((byte_of(s2, j) & 15u) | ((byte_of(s0, j) >> 6) << 4));
        mn = (int)((byte_of(s2, j) >> 4) | ((byte_of(s1, j) >> 6) << 4));
    }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Sum over the 64 lanes of a wavefront in a fixed order, result valid in
// lane 63: DPP butterflies inside each row of 16 lanes, then the row
// broadcasts of lane 15 / lane 31.
// silu(v) = v * sigmoid(v) = v / (1 + e^-v) (page "cera 0.5.2
// src/backend/cpu.rs", activation functions), evaluated with e = e^-|v| so
// that the exponential never overflows: v / (1 + e) for v >= 0 and
// v e / (1 + e) for v < 0 (the same function; tiny negative tails keep their
// value instead of becoming -0 where e^-v would overflow).
__device__ __forceinline__ float silu(float v) {
    const float e = expf(-fabsf(v));
    return (v >= 0.f ? v : v * e) / (1.0f + e);
}

__device__ __forceinline__ float wave_sum_to_lane63(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));  // quad_perm 1,0,3,2
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));  // quad_perm 2,3,0,1
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true)); // row_half_mirror
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true)); // row_mirror
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false)); // row_bcast15
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false)); // row_bcast31
    return v;
}

// The f16 pairs {1024 + byte0, 1024 + byte2} and {1024 + byte1, 1024 + byte3}
// of a dword, one v_perm_b32 each: 0x64 is the high byte of f16 1024.0 and the
// byte lands in the low mantissa bits, so byte b becomes exactly 1024 + b.
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ half2_t bytes02_as_f16(uint32_t v) {
    return __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, v, 0x04020400u));
}
__device__ __forceinline__ half2_t bytes13_as_f16(uint32_t v) {
    return __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, v, 0x04030401u));
}

// Bounds-checked buffer loads: a resource covers [base, base + bytes); any
// dword at or past the byte count reads as 0 without a memory access, so
// out-of-range rows, tokens and row groups need no branch around a load (a
// branch around a load makes the compiler's wait counts conservative).
typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ Rsrc make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// The same from values known to be wave-uniform but not provably so to the
// compiler: without the explicit readfirstlane it keeps the descriptor in
// VGPRs and wraps every load in a waterfall loop.
__device__ __forceinline__ Rsrc make_rsrc_uniform(const void *base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b), hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint64_t u = ((uint64_t)hi << 32) | lo;
    return make_rsrc(reinterpret_cast<const void *>(u), __builtin_amdgcn_readfirstlane(bytes));
}

// N dwords at byte offset voff (per lane) + soff (uniform)
template <int N>
__device__ __forceinline__ void ldb(Rsrc rs, uint32_t voff, uint32_t soff, uint32_t (&v)[N]) {
    int i = 0;
#pragma unroll
    for (; i + 4 <= N; i += 4) {
        const u32x4_t q = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 4 * i, soff, 0);
        v[i] = q.x; v[i + 1] = q.y; v[i + 2] = q.z; v[i + 3] = q.w;
    }
    if constexpr (N % 4 == 3) {
        const u32x3_t q = __builtin_amdgcn_raw_buffer_load_b96(rs, voff + 4 * i, soff, 0);
        v[i] = q.x; v[i + 1] = q.y; v[i + 2] = q.z;
    } else if constexpr (N % 4 == 2) {
        const u32x2_t q = __builtin_amdgcn_raw_buffer_load_b64(rs, voff + 4 * i, soff, 0);
        v[i] = q.x; v[i + 1] = q.y;
    } else if constexpr (N % 4 == 1) {
        v[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff + 4 * i, soff, 0);
    }
}

}  // namespace qmm
