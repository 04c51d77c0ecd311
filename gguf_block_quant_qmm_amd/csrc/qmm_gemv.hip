// qmm_gemv.hip -- decode GEMV kernels, y[m] = sum_k W[m][k] x[k], f32 arithmetic.
//
// Decode is a stream of the packed weight (page "cera 0.3.1
// src/model/gpu_lfm2.rs", forward_inner_compute: decode is memory-bound inside
// the quantized GEMVs).  Design for gfx950:
//   * a workgroup owns R rows at a time and walks row groups with a grid stride;
//   * its threads split each row into 64-weight units, every thread keeps the
//     64 activations of its unit in registers and reuses them for all R rows
//     (when a row has no more units than the workgroup has threads, the
//     activations are loaded once for the workgroup's whole life);
//   * weight bytes arrive as aligned dword loads; 18/34/210-byte blocks that
//     straddle dwords are realigned in registers with v_alignbyte;
//   * each unit is decoded in registers and accumulated with f32 FMAs in short
//     chains (16 terms per chain), then reduced across the wavefront with
//     cross-lane shuffles and across wavefronts through LDS, in a fixed order.
// The per-element weight is exact in f32 for Q8_0, Q4_0 and Q6_K and rounded
// once for Q4_K (fma(d*sc, q, -dmin*m)).
#include <algorithm>
#include <cstdlib>

#include "qmm_device.hpp"
#include "qmm_internal.hpp"

namespace qmm {

// ----------------------------------------------------------------- units ----
// A unit is 64 weights of one row.  Q8_0/Q4_0: a pair of consecutive blocks
// (needs an even number of blocks per row so every pair is dword aligned).
// Q4_K: one 64-weight chunk of a super-block (sub-blocks 2c and 2c+1).
// Q6_K: the 64 weights {128h + 32g + 16lh + i : g < 4, i < 16} of one
// super-block, which share one 16-byte slice of each ql half and of qh.

template <int DT> struct Unit;

// Exact f16 of a small integer code c: bytes02/13_as_f16 give 1024 + c, and
// one packed f16 add of -(1024 + bias) leaves c - bias with no rounding (all
// values are integers below 2048).  v_fma_mix_f32 then multiplies the f16 by
// the f32 activation inside an f32 FMA, so every product and sum is f32.
__device__ __forceinline__ float fma_h(_Float16 h, float x, float acc) { return fmaf((float)h, x, acc); }

template <> struct Unit<QMM_Q4_0> {
    static constexpr int NDW = 9;
    template <bool NT>
    __device__ static void load(const uint8_t *row, int u, uint32_t (&v)[NDW]) { fetch_al<NDW, NT>(row + 36 * u, v); }
    __device__ static void load_x(const float *x, int u, float (&xv)[64]) {
        const floatx4 *p = reinterpret_cast<const floatx4 *>(x + 64 * u);
#pragma unroll
        for (int i = 0; i < 16; i++) {
            floatx4 t = p[i];
            xv[4 * i] = t.x; xv[4 * i + 1] = t.y; xv[4 * i + 2] = t.z; xv[4 * i + 3] = t.w;
        }
    }
    __device__ static float dot(const uint32_t (&v)[NDW], const float (&xv)[64], int) {
        const half2_t bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};  // q - 8
        float total = 0.f;
#pragma unroll
        for (int b = 0; b < 2; b++) {
            const float d = b == 0 ? h2f(v[0]) : h2f(v[4] >> 16);
            float slo = 0.f, shi = 0.f;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint32_t q = b == 0 ? __builtin_amdgcn_alignbyte(v[i + 1], v[i], 2) : v[5 + i];
                const uint32_t L = q & 0x0F0F0F0Fu, H = (q >> 4) & 0x0F0F0F0Fu;
                const half2_t l02 = bytes02_as_f16(L) + bias, l13 = bytes13_as_f16(L) + bias;
                const half2_t h02 = bytes02_as_f16(H) + bias, h13 = bytes13_as_f16(H) + bias;
                const float *xl = xv + 32 * b + 4 * i, *xh = xl + 16;
                slo = fma_h(l02.x, xl[0], slo); slo = fma_h(l13.x, xl[1], slo);
                slo = fma_h(l02.y, xl[2], slo); slo = fma_h(l13.y, xl[3], slo);
                shi = fma_h(h02.x, xh[0], shi); shi = fma_h(h13.x, xh[1], shi);
                shi = fma_h(h02.y, xh[2], shi); shi = fma_h(h13.y, xh[3], shi);
            }
            total = fmaf(d, slo + shi, total);
        }
        return total;
    }
};

template <> struct Unit<QMM_Q8_0> {
    static constexpr int NDW = 17;
    template <bool NT>
    __device__ static void load(const uint8_t *row, int u, uint32_t (&v)[NDW]) { fetch_al<NDW, NT>(row + 68 * u, v); }
    __device__ static void load_x(const float *x, int u, float (&xv)[64]) { Unit<QMM_Q4_0>::load_x(x, u, xv); }
    __device__ static float dot(const uint32_t (&v)[NDW], const float (&xv)[64], int) {
        const half2_t bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};  // (q + 128) - 128
        float total = 0.f;
#pragma unroll
        for (int b = 0; b < 2; b++) {
            const float d = b == 0 ? h2f(v[0]) : h2f(v[8] >> 16);
            float s0 = 0.f, s1 = 0.f;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const uint32_t q = (b == 0 ? __builtin_amdgcn_alignbyte(v[i + 1], v[i], 2) : v[9 + i]) ^ 0x80808080u;
                const half2_t p02 = bytes02_as_f16(q) + bias, p13 = bytes13_as_f16(q) + bias;
                const float *xp = xv + 32 * b + 4 * i;
                float &s = i < 4 ? s0 : s1;
                s = fma_h(p02.x, xp[0], s); s = fma_h(p13.x, xp[1], s);
                s = fma_h(p02.y, xp[2], s); s = fma_h(p13.y, xp[3], s);
            }
            total = fmaf(d, s0 + s1, total);
        }
        return total;
    }
};

template <> struct Unit<QMM_Q4_K> {
    static constexpr int NDW = 12;  // 4 header dwords (d, dmin, 12 scale bytes) + 8 nibble dwords
    template <bool NT>
    __device__ static void load(const uint8_t *row, int u, uint32_t (&v)[NDW]) {
        const uint8_t *sb = row + 144 * (u >> 2);
        uint32_t h[4], q[8];
        fetch_al<4, NT>(sb, h);
        fetch_al<8, NT>(sb + 16 + 32 * (u & 3), q);
#pragma unroll
        for (int i = 0; i < 4; i++) v[i] = h[i];
#pragma unroll
        for (int i = 0; i < 8; i++) v[4 + i] = q[i];
    }
    __device__ static void load_x(const float *x, int u, float (&xv)[64]) { Unit<QMM_Q4_0>::load_x(x, u, xv); }
    __device__ static float dot(const uint32_t (&v)[NDW], const float (&xv)[64], int u) {
        const half2_t bias = {(_Float16)-1024.0f, (_Float16)-1024.0f};  // q
        const float d = h2f(v[0]), dmin = h2f(v[0] >> 16);
        const int c = u & 3;
        float total = 0.f;
#pragma unroll
        for (int half = 0; half < 2; half++) {  // sub-block 2c (low nibbles), 2c+1 (high nibbles)
            int sc, mn;
            q4k_scale_min(v[1], v[2], v[3], 2 * c + half, sc, mn);
            const float dsc = d * (float)sc, ndm = -(dmin * (float)mn);
            float s0 = 0.f, s1 = 0.f;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const uint32_t n = (v[4 + i] >> (4 * half)) & 0x0F0F0F0Fu;
                const half2_t q02 = bytes02_as_f16(n) + bias, q13 = bytes13_as_f16(n) + bias;
                const float *xp = xv + 32 * half + 4 * i;
                float &s = i < 4 ? s0 : s1;
                // weight = d*sc*q - dmin*m, one f32 rounding; then the f32 FMA with x
                s = fmaf(fmaf(dsc, (float)q02.x, ndm), xp[0], s);
                s = fmaf(fmaf(dsc, (float)q13.x, ndm), xp[1], s);
                s = fmaf(fmaf(dsc, (float)q02.y, ndm), xp[2], s);
                s = fmaf(fmaf(dsc, (float)q13.y, ndm), xp[3], s);
            }
            total += s0 + s1;
        }
        return total;
    }
};

template <> struct Unit<QMM_Q6_K> {
    // A = ql[64h+16lh ..+16], B = ql[64h+32+16lh ..+16], C = qh[32h+16lh ..+16],
    // S = sc[8h .. 8h+8), D = dword holding d.  Needs an even number of
    // super-blocks per row so that only even (4-aligned) blocks read past
    // their own last byte, and never past the blob.
    static constexpr int NDW = 4 + 4 + 4 + 2 + 1;
    template <bool NT>
    __device__ static void load(const uint8_t *row, int u, uint32_t (&v)[NDW]) {
        const uint8_t *p = row + 210 * (u >> 2);
        const int h = (u >> 1) & 1, lh = u & 1;
        uint32_t a[4], b[4], c[4], s[2];
        fetch_un<4, NT>(p + 64 * h + 16 * lh, a);
        fetch_un<4, NT>(p + 64 * h + 32 + 16 * lh, b);
        fetch_un<4, NT>(p + 128 + 32 * h + 16 * lh, c);
        fetch_un<2, NT>(p + 192 + 8 * h, s);
        const uint8_t *pd = p + 208;
        const uint32_t *pdw = dword_at(pd);
        const uint32_t dw = NT ? __builtin_nontemporal_load(pdw) : *pdw;
#pragma unroll
        for (int i = 0; i < 4; i++) { v[i] = a[i]; v[4 + i] = b[i]; v[8 + i] = c[i]; }
        v[12] = s[0]; v[13] = s[1];
        v[14] = dw >> (8 * ((uintptr_t)pd & 3));
    }
    __device__ static void load_x(const float *x, int u, float (&xv)[64]) {
        const int h = (u >> 1) & 1, lh = u & 1;
        const float *base = x + 256 * (u >> 2) + 128 * h + 16 * lh;
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const floatx4 *p = reinterpret_cast<const floatx4 *>(base + 32 * g);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                floatx4 t = p[i];
                xv[16 * g + 4 * i] = t.x; xv[16 * g + 4 * i + 1] = t.y;
                xv[16 * g + 4 * i + 2] = t.z; xv[16 * g + 4 * i + 3] = t.w;
            }
        }
    }
    __device__ static float dot(const uint32_t (&v)[NDW], const float (&xv)[64], int u) {
        const half2_t bias = {(_Float16)-1056.0f, (_Float16)-1056.0f};  // q - 32
        const int lh = u & 1;
        const float d = h2f(v[14]);
        float total = 0.f;
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const int sidx = 2 * g + lh;  // byte of sc[8h .. 8h+8)
            const float dsc = d * (float)(int8_t)(uint8_t)byte_of(v[12 + (sidx >> 2)], sidx & 3);
            float s = 0.f;
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const uint32_t L = (g & 1) ? v[4 + t] : v[t];
                const uint32_t lo = (g < 2 ? L : (L >> 4)) & 0x0F0F0F0Fu;
                const uint32_t C = v[8 + t];
                const uint32_t hi = (g < 2 ? (C << (4 - 2 * g)) : (C >> (2 * g - 4))) & 0x30303030u;
                const uint32_t q = lo | hi;  // four 6-bit codes, one per byte
                const half2_t q02 = bytes02_as_f16(q) + bias, q13 = bytes13_as_f16(q) + bias;
                const float *xp = xv + 16 * g + 4 * t;
                s = fma_h(q02.x, xp[0], s); s = fma_h(q13.x, xp[1], s);
                s = fma_h(q02.y, xp[2], s); s = fma_h(q13.y, xp[3], s);
            }
            total = fmaf(dsc, s, total);
        }
        return total;
    }
};

// ----------------------------------------------------------- fast kernel ----
// Every thread owns at most one unit of the row (U <= blockDim.x), so its 64
// activations are loaded once and stay in registers while the workgroup
// walks its row groups (R rows each, grid stride).  The raw bytes of the next
// row group are fetched before the current one is decoded (two register
// buffers, loop unrolled by two so neither is indexed dynamically).
template <int DT, int R>
__global__ void __launch_bounds__(256) gemv_kernel(const uint8_t *__restrict__ blob, int64_t M,
                                                   int64_t row_bytes, int U,
                                                   const float *__restrict__ x, float *__restrict__ y) {
    constexpr int NDW = Unit<DT>::NDW;
    __shared__ float red[2][R][4];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, nwaves = blockDim.x >> 6;
    const bool active = t < U;
    const int64_t nrg = (M + R - 1) / R;
    float xv[64];
    if (active) Unit<DT>::load_x(x, t, xv);

    auto fetch = [&](int64_t g, uint32_t (&raw)[R][NDW]) {
#pragma unroll
        for (int r = 0; r < R; r++) {
            const int64_t row = g * R + r;
            if (active && row < M) Unit<DT>::template load<false>(blob + row * row_bytes, t, raw[r]);
        }
    };
    auto finish = [&](int64_t g, const uint32_t (&raw)[R][NDW], int parity) {
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; r++) {
            acc[r] = (active && g * R + r < M) ? Unit<DT>::dot(raw[r], xv, t) : 0.f;
            acc[r] = wave_sum_to_lane63(acc[r]);
        }
        if (nwaves == 1) {
            if (lane == 63) {
#pragma unroll
                for (int r = 0; r < R; r++)
                    if (g * R + r < M) y[g * R + r] = acc[r];
            }
        } else {
            if (lane == 63) {
#pragma unroll
                for (int r = 0; r < R; r++) red[parity][r][wave] = acc[r];
            }
            __syncthreads();
            if (t < R && g * R + t < M) {
                float s = red[parity][t][0];
                for (int w = 1; w < nwaves; w++) s += red[parity][t][w];
                y[g * R + t] = s;
            }
        }
    };

    uint32_t ra[R][NDW], rb[R][NDW];
    int64_t g = blockIdx.x;
    if (g < nrg) fetch(g, ra);
    while (g < nrg) {
        const int64_t g1 = g + gridDim.x;
        if (g1 < nrg) fetch(g1, rb);
        finish(g, ra, 0);
        if (g1 >= nrg) break;
        const int64_t g2 = g1 + gridDim.x;
        if (g2 < nrg) fetch(g2, ra);
        finish(g1, rb, 1);
        g = g2;
    }
}

// More units than threads (K > 64 * 256): each thread loops over its units
// and reloads their activations for every row group.
template <int DT, int R>
__global__ void __launch_bounds__(256) gemv_multi_kernel(const uint8_t *__restrict__ blob, int64_t M,
                                                         int64_t row_bytes, int U,
                                                         const float *__restrict__ x, float *__restrict__ y) {
    __shared__ float red[R][4];
    const int t = threadIdx.x, T = blockDim.x, lane = t & 63, wave = t >> 6, nwaves = T >> 6;
    const int64_t nrg = (M + R - 1) / R;
    float xv[64];
    for (int64_t rg = blockIdx.x; rg < nrg; rg += gridDim.x) {
        const int64_t row0 = rg * R;
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; r++) acc[r] = 0.f;
        for (int u = t; u < U; u += T) {
            Unit<DT>::load_x(x, u, xv);
            uint32_t raw[R][Unit<DT>::NDW];
#pragma unroll
            for (int r = 0; r < R; r++)
                if (row0 + r < M) Unit<DT>::template load<false>(blob + (row0 + r) * row_bytes, u, raw[r]);
#pragma unroll
            for (int r = 0; r < R; r++)
                if (row0 + r < M) acc[r] += Unit<DT>::dot(raw[r], xv, u);
        }
#pragma unroll
        for (int r = 0; r < R; r++) {
            const float s = wave_sum_to_lane63(acc[r]);
            if (lane == 63) red[r][wave] = s;
        }
        __syncthreads();
        if (t < R && row0 + t < M) {
            float s = red[t][0];
            for (int w = 1; w < nwaves; w++) s += red[t][w];
            y[row0 + t] = s;
        }
        __syncthreads();
    }
}

// -------------------------------------------------------- generic kernel ----
// Any K that is a multiple of the block size (used when the fast kernel's
// alignment conditions do not hold): one block per thread, byte loads, the
// same f32 arithmetic per block.
template <int DT>
__device__ float block_dot_generic(const uint8_t *blk, const float *x);

template <>
__device__ float block_dot_generic<QMM_Q4_0>(const uint8_t *p, const float *x) {
    const float d = h2f((uint32_t)p[0] | ((uint32_t)p[1] << 8));
    float slo = 0.f, shi = 0.f;
    for (int j = 0; j < 16; j++) {
        slo = fmaf((float)((int)(p[2 + j] & 15) - 8), x[j], slo);
        shi = fmaf((float)((int)(p[2 + j] >> 4) - 8), x[16 + j], shi);
    }
    return d * (slo + shi);
}

template <>
__device__ float block_dot_generic<QMM_Q8_0>(const uint8_t *p, const float *x) {
    const float d = h2f((uint32_t)p[0] | ((uint32_t)p[1] << 8));
    float s0 = 0.f, s1 = 0.f;
    for (int j = 0; j < 16; j++) {
        s0 = fmaf((float)(int8_t)p[2 + j], x[j], s0);
        s1 = fmaf((float)(int8_t)p[18 + j], x[16 + j], s1);
    }
    return d * (s0 + s1);
}

template <>
__device__ float block_dot_generic<QMM_Q4_K>(const uint8_t *p, const float *x) {
    const float d = h2f((uint32_t)p[0] | ((uint32_t)p[1] << 8));
    const float dmin = h2f((uint32_t)p[2] | ((uint32_t)p[3] << 8));
    uint32_t s[3];
    for (int i = 0; i < 3; i++)
        s[i] = (uint32_t)p[4 + 4 * i] | ((uint32_t)p[5 + 4 * i] << 8) | ((uint32_t)p[6 + 4 * i] << 16) |
               ((uint32_t)p[7 + 4 * i] << 24);
    float total = 0.f;
    for (int i = 0; i < 8; i++) {
        int sc, mn;
        q4k_scale_min(s[0], s[1], s[2], i, sc, mn);
        const float dsc = d * (float)sc, ndm = -(dmin * (float)mn);
        float s0 = 0.f, s1 = 0.f;
        for (int e = 0; e < 16; e++) {
            const uint8_t b0 = p[16 + 32 * (i >> 1) + e], b1 = p[16 + 32 * (i >> 1) + 16 + e];
            const float q0 = (float)((i & 1) ? (b0 >> 4) : (b0 & 15));
            const float q1 = (float)((i & 1) ? (b1 >> 4) : (b1 & 15));
            s0 = fmaf(fmaf(dsc, q0, ndm), x[32 * i + e], s0);
            s1 = fmaf(fmaf(dsc, q1, ndm), x[32 * i + 16 + e], s1);
        }
        total += s0 + s1;
    }
    return total;
}

template <>
__device__ float block_dot_generic<QMM_Q6_K>(const uint8_t *p, const float *x) {
    const float d = h2f((uint32_t)p[208] | ((uint32_t)p[209] << 8));
    float total = 0.f;
    for (int s = 0; s < 16; s++) {  // 16 groups of 16 weights sharing one sub-scale
        const float dsc = d * (float)(int8_t)p[192 + s];
        float acc = 0.f;
        for (int i = 0; i < 16; i++) {
            const int j = 16 * s + i, h = j >> 7, g = (j & 127) >> 5, l = j & 31;
            const uint8_t lb = p[64 * h + 32 * (g & 1) + l];
            const int lo = (g < 2) ? (lb & 15) : (lb >> 4);
            const int hi = (p[128 + 32 * h + l] >> (2 * g)) & 3;
            acc = fmaf((float)((lo | (hi << 4)) - 32), x[j], acc);
        }
        total = fmaf(dsc, acc, total);
    }
    return total;
}

template <int DT, int R>
__global__ void __launch_bounds__(256) gemv_generic_kernel(const uint8_t *__restrict__ blob, int64_t M,
                                                           int64_t K, const float *__restrict__ x,
                                                           float *__restrict__ y) {
    constexpr int BS = Geo<DT>::BS, BB = Geo<DT>::BB;
    __shared__ float red[R][4];
    const int t = threadIdx.x, T = blockDim.x, lane = t & 63, wave = t >> 6, nwaves = T >> 6;
    const int64_t nb = K / BS, row_bytes = nb * BB, nrg = (M + R - 1) / R;
    for (int64_t rg = blockIdx.x; rg < nrg; rg += gridDim.x) {
        const int64_t row0 = rg * R;
        float acc[R];
        for (int r = 0; r < R; r++) acc[r] = 0.f;
        for (int64_t b = t; b < nb; b += T)
            for (int r = 0; r < R; r++)
                if (row0 + r < M) acc[r] += block_dot_generic<DT>(blob + (row0 + r) * row_bytes + b * BB, x + b * BS);
        for (int r = 0; r < R; r++) {
            const float s = wave_sum_to_lane63(acc[r]);
            if (lane == 63) red[r][wave] = s;
        }
        __syncthreads();
        if (t < R && row0 + t < M) {
            float s = 0.f;
            for (int w = 0; w < nwaves; w++) s += red[t][w];
            y[row0 + t] = s;
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------- launcher ----

static bool fast_layout_ok(int dtype, int64_t nb) {
    switch (dtype) {
    case QMM_Q4_0:
    case QMM_Q8_0:
    case QMM_Q6_K: return (nb % 2) == 0;
    case QMM_Q4_K: return true;
    default: return false;
    }
}

// Resident workgroups per CU for the persistent GEMV; QMM_GEMV_WAVES_PER_CU
// overrides the default (a tuning lever, read once).
static int gemv_waves_per_cu() {
    static int v = [] {
        const char *e = getenv("QMM_GEMV_WAVES_PER_CU");
        const int n = e ? atoi(e) : 0;
        return (n >= 1 && n <= 32) ? n : 8;
    }();
    return v;
}

template <int DT, int R>
static hipError_t launch_fast(const uint8_t *blob, int64_t M, int64_t K, const float *x, float *y,
                              hipStream_t st, int cus) {
    constexpr int BS = Geo<DT>::BS, BB = Geo<DT>::BB;
    const int64_t nb = K / BS, row_bytes = nb * BB;
    const int64_t U64 = K / 64;
    const int T = (int)(U64 >= 256 ? 256 : ((U64 + 63) / 64) * 64);
    const int U = (int)U64;
    const int64_t nrg = (M + R - 1) / R;
    const int64_t wg_per_cu = std::max<int64_t>(1, gemv_waves_per_cu() / (T / 64));
    const int64_t grid = std::min<int64_t>(nrg, (int64_t)cus * wg_per_cu);
    if (U64 <= 256)
        hipLaunchKernelGGL((gemv_kernel<DT, R>), dim3((unsigned)grid), dim3(T), 0, st, blob, M, row_bytes, U, x, y);
    else
        hipLaunchKernelGGL((gemv_multi_kernel<DT, R>), dim3((unsigned)grid), dim3(T), 0, st, blob, M, row_bytes, U, x, y);
    return hipGetLastError();
}

template <int DT>
static hipError_t launch_generic(const uint8_t *blob, int64_t M, int64_t K, const float *x, float *y,
                                 hipStream_t st, int cus) {
    constexpr int R = 4;
    const int64_t nrg = (M + R - 1) / R;
    const int64_t grid = nrg < (int64_t)cus * 8 ? nrg : (int64_t)cus * 8;
    hipLaunchKernelGGL((gemv_generic_kernel<DT, R>), dim3((unsigned)grid), dim3(256), 0, st, blob, M, K, x, y);
    return hipGetLastError();
}

hipError_t launch_gemv(int dtype, const void *blob_v, int64_t M, int64_t K, const float *x, float *y,
                       hipStream_t st, int cus) {
    const uint8_t *blob = static_cast<const uint8_t *>(blob_v);
    const int64_t bs = (dtype == QMM_Q4_K || dtype == QMM_Q6_K) ? 256 : 32;
    const bool fast = fast_layout_ok(dtype, K / bs) && (K % 64) == 0;
    switch (dtype) {
    case QMM_Q4_0: return fast ? launch_fast<QMM_Q4_0, 4>(blob, M, K, x, y, st, cus) : launch_generic<QMM_Q4_0>(blob, M, K, x, y, st, cus);
    case QMM_Q8_0: return fast ? launch_fast<QMM_Q8_0, 4>(blob, M, K, x, y, st, cus) : launch_generic<QMM_Q8_0>(blob, M, K, x, y, st, cus);
    case QMM_Q4_K: return fast ? launch_fast<QMM_Q4_K, 4>(blob, M, K, x, y, st, cus) : launch_generic<QMM_Q4_K>(blob, M, K, x, y, st, cus);
    case QMM_Q6_K: return fast ? launch_fast<QMM_Q6_K, 4>(blob, M, K, x, y, st, cus) : launch_generic<QMM_Q6_K>(blob, M, K, x, y, st, cus);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qmm
