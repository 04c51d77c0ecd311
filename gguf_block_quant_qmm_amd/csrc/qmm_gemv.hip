// qmm_gemv.hip -- decode GEMV kernels, y[m] = sum_k W[m][k] x[k], f32 arithmetic.
//
// Decode is a stream of the packed weight (page "cera 0.3.1
// src/model/gpu_lfm2.rs", forward_inner_compute: decode is memory-bound inside
// the quantized GEMVs).  Design for gfx950:
//   * a row is cut into 64-weight units, one per lane; every lane keeps the 64
//     activations of its unit in registers for the whole kernel (staged once
//     per workgroup through LDS with coalesced loads);
//   * a wavefront (K <= 4096) or a workgroup of up to 4 wavefronts splitting K
//     (K <= 16384) owns a balanced contiguous range of row groups (R rows) and
//     keeps D row groups in flight in registers while it decodes the current
//     one, so memory and ALU work overlap;
//   * weight bytes arrive as dword loads addressed from a uniform row pointer
//     plus a per-lane 32-bit offset; 18/34/210-byte blocks that straddle
//     dwords are realigned in registers with v_alignbyte;
//   * codes become exact f16 values (v_perm_b32 + one packed f16 subtract) and
//     multiply the f32 activations inside v_fma_mix_f32 (f32 FMA), in chains
//     of 16 terms, reduced across the wavefront with DPP in a fixed order.
// The per-element weight is exact in f32 for Q8_0, Q4_0 and Q6_K and rounded
// once for Q4_K (fma(d*sc, q, -dmin*m)).
#include <algorithm>
#include <cstdlib>

#include "qmm_device.hpp"
#include "qmm_internal.hpp"

namespace qmm {

__device__ __forceinline__ float fma_h(_Float16 h, float x, float acc) { return fmaf((float)h, x, acc); }


// ----------------------------------------------------------------- units ----
// A unit is 64 weights of one row.  Q8_0/Q4_0: a pair of consecutive blocks
// (an even number of blocks per row keeps every pair dword aligned).  Q4_K:
// one 64-weight chunk of a super-block (sub-blocks 2c and 2c+1).  Q6_K: the 64
// weights {128h + 32g + 16lh + i : g < 4, i < 16} of one super-block, which
// share one 16-byte slice of each ql half and of qh.
//   Off          per-lane byte offsets inside a row (computed once)
//   load(row,o)  the unit's raw dwords (row pointer uniform across the wave)
//   x4(u, i)     float4 index of local activations 4i..4i+3 of unit u
//   dot(v,x,o)   the unit's dot product, f32

template <int DT> struct Unit;

// 4-bit codes enter the f32 arithmetic (v_fma_mix_f32) as f16 subnormals: a
// dword masked with 0x000F000F holds two codes c as c * 2^-24, masked with
// 0x00F000F0 as c * 2^-20 -- one VOP2 instruction per two codes, exact.  Every
// weight is formed exactly (Q4_0, Q8_0, Q6_K) or with one rounding (Q4_K)
// before it meets its activation, so the usual f32 dot-product error bound
// relative to sum |w x| holds: no offset is ever taken out through a sum of
// activations (that would cancel when the weights do).
__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

constexpr float TWO24 = 16777216.0f, TWO20 = 1048576.0f;

template <> struct Unit<QMM_Q4_0> {
    static constexpr int NL = 9;
    struct Off { uint32_t a; };
    __device__ static Off lane_off(int u) { return {36u * u}; }
    __device__ static void load(Rsrc rs, uint32_t row, const Off &o, uint32_t (&v)[NL]) { ldb(rs, o.a, row, v); }
    __device__ static int x4(int u, int i) { return 16 * u + i; }
    __device__ static float dot(const uint32_t (&v)[NL], const float (&xv)[64], const Off &) {
        // The unit is two blocks, 36 bytes: d0 qs0[16] d1 qs1[16].  Block 0's
        // codes sit in dwords [qs0 qs1 qs14 qs15] (realigned from v0, v4) and
        // v1..v3 = qs2..13; block 1's in v5..v8.  Element e < 16 is the low
        // nibble of qs[e], element e + 16 its high nibble.  Low nibbles become
        // (q - 8) 2^-24, high nibbles (q - 8) 2^-20: exact f16 subnormals.
        const half2_t b24 = as_h2(0x80088008u), b20 = as_h2(0x80808080u);  // -8 * 2^-24, -128 * 2^-24
        const uint32_t D[2][4] = {{__builtin_amdgcn_alignbyte(v[4], v[0], 2), v[1], v[2], v[3]},
                                  {v[5], v[6], v[7], v[8]}};
        float lo[2][2], hi[2][2];
#pragma unroll
        for (int b = 0; b < 2; b++) {
            const float *xb = xv + 32 * b;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                // qs index of the dword's bytes 0..3
                const int e0 = b == 1 ? 4 * i : (i == 0 ? 0 : 4 * i - 2);
                const int e1 = e0 + 1;
                const int e2 = (b == 0 && i == 0) ? 14 : e0 + 2, e3 = e2 + 1;
                const uint32_t d = D[b][i], t = d >> 8;
                const half2_t p0 = as_h2(d & 0x000F000Fu) + b24, p1 = as_h2(d & 0x00F000F0u) + b20;
                const half2_t p2 = as_h2(t & 0x000F000Fu) + b24, p3 = as_h2(t & 0x00F000F0u) + b20;
                const int c = i & 1;
                float l = i < 2 ? 0.f : lo[b][c], h = i < 2 ? 0.f : hi[b][c];
                l = fma_h(p0.x, xb[e0], l); h = fma_h(p1.x, xb[16 + e0], h);
                l = fma_h(p0.y, xb[e2], l); h = fma_h(p1.y, xb[16 + e2], h);
                l = fma_h(p2.x, xb[e1], l); h = fma_h(p3.x, xb[16 + e1], h);
                l = fma_h(p2.y, xb[e3], l); h = fma_h(p3.y, xb[16 + e3], h);
                lo[b][c] = l; hi[b][c] = h;
            }
        }
        const float s0 = fmaf(lo[0][0] + lo[0][1], TWO24, (hi[0][0] + hi[0][1]) * TWO20);
        const float s1 = fmaf(lo[1][0] + lo[1][1], TWO24, (hi[1][0] + hi[1][1]) * TWO20);
        return fmaf(h2f(v[4] >> 16), s1, h2f(v[0]) * s0);
    }
};

template <> struct Unit<QMM_Q4_1> {
    // The unit is two 20-byte blocks (d, m, qs[16]) -- every dword aligned:
    // v0 = d0|m0, v1..v4 = qs0[0..16), v5 = d1|m1, v6..v9 = qs1.  Codes enter
    // as exact f16 subnormals (low nibbles c 2^-24, high nibbles c 2^-20); each
    // weight d*q + m is formed with one rounding (v_fma_mix_f32 with d*2^24 or
    // d*2^20 and m), then multiplied into x with an f32 FMA -- as for Q4_K.
    static constexpr int NL = 10;
    struct Off { uint32_t a; };
    __device__ static Off lane_off(int u) { return {40u * u}; }
    __device__ static void load(Rsrc rs, uint32_t row, const Off &o, uint32_t (&v)[NL]) { ldb(rs, o.a, row, v); }
    __device__ static int x4(int u, int i) { return 16 * u + i; }
    __device__ static float dot(const uint32_t (&v)[NL], const float (&xv)[64], const Off &) {
        float acc[4];
#pragma unroll
        for (int b = 0; b < 2; b++) {
            const float d = h2f(v[5 * b]), m = h2f(v[5 * b] >> 16);
            const float s24 = d * TWO24, s20 = d * TWO20;
            const float *xb = xv + 32 * b;
            float l = 0.f, h = 0.f;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                // qs[4i .. 4i+4): elements 4i..4i+3 (low nibbles), 16+4i.. (high)
                const uint32_t dw = v[5 * b + 1 + i], t = dw >> 8;
                const half2_t p0 = as_h2(dw & 0x000F000Fu), p1 = as_h2(dw & 0x00F000F0u);
                const half2_t p2 = as_h2(t & 0x000F000Fu), p3 = as_h2(t & 0x00F000F0u);
                l = fmaf(fma_h(p0.x, s24, m), xb[4 * i], l);     h = fmaf(fma_h(p1.x, s20, m), xb[16 + 4 * i], h);
                l = fmaf(fma_h(p0.y, s24, m), xb[4 * i + 2], l); h = fmaf(fma_h(p1.y, s20, m), xb[16 + 4 * i + 2], h);
                l = fmaf(fma_h(p2.x, s24, m), xb[4 * i + 1], l); h = fmaf(fma_h(p3.x, s20, m), xb[16 + 4 * i + 1], h);
                l = fmaf(fma_h(p2.y, s24, m), xb[4 * i + 3], l); h = fmaf(fma_h(p3.y, s20, m), xb[16 + 4 * i + 3], h);
            }
            acc[2 * b] = l;
            acc[2 * b + 1] = h;
        }
        return (acc[0] + acc[1]) + (acc[2] + acc[3]);
    }
};
template <> struct Unit<QMM_Q8_0> {
    static constexpr int NL = 17;
    struct Off { uint32_t a; };
    __device__ static Off lane_off(int u) { return {68u * u}; }
    __device__ static void load(Rsrc rs, uint32_t row, const Off &o, uint32_t (&v)[NL]) { ldb(rs, o.a, row, v); }
    __device__ static int x4(int u, int i) { return 16 * u + i; }
    __device__ static float dot(const uint32_t (&v)[NL], const float (&xv)[64], const Off &) {
        const half2_t bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};  // (q + 128) - 128
        float blk[2];
#pragma unroll
        for (int b = 0; b < 2; b++) {
            half2_t w[8][2];  // [dword][p02, p13]
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const uint32_t q = (b == 0 ? __builtin_amdgcn_alignbyte(v[i + 1], v[i], 2) : v[9 + i]) ^ 0x80808080u;
                w[i][0] = bytes02_as_f16(q) + bias; w[i][1] = bytes13_as_f16(q) + bias;
            }
            const float *xb = xv + 32 * b;
            float s8[8];
#pragma unroll
            for (int i = 0; i < 8; i++) s8[i] = fma_h(w[i][0].x, xb[4 * i], 0.f);
#pragma unroll
            for (int i = 0; i < 8; i++) s8[i] = fma_h(w[i][1].x, xb[4 * i + 1], s8[i]);
#pragma unroll
            for (int i = 0; i < 8; i++) s8[i] = fma_h(w[i][0].y, xb[4 * i + 2], s8[i]);
#pragma unroll
            for (int i = 0; i < 8; i++) s8[i] = fma_h(w[i][1].y, xb[4 * i + 3], s8[i]);
            blk[b] = ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
        }
        return fmaf(h2f(v[8] >> 16), blk[1], h2f(v[0]) * blk[0]);
    }
};

template <> struct Unit<QMM_Q4_K> {
    static constexpr int NL = 12;  // 4 header dwords (d, dmin, 12 scale bytes) + 8 nibble dwords
    struct Off { uint32_t hdr, qs; int c; };
    __device__ static Off lane_off(int u) {
        const uint32_t h = 144u * (u >> 2);
        return {h, h + 16u + 32u * (u & 3), u & 3};
    }
    __device__ static void load(Rsrc rs, uint32_t row, const Off &o, uint32_t (&v)[NL]) {
        uint32_t h[4], q[8];
        ldb(rs, o.hdr, row, h);
        ldb(rs, o.qs, row, q);
#pragma unroll
        for (int i = 0; i < 4; i++) v[i] = h[i];
#pragma unroll
        for (int i = 0; i < 8; i++) v[4 + i] = q[i];
    }

    __device__ static int x4(int u, int i) { return 16 * u + i; }
    __device__ static float dot(const uint32_t (&v)[NL], const float (&xv)[64], const Off &o) {
        // sub-block 2c = low nibbles of qs[32c + j], 2c+1 = high nibbles.  Each
        // weight d*sc*q - dmin*m is formed with one rounding (v_fma_mix_f32 of
        // the subnormal code c*2^-24 or c*2^-20 with d*sc*2^24 or d*sc*2^20),
        // then multiplied into x with an f32 FMA.
        const float d = h2f(v[0]), dmin = h2f(v[0] >> 16);
        int sc0, m0, sc1, m1;
        q4k_scale_min(v[1], v[2], v[3], 2 * o.c, sc0, m0);
        q4k_scale_min(v[1], v[2], v[3], 2 * o.c + 1, sc1, m1);
        const float s0 = d * (float)sc0 * TWO24, n0 = -(dmin * (float)m0);
        const float s1 = d * (float)sc1 * TWO20, n1 = -(dmin * (float)m1);
        float acc[4];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t dw = v[4 + i], t = dw >> 8;
            const half2_t p0 = as_h2(dw & 0x000F000Fu), p1 = as_h2(dw & 0x00F000F0u);
            const half2_t p2 = as_h2(t & 0x000F000Fu), p3 = as_h2(t & 0x00F000F0u);
            const int c = 2 * (i & 1);
            float l = i < 2 ? 0.f : acc[c], h = i < 2 ? 0.f : acc[c + 1];
            l = fmaf(fma_h(p0.x, s0, n0), xv[4 * i], l);     h = fmaf(fma_h(p1.x, s1, n1), xv[32 + 4 * i], h);
            l = fmaf(fma_h(p0.y, s0, n0), xv[4 * i + 2], l); h = fmaf(fma_h(p1.y, s1, n1), xv[32 + 4 * i + 2], h);
            l = fmaf(fma_h(p2.x, s0, n0), xv[4 * i + 1], l); h = fmaf(fma_h(p3.x, s1, n1), xv[32 + 4 * i + 1], h);
            l = fmaf(fma_h(p2.y, s0, n0), xv[4 * i + 3], l); h = fmaf(fma_h(p3.y, s1, n1), xv[32 + 4 * i + 3], h);
            acc[c] = l; acc[c + 1] = h;
        }
        return (acc[0] + acc[2]) + (acc[1] + acc[3]);
    }
};

template <> struct Unit<QMM_Q5_K> {
    // As Q4_K (unit = 64-weight chunk c of a super-block: sub-blocks 2c, 2c+1),
    // plus the fifth bit of every weight: bit i of qh[e] for element e of
    // sub-block i.  The bit joins the code while it is still an exact f16
    // subnormal: bit 4 of a low-nibble pair (c 2^-24), bit 8 of a high-nibble
    // pair (c 2^-20).  Super-blocks are 176 = 11 * 16 bytes: 16-byte aligned.
    static constexpr int NL = 20;  // 4 header dwords, 8 qh dwords, 8 nibble dwords
    struct Off { uint32_t hdr, qs; int c; };
    __device__ static Off lane_off(int u) {
        const uint32_t h = 176u * (u >> 2);
        return {h, h + 48u + 32u * (u & 3), u & 3};
    }
    __device__ static void load(Rsrc rs, uint32_t row, const Off &o, uint32_t (&v)[NL]) {
        uint32_t h[12], q[8];
        ldb(rs, o.hdr, row, h);  // d, dmin, scales, qh
        ldb(rs, o.qs, row, q);
#pragma unroll
        for (int i = 0; i < 12; i++) v[i] = h[i];
#pragma unroll
        for (int i = 0; i < 8; i++) v[12 + i] = q[i];
    }
    __device__ static int x4(int u, int i) { return 16 * u + i; }
    __device__ static float dot(const uint32_t (&v)[NL], const float (&xv)[64], const Off &o) {
        const float d = h2f(v[0]), dmin = h2f(v[0] >> 16);
        int sc0, m0, sc1, m1;
        q4k_scale_min(v[1], v[2], v[3], 2 * o.c, sc0, m0);
        q4k_scale_min(v[1], v[2], v[3], 2 * o.c + 1, sc1, m1);
        const float s0 = d * (float)sc0 * TWO24, n0 = -(dmin * (float)m0);
        const float s1 = d * (float)sc1 * TWO20, n1 = -(dmin * (float)m1);
        float acc[4];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t dw = v[12 + i], t = dw >> 8;
            const uint32_t hq = v[4 + i] >> (2 * o.c), ht = hq >> 8;  // qh[4i .. 4i+4), bits 2c and 2c+1 at 0, 1
            const half2_t p0 = as_h2((dw & 0x000F000Fu) | ((hq << 4) & 0x00100010u));
            const half2_t p1 = as_h2((dw & 0x00F000F0u) | ((hq << 7) & 0x01000100u));
            const half2_t p2 = as_h2((t & 0x000F000Fu) | ((ht << 4) & 0x00100010u));
            const half2_t p3 = as_h2((t & 0x00F000F0u) | ((ht << 7) & 0x01000100u));
            const int c = 2 * (i & 1);
            float l = i < 2 ? 0.f : acc[c], h = i < 2 ? 0.f : acc[c + 1];
            l = fmaf(fma_h(p0.x, s0, n0), xv[4 * i], l);     h = fmaf(fma_h(p1.x, s1, n1), xv[32 + 4 * i], h);
            l = fmaf(fma_h(p0.y, s0, n0), xv[4 * i + 2], l); h = fmaf(fma_h(p1.y, s1, n1), xv[32 + 4 * i + 2], h);
            l = fmaf(fma_h(p2.x, s0, n0), xv[4 * i + 1], l); h = fmaf(fma_h(p3.x, s1, n1), xv[32 + 4 * i + 1], h);
            l = fmaf(fma_h(p2.y, s0, n0), xv[4 * i + 3], l); h = fmaf(fma_h(p3.y, s1, n1), xv[32 + 4 * i + 3], h);
            acc[c] = l; acc[c + 1] = h;
        }
        return (acc[0] + acc[2]) + (acc[1] + acc[3]);
    }
};
template <> struct Unit<QMM_Q6_K> {
    // Unit u = 4 sb + 2 h + lh: the 64 weights {128h + 32g + 16lh + i : g < 4,
    // i < 16} of super-block sb, which share one 16-byte slice of each ql half
    // and of qh.  Loads: A = ql[64h+16lh ..+16], B = ql[64h+32+16lh ..+16],
    // C = qh[32h+16lh ..+16], S = sc[8h ..+8], D = d.  Super-blocks are 210
    // bytes, so odd ones start 2 bytes off a dword: the loads are byte-
    // addressed (unaligned buffer loads), which keeps every window at its
    // own size and needs no realignment.
    static constexpr int NL = 4 + 4 + 4 + 2 + 1;
    struct Off { uint32_t a, c, s, d; int lh; };
    __device__ static Off lane_off(int u) {
        const int h = (u >> 1) & 1, lh = u & 1;
        const uint32_t base = 210u * (u >> 2);
        return {base + 64u * h + 16u * lh, base + 128u + 32u * h + 16u * lh, base + 192u + 8u * h, base + 208u, lh};
    }
    __device__ static void load(Rsrc rs, uint32_t row, const Off &o, uint32_t (&v)[NL]) {
        const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(rs, o.a, row, 0);
        const u32x4_t b = __builtin_amdgcn_raw_buffer_load_b128(rs, o.a + 32u, row, 0);
        const u32x4_t c = __builtin_amdgcn_raw_buffer_load_b128(rs, o.c, row, 0);
        const u32x2_t sc = __builtin_amdgcn_raw_buffer_load_b64(rs, o.s, row, 0);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        v[8] = c.x; v[9] = c.y; v[10] = c.z; v[11] = c.w;
        v[12] = sc.x; v[13] = sc.y;
        v[14] = __builtin_amdgcn_raw_buffer_load_b16(rs, o.d, row, 0);
    }
    __device__ static int x4(int u, int i) {
        // unit u = 4b + 2h + lh covers x[256b + 128h + 32g + 16lh + j], g < 4, j < 16
        return 64 * (u >> 2) + 32 * ((u >> 1) & 1) + 8 * (i >> 2) + 4 * (u & 1) + (i & 3);
    }
    __device__ static float dot(const uint32_t (&v)[NL], const float (&xv)[64], const Off &o) {
        // code q = lo4 | hi2 << 4 per byte; (q - 32) 2^-24 as an exact f16 subnormal
        const half2_t b32 = as_h2(0x80208020u);  // -32 * 2^-24
        const float d = h2f(v[14]);
        float grp[4];
#pragma unroll
        for (int gp = 0; gp < 4; gp += 2) {  // two groups at a time: 8 independent chains
            half2_t w[2][4][2];  // [group][dword][bytes 0,2 | bytes 1,3]
#pragma unroll
            for (int k = 0; k < 2; k++) {
                const int g = gp + k;
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    const uint32_t L = (g & 1) ? v[4 + t] : v[t];
                    const uint32_t C = v[8 + t];
                    const uint32_t hi = (g < 2 ? (C << (4 - 2 * g)) : (C >> (2 * g - 4))) & 0x30303030u;
                    const uint32_t q = ((g < 2 ? L : (L >> 4)) & 0x0F0F0F0Fu) | hi;
                    w[k][t][0] = as_h2(q & 0x00FF00FFu) + b32;
                    w[k][t][1] = as_h2(__builtin_amdgcn_perm(0u, q, 0x0C030C01u)) + b32;
                }
            }
            float s8[8];
#pragma unroll
            for (int k = 0; k < 2; k++)
#pragma unroll
                for (int t = 0; t < 4; t++) s8[4 * k + t] = fma_h(w[k][t][0].x, xv[16 * (gp + k) + 4 * t], 0.f);
#pragma unroll
            for (int k = 0; k < 2; k++)
#pragma unroll
                for (int t = 0; t < 4; t++) s8[4 * k + t] = fma_h(w[k][t][1].x, xv[16 * (gp + k) + 4 * t + 1], s8[4 * k + t]);
#pragma unroll
            for (int k = 0; k < 2; k++)
#pragma unroll
                for (int t = 0; t < 4; t++) s8[4 * k + t] = fma_h(w[k][t][0].y, xv[16 * (gp + k) + 4 * t + 2], s8[4 * k + t]);
#pragma unroll
            for (int k = 0; k < 2; k++)
#pragma unroll
                for (int t = 0; t < 4; t++) s8[4 * k + t] = fma_h(w[k][t][1].y, xv[16 * (gp + k) + 4 * t + 3], s8[4 * k + t]);
            grp[gp] = (s8[0] + s8[1]) + (s8[2] + s8[3]);
            grp[gp + 1] = (s8[4] + s8[5]) + (s8[6] + s8[7]);
        }
        float total = 0.f;
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const uint32_t scw = (g < 2) ? v[12] : v[13];  // sc[8h .. 8h+4), sc[8h+4 .. 8h+8)
            const int sbyte = (int)__builtin_amdgcn_sbfe((int)scw, 16 * (g & 1) + 8 * o.lh, 8);  // sc[8h + 2g + lh]
            total = fmaf(d * 16777216.0f * (float)sbyte, grp[g], total);
        }
        return total;
    }
};

// ------------------------------------------ Q8_0-quantized activations ----
// The int8-activation variant (page "cera 0.5.2 src/backend/cpu.rs", the
// Q8_0 activation path: the activations are quantized to blocks of 32 int8
// codes with one scale each, and every weight block meets them in integer
// dot products).  A lane keeps, per token, the 64 activation codes of its
// unit (16 dwords, bytes ordered like the unit's weight bytes), the scales of
// the activation blocks the unit touches and the per-block code sums that
// the weights' offsets need.  Per activation block (per 16-weight sub-scale
// group for Q6_K) the integer sum of code products is exact
// (v_dot4_i32_i8); it is scaled once in f32:
//   Q8_0  (d xs) * sum q c                  Q4_0  (d xs) * (sum q c - 8 sum c)
//   Q4_1  (d xs) * sum q c + (m xs) * sum c
//   Q4_K, Q5_K  (d xs) * (sc * sum q c) - (dmin xs) * (m * sum c)
//   Q6_K  (d xs) * (sc * (sum q c - 32 sum c))
// The offsets -8 and -32 stay inside the exact integer sums; the Q4_1 and
// K-quant minimum terms are scaled separately, so their rounding is relative
// to sum |w - o| |xq| + sum |o| |xq| (o the weight's offset part).
struct XA {
    uint32_t c[16];  // codes, in the byte order dot() pairs them with
    float s[4];      // activation scales (2 used, 4 for Q6_K)
    int o[4];        // per-block integer offsets (see prep)
};

// Q8_0 quantization of four activations of a block whose other 28 sit in the
// seven neighbouring lanes (lanes 8j .. 8j+7 hold one block): the block's
// amax (a NaN never wins the comparison), d = amax/127, id = 1/d unless d is
// 0 or 1/d is not finite, codes = rint(v * id) clamped to [-128, 127] (NaN ->
// 0), packed little-endian; *d_out = d (the caller stores it rounded to f16).
// Every lane of the wavefront must call it.
//
// The lane maxima are combined across the 8 lanes with DPP moves inside the
// VALU (swap neighbours, swap pairs, mirror the half-row of 8: the same
// pattern as the first three steps of the wavefront sum), not with LDS
// permutes; a lane maximum is never NaN, so a plain max is exact there.  The
// clamp is done on the float before the conversion (NaN replaced first), so
// it compiles to selects, not branches.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
// the block maximum of |v| over the 8 lanes of the block
__device__ __forceinline__ float q8_block_amax(const floatx4 &v) {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const float a = fabsf(v[i]);
        amax = a > amax ? a : amax;
    }
    amax = fmaxf(amax, dpp_f<0xB1>(amax));   // quad_perm 1,0,3,2
    amax = fmaxf(amax, dpp_f<0x4E>(amax));   // quad_perm 2,3,0,1
    return fmaxf(amax, dpp_f<0x141>(amax));  // row_half_mirror
}
__device__ __forceinline__ void q8_scale(float amax, float &d, float &id) {
    d = amax / 127.0f;
    const float r = 1.0f / d;
    id = (d != 0.0f && __builtin_isfinite(r)) ? r : 0.0f;
}
__device__ __forceinline__ uint32_t q8_codes4(const floatx4 &v, float id) {
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const float q = rintf(v[i] * id);
        const float qc = q != q ? 0.0f : fminf(fmaxf(q, -128.0f), 127.0f);
        packed |= ((uint32_t)(int)qc & 0xFFu) << (8 * i);
    }
    return packed;
}
__device__ __forceinline__ uint32_t q8_quant4(const floatx4 &v, float *d_out) {
    float d, id;
    q8_scale(q8_block_amax(v), d, id);
    *d_out = d;
    return q8_codes4(v, id);
}
// v of lane k of each group of 8 lanes, to all 8: a quad_perm broadcast of
// lane k & 3 within each quad, then the other quad's copy by mirroring the
// half-row
template <int K>
__device__ __forceinline__ float bcast8(float v) {
    const float t = dpp_f<0x55 * (K & 3)>(v);
    const float u = dpp_f<0x141>(t);
    return (((threadIdx.x & 4) != 0) == (K >= 4)) ? t : u;
}
__device__ __forceinline__ float bcast8_k(float v, int k) {  // k a constant after unrolling
    switch (k) {
    case 0: return bcast8<0>(v);
    case 1: return bcast8<1>(v);
    case 2: return bcast8<2>(v);
    case 3: return bcast8<3>(v);
    case 4: return bcast8<4>(v);
    case 5: return bcast8<5>(v);
    case 6: return bcast8<6>(v);
    default: return bcast8<7>(v);
    }
}

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int acc) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, acc, false);
}
// sum of the 4 signed bytes of v
__device__ __forceinline__ int bsum4(uint32_t v, int acc) { return dot4(v, 0x01010101u, acc); }

template <int DT> struct U8;

template <> struct U8<QMM_Q4_0> {
    static constexpr int NS = 2;
    __device__ static int s_index(int u) { return 2 * u; }
    __device__ static void prep(XA &a) {
        // block 0's weight dwords are [qs0 qs1 qs14 qs15], qs2..5, qs6..9,
        // qs10..13 (the unit starts with d0); block 1's are natural
        int s[2] = {0, 0};
#pragma unroll
        for (int i = 0; i < 16; i++) s[i >> 3] = bsum4(a.c[i], s[i >> 3]);
        a.o[0] = -8 * s[0];
        a.o[1] = -8 * s[1];
#pragma unroll
        for (int h = 0; h < 2; h++) {  // low nibbles: codes 0..15, high: 16..31
            const uint32_t c0 = a.c[4 * h], c1 = a.c[4 * h + 1], c2 = a.c[4 * h + 2], c3 = a.c[4 * h + 3];
            a.c[4 * h] = __builtin_amdgcn_perm(c3, c0, 0x07060100u);
            a.c[4 * h + 1] = __builtin_amdgcn_alignbyte(c1, c0, 2);
            a.c[4 * h + 2] = __builtin_amdgcn_alignbyte(c2, c1, 2);
            a.c[4 * h + 3] = __builtin_amdgcn_alignbyte(c3, c2, 2);
        }
    }
    __device__ static float dot(const uint32_t (&v)[Unit<QMM_Q4_0>::NL], const XA &a, const Unit<QMM_Q4_0>::Off &) {
        const uint32_t D[2][4] = {{__builtin_amdgcn_alignbyte(v[4], v[0], 2), v[1], v[2], v[3]},
                                  {v[5], v[6], v[7], v[8]}};
        int s[2];
#pragma unroll
        for (int b = 0; b < 2; b++) {
            int acc = a.o[b];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                acc = dot4(D[b][i] & 0x0F0F0F0Fu, a.c[8 * b + i], acc);
                acc = dot4((D[b][i] >> 4) & 0x0F0F0F0Fu, a.c[8 * b + 4 + i], acc);
            }
            s[b] = acc;
        }
        return fmaf(h2f(v[4] >> 16) * a.s[1], (float)s[1], (h2f(v[0]) * a.s[0]) * (float)s[0]);
    }
};

template <> struct U8<QMM_Q4_1> {
    static constexpr int NS = 2;
    __device__ static int s_index(int u) { return 2 * u; }
    __device__ static void prep(XA &a) {
        int s[2] = {0, 0};
#pragma unroll
        for (int i = 0; i < 16; i++) s[i >> 3] = bsum4(a.c[i], s[i >> 3]);
        a.o[0] = s[0];
        a.o[1] = s[1];
    }
    __device__ static float dot(const uint32_t (&v)[Unit<QMM_Q4_1>::NL], const XA &a, const Unit<QMM_Q4_1>::Off &) {
        float t[2];
#pragma unroll
        for (int b = 0; b < 2; b++) {
            int acc = 0;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint32_t dw = v[5 * b + 1 + i];
                acc = dot4(dw & 0x0F0F0F0Fu, a.c[8 * b + i], acc);
                acc = dot4((dw >> 4) & 0x0F0F0F0Fu, a.c[8 * b + 4 + i], acc);
            }
            const float d = h2f(v[5 * b]), m = h2f(v[5 * b] >> 16);
            t[b] = fmaf(d * a.s[b], (float)acc, (m * a.s[b]) * (float)a.o[b]);
        }
        return t[0] + t[1];
    }
};

template <> struct U8<QMM_Q8_0> {
    static constexpr int NS = 2;
    __device__ static int s_index(int u) { return 2 * u; }
    __device__ static void prep(XA &) {}
    __device__ static float dot(const uint32_t (&v)[Unit<QMM_Q8_0>::NL], const XA &a, const Unit<QMM_Q8_0>::Off &) {
        int s[2];
#pragma unroll
        for (int b = 0; b < 2; b++) {
            int acc = 0;
#pragma unroll
            for (int i = 0; i < 8; i++)
                acc = dot4(b == 0 ? __builtin_amdgcn_alignbyte(v[i + 1], v[i], 2) : v[9 + i], a.c[8 * b + i], acc);
            s[b] = acc;
        }
        return fmaf(h2f(v[8] >> 16) * a.s[1], (float)s[1], (h2f(v[0]) * a.s[0]) * (float)s[0]);
    }
};

// Q4_K and Q5_K: the unit is chunk c of a super-block, sub-blocks 2c (low
// nibbles) and 2c+1 (high nibbles), activation blocks 2u and 2u+1.
__device__ __forceinline__ float kquant_pair(float d, float dmin, uint32_t s0w, uint32_t s1w, uint32_t s2w, int c,
                                             int acc0, int acc1, const XA &a) {
    int sc0, m0, sc1, m1;
    q4k_scale_min(s0w, s1w, s2w, 2 * c, sc0, m0);
    q4k_scale_min(s0w, s1w, s2w, 2 * c + 1, sc1, m1);
    // sc * acc (< 2^22) and m * sum (< 2^19) are exact as f32 products of
    // their exact f32 factors: the same values as the integer products, without
    // the quarter-rate integer multiply
    const float t0 = fmaf(d * a.s[0], (float)sc0 * (float)acc0, -((dmin * a.s[0]) * ((float)m0 * (float)a.o[0])));
    const float t1 = fmaf(d * a.s[1], (float)sc1 * (float)acc1, -((dmin * a.s[1]) * ((float)m1 * (float)a.o[1])));
    return t0 + t1;
}

template <> struct U8<QMM_Q4_K> {
    static constexpr int NS = 2;
    __device__ static int s_index(int u) { return 2 * u; }
    __device__ static void prep(XA &a) { U8<QMM_Q4_1>::prep(a); }
    __device__ static float dot(const uint32_t (&v)[Unit<QMM_Q4_K>::NL], const XA &a, const Unit<QMM_Q4_K>::Off &o) {
        int acc0 = 0, acc1 = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t dw = v[4 + i];
            acc0 = dot4(dw & 0x0F0F0F0Fu, a.c[i], acc0);
            acc1 = dot4((dw >> 4) & 0x0F0F0F0Fu, a.c[8 + i], acc1);
        }
        return kquant_pair(h2f(v[0]), h2f(v[0] >> 16), v[1], v[2], v[3], o.c, acc0, acc1, a);
    }
};

template <> struct U8<QMM_Q5_K> {
    static constexpr int NS = 2;
    __device__ static int s_index(int u) { return 2 * u; }
    __device__ static void prep(XA &a) { U8<QMM_Q4_1>::prep(a); }
    __device__ static float dot(const uint32_t (&v)[Unit<QMM_Q5_K>::NL], const XA &a, const Unit<QMM_Q5_K>::Off &o) {
        int acc0 = 0, acc1 = 0;
        const int sh = 2 * o.c;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t dw = v[12 + i], hq = v[4 + i] >> sh;  // qh bits 2c, 2c+1 at 0, 1
            acc0 = dot4((dw & 0x0F0F0F0Fu) | ((hq & 0x01010101u) << 4), a.c[i], acc0);
            acc1 = dot4(((dw >> 4) & 0x0F0F0F0Fu) | ((hq & 0x02020202u) << 3), a.c[8 + i], acc1);
        }
        return kquant_pair(h2f(v[0]), h2f(v[0] >> 16), v[1], v[2], v[3], o.c, acc0, acc1, a);
    }
};

template <> struct U8<QMM_Q6_K> {
    // unit u = 4b + 2h + lh: group g (16 weights, sub-scale sc[8h + 2g + lh])
    // lies in activation block 8b + 4h + g; codes dword 4g + t of the unit
    static constexpr int NS = 4;
    __device__ static int s_index(int u) { return 8 * (u >> 2) + 4 * ((u >> 1) & 1); }
    __device__ static void prep(XA &a) {
#pragma unroll
        for (int g = 0; g < 4; g++) {
            int s = 0;
#pragma unroll
            for (int t = 0; t < 4; t++) s = bsum4(a.c[4 * g + t], s);
            a.o[g] = -32 * s;
        }
    }
    __device__ static float dot(const uint32_t (&v)[Unit<QMM_Q6_K>::NL], const XA &a, const Unit<QMM_Q6_K>::Off &o) {
        const float d = h2f(v[14]);
        float total = 0.f;
#pragma unroll
        for (int g = 0; g < 4; g++) {
            int acc = a.o[g];
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const uint32_t L = (g & 1) ? v[4 + t] : v[t];
                const uint32_t C = v[8 + t];
                const uint32_t hi = (g < 2 ? (C << (4 - 2 * g)) : (C >> (2 * g - 4))) & 0x30303030u;
                const uint32_t q = ((g < 2 ? L : (L >> 4)) & 0x0F0F0F0Fu) | hi;
                acc = dot4(q, a.c[4 * g + t], acc);
            }
            const uint32_t scw = (g < 2) ? v[12] : v[13];
            const int sbyte = (int)__builtin_amdgcn_sbfe((int)scw, 16 * (g & 1) + 8 * o.lh, 8);  // sc[8h + 2g + lh]
            // |sc * acc| < 2^22: the f32 product of the exact factors is exact
            total = fmaf(d * a.s[g], (float)sbyte * (float)acc, total);
        }
        return total;
    }
};

// Issue the loads of one token's codes and scales for unit u (K = 64 U
// codes, K / 32 scales); U8<DT>::prep finishes the set once they arrive.
template <int DT>
__device__ __forceinline__ void load_xa(const int8_t *xq, const float *xsc, int u, XA &a) {
    const u32x4_t *q = reinterpret_cast<const u32x4_t *>(xq);
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const u32x4_t v = q[Unit<DT>::x4(u, 4 * j) >> 2];
        a.c[4 * j] = v.x; a.c[4 * j + 1] = v.y; a.c[4 * j + 2] = v.z; a.c[4 * j + 3] = v.w;
    }
    const int si = U8<DT>::s_index(u);
    if constexpr (U8<DT>::NS == 4) {
        const floatx4 s = *reinterpret_cast<const floatx4 *>(xsc + si);
        a.s[0] = s.x; a.s[1] = s.y; a.s[2] = s.z; a.s[3] = s.w;
    } else {
        const float2 s = *reinterpret_cast<const float2 *>(xsc + si);
        a.s[0] = s.x; a.s[1] = s.y; a.s[2] = 0.f; a.s[3] = 0.f;
    }
}

// Activations go through LDS laid out so that the 16 lanes of a read phase,
// each reading its own unit, hit distinct banks:
//   PAD    one float4 of padding after every 16 (17 float4s per 64 values):
//          a lane's 16 reads are one base address plus constant offsets
//          (whole-row wavefronts, 272 bytes per unit);
//   else   the float4 index XOR-swizzled within groups of 16 (256 bytes per
//          unit; per-read address arithmetic).
template <bool PAD>
__device__ __forceinline__ int xslot(int f) {
    if constexpr (PAD) return f + (f >> 4);
    else return (f & ~15) | ((f & 15) ^ ((f >> 4) & 15));
}
constexpr size_t xs_unit_bytes(bool pad) { return pad ? 272 : 256; }

// The activations are fetched into registers before any weight load is
// issued and written to LDS afterwards: vector-memory loads return in order,
// so fetching x after the weight prefetch would make the first product wait
// for every prefetched weight byte.  Callers put a scheduling barrier between
// load_x and the weight fetches: left alone, the compiler moves weight loads
// ahead of activation loads.  XPT = float4 per thread (16 U <= XPT *
// blockDim).
template <int XPT>
__device__ __forceinline__ void load_x(const float *x, int U, floatx4 (&r)[XPT]) {
    const floatx4 *xg = reinterpret_cast<const floatx4 *>(x);
    const int last = 16 * U - 1;
#pragma unroll
    for (int i = 0; i < XPT; i++) {
        const int f = threadIdx.x + i * blockDim.x;
        r[i] = xg[f < last ? f : last];  // unconditional: no divergent load to wait on
    }
}
// Stores past the last float4 go to the last one with its own value (load_x
// read it there): no branch, so the compiler cannot sink a load into one and
// make its store wait for every load issued after it.
template <bool PAD, int XPT>
__device__ __forceinline__ void store_x(const floatx4 (&r)[XPT], int U, floatx4 *xs) {
    const int last = 16 * U - 1;
#pragma unroll
    for (int i = 0; i < XPT; i++) {
        const int f = threadIdx.x + i * blockDim.x;
        xs[xslot<PAD>(f < last ? f : last)] = r[i];
    }
}

// With PAD the offsets of a unit's float4s from its first one do not depend
// on the lane: every unit layout starts at a multiple of 16 or at 4 more, and
// its float4s lie at offsets o (< 28) with (first % 16) + (o % 16) < 16, so
// xslot(first + o) = xslot(first) + o + o / 16.
template <int DT, bool PAD>
__device__ __forceinline__ void x_from_lds(const floatx4 *xs, int u, float (&xv)[64]) {
    const int first = Unit<DT>::x4(u, 0);
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int o = Unit<DT>::x4(u, i) - first;
        const floatx4 v = PAD ? xs[xslot<true>(first) + o + (o >> 4)] : xs[xslot<false>(Unit<DT>::x4(u, i))];
        xv[4 * i] = v.x; xv[4 * i + 1] = v.y; xv[4 * i + 2] = v.z; xv[4 * i + 3] = v.w;
    }
}

// ------------------------------------------------------------ fast kernel ----
// WAVE_ROWS: K <= 4096, independent wavefronts (4 per workgroup; 8 for most
// int8 one-launch calls, see gemv_block_threads), each with its
// own range of row groups.  Otherwise the workgroup's ceil(U/64) wavefronts
// split K and reduce each row group through LDS.  D row groups are in flight
// while one is decoded (a ring of D+1 register buffers, unrolled so that no
// buffer is indexed dynamically).
//
// Every weight fetch is issued unconditionally as bounds-checked buffer loads
// (rows past M and row groups past the wavefront's range read as zeros
// without touching memory), so the loop has no branch around a load and the
// compiler's wait counts stay exact: each decode waits for its own row group
// only, never for the whole ring.
//
// FLAT: every wavefront (or workgroup) owns at most D+1 row groups; all of
// them are fetched up front and decoded in order, with no fetch in the loop.
//
// MODE selects what a row group is and where its results go:
//   GEMV_ONE     R rows of one matrix;  y = W x.
//   GEMV_CONCAT  up to GEMV_MAX_MATS matrices that share K and x, run as one
//                range of row groups, matrix after matrix (a matrix of M_i
//                rows owns groups [g_lo[i], g_lo[i+1])); y_i = W_i x.  Each
//                row's arithmetic is the single-matrix kernel's, so the bits
//                match separate calls (page "cera 0.5.2 src/backend/cpu.rs",
//                the fused dual and concatenated three-matrix GEMVs: one
//                dispatch and one read of x for several projections).
//   GEMV_SWIGLU  R rows of the gate matrix and the same R rows of the up
//                matrix; out = silu(W_gate x) * (W_up x) (same page, the
//                fused gate + up GEMV with in-register SwiGLU).
//   GEMV_PAIR    two matrices of equal M (the concatenated call's gate + up
//                case): a group holds R rows of the first and the same R rows
//                of the second, as GEMV_SWIGLU, and both sums are stored
//                (y_0 = W_0 x, y_1 = W_1 x, the single-matrix bits).  Reading
//                the two matrices' rows side by side was measured faster than
//                running them one after the other (2 x 14336 x 4096 Q4_0:
//                13.8 against 15.2 us).
//   GEMV_ARGMAX  R rows of one matrix; nothing is stored per row: every
//                workgroup writes the best (value, row) of its rows to
//                part[blockIdx.x] and gemv_argmax_finish picks the overall
//                winner (same page, the greedy argmax GEMV that returns the
//                index without storing the logits).  The values compared are
//                the single-matrix kernel's f32 sums, bit for bit.
enum { GEMV_ONE = 0, GEMV_CONCAT = 1, GEMV_SWIGLU = 2, GEMV_ARGMAX = 3, GEMV_PAIR = 4 };
// modes whose row group holds R rows of each of two matrices
constexpr bool gemv_two_mats(int mode) { return mode == GEMV_SWIGLU || mode == GEMV_PAIR; }
constexpr int GEMV_MAX_MATS = 4;

struct GemvMats {
    const uint8_t *blob[GEMV_MAX_MATS];
    float *y[GEMV_MAX_MATS];
    int64_t M[GEMV_MAX_MATS];
    int64_t g_lo[GEMV_MAX_MATS + 1];  // unused entries hold the total group count
    float2 *part;                     // GEMV_ARGMAX: one (value, row bits) per workgroup
};

// The argmax order: a larger value wins; equal values go to the smaller row;
// NaN never wins; row < 0 marks "nothing yet".
__device__ __forceinline__ bool beats(float v, int row, float bv, int brow) {
    return row >= 0 && v == v && (brow < 0 || v > bv || (v == bv && row < brow));
}

// Field i of a kernel-argument array, by selects (a dynamic index would copy
// the argument block to scratch).
template <typename T>
__device__ __forceinline__ T pick(const T (&a)[GEMV_MAX_MATS], int i) {
    T v = a[0];
#pragma unroll
    for (int j = 1; j < GEMV_MAX_MATS; j++) v = i == j ? a[j] : v;
    return v;
}
__device__ __forceinline__ int mat_of(const GemvMats &m, int64_t g) {
    int i = 0;
#pragma unroll
    for (int j = 1; j < GEMV_MAX_MATS; j++) i = g >= m.g_lo[j] ? j : i;
    return i;
}
__device__ __forceinline__ int64_t lo_of(const GemvMats &m, int i) {
    int64_t v = 0;
#pragma unroll
    for (int j = 1; j < GEMV_MAX_MATS; j++) v = i == j ? m.g_lo[j] : v;
    return v;
}

//
// NT = 0: f32 activations x.  NT >= 1: Q8_0-quantized activations of NT
// tokens per weight read (codes xq [ntok][K], scales xsc [ntok][K/32]; token
// group blockIdx.y covers tokens NT*blockIdx.y ..; outputs y[tok][M]); GEMV_ONE
// only.  NT = -1: one token of f32 activations x, quantized to Q8_0 by the
// workgroup itself (into LDS, the quantizer kernel's arithmetic, so the codes
// are the ones qmm_quantize_q8_0 writes), then the int8 dots; every MODE.
//
// Workgroup size: 256 threads, except whole-row wavefronts with x quantized
// in the launch (not Q6_K, whose head runs 4 wavefronts per CU): 512, so the
// quantization of x, done once per workgroup, is shared by 8 wavefronts and
// each thread quantizes 2 float4 rounds instead of 4.
constexpr int gemv_block_threads(int dt, bool wave_rows, int nt) {
    return (wave_rows && nt < 0 && dt != QMM_Q6_K) ? 512 : 256;
}
template <int DT, int R, int D, bool WAVE_ROWS, bool FLAT, int MODE, int NT, int PH = 1>
__global__ void __launch_bounds__(gemv_block_threads(DT, WAVE_ROWS, NT) * PH) gemv_kernel(const GemvMats mats, int64_t row_bytes, int U,
                                                   const float *__restrict__ x, int64_t per_owner, int64_t extra,
                                                   const int8_t *__restrict__ xq, const float *__restrict__ xsc,
                                                   int64_t ntok) {
    static_assert(NT <= 0 || MODE == GEMV_ONE, "several int8 tokens: one matrix");
    static_assert(PH == 1 || (!WAVE_ROWS && MODE == GEMV_ONE && NT == 0), "row phases: f32 K-split, one matrix");
    constexpr int NL = Unit<DT>::NL;
    constexpr int RR = gemv_two_mats(MODE) ? 2 * R : R;  // row dots per row group
    constexpr int TK = NT > 0 ? NT : 1;                  // tokens per row dot
    extern __shared__ __attribute__((aligned(16))) floatx4 xs[];
    constexpr int RED_G = 16;
    __shared__ float red[PH][WAVE_ROWS ? 1 : RED_G][RR * TK][4];
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6), nwaves = blockDim.x >> 6;
    // K-split: PH row phases of nwaves / PH wavefronts each; a phase is an
    // owner of its own (the workgroup stages x once for all of them)
    const int kw = nwaves / PH;                               // wavefronts per row
    const int phase = WAVE_ROWS ? 0 : wave / kw;
    const int wk = wave - phase * kw;                         // K slice of the wavefront
    const int tp = t - phase * 64 * kw;                       // thread within its phase
    const int u = WAVE_ROWS ? lane : tp;
    const bool active = u < U;
    // owner o gets per_owner row groups, plus one more for the first `extra` owners
    const int64_t owner = WAVE_ROWS ? (int64_t)blockIdx.x * nwaves + wave : (int64_t)blockIdx.x * PH + phase;
    const int64_t g0 = owner * per_owner + (owner < extra ? owner : extra);
    const int64_t n = per_owner + (owner < extra ? 1 : 0);
    // row-group steps: with phases every phase takes the most any owner has
    // (an owner with one fewer decodes zeros once and stores nothing), so all
    // wavefronts meet the same barriers
    const int64_t nloop = PH > 1 ? per_owner + (extra > 0 ? 1 : 0) : n;
    const int64_t nrg = mats.g_lo[GEMV_MAX_MATS];
    const int64_t gend = g0 + n < nrg ? g0 + n : nrg;  // past the wavefront's last row group
    const typename Unit<DT>::Off off = Unit<DT>::lane_off(active ? u : 0);

    uint32_t buf[D + 1][RR][NL];
    auto fetch = [&](int64_t g, uint32_t (&b)[RR][NL]) {
        const bool in = g < gend;
        const int mi = (MODE == GEMV_CONCAT && in) ? mat_of(mats, g) : 0;
        const int64_t lg = in ? g - (MODE == GEMV_CONCAT ? lo_of(mats, mi) : 0) : 0;  // group within its matrix
        const int64_t Mi = MODE == GEMV_CONCAT ? pick(mats.M, mi) : mats.M[0];
        // rows of the group that exist; none when g is past the range
        const int64_t rows = in ? (Mi - lg * R < R ? Mi - lg * R : R) : 0;
        const uint8_t *base = MODE == GEMV_CONCAT ? pick(mats.blob, mi) : mats.blob[0];
        const Rsrc rs = make_rsrc(base + lg * R * row_bytes, (uint32_t)(rows * row_bytes));
#pragma unroll
        for (int r = 0; r < R; r++) Unit<DT>::load(rs, (uint32_t)(r * row_bytes), off, b[r]);
        if constexpr (gemv_two_mats(MODE)) {
            const Rsrc ru = make_rsrc(mats.blob[1] + lg * R * row_bytes, (uint32_t)(rows * row_bytes));
#pragma unroll
            for (int r = 0; r < R; r++) Unit<DT>::load(ru, (uint32_t)(r * row_bytes), off, b[R + r]);
        }
    };
    // results of row r of group g (every lane that calls holds the sums)
    float best_v = 0.f;  // GEMV_ARGMAX: this thread's best row so far (rows < 2^31)
    int best_row = -1;
    const int64_t tok0 = (int64_t)blockIdx.y * TK;
    auto put = [&](int64_t g, int r, float v, float vu, int tn) {
        if constexpr (NT > 0) {
            const int64_t row = g * R + r;
            if (row < mats.M[0] && tok0 + tn < ntok) mats.y[0][(tok0 + tn) * mats.M[0] + row] = v;
        } else if constexpr (MODE == GEMV_ARGMAX) {
            const int64_t row = g * R + r;
            if (row < mats.M[0] && beats(v, (int)row, best_v, best_row)) {
                best_v = v;
                best_row = (int)row;
            }
        } else if constexpr (MODE == GEMV_SWIGLU) {
            const int64_t row = g * R + r;
            if (row < mats.M[0]) mats.y[0][row] = silu(v) * vu;
        } else if constexpr (MODE == GEMV_PAIR) {
            const int64_t row = g * R + r;
            if (row < mats.M[0]) {
                mats.y[0][row] = v;
                mats.y[1][row] = vu;
            }
        } else {
            const int mi = MODE == GEMV_CONCAT ? mat_of(mats, g) : 0;
            const int64_t row = (g - (MODE == GEMV_CONCAT ? lo_of(mats, mi) : 0)) * R + r;
            if (row < (MODE == GEMV_CONCAT ? pick(mats.M, mi) : mats.M[0]))
                (MODE == GEMV_CONCAT ? pick(mats.y, mi) : mats.y[0])[row] = v;
        }
    };
    float xv[NT != 0 ? 1 : 64];
    XA xa[TK];
    if constexpr (NT < 0) {
        // x f32 -> Q8_0 codes (dwords [0, 16U)) and scales (floats after
        // them) in LDS; eight consecutive threads share a block
        // float4 of x per thread: 16 U <= QPT * blockDim (U <= 64 with whole rows)
        constexpr int QPT = WAVE_ROWS ? 1024 / gemv_block_threads(DT, WAVE_ROWS, NT) : 16;
        const int nf = 16 * U;
        const floatx4 *xg = reinterpret_cast<const floatx4 *>(x);
        floatx4 xr[QPT];
#pragma unroll
        for (int i = 0; i < QPT; i++) {
            const int f = t + i * (int)blockDim.x;
            xr[i] = xg[f < nf ? f : nf - 1];  // whole 8-lane groups are in or out of range
        }
#pragma unroll
        for (int s = 0; s < (FLAT ? D + 1 : D); s++) fetch(g0 + s, buf[s]);
        uint32_t *cs = reinterpret_cast<uint32_t *>(xs);
        float *ss = reinterpret_cast<float *>(cs + nf);
        // every float4 round i quantizes one block per 8 lanes.  The block
        // maxima of 8 rounds are gathered so that lane k of a group of 8
        // holds round 8j + k's, one division pair serves all 8 rounds, that
        // lane stores the block's scale, and the reciprocal goes back to the
        // block's 8 lanes (same arithmetic as q8_quant4, one division per 8)
        float am[QPT];
#pragma unroll
        for (int i = 0; i < QPT; i++) am[i] = q8_block_amax(xr[i]);
        const int k8 = lane & 7;
#pragma unroll
        for (int j = 0; j < (QPT + 7) / 8; j++) {
            float g = 0.f;
#pragma unroll
            for (int k = 0; k < 8 && 8 * j + k < QPT; k++) g = k8 == k ? am[8 * j + k] : g;
            float d, id;
            q8_scale(g, d, id);
            const int fb = (t & ~7) + (8 * j + k8) * (int)blockDim.x;  // first float4 of that block
            if (8 * j + k8 < QPT && fb < nf) ss[fb >> 3] = (float)(_Float16)d;
#pragma unroll
            for (int k = 0; k < 8 && 8 * j + k < QPT; k++) {
                const int i = 8 * j + k, f = t + i * (int)blockDim.x;
                const uint32_t packed = q8_codes4(xr[i], bcast8_k(id, k));
                if (f < nf) cs[f] = packed;
            }
        }
        __syncthreads();
        const int uu = active ? u : 0;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const u32x4_t v = *reinterpret_cast<const u32x4_t *>(cs + Unit<DT>::x4(uu, 4 * j));
            xa[0].c[4 * j] = v.x; xa[0].c[4 * j + 1] = v.y; xa[0].c[4 * j + 2] = v.z; xa[0].c[4 * j + 3] = v.w;
        }
        const int si = U8<DT>::s_index(uu);
#pragma unroll
        for (int j = 0; j < 4; j++) xa[0].s[j] = j < U8<DT>::NS ? ss[si + j] : 0.f;
        U8<DT>::prep(xa[0]);
    } else if constexpr (NT > 0) {
        // every lane fetches its own unit's codes (64 bytes per token) before
        // the weights; tokens past the end repeat the last one (not stored)
        const int64_t K = 64 * (int64_t)U;
#pragma unroll
        for (int n = 0; n < TK; n++) {
            const int64_t tk = tok0 + n < ntok ? tok0 + n : ntok - 1;
            load_xa<DT>(xq + tk * K, xsc + tk * (K / 32), active ? u : 0, xa[n]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < (FLAT ? D + 1 : D); s++) fetch(g0 + s, buf[s]);
#pragma unroll
        for (int n = 0; n < TK; n++) U8<DT>::prep(xa[n]);
    } else if constexpr (WAVE_ROWS) {
        // 256 threads x 4 float4 = 64 units, every slot of the padded LDS
        // layout (sized for 64 units): bounds-checked buffer loads return
        // zeros past 16 U float4s, stored where no lane reads, so the
        // addresses are one lane offset plus constants and nothing is clamped
        static_assert(gemv_block_threads(DT, true, NT) == 256, "4 float4 of x per thread");
        const Rsrc xrs = make_rsrc(x, (uint32_t)U * 256u);
        floatx4 xr[4];
#pragma unroll
        for (int i = 0; i < 4; i++)
            xr[i] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(xrs, 16u * t, 4096u * i, 0));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < (FLAT ? D + 1 : D); s++) fetch(g0 + s, buf[s]);
#pragma unroll
        for (int i = 0; i < 4; i++) xs[xslot<true>(t + 256 * i)] = xr[i];
        __syncthreads();
        x_from_lds<DT, true>(xs, active ? u : 0, xv);
        // the activation reads go out before the wait for the first weights
        __builtin_amdgcn_sched_barrier(0);
    } else {
        floatx4 xr[16 / PH];  // 16 U <= (16 / PH) * blockDim
        load_x(x, U, xr);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < (FLAT ? D + 1 : D); s++) fetch(g0 + s, buf[s]);
        store_x<false>(xr, U, xs);
        __syncthreads();
        x_from_lds<DT, false>(xs, active ? u : 0, xv);
    }

    // one matrix, whole-row wavefronts with a ring of row groups: a
    // wavefront's rows are consecutive, so their sums are parked one per lane
    // and written 64 at a time with one coalesced store (single-lane 4-byte
    // stores are partial-line writes).  Wavefronts owning at most D + 1
    // groups (FLAT) store from lane 63 instead: the parking costs ~15 VALU
    // instructions per row and saves little on one or two rows (14336 x 4096
    // Q4_0 9.4 -> 9.1 us, 4096 x 4096 4.5 -> 4.4 us).
    constexpr bool BATCH = WAVE_ROWS && MODE == GEMV_ONE && NT <= 1 && !FLAT;
    float obuf = 0.f;
    const int64_t orow0 = g0 * R;  // first row of the wavefront's range
    auto flush = [&](int64_t k0, int cnt) {  // rows orow0 + k0 + [0, cnt) from lanes [0, cnt)
        const int64_t row = orow0 + k0 + lane;
        if (lane < cnt && row < mats.M[0]) mats.y[0][row] = obuf;
    };
    for (int64_t i0 = 0; i0 < nloop; i0 += D + 1) {
#pragma unroll
        for (int s = 0; s <= D; s++) {
            const int64_t i = i0 + s;
            if (!FLAT) fetch(g0 + i + D, buf[(s + D) % (D + 1)]);
            if (i < nloop) {
                float acc[RR * TK];  // [row][token]
#pragma unroll
                for (int r = 0; r < RR; r++) {
#pragma unroll
                    for (int tn = 0; tn < TK; tn++) {
                        float d;
                        if constexpr (NT != 0) d = U8<DT>::dot(buf[s][r], xa[tn], off);
                        else d = Unit<DT>::dot(buf[s][r], xv, off);
                        acc[r * TK + tn] = wave_sum_to_lane63(active ? d : 0.f);
                    }
                }
                if constexpr (BATCH) {
#pragma unroll
                    for (int r = 0; r < R; r++) {
                        const int64_t k = i * R + r;  // row offset in the range
                        const float v = __builtin_bit_cast(
                            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, acc[r]), 63));
                        if (lane == (int)(k & 63)) obuf = v;
                        if ((k & 63) == 63) flush(k - 63, 64);
                    }
                } else if (WAVE_ROWS) {
                    if (lane == 63) {
#pragma unroll
                        for (int r = 0; r < R; r++)
#pragma unroll
                            for (int tn = 0; tn < TK; tn++)
                                put(g0 + i, r, acc[r * TK + tn], acc[gemv_two_mats(MODE) ? R + r : r], tn);
                    }
                } else {
                    // partial sums of up to RED_G row groups wait in LDS; one
                    // barrier pair per RED_G groups (the count is uniform
                    // across the workgroup)
                    const int slot = (int)(i % RED_G);
                    if (lane == 63) {
#pragma unroll
                        for (int r = 0; r < RR * TK; r++) red[phase][slot][r][wk] = acc[r];
                    }
                    if (slot == RED_G - 1 || i == nloop - 1) {
                        __syncthreads();
                        // groups past the owner's count (phases only) are not stored
                        if (tp < (slot + 1) * R * TK && i - slot + tp / (R * TK) < n) {
                            const int gi = tp / (R * TK), r = (tp % (R * TK)) / TK, tn = tp % TK;
                            float sum = red[phase][gi][r * TK + tn][0], su = 0.f;
                            for (int w = 1; w < kw; w++) sum += red[phase][gi][r * TK + tn][w];
                            if constexpr (gemv_two_mats(MODE)) {
                                su = red[phase][gi][R + r][0];
                                for (int w = 1; w < kw; w++) su += red[phase][gi][R + r][w];
                            }
                            put(g0 + i - slot + gi, r, sum, su, tn);
                        }
                        __syncthreads();
                    }
                }
            }
        }
    }
    if constexpr (BATCH) {
        const int64_t total = n * R;  // rows of the range (past-M rows are not stored)
        if ((total & 63) != 0) flush(total & ~(int64_t)63, (int)(total & 63));
    }
    if constexpr (MODE == GEMV_ARGMAX) {
        // the best of the workgroup: lane 63 of every wavefront (whole rows) or
        // the reducing threads (split K) hold candidates
        constexpr int NC = WAVE_ROWS ? gemv_block_threads(DT, WAVE_ROWS, NT) / 64 : RED_G * R;
        __shared__ float cv[NC];
        __shared__ int cr[NC];
        const int c = WAVE_ROWS ? (lane == 63 ? wave : -1) : (t < NC ? t : -1);
        if (c >= 0) {
            cv[c] = best_v;
            cr[c] = best_row;
        }
        __syncthreads();
        if (t == 0) {
            float bv = 0.f;
            int br = -1;
            const int nc = WAVE_ROWS ? nwaves : NC;
            for (int i = 0; i < nc; i++)
                if (beats(cv[i], cr[i], bv, br)) {
                    bv = cv[i];
                    br = cr[i];
                }
            mats.part[blockIdx.x] = float2{bv, __int_as_float(br)};
        }
    }
}

// The winner among the workgroups' candidates: one workgroup, a strided scan
// per thread, then a tree over the threads with the same order.
__global__ void __launch_bounds__(256) gemv_argmax_finish(const float2 *__restrict__ part, int nparts,
                                                          int64_t *__restrict__ index, float *__restrict__ value) {
    __shared__ float sv[256];
    __shared__ int sr[256];
    const int t = threadIdx.x;
    float bv = 0.f;
    int br = -1;
    for (int i = t; i < nparts; i += 256) {
        const float2 p = part[i];
        const int r = __float_as_int(p.y);
        if (beats(p.x, r, bv, br)) {
            bv = p.x;
            br = r;
        }
    }
    sv[t] = bv;
    sr[t] = br;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (t < w && beats(sv[t + w], sr[t + w], sv[t], sr[t])) {
            sv[t] = sv[t + w];
            sr[t] = sr[t + w];
        }
        __syncthreads();
    }
    if (t == 0) {
        *index = sr[0];
        if (value) *value = sr[0] >= 0 ? sv[0] : __builtin_nanf("");
    }
}

// ------------------------------------------------------- several tokens ----
// Y[j][m] for up to NT tokens with whole-row wavefronts (K <= 4096): the
// weights stream once for all of them, and every token's dot product is
// computed with exactly the single-token kernel's arithmetic (the same unit
// dot, the same cross-lane sum), so each output has the bits the GEMV
// returns for that token alone -- a batch of draft tokens is verified with
// the numbers greedy decoding produced (page "cera 0.5.0 src/model/llama.rs",
// project_logits_batched: one read of the LM head for all verified
// positions; page "cera 0.5.2 src/backend/cpu.rs": decode and prefill must
// give the same bits).  The activations of all tokens wait in LDS; each
// token's 64 values per lane are read back once per row group and shared by
// the group's R rows.  Tokens past ntok are never computed or stored.
template <int DT, int R, int D, int NT>
__global__ void __launch_bounds__(256) gemv_tokens_kernel(const uint8_t *__restrict__ blob, int64_t M,
                                                          int64_t row_bytes, int U, const float *__restrict__ X,
                                                          float *__restrict__ Y, int ntok, int64_t per_owner,
                                                          int64_t extra) {
    constexpr int NL = Unit<DT>::NL;
    extern __shared__ __attribute__((aligned(16))) floatx4 xs[];  // NT blocks of 16 U float4
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6), nwaves = blockDim.x >> 6;
    const bool active = lane < U;
    const int64_t owner = (int64_t)blockIdx.x * nwaves + wave;
    const int64_t g0 = owner * per_owner + (owner < extra ? owner : extra);
    const int64_t n = per_owner + (owner < extra ? 1 : 0);
    const int64_t nrg = (M + R - 1) / R;
    const int64_t gend = g0 + n < nrg ? g0 + n : nrg;
    const typename Unit<DT>::Off off = Unit<DT>::lane_off(active ? lane : 0);
    const int64_t K = (int64_t)U * 64;

    uint32_t buf[D + 1][R][NL];
    auto fetch = [&](int64_t g, uint32_t (&b)[R][NL]) {
        const int64_t rows = g < gend ? (M - g * R < R ? M - g * R : R) : 0;
        const Rsrc rs = make_rsrc(blob + (g < gend ? g : 0) * R * row_bytes, (uint32_t)(rows * row_bytes));
#pragma unroll
        for (int r = 0; r < R; r++) Unit<DT>::load(rs, (uint32_t)(r * row_bytes), off, b[r]);
    };
    {
        floatx4 xr[NT][4];
#pragma unroll
        for (int j = 0; j < NT; j++) load_x(X + (j < ntok ? j : ntok - 1) * K, U, xr[j]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < D; s++) fetch(g0 + s, buf[s]);
#pragma unroll
        for (int j = 0; j < NT; j++) store_x<false>(xr[j], U, xs + j * 16 * U);
    }
    __syncthreads();
    float xv[64];

    for (int64_t i0 = 0; i0 < n; i0 += D + 1) {
#pragma unroll
        for (int s = 0; s <= D; s++) {
            const int64_t i = i0 + s;
            fetch(g0 + i + D, buf[(s + D) % (D + 1)]);
            if (i < n) {
                const int64_t row0 = (g0 + i) * R;
#pragma unroll
                for (int j = 0; j < NT; j++) {
                    if (j < ntok) {
                        x_from_lds<DT, false>(xs + j * 16 * U, active ? lane : 0, xv);
                        float acc[R];
#pragma unroll
                        for (int r = 0; r < R; r++) {
                            const float d = Unit<DT>::dot(buf[s][r], xv, off);
                            acc[r] = wave_sum_to_lane63(active ? d : 0.f);
                        }
                        if (lane == 63) {
#pragma unroll
                            for (int r = 0; r < R; r++)
                                if (row0 + r < M) Y[j * M + row0 + r] = acc[r];
                        }
                    }
                }
            }
        }
    }
}

// More units than 4 wavefronts of lanes (K > 16384): each thread loops over
// its units and reloads their activations for every row group.
template <int DT, int R>
__global__ void __launch_bounds__(256) gemv_multi_kernel(const uint8_t *__restrict__ blob, int64_t M,
                                                         int64_t row_bytes, int U,
                                                         const float *__restrict__ x, float *__restrict__ y) {
    __shared__ float red[R][4];
    const int t = threadIdx.x, T = blockDim.x, lane = t & 63, wave = t >> 6, nwaves = T >> 6;
    const int64_t nrg = (M + R - 1) / R;
    const floatx4 *xg = reinterpret_cast<const floatx4 *>(x);
    float xv[64];
    for (int64_t rg = blockIdx.x; rg < nrg; rg += gridDim.x) {
        const int64_t row0 = rg * R;
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; r++) acc[r] = 0.f;
        for (int u = t; u < U; u += T) {
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const floatx4 v = xg[Unit<DT>::x4(u, i)];
                xv[4 * i] = v.x; xv[4 * i + 1] = v.y; xv[4 * i + 2] = v.z; xv[4 * i + 3] = v.w;
            }
            const typename Unit<DT>::Off off = Unit<DT>::lane_off(u);
            uint32_t raw[R][Unit<DT>::NL];
            const int64_t rows = M - row0 < R ? M - row0 : R;
            const Rsrc rs = make_rsrc(blob + row0 * row_bytes, (uint32_t)(rows * row_bytes));
#pragma unroll
            for (int r = 0; r < R; r++) Unit<DT>::load(rs, (uint32_t)(r * row_bytes), off, raw[r]);
#pragma unroll
            for (int r = 0; r < R; r++)
                if (row0 + r < M) acc[r] += Unit<DT>::dot(raw[r], xv, off);
        }
#pragma unroll
        for (int r = 0; r < R; r++) {
            const float sum = wave_sum_to_lane63(acc[r]);
            if (lane == 63) red[r][wave] = sum;
        }
        __syncthreads();
        if (t < R && row0 + t < M) {
            float sum = red[t][0];
            for (int w = 1; w < nwaves; w++) sum += red[t][w];
            y[row0 + t] = sum;
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
__device__ float block_dot_generic<QMM_Q4_1>(const uint8_t *p, const float *x) {
    const float d = h2f((uint32_t)p[0] | ((uint32_t)p[1] << 8));
    const float m = h2f((uint32_t)p[2] | ((uint32_t)p[3] << 8));
    float slo = 0.f, shi = 0.f;
    for (int j = 0; j < 16; j++) {
        slo = fmaf(fmaf(d, (float)(p[4 + j] & 15), m), x[j], slo);
        shi = fmaf(fmaf(d, (float)(p[4 + j] >> 4), m), x[16 + j], shi);
    }
    return slo + shi;
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
__device__ float block_dot_generic<QMM_Q5_K>(const uint8_t *p, const float *x) {
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
            const uint8_t b0 = p[48 + 32 * (i >> 1) + e], b1 = p[48 + 32 * (i >> 1) + 16 + e];
            const int h0 = (p[16 + e] >> i) & 1, h1 = (p[32 + e] >> i) & 1;
            const float q0 = (float)(((i & 1) ? (b0 >> 4) : (b0 & 15)) | (h0 << 4));
            const float q1 = (float)(((i & 1) ? (b1 >> 4) : (b1 & 15)) | (h1 << 4));
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
    case QMM_Q4_1:
    case QMM_Q8_0:
    case QMM_Q6_K: return (nb % 2) == 0;
    case QMM_Q4_K:
    case QMM_Q5_K: return true;
    default: return false;
    }
}

// How many wavefronts own row groups (measured on 4096- and 14336-row
// matrices, single and concatenated, and a 128256-row head):
//   * whole-row wavefronts (K <= 4096) and at most 64 row groups per CU: one
//     row group per wavefront -- every group's loads are in flight at once
//     and no wavefront waits for a second group (up to 1.4x faster than a
//     ring for 14336 x 4096 and for concatenated gate + up);
//   * larger matrices: a ring per wavefront, 16 wavefronts per CU for Q4_0
//     and Q8_0, else 8;
//   * a workgroup splitting K: 8 wavefronts per CU (one workgroup per CU
//     for Q4_0 and Q4_K with x quantized in the launch; see launch_fast).
// A measurement build (QMM_TUNING) takes QMM_GEMV_WAVES_PER_CU = n (1..4096)
// to replace all of this with n per CU.
static int gemv_waves_lever() {
    static const int v = [] {
        const int n = tuning_lever("QMM_GEMV_WAVES_PER_CU", 0);
        return (n >= 1 && n <= 4096) ? n : 0;
    }();
    return v;
}
// Row phases of a K-split workgroup (f32, one matrix).  Rows of 2 wavefronts
// (4097 <= K <= 8192) run 2 phases: 4 workgroups of 4 wavefronts per CU, each
// staging x once for both phases (16 wavefronts per CU), instead of 4
// workgroups of 2 wavefronts (8 per CU): 4096 x 8192 Q4_0 8.25 -> 7.0 us,
// Q4_K 9.8 -> 7.4, Q6_K 11.4 -> 9.0, Q8_0 11.8 -> 9.6, 8192 x 8192 Q4_0
// 13.8 -> 10.3, 4096 x 6144 7.5 -> 6.4.  Longer rows measured no better with
// phases.  A measurement build takes QMM_GEMV_PHASES = 1, 2 or 4 (at most 16
// wavefronts per workgroup).
static int gemv_phases(int W) {
    static const int lever = [] {
        const int n = tuning_lever("QMM_GEMV_PHASES", 0);
        return (n == 1 || n == 2 || n == 4) ? n : 0;
    }();
    int ph = lever ? lever : (W == 2 ? 2 : 1);
    while (ph > 1 && W * ph > 16) ph /= 2;
    return ph;
}
static int64_t gemv_wave_owners(int dtype, int64_t nrg, int cus, bool q8_in_launch = false) {
    const int lever = gemv_waves_lever();
    if (lever) return std::min<int64_t>(nrg, (int64_t)cus * lever);
    if (nrg <= (int64_t)cus * 64) return nrg;
    // Q6_K with x quantized in the launch (the 128256-row head): 4 per CU with
    // a ring of 2, 76.5-77.2 us against 78.7-78.9 at 8 per CU with a ring of 4
    // (pre-quantized codes keep 8 per CU and a ring of 4: 81-82 against 86-88)
    if (q8_in_launch && dtype == QMM_Q6_K) return (int64_t)cus * 4;
    return (int64_t)cus * ((dtype == QMM_Q4_0 || dtype == QMM_Q8_0) ? 16 : 8);
}

// Q8_0-quantized activations of ntok tokens (codes [ntok][K], scales
// [ntok][K/32]); unused (q == nullptr) for f32 activations.
struct XQ8 {
    const int8_t *q;
    const float *s;
    int64_t ntok;
};

// Launch one fast-kernel variant: FLAT with D+1 = the most row groups an
// owner gets when that is at most 4, else the ring with D row groups ahead.
template <int DT, int R, int D, bool WAVE_ROWS, int MODE, int NT, int PH = 1>
static void launch_variant(int64_t nmax, dim3 grid, dim3 block, size_t lds, hipStream_t st, const GemvMats &mats,
                           int64_t row_bytes, int U, const float *x, int64_t per_owner, int64_t extra,
                           const XQ8 &xq8) {
#define QMM_GEMV_LAUNCH(F, DD) \
    hipLaunchKernelGGL((gemv_kernel<DT, R, DD, WAVE_ROWS, F, MODE, NT, PH>), grid, block, lds, st, mats, row_bytes, U, x, \
                       per_owner, extra, xq8.q, xq8.s, xq8.ntok)
    // Q4_K: with more than one row group fetched up front the compiler hoists
    // the scale unpacking of all of them and runs out of registers
    constexpr int64_t flat_max = (DT == QMM_Q4_K || DT == QMM_Q5_K) ? 1 : 4;
    switch (nmax <= flat_max ? nmax : 0) {
    case 1: QMM_GEMV_LAUNCH(true, 0); break;
    case 2: if constexpr (flat_max >= 2) QMM_GEMV_LAUNCH(true, 1); break;
    case 3: if constexpr (flat_max >= 3) QMM_GEMV_LAUNCH(true, 2); break;
    case 4: if constexpr (flat_max >= 4) QMM_GEMV_LAUNCH(true, 3); break;
    default: QMM_GEMV_LAUNCH(false, D); break;
    }
#undef QMM_GEMV_LAUNCH
}

// Workgroup candidates the argmax workspace holds (QMM_ARGMAX_WORK_BYTES / 8).
constexpr int64_t ARGMAX_PARTS = 4096;

// The fast kernel over the row groups of `mats` (g_lo filled in by the
// caller); *grid_out receives the workgroup count.
//
// NT >= 1: int8 activations from xq8, NT tokens per weight read, one token
// group per grid row.
template <int DT, int R, int D, int MODE, int NT = 0>
static hipError_t launch_fast(const GemvMats &mats, int64_t K, const float *x, hipStream_t st, int cus,
                              int64_t *grid_out = nullptr, const XQ8 &xq8 = XQ8{nullptr, nullptr, 1}) {
    constexpr int BS = Geo<DT>::BS, BB = Geo<DT>::BB;
    const int64_t row_bytes = (K / BS) * BB;
    const int U = (int)(K / 64);
    const int64_t nrg = mats.g_lo[GEMV_MAX_MATS];
    // the f32 activations; none for pre-quantized codes; codes + scales when
    // the workgroup quantizes
    // whole-row wavefronts (U <= 64) take the padded layout, sized for 64 units
    const size_t lds = NT > 0 ? 0 : (NT < 0 ? (size_t)U * 72 : (U <= 64 ? 64 * xs_unit_bytes(true) : (size_t)U * 256));
    const unsigned gy = NT > 0 ? (unsigned)((xq8.ntok + NT - 1) / NT) : 1u;
    if (U <= 64) {
        const int64_t waves = gemv_wave_owners(DT, nrg, cus, NT < 0);
        constexpr int WPB = gemv_block_threads(DT, true, NT) / 64;  // wavefronts per workgroup
        const int64_t grid = (waves + WPB - 1) / WPB, owners = grid * WPB;
        const int64_t per = nrg / owners, extra = nrg % owners;
        if (MODE == GEMV_ARGMAX && grid > ARGMAX_PARTS) return hipErrorInvalidConfiguration;
        if (grid_out) *grid_out = grid;
        launch_variant<DT, R, D, true, MODE, NT>(per + (extra ? 1 : 0), dim3((unsigned)grid, gy), dim3(64 * WPB), lds, st,
                                                 mats, row_bytes, U, x, per, extra, xq8);
    } else if (U <= 256) {
        const int W = (U + 63) / 64;
        const int lever = gemv_waves_lever();
        // 8 wavefronts per CU; but with x quantized in the launch every
        // workgroup quantizes all of it, and for Q4_0 and Q4_K with 3-4
        // wavefronts per row one workgroup per CU is faster (4096 x 14336:
        // Q4_0 10.3 against 12.3 us, Q4_K 10.8-11.1 against 13.0; 4096 x
        // 12288 Q4_K 10.0 against 11.7; Q8_0 and Q6_K measured no better)
        const bool q8_one = NT < 0 && (DT == QMM_Q4_0 || DT == QMM_Q4_K) && W >= 3;
        // row phases (f32, one matrix): ph groups of W wavefronts share one
        // staging of x
        const int ph = (MODE == GEMV_ONE && NT == 0) ? gemv_phases(W) : 1;
        const int per_cu = lever ? std::max(1, lever / (W * ph))
                                 : (q8_one ? 1 : std::max(1, (ph > 1 ? 16 : 8) / (W * ph)));
        const int64_t grid = std::min<int64_t>((nrg + ph - 1) / ph, (int64_t)cus * per_cu);
        const int64_t owners = grid * ph, per = nrg / owners, extra = nrg % owners;
        if (MODE == GEMV_ARGMAX && grid > ARGMAX_PARTS) return hipErrorInvalidConfiguration;
        if (grid_out) *grid_out = grid;
#define QMM_GEMV_PHASED(P)                                                                                            \
    launch_variant<DT, R, D, false, MODE, NT, P>(per + (extra ? 1 : 0), dim3((unsigned)grid, gy), dim3(64 * W * P), lds, \
                                                 st, mats, row_bytes, U, x, per, extra, xq8)
        if constexpr (MODE == GEMV_ONE && NT == 0) {
            switch (ph) {
            case 2: QMM_GEMV_PHASED(2); break;
#ifdef QMM_TUNING
            case 4: QMM_GEMV_PHASED(4); break;
#endif
            default: QMM_GEMV_PHASED(1); break;
            }
        } else {
            QMM_GEMV_PHASED(1);
        }
#undef QMM_GEMV_PHASED
    } else {
        if constexpr (MODE != GEMV_ONE || NT != 0) return hipErrorNotSupported;
        const int64_t M = mats.M[0];
        const int64_t grid = std::min<int64_t>(nrg, (int64_t)cus * 2);
        hipLaunchKernelGGL((gemv_multi_kernel<DT, R>), dim3((unsigned)grid), dim3(256), 0, st, mats.blob[0], M,
                           row_bytes, U, x, mats.y[0]);
    }
    return hipGetLastError();
}

template <int DT, int R, int D>
static hipError_t launch_one(const uint8_t *blob, int64_t M, int64_t K, const float *x, float *y, hipStream_t st,
                             int cus) {
    GemvMats m{};
    m.blob[0] = blob;
    m.y[0] = y;
    m.M[0] = M;
    for (int j = 1; j <= GEMV_MAX_MATS; j++) m.g_lo[j] = (M + R - 1) / R;
    return launch_fast<DT, R, D, GEMV_ONE>(m, K, x, st, cus);
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

// Several matrices (CONCAT) or a gate/up pair (SWIGLU) in one launch.
template <int DT, int R, int D, int MODE, int NT = 0>
static hipError_t launch_mats(int n, const void *const *blobs, const int64_t *Ms, int64_t K, const float *x,
                              float *const *ys, hipStream_t st, int cus, float2 *part = nullptr,
                              int64_t *grid_out = nullptr) {
    GemvMats m{};
    m.part = part;
    int64_t g = 0;
    for (int i = 0; i < GEMV_MAX_MATS; i++) {
        m.g_lo[i] = g;
        if (i < n) {
            m.blob[i] = static_cast<const uint8_t *>(blobs[i]);
            m.y[i] = ys[i];
            m.M[i] = Ms[i];
            if (MODE == GEMV_CONCAT || i == 0) g += (Ms[i] + R - 1) / R;
        }
    }
    m.g_lo[GEMV_MAX_MATS] = g;
    return launch_fast<DT, R, D, MODE, NT>(m, K, x, st, cus, grid_out);
}

// A measurement build takes QMM_GEMV_PAIR = 0 to run two equal matrices
// through the one-after-the-other concatenation instead.
static bool gemv_pair_lever() {
    static const bool v = tuning_lever("QMM_GEMV_PAIR", 1) != 0;
    return v;
}

bool gemv_fused_ok(int dtype, int64_t K) {
    const int64_t bs = (dtype == QMM_Q4_K || dtype == QMM_Q5_K || dtype == QMM_Q6_K) ? 256 : 32;
    return fast_layout_ok(dtype, K / bs) && (K % 64) == 0 && K / 64 <= 256;
}

hipError_t launch_gemv_concat(int n, const void *const *blobs, const int64_t *Ms, int dtype, int64_t K,
                              const float *x, float *const *ys, hipStream_t st, int cus) {
    if (n < 1 || n > GEMV_MAX_MATS) return hipErrorInvalidValue;
    if (!gemv_fused_ok(dtype, K)) {
        // layouts the fast kernel does not take: one launch per matrix, same bits
        for (int i = 0; i < n; i++) {
            const hipError_t e = launch_gemv(dtype, blobs[i], Ms[i], K, x, ys[i], st, cus);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    if (n == 2 && Ms[0] == Ms[1] && gemv_pair_lever()) {
        // two matrices of one shape (gate + up): their rows side by side
        switch (dtype) {
        case QMM_Q4_0: return launch_mats<QMM_Q4_0, 1, 3, GEMV_PAIR>(2, blobs, Ms, K, x, ys, st, cus);
        case QMM_Q4_1: return launch_mats<QMM_Q4_1, 1, 3, GEMV_PAIR>(2, blobs, Ms, K, x, ys, st, cus);
        case QMM_Q8_0: return launch_mats<QMM_Q8_0, 1, 2, GEMV_PAIR>(2, blobs, Ms, K, x, ys, st, cus);
        case QMM_Q4_K: return launch_mats<QMM_Q4_K, 1, 3, GEMV_PAIR>(2, blobs, Ms, K, x, ys, st, cus);
        case QMM_Q5_K: return launch_mats<QMM_Q5_K, 1, 2, GEMV_PAIR>(2, blobs, Ms, K, x, ys, st, cus);
        case QMM_Q6_K: return launch_mats<QMM_Q6_K, 1, 2, GEMV_PAIR>(2, blobs, Ms, K, x, ys, st, cus);
        default: return hipErrorInvalidValue;
        }
    }
    switch (dtype) {
    case QMM_Q4_0: return launch_mats<QMM_Q4_0, 2, 3, GEMV_CONCAT>(n, blobs, Ms, K, x, ys, st, cus);
    case QMM_Q4_1: return launch_mats<QMM_Q4_1, 2, 3, GEMV_CONCAT>(n, blobs, Ms, K, x, ys, st, cus);
    case QMM_Q8_0: return launch_mats<QMM_Q8_0, 1, 4, GEMV_CONCAT>(n, blobs, Ms, K, x, ys, st, cus);
    case QMM_Q4_K: return launch_mats<QMM_Q4_K, 2, 3, GEMV_CONCAT>(n, blobs, Ms, K, x, ys, st, cus);
    case QMM_Q5_K: return launch_mats<QMM_Q5_K, 1, 3, GEMV_CONCAT>(n, blobs, Ms, K, x, ys, st, cus);
    case QMM_Q6_K: return launch_mats<QMM_Q6_K, 1, 4, GEMV_CONCAT>(n, blobs, Ms, K, x, ys, st, cus);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv_swiglu(int dtype, const void *gate, const void *up, int64_t M, int64_t K, const float *x,
                              float *out, hipStream_t st, int cus) {
    if (!gemv_fused_ok(dtype, K)) return hipErrorInvalidValue;
    const void *blobs[2] = {gate, up};
    const int64_t Ms[2] = {M, M};
    float *ys[2] = {out, out};
    // one row of each matrix per group: the register footprint of two rows
    switch (dtype) {
    case QMM_Q4_0: return launch_mats<QMM_Q4_0, 1, 3, GEMV_SWIGLU>(2, blobs, Ms, K, x, ys, st, cus);
    case QMM_Q4_1: return launch_mats<QMM_Q4_1, 1, 3, GEMV_SWIGLU>(2, blobs, Ms, K, x, ys, st, cus);
    case QMM_Q8_0: return launch_mats<QMM_Q8_0, 1, 2, GEMV_SWIGLU>(2, blobs, Ms, K, x, ys, st, cus);
    case QMM_Q4_K: return launch_mats<QMM_Q4_K, 1, 3, GEMV_SWIGLU>(2, blobs, Ms, K, x, ys, st, cus);
    case QMM_Q5_K: return launch_mats<QMM_Q5_K, 1, 2, GEMV_SWIGLU>(2, blobs, Ms, K, x, ys, st, cus);
    case QMM_Q6_K: return launch_mats<QMM_Q6_K, 1, 2, GEMV_SWIGLU>(2, blobs, Ms, K, x, ys, st, cus);
    default: return hipErrorInvalidValue;
    }
}

// NT = 0: f32 activations; NT = -1: x quantized to Q8_0 inside the launch.
template <int NT>
static hipError_t launch_argmax_nt(int dtype, const void *blob, int64_t M, int64_t K, const float *x, void *work,
                                   int64_t *index, float *value, hipStream_t st, int cus) {
    if (!gemv_fused_ok(dtype, K)) return hipErrorInvalidValue;
    const void *blobs[1] = {blob};
    const int64_t Ms[1] = {M};
    float *ys[1] = {nullptr};
    float2 *part = static_cast<float2 *>(work);
    int64_t grid = 0;
    hipError_t e;
    constexpr int DQ6 = NT < 0 ? 2 : 4;  // the int8 head's ring depth, as qmm_gemv_q8act
    switch (dtype) {
    case QMM_Q4_0: e = launch_mats<QMM_Q4_0, 2, 3, GEMV_ARGMAX, NT>(1, blobs, Ms, K, x, ys, st, cus, part, &grid); break;
    case QMM_Q4_1: e = launch_mats<QMM_Q4_1, 2, 3, GEMV_ARGMAX, NT>(1, blobs, Ms, K, x, ys, st, cus, part, &grid); break;
    case QMM_Q8_0: e = launch_mats<QMM_Q8_0, 1, 4, GEMV_ARGMAX, NT>(1, blobs, Ms, K, x, ys, st, cus, part, &grid); break;
    case QMM_Q4_K: e = launch_mats<QMM_Q4_K, 2, 3, GEMV_ARGMAX, NT>(1, blobs, Ms, K, x, ys, st, cus, part, &grid); break;
    case QMM_Q5_K: e = launch_mats<QMM_Q5_K, 1, 3, GEMV_ARGMAX, NT>(1, blobs, Ms, K, x, ys, st, cus, part, &grid); break;
    case QMM_Q6_K: e = launch_mats<QMM_Q6_K, 1, DQ6, GEMV_ARGMAX, NT>(1, blobs, Ms, K, x, ys, st, cus, part, &grid); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gemv_argmax_finish, dim3(1), dim3(256), 0, st, static_cast<const float2 *>(part), (int)grid,
                       index, value);
    return hipGetLastError();
}

hipError_t launch_gemv_argmax(int dtype, const void *blob, int64_t M, int64_t K, const float *x, void *work,
                              int64_t *index, float *value, hipStream_t st, int cus, bool q8) {
    return q8 ? launch_argmax_nt<-1>(dtype, blob, M, K, x, work, index, value, st, cus)
              : launch_argmax_nt<0>(dtype, blob, M, K, x, work, index, value, st, cus);
}

// Tokens per pass of the several-token kernel and its shape limits.  Rows
// per group (measured): 2 for Q4_0 and Q8_0, 1 for Q4_K and Q6_K (the
// compiler keeps each row's decoded codes across the token loop, so more
// rows cost occupancy).
constexpr int GEMV_TOKENS = 4;

bool gemv_tokens_ok(int dtype, int64_t K) {
    const int64_t bs = (dtype == QMM_Q4_K || dtype == QMM_Q5_K || dtype == QMM_Q6_K) ? 256 : 32;
    return fast_layout_ok(dtype, K / bs) && (K % 64) == 0 && K / 64 <= 64;
}

template <int DT, int R, int D>
static hipError_t launch_tokens(const uint8_t *blob, int64_t M, int64_t K, int ntok, const float *X, float *Y,
                                hipStream_t st, int cus) {
    constexpr int BS = Geo<DT>::BS, BB = Geo<DT>::BB;
    const int64_t row_bytes = (K / BS) * BB;
    const int U = (int)(K / 64);
    const int64_t nrg = (M + R - 1) / R;
    const int64_t waves = std::min<int64_t>(nrg, (int64_t)cus * 8);
    const int64_t grid = (waves + 3) / 4, owners = grid * 4;
    const int64_t per = nrg / owners, extra = nrg % owners;
    const size_t lds = (size_t)U * 256;  // per token
    if (ntok <= 2)
        hipLaunchKernelGGL((gemv_tokens_kernel<DT, R, D, 2>), dim3((unsigned)grid), dim3(256), 2 * lds, st, blob, M,
                           row_bytes, U, X, Y, ntok, per, extra);
    else
        hipLaunchKernelGGL((gemv_tokens_kernel<DT, R, D, GEMV_TOKENS>), dim3((unsigned)grid), dim3(256),
                           GEMV_TOKENS * lds, st, blob, M, row_bytes, U, X, Y, ntok, per, extra);
    return hipGetLastError();
}

hipError_t launch_gemv_tokens(int dtype, const void *blob_v, int64_t M, int64_t K, int64_t N, const float *X,
                              float *Y, hipStream_t st, int cus) {
    if (!gemv_tokens_ok(dtype, K)) return hipErrorInvalidValue;
    const uint8_t *blob = static_cast<const uint8_t *>(blob_v);
    for (int64_t n0 = 0; n0 < N; n0 += GEMV_TOKENS) {
        const int nt = (int)std::min<int64_t>(GEMV_TOKENS, N - n0);
        const float *Xp = X + n0 * K;
        float *Yp = Y + n0 * M;
        hipError_t e;
        switch (dtype) {
        case QMM_Q4_0: e = launch_tokens<QMM_Q4_0, 2, 1>(blob, M, K, nt, Xp, Yp, st, cus); break;
        case QMM_Q4_1: e = launch_tokens<QMM_Q4_1, 2, 1>(blob, M, K, nt, Xp, Yp, st, cus); break;
        case QMM_Q8_0: e = launch_tokens<QMM_Q8_0, 2, 1>(blob, M, K, nt, Xp, Yp, st, cus); break;
        case QMM_Q4_K: e = launch_tokens<QMM_Q4_K, 1, 1>(blob, M, K, nt, Xp, Yp, st, cus); break;
        case QMM_Q5_K: e = launch_tokens<QMM_Q5_K, 1, 1>(blob, M, K, nt, Xp, Yp, st, cus); break;
        case QMM_Q6_K: e = launch_tokens<QMM_Q6_K, 1, 1>(blob, M, K, nt, Xp, Yp, st, cus); break;
        default: return hipErrorInvalidValue;
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_gemv(int dtype, const void *blob_v, int64_t M, int64_t K, const float *x, float *y,
                       hipStream_t st, int cus) {
    const uint8_t *blob = static_cast<const uint8_t *>(blob_v);
    const int64_t bs = (dtype == QMM_Q4_K || dtype == QMM_Q5_K || dtype == QMM_Q6_K) ? 256 : 32;
    const bool fast = fast_layout_ok(dtype, K / bs) && (K % 64) == 0;
    // Long rows split over 3+ wavefronts (K > 8192) on 2048+ rows: one row per
    // group and a short ring (row sums have the same bits for any grouping).
    // 4096 x 14336: Q4_0 12.3 -> 11.6 us, Q4_1 13.6 -> 12.3, Q4_K 14.3 -> 12.2;
    // 4096 x 12288 Q4_0 12.6 -> 11.1 us.  K = 8192 and 1024 rows keep 2 rows.
    const bool long_rows = fast && K / 64 > 128 && M >= 2048;
    switch (dtype) {
    case QMM_Q4_0:
        if (long_rows) return launch_one<QMM_Q4_0, 1, 2>(blob, M, K, x, y, st, cus);
        // whole-row wavefronts on up to 8192 rows: one row per wavefront
        // (4096 x 4096: 4.74 against 4.98 us; 12289 rows and up keep 2)
        if (fast && K / 64 <= 64 && M <= 8192) return launch_one<QMM_Q4_0, 1, 3>(blob, M, K, x, y, st, cus);
        return fast ? launch_one<QMM_Q4_0, 2, 3>(blob, M, K, x, y, st, cus) : launch_generic<QMM_Q4_0>(blob, M, K, x, y, st, cus);
    case QMM_Q4_1:
        if (long_rows) return launch_one<QMM_Q4_1, 1, 1>(blob, M, K, x, y, st, cus);
        return fast ? launch_one<QMM_Q4_1, 2, 3>(blob, M, K, x, y, st, cus) : launch_generic<QMM_Q4_1>(blob, M, K, x, y, st, cus);
    case QMM_Q8_0: return fast ? launch_one<QMM_Q8_0, 1, 4>(blob, M, K, x, y, st, cus) : launch_generic<QMM_Q8_0>(blob, M, K, x, y, st, cus);
    case QMM_Q4_K:
        if (long_rows) return launch_one<QMM_Q4_K, 1, 1>(blob, M, K, x, y, st, cus);
        return fast ? launch_one<QMM_Q4_K, 2, 3>(blob, M, K, x, y, st, cus) : launch_generic<QMM_Q4_K>(blob, M, K, x, y, st, cus);
    case QMM_Q5_K: return fast ? launch_one<QMM_Q5_K, 1, 3>(blob, M, K, x, y, st, cus) : launch_generic<QMM_Q5_K>(blob, M, K, x, y, st, cus);
    case QMM_Q6_K: return fast ? launch_one<QMM_Q6_K, 1, 4>(blob, M, K, x, y, st, cus) : launch_generic<QMM_Q6_K>(blob, M, K, x, y, st, cus);
    default: return hipErrorInvalidValue;
    }
}


// ------------------------------------------------------ read ceiling ----
// A plain streaming read of a buffer (the ceiling a launch that reads the same
// bytes can reach), in the fastest pattern measured for a plain read: every
// workgroup reads whole 32 KB pieces, eight 16-byte non-temporal loads per
// thread in flight (each load instruction of a wavefront 1 KB in a row),
// pieces spread over at most QMM_READ_PROBE_OUT_FLOATS / 4 workgroups.  Each
// wavefront folds what it read into one value (a cross-lane XOR, no LDS and
// no barrier) so that no load is dead.  Loads past the end are bounds-checked
// zeros.
__global__ void __launch_bounds__(256) read_probe_kernel(const uint8_t *__restrict__ buf, int64_t bytes,
                                                         float *__restrict__ out) {
    constexpr int64_t window = (int64_t)1 << 30;  // bytes per buffer resource
    constexpr uint32_t piece = 32768;
    uint32_t acc = 0;
    for (int64_t base = 0; base < bytes; base += window) {
        const int64_t n = bytes - base < window ? bytes - base : window;
        const Rsrc rs = make_rsrc(buf + base, (uint32_t)n);
        const uint32_t pieces = (uint32_t)((n + piece - 1) / piece);
        for (uint32_t p = blockIdx.x; p < pieces; p += gridDim.x) {
            u32x4_t v[8];
#pragma unroll
            for (int u = 0; u < 8; u++)
                v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, p * piece + 4096u * u + 16u * threadIdx.x, 0,
                                                              2 /* non-temporal */);
#pragma unroll
            for (int u = 0; u < 8; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, 64);
    if ((threadIdx.x & 63) == 0) out[4 * blockIdx.x + (threadIdx.x >> 6)] = __uint_as_float(acc);
}

hipError_t launch_read_probe(const void *buf, int64_t bytes, float *out, hipStream_t st, int) {
    const int64_t first = bytes < ((int64_t)1 << 30) ? bytes : ((int64_t)1 << 30);
    int64_t grid = std::min<int64_t>(QMM_READ_PROBE_OUT_FLOATS / 4, (first + 32767) / 32768);
    grid = std::max<int64_t>(grid, 1);
    hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)grid), dim3(256), 0, st,
                       static_cast<const uint8_t *>(buf), bytes, out);
    return hipGetLastError();
}

// ------------------------------------------------ Q8_0 activation path ----
// Quantizer (page "cera 0.5.2 src/backend/cpu.rs", the portable Q8_0
// quantizer): per block of 32 activations, in f32,
//   amax = max |v| (NaN elements never win the comparison),
//   d = amax / 127, id = 1 / d when d != 0 and 1 / d is finite, else 0,
//   code = round-to-nearest-even(v * id), clamped to [-128, 127], NaN -> 0,
//   stored scale = d rounded to f16 (and widened back to f32).
// The codes use the unrounded 1/d and the stored scale the rounded d, as on
// the page.  Eight lanes share a block (one float4 each); the block maximum
// is exchanged with three xor shuffles.  Division and reciprocal are the
// correctly rounded f32 operations, so every code and scale is the unique
// result the definition gives.
__global__ void __launch_bounds__(256) quantize_q8_0_kernel(const floatx4 *__restrict__ X, int64_t nblocks,
                                                            float *__restrict__ scales,
                                                            uint32_t *__restrict__ quants) {
    const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t b = gt >> 3;
    const bool in = b < nblocks;
    const floatx4 v = in ? X[gt] : floatx4{0.f, 0.f, 0.f, 0.f};
    float d;
    const uint32_t packed = q8_quant4(v, &d);
    if (in) {
        quants[gt] = packed;
        if ((gt & 7) == 0) scales[b] = (float)(_Float16)d;
    }
}

hipError_t launch_quantize_q8_0(const float *X, int64_t N, int64_t K, float *scales, int8_t *quants,
                                hipStream_t st) {
    const int64_t nblocks = N * (K / 32);
    // a dispatch counts its work-items in 32 bits: at most 2^29 per launch
    const int64_t max_blocks = (int64_t)1 << 26;
    for (int64_t b0 = 0; b0 < nblocks; b0 += max_blocks) {
        const int64_t nb = std::min<int64_t>(max_blocks, nblocks - b0);
        const int64_t grid = (nb * 8 + 255) / 256;
        hipLaunchKernelGGL(quantize_q8_0_kernel, dim3((unsigned)grid), dim3(256), 0, st,
                           reinterpret_cast<const floatx4 *>(X) + b0 * 8, nb, scales + b0,
                           reinterpret_cast<uint32_t *>(quants) + b0 * 8);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Any layout (one weight block per thread, byte loads): the same integer
// sums per activation block and the same scaling as the fast kernel.
// c = the block's activation codes, s = their scales (one per 32).
template <int DT>
__device__ float block_dot8_generic(const uint8_t *p, const int8_t *c, const float *s);

template <>
__device__ float block_dot8_generic<QMM_Q4_0>(const uint8_t *p, const int8_t *c, const float *s) {
    int acc = 0;
    for (int j = 0; j < 16; j++) acc += ((int)(p[2 + j] & 15) - 8) * c[j] + ((int)(p[2 + j] >> 4) - 8) * c[16 + j];
    return (h2f((uint32_t)p[0] | ((uint32_t)p[1] << 8)) * s[0]) * (float)acc;
}

template <>
__device__ float block_dot8_generic<QMM_Q4_1>(const uint8_t *p, const int8_t *c, const float *s) {
    int acc = 0, cs = 0;
    for (int j = 0; j < 16; j++) {
        acc += (int)(p[4 + j] & 15) * c[j] + (int)(p[4 + j] >> 4) * c[16 + j];
        cs += c[j] + c[16 + j];
    }
    const float d = h2f((uint32_t)p[0] | ((uint32_t)p[1] << 8)), m = h2f((uint32_t)p[2] | ((uint32_t)p[3] << 8));
    return fmaf(d * s[0], (float)acc, (m * s[0]) * (float)cs);
}

template <>
__device__ float block_dot8_generic<QMM_Q8_0>(const uint8_t *p, const int8_t *c, const float *s) {
    int acc = 0;
    for (int j = 0; j < 32; j++) acc += (int)(int8_t)p[2 + j] * c[j];
    return (h2f((uint32_t)p[0] | ((uint32_t)p[1] << 8)) * s[0]) * (float)acc;
}

template <int DT>
__device__ float kquant_dot8_generic(const uint8_t *p, const int8_t *c, const float *s) {
    constexpr int QS = DT == QMM_Q5_K ? 48 : 16;  // offset of the nibbles
    const float d = h2f((uint32_t)p[0] | ((uint32_t)p[1] << 8));
    const float dmin = h2f((uint32_t)p[2] | ((uint32_t)p[3] << 8));
    uint32_t w[3];
    for (int i = 0; i < 3; i++)
        w[i] = (uint32_t)p[4 + 4 * i] | ((uint32_t)p[5 + 4 * i] << 8) | ((uint32_t)p[6 + 4 * i] << 16) |
               ((uint32_t)p[7 + 4 * i] << 24);
    float total = 0.f;
#pragma unroll 1
    for (int i = 0; i < 8; i++) {
        int sc, mn;
        q4k_scale_min(w[0], w[1], w[2], i, sc, mn);
        int acc = 0, cs = 0;
        for (int e = 0; e < 32; e++) {
            const uint8_t b = p[QS + 32 * (i >> 1) + e];
            int q = (i & 1) ? (b >> 4) : (b & 15);
            if (DT == QMM_Q5_K) q |= ((p[16 + e] >> i) & 1) << 4;
            acc += q * c[32 * i + e];
            cs += c[32 * i + e];
        }
        total += fmaf(d * s[i], (float)(sc * acc), -((dmin * s[i]) * (float)(mn * cs)));
    }
    return total;
}
template <>
__device__ float block_dot8_generic<QMM_Q4_K>(const uint8_t *p, const int8_t *c, const float *s) {
    return kquant_dot8_generic<QMM_Q4_K>(p, c, s);
}
template <>
__device__ float block_dot8_generic<QMM_Q5_K>(const uint8_t *p, const int8_t *c, const float *s) {
    return kquant_dot8_generic<QMM_Q5_K>(p, c, s);
}

template <>
__device__ float block_dot8_generic<QMM_Q6_K>(const uint8_t *p, const int8_t *c, const float *s) {
    const float d = h2f((uint32_t)p[208] | ((uint32_t)p[209] << 8));
    float total = 0.f;
    for (int g = 0; g < 16; g++) {  // 16 groups of 16 weights sharing one sub-scale
        int acc = 0;
        for (int i = 0; i < 16; i++) {
            const int j = 16 * g + i, h = j >> 7, q4 = (j & 127) >> 5, l = j & 31;
            const uint8_t lb = p[64 * h + 32 * (q4 & 1) + l];
            const int lo = (q4 < 2) ? (lb & 15) : (lb >> 4);
            const int hi = (p[128 + 32 * h + l] >> (2 * q4)) & 3;
            acc += ((lo | (hi << 4)) - 32) * c[j];
        }
        total = fmaf(d * s[g >> 1], (float)((int)(int8_t)p[192 + g] * acc), total);
    }
    return total;
}

// Y[tok][m] for the tokens of grid row blockIdx.y (one each).
template <int DT, int R>
__global__ void __launch_bounds__(256) gemv_q8_generic_kernel(const uint8_t *__restrict__ blob, int64_t M, int64_t K,
                                                              const int8_t *__restrict__ xq,
                                                              const float *__restrict__ xsc, float *__restrict__ Y) {
    constexpr int BS = Geo<DT>::BS, BB = Geo<DT>::BB;
    __shared__ float red[R][4];
    const int t = threadIdx.x, T = blockDim.x, lane = t & 63, wave = t >> 6, nwaves = T >> 6;
    const int64_t tok = blockIdx.y;
    const int8_t *c = xq + tok * K;
    const float *s = xsc + tok * (K / 32);
    float *y = Y + tok * M;
    const int64_t nb = K / BS, row_bytes = nb * BB, nrg = (M + R - 1) / R;
    for (int64_t rg = blockIdx.x; rg < nrg; rg += gridDim.x) {
        const int64_t row0 = rg * R;
        float acc[R];
        for (int r = 0; r < R; r++) acc[r] = 0.f;
        for (int64_t b = t; b < nb; b += T)
            for (int r = 0; r < R; r++)
                if (row0 + r < M)
                    acc[r] += block_dot8_generic<DT>(blob + (row0 + r) * row_bytes + b * BB, c + b * BS,
                                                     s + b * (BS / 32));
        for (int r = 0; r < R; r++) {
            const float v = wave_sum_to_lane63(acc[r]);
            if (lane == 63) red[r][wave] = v;
        }
        __syncthreads();
        if (t < R && row0 + t < M) {
            float v = 0.f;
            for (int w = 0; w < nwaves; w++) v += red[t][w];
            y[row0 + t] = v;
        }
        __syncthreads();
    }
}

// Tokens per weight read of the int8-activation fast kernel.
constexpr int Q8A_TOKENS = 4;

template <int DT, int R, int D, int NT>
static hipError_t launch_q8a_fast(const uint8_t *blob, int64_t M, int64_t K, int64_t N, const int8_t *xq,
                                  const float *xsc, float *Y, hipStream_t st, int cus) {
    GemvMats m{};
    m.blob[0] = blob;
    m.y[0] = Y;
    m.M[0] = M;
    for (int j = 1; j <= GEMV_MAX_MATS; j++) m.g_lo[j] = (M + R - 1) / R;
    return launch_fast<DT, R, D, GEMV_ONE, NT>(m, K, nullptr, st, cus, nullptr, XQ8{xq, xsc, N});
}

template <int DT, int R1, int D1>
static hipError_t launch_q8a_dt(const uint8_t *blob, int64_t M, int64_t K, int64_t N, const int8_t *xq,
                                const float *xsc, float *Y, hipStream_t st, int cus) {
    if (N == 1) return launch_q8a_fast<DT, R1, D1, 1>(blob, M, K, N, xq, xsc, Y, st, cus);
    return launch_q8a_fast<DT, 1, 1, Q8A_TOKENS>(blob, M, K, N, xq, xsc, Y, st, cus);
}

template <int DT>
static hipError_t launch_q8a_generic(const uint8_t *blob, int64_t M, int64_t K, int64_t N, const int8_t *xq,
                                     const float *xsc, float *Y, hipStream_t st, int cus) {
    constexpr int R = 4;
    const int64_t nrg = (M + R - 1) / R;
    const int64_t grid = nrg < (int64_t)cus * 8 ? nrg : (int64_t)cus * 8;
    hipLaunchKernelGGL((gemv_q8_generic_kernel<DT, R>), dim3((unsigned)grid, (unsigned)N), dim3(256), 0, st, blob, M,
                       K, xq, xsc, Y);
    return hipGetLastError();
}

// One token of f32 activations, quantized inside the launch: MODE GEMV_ONE
// (n = 1), GEMV_CONCAT (n <= 4 matrices of one K) or GEMV_SWIGLU (gate, up).
// Rows per group and ring depth as the f32 GEMV's.  Needs gemv_fused_ok.
hipError_t launch_gemv_q8in(int mode, int n, const void *const *blobs, const int64_t *Ms, int dtype, int64_t K,
                            const float *x, float *const *ys, hipStream_t st, int cus) {
    if (!gemv_fused_ok(dtype, K) || n < 1 || n > GEMV_MAX_MATS) return hipErrorInvalidValue;
#define QMM_Q8IN(DT, R, D, RS, DS)                                                                            \
    switch (mode) {                                                                                         \
    case GEMV_ONE: return launch_mats<DT, R, D, GEMV_ONE, -1>(1, blobs, Ms, K, x, ys, st, cus);            \
    case GEMV_CONCAT:                                                                                       \
        if (pair) return launch_mats<DT, RS, DS, GEMV_PAIR, -1>(2, blobs, Ms, K, x, ys, st, cus);          \
        return launch_mats<DT, R, D, GEMV_CONCAT, -1>(n, blobs, Ms, K, x, ys, st, cus);                    \
    case GEMV_SWIGLU: return launch_mats<DT, RS, DS, GEMV_SWIGLU, -1>(2, blobs, Ms, K, x, ys, st, cus);    \
    default: return hipErrorInvalidValue;                                                                   \
    }
    // two matrices of one shape (gate + up) side by side, as the f32 concat
    const bool pair = mode == GEMV_CONCAT && n == 2 && Ms[0] == Ms[1] && gemv_pair_lever();
    // Q4_1 rows split over 3+ wavefronts on 2048+ rows: one row per group
    // (4096 x 14336: 12.9 -> 10.7 us; Q4_0 and Q4_K, one workgroup per CU,
    // measured best with two)
    if (mode == GEMV_ONE && dtype == QMM_Q4_1 && K / 64 > 128 && Ms[0] >= 2048)
        return launch_mats<QMM_Q4_1, 1, 2, GEMV_ONE, -1>(1, blobs, Ms, K, x, ys, st, cus);
    switch (dtype) {
    case QMM_Q4_0: QMM_Q8IN(QMM_Q4_0, 2, 3, 1, 3)
    case QMM_Q4_1: QMM_Q8IN(QMM_Q4_1, 2, 3, 1, 3)
    case QMM_Q8_0: QMM_Q8IN(QMM_Q8_0, 1, 4, 1, 2)
    case QMM_Q4_K: QMM_Q8IN(QMM_Q4_K, 2, 3, 1, 3)
    case QMM_Q5_K: QMM_Q8IN(QMM_Q5_K, 1, 3, 1, 2)
    case QMM_Q6_K: QMM_Q8IN(QMM_Q6_K, 1, 2, 1, 2)
    default: return hipErrorInvalidValue;
    }
#undef QMM_Q8IN
}

// Whether qmm_gemm_q8act runs on the int8 matrix cores (where gemm_i8_ok
// holds) or in token groups of 4 per weight read (each token then has the bits
// of its single-token call).  Measured at K = 4096 (14336 and 4096 rows): a
// token-group launch costs about max(5.5, 1.2e-3 M) us (Q8_0: 1.45e-3 M), one
// round of matrix-core workgroups (256 rows x 64 tokens, 256 at a time) about
// 110 us (Q4_K), 130 (Q4_0), 160 (Q8_0); both scale with K.  E.g. 14336 x 4096
// Q4_K: N = 16 70 vs 110 us, N = 32 133 vs 111, N = 512 1988 vs 238; 4096 x
// 4096: N = 32 41 vs 109, N = 128 153 vs 109.  Below 32 tokens the token
// groups always run.  A measurement build (QMM_TUNING) takes
// QMM_Q8_MFMA_FROM_N = n to use the matrix cores from n tokens on instead.
bool q8_use_mfma(int dtype, int64_t M, int64_t K, int64_t N) {
    if (!gemm_i8_ok(dtype, M, K, N)) return false;
    static const int lever = tuning_lever("QMM_Q8_MFMA_FROM_N", 0);
    if (lever > 0) return N >= lever;
    if (N < 32) return false;
    const double t_group = std::max(5.5, (dtype == QMM_Q8_0 ? 1.45e-3 : 1.2e-3) * (double)M);
    const double t_old = (double)((N + 3) / 4) * t_group;
    const double t_round = dtype == QMM_Q4_K ? 110.0 : dtype == QMM_Q4_0 ? 130.0 : 160.0;
    const double rounds = (double)((((M + 255) / 256) * ((N + 63) / 64) + 255) / 256);
    return t_old > t_round * rounds;
}

hipError_t launch_gemm_q8act(int dtype, const void *blob_v, int64_t M, int64_t K, int64_t N, const float *xsc,
                             const int8_t *xq, float *Y, hipStream_t st, int cus) {
    const uint8_t *blob = static_cast<const uint8_t *>(blob_v);
    if (q8_use_mfma(dtype, M, K, N)) return launch_gemm_q8act_mfma(dtype, blob_v, M, K, N, xsc, xq, Y, st);
    const bool fast = gemv_fused_ok(dtype, K);
    // the grid's second dimension holds token groups: at most 65535 per launch
    const int64_t chunk = fast ? (N == 1 ? 1 : (int64_t)65535 * Q8A_TOKENS) : 65535;
    for (int64_t n0 = 0; n0 < N; n0 += chunk) {
        const int64_t nt = std::min<int64_t>(chunk, N - n0);
        const int8_t *q = xq + n0 * K;
        const float *s = xsc + n0 * (K / 32);
        float *y = Y + n0 * M;
        hipError_t e;
        switch (dtype) {
        case QMM_Q4_0: e = fast ? launch_q8a_dt<QMM_Q4_0, 2, 3>(blob, M, K, nt, q, s, y, st, cus) : launch_q8a_generic<QMM_Q4_0>(blob, M, K, nt, q, s, y, st, cus); break;
        case QMM_Q4_1: e = fast ? launch_q8a_dt<QMM_Q4_1, 2, 3>(blob, M, K, nt, q, s, y, st, cus) : launch_q8a_generic<QMM_Q4_1>(blob, M, K, nt, q, s, y, st, cus); break;
        case QMM_Q8_0: e = fast ? launch_q8a_dt<QMM_Q8_0, 1, 4>(blob, M, K, nt, q, s, y, st, cus) : launch_q8a_generic<QMM_Q8_0>(blob, M, K, nt, q, s, y, st, cus); break;
        case QMM_Q4_K: e = fast ? launch_q8a_dt<QMM_Q4_K, 2, 3>(blob, M, K, nt, q, s, y, st, cus) : launch_q8a_generic<QMM_Q4_K>(blob, M, K, nt, q, s, y, st, cus); break;
        case QMM_Q5_K: e = fast ? launch_q8a_dt<QMM_Q5_K, 1, 3>(blob, M, K, nt, q, s, y, st, cus) : launch_q8a_generic<QMM_Q5_K>(blob, M, K, nt, q, s, y, st, cus); break;
        case QMM_Q6_K: e = fast ? launch_q8a_dt<QMM_Q6_K, 1, 4>(blob, M, K, nt, q, s, y, st, cus) : launch_q8a_generic<QMM_Q6_K>(blob, M, K, nt, q, s, y, st, cus); break;
        default: return hipErrorInvalidValue;
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace qmm
