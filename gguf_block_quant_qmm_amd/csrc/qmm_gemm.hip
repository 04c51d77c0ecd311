// qmm_gemm.hip -- prefill / verify GEMM on the matrix cores,
//     Y[n][m] = sum_k W[m][k] X[n][k]   (X f32 [N][K], Y f32 [N][M]).
//
// The weights are decoded once per 64-deep k-tile into an f16 tile in LDS and
// that tile is reused for every token column of the workgroup (page "cera
// 0.3.1 src/model/gpu_lfm2.rs", build_mul_mat_pipeline: decode to shared
// memory once per k-tile, reuse across all token columns -- the reuse is what
// beats kernels that re-decode per token).  What is MI355X-specific:
//   * the contraction runs on v_mfma_f32_32x32x16_f16 (f16 operands, f32
//     accumulation) with the activations as the A operand (32 tokens) and the
//     decoded weights as the B operand (32 rows), so a wavefront's result
//     lanes hold 32 consecutive output rows of one token: the stores of
//     Y[n][m] are 128-byte coalesced;
//   * each k-tile's f32 activations are converted to f16 on the way into LDS
//     (no separate conversion pass and no workspace);
//   * the next k-tile's raw weight bytes and activations are fetched into
//     registers while the matrix cores work on the current one;
//   * LDS rows are padded by 16 bytes so the 16-byte operand reads of 8
//     consecutive lanes hit distinct banks.
// Each weight is rounded once to f16 from its exact value (Q4_K: from the
// f32 fma(d*sc, q, -dmin*m)); activations are rounded to nearest f16.
#include <cstdlib>

#include "qmm_device.hpp"
#include "qmm_internal.hpp"

namespace qmm {

constexpr int BK = 64;        // k-tile depth (weights)
constexpr int LDK = BK + 8;   // LDS row stride in halves (16-byte pad)

// ------------------------------------------------------ weight k-tiles ----
// One "item" is half of a row's 64-weight k-tile (part 0 or 1); load() pulls
// its raw bytes into registers, store() decodes them to 32 f16 weights in the
// LDS row.  GEN selects byte loads (any alignment) over dword loads.

template <int DT, bool GEN> struct WTile;

template <bool GEN> struct WTile<QMM_Q4_0, GEN> {
    // part = block 2*(k0/64) + part; 18 bytes: d, 16 nibble bytes
    static constexpr int NDW = 5;
    __device__ static bool exists(int64_t K, int64_t k0, int part) { return k0 + 32 * part < K; }
    __device__ static void load(const uint8_t *row, int64_t k0, int part, uint32_t (&v)[NDW]) {
        const uint8_t *p = row + 18 * (k0 / 32 + part);
        uint32_t w[5];
        uint32_t sh = 0;
        if (GEN) {
            fetch_bytes(p, 18, w);
        } else {
            sh = (uint32_t)((uintptr_t)p & 3u);
            fetch_al(reinterpret_cast<const uint8_t *>(dword_at(p)), w);
        }
        v[0] = w[0] >> (8 * sh);
#pragma unroll
        for (int i = 0; i < 4; i++) v[1 + i] = sh ? w[i + 1] : __builtin_amdgcn_alignbyte(w[i + 1], w[i], 2);
    }
    __device__ static void store(const uint32_t (&v)[NDW], int part, _Float16 *wrow) {
        const float d = h2f(v[0]);
        half8 lo[2], hi[2];
#pragma unroll
        for (int i = 0; i < 4; i++) {
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const int e = 4 * i + c;
                lo[e >> 3][e & 7] = (_Float16)(d * (float)((int)((v[1 + i] >> (8 * c)) & 15u) - 8));
                hi[e >> 3][e & 7] = (_Float16)(d * (float)((int)((v[1 + i] >> (8 * c + 4)) & 15u) - 8));
            }
        }
        half8 *dst = reinterpret_cast<half8 *>(wrow + 32 * part);
        dst[0] = lo[0]; dst[1] = lo[1]; dst[2] = hi[0]; dst[3] = hi[1];
    }
};

template <bool GEN> struct WTile<QMM_Q8_0, GEN> {
    // part = block 2*(k0/64) + part; 34 bytes: d, 32 int8
    static constexpr int NDW = 9;
    __device__ static bool exists(int64_t K, int64_t k0, int part) { return k0 + 32 * part < K; }
    __device__ static void load(const uint8_t *row, int64_t k0, int part, uint32_t (&v)[NDW]) {
        const uint8_t *p = row + 34 * (k0 / 32 + part);
        uint32_t w[9];
        uint32_t sh = 0;
        if (GEN) {
            fetch_bytes(p, 34, w);
        } else {
            sh = (uint32_t)((uintptr_t)p & 3u);
            fetch_al(reinterpret_cast<const uint8_t *>(dword_at(p)), w);
        }
        v[0] = w[0] >> (8 * sh);
#pragma unroll
        for (int i = 0; i < 8; i++) v[1 + i] = sh ? w[i + 1] : __builtin_amdgcn_alignbyte(w[i + 1], w[i], 2);
    }
    __device__ static void store(const uint32_t (&v)[NDW], int part, _Float16 *wrow) {
        const float d = h2f(v[0]);
        half8 o[4];
#pragma unroll
        for (int i = 0; i < 8; i++) {
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const int e = 4 * i + c;
                o[e >> 3][e & 7] = (_Float16)(d * (float)(int8_t)(uint8_t)((v[1 + i] >> (8 * c)) & 0xFFu));
            }
        }
        half8 *dst = reinterpret_cast<half8 *>(wrow + 32 * part);
#pragma unroll
        for (int i = 0; i < 4; i++) dst[i] = o[i];
    }
};

template <bool GEN> struct WTile<QMM_Q4_K, GEN> {
    // k-tile = chunk c = (k0%256)/64 of super-block k0/256 (sub-blocks 2c, 2c+1);
    // part = which 16 of the chunk's 32 nibble bytes.  Super-blocks are
    // 16-byte aligned whenever the blob is (144 = 9*16).
    static constexpr int NDW = 8;  // 4 header dwords + 4 nibble dwords
    __device__ static bool exists(int64_t, int64_t, int) { return true; }
    __device__ static void load(const uint8_t *row, int64_t k0, int part, uint32_t (&v)[NDW]) {
        const uint8_t *sb = row + 144 * (k0 / 256);
        const int c = (int)((k0 % 256) / 64);
        uint32_t h[4], q[4];
        if (GEN) {
            fetch_bytes(sb, 16, h);
            fetch_bytes(sb + 16 + 32 * c + 16 * part, 16, q);
        } else {
            fetch_al(sb, h);
            fetch_al(sb + 16 + 32 * c + 16 * part, q);
        }
#pragma unroll
        for (int i = 0; i < 4; i++) { v[i] = h[i]; v[4 + i] = q[i]; }
    }
    __device__ static void store(const uint32_t (&v)[NDW], int part, _Float16 *wrow, int c) {
        const float d = h2f(v[0]), dmin = h2f(v[0] >> 16);
#pragma unroll
        for (int half = 0; half < 2; half++) {
            int sc, mn;
            q4k_scale_min(v[1], v[2], v[3], 2 * c + half, sc, mn);
            const float dsc = d * (float)sc, ndm = -(dmin * (float)mn);
            half8 o[2];
#pragma unroll
            for (int i = 0; i < 4; i++) {
#pragma unroll
                for (int b = 0; b < 4; b++) {
                    const int e = 4 * i + b;
                    const float q = (float)((v[4 + i] >> (8 * b + 4 * half)) & 15u);
                    o[e >> 3][e & 7] = (_Float16)fmaf(dsc, q, ndm);
                }
            }
            half8 *dst = reinterpret_cast<half8 *>(wrow + 32 * half + 16 * part);
            dst[0] = o[0]; dst[1] = o[1];
        }
    }
};

template <bool GEN> struct WTile<QMM_Q6_K, GEN> {
    // k-tile = quarter qq = (k0%256)/64 of the super-block: h = qq/2,
    // groups g = 2(qq&1) + part, elements l = 0..31 of each group.
    static constexpr int NDW = 8 + 8 + 1;  // ql slice, qh slice, (sc | d<<16)
    __device__ static bool exists(int64_t, int64_t, int) { return true; }
    __device__ static void load(const uint8_t *row, int64_t k0, int part, uint32_t (&v)[NDW]) {
        const uint8_t *p = row + 210 * (k0 / 256);
        const int qq = (int)((k0 % 256) / 64), h = qq >> 1, g = 2 * (qq & 1) + part;
        uint32_t a[8], c[8];
        uint32_t scd;
        if (GEN) {
            fetch_bytes(p + 64 * h + 32 * (g & 1), 32, a);
            fetch_bytes(p + 128 + 32 * h, 32, c);
            const uint8_t *ps = p + 192 + 8 * h + 2 * g;
            scd = (uint32_t)ps[0] | ((uint32_t)ps[1] << 8) | ((uint32_t)p[208] << 16) | ((uint32_t)p[209] << 24);
        } else {
            fetch_un(p + 64 * h + 32 * (g & 1), a);
            fetch_un(p + 128 + 32 * h, c);
            const uint8_t *ps = p + 192 + 8 * h + 2 * g;
            const uint32_t sw = *dword_at(ps);
            const uint8_t *pd = p + 208;
            const uint32_t dw = *dword_at(pd);
            scd = ((sw >> (8 * ((uintptr_t)ps & 3))) & 0xFFFFu) | ((dw >> (8 * ((uintptr_t)pd & 3))) << 16);
        }
#pragma unroll
        for (int i = 0; i < 8; i++) { v[i] = a[i]; v[8 + i] = c[i]; }
        v[16] = scd;
    }
    __device__ static void store(const uint32_t (&v)[NDW], int part, _Float16 *wrow, int qq) {
        const int g = 2 * (qq & 1) + part;
        const float d = h2f(v[16] >> 16);
        const float dsc0 = d * (float)(int8_t)(uint8_t)(v[16] & 0xFFu);         // l < 16
        const float dsc1 = d * (float)(int8_t)(uint8_t)((v[16] >> 8) & 0xFFu);  // l >= 16
        half8 o[4];
#pragma unroll
        for (int i = 0; i < 8; i++) {
#pragma unroll
            for (int b = 0; b < 4; b++) {
                const int l = 4 * i + b;
                const uint32_t lo = (v[i] >> (8 * b + (g >= 2 ? 4 : 0))) & 15u;
                const uint32_t hi = (v[8 + i] >> (8 * b + 2 * g)) & 3u;
                const float q = (float)((int)(lo | (hi << 4)) - 32);
                o[l >> 3][l & 7] = (_Float16)((l < 16 ? dsc0 : dsc1) * q);
            }
        }
        half8 *dst = reinterpret_cast<half8 *>(wrow + 32 * part);
#pragma unroll
        for (int i = 0; i < 4; i++) dst[i] = o[i];
    }
};

template <int DT, bool GEN>
__device__ __forceinline__ void wtile_store(const uint32_t (&v)[WTile<DT, GEN>::NDW], int part, _Float16 *wrow,
                                            int64_t k0) {
    if constexpr (DT == QMM_Q4_K || DT == QMM_Q6_K)
        WTile<DT, GEN>::store(v, part, wrow, (int)((k0 % 256) / 64));
    else
        WTile<DT, GEN>::store(v, part, wrow);
}

// ------------------------------------------------------------- kernel ----
// Workgroup tile: BN tokens x BM weight rows, 4 wavefronts arranged WN x WM,
// each owning (BN/WN) x (BM/WM) outputs as 32x32 MFMA blocks.
template <int DT, int BM, int BN, int WN, int WM, bool GEN>
__global__ void __launch_bounds__(256) gemm_kernel(const uint8_t *__restrict__ blob, int64_t M, int64_t K, int64_t N,
                                                   int64_t row_bytes, const float *__restrict__ X,
                                                   float *__restrict__ Y, int n_ntiles) {
    static_assert(WN * WM == 4, "4 wavefronts");
    constexpr int TN = BN / WN, TM = BM / WM, FN = TN / 32, FM = TM / 32;
    static_assert(FN >= 1 && FM >= 1 && TN % 32 == 0 && TM % 32 == 0, "tile shape");
    constexpr int NXF = BN * (BK / 4) / 256;       // float4 of X per thread per k-tile
    static_assert(NXF >= 1, "BN too small");
    constexpr int NWI = (BM * 2 + 255) / 256;      // weight items per thread per k-tile
    using WT = WTile<DT, GEN>;

    __shared__ __attribute__((aligned(16))) _Float16 Xs[BN * LDK];
    __shared__ __attribute__((aligned(16))) _Float16 Ws[BM * LDK];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wn = wave / WM, wm = wave % WM;
    const int64_t mt = blockIdx.x / n_ntiles, nt = blockIdx.x % n_ntiles;
    const int64_t m0 = mt * BM, n0 = nt * BN;
    const int64_t nkt = (K + BK - 1) / BK;

    floatx4 xr[NXF];
    uint32_t wr[NWI][WT::NDW];

    auto gload = [&](int64_t kt) {
        const int64_t k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < NXF; i++) {
            const int f = t + 256 * i, r = f >> 4, c4 = f & 15;
            const int64_t n = n0 + r, k = k0 + 4 * c4;
            if (n < N && k < K)
                xr[i] = *reinterpret_cast<const floatx4 *>(X + n * K + k);
            else
                xr[i] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int i = 0; i < NWI; i++) {
            const int w = t + 256 * i, r = w >> 1, part = w & 1;
            const int64_t m = m0 + r;
            if (w < BM * 2 && m < M && WT::exists(K, k0, part)) {
                WT::load(blob + m * row_bytes, k0, part, wr[i]);
            } else {
#pragma unroll
                for (int j = 0; j < WT::NDW; j++) wr[i][j] = 0u;
            }
        }
    };
    auto sstore = [&](int64_t kt) {
        const int64_t k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < NXF; i++) {
            const int f = t + 256 * i, r = f >> 4, c4 = f & 15;
            half4 hv = {(_Float16)xr[i].x, (_Float16)xr[i].y, (_Float16)xr[i].z, (_Float16)xr[i].w};
            *reinterpret_cast<half4 *>(Xs + r * LDK + 4 * c4) = hv;
        }
#pragma unroll
        for (int i = 0; i < NWI; i++) {
            const int w = t + 256 * i, r = w >> 1, part = w & 1;
            if (w < BM * 2) wtile_store<DT, GEN>(wr[i], part, Ws + r * LDK, k0);
        }
    };

    floatx16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; i++)
#pragma unroll
        for (int j = 0; j < FM; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

    gload(0);
    for (int64_t kt = 0; kt < nkt; kt++) {
        if (kt) __syncthreads();
        sstore(kt);
        __syncthreads();
        if (kt + 1 < nkt) gload(kt + 1);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ks++) {
            half8 a[FN], b[FM];
            const int kk = ks * 16 + 8 * (lane >> 5);
#pragma unroll
            for (int i = 0; i < FN; i++)
                a[i] = *reinterpret_cast<const half8 *>(Xs + (wn * TN + 32 * i + (lane & 31)) * LDK + kk);
#pragma unroll
            for (int j = 0; j < FM; j++)
                b[j] = *reinterpret_cast<const half8 *>(Ws + (wm * TM + 32 * j + (lane & 31)) * LDK + kk);
#pragma unroll
            for (int i = 0; i < FN; i++)
#pragma unroll
                for (int j = 0; j < FM; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }

    // D[n][m]: lane holds column m = lane%32, rows 8*(v/4) + 4*(lane/32) + v%4.
#pragma unroll
    for (int i = 0; i < FN; i++) {
#pragma unroll
        for (int j = 0; j < FM; j++) {
            const int64_t m = m0 + wm * TM + 32 * j + (lane & 31);
            if (m >= M) continue;
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int64_t n = n0 + wn * TN + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (n < N) Y[n * M + m] = acc[i][j][v];
            }
        }
    }
}

// ================================================= register-B GEMM ====
// Each wavefront owns TM weight rows and decodes their k-tiles straight into
// the B operand registers of v_mfma_f32_32x32x16_f16 (lane l: row l%32 of a
// 32-row block, 8 consecutive k at 8*(l/32) of every 16-deep step), so a
// weight is decoded exactly once per token tile and never passes through
// LDS.  The f32 activations of a k-tile are converted once per workgroup
// into a double-buffered f16 LDS tile that the 4 wavefronts share as the A
// operand.  Raw weight bytes are prefetched WD k-tiles ahead, activations 2.
//
// Exact decode to f16: a code c (< 1024) placed in a 16-bit lane is the f16
// subnormal c * 2^-24, so v_fma_mix_f32(c, scale * 2^24, bias) computes
// scale * c + bias exactly and rounds once to f32 (then once to f16).

__device__ __forceinline__ float sub_code(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits16 & 0xFFFFu));
}

// 8 weights from two dwords of byte codes (bytes 0..3 of q0, then of q1):
// w_j = scale * code_j + bias, rounded to f16.
__device__ __forceinline__ half8 dec8(uint32_t q0, uint32_t q1, float scale24, float bias) {
    const uint32_t a = q0 & 0x00FF00FFu, b = (q0 >> 8) & 0x00FF00FFu;
    const uint32_t c = q1 & 0x00FF00FFu, d = (q1 >> 8) & 0x00FF00FFu;
    half8 w;
    w[0] = (_Float16)fmaf(sub_code(a), scale24, bias);
    w[1] = (_Float16)fmaf(sub_code(b), scale24, bias);
    w[2] = (_Float16)fmaf(sub_code(a >> 16), scale24, bias);
    w[3] = (_Float16)fmaf(sub_code(b >> 16), scale24, bias);
    w[4] = (_Float16)fmaf(sub_code(c), scale24, bias);
    w[5] = (_Float16)fmaf(sub_code(d), scale24, bias);
    w[6] = (_Float16)fmaf(sub_code(c >> 16), scale24, bias);
    w[7] = (_Float16)fmaf(sub_code(d >> 16), scale24, bias);
    return w;
}

constexpr float TWO24 = 16777216.0f;

// BDec<DT>: raw bytes of one row's 64-deep k-tile that lane half kh needs
// (its k = 16s + 8kh + j, s < 4, j < 8), and their decode to 4 half8.
template <int DT> struct BDec;

template <> struct BDec<QMM_Q4_0> {
    // blocks b0 = k0/32 (k < 32) and b0+1: a 36-byte dword-aligned pair
    static constexpr int NW = 9;
    __device__ static void load(const uint8_t *row, int64_t k0, int, uint32_t (&r)[NW]) {
        const uint32_t *p = reinterpret_cast<const uint32_t *>(row + 18 * (k0 / 32));
#pragma unroll
        for (int i = 0; i < NW; i++) r[i] = p[i];
    }
    __device__ static void decode(const uint32_t (&r)[NW], int kh, int64_t, half8 (&f)[4]) {
        // block 0: qs at bytes 2..17; block 1: d at bytes 18..19, qs at 20..35
        const float d0 = h2f(r[0]), d1 = h2f(r[4] >> 16);
        const uint32_t a0 = __builtin_amdgcn_alignbyte(r[1], r[0], 2), a1 = __builtin_amdgcn_alignbyte(r[2], r[1], 2);
        const uint32_t a2 = __builtin_amdgcn_alignbyte(r[3], r[2], 2), a3 = __builtin_amdgcn_alignbyte(r[4], r[3], 2);
        const uint32_t p0 = kh ? a2 : a0, p1 = kh ? a3 : a1;             // qs[8kh .. 8kh+8) of block 0
        const uint32_t q0 = kh ? r[7] : r[5], q1 = kh ? r[8] : r[6];      // of block 1
        // element e < 16: low nibble of qs[e]; e >= 16: high nibble of qs[e-16]
        f[0] = dec8(p0 & 0x0F0F0F0Fu, p1 & 0x0F0F0F0Fu, d0 * TWO24, -8.f * d0);
        f[1] = dec8((p0 >> 4) & 0x0F0F0F0Fu, (p1 >> 4) & 0x0F0F0F0Fu, d0 * TWO24, -8.f * d0);
        f[2] = dec8(q0 & 0x0F0F0F0Fu, q1 & 0x0F0F0F0Fu, d1 * TWO24, -8.f * d1);
        f[3] = dec8((q0 >> 4) & 0x0F0F0F0Fu, (q1 >> 4) & 0x0F0F0F0Fu, d1 * TWO24, -8.f * d1);
    }
};

template <> struct BDec<QMM_Q8_0> {
    // blocks b0 = k0/32 and b0+1: a 68-byte dword-aligned pair
    static constexpr int NW = 17;
    __device__ static void load(const uint8_t *row, int64_t k0, int, uint32_t (&r)[NW]) {
        const uint32_t *p = reinterpret_cast<const uint32_t *>(row + 34 * (k0 / 32));
#pragma unroll
        for (int i = 0; i < NW; i++) r[i] = p[i];
    }
    __device__ static void decode(const uint32_t (&r)[NW], int kh, int64_t, half8 (&f)[4]) {
        const float d0 = h2f(r[0]), d1 = h2f(r[8] >> 16);
        // block 0: q at bytes 2..33 -> realigned dwords; block 1: q at bytes 36..67 = r[9..16]
        uint32_t b0[8];
#pragma unroll
        for (int i = 0; i < 8; i++) b0[i] = __builtin_amdgcn_alignbyte(r[i + 1], r[i], 2);
        const int o = 2 * kh;  // dword offset of q[8kh] within a 32-byte run
        const uint32_t flip = 0x80808080u;  // q + 128 as an unsigned code
        f[0] = dec8((kh ? b0[2] : b0[0]) ^ flip, (kh ? b0[3] : b0[1]) ^ flip, d0 * TWO24, -128.f * d0);
        f[1] = dec8((kh ? b0[6] : b0[4]) ^ flip, (kh ? b0[7] : b0[5]) ^ flip, d0 * TWO24, -128.f * d0);
        f[2] = dec8((kh ? r[11] : r[9]) ^ flip, (kh ? r[12] : r[10]) ^ flip, d1 * TWO24, -128.f * d1);
        f[3] = dec8((kh ? r[15] : r[13]) ^ flip, (kh ? r[16] : r[14]) ^ flip, d1 * TWO24, -128.f * d1);
        (void)o;
    }
};

template <> struct BDec<QMM_Q4_K> {
    // header (d, dmin, 12 scale bytes) + qs[32c + 8kh ..+8) + qs[32c + 16 + 8kh ..+8)
    static constexpr int NW = 8;
    __device__ static void load(const uint8_t *row, int64_t k0, int kh, uint32_t (&r)[NW]) {
        const uint8_t *sb = row + 144 * (k0 / 256);
        const int c = (int)((k0 % 256) / 64);
        const uint32_t *h = reinterpret_cast<const uint32_t *>(sb);
        const uint32_t *q = reinterpret_cast<const uint32_t *>(sb + 16 + 32 * c + 8 * kh);
        r[0] = h[0]; r[1] = h[1]; r[2] = h[2]; r[3] = h[3];
        r[4] = q[0]; r[5] = q[1]; r[6] = q[4]; r[7] = q[5];
    }
    __device__ static void decode(const uint32_t (&r)[NW], int, int64_t k0, half8 (&f)[4]) {
        const int c = (int)((k0 % 256) / 64);
        const float d = h2f(r[0]), dmin = h2f(r[0] >> 16);
        int sc0, m0, sc1, m1;
        q4k_scale_min(r[1], r[2], r[3], 2 * c, sc0, m0);
        q4k_scale_min(r[1], r[2], r[3], 2 * c + 1, sc1, m1);
        const float s0 = d * (float)sc0 * TWO24, b0 = -(dmin * (float)m0);
        const float s1 = d * (float)sc1 * TWO24, b1 = -(dmin * (float)m1);
        // sub-block 2c = low nibbles (k < 32), 2c+1 = high nibbles
        f[0] = dec8(r[4] & 0x0F0F0F0Fu, r[5] & 0x0F0F0F0Fu, s0, b0);
        f[1] = dec8(r[6] & 0x0F0F0F0Fu, r[7] & 0x0F0F0F0Fu, s0, b0);
        f[2] = dec8((r[4] >> 4) & 0x0F0F0F0Fu, (r[5] >> 4) & 0x0F0F0F0Fu, s1, b1);
        f[3] = dec8((r[6] >> 4) & 0x0F0F0F0Fu, (r[7] >> 4) & 0x0F0F0F0Fu, s1, b1);
    }
};

template <> struct BDec<QMM_Q6_K> {
    // quarter qq of the super-block: h = qq/2, groups g0 = 2(qq&1) and g0+1.
    // Windows aligned down to the dword (odd super-blocks start 2 bytes into
    // one): ql[64h + 16s' + 8kh ..+8) for s' = 0..3 (3 dwords each),
    // qh[32h + 16s'' + 8kh ..+8) for s'' = 0,1 (3 dwords each), the 4 sub-scales
    // sc[8h + 2g0 ..+4) (2 dwords) and the dword holding d.
    static constexpr int NW = 4 * 3 + 2 * 3 + 2 + 1;
    __device__ static void load(const uint8_t *row, int64_t k0, int kh, uint32_t (&r)[NW]) {
        const int64_t sb = k0 / 256;
        const int qq = (int)((k0 % 256) / 64), h = qq >> 1, g0 = 2 * (qq & 1);
        const uint32_t sh = (uint32_t)(2 * (sb & 1));
        const uint8_t *base = row + 210 * sb - sh;  // dword aligned
        auto ld3 = [&](int off, int at) {
            const uint32_t *p = reinterpret_cast<const uint32_t *>(base + off);
            r[at] = p[0]; r[at + 1] = p[1]; r[at + 2] = p[2];
        };
#pragma unroll
        for (int s = 0; s < 4; s++) ld3(64 * h + 16 * s + 8 * kh, 3 * s);
        ld3(128 + 32 * h + 8 * kh, 12);
        ld3(128 + 32 * h + 16 + 8 * kh, 15);
        const uint32_t *ps = reinterpret_cast<const uint32_t *>(base + 192 + 8 * h + 2 * g0 - (2 * g0 & 3));
        r[18] = ps[0]; r[19] = ps[1];
        r[20] = *reinterpret_cast<const uint32_t *>(base + 208);
        (void)g0;
    }
    __device__ static void decode(const uint32_t (&r)[NW], int, int64_t k0, half8 (&f)[4]) {
        const int64_t sb = k0 / 256;
        const int qq = (int)((k0 % 256) / 64), g0 = 2 * (qq & 1);
        const uint32_t sh = (uint32_t)(2 * (sb & 1));
        const float d = h2f(r[20] >> (8 * sh));
        // the 4 sub-scales sc[8h + 2g0 + i], i = 0..3, start (sh + (2g0 & 3)) bytes into r[18]
        const uint32_t scw = __builtin_amdgcn_alignbyte(r[19], r[18], sh + (uint32_t)(2 * g0 & 3));
        uint32_t qh[2][2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
            qh[i][0] = __builtin_amdgcn_alignbyte(r[12 + 3 * i + 1], r[12 + 3 * i], sh);
            qh[i][1] = __builtin_amdgcn_alignbyte(r[12 + 3 * i + 2], r[12 + 3 * i + 1], sh);
        }
#pragma unroll
        for (int s = 0; s < 4; s++) {
            // s = 0,1: group g0, l = 16s + 8kh + j (ql pieces 0,1); s = 2,3: group g0+1 (pieces 2,3)
            const int gi = s >> 1, li = s & 1;
            const int g = g0 + gi;
            const uint32_t l0 = __builtin_amdgcn_alignbyte(r[3 * (2 * gi + li) + 1], r[3 * (2 * gi + li)], sh);
            const uint32_t l1 = __builtin_amdgcn_alignbyte(r[3 * (2 * gi + li) + 2], r[3 * (2 * gi + li) + 1], sh);
            const uint32_t lo0 = (g >= 2 ? (l0 >> 4) : l0) & 0x0F0F0F0Fu, lo1 = (g >= 2 ? (l1 >> 4) : l1) & 0x0F0F0F0Fu;
            const uint32_t hi0 = ((qh[li][0] >> (2 * g)) & 0x03030303u) << 4;
            const uint32_t hi1 = ((qh[li][1] >> (2 * g)) & 0x03030303u) << 4;
            const float dsc = d * (float)(int)__builtin_amdgcn_sbfe((int)scw, 8 * (2 * gi + li), 8);  // the builtin returns unsigned
            f[s] = dec8(lo0 | hi0, lo1 | hi1, dsc * TWO24, -32.f * dsc);
        }
    }
};

// Workgroup: W wavefronts x TM weight rows, BN tokens; k-tiles of 64.  The
// decode of k-tile kt+1 is issued in four slices between the four 16-deep
// MFMA steps of k-tile kt, so the matrix cores and the vector ALUs overlap.
template <int DT, int TM, int BN, int WD, int W>
__global__ void __launch_bounds__(64 * W) gemm_wreg_kernel(const uint8_t *__restrict__ blob, int64_t M, int64_t K,
                                                          int64_t N, int64_t row_bytes, const float *__restrict__ X,
                                                          float *__restrict__ Y, int n_ntiles) {
    constexpr int FM = TM / 32, FN = BN / 32;
    constexpr int NT = 64 * W;
    constexpr int NXF = BN * (BK / 4) / NT;  // float4 of X per thread per k-tile
    static_assert(NXF >= 1 && BN * (BK / 4) % NT == 0, "activation tile split");
    constexpr int XD = 2;                     // activation k-tiles in flight
    using BD = BDec<DT>;
    __shared__ __attribute__((aligned(16))) _Float16 Xs[2][BN * LDK];

    const int t = threadIdx.x, lane = t & 63, kh = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int64_t mt = blockIdx.x / n_ntiles, nt = blockIdx.x % n_ntiles;
    const int64_t n0 = nt * BN, mw = mt * (W * TM) + wave * TM;
    const int64_t nkt = K / BK;

    uint32_t wr[WD][FM][BD::NW];
    floatx4 xr[XD][NXF];
    half8 bf[2][FM][4];

    auto wload = [&](int64_t kt, uint32_t (&w)[FM][BD::NW]) {
#pragma unroll
        for (int j = 0; j < FM; j++) {
            const int64_t m = mw + 32 * j + (lane & 31);
            if (m < M) {
                BD::load(blob + m * row_bytes, kt * BK, kh, w[j]);
            } else {
#pragma unroll
                for (int i = 0; i < BD::NW; i++) w[j][i] = 0u;
            }
        }
    };
    auto xload = [&](int64_t kt, floatx4 (&x)[NXF]) {
#pragma unroll
        for (int i = 0; i < NXF; i++) {
            const int f = t + NT * i, r = f >> 4, c4 = f & 15;
            const int64_t n = n0 + r;
            x[i] = n < N ? *reinterpret_cast<const floatx4 *>(X + n * K + kt * BK + 4 * c4) : floatx4{0.f, 0.f, 0.f, 0.f};
        }
    };
    auto xstore = [&](const floatx4 (&x)[NXF], _Float16 *xs) {
#pragma unroll
        for (int i = 0; i < NXF; i++) {
            const int f = t + NT * i, r = f >> 4, c4 = f & 15;
            half4 hv = {(_Float16)x[i].x, (_Float16)x[i].y, (_Float16)x[i].z, (_Float16)x[i].w};
            *reinterpret_cast<half4 *>(xs + r * LDK + 4 * c4) = hv;
        }
    };

    floatx16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; i++)
#pragma unroll
        for (int j = 0; j < FM; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

    // prologue: weights k-tiles 0..WD-1, activations 0..XD-1 in flight;
    // k-tile 0 decoded and staged
#pragma unroll
    for (int d = 0; d < WD; d++)
        if (d < nkt) wload(d, wr[d]);
#pragma unroll
    for (int d = 0; d < XD; d++)
        if (d < nkt) xload(d, xr[d]);
#pragma unroll
    for (int j = 0; j < FM; j++) BD::decode(wr[0][j], kh, 0, bf[0][j]);
    xstore(xr[0], Xs[0]);
    if (WD < nkt) wload(WD, wr[0]);
    if (XD < nkt) xload(XD, xr[0]);
    __syncthreads();

    constexpr int UNR = (WD % 2 == 0) ? WD : 2 * WD;  // multiple of WD, XD (=2) and 2
    for (int64_t kb = 0; kb < nkt; kb += UNR) {
#pragma unroll
        for (int u = 0; u < UNR; u++) {
            const int64_t kt = kb + u;
            if (kt < nkt) {
                // this k-tile on the matrix cores, with the next k-tile's weight
                // decode (one slice per 16-deep step) and activation staging in
                // between
                const bool more = kt + 1 < nkt;
                const _Float16 *xs = Xs[u & 1];
                half8 nb[FM][4];
#pragma unroll
                for (int s = 0; s < BK / 16; s++) {
                    half8 a[FN];
#pragma unroll
                    for (int i = 0; i < FN; i++)
                        a[i] = *reinterpret_cast<const half8 *>(xs + (32 * i + (lane & 31)) * LDK + 16 * s + 8 * kh);
#pragma unroll
                    for (int i = 0; i < FN; i++)
#pragma unroll
                        for (int j = 0; j < FM; j++)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], bf[u & 1][j][s], acc[i][j], 0, 0, 0);
                    if (more) {
                        if (s == 0) {
#pragma unroll
                            for (int j = 0; j < FM; j++) BD::decode(wr[(u + 1) % WD][j], kh, (kt + 1) * BK, nb[j]);
                        }
                        if (s == 1) {
#pragma unroll
                            for (int j = 0; j < FM; j++)
#pragma unroll
                                for (int q = 0; q < 4; q++) bf[(u + 1) & 1][j][q] = nb[j][q];
                            if (kt + 1 + WD < nkt) wload(kt + 1 + WD, wr[(u + 1) % WD]);
                        }
                        if (s == 2) xstore(xr[(u + 1) % XD], Xs[(u + 1) & 1]);
                        if (s == 3 && kt + 1 + XD < nkt) xload(kt + 1 + XD, xr[(u + 1) % XD]);
                    }
                }
                __syncthreads();
            }
        }
    }

#pragma unroll
    for (int i = 0; i < FN; i++) {
#pragma unroll
        for (int j = 0; j < FM; j++) {
            const int64_t m = mw + 32 * j + (lane & 31);
            if (m >= M) continue;
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int64_t n = n0 + 32 * i + 8 * (v >> 2) + 4 * kh + (v & 3);
                if (n < N) Y[n * M + m] = acc[i][j][v];
            }
        }
    }
}

// ------------------------------------------------------------ launcher ----

static bool aligned_layout(int dtype, int64_t nb) {
    switch (dtype) {
    case QMM_Q4_0:
    case QMM_Q8_0:
    case QMM_Q6_K: return (nb % 2) == 0;
    case QMM_Q4_K: return true;
    default: return false;
    }
}

template <int DT, int BM, int BN, int WN, int WM>
static hipError_t launch_tile(const uint8_t *blob, int64_t M, int64_t K, int64_t N, const float *X, float *Y,
                              hipStream_t st, bool gen) {
    constexpr int BS = Geo<DT>::BS, BB = Geo<DT>::BB;
    const int64_t row_bytes = (K / BS) * BB;
    const int64_t mtiles = (M + BM - 1) / BM, ntiles = (N + BN - 1) / BN;
    const int64_t grid = mtiles * ntiles;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    if (gen)
        hipLaunchKernelGGL((gemm_kernel<DT, BM, BN, WN, WM, true>), dim3((unsigned)grid), dim3(256), 0, st, blob, M, K, N,
                           row_bytes, X, Y, (int)ntiles);
    else
        hipLaunchKernelGGL((gemm_kernel<DT, BM, BN, WN, WM, false>), dim3((unsigned)grid), dim3(256), 0, st, blob, M, K,
                           N, row_bytes, X, Y, (int)ntiles);
    return hipGetLastError();
}

template <int DT, int TM, int BN, int WD, int W>
static hipError_t launch_wreg(const uint8_t *blob, int64_t M, int64_t K, int64_t N, const float *X, float *Y,
                              hipStream_t st) {
    constexpr int BS = Geo<DT>::BS, BB = Geo<DT>::BB;
    const int64_t row_bytes = (K / BS) * BB;
    const int64_t mtiles = (M + W * TM - 1) / (W * TM), ntiles = (N + BN - 1) / BN;
    const int64_t grid = mtiles * ntiles;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gemm_wreg_kernel<DT, TM, BN, WD, W>), dim3((unsigned)grid), dim3(64 * W), 0, st, blob, M, K,
                       N, row_bytes, X, Y, (int)ntiles);
    return hipGetLastError();
}

// Large-N kernel choice.  Measured on 14336 x 4096 at N = 512: the register-B
// kernel with 8 wavefronts x 32 rows wins for the 4-bit formats once its grid
// (M/256 x N/128 workgroups) nearly fills the chip; the LDS-staged kernel wins
// otherwise.  QMM_GEMM_KERNEL = 0 / 1 / 2 forces LDS-staged / register-B 4x64
// rows / register-B 8x32 rows (for measurement).
static int gemm_kernel_choice() {
    static int v = [] {
        const char *e = getenv("QMM_GEMM_KERNEL");
        return e ? atoi(e) : -1;
    }();
    return v;
}

template <int DT>
static hipError_t launch_dt(const uint8_t *blob, int64_t M, int64_t K, int64_t N, const float *X, float *Y,
                            hipStream_t st) {
    const bool gen = !aligned_layout(DT, K / Geo<DT>::BS);
    const bool wreg_ok = !gen && N > 64 && (K % BK) == 0;
    int choice = gemm_kernel_choice();
    if (choice < 0) {
        const bool four_bit = DT == QMM_Q4_0 || DT == QMM_Q4_K;
        choice = (four_bit && ((M + 255) / 256) * ((N + 127) / 128) >= 224) ? 2 : 0;
    }
    if (wreg_ok && choice == 1) {
        if constexpr (DT == QMM_Q6_K || DT == QMM_Q8_0) return launch_wreg<DT, 32, 128, 2, 4>(blob, M, K, N, X, Y, st);
        else return launch_wreg<DT, 64, 128, 4, 4>(blob, M, K, N, X, Y, st);
    }
    if (wreg_ok && choice == 2) {
        if constexpr (DT == QMM_Q6_K) return launch_wreg<DT, 32, 128, 2, 8>(blob, M, K, N, X, Y, st);
        else return launch_wreg<DT, 32, 128, 3, 8>(blob, M, K, N, X, Y, st);
    }
    if (N <= 32) return launch_tile<DT, 128, 32, 1, 4>(blob, M, K, N, X, Y, st, gen);
    if (N <= 64) return launch_tile<DT, 128, 64, 1, 4>(blob, M, K, N, X, Y, st, gen);
    return launch_tile<DT, 128, 128, 2, 2>(blob, M, K, N, X, Y, st, gen);
}

hipError_t launch_gemm_mfma(int dtype, const void *blob_v, int64_t M, int64_t K, int64_t N, const float *X, float *Y,
                            hipStream_t st) {
    const uint8_t *blob = static_cast<const uint8_t *>(blob_v);
    switch (dtype) {
    case QMM_Q4_0: return launch_dt<QMM_Q4_0>(blob, M, K, N, X, Y, st);
    case QMM_Q8_0: return launch_dt<QMM_Q8_0>(blob, M, K, N, X, Y, st);
    case QMM_Q4_K: return launch_dt<QMM_Q4_K>(blob, M, K, N, X, Y, st);
    case QMM_Q6_K: return launch_dt<QMM_Q6_K>(blob, M, K, N, X, Y, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qmm
