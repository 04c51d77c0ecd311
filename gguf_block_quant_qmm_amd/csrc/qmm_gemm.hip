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

template <bool GEN> struct WTile<QMM_Q4_1, GEN> {
    // part = block 2*(k0/64) + part; 20 bytes: d, m, 16 nibble bytes.  Every
    // block of a 16-byte aligned blob is dword aligned (20 = 5 dwords).
    static constexpr int NDW = 5;
    __device__ static bool exists(int64_t K, int64_t k0, int part) { return k0 + 32 * part < K; }
    __device__ static void load(const uint8_t *row, int64_t k0, int part, uint32_t (&v)[NDW]) {
        const uint8_t *p = row + 20 * (k0 / 32 + part);
        if (GEN) fetch_bytes(p, 20, v);
        else fetch_al(p, v);
    }
    __device__ static void store(const uint32_t (&v)[NDW], int part, _Float16 *wrow) {
        const float d = h2f(v[0]), m = h2f(v[0] >> 16);
        half8 lo[2], hi[2];
#pragma unroll
        for (int i = 0; i < 4; i++) {
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const int e = 4 * i + c;
                lo[e >> 3][e & 7] = (_Float16)fmaf(d, (float)((v[1 + i] >> (8 * c)) & 15u), m);
                hi[e >> 3][e & 7] = (_Float16)fmaf(d, (float)((v[1 + i] >> (8 * c + 4)) & 15u), m);
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

template <bool GEN> struct WTile<QMM_Q5_K, GEN> {
    // As Q4_K's k-tile (chunk c, part = which 16 of its 32 nibble bytes), plus
    // the 16 qh bytes of those elements (bit 2c: sub-block 2c, bit 2c+1: 2c+1).
    // Super-blocks are 16-byte aligned whenever the blob is (176 = 11*16).
    static constexpr int NDW = 12;  // 4 header dwords + 4 qh dwords + 4 nibble dwords
    __device__ static bool exists(int64_t, int64_t, int) { return true; }
    __device__ static void load(const uint8_t *row, int64_t k0, int part, uint32_t (&v)[NDW]) {
        const uint8_t *sb = row + 176 * (k0 / 256);
        const int c = (int)((k0 % 256) / 64);
        uint32_t h[4], qh[4], q[4];
        if (GEN) {
            fetch_bytes(sb, 16, h);
            fetch_bytes(sb + 16 + 16 * part, 16, qh);
            fetch_bytes(sb + 48 + 32 * c + 16 * part, 16, q);
        } else {
            fetch_al(sb, h);
            fetch_al(sb + 16 + 16 * part, qh);
            fetch_al(sb + 48 + 32 * c + 16 * part, q);
        }
#pragma unroll
        for (int i = 0; i < 4; i++) { v[i] = h[i]; v[4 + i] = qh[i]; v[8 + i] = q[i]; }
    }
    __device__ static void store(const uint32_t (&v)[NDW], int part, _Float16 *wrow, int c) {
        const float d = h2f(v[0]), dmin = h2f(v[0] >> 16);
#pragma unroll
        for (int half = 0; half < 2; half++) {
            const int sub = 2 * c + half;
            int sc, mn;
            q4k_scale_min(v[1], v[2], v[3], sub, sc, mn);
            const float dsc = d * (float)sc, ndm = -(dmin * (float)mn);
            half8 o[2];
#pragma unroll
            for (int i = 0; i < 4; i++) {
#pragma unroll
                for (int b = 0; b < 4; b++) {
                    const int e = 4 * i + b;
                    const uint32_t lo = (v[8 + i] >> (8 * b + 4 * half)) & 15u;
                    const uint32_t hi = (v[4 + i] >> (8 * b + sub)) & 1u;
                    o[e >> 3][e & 7] = (_Float16)fmaf(dsc, (float)(lo | (hi << 4)), ndm);
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
    if constexpr (DT == QMM_Q4_K || DT == QMM_Q5_K || DT == QMM_Q6_K)
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

// ================================================ weight decoders ====
// Each wavefront decodes the k-tiles of its weight rows straight into the B
// operand registers of v_mfma_f32_32x32x16_f16 (lane l: row l % 32 of a
// 32-row block, 8 k values for lane half kh = l / 32 in every 16-deep step),
// so a weight is decoded once per token tile and never passes through LDS.
// Exact decode to f16: a code c placed in the low mantissa bits of a 16-bit
// lane is an f16 subnormal (c * 2^-24, or c * 2^-20 for bits 4..7), so one
// v_fma_mix_f32 with the scale * 2^24 (or 2^20) and the bias forms
// scale * c + bias exactly before its single rounding.

constexpr float TWO24 = 16777216.0f;

// Two weights (scale * code + bias, each rounded once to f16) from the two
// f16 code lanes of a dword.  Written as plain code (the compiler forms
// v_fma_mix_f32 / v_fma_mixlo_f16 pairs and the conversions itself): an
// inline-asm form hides its register writes from the compiler's hazard
// checks next to the matrix-core instructions reading the same registers,
// and was measured to give wrong sums in one register allocation.
__device__ __forceinline__ uint32_t mix_pair(uint32_t codes, float scale, float bias) {
    const half2_t c = __builtin_bit_cast(half2_t, codes);
    half2_t o;
    o.x = (_Float16)fmaf((float)c.x, scale, bias);
    o.y = (_Float16)fmaf((float)c.y, scale, bias);
    return __builtin_bit_cast(uint32_t, o);
}
// four weights from the two code pairs of a dword, into f[at .. at+4)
__device__ __forceinline__ void quad(uint32_t p02, uint32_t p13, float scale, float bias, half8 &f, int at) {
    const half2_t a = __builtin_bit_cast(half2_t, mix_pair(p02, scale, bias));
    const half2_t b = __builtin_bit_cast(half2_t, mix_pair(p13, scale, bias));
    f[at] = a.x;
    f[at + 1] = a.y;
    f[at + 2] = b.x;
    f[at + 3] = b.y;
}

// BDec<DT>: raw bytes of one row's 64-deep k-tile that lane half kh needs
// (its k = 16s + 8kh + j, s < 4, j < 8), and their decode to 4 half8.
template <int DT> struct BDec;




template <> struct BDec<QMM_Q6_K> {
    // 8 consecutive k per step, in sigma order within each group of 4
    static constexpr bool SWAP = true;
    __device__ static int xpos(int c4) { return 4 * c4; }
    struct State {};
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
    __device__ static void loadb(Rsrc rs, uint32_t roff, int64_t k0, int kh, int, uint32_t (&r)[NW]) {
        const int64_t sb = k0 / 256;
        const int qq = (int)((k0 % 256) / 64), h = qq >> 1, g0 = 2 * (qq & 1);
        const uint32_t base = (uint32_t)(210 * sb - 2 * (sb & 1));  // dword aligned
        uint32_t w3[3], w2[2], w1[1];
#pragma unroll
        for (int s = 0; s < 4; s++) {
            ldb(rs, roff + 8u * kh, base + 64u * h + 16u * s, w3);
            r[3 * s] = w3[0]; r[3 * s + 1] = w3[1]; r[3 * s + 2] = w3[2];
        }
        ldb(rs, roff + 8u * kh, base + 128u + 32u * h, w3);
        r[12] = w3[0]; r[13] = w3[1]; r[14] = w3[2];
        ldb(rs, roff + 8u * kh, base + 128u + 32u * h + 16u, w3);
        r[15] = w3[0]; r[16] = w3[1]; r[17] = w3[2];
        ldb(rs, roff, base + 192u + 8u * h + 2u * g0 - (2u * g0 & 3u), w2);
        r[18] = w2[0]; r[19] = w2[1];
        ldb(rs, roff, base + 208u, w1);
        r[20] = w1[0];
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
            const uint32_t q0 = lo0 | hi0, q1 = lo1 | hi1;  // four 6-bit codes each, one per byte
            quad(q0 & 0x00FF00FFu, (q0 >> 8) & 0x00FF00FFu, dsc * TWO24, -32.f * dsc, f[s], 0);
            quad(q1 & 0x00FF00FFu, (q1 >> 8) & 0x00FF00FFu, dsc * TWO24, -32.f * dsc, f[s], 4);
        }
    }
    __device__ static void decode(const uint32_t (&r)[NW], State &, int kh, int, int64_t k0, half8 (&f)[4]) {
        decode(r, kh, k0, f);
    }
};

// ------------------------------------------- permuted-k decoders ----
// The contraction only needs the A and B fragments of a 16-deep step to agree
// on which k each of a lane's 8 elements is.  These decoders take each
// lane's bytes in the order that is cheapest to unpack -- a dword d gives
// the element pairs (byte 0, byte 2) = d & mask and (byte 1, byte 3) =
// (d >> 8) & mask, one VOP2 instruction per two codes, low nibbles as
// c * 2^-24 and high nibbles as c * 2^-20 (exact f16 subnormals) -- and the
// activations are written to LDS in the same order: within every group of 8
// the k order is sigma = (0 2 1 3 4 6 5 7), so a float4 of consecutive k
// lands as [x0 x2 x1 x3] in 4 consecutive LDS slots.  Each weight is formed
// by one v_fma_mix (scale * code + bias, then one rounding to f16).
template <int DT> struct PDec;

template <> struct PDec<QMM_Q4_K> {
    // lane half kh: qs[32c + 16kh ..+16) of chunk c; step s: k = 32 (s >> 1) +
    // 16 kh + 8 (s & 1) + sigma(j)  (low nibbles: sub-block 2c, high: 2c+1).
    // The super-block header (d, dmin, 12 scale bytes) comes with chunk 0 and
    // is unpacked once into State for the four chunks.
    static constexpr int NW = 8;
    static constexpr bool SWAP = true;
    struct State { float s[8], n[8]; };
    __device__ static int xpos(int c4) {
        return 16 * (2 * (c4 >> 3) + ((c4 >> 1) & 1)) + 8 * ((c4 >> 2) & 1) + 4 * (c4 & 1);
    }
    __device__ static void loadb(Rsrc rs, uint32_t roff, int64_t k0, int kh, int c, uint32_t (&r)[NW]) {
        const uint32_t sb = (uint32_t)(144 * (k0 / 256));
        if (c == 0) {
            uint32_t h[4];
            ldb(rs, roff, sb, h);
#pragma unroll
            for (int i = 0; i < 4; i++) r[i] = h[i];
        }
        uint32_t q[4];
        ldb(rs, roff + 16u * kh, sb + 16u + 32u * (uint32_t)c, q);
#pragma unroll
        for (int i = 0; i < 4; i++) r[4 + i] = q[i];
    }
    __device__ static void decode(const uint32_t (&r)[NW], State &st, int, int c, int64_t, half8 (&f)[4]) {
        if (c == 0) {
            const float d = h2f(r[0]), dmin = h2f(r[0] >> 16);
#pragma unroll
            for (int i = 0; i < 8; i++) {
                int sc, mn;
                q4k_scale_min(r[1], r[2], r[3], i, sc, mn);
                st.s[i] = d * (float)sc * ((i & 1) ? 1048576.0f : TWO24);  // high nibbles enter as c * 2^-20
                st.n[i] = -(dmin * (float)mn);
            }
        }
        const float s0 = st.s[2 * c], n0 = st.n[2 * c], s1 = st.s[2 * c + 1], n1 = st.n[2 * c + 1];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t w = r[4 + i], t = w >> 8;
            quad(w & 0x000F000Fu, t & 0x000F000Fu, s0, n0, f[i >> 1], 4 * (i & 1));
            quad(w & 0x00F000F0u, t & 0x00F000F0u, s1, n1, f[2 + (i >> 1)], 4 * (i & 1));
        }
    }
};

template <> struct PDec<QMM_Q5_K> {
    // As PDec<QMM_Q4_K> (lane half kh: qs[32c + 16kh ..+16), the header with
    // chunk 0, unpacked once into State), plus qh[16kh ..+16) with every
    // chunk: bits 2c and 2c+1 join the codes as bit 4 (low nibbles, c 2^-24)
    // and bit 8 (high nibbles, c 2^-20).
    static constexpr int NW = 12;
    static constexpr bool SWAP = true;
    struct State { float s[8], n[8]; };
    __device__ static int xpos(int c4) { return PDec<QMM_Q4_K>::xpos(c4); }
    __device__ static void loadb(Rsrc rs, uint32_t roff, int64_t k0, int kh, int c, uint32_t (&r)[NW]) {
        const uint32_t sb = (uint32_t)(176 * (k0 / 256));
        if (c == 0) {
            uint32_t h[4];
            ldb(rs, roff, sb, h);
#pragma unroll
            for (int i = 0; i < 4; i++) r[i] = h[i];
        }
        uint32_t qh[4], q[4];
        ldb(rs, roff + 16u * kh, sb + 16u, qh);
        ldb(rs, roff + 16u * kh, sb + 48u + 32u * (uint32_t)c, q);
#pragma unroll
        for (int i = 0; i < 4; i++) { r[4 + i] = q[i]; r[8 + i] = qh[i]; }
    }
    __device__ static void decode(const uint32_t (&r)[NW], State &st, int, int c, int64_t, half8 (&f)[4]) {
        if (c == 0) {
            const float d = h2f(r[0]), dmin = h2f(r[0] >> 16);
#pragma unroll
            for (int i = 0; i < 8; i++) {
                int sc, mn;
                q4k_scale_min(r[1], r[2], r[3], i, sc, mn);
                st.s[i] = d * (float)sc * ((i & 1) ? 1048576.0f : TWO24);  // high nibbles enter as c * 2^-20
                st.n[i] = -(dmin * (float)mn);
            }
        }
        const float s0 = st.s[2 * c], n0 = st.n[2 * c], s1 = st.s[2 * c + 1], n1 = st.n[2 * c + 1];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t w = r[4 + i], t = w >> 8;
            const uint32_t hq = r[8 + i] >> (2 * c), ht = hq >> 8;
            quad((w & 0x000F000Fu) | ((hq << 4) & 0x00100010u), (t & 0x000F000Fu) | ((ht << 4) & 0x00100010u),
                        s0, n0, f[i >> 1], 4 * (i & 1));
            quad((w & 0x00F000F0u) | ((hq << 7) & 0x01000100u), (t & 0x00F000F0u) | ((ht << 7) & 0x01000100u),
                        s1, n1, f[2 + (i >> 1)], 4 * (i & 1));
        }
    }
};

template <> struct PDec<QMM_Q4_0> {
    // lane half kh: block 2 kt + kh (18 bytes, read from the dword at or just
    // below it); step s: k = 32 kh + 8 s + sigma(j)
    static constexpr int NW = 5;
    static constexpr bool SWAP = true;
    __device__ static int xpos(int c4) { return 16 * ((c4 >> 1) & 3) + 8 * (c4 >> 3) + 4 * (c4 & 1); }
    struct State {};
    __device__ static void loadb(Rsrc rs, uint32_t roff, int64_t k0, int kh, int, uint32_t (&r)[NW]) {
        ldb(rs, roff + 16u * kh, (uint32_t)(36 * (k0 / 64)), r);
    }
    __device__ static void decode(const uint32_t (&r)[NW], State &, int kh, int, int64_t, half8 (&f)[4]) {
        // block 0 starts at byte 0 of r (codes 2 bytes in), block 1 at byte 2
        // (codes dword aligned from r[1])
        const uint32_t sel = kh ? 0x07060504u : 0x05040302u;
        const float d = h2f(kh ? r[0] >> 16 : r[0]);
        const float s24 = d * TWO24, s20 = d * 1048576.0f, n = -8.f * d;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t w = __builtin_amdgcn_perm(r[i + 1], r[i], sel), t = w >> 8;  // qs[4i .. 4i+4)
            quad(w & 0x000F000Fu, t & 0x000F000Fu, s24, n, f[i >> 1], 4 * (i & 1));
            quad(w & 0x00F000F0u, t & 0x00F000F0u, s20, n, f[2 + (i >> 1)], 4 * (i & 1));
        }
    }
};

template <> struct PDec<QMM_Q4_1> {
    // lane half kh: block 2 kt + kh (20 bytes, dword aligned: r[0] = d|m,
    // r[1..4] = qs); step s: k = 32 kh + 8 s + sigma(j), as for Q4_0
    static constexpr int NW = 5;
    static constexpr bool SWAP = true;
    __device__ static int xpos(int c4) { return 16 * ((c4 >> 1) & 3) + 8 * (c4 >> 3) + 4 * (c4 & 1); }
    struct State {};
    __device__ static void loadb(Rsrc rs, uint32_t roff, int64_t k0, int kh, int, uint32_t (&r)[NW]) {
        ldb(rs, roff + 20u * kh, (uint32_t)(40 * (k0 / 64)), r);
    }
    __device__ static void decode(const uint32_t (&r)[NW], State &, int, int, int64_t, half8 (&f)[4]) {
        const float d = h2f(r[0]), m = h2f(r[0] >> 16);
        const float s24 = d * TWO24, s20 = d * 1048576.0f;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t w = r[1 + i], t = w >> 8;  // qs[4i .. 4i+4)
            quad(w & 0x000F000Fu, t & 0x000F000Fu, s24, m, f[i >> 1], 4 * (i & 1));
            quad(w & 0x00F000F0u, t & 0x00F000F0u, s20, m, f[2 + (i >> 1)], 4 * (i & 1));
        }
    }
};

template <> struct PDec<QMM_Q8_0> {
    // lane half kh: block 2 kt + kh (34 bytes); step s: k = 32 kh + 8 s + sigma(j)
    static constexpr int NW = 9;
    static constexpr bool SWAP = true;
    __device__ static int xpos(int c4) { return 16 * ((c4 >> 1) & 3) + 8 * (c4 >> 3) + 4 * (c4 & 1); }
    struct State {};
    __device__ static void loadb(Rsrc rs, uint32_t roff, int64_t k0, int kh, int, uint32_t (&r)[NW]) {
        ldb(rs, roff + 32u * kh, (uint32_t)(68 * (k0 / 64)), r);
    }
    __device__ static void decode(const uint32_t (&r)[NW], State &, int kh, int, int64_t, half8 (&f)[4]) {
        const uint32_t sel = kh ? 0x07060504u : 0x05040302u;
        const float d = h2f(kh ? r[0] >> 16 : r[0]);
        const float s24 = d * TWO24, n = -128.f * d;  // codes enter as q + 128
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t w = __builtin_amdgcn_perm(r[i + 1], r[i], sel) ^ 0x80808080u;  // q[4i .. 4i+4) + 128
            quad(w & 0x00FF00FFu, (w >> 8) & 0x00FF00FFu, s24, n, f[i >> 1], 4 * (i & 1));
        }
    }
};

template <> struct PDec<QMM_Q6_K_R> {
    // The repacked Q6_K layout: per super-block 256 code bytes, then the 16
    // sub-block scales d * sc as f32.  In k-tile c lane half kh reads the 32
    // code bytes at 64c + 32kh; byte 8s + j is the code of k = 64c + 16s +
    // 8kh + j, so every lane and step holds the k that BDec<QMM_Q6_K> gives
    // it, and step s lies in sub-block 4c + s.  Each weight is the same
    // single rounding of d * sc * (q - 32) as from the GGUF bytes: the
    // matrix-core steps get the same operands and the sums the same bits.
    static constexpr int NW = 12;
    static constexpr bool SWAP = true;
    __device__ static int xpos(int c4) { return BDec<QMM_Q6_K>::xpos(c4); }
    struct State {};
    __device__ static void loadb(Rsrc rs, uint32_t roff, int64_t k0, int kh, int c, uint32_t (&r)[NW]) {
        const uint32_t sb = (uint32_t)(320 * (k0 / 256));
        uint32_t q[8], sc[4];
        ldb(rs, roff + 32u * kh, sb + 64u * (uint32_t)c, q);
        ldb(rs, roff, sb + 256u + 16u * (uint32_t)c, sc);
#pragma unroll
        for (int i = 0; i < 8; i++) r[i] = q[i];
#pragma unroll
        for (int i = 0; i < 4; i++) r[8 + i] = sc[i];
    }
    __device__ static void decode(const uint32_t (&r)[NW], State &, int, int, int64_t, half8 (&f)[4]) {
#pragma unroll
        for (int s = 0; s < 4; s++) {
            const float dsc = __builtin_bit_cast(float, r[8 + s]);
            const float s24 = dsc * TWO24, n = -32.f * dsc;
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const uint32_t w = r[2 * s + h];  // codes of j = 4h .. 4h + 3
                quad(w & 0x00FF00FFu, (w >> 8) & 0x00FF00FFu, s24, n, f[s], 4 * h);
            }
        }
    }
};

template <> struct PDec<QMM_Q8_0_R> {
    // The repacked Q8_0 layout: per k-tile (two GGUF blocks) 64 code bytes
    // q + 128, then d of both blocks as f32.  Lane half kh reads block kh's
    // 32 codes at 32kh; step s takes k = 32kh + 8s + sigma(j), the k that
    // PDec<QMM_Q8_0> gives it, and each weight is the same single rounding of
    // d * q to f16, so the matrix-core steps see the same operands.
    static constexpr int NW = 9;
    static constexpr bool SWAP = true;
    __device__ static int xpos(int c4) { return PDec<QMM_Q8_0>::xpos(c4); }
    struct State {};
    __device__ static void loadb(Rsrc rs, uint32_t roff, int64_t k0, int kh, int, uint32_t (&r)[NW]) {
        const uint32_t base = (uint32_t)(72 * (k0 / 64));
        uint32_t q[8], d[1];
        ldb(rs, roff + 32u * kh, base, q);
        ldb(rs, roff + 4u * kh, base + 64u, d);
#pragma unroll
        for (int i = 0; i < 8; i++) r[i] = q[i];
        r[8] = d[0];
    }
    __device__ static void decode(const uint32_t (&r)[NW], State &, int, int, int64_t, half8 (&f)[4]) {
        const float d = __builtin_bit_cast(float, r[8]);
        const float s24 = d * TWO24, n = -128.f * d;  // codes enter as q + 128
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t w = r[i];
            quad(w & 0x00FF00FFu, (w >> 8) & 0x00FF00FFu, s24, n, f[i >> 1], 4 * (i & 1));
        }
    }
};

template <int DT> struct WbDec { using type = PDec<DT>; };
template <> struct WbDec<QMM_Q6_K> { using type = BDec<QMM_Q6_K>; };

// ============================================= register-B GEMM, buffered ====
// The register-B design above with every global access a bounds-checked
// buffer load: weight rows past M and token rows past N read as zeros, and
// the prefetch of k-tiles past the end is clamped onto the last one, so the
// k-loop has no branch at all (K is a multiple of UNR k-tiles) and every
// wait is for exactly the data the next step consumes.  Workgroups are
// ordered so that the ones sharing a weight tile run on the same XCD (the
// dispatcher sends workgroup b to XCD b % 8), whose L2 then serves the
// weights to all token tiles.
//
// SWI (gate/up projection with SwiGLU, page "cera 0.5.2 src/backend/cpu.rs":
// the fused gate + up + SiLU GEMM dispatch), neither projection ever stored:
//   TM = 64: each wavefront's two 32-row fragments are the same 32 rows of
//     the gate matrix (blob) and of the up matrix (blob_up); the epilogue
//     writes silu(gate) * up for those 32 output rows;
//   TM = 32 (the wavefront pair form): wavefront w < W/2 computes 32 rows of
//     the gate matrix and wavefront w + W/2 the same rows of the up matrix,
//     each the plain kernel's tile; the up tiles go through LDS to their gate
//     partners, which write silu(gate) * up.  The registers of the plain
//     8 x 32-row x 128-token tile, where a wavefront holding both fragments
//     of 128 tokens would not fit two per SIMD.
//
// BE: one workgroup barrier every BE k-tiles.  The activation tiles sit in
// 2 BE LDS buffers and each is stored BE k-tiles ahead of its use, so that a
// barrier always separates a tile's stores from its reads and its reads from
// the next store into the same buffer.
template <int DT, int TM, int BN, int WD, int W, int INTERLEAVE, int XD, bool SWI = false, int BE = 1>
__global__ void __launch_bounds__(64 * W) gemm_wb_kernel(const uint8_t *__restrict__ blob,
                                                        const uint8_t *__restrict__ blob_up, int64_t M, int64_t K,
                                                        int64_t N, int64_t row_bytes, const float *__restrict__ X,
                                                        float *__restrict__ Y, int n_mtiles, int n_ntiles) {
    constexpr int FM = TM / 32, FN = BN / 32;
    constexpr bool PAIR = SWI && FM == 1;  // gate and up in two wavefronts
    constexpr int OT = SWI ? 32 : TM;      // output rows per wavefront
    constexpr int OW = PAIR ? W / 2 : W;   // wavefronts per workgroup with distinct output rows
    static_assert(!SWI || FM == 2 || (FM == 1 && W % 2 == 0), "the SwiGLU forms pair a gate and an up fragment");
    constexpr int NT = 64 * W;
    constexpr int NX4 = BN * (BK / 4);          // float4 of X per k-tile
    constexpr int NXF = (NX4 + NT - 1) / NT;    // per thread (the last ones repeat a valid float4)
    constexpr int UNR = 4;  // k-tiles per trip: a Q4_K super-block; K is a multiple of 4 k-tiles
    static_assert(UNR % WD == 0 && UNR % XD == 0, "ring sizes");
    using BD = typename WbDec<DT>::type;
    // (2 BE buffers indexed by the k-tile's place in the unrolled trip)
    static_assert((BE == 1 || BE == 2) && BE <= XD, "barrier cadence and activation ring");
    constexpr int NB = 2 * BE, SD = BE;  // LDS activation buffers; store distance in k-tiles
    __shared__ __attribute__((aligned(16))) _Float16 Xs[NB][BN * LDK];

    const int t = threadIdx.x, lane = t & 63, kh = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int total = n_mtiles * n_ntiles, b = blockIdx.x, xcd = b & 7, local = b >> 3;
    const int tile = xcd * (total >> 3) + (xcd < (total & 7) ? xcd : (total & 7)) + local;
    const int64_t mt = tile / n_ntiles, nt = tile % n_ntiles;
    const int half = PAIR ? wave / OW : 0;  // PAIR: 0 gate, 1 up (wave-uniform)
    const int64_t n0 = nt * BN, mw = mt * (OW * OT) + (wave % OW) * OT;
    const int64_t nkt = K / BK;

    const int64_t wrows = M - mw < 0 ? 0 : (M - mw < OT ? M - mw : OT);
    const Rsrc wrs = make_rsrc_uniform((PAIR && half ? blob_up : blob) + (wrows ? mw : 0) * row_bytes,
                                       (uint32_t)(wrows * row_bytes));
    const Rsrc wrs_up = make_rsrc_uniform((SWI ? blob_up : blob) + (wrows ? mw : 0) * row_bytes,
                                          (uint32_t)(wrows * row_bytes));
    uint32_t roff[FM];
#pragma unroll
    for (int j = 0; j < FM; j++) roff[j] = (uint32_t)(((SWI ? 0 : 32 * j) + (lane & 31)) * row_bytes);
    const int64_t xrows = N - n0 < BN ? N - n0 : BN;
    const Rsrc xrs = make_rsrc_uniform(X + n0 * K, (uint32_t)(xrows * K * 4));
    uint32_t xoff[NXF];
#pragma unroll
    for (int i = 0; i < NXF; i++) {
        const int f = t + NT * i < NX4 ? t + NT * i : NX4 - 1, r = f >> 4, c4 = f & 15;
        xoff[i] = (uint32_t)((r * K + 4 * c4) * 4);
    }

    uint32_t wr[WD][FM][BD::NW];
    floatx4 xr[XD][NXF];
    half8 bf[2][FM][4];
    typename BD::State st[FM];

    // c = kt % 4 (a compile-time constant at every call)
    auto wload = [&](int64_t kt, int c, uint32_t (&w)[FM][BD::NW]) {
        const int64_t kc = kt < nkt ? kt : nkt - 4 + c;
#pragma unroll
        for (int j = 0; j < FM; j++) BD::loadb(SWI && j ? wrs_up : wrs, roff[j], kc * BK, kh, c, w[j]);
    };
    auto xload = [&](int64_t kt, floatx4 (&x)[NXF]) {
        const uint32_t kb = (uint32_t)((kt < nkt ? kt : nkt - 1) * BK * 4);
#pragma unroll
        for (int i = 0; i < NXF; i++)
            x[i] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xoff[i], kb, 0));
    };
    auto xstore = [&](const floatx4 (&x)[NXF], _Float16 *xs) {
#pragma unroll
        for (int i = 0; i < NXF; i++) {
            // a clamped repeat writes the same value to the same slot
            const int f = t + NT * i < NX4 ? t + NT * i : NX4 - 1, r = f >> 4, c4 = f & 15;
            half4 hv;
            if constexpr (BD::SWAP)
                hv = half4{(_Float16)x[i].x, (_Float16)x[i].z, (_Float16)x[i].y, (_Float16)x[i].w};
            else
                hv = half4{(_Float16)x[i].x, (_Float16)x[i].y, (_Float16)x[i].z, (_Float16)x[i].w};
            *reinterpret_cast<half4 *>(xs + r * LDK + BD::xpos(c4)) = hv;
        }
    };

    floatx16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; i++)
#pragma unroll
        for (int j = 0; j < FM; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

#pragma unroll
    for (int d = 0; d < WD; d++) wload(d, d % 4, wr[d]);
#pragma unroll
    for (int d = 0; d < XD; d++) xload(d, xr[d]);
#pragma unroll
    for (int j = 0; j < FM; j++) BD::decode(wr[0][j], st[j], kh, 0, 0, bf[0][j]);
    wload(WD, WD % 4, wr[0]);
    // the first SD activation tiles into LDS; the ring then holds tiles SD ..
#pragma unroll
    for (int d = 0; d < SD; d++) {
        xstore(xr[d], Xs[d]);
        xload(d + XD, xr[d]);
    }
    __syncthreads();

    for (int64_t kb = 0; kb < nkt; kb += UNR) {
#pragma unroll
        for (int u = 0; u < UNR; u++) {
            const int64_t kt = kb + u;
            const _Float16 *xs = Xs[u % NB];
            // all A fragments of the k-tile are read up front, so the MFMAs
            // wait for LDS only once per k-tile
            half8 a[BK / 16][FN];
#pragma unroll
            for (int s = 0; s < BK / 16; s++)
#pragma unroll
                for (int i = 0; i < FN; i++)
                    a[s][i] = *reinterpret_cast<const half8 *>(xs + (32 * i + (lane & 31)) * LDK + 16 * s + 8 * kh);
            __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs
#pragma unroll
            for (int s = 0; s < BK / 16; s++) {
#pragma unroll
                for (int i = 0; i < FN; i++)
#pragma unroll
                    for (int j = 0; j < FM; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[s][i], bf[u & 1][j][s], acc[i][j], 0, 0, 0);
                // the next k-tile (its data for kt + 1 = nkt is a clamped repeat, never used)
                if (s == 0) {
#pragma unroll
                    for (int j = 0; j < FM; j++)
                        BD::decode(wr[(u + 1) % WD][j], st[j], kh, (u + 1) % 4, (kt + 1) * BK, bf[(u + 1) & 1][j]);
                }
                if (s == 1) wload(kt + 1 + WD, (u + 1 + WD) % 4, wr[(u + 1) % WD]);
                // activation tile kt + SD into LDS, tile kt + SD + XD into its ring slot
                if (s == 2) xstore(xr[(u + SD) % XD], Xs[(u + SD) % NB]);
                if (s == 3) xload(kt + SD + XD, xr[(u + SD) % XD]);
            }
            if constexpr (INTERLEAVE > 0) {
                // one MFMA, then INTERLEAVE vector instructions, repeated
#pragma unroll
                for (int q = 0; q < (BK / 16) * FN * FM; q++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, INTERLEAVE, 0);
                }
            }
            if (u % BE == BE - 1) __syncthreads();
        }
    }

    if constexpr (PAIR) {
        // the up tiles reach their gate partners through the activation
        // buffer (free after the k-loop's last barrier), two token fragments
        // at a time: [OW][2][16][64] floats = 32 KB for W = 8
        static_assert(OW * 2 * 16 * 64 * 4 <= 2 * BN * LDK * 2, "exchange fits the activation buffer");
        float *ex = reinterpret_cast<float *>(&Xs[0][0]);
#pragma unroll
        for (int i0 = 0; i0 < FN; i0 += 2) {
            if (half) {
#pragma unroll
                for (int ii = 0; ii < 2 && i0 + ii < FN; ii++)
#pragma unroll
                    for (int v = 0; v < 16; v++)
                        ex[(((wave - OW) * 2 + ii) * 16 + v) * 64 + lane] = acc[i0 + ii][0][v];
            }
            __syncthreads();
            if (!half) {
                const int64_t m = mw + (lane & 31);
#pragma unroll
                for (int ii = 0; ii < 2 && i0 + ii < FN; ii++)
#pragma unroll
                    for (int v = 0; v < 16; v++) {
                        const int64_t n = n0 + 32 * (i0 + ii) + 8 * (v >> 2) + 4 * kh + (v & 3);
                        const float u = ex[((wave * 2 + ii) * 16 + v) * 64 + lane];
                        if (m < M && n < N) Y[n * M + m] = silu(acc[i0 + ii][0][v]) * u;
                    }
            }
            __syncthreads();
        }
    } else if constexpr (SWI) {
#pragma unroll
        for (int i = 0; i < FN; i++) {
            const int64_t m = mw + (lane & 31);
            if (m >= M) continue;
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int64_t n = n0 + 32 * i + 8 * (v >> 2) + 4 * kh + (v & 3);
                if (n < N) Y[n * M + m] = silu(acc[i][0][v]) * acc[i][1][v];
            }
        }
    } else {
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
}

// ============================================= skinny split-K GEMM ====
// Small N (verify batches, N <= 64) and small grids: a workgroup owns 32
// weight rows and BN tokens, and its W wavefronts split K into contiguous
// ranges of whole super-blocks.  Each wavefront stages its own activations
// in a private double-buffered LDS region (LDS operations of one wavefront
// complete in order), so the k-loop has no barrier at all; the W partial
// 32 x BN tiles are summed once at the end through LDS, in wavefront order
// (deterministic).  Weights and activations use the same bounds-checked
// buffer loads, decoders and permuted-k layout as the kernel above.
//
// FM weight-row fragments of 32 per wavefront (a workgroup owns 32 FM rows):
// every activation fragment read from LDS feeds FM matrix-core steps, so the
// activation traffic per weight row falls by FM.  Each output's sum has the
// same order for every FM (same k-steps, same wavefront order).
template <int DT, int BN, int W, int WD, int XD, int FM = 1>
__global__ void __launch_bounds__(64 * W) gemm_sk_kernel(const uint8_t *__restrict__ blob, int64_t M, int64_t K,
                                                        int64_t N, int64_t row_bytes, const float *__restrict__ X,
                                                        float *__restrict__ Y, int n_ntiles) {
    constexpr int FN = BN / 32;
    constexpr int NX4 = BN * (BK / 4);  // float4 of X per k-tile
    constexpr int NXF = NX4 / 64;       // per lane
    constexpr int UNR = 4;
    static_assert(UNR % WD == 0 && UNR % XD == 0 && NX4 % 64 == 0, "ring sizes");
    using BD = typename WbDec<DT>::type;
    extern __shared__ __attribute__((aligned(16))) _Float16 sk_lds[];

    const int t = threadIdx.x, lane = t & 63, kh = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int64_t mt = blockIdx.x / n_ntiles, nt = blockIdx.x % n_ntiles;
    const int64_t m0 = mt * (32 * FM), n0 = nt * BN;
    const int64_t per = (K / BK) / W, kt0 = wave * per;  // per is a multiple of 4
    _Float16 *xw = sk_lds + wave * (2 * BN * LDK);

    const int64_t wrows = M - m0 < 32 * FM ? M - m0 : 32 * FM;
    const Rsrc wrs = make_rsrc_uniform(blob + m0 * row_bytes, (uint32_t)(wrows * row_bytes));
    uint32_t roff[FM];
#pragma unroll
    for (int j = 0; j < FM; j++) roff[j] = (uint32_t)((32 * j + (lane & 31)) * row_bytes);
    const int64_t xrows = N - n0 < BN ? N - n0 : BN;
    const Rsrc xrs = make_rsrc_uniform(X + n0 * K, (uint32_t)(xrows * K * 4));
    uint32_t xoff[NXF];
#pragma unroll
    for (int i = 0; i < NXF; i++) {
        const int f = lane + 64 * i, r = f >> 4, c4 = f & 15;
        xoff[i] = (uint32_t)((r * K + 4 * c4) * 4);
    }

    uint32_t wr[WD][FM][BD::NW];
    floatx4 xr[XD][NXF];
    half8 bf[2][FM][4];
    typename BD::State st[FM];
    const int64_t kend = kt0 + per;
    // c = kt % 4 (a compile-time constant at every call); tiles past the
    // range repeat its last super-block (never used)
    auto wload = [&](int64_t kt, int c, uint32_t (&w)[FM][BD::NW]) {
        const int64_t kc = kt < kend ? kt : kend - 4 + c;
#pragma unroll
        for (int j = 0; j < FM; j++) BD::loadb(wrs, roff[j], kc * BK, kh, c, w[j]);
    };
    auto xload = [&](int64_t kt, floatx4 (&x)[NXF]) {
        const uint32_t kb = (uint32_t)((kt < kend ? kt : kend - 1) * BK * 4);
#pragma unroll
        for (int i = 0; i < NXF; i++)
            x[i] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xoff[i], kb, 0));
    };
    auto xstore = [&](const floatx4 (&x)[NXF], _Float16 *xs) {
#pragma unroll
        for (int i = 0; i < NXF; i++) {
            const int f = lane + 64 * i, r = f >> 4, c4 = f & 15;
            half4 hv;
            if constexpr (BD::SWAP)
                hv = half4{(_Float16)x[i].x, (_Float16)x[i].z, (_Float16)x[i].y, (_Float16)x[i].w};
            else
                hv = half4{(_Float16)x[i].x, (_Float16)x[i].y, (_Float16)x[i].z, (_Float16)x[i].w};
            *reinterpret_cast<half4 *>(xs + r * LDK + BD::xpos(c4)) = hv;
        }
    };

    floatx16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; i++)
#pragma unroll
        for (int j = 0; j < FM; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

#pragma unroll
    for (int d = 0; d < WD; d++) wload(kt0 + d, d % 4, wr[d]);
#pragma unroll
    for (int d = 0; d < XD; d++) xload(kt0 + d, xr[d]);
#pragma unroll
    for (int j = 0; j < FM; j++) BD::decode(wr[0][j], st[j], kh, 0, kt0 * BK, bf[0][j]);
    xstore(xr[0], xw);
    wload(kt0 + WD, WD % 4, wr[0]);
    xload(kt0 + XD, xr[0]);

    for (int64_t kb = kt0; kb < kend; kb += UNR) {
#pragma unroll
        for (int u = 0; u < UNR; u++) {
            const int64_t kt = kb + u;
            const _Float16 *xs = xw + (u & 1) * (BN * LDK);
            half8 a[BK / 16][FN];
#pragma unroll
            for (int s = 0; s < BK / 16; s++)
#pragma unroll
                for (int i = 0; i < FN; i++)
                    a[s][i] = *reinterpret_cast<const half8 *>(xs + (32 * i + (lane & 31)) * LDK + 16 * s + 8 * kh);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < BK / 16; s++) {
#pragma unroll
                for (int i = 0; i < FN; i++)
#pragma unroll
                    for (int j = 0; j < FM; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[s][i], bf[u & 1][j][s], acc[i][j], 0, 0, 0);
                if (s == 0) {
#pragma unroll
                    for (int j = 0; j < FM; j++)
                        BD::decode(wr[(u + 1) % WD][j], st[j], kh, (u + 1) % 4, (kt + 1) * BK, bf[(u + 1) & 1][j]);
                }
                if (s == 1) wload(kt + 1 + WD, (u + 1 + WD) % 4, wr[(u + 1) % WD]);
                if (s == 2) xstore(xr[(u + 1) % XD], xw + ((u + 1) & 1) * (BN * LDK));
                if (s == 3) xload(kt + 1 + XD, xr[(u + 1) % XD]);
            }
        }
    }

    // sum the W partial tiles in wavefront order
    __syncthreads();
    constexpr int NF = FN * FM;  // 32 x 32 fragments per wavefront, index i * FM + j
    float *red = reinterpret_cast<float *>(sk_lds);  // [W][NF * 16][64]
#pragma unroll
    for (int i = 0; i < FN; i++)
#pragma unroll
        for (int j = 0; j < FM; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) red[(wave * NF * 16 + (i * FM + j) * 16 + v) * 64 + lane] = acc[i][j][v];
    __syncthreads();
    for (int o = t; o < NF * 16 * 64; o += 64 * W) {
        float sum = red[o];
        for (int w = 1; w < W; w++) sum += red[w * NF * 16 * 64 + o];
        const int L = o & 63, v = (o >> 6) & 15, f = o >> 10, i = f / FM, j = f % FM;
        const int64_t m = m0 + 32 * j + (L & 31), n = n0 + 32 * i + 8 * (v >> 2) + 4 * (L >> 5) + (v & 3);
        if (m < M && n < N) Y[n * M + m] = sum;
    }
}

template <int DT, int BN, int W, int WD, int XD, int FM = 1>
static hipError_t launch_sk(const uint8_t *blob, int64_t M, int64_t K, int64_t N, const float *X, float *Y,
                            hipStream_t st) {
    constexpr int BS = Geo<DT>::BS, BB = Geo<DT>::BB;
    const int64_t row_bytes = (K / BS) * BB;
    const int64_t mtiles = (M + 32 * FM - 1) / (32 * FM), ntiles = (N + BN - 1) / BN;
    const int64_t grid = mtiles * ntiles;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    constexpr size_t xs_bytes = (size_t)W * 2 * BN * LDK * 2, red_bytes = (size_t)W * (BN / 32) * FM * 16 * 64 * 4;
    constexpr size_t lds = xs_bytes > red_bytes ? xs_bytes : red_bytes;
    if (lds > 64 * 1024) {
        static const hipError_t attr = hipFuncSetAttribute(
            reinterpret_cast<const void *>(&gemm_sk_kernel<DT, BN, W, WD, XD, FM>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (attr != hipSuccess) return attr;
    }
    hipLaunchKernelGGL((gemm_sk_kernel<DT, BN, W, WD, XD, FM>), dim3((unsigned)grid), dim3(64 * W), lds, st, blob, M,
                       K, N, row_bytes, X, Y, (int)ntiles);
    return hipGetLastError();
}

// ------------------------------------------------------------ launcher ----

static bool aligned_layout(int dtype, int64_t nb) {
    switch (dtype) {
    case QMM_Q4_0:
    case QMM_Q8_0:
    case QMM_Q6_K: return (nb % 2) == 0;
    case QMM_Q4_1:
    case QMM_Q4_K:
    case QMM_Q5_K:
    case QMM_Q6_K_R:
    case QMM_Q8_0_R: return true;
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


template <int DT, int TM, int BN, int WD, int W, int IL = 0, int XD = 2, bool SWI = false, int BE = 1>
static hipError_t launch_wb(const uint8_t *blob, int64_t M, int64_t K, int64_t N, const float *X, float *Y,
                            hipStream_t st, const uint8_t *blob_up = nullptr) {
    constexpr int BS = Geo<DT>::BS, BB = Geo<DT>::BB;
    constexpr int OT = SWI ? 32 : TM;
    constexpr int OW = (SWI && TM == 32) ? W / 2 : W;  // the wavefront pair form: W/2 output row groups
    const int64_t row_bytes = (K / BS) * BB;
    const int64_t mtiles = (M + OW * OT - 1) / (OW * OT), ntiles = (N + BN - 1) / BN;
    const int64_t grid = mtiles * ntiles;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gemm_wb_kernel<DT, TM, BN, WD, W, IL, XD, SWI, BE>), dim3((unsigned)grid), dim3(64 * W), 0, st,
                       blob, blob_up, M, K, N, row_bytes, X, Y, (int)mtiles, (int)ntiles);
    return hipGetLastError();
}

// Kernel ids (gemm_kernel_choice): the LDS-staged kernel, the register-B
// kernel at three tile shapes, the skinny split-K kernel at four.
enum {
    GEMM_K_LDS = 0,       // gemm_kernel: weights decoded into an LDS tile
    GEMM_K_WB_8x128 = 1,  // gemm_wb_kernel, 8 wavefronts x 32 rows x 128 tokens
    GEMM_K_WB_4x64 = 2,   // gemm_wb_kernel, 4 wavefronts x 32 rows x 64 tokens
    GEMM_K_WB_4x32 = 3,   // gemm_wb_kernel, 4 wavefronts x 32 rows x 32 tokens
    GEMM_K_SK = 4,        // gemm_sk_kernel, 32 rows x 32 tokens
    GEMM_K_SK_FM2 = 5,    // gemm_sk_kernel, 64 rows x 32 tokens
    GEMM_K_SK_64 = 6,     // gemm_sk_kernel, 32 rows x 64 tokens
    GEMM_K_SK_FM2_64 = 7, // gemm_sk_kernel, 64 rows x 64 tokens
    GEMM_K_COUNT = 8
};

// Kernel choice (measured on 4096 x 4096 and 14336 x 4096 weights):
//   * the skinny split-K kernel (32 rows x 32 tokens, 4 wavefronts splitting
//     K) when the 32 x 32 tile grid is small, or N <= 32 with at most 1024
//     row tiles -- small N leaves too few row x token tiles to fill the chip
//     otherwise; taller matrices (a 128256-row head) have tiles enough and
//     run 4 x 32 rows x 32 tokens without the split (240 vs 300 us there);
//   * the skinny kernel with two 32-row fragments per wavefront for N <= 32
//     when that still gives >= 192 workgroups (half the activation traffic);
//   * for N > 32, the skinny kernel with 64-token tiles (32 or 64 rows) when
//     it fits one round of <= 256 workgroups and the 32-token tile does not
//     (4096 x 4096 Q4_K N = 128: 32-row tiles 20.7 vs 23.8 us; N = 256:
//     64-row tiles 28.6 vs 35.4 us; 14336 x 4096 N = 64: 30.2 vs 36.6 us);
//   * the buffered kernel with 8 wavefronts x 32 rows x 128 tokens when that
//     grid gives at least 160 workgroups, else 4 x 32 rows x 64 tokens;
//   * the LDS-staged kernel when the layout rules the others out (K not a
//     multiple of 256, odd block counts).
// A measurement build (QMM_TUNING) takes QMM_GEMM_KERNEL = an id to force
// where the layout allows.
template <int DT>
static int choice_dt(int64_t M, int64_t K, int64_t N) {
    const bool gen = !aligned_layout(DT, K / Geo<DT>::BS);
    // buffer resources cover at most 128 token rows of X: 32-bit byte counts
    const bool wb_ok = !gen && (K % (4 * BK)) == 0 && K * 4 * 128 < ((int64_t)1 << 31);
    const bool sk_ok = wb_ok && (K / BK) % 16 == 0;  // 4 wavefronts x whole super-blocks
    int choice = tuning_lever("QMM_GEMM_KERNEL", -1);
    if (choice >= GEMM_K_SK && choice < GEMM_K_COUNT && !sk_ok) choice = -1;
    if (choice > GEMM_K_LDS && choice < GEMM_K_COUNT && !wb_ok) choice = -1;
    if (choice >= 0 && choice < GEMM_K_COUNT) return choice;
    const int64_t mt32 = (M + 31) / 32, mt64 = (M + 63) / 64, nt32 = (N + 31) / 32, nt64 = (N + 63) / 64;
    if (!wb_ok) return GEMM_K_LDS;
    if (sk_ok && N > 32 && mt32 * nt32 > 256 && mt32 * nt64 <= 256) return GEMM_K_SK_64;
    if (sk_ok && N > 32 && mt32 * nt32 > 256 && mt64 * nt64 <= 256) return GEMM_K_SK_FM2_64;
    if (sk_ok && ((N <= 32 && mt32 <= 1024) || mt32 * nt32 <= 512))
        // two row fragments per wavefront halve the activation traffic
        // where they still give >= 192 workgroups (14336 x 4096 Q4_K:
        // N = 32 21.3 vs 26.1 us, N = 16 19.0 vs 22.7 us; on 4096 rows
        // the 64 workgroups leave CUs idle: 20.3 vs 13.6 us)
        return (N <= 32 && mt64 >= 192) ? GEMM_K_SK_FM2 : GEMM_K_SK;
    if (N <= 32) return GEMM_K_WB_4x32;
    // 14336 x 4096 Q4_K: N = 320 81 vs 98 us, N = 384 85 vs 105 us (Q4_0 88
    // vs 108, Q6_K 155 vs 192); N = 256 66 vs 73 us the other way
    if (((M + 255) / 256) * ((N + 127) / 128) >= 160) return GEMM_K_WB_8x128;
    return GEMM_K_WB_4x64;
}

template <int DT>
static hipError_t launch_dt(const uint8_t *blob, int64_t M, int64_t K, int64_t N, const float *X, float *Y,
                            hipStream_t st) {
    const bool gen = !aligned_layout(DT, K / Geo<DT>::BS);
    switch (choice_dt<DT>(M, K, N)) {
    // a barrier every 2 k-tiles (14336 x 4096 N = 512: Q4_K 93 -> 86-93 us,
    // Q6_K 165 -> 154, Q8_0 124 -> 120; 4096 x 4096 N = 256 35.2 -> 32.6)
    case GEMM_K_WB_8x128: return launch_wb<DT, 32, 128, 2, 8, 4, 2, false, 2>(blob, M, K, N, X, Y, st);
    case GEMM_K_WB_4x64: return launch_wb<DT, 32, 64, 4, 4, 0, 4, false, 2>(blob, M, K, N, X, Y, st);
    case GEMM_K_WB_4x32: return launch_wb<DT, 32, 32, 4, 4, 0, 4, false, 2>(blob, M, K, N, X, Y, st);
    case GEMM_K_SK: return launch_sk<DT, 32, 4, 2, 2>(blob, M, K, N, X, Y, st);
    case GEMM_K_SK_FM2: return launch_sk<DT, 32, 4, 2, 2, 2>(blob, M, K, N, X, Y, st);
    case GEMM_K_SK_64: return launch_sk<DT, 64, 4, 2, 2, 1>(blob, M, K, N, X, Y, st);
    case GEMM_K_SK_FM2_64: return launch_sk<DT, 64, 4, 2, 2, 2>(blob, M, K, N, X, Y, st);
    default: break;
    }
    if constexpr (DT == QMM_Q6_K_R || DT == QMM_Q8_0_R) {
        return hipErrorInvalidValue;  // no LDS-tile decoder
    } else {
        if (N <= 32) return launch_tile<DT, 128, 32, 1, 4>(blob, M, K, N, X, Y, st, gen);
        if (N <= 64) return launch_tile<DT, 128, 64, 1, 4>(blob, M, K, N, X, Y, st, gen);
        return launch_tile<DT, 128, 128, 2, 2>(blob, M, K, N, X, Y, st, gen);
    }
}

int gemm_kernel_choice(int dtype, int64_t M, int64_t K, int64_t N) {
    switch (dtype) {
    case QMM_Q4_0: return choice_dt<QMM_Q4_0>(M, K, N);
    case QMM_Q4_1: return choice_dt<QMM_Q4_1>(M, K, N);
    case QMM_Q8_0: return choice_dt<QMM_Q8_0>(M, K, N);
    case QMM_Q4_K: return choice_dt<QMM_Q4_K>(M, K, N);
    case QMM_Q5_K: return choice_dt<QMM_Q5_K>(M, K, N);
    case QMM_Q6_K: return choice_dt<QMM_Q6_K>(M, K, N);
    default: return -1;
    }
}

// The repacked layouts run the register-B and split-K kernels only (they
// have no LDS-tile decoder): K must give the register-B layout.
bool gemm_repacked_ok(int dtype, int64_t K) {
    return (dtype == QMM_Q6_K || dtype == QMM_Q8_0) && (K % (4 * BK)) == 0 && K * 4 * 128 < ((int64_t)1 << 31);
}

int gemm_repacked_kernel_choice(int dtype, int64_t M, int64_t K, int64_t N) {
    return dtype == QMM_Q6_K ? choice_dt<QMM_Q6_K_R>(M, K, N) : choice_dt<QMM_Q8_0_R>(M, K, N);
}

hipError_t launch_gemm_repacked(int dtype, const void *packed, int64_t M, int64_t K, int64_t N, const float *X,
                                float *Y, hipStream_t st) {
    if (!gemm_repacked_ok(dtype, K)) return hipErrorInvalidValue;
    const uint8_t *p = static_cast<const uint8_t *>(packed);
    return dtype == QMM_Q6_K ? launch_dt<QMM_Q6_K_R>(p, M, K, N, X, Y, st) : launch_dt<QMM_Q8_0_R>(p, M, K, N, X, Y, st);
}

// The gate/up projection with SwiGLU on the matrix cores: 4 wavefronts x 32
// output rows (64 decoded weight rows each) x 64 tokens.  Needs K a multiple
// of 256 with the register-B layout (gemm_swiglu_ok).
bool gemm_swiglu_ok(int dtype, int64_t K) {
    const int64_t bs = (dtype == QMM_Q4_K || dtype == QMM_Q5_K || dtype == QMM_Q6_K) ? 256 : 32;
    return aligned_layout(dtype, K / bs) && (K % (4 * BK)) == 0 && K * 4 * 128 < ((int64_t)1 << 31);
}

static int swiglu_choice() {
    static const int v = tuning_lever("QMM_SWIGLU_KERNEL", 0);
    return v;
}

// Tile of the SwiGLU form, measured on the 14336 x 4096 Q4_K gate/up pair
// (us; two plain GEMMs in brackets) and on 4096 x 4096:
//   1  4 wavefronts x 32 output rows x 32 tokens, both fragments per wavefront
//   2  the same with 64 tokens
//   3  the same with 128 tokens
//   4  8 wavefronts x 32 output rows x 64 tokens
//   5  the wavefront pair form: 8 wavefronts, 4 x 32 gate rows and the same
//      4 x 32 up rows, 128 tokens
//   N <= 64: 1 (N = 64: 51.6 vs 71.8).  4096 rows: 2 (N = 256: 58 vs 74 with
//   3, 69 with 5; N = 512: 64 vs 79 with 3, 74 with 5 (77)).  14336 rows:
//   N <= 128: 2 (N = 128: 67 vs 78 with 5 (78)); above, 5 where its
//   workgroups fill one round (112 x ceil(N/128) <= 256: N = 192 83 vs 101
//   with 2, 90 with 3 (116); N = 256 88 vs 93 with 3 (123)) or well over one
//   (N = 448 166 vs 194 with 2 (157); N = 512 171 vs 182 with 3 (162)), else 2
//   (N = 320 151 vs 155 with 5 (178); N = 384 158 vs 162 (186)).
// A measurement build (QMM_TUNING) takes QMM_SWIGLU_KERNEL = 1..5.
int swiglu_tile(int64_t M, int64_t N) {
    const int lever = swiglu_choice();
    if (lever >= 1 && lever <= 5) return lever;
    if (N <= 64) return 1;
    if (M >= 12288 && N > 128) {
        const int64_t t5 = ((M + 127) / 128) * ((N + 127) / 128);  // pair-form workgroups
        if (t5 <= 256 || t5 > 384) return 5;
    }
    return 2;
}

template <int DT>
static hipError_t launch_swiglu_dt(const uint8_t *g, const uint8_t *u, int64_t M, int64_t K, int64_t N,
                                   const float *X, float *Y, hipStream_t st) {
    switch (swiglu_tile(M, N)) {
    case 1: return launch_wb<DT, 64, 32, 2, 4, 0, 2, true, 2>(g, M, K, N, X, Y, st, u);
    case 2: return launch_wb<DT, 64, 64, 2, 4, 0, 2, true, 2>(g, M, K, N, X, Y, st, u);
    case 3: return launch_wb<DT, 64, 128, 2, 4, 4, 2, true, 2>(g, M, K, N, X, Y, st, u);
    case 5: return launch_wb<DT, 32, 128, 2, 8, 4, 2, true, 2>(g, M, K, N, X, Y, st, u);
    default: return launch_wb<DT, 64, 64, 2, 8, 0, 2, true, 2>(g, M, K, N, X, Y, st, u);
    }
}

hipError_t launch_gemm_swiglu(int dtype, const void *gate, const void *up, int64_t M, int64_t K, int64_t N,
                              const float *X, float *Y, hipStream_t st) {
    if (!gemm_swiglu_ok(dtype, K)) return hipErrorInvalidValue;
    const uint8_t *g = static_cast<const uint8_t *>(gate), *u = static_cast<const uint8_t *>(up);
    switch (dtype) {
    case QMM_Q4_0: return launch_swiglu_dt<QMM_Q4_0>(g, u, M, K, N, X, Y, st);
    case QMM_Q4_1: return launch_swiglu_dt<QMM_Q4_1>(g, u, M, K, N, X, Y, st);
    case QMM_Q8_0: return launch_swiglu_dt<QMM_Q8_0>(g, u, M, K, N, X, Y, st);
    case QMM_Q4_K: return launch_swiglu_dt<QMM_Q4_K>(g, u, M, K, N, X, Y, st);
    case QMM_Q5_K: return launch_swiglu_dt<QMM_Q5_K>(g, u, M, K, N, X, Y, st);
    case QMM_Q6_K: return launch_swiglu_dt<QMM_Q6_K>(g, u, M, K, N, X, Y, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm_mfma(int dtype, const void *blob_v, int64_t M, int64_t K, int64_t N, const float *X, float *Y,
                            hipStream_t st) {
    const uint8_t *blob = static_cast<const uint8_t *>(blob_v);
    switch (dtype) {
    case QMM_Q4_0: return launch_dt<QMM_Q4_0>(blob, M, K, N, X, Y, st);
    case QMM_Q4_1: return launch_dt<QMM_Q4_1>(blob, M, K, N, X, Y, st);
    case QMM_Q8_0: return launch_dt<QMM_Q8_0>(blob, M, K, N, X, Y, st);
    case QMM_Q4_K: return launch_dt<QMM_Q4_K>(blob, M, K, N, X, Y, st);
    case QMM_Q5_K: return launch_dt<QMM_Q5_K>(blob, M, K, N, X, Y, st);
    case QMM_Q6_K: return launch_dt<QMM_Q6_K>(blob, M, K, N, X, Y, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qmm
