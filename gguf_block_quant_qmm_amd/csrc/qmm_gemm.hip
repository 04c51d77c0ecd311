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

template <int DT>
static hipError_t launch_dt(const uint8_t *blob, int64_t M, int64_t K, int64_t N, const float *X, float *Y,
                            hipStream_t st) {
    const bool gen = !aligned_layout(DT, K / Geo<DT>::BS);
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
