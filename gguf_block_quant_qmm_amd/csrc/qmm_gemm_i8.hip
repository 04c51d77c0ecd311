// qmm_gemm_i8.hip -- the int8-activation matmul on the matrix cores,
//     Y[n][m] = sum_k W[m][k] * xs[n][k/32] * xq[n][k]
// for many tokens (page "cera 0.5.2 src/backend/cpu.rs": the int8 GEMMs over
// Q8_0-quantized activations, one integer dot per 32-element activation block,
// scaled once; the minimum term of the K-quants through the activation code
// sums).
//
// One v_mfma_i32_32x32x32_i8 contracts exactly one activation block (32 k)
// with one weight block of 32 tokens x 32 rows: the integer block sums are
// exact, and each is scaled once in f32 (the activation block's scale times
// the weight block's scale) and added to the output:
//   Q8_0  y += (d xs) * sum q c
//   Q4_0  y += (d xs) * sum (q - 8) c      (the -8 through a second matrix step
//                                          against a constant -8 operand: exact)
//   Q4_K  y += (d sc xs) * sum q c - (dmin m) * (xs * sum c)
// Each output accumulates its blocks in two levels (8 blocks, then the sums of
// 8), so an output of K = 16384 sees at most 72 f32 roundings of its terms:
// |err| <= ~80 * 2^-24 * Splus, inside 1e-5 * Splus (Splus = sum over k of
// (|w - o| + |o|) |xq|, o the weight's offset part).  The rounding order
// differs from the few-token kernels (one token's bits are not those of a
// single-token call on this path).
//
// Workgroup: 8 wavefronts x 32 weight rows x 64 tokens (two 32-token
// fragments per wavefront; the output sums of both levels stay in registers).  The activation codes of a 64-deep k-tile, their
// block scales and (Q4_K) scale x code sum are staged once per workgroup in
// LDS (double-buffered) and shared by the 8 wavefronts; the weight codes go
// straight from bounds-checked buffer loads into the matrix-core B registers.
#include "qmm_device.hpp"
#include "qmm_internal.hpp"

namespace qmm {

typedef int intx16 __attribute__((ext_vector_type(16)));
typedef int intx4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int BN8 = 64;       // tokens per workgroup
constexpr int W8 = 8;         // wavefronts, 32 rows each
constexpr int LDC = 80;       // LDS bytes per token row of codes (64 + 16 pad)

// Weight codes of one 64-deep k-tile for lane half kh: per block (2 per
// k-tile) 16 int8 codes (4 dwords) and the block's scale terms.
template <int DT> struct I8W;

template <> struct I8W<QMM_Q8_0> {
    // block pair kt: 68 bytes; block 0 codes at 2..34, block 1 codes at 36..68
    static constexpr int NW = 11;
    static constexpr bool OFF8 = false, MIN = false;
    struct State {};
    __device__ static void load(Rsrc rs, uint32_t roff, int kt, int kh, int, uint32_t (&r)[NW]) {
        const uint32_t base = 68u * (uint32_t)kt;
        uint32_t a[5], b[4], d0[1], d1[1];
        ldb(rs, roff + 16u * kh, base, a);          // bytes 16kh .. 16kh+20: block-0 codes at +2
        ldb(rs, roff + 16u * kh, base + 36u, b);    // block-1 codes 16kh .. +16
        ldb(rs, roff, base, d0);                    // d of block 0 (low half)
        ldb(rs, roff, base + 32u, d1);              // d of block 1 (high half)
#pragma unroll
        for (int i = 0; i < 5; i++) r[i] = a[i];
#pragma unroll
        for (int i = 0; i < 4; i++) r[5 + i] = b[i];
        r[9] = d0[0];
        r[10] = d1[0];
    }
    __device__ static void decode(const uint32_t (&r)[NW], State &, int, int, int blk, intx4 &c, float &s,
                                  float &mn) {
        if (blk == 0) {
#pragma unroll
            for (int i = 0; i < 4; i++) c[i] = (int)__builtin_amdgcn_alignbyte(r[i + 1], r[i], 2);
            s = h2f(r[9]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++) c[i] = (int)r[5 + i];
            s = h2f(r[10] >> 16);
        }
        mn = 0.f;
    }
};

template <> struct I8W<QMM_Q4_0> {
    // block pair kt: 36 bytes; block 0: d at 0, qs at 2..18; block 1: d at 18,
    // qs at 20..36.  Lane half 0 takes the low nibbles (k 0..15), half 1 the
    // high nibbles (k 16..31) of the block's 16 bytes.
    static constexpr int NW = 9;
    static constexpr bool OFF8 = true, MIN = false;
    struct State {};
    __device__ static void load(Rsrc rs, uint32_t roff, int kt, int, int, uint32_t (&r)[NW]) {
        ldb(rs, roff, 36u * (uint32_t)kt, r);
    }
    __device__ static void decode(const uint32_t (&r)[NW], State &, int kh, int, int blk, intx4 &c, float &s,
                                  float &mn) {
        const uint32_t sh = 4u * (uint32_t)kh;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t w = blk == 0 ? __builtin_amdgcn_alignbyte(r[i + 1], r[i], 2) : r[5 + i];
            c[i] = (int)((w >> sh) & 0x0F0F0F0Fu);
        }
        s = blk == 0 ? h2f(r[0]) : h2f(r[4] >> 16);
        mn = 0.f;
    }
};

template <> struct I8W<QMM_Q4_K> {
    // k-tile = chunk c of a super-block: block 0 = sub-block 2c (low nibbles of
    // qs[32c .. 32c+32)), block 1 = sub-block 2c+1 (high nibbles); lane half kh
    // takes bytes 16kh .. 16kh+16 of the chunk.  The header (d, dmin, the 12
    // scale bytes) comes with chunk 0 and is kept in State for the four chunks.
    static constexpr int NW = 8;
    static constexpr bool OFF8 = false, MIN = true;
    struct State { uint32_t h[4]; };
    __device__ static void load(Rsrc rs, uint32_t roff, int kt, int kh, int c, uint32_t (&r)[NW]) {
        const uint32_t sb = 144u * (uint32_t)(kt >> 2);
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
    __device__ static void decode(const uint32_t (&r)[NW], State &st, int, int c, int blk, intx4 &cd, float &s,
                                  float &mn) {
        if (c == 0 && blk == 0) {
#pragma unroll
            for (int i = 0; i < 4; i++) st.h[i] = r[i];
        }
        const uint32_t sh = 4u * (uint32_t)blk;
#pragma unroll
        for (int i = 0; i < 4; i++) cd[i] = (int)((r[4 + i] >> sh) & 0x0F0F0F0Fu);
        int sc, m;
        q4k_scale_min(st.h[1], st.h[2], st.h[3], 2 * c + blk, sc, m);
        s = h2f(st.h[0]) * (float)sc;           // exact: an f16 times a 6-bit integer
        mn = h2f(st.h[0] >> 16) * (float)m;     // exact likewise
    }
};

template <int DT>
__global__ void __launch_bounds__(64 * W8, 2) gemm_i8_kernel(const uint8_t *__restrict__ blob, int64_t M, int64_t K,
                                                             int64_t N, int64_t row_bytes,
                                                             const int8_t *__restrict__ xq,
                                                             const float *__restrict__ xsc, float *__restrict__ Y,
                                                             int n_mtiles, int n_ntiles) {
    using WD = I8W<DT>;
    constexpr int FN = BN8 / 32;
    __shared__ __attribute__((aligned(16))) uint8_t cs[2][BN8 * LDC];  // codes, token-major
    __shared__ __attribute__((aligned(16))) float ss[2][2][BN8];       // [buf][block][token] scale
    __shared__ __attribute__((aligned(16))) float qs[2][2][BN8];       // [buf][block][token] scale x code sum

    const int t = threadIdx.x, lane = t & 63, kh = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int total = n_mtiles * n_ntiles, b = blockIdx.x, xcd = b & 7, local = b >> 3;
    const int tile = xcd * (total >> 3) + (xcd < (total & 7) ? xcd : (total & 7)) + local;
    const int64_t mt = tile / n_ntiles, nt = tile % n_ntiles;
    const int64_t n0 = nt * BN8, mw = mt * (W8 * 32) + wave * 32;
    const int nkt = (int)(K / 64);

    const int64_t wrows = M - mw < 0 ? 0 : (M - mw < 32 ? M - mw : 32);
    const Rsrc wrs = make_rsrc_uniform(blob + (wrows ? mw : 0) * row_bytes, (uint32_t)(wrows * row_bytes));
    const uint32_t roff = (uint32_t)((lane & 31) * row_bytes);
    // staging: thread t < 2 BN8 moves token t >> 1, block t & 1 of every k-tile
    const int64_t xrows = N - n0 < BN8 ? N - n0 : BN8;
    const Rsrc qrs = make_rsrc_uniform(xq + n0 * K, (uint32_t)(xrows * K));
    const Rsrc srs = make_rsrc_uniform(xsc + n0 * (K / 32), (uint32_t)(xrows * (K / 32) * 4));
    const int sr = (t >> 1) & (BN8 - 1), sb = t & 1;
    const bool stager = t < 2 * BN8;
    const uint32_t qoff = (uint32_t)(sr * K + 32 * sb), soff = (uint32_t)((sr * (K / 32) + sb) * 4);

    u32x4_t xr[2];
    float xsr = 0.f;
    auto xload = [&](int kt) {
        if (!stager) return;  // wave-uniform: the first 2 BN8 / 64 wavefronts stage
        const int kc = kt < nkt ? kt : nkt - 1;
        xr[0] = __builtin_amdgcn_raw_buffer_load_b128(qrs, qoff, (uint32_t)(64 * kc), 0);
        xr[1] = __builtin_amdgcn_raw_buffer_load_b128(qrs, qoff + 16u, (uint32_t)(64 * kc), 0);
        xsr = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, soff, (uint32_t)(8 * kc), 0));
    };
    auto xstore = [&](int buf) {
        if (stager) {
            u32x4_t *dst = reinterpret_cast<u32x4_t *>(&cs[buf][sr * LDC + 32 * sb]);
            dst[0] = xr[0];
            dst[1] = xr[1];
            ss[buf][sb][sr] = xsr;
            if constexpr (WD::MIN) {
                int sum = 0;
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    sum = __builtin_amdgcn_sdot4((int)xr[h].x, 0x01010101, sum, false);
                    sum = __builtin_amdgcn_sdot4((int)xr[h].y, 0x01010101, sum, false);
                    sum = __builtin_amdgcn_sdot4((int)xr[h].z, 0x01010101, sum, false);
                    sum = __builtin_amdgcn_sdot4((int)xr[h].w, 0x01010101, sum, false);
                }
                qs[buf][sb][sr] = xsr * (float)sum;
            }
        }
    };

    uint32_t wr[2][WD::NW];
    typename WD::State st;
    float y[FN][16], yt[FN][16];
#pragma unroll
    for (int i = 0; i < FN; i++)
#pragma unroll
        for (int v = 0; v < 16; v++) y[i][v] = yt[i][v] = 0.f;
    const intx4 neg8 = {(int)0xF8F8F8F8u, (int)0xF8F8F8F8u, (int)0xF8F8F8F8u, (int)0xF8F8F8F8u};
    const intx16 zero16 = {};

    WD::load(wrs, roff, 0, kh, 0, wr[0]);
    xload(0);
    xstore(0);
    xload(1);
    __syncthreads();

    for (int kt = 0; kt < nkt; kt++) {
        const int c = kt & 3, buf = kt & 1;
        // the next k-tile's weights (clamped past the end: never used)
        WD::load(wrs, roff, kt + 1 < nkt ? kt + 1 : kt, kh, (kt + 1 < nkt ? kt + 1 : kt) & 3, wr[(kt + 1) & 1]);
#pragma unroll
        for (int blk = 0; blk < 2; blk++) {
            intx4 bq;
            float s, mn;
            WD::decode(wr[kt & 1], st, kh, c, blk, bq, s, mn);
#pragma unroll
            for (int i = 0; i < FN; i++) {
                const int tr = 32 * i + (lane & 31);
                const intx4 a = *reinterpret_cast<const intx4 *>(&cs[buf][tr * LDC + 32 * blk + 16 * kh]);
                intx16 acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bq, zero16, 0, 0, 0);
                if constexpr (WD::OFF8) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, neg8, acc, 0, 0, 0);
                // this lane's tokens: 32 i + 8 g + 4 kh + r, r = 0..3 (output v = 4 g + r)
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    const floatx4 sx = *reinterpret_cast<const floatx4 *>(&ss[buf][blk][32 * i + 8 * g + 4 * kh]);
                    floatx4 qx = {0.f, 0.f, 0.f, 0.f};
                    if constexpr (WD::MIN) qx = *reinterpret_cast<const floatx4 *>(&qs[buf][blk][32 * i + 8 * g + 4 * kh]);
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        const int v = 4 * g + r;
                        float term = (float)acc[v] * (s * sx[r]);
                        if constexpr (WD::MIN) term = fmaf(-mn, qx[r], term);
                        yt[i][v] += term;
                    }
                }
            }
        }
        // the second level: every 4 k-tiles (8 blocks) into the output sums
        if (c == 3 || kt == nkt - 1) {
#pragma unroll
            for (int i = 0; i < FN; i++)
#pragma unroll
                for (int v = 0; v < 16; v++) {
                    y[i][v] += yt[i][v];
                    yt[i][v] = 0.f;
                }
        }
        if (kt + 1 < nkt) {
            xstore(buf ^ 1);
            xload(kt + 2);
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < FN; i++) {
        const int64_t m = mw + (lane & 31);
        if (m >= M) continue;
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int64_t n = n0 + 32 * i + 8 * (v >> 2) + 4 * kh + (v & 3);
            if (n < N) Y[n * M + m] = y[i][v];
        }
    }
}

template <int DT>
hipError_t launch_i8(const uint8_t *blob, int64_t M, int64_t K, int64_t N, const int8_t *xq, const float *xsc,
                     float *Y, hipStream_t st) {
    constexpr int BS = Geo<DT>::BS, BB = Geo<DT>::BB;
    const int64_t row_bytes = (K / BS) * BB;
    const int64_t mtiles = (M + W8 * 32 - 1) / (W8 * 32), ntiles = (N + BN8 - 1) / BN8;
    const int64_t grid = mtiles * ntiles;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gemm_i8_kernel<DT>), dim3((unsigned)grid), dim3(64 * W8), 0, st, blob, M, K, N, row_bytes,
                       xq, xsc, Y, (int)mtiles, (int)ntiles);
    return hipGetLastError();
}

}  // namespace

bool gemm_i8_ok(int dtype, int64_t M, int64_t K, int64_t N) {
    // the matrix-core int8 kernel: Q8_0, Q4_0 (an even block count: K a
    // multiple of 64) and Q4_K; K up to 16384 (the two-level sum's bound) and
    // resources of 128 token rows of codes and scales under 2^31 bytes
    if (K % 64 != 0 || K > 16384 || M < 1 || N < 1) return false;
    return dtype == QMM_Q8_0 || dtype == QMM_Q4_0 || (dtype == QMM_Q4_K && K % 256 == 0);
}

hipError_t launch_gemm_q8act_mfma(int dtype, const void *blob_v, int64_t M, int64_t K, int64_t N, const float *xsc,
                                  const int8_t *xq, float *Y, hipStream_t st) {
    if (!gemm_i8_ok(dtype, M, K, N)) return hipErrorInvalidValue;
    const uint8_t *blob = static_cast<const uint8_t *>(blob_v);
    switch (dtype) {
    case QMM_Q8_0: return launch_i8<QMM_Q8_0>(blob, M, K, N, xq, xsc, Y, st);
    case QMM_Q4_0: return launch_i8<QMM_Q4_0>(blob, M, K, N, xq, xsc, Y, st);
    case QMM_Q4_K: return launch_i8<QMM_Q4_K>(blob, M, K, N, xq, xsc, Y, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qmm
