// lowrank_factor.hip - rank-32 truncated SVD of cache matrices (gfx950).
//
// KVCMAS, "what differs": the base caches and delta corrections an anchor
// stores are kept as truncated SVDs, Z ~ U_r S_r R_r^T, with A = U_r S_r
// (T x r) and R = R_r (D x r); r = 32 by default. The page does not say how
// the truncated SVD is computed. Here it is the randomized range finder of
// Halko, Martinsson and Tropp ("Finding structure with randomness", 2011:
// Gaussian sketch, power iteration, Rayleigh-Ritz on the small projected
// matrix), with a Gaussian test matrix Omega (D x 48) supplied by the caller
// (rank 32 plus 16 oversampling columns) and one power iteration:
//
//   Y = Z Omega;  Q = orth(Y);  W = orth(Z^T Q);  Y = Z W;  Q = orth(Y)
//   W = Z^T Q (= B^T, B = Q^T Z);  C = W^T W = U Lambda U^T (Jacobi)
//   A = Q U_r Lambda_r^(1/2),  R = W U_r Lambda_r^(-1/2)
//
// orth() is CholeskyQR (Gram matrix and Cholesky factor in binary64, a
// pivot at or below 1e-12 of the largest diagonal drops its column), once
// inside the power iteration and twice for the final Q; the products with Z
// run on the matrix cores (Z is bf16; the binary32 operand enters as two
// bf16 parts, binary32 accumulation), and the 48 x 48 eigenproblem is
// solved by parallel cyclic Jacobi in binary64. A and R are rounded once to
// bf16.
//
// Z is a matrix view of the cache layout: row t, column h*d + c of matrix m
// is element [m][h][t][c] of a bf16 [M][H][T][d] tensor.
#include "kernels_common.h"
#include "launch.h"

namespace kvc {
namespace {

constexpr int kFK = kLowrankSketch;  // 48 sketch columns
constexpr int kFR = 32;              // rank
constexpr int kFChunk = 1024;        // tokens per partial product of Z^T Q
constexpr int kFThreads = 256;
constexpr int kFSweeps = 16;         // Jacobi sweep limit
// The small eigenproblem's workgroup: a Jacobi step is a chain of two
// barriers and 1728 independent updates (576 2 x 2 blocks of A, 1152 rows of
// V), so more threads shorten every step of the chain; its 32 workgroups do
// not fill the chip in any case.
constexpr int kSvdThreads = 1024;

typedef __bf16 fbf16x8 __attribute__((ext_vector_type(8)));
typedef float ff32x4 __attribute__((ext_vector_type(4)));

// A binary32 operand of the matrix-core products as two bf16 parts: hi =
// bf16(x) (nearest, ties to even) and lo = bf16(x - hi) (x - hi is exact),
// so hi + lo is within 2^-17 |x| of x; a product Z (hi + lo) is two matrix
// instructions accumulating in binary32. Z itself is bf16 and exact.
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
    hi = (__bf16)x;
    lo = (__bf16)(x - (float)hi);
}

__device__ __forceinline__ ff32x4 mfma_bf16(const uint4& a, const uint4& b, ff32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(fbf16x8, a), __builtin_bit_cast(fbf16x8, b), c,
                                                   0, 0, 0);
}

// v_mfma_f32_16x16x32_bf16 operand layout: lane l supplies row l % 16 of A
// and column l % 16 of B, each with k = 8 (l / 16) .. 8 (l / 16) + 7, and
// receives rows 4 (l / 16) .. 4 (l / 16) + 3 of column l % 16 of the result.

// Y[m](t, :) = Z[m](t, :) X[m] on the matrix cores; X is D x 48 row-major
// binary32, x_stride elements apart per matrix (0: one X for all). Block:
// 256 tokens, wave w rows 64 w .. 64 w + 63 (four 16-row tiles) by all 48
// columns (three tiles). The contraction runs over the channels, which are
// contiguous in Z: A fragments are 16-byte loads straight from memory. The
// rows of X for one head pass through LDS as bf16 B fragments (hi and lo).
template <int D>
__global__ __launch_bounds__(kFThreads) void fac_zx_kernel(const uint16_t* z, const float* x, uint64_t x_stride,
                                                           float* y, uint32_t H, uint32_t T) {
    constexpr int KS = D / 32;  // k-steps per head
    __shared__ uint4 xb[2][KS][3][kWave];
    const uint32_t m = blockIdx.y;
    const uint32_t lane = lane_id(), w = wave_uniform(threadIdx.x / kWave);
    const uint32_t tb = blockIdx.x * 256 + w * 64;
    const uint16_t* zm = z + (uint64_t)m * H * T * D;
    const float* xm = x + (uint64_t)m * x_stride;
    ff32x4 acc[4][3];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < 3; ++ct) acc[rt][ct] = ff32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // this lane's A fragments of head h: rows tb + 16 rt + lane % 16
    // (clamped to the last token), channels 32 ks + 8 (lane / 16) ..
    auto load_a = [&](uint32_t h, uint4 (&a)[KS][4]) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                uint32_t t = tb + rt * 16 + lane % 16;
                t = t < T ? t : T - 1;
                a[ks][rt] = *reinterpret_cast<const uint4*>(zm + ((uint64_t)h * T + t) * D + ks * 32 + 8 * (lane / 16));
            }
    };
    uint4 a[KS][4], an[KS][4];
    load_a(0, an);
    for (uint32_t h = 0; h < H; ++h) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) a[ks][rt] = an[ks][rt];
        __syncthreads();
        for (uint32_t f = threadIdx.x; f < (uint32_t)KS * 3 * kWave; f += kFThreads) {
            const uint32_t ks = f / (3 * kWave), ct = (f / kWave) % 3, l = f % kWave;
            const float* xr = xm + ((uint64_t)h * D + ks * 32 + 8 * (l / 16)) * kFK + ct * 16 + l % 16;
            __bf16 hi[8], lo[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) split_bf16(xr[i * kFK], hi[i], lo[i]);
            xb[0][ks][ct][l] = __builtin_bit_cast(uint4, hi);
            xb[1][ks][ct][l] = __builtin_bit_cast(uint4, lo);
        }
        __syncthreads();
        if (h + 1 < H) load_a(h + 1, an);  // the next head's rows, in flight during this head's products
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 bh[3], bl[3];
#pragma unroll
            for (int ct = 0; ct < 3; ++ct) {
                bh[ct] = xb[0][ks][ct][lane];
                bl[ct] = xb[1][ks][ct][lane];
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int ct = 0; ct < 3; ++ct) {
                    acc[rt][ct] = mfma_bf16(a[ks][rt], bh[ct], acc[rt][ct]);
                    acc[rt][ct] = mfma_bf16(a[ks][rt], bl[ct], acc[rt][ct]);
                }
        }
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t t = tb + rt * 16 + 4 * (lane / 16) + e;
            if (t < T) {
                float* yr = y + ((uint64_t)m * T + t) * kFK + lane % 16;
#pragma unroll
                for (int ct = 0; ct < 3; ++ct) yr[ct * 16] = acc[rt][ct][e];
            }
        }
}

// Partial products P[m][chunk](h*d + c, :) = sum over the chunk's tokens t
// of Z[m](t, h*d + c) Q[m](t, :), on the matrix cores. The contraction runs
// over tokens, which are not contiguous in Z: a 128-token tile of the head
// is staged in LDS as it lies ([t][c], coalesced) and each lane gathers its
// A fragment (8 tokens of one channel) with 2-byte reads; the tile's rows of
// Q pass through LDS as bf16 B fragments (hi and lo). Block: one chunk of
// tokens of one head; wave w owns channel tiles w * D/64 .. of the head.
constexpr int kZtqSub = 128;
template <int D>
__global__ __launch_bounds__(kFThreads) void fac_ztq_kernel(const uint16_t* z, const float* q, float* part,
                                                            uint32_t H, uint32_t T, uint32_t nchunks) {
    constexpr int CTW = D / 64;          // channel tiles per wave: 2 (d = 128) or 1 (d = 64)
    constexpr int KS = kZtqSub / 32;     // k-steps per sub-tile
    constexpr int ZR = D + 8;            // LDS row of the Z tile, in bf16 (16-byte multiple, spreads banks)
    __shared__ __attribute__((aligned(16))) uint16_t zs[kZtqSub * ZR];
    __shared__ uint4 qb[2][KS][3][kWave];
    const uint32_t chunk = blockIdx.x, h = blockIdx.y % H, m = blockIdx.y / H;
    const uint32_t lane = lane_id(), w = wave_uniform(threadIdx.x / kWave);
    const uint32_t tbeg = chunk * kFChunk;
    const uint32_t tend = (T - tbeg < (uint32_t)kFChunk) ? T : tbeg + kFChunk;
    const uint16_t* zh = z + ((uint64_t)m * H + h) * T * D;
    const float* qm = q + (uint64_t)m * T * kFK;
    ff32x4 acc[CTW][3];
#pragma unroll
    for (int c = 0; c < CTW; ++c)
#pragma unroll
        for (int jt = 0; jt < 3; ++jt) acc[c][jt] = ff32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // A sub-tile's share of each thread: ZN 16-byte pieces of the Z tile
    // (piece i = threadIdx.x + 256 n: row i / (D/8), 8 channels) and QN
    // B fragments' 8 values of Q (fragment f = threadIdx.x + 256 n), loaded
    // into registers one sub-tile ahead, then placed in LDS.
    constexpr int ZN = kZtqSub * D / 8 / kFThreads;
    constexpr int QN = KS * 3 * kWave / kFThreads;
    uint4 zr[ZN];
    float qv[QN][8];
    auto load_tile = [&](uint32_t t0) {
        const uint32_t nt = (tend - t0 < (uint32_t)kZtqSub) ? tend - t0 : (uint32_t)kZtqSub;
#pragma unroll
        for (int n = 0; n < ZN; ++n) {
            const uint32_t i = threadIdx.x + n * kFThreads, r = i / (D / 8), c8 = i % (D / 8);
            zr[n] = r < nt ? *reinterpret_cast<const uint4*>(zh + (uint64_t)(t0 + r) * D + c8 * 8)
                           : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int n = 0; n < QN; ++n) {
            const uint32_t f = threadIdx.x + n * kFThreads;
            const uint32_t ks = f / (3 * kWave), jt = (f / kWave) % 3, l = f % kWave;
            const uint32_t tr = ks * 32 + 8 * (l / 16);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                qv[n][i] = tr + i < nt ? qm[(uint64_t)(t0 + tr + i) * kFK + jt * 16 + l % 16] : 0.0f;
        }
    };
    load_tile(tbeg);
    for (uint32_t t0 = tbeg; t0 < tend; t0 += kZtqSub) {
        __syncthreads();  // the previous sub-tile's LDS reads are done
#pragma unroll
        for (int n = 0; n < ZN; ++n) {
            const uint32_t i = threadIdx.x + n * kFThreads, r = i / (D / 8), c8 = i % (D / 8);
            *reinterpret_cast<uint4*>(zs + r * ZR + c8 * 8) = zr[n];
        }
#pragma unroll
        for (int n = 0; n < QN; ++n) {
            const uint32_t f = threadIdx.x + n * kFThreads;
            const uint32_t ks = f / (3 * kWave), jt = (f / kWave) % 3, l = f % kWave;
            __bf16 hi[8], lo[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) split_bf16(qv[n][i], hi[i], lo[i]);
            qb[0][ks][jt][l] = __builtin_bit_cast(uint4, hi);
            qb[1][ks][jt][l] = __builtin_bit_cast(uint4, lo);
        }
        __syncthreads();
        if (t0 + kZtqSub < tend) load_tile(t0 + kZtqSub);  // in flight during this sub-tile's products
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 bh[3], bl[3];
#pragma unroll
            for (int jt = 0; jt < 3; ++jt) {
                bh[jt] = qb[0][ks][jt][lane];
                bl[jt] = qb[1][ks][jt][lane];
            }
#pragma unroll
            for (int c = 0; c < CTW; ++c) {
                const uint32_t ch = (w * CTW + c) * 16 + lane % 16;
                const uint16_t* col = zs + (ks * 32 + 8 * (lane / 16)) * ZR + ch;
                uint16_t av[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) av[i] = col[i * ZR];
                const uint4 a = __builtin_bit_cast(uint4, av);
#pragma unroll
                for (int jt = 0; jt < 3; ++jt) {
                    acc[c][jt] = mfma_bf16(a, bh[jt], acc[c][jt]);
                    acc[c][jt] = mfma_bf16(a, bl[jt], acc[c][jt]);
                }
            }
        }
    }
    float* pm = part + (((uint64_t)m * nchunks + chunk) * H + h) * (uint64_t)D * kFK;
#pragma unroll
    for (int c = 0; c < CTW; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t ch = (w * CTW + c) * 16 + 4 * (lane / 16) + e;
#pragma unroll
            for (int jt = 0; jt < 3; ++jt) pm[(uint64_t)ch * kFK + jt * 16 + lane % 16] = acc[c][jt][e];
        }
}

// W[m] = sum over chunks of P[m][chunk], chunks in order.
__global__ __launch_bounds__(kFThreads) void fac_reduce_kernel(const float* part, float* w, uint32_t M,
                                                               uint64_t per_matrix, uint32_t nchunks) {
    const uint64_t i = (uint64_t)blockIdx.x * kFThreads + threadIdx.x;
    if (i >= (uint64_t)M * per_matrix) return;
    const uint64_t m = i / per_matrix, e = i % per_matrix;
    const float* p = part + m * nchunks * per_matrix + e;
    float s = 0.0f;
    for (uint32_t c = 0; c < nchunks; ++c) s += p[(uint64_t)c * per_matrix];
    w[i] = s;
}

// Partial Gram matrices: Gp[m][chunk] = Y_chunk^T Y_chunk (48 x 48,
// binary64) over chunks of kGChunk rows, one block per (chunk, matrix), on
// the matrix cores in binary64 (v_mfma_f64_16x16x4_f64: lane l supplies
// A(l % 16, l / 16) and B(l / 16, l % 16), one double each, and its result
// entry e is row l / 16 + 4 e of column l % 16 - measured on the GPU with a
// probe whose entries encode their own row and column). With
// A = Y^T and B = Y both operands of a k-step are 4 rows of Y, lane l
// reading 16 consecutive columns of row l / 16; the six tiles (a, b), a <= b,
// of the 3 x 3 tiling are accumulated. Wave w takes the k-steps of rows
// 4 w + 16 s .. + 3; the four waves' sums are added in LDS, in wave order,
// and the block writes the full symmetric matrix.
constexpr int kGChunk = 256;

typedef double fd4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kFThreads) void fac_gram_partial_kernel(const float* y, uint32_t N, uint32_t nchunks,
                                                                     double* gpart) {
    __shared__ double red[kFThreads / kWave][6][kWave][4];
    const uint32_t chunk = blockIdx.x, m = blockIdx.y;
    const uint32_t lane = lane_id(), w = wave_uniform(threadIdx.x / kWave);
    const uint32_t cbeg = chunk * kGChunk;
    const uint32_t cend = (N - cbeg < (uint32_t)kGChunk) ? N : cbeg + kGChunk;
    const float* ym = y + (uint64_t)m * N * kFK;
    fd4 acc[6];
#pragma unroll
    for (int t = 0; t < 6; ++t) acc[t] = fd4{0.0, 0.0, 0.0, 0.0};
    // k-steps of 4 rows, wave w every fourth (16 steps of a 256-row chunk);
    // all of a wave's values loaded at once, then its matrix instructions
    constexpr int kSteps = kGChunk / 16;
    float v[kSteps][3];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        const uint32_t row = cbeg + 4 * w + 16 * s + lane / 16;
#pragma unroll
        for (int c = 0; c < 3; ++c) v[s][c] = row < cend ? ym[(uint64_t)row * kFK + 16 * c + lane % 16] : 0.0f;
    }
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        int t = 0;
#pragma unroll
        for (int a = 0; a < 3; ++a)
#pragma unroll
            for (int b = a; b < 3; ++b, ++t)
                acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)v[s][a], (double)v[s][b], acc[t], 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < 6; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[w][t][lane][e] = acc[t][e];
    __syncthreads();
    double* out = gpart + ((uint64_t)m * nchunks + chunk) * kFK * kFK;
    // thread -> (tile t, lane l, entry e): 6 x 64 x 4 = 1536 sums of 4 waves
    for (uint32_t k = threadIdx.x; k < 6u * kWave * 4u; k += kFThreads) {
        const uint32_t t = k / (kWave * 4), l = (k / 4) % kWave, e = k % 4;
        double sum = 0.0;
#pragma unroll
        for (int ww = 0; ww < kFThreads / kWave; ++ww) sum += red[ww][t][l][e];
        const uint32_t a = t < 3 ? 0u : (t < 5 ? 1u : 2u);
        const uint32_t b = t < 3 ? t : (t < 5 ? t - 2 : 2u);
        const uint32_t i = 16 * a + l / 16 + 4 * e, jj = 16 * b + l % 16;
        // in a diagonal tile (i, j) and (j, i) are separate sums: the upper
        // one is written to both places (one writer per address)
        if (i <= jj) {
            out[i * kFK + jj] = sum;
            out[jj * kFK + i] = sum;
        }
    }
}

// g = sum of the chunks' partial Gram matrices, chunks in order
template <int NT>
__device__ __forceinline__ void sum_gram(const double* gpart, uint32_t m, uint32_t nchunks, double* g) {
    const double* gp = gpart + (uint64_t)m * nchunks * kFK * kFK;
    // a thread's elements side by side, chunk after chunk: each element is
    // still summed in chunk order, while the loads of several chunks and
    // elements are in flight together
    constexpr int kPer = (kFK * kFK + NT - 1) / NT;
    double acc[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) acc[e] = 0.0;
#pragma unroll 4
    for (uint32_t c = 0; c < nchunks; ++c) {
        const double* gc = gp + (uint64_t)c * kFK * kFK;
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const uint32_t i = threadIdx.x + (uint32_t)e * NT;
            if (i < (uint32_t)(kFK * kFK)) acc[e] += gc[i];
        }
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        const uint32_t i = threadIdx.x + (uint32_t)e * NT;
        if (i < (uint32_t)(kFK * kFK)) g[i] = acc[e];
    }
    __syncthreads();
}

// Broadcast of lane `src`'s binary64 value to the wave (two readlanes).
__device__ __forceinline__ double bcast_f64(double v, uint32_t src) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, (int)src);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), (int)src);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// One CholeskyQR step, factor part: G = Y^T Y = L L^T, then Rinv = (L^T)^-1
// (upper triangular), binary64. A pivot at or below 1e-12 of the largest
// diagonal entry drops its column: its row and column of Rinv are zero.
// After the block sums the partial Gram matrices, one wave does both parts
// in registers, lane i holding row i (48 binary64), fully unrolled so that
// every register index is a constant: right-looking, column j of L is the
// pivot column scaled by 1/sqrt(pivot) and the trailing rows lose its outer
// product, the entries of column j reaching the other lanes by readlane;
// then M = L^-1 (Rinv = M^T) row by row, row k final once divided by
// L[k][k], the rows below updated with it. No barrier inside either part.
__global__ __launch_bounds__(kFThreads) void fac_chol_kernel(const double* gpart, uint32_t nchunks, double* rinv) {
    __shared__ double g[kFK * kFK];
    const uint32_t m = blockIdx.x;
    sum_gram<kFThreads>(gpart, m, nchunks, g);
    if (threadIdx.x >= (uint32_t)kWave) return;  // no barrier follows
    const uint32_t lane = threadIdx.x;
    const uint32_t row = lane < (uint32_t)kFK ? lane : 0u;
    double maxdiag = 0.0;
    for (int k = 0; k < kFK; ++k) maxdiag = fmax(maxdiag, g[k * kFK + k]);
    const double tol = 1e-12 * maxdiag;
    double a[kFK];  // row `row` of G, then of L (lower part; the rest stays unused)
#pragma unroll
    for (int k = 0; k < kFK; ++k) a[k] = g[row * kFK + k];
    double diag[kFK];  // L[j][j], uniform
#pragma unroll
    for (int j = 0; j < kFK; ++j) {
        const double s = bcast_f64(a[j], j);  // the pivot, updated by columns 0 .. j-1
        const bool keep = s > tol;
        const double ljj = keep ? sqrt(s) : 0.0;
        diag[j] = ljj;
        // this lane's entry of column j (rows below j), then its trailing
        // row; lanes at or above j carry lij = 0, and what they change above
        // their diagonal is never read
        const double rj = keep ? 1.0 / ljj : 0.0;
        const double lij = lane > (uint32_t)j ? a[j] * rj : 0.0;
        a[j] = lane == (uint32_t)j ? ljj : lij;
#pragma unroll
        for (int k = j + 1; k < kFK; ++k) a[k] = fma(-lij, bcast_f64(lij, k), a[k]);
    }
    // M = L^-1: lane r holds row r of M (b) and of L (a)
    double b[kFK];
#pragma unroll
    for (int c = 0; c < kFK; ++c) b[c] = (row == (uint32_t)c) ? 1.0 : 0.0;
#pragma unroll
    for (int k = 0; k < kFK; ++k) {
        const double rk = diag[k] != 0.0 ? 1.0 / diag[k] : 0.0;
        const double sk = lane == (uint32_t)k ? rk : 1.0;
#pragma unroll
        for (int c = 0; c <= k; ++c) b[c] *= sk;
        const double lrk = lane > (uint32_t)k ? a[k] : 0.0;
#pragma unroll
        for (int c = 0; c <= k; ++c) b[c] = fma(-lrk, bcast_f64(b[c], k), b[c]);
    }
    // Rinv(r, c) = M(c, r): lane c holds row c of M, i.e. column c of Rinv
    double* out = rinv + (uint64_t)m * kFK * kFK;
    if (lane < (uint32_t)kFK) {
#pragma unroll
        for (int r = 0; r < kFK; ++r) out[r * kFK + lane] = (uint32_t)r <= lane ? b[r] : 0.0;
    }
}

// Y <- Y Rinv (rows independent, in place), binary64 sums.
__global__ __launch_bounds__(kFThreads) void fac_apply_rinv_kernel(float* y, uint32_t N, const double* rinv) {
    __shared__ double r[kFK * kFK];
    const uint32_t m = blockIdx.y;
    const double* rm = rinv + (uint64_t)m * kFK * kFK;
    for (uint32_t i = threadIdx.x; i < kFK * kFK; i += kFThreads) r[i] = rm[i];
    __syncthreads();
    const uint32_t n = blockIdx.x * kFThreads + threadIdx.x;
    if (n >= N) return;
    float4* yr = reinterpret_cast<float4*>(y + ((uint64_t)m * N + n) * kFK);
    float v[kFK];
#pragma unroll
    for (int q = 0; q < kFK / 4; ++q) {
        const float4 t = yr[q];
        v[4 * q] = t.x;
        v[4 * q + 1] = t.y;
        v[4 * q + 2] = t.z;
        v[4 * q + 3] = t.w;
    }
    float o[kFK];
#pragma unroll
    for (int j = 0; j < kFK; ++j) {
        double s = 0.0;
#pragma unroll
        for (int i = 0; i <= j; ++i) s = fma((double)v[i], r[i * kFK + j], s);
        o[j] = (float)s;
    }
#pragma unroll
    for (int q = 0; q < kFK / 4; ++q) yr[q] = make_float4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
}

// C = W^T W (from its partial Gram matrices), eigenpairs by parallel cyclic
// Jacobi (round-robin pairing: 24 disjoint rotations per step, 47 steps per
// sweep; each thread applies both sides of the rotations to whole 2 x 2
// blocks, so a step is one pass), binary64, until the off-diagonal part is
// below 1e-9 of the diagonal (in norm); writes ua = U_r diag(sigma),
// ur = U_r diag(1/sigma) (0 where sigma = 0), both 48 x 32 binary32, and
// sigma (descending).
__global__ __launch_bounds__(kSvdThreads) void fac_small_svd_kernel(const double* gpart, uint32_t nchunks, float* ua,
                                                                  float* ur, float* sigma) {
    __shared__ double a[kFK * kFK];
    __shared__ double v[kFK * kFK];
    __shared__ double rc[kFK / 2], rs[kFK / 2];
    __shared__ uint32_t rp[kFK / 2], rq[kFK / 2];
    __shared__ double red[2][kSvdThreads / kWave];
    __shared__ uint32_t order[kFK];
    const uint32_t m = blockIdx.x;
    sum_gram<kSvdThreads>(gpart, m, nchunks, a);
    for (uint32_t i = threadIdx.x; i < kFK * kFK; i += kSvdThreads) v[i] = (i / kFK == i % kFK) ? 1.0 : 0.0;
    __syncthreads();
    for (int sweep = 0; sweep < kFSweeps; ++sweep) {
        double off = 0.0, dia = 0.0;
        for (uint32_t i = threadIdx.x; i < kFK * kFK; i += kSvdThreads) {
            const double x = a[i];
            if (i / kFK == i % kFK) dia += x * x;
            else off += x * x;
        }
        for (int o = 32; o > 0; o >>= 1) {
            off += __shfl_xor(off, o);
            dia += __shfl_xor(dia, o);
        }
        if (threadIdx.x % kWave == 0) {
            red[0][threadIdx.x / kWave] = off;
            red[1][threadIdx.x / kWave] = dia;
        }
        __syncthreads();
        double so = 0.0, sd = 0.0;
        for (int k = 0; k < kSvdThreads / kWave; ++k) {
            so += red[0][k];
            sd += red[1][k];
        }
        __syncthreads();  // red is rewritten at the next sweep
        // off-diagonal norm below 1e-9 of the diagonal's: the eigenvalues
        // are then exact to about 1e-14 relative of the largest, the vectors
        // to far better than the bf16 factors keep
        if (so <= 1e-18 * sd) break;  // every thread takes the same branch
        for (uint32_t step = 0; step < (uint32_t)kFK - 1; ++step) {
            // pairs: position 0 holds index 0, positions 1..47 rotate
            if (threadIdx.x < (uint32_t)kFK / 2) {
                const uint32_t i = threadIdx.x;
                const uint32_t pa = i, pb = kFK - 1 - i;
                uint32_t p = pa == 0 ? 0u : 1u + (pa - 1 + step) % (kFK - 1);
                uint32_t q = 1u + (pb - 1 + step) % (kFK - 1);
                if (p > q) {
                    const uint32_t t = p;
                    p = q;
                    q = t;
                }
                const double apq = a[p * kFK + q];
                double c = 1.0, sn = 0.0;
                if (apq != 0.0) {
                    // t = tan(theta), the smaller root of t^2 + 2 tau t - 1 = 0
                    // with tau = x / y: t = sgn(x y) |y| / (|x| + hypot(x, y));
                    // c = (1 + t^2)^(-1/2) from the hardware estimate and two
                    // Newton steps (each doubles the correct bits)
                    const double x = a[q * kFK + q] - a[p * kFK + p], y = 2.0 * apq;
                    const double r = sqrt(fma(x, x, y * y));
                    const double t = copysign(fabs(y) / (fabs(x) + r), x * y);
                    const double u = fma(t, t, 1.0);
                    double c0 = __builtin_amdgcn_rsq(u);
                    c0 = c0 * fma(-0.5 * u, c0 * c0, 1.5);
                    c0 = c0 * fma(-0.5 * u, c0 * c0, 1.5);
                    c = c0;
                    sn = t * c;
                }
                rp[i] = p;
                rq[i] = q;
                rc[i] = c;
                rs[i] = sn;
            }
            __syncthreads();
            // A <- J^T A J on 2 x 2 blocks (pair P rows, pair Q columns), and
            // V <- V J on rows j, pair Q
            constexpr uint32_t NP = kFK / 2;
            for (uint32_t k = threadIdx.x; k < NP * NP + kFK * NP; k += kSvdThreads) {
                if (k < NP * NP) {
                    const uint32_t P = k / NP, Q = k % NP;
                    const uint32_t p0 = rp[P], p1 = rq[P], q0 = rp[Q], q1 = rq[Q];
                    const double cP = rc[P], sP = rs[P], cQ = rc[Q], sQ = rs[Q];
                    const double m00 = a[p0 * kFK + q0], m01 = a[p0 * kFK + q1];
                    const double m10 = a[p1 * kFK + q0], m11 = a[p1 * kFK + q1];
                    // rows: J^T M
                    const double r00 = cP * m00 - sP * m10, r01 = cP * m01 - sP * m11;
                    const double r10 = sP * m00 + cP * m10, r11 = sP * m01 + cP * m11;
                    // columns: (J^T M) J
                    a[p0 * kFK + q0] = cQ * r00 - sQ * r01;
                    a[p0 * kFK + q1] = sQ * r00 + cQ * r01;
                    a[p1 * kFK + q0] = cQ * r10 - sQ * r11;
                    a[p1 * kFK + q1] = sQ * r10 + cQ * r11;
                } else {
                    const uint32_t t = k - NP * NP;
                    const uint32_t j = t / NP, Q = t % NP;
                    const uint32_t q0 = rp[Q], q1 = rq[Q];
                    const double c = rc[Q], sn = rs[Q];
                    const double x = v[j * kFK + q0], y2 = v[j * kFK + q1];
                    v[j * kFK + q0] = c * x - sn * y2;
                    v[j * kFK + q1] = sn * x + c * y2;
                }
            }
            __syncthreads();
        }
    }
    // eigenvalues in descending order (ties by index)
    if (threadIdx.x < (uint32_t)kFK) {
        const uint32_t i = threadIdx.x;
        const double li = a[i * kFK + i];
        uint32_t rank = 0;
        for (uint32_t k = 0; k < (uint32_t)kFK; ++k) {
            const double lk = a[k * kFK + k];
            rank += (lk > li || (lk == li && k < i)) ? 1u : 0u;
        }
        order[rank] = i;
    }
    __syncthreads();
    for (uint32_t k = threadIdx.x; k < (uint32_t)kFK * kFR; k += kSvdThreads) {
        const uint32_t j = k / kFR, col = k % kFR;
        const uint32_t e = order[col];
        const double lam = a[e * kFK + e];
        const double sg = lam > 0.0 ? sqrt(lam) : 0.0;
        const double u = v[j * kFK + e];
        ua[((uint64_t)m * kFK + j) * kFR + col] = (float)(u * sg);
        ur[((uint64_t)m * kFK + j) * kFR + col] = sg > 0.0 ? (float)(u / sg) : 0.0f;
    }
    if (threadIdx.x < (uint32_t)kFR) {
        const uint32_t e = order[threadIdx.x];
        const double lam = a[e * kFK + e];
        sigma[(uint64_t)m * kFR + threadIdx.x] = lam > 0.0 ? (float)sqrt(lam) : 0.0f;
    }
}

// out[m](n, :) = bf16( X[m](n, :) U[m] ) for X N x 48 and U 48 x 32, rows
// out_stride elements apart per matrix.
__global__ __launch_bounds__(kFThreads) void fac_finalize_kernel(const float* x, uint32_t N, const float* u,
                                                                 uint16_t* out, uint64_t out_stride) {
    __shared__ float us[kFK * kFR];
    const uint32_t m = blockIdx.y;
    for (uint32_t i = threadIdx.x; i < kFK * kFR; i += kFThreads) us[i] = u[(uint64_t)m * kFK * kFR + i];
    __syncthreads();
    const uint32_t n = blockIdx.x * kFThreads + threadIdx.x;
    if (n >= N) return;
    const float4* xr = reinterpret_cast<const float4*>(x + ((uint64_t)m * N + n) * kFK);
    float xv[kFK];
#pragma unroll
    for (int q = 0; q < kFK / 4; ++q) {
        const float4 t = xr[q];
        xv[4 * q] = t.x;
        xv[4 * q + 1] = t.y;
        xv[4 * q + 2] = t.z;
        xv[4 * q + 3] = t.w;
    }
    uint32_t o[kFR / 2];
#pragma unroll
    for (int c2 = 0; c2 < kFR / 2; ++c2) {
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int j = 0; j < kFK; ++j) {
            s0 = fmaf(xv[j], us[j * kFR + 2 * c2], s0);
            s1 = fmaf(xv[j], us[j * kFR + 2 * c2 + 1], s1);
        }
        o[c2] = pack_bf16x2(s0, s1);
    }
    uint4* dst = reinterpret_cast<uint4*>(out + (uint64_t)m * out_stride + (uint64_t)n * kFR);
#pragma unroll
    for (int q = 0; q < kFR / 8; ++q) dst[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
}

}  // namespace

LowrankFactorWs lowrank_factor_ws(uint32_t M, uint32_t H, uint32_t T, uint32_t d) {
    LowrankFactorWs w{};
    const uint64_t Dt = (uint64_t)H * d;
    const uint64_t nchunks = ((uint64_t)T + kFChunk - 1) / kFChunk;
    uint64_t off = 0;
    auto take = [&](uint64_t bytes) {
        const uint64_t at = off;
        off = (off + bytes + 255) & ~255ull;
        return at;
    };
    w.y = take((uint64_t)M * T * kFK * 4);
    w.w = take((uint64_t)M * Dt * kFK * 4);
    w.part = take((uint64_t)M * nchunks * Dt * kFK * 4);
    w.rinv = take((uint64_t)M * kFK * kFK * 8);
    const uint64_t gchunks = (((uint64_t)T > Dt ? (uint64_t)T : Dt) + kGChunk - 1) / kGChunk;
    w.gpart = take((uint64_t)M * gchunks * kFK * kFK * 8);
    w.ua = take((uint64_t)M * kFK * kFR * 4);
    w.ur = take((uint64_t)M * kFK * kFR * 4);
    w.sigma = take((uint64_t)M * kFR * 4);
    w.total = off;
    return w;
}

hipError_t launch_lowrank_factor(uint32_t M, uint32_t H, uint32_t T, uint32_t d, const void* z, const float* omega,
                                 void* a_out, uint64_t a_stride, void* r_out, uint64_t r_stride, float* sigma_out,
                                 void* ws, hipStream_t stream) {
    const LowrankFactorWs L = lowrank_factor_ws(M, H, T, d);
    uint8_t* base = static_cast<uint8_t*>(ws);
    float* Y = reinterpret_cast<float*>(base + L.y);
    float* W = reinterpret_cast<float*>(base + L.w);
    float* P = reinterpret_cast<float*>(base + L.part);
    double* Rinv = reinterpret_cast<double*>(base + L.rinv);
    double* Gp = reinterpret_cast<double*>(base + L.gpart);
    float* UA = reinterpret_cast<float*>(base + L.ua);
    float* UR = reinterpret_cast<float*>(base + L.ur);
    float* sig = sigma_out ? sigma_out : reinterpret_cast<float*>(base + L.sigma);
    const uint16_t* Z = static_cast<const uint16_t*>(z);
    const uint32_t Dt = H * d;
    const uint32_t nchunks = (T + kFChunk - 1) / kFChunk;
    const dim3 blk(kFThreads);
    hipError_t e = hipSuccess;
    auto zx = [&](const float* x, uint64_t x_stride) {
        if (e != hipSuccess) return;
        const dim3 grid((T + 255) / 256, M);
        e = d == 64 ? launch_kernel(fac_zx_kernel<64>, grid, blk, stream, Z, x, x_stride, Y, H, T)
                    : launch_kernel(fac_zx_kernel<128>, grid, blk, stream, Z, x, x_stride, Y, H, T);
    };
    auto ztq = [&]() {
        if (e != hipSuccess) return;
        const dim3 grid(nchunks, M * H);
        e = d == 64 ? launch_kernel(fac_ztq_kernel<64>, grid, blk, stream, Z, (const float*)Y, P, H, T, nchunks)
                    : launch_kernel(fac_ztq_kernel<128>, grid, blk, stream, Z, (const float*)Y, P, H, T, nchunks);
        if (e != hipSuccess) return;
        const uint64_t per = (uint64_t)Dt * kFK;
        const uint64_t n = (uint64_t)M * per;
        e = launch_kernel(fac_reduce_kernel, dim3((uint32_t)((n + kFThreads - 1) / kFThreads)), blk, stream,
                          (const float*)P, W, M, per, nchunks);
    };
    auto gram = [&](const float* x, uint32_t N) -> uint32_t {
        const uint32_t nc = (N + kGChunk - 1) / kGChunk;
        if (e == hipSuccess) e = launch_kernel(fac_gram_partial_kernel, dim3(nc, M), blk, stream, x, N, nc, Gp);
        return nc;
    };
    auto orth = [&](float* x, uint32_t N, int reps) {
        for (int rep = 0; rep < reps && e == hipSuccess; ++rep) {
            const uint32_t nc = gram(x, N);
            if (e != hipSuccess) return;
            e = launch_kernel(fac_chol_kernel, dim3(M), blk, stream, (const double*)Gp, nc, Rinv);
            if (e != hipSuccess) return;
            e = launch_kernel(fac_apply_rinv_kernel, dim3((N + kFThreads - 1) / kFThreads, M), blk, stream, x, N,
                              (const double*)Rinv);
        }
    };
    // the power iteration's bases only need to be well conditioned (one
    // CholeskyQR pass); the final Q is orthonormalised twice
    zx(omega, 0);               // Y = Z Omega
    orth(Y, T, 1);              // Q
    ztq();                      // W = Z^T Q
    orth(W, Dt, 1);             // orth(W)
    zx(W, (uint64_t)Dt * kFK);  // Y = Z W
    orth(Y, T, 2);              // Q
    ztq();                      // W = Z^T Q = B^T
    {
        const uint32_t nc = gram(W, Dt);
        if (e == hipSuccess)
            e = launch_kernel(fac_small_svd_kernel, dim3(M), dim3(kSvdThreads), stream, (const double*)Gp, nc, UA, UR, sig);
    }
    if (e == hipSuccess)
        e = launch_kernel(fac_finalize_kernel, dim3((T + kFThreads - 1) / kFThreads, M), blk, stream, (const float*)Y,
                          T, (const float*)UA, static_cast<uint16_t*>(a_out), a_stride);
    if (e == hipSuccess)
        e = launch_kernel(fac_finalize_kernel, dim3((Dt + kFThreads - 1) / kFThreads, M), blk, stream, (const float*)W,
                          Dt, (const float*)UR, static_cast<uint16_t*>(r_out), r_stride);
    return e;
}

}  // namespace kvc
