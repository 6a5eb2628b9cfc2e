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
// inside the power iteration and twice for the final Q, the products with Z run in binary32 on the vector units (Z is
// bf16, exact in binary32), and the 48 x 48 eigenproblem is solved by
// parallel cyclic Jacobi in binary64. A and R are rounded once to bf16.
//
// Z is a matrix view of the cache layout: row t, column h*d + c of matrix m
// is element [m][h][t][c] of a bf16 [M][H][T][d] tensor.
#include "kernels_common.h"
#include "launch.h"

namespace kvc {
namespace {

constexpr int kFK = kLowrankSketch;  // 48 sketch columns
constexpr int kFR = 32;              // rank
constexpr int kFChunk = 256;         // tokens per partial product of Z^T Q
constexpr int kFThreads = 256;
constexpr int kFSweeps = 16;         // Jacobi sweep limit
// The small eigenproblem's workgroup: a Jacobi step is a chain of two
// barriers and 1728 independent updates (576 2 x 2 blocks of A, 1152 rows of
// V), so more threads shorten every step of the chain; its 32 workgroups do
// not fill the chip in any case.
constexpr int kSvdThreads = 1024;

// Y[m](t, :) = Z[m](t, :) X[m]; X is D x 48 row-major binary32, x_stride
// elements apart per matrix (0: one X for all). Block: 64 tokens x 4 waves
// of 12 columns; the rows of X for one head at a time pass through LDS.
template <int D>
__global__ __launch_bounds__(kFThreads) void fac_zx_kernel(const uint16_t* z, const float* x, uint64_t x_stride,
                                                           float* y, uint32_t H, uint32_t T) {
    __shared__ float4 xs[D * kFK / 4];
    const uint32_t m = blockIdx.y;
    const uint32_t t = blockIdx.x * 64 + threadIdx.x % 64;
    const uint32_t cg = wave_uniform(threadIdx.x / 64);  // columns 12 cg .. 12 cg + 11
    const uint32_t tc = t < T ? t : T - 1;
    const uint16_t* zm = z + (uint64_t)m * H * T * D;
    const float* xm = x + (uint64_t)m * x_stride;
    float acc[12];
#pragma unroll
    for (int j = 0; j < 12; ++j) acc[j] = 0.0f;
    for (uint32_t h = 0; h < H; ++h) {
        __syncthreads();
        const float4* xh = reinterpret_cast<const float4*>(xm + (uint64_t)h * D * kFK);
        for (uint32_t i = threadIdx.x; i < D * kFK / 4; i += kFThreads) xs[i] = xh[i];
        __syncthreads();
        const uint4* zr = reinterpret_cast<const uint4*>(zm + ((uint64_t)h * T + tc) * D);
        for (int q = 0; q < D / 8; ++q) {
            const uint4 w = zr[q];
            const float zz[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                                 bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float4* xr = xs + ((q * 8 + e) * kFK + cg * 12) / 4;
#pragma unroll
                for (int v = 0; v < 3; ++v) {
                    const float4 xv = xr[v];
                    acc[4 * v] = fmaf(zz[e], xv.x, acc[4 * v]);
                    acc[4 * v + 1] = fmaf(zz[e], xv.y, acc[4 * v + 1]);
                    acc[4 * v + 2] = fmaf(zz[e], xv.z, acc[4 * v + 2]);
                    acc[4 * v + 3] = fmaf(zz[e], xv.w, acc[4 * v + 3]);
                }
            }
        }
    }
    if (t < T) {
        float4* yr = reinterpret_cast<float4*>(y + ((uint64_t)m * T + t) * kFK + cg * 12);
#pragma unroll
        for (int v = 0; v < 3; ++v) yr[v] = make_float4(acc[4 * v], acc[4 * v + 1], acc[4 * v + 2], acc[4 * v + 3]);
    }
}

// Partial products P[m][chunk](h*d + c, :) = sum over the chunk's tokens t
// of Z[m](t, h*d + c) Q[m](t, :). Block: one chunk of one head; thread c of
// each group of d threads takes one channel and 48/G columns.
template <int D>
__global__ __launch_bounds__(kFThreads) void fac_ztq_kernel(const uint16_t* z, const float* q, float* part,
                                                            uint32_t H, uint32_t T, uint32_t nchunks) {
    constexpr int G = kFThreads / D;  // column groups: 2 (d = 128) or 4 (d = 64)
    constexpr int CW = kFK / G;       // 24 or 12 columns per thread
    __shared__ float4 qs[kFChunk * kFK / 4];
    const uint32_t chunk = blockIdx.x, h = blockIdx.y % H, m = blockIdx.y / H;
    const uint32_t c = threadIdx.x % D, g = wave_uniform(threadIdx.x / D);
    const uint32_t t0 = chunk * kFChunk;
    const uint32_t nt = (T - t0 < (uint32_t)kFChunk) ? T - t0 : (uint32_t)kFChunk;
    const float4* qm = reinterpret_cast<const float4*>(q + ((uint64_t)m * T + t0) * kFK);
    for (uint32_t i = threadIdx.x; i < nt * kFK / 4; i += kFThreads) qs[i] = qm[i];
    __syncthreads();
    const uint16_t* zm = z + (((uint64_t)m * H + h) * T + t0) * D + c;
    float acc[CW];
#pragma unroll
    for (int j = 0; j < CW; ++j) acc[j] = 0.0f;
    uint32_t t = 0;
    for (; t + 8 <= nt; t += 8) {
        float zz[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) zz[u] = __uint_as_float((uint32_t)zm[(uint64_t)(t + u) * D] << 16);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float4* qr = qs + ((t + u) * kFK + g * CW) / 4;
#pragma unroll
            for (int v = 0; v < CW / 4; ++v) {
                const float4 qv = qr[v];
                acc[4 * v] = fmaf(zz[u], qv.x, acc[4 * v]);
                acc[4 * v + 1] = fmaf(zz[u], qv.y, acc[4 * v + 1]);
                acc[4 * v + 2] = fmaf(zz[u], qv.z, acc[4 * v + 2]);
                acc[4 * v + 3] = fmaf(zz[u], qv.w, acc[4 * v + 3]);
            }
        }
    }
    for (; t < nt; ++t) {
        const float zz = __uint_as_float((uint32_t)zm[(uint64_t)t * D] << 16);
        const float4* qr = qs + (t * kFK + g * CW) / 4;
#pragma unroll
        for (int v = 0; v < CW / 4; ++v) {
            const float4 qv = qr[v];
            acc[4 * v] = fmaf(zz, qv.x, acc[4 * v]);
            acc[4 * v + 1] = fmaf(zz, qv.y, acc[4 * v + 1]);
            acc[4 * v + 2] = fmaf(zz, qv.z, acc[4 * v + 2]);
            acc[4 * v + 3] = fmaf(zz, qv.w, acc[4 * v + 3]);
        }
    }
    float4* pr = reinterpret_cast<float4*>(part + (((uint64_t)m * nchunks + chunk) * ((uint64_t)H * D) +
                                                   (uint64_t)h * D + c) * kFK + g * CW);
#pragma unroll
    for (int v = 0; v < CW / 4; ++v) pr[v] = make_float4(acc[4 * v], acc[4 * v + 1], acc[4 * v + 2], acc[4 * v + 3]);
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
// binary64) over chunks of 256 rows, one block per (chunk, matrix); the
// chunk's rows pass through LDS and each thread owns a 3 x 3 tile of the
// upper triangle of tiles.
constexpr int kGRows = 256;
constexpr int kGTile = 3;
constexpr int kGTiles = kFK / kGTile;                    // 16 tiles per side
constexpr int kGTilePairs = kGTiles * (kGTiles + 1) / 2;  // 136

__global__ __launch_bounds__(kFThreads) void fac_gram_partial_kernel(const float* y, uint32_t N, uint32_t nchunks,
                                                                     double* gpart) {
    __shared__ float4 ys[kGRows * kFK / 4];
    const uint32_t chunk = blockIdx.x, m = blockIdx.y;
    const uint32_t r0 = chunk * kGRows;
    const uint32_t nr = (N - r0 < (uint32_t)kGRows) ? N - r0 : (uint32_t)kGRows;
    const float4* src = reinterpret_cast<const float4*>(y + ((uint64_t)m * N + r0) * kFK);
    for (uint32_t i = threadIdx.x; i < nr * kFK / 4; i += kFThreads) ys[i] = src[i];
    __syncthreads();
    double* out = gpart + ((uint64_t)m * nchunks + chunk) * kFK * kFK;
    if (threadIdx.x >= (uint32_t)kGTilePairs) return;  // no barrier follows
    uint32_t ti = 0, e = threadIdx.x, n = kGTiles;
    while (e >= n) {
        e -= n;
        ++ti;
        --n;
    }
    const uint32_t tj = ti + e;  // tile (ti, tj), ti <= tj
    const float* yf = reinterpret_cast<const float*>(ys);
    double acc[kGTile][kGTile];
#pragma unroll
    for (int a = 0; a < kGTile; ++a)
#pragma unroll
        for (int b = 0; b < kGTile; ++b) acc[a][b] = 0.0;
    for (uint32_t r = 0; r < nr; ++r) {
        double u[kGTile], v[kGTile];
#pragma unroll
        for (int a = 0; a < kGTile; ++a) {
            u[a] = yf[r * kFK + ti * kGTile + a];
            v[a] = yf[r * kFK + tj * kGTile + a];
        }
#pragma unroll
        for (int a = 0; a < kGTile; ++a)
#pragma unroll
            for (int b = 0; b < kGTile; ++b) acc[a][b] = fma(u[a], v[b], acc[a][b]);
    }
#pragma unroll
    for (int a = 0; a < kGTile; ++a)
#pragma unroll
        for (int b = 0; b < kGTile; ++b) {
            const uint32_t i = ti * kGTile + a, j = tj * kGTile + b;
            out[i * kFK + j] = acc[a][b];
            out[j * kFK + i] = acc[a][b];
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

// One CholeskyQR step, factor part: G = Y^T Y = L L^T, then Rinv = (L^T)^-1
// (upper triangular), binary64. A pivot at or below 1e-12 of the largest
// diagonal entry drops its column: its row and column of Rinv are zero.
__global__ __launch_bounds__(kFThreads) void fac_chol_kernel(const double* gpart, uint32_t nchunks, double* rinv) {
    __shared__ double g[kFK * kFK];
    __shared__ double L[kFK * kFK];
    const uint32_t m = blockIdx.x;
    sum_gram<kFThreads>(gpart, m, nchunks, g);
    for (uint32_t i = threadIdx.x; i < kFK * kFK; i += kFThreads) L[i] = 0.0;
    __syncthreads();
    if (threadIdx.x < kWave) {
        const uint32_t i = threadIdx.x;  // row handled by this lane
        double maxdiag = 0.0;
        for (int k = 0; k < kFK; ++k) maxdiag = fmax(maxdiag, g[k * kFK + k]);
        const double tol = 1e-12 * maxdiag;
        const uint32_t ri = i < (uint32_t)kFK ? i : 0u;
        for (uint32_t j = 0; j < (uint32_t)kFK; ++j) {
            // the pivot's sum and this row's sum in one loop: two independent
            // chains of subtractions, each in its own order of k
            double s = g[j * kFK + j];
            double v = g[ri * kFK + j];
            for (uint32_t k = 0; k < j; ++k) {
                const double ljk = L[j * kFK + k];
                s -= ljk * ljk;
                v -= L[ri * kFK + k] * ljk;
            }
            const bool keep = s > tol;
            const double ljj = keep ? sqrt(s) : 0.0;
            if (keep && i > j && i < (uint32_t)kFK) v /= ljj;
            else v = 0.0;
            __builtin_amdgcn_wave_barrier();
            if (i == j) L[j * kFK + j] = ljj;
            if (i > j && i < (uint32_t)kFK) L[i * kFK + j] = v;
            __builtin_amdgcn_wave_barrier();
        }
        // column i of Rinv (R = L^T, R(a, b) = L[b][a]): back substitution,
        // in g (the Gram matrix is no longer needed)
        __builtin_amdgcn_wave_barrier();
        if (i < (uint32_t)kFK) {
            for (int a = kFK - 1; a >= 0; --a) {
                double xa = 0.0;
                if ((uint32_t)a <= i && L[a * kFK + a] != 0.0) {
                    double s = (a == (int)i) ? 1.0 : 0.0;
                    for (uint32_t b = a + 1; b <= i; ++b) s -= L[b * kFK + a] * g[b * kFK + i];
                    xa = s / L[a * kFK + a];
                }
                g[a * kFK + i] = xa;
            }
        }
    }
    __syncthreads();
    double* out = rinv + (uint64_t)m * kFK * kFK;
    for (uint32_t i = threadIdx.x; i < kFK * kFK; i += kFThreads) out[i] = g[i];
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
// below 1e-12 of the diagonal (in norm); writes ua = U_r diag(sigma),
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
        if (so <= 1e-24 * sd) break;  // every thread takes the same branch
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
                    const double tau = (a[q * kFK + q] - a[p * kFK + p]) / (2.0 * apq);
                    const double t = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
                    c = 1.0 / sqrt(1.0 + t * t);
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
    const uint64_t gchunks = (((uint64_t)T > Dt ? (uint64_t)T : Dt) + kGRows - 1) / kGRows;
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
        const dim3 grid((T + 63) / 64, M);
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
        const uint32_t nc = (N + kGRows - 1) / kGRows;
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
