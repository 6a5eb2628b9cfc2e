// realign_kernels.hip - key position re-alignment for gfx950.
//
// KVCMAS (cache reuse across agents), procedure: before a shared segment's
// cache is reused by another agent, its key positions are re-aligned to the
// target's; a QKVShare CacheCard carries the source position offset for
// this. Rotary keys at position p hold each channel pair j rotated by
// p * f_j, so moving them by delta positions rotates pair j by delta * f_j
// more. The pairing of channels and the inverse frequencies f_j belong to
// the model and are inputs. Each workgroup takes cos and sin of
// delta * f_j (the product in binary64, exact as the host's) in binary64
// with the device math library, one pair per thread, into LDS. Each
// rotated value is a*c - b*s (or a*s + b*c) in binary64, two products and
// a difference, then rounded once to bf16: binary32 cos and sin lose too
// much when the two products nearly cancel.
//
// Work mapping: a lane rotates 8 channel pairs of one vector, so d/16 lanes
// cover a vector (8 vectors per wave at d = 128); every access is a 16-byte
// load or store, in place allowed (a lane reads its chunks before writing
// them, and no chunk is shared between lanes). A lane always handles the
// same 8 pairs, so the grid is persistent: each lane takes its 16 cos and
// sin values from LDS once, into registers, and then streams vector groups,
// two at a time.
#include "kernels_common.h"
#include "launch.h"

namespace kvc {
namespace {

constexpr uint64_t kRealignMaxBlocks = 2048;

struct RealignParams {
    const uint16_t* k_in;
    uint16_t* k_out;
    uint64_t vecs;      // L * H * T
    uint32_t pairing;   // 0: (j, j + d/2); 1: (2j, 2j + 1)
    int64_t delta;      // positions to move by
    float f[kMaxRealignPairs];  // inverse frequency of each pair
};

// Binary64 to bf16, round to nearest even, with one correct rounding: the
// value is first rounded to binary32 by round-to-odd (round to nearest, then,
// if inexact and the result is even, one step towards the exact value), which
// keeps the information the second rounding needs (binary32 has more than
// 8 + 2 significant bits), then rounded to bf16 by the hardware conversion.
__device__ __forceinline__ float to_odd_binary32(double x) {
    const float r = (float)x;
    uint32_t u = __float_as_uint(r);
    if ((double)r != x && (u & 1u) == 0u) {
        if (r == 0.0f)
            u = x < 0.0 ? 0x80000001u : 1u;
        else
            u += ((x > (double)r) == (r > 0.0f)) ? 1u : 0xFFFFFFFFu;
    }
    return __uint_as_float(u);
}

__device__ __forceinline__ void rotate_pair(float a, float b, double c, double s, float& ra, float& rb) {
    const double da = a, db = b;
    ra = to_odd_binary32(da * c - db * s);
    rb = to_odd_binary32(da * s + db * c);
}

template <int D>
__device__ __forceinline__ void realign_group(const RealignParams& p, uint64_t vec, uint32_t i, const double (&c)[8],
                                              const double (&sn)[8], uint32_t oa, uint32_t ob, const uint4& A,
                                              const uint4& B) {
    uint16_t* y = p.k_out + vec * D;
    const uint32_t wa[4] = {A.x, A.y, A.z, A.w}, wb[4] = {B.x, B.y, B.z, B.w};
    uint32_t ra[4], rb[4];
    if (p.pairing == 0) {
        // chunk A holds the 8 first members, chunk B the 8 second members
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            float a0, b0, a1, b1;
            rotate_pair(bf16_lo(wa[t]), bf16_lo(wb[t]), c[2 * t], sn[2 * t], a0, b0);
            rotate_pair(bf16_hi(wa[t]), bf16_hi(wb[t]), c[2 * t + 1], sn[2 * t + 1], a1, b1);
            ra[t] = pack_bf16x2(a0, a1);
            rb[t] = pack_bf16x2(b0, b1);
        }
    } else {
        // word t of a chunk is one pair (first member low, second high)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            float a0, b0, a1, b1;
            rotate_pair(bf16_lo(wa[t]), bf16_hi(wa[t]), c[t], sn[t], a0, b0);
            rotate_pair(bf16_lo(wb[t]), bf16_hi(wb[t]), c[4 + t], sn[4 + t], a1, b1);
            ra[t] = pack_bf16x2(a0, b0);
            rb[t] = pack_bf16x2(a1, b1);
        }
    }
    st_stream(reinterpret_cast<uint4*>(y + oa), make_uint4(ra[0], ra[1], ra[2], ra[3]));
    st_stream(reinterpret_cast<uint4*>(y + ob), make_uint4(rb[0], rb[1], rb[2], rb[3]));
}

template <int D>
__global__ __launch_bounds__(kBlockThreads) void realign_keys_kernel(RealignParams p) {
    constexpr uint32_t LPV = D / 16;         // lanes per vector (8 pairs each)
    constexpr uint32_t VPW = kWave / LPV;    // vectors per wave
    const uint32_t lane = lane_id();
    const uint64_t wave0 = (uint64_t)blockIdx.x * (kBlockThreads / kWave) + wave_uniform(threadIdx.x / kWave);
    const uint64_t nwaves = (uint64_t)gridDim.x * (kBlockThreads / kWave);
    const uint64_t groups = (p.vecs + VPW - 1) / VPW;  // VPW vectors each
    const uint32_t i = lane % LPV;           // pairs 8i .. 8i + 7
    // cos and sin of every pair's angle, once per workgroup
    __shared__ double cs_lds[D / 2], sn_lds[D / 2];
    if (threadIdx.x < D / 2) {
        const double phi = (double)p.delta * (double)p.f[threadIdx.x];
        cs_lds[threadIdx.x] = cos(phi);
        sn_lds[threadIdx.x] = sin(phi);
    }
    __syncthreads();
    // pair set 8i .. 8i + 7 in both pairings
    double c[8], sn[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        c[u] = cs_lds[8 * i + u];
        sn[u] = sn_lds[8 * i + u];
    }
    const uint32_t oa = p.pairing == 0 ? 8 * i : 16 * i;
    const uint32_t ob = p.pairing == 0 ? D / 2 + 8 * i : 16 * i + 8;
    for (uint64_t gw = wave0; gw < groups; gw += 2 * nwaves) {
        // two groups per pass; a lane past the last vector reloads its own
        // group's first vector and does not store
        const uint64_t g2 = gw + nwaves;
        const uint64_t v1 = gw * VPW + lane / LPV, v2 = g2 * VPW + lane / LPV;
        const bool ok1 = v1 < p.vecs, ok2 = v2 < p.vecs;
        const uint16_t* x1 = p.k_in + (ok1 ? v1 : gw * VPW) * D;
        const uint16_t* x2 = p.k_in + (ok2 ? v2 : gw * VPW) * D;
        const uint4 A1 = *reinterpret_cast<const uint4*>(x1 + oa), B1 = *reinterpret_cast<const uint4*>(x1 + ob);
        const uint4 A2 = *reinterpret_cast<const uint4*>(x2 + oa), B2 = *reinterpret_cast<const uint4*>(x2 + ob);
        if (ok1) realign_group<D>(p, v1, i, c, sn, oa, ob, A1, B1);
        if (ok2) realign_group<D>(p, v2, i, c, sn, oa, ob, A2, B2);
    }
}

}  // namespace

hipError_t launch_realign_keys(const Shape& s, const void* k_in, void* k_out, int64_t delta, const float* inv_freq,
                               uint32_t pairing, hipStream_t stream) {
    RealignParams p{};
    p.k_in = static_cast<const uint16_t*>(k_in);
    p.k_out = static_cast<uint16_t*>(k_out);
    p.vecs = (uint64_t)s.L * s.H * s.T;
    p.pairing = pairing;
    p.delta = delta;
    for (uint32_t j = 0; j < s.d / 2; ++j) p.f[j] = inv_freq[j];
    const uint32_t vpw = kWave / (s.d / 16);
    const uint64_t groups = (p.vecs + vpw - 1) / vpw;
    // persistent: 8 workgroups of 4 waves per CU, fewer for small inputs
    const uint64_t want = (groups + 3) / 4;
    const uint32_t nblocks = (uint32_t)(want < kRealignMaxBlocks ? want : kRealignMaxBlocks);
    return launch_kernel(s.d == 64 ? realign_keys_kernel<64> : realign_keys_kernel<128>, dim3(nblocks),
                         dim3(kBlockThreads), stream, p);
}

}  // namespace kvc
