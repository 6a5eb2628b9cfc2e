// pool_kernels.hip - shared-pool encode and decode for gfx950.
//
// PolyKV (gist.science/ko/paper/2604.24971) section 2.A: one compressed pool
// is written once and read by every agent; section 2.B item 1: int8 keys with
// one scale per tensor (per layer); section 2.B item 2: values rotated by the
// fast Walsh-Hadamard transform and mapped to 3-bit Lloyd-Max levels of
// N(0,1), decoded by level lookup and the inverse transform.
//
// Work mapping. One wave64 handles one 16-token block of one (layer, head):
// lane 4t+m holds channels [m*d/4, (m+1)*d/4) of token t, i.e. 32 consecutive
// bf16 (64 bytes) for d = 128 and 16 (32 bytes) for d = 64. So
//  - HBM traffic is contiguous per wave (4 KiB of K and of V for d = 128);
//  - the first log2(d/4) butterfly stages and the first levels of the
//    pairwise sum of squares run inside a lane, the last two across the quad
//    through DPP quad permutes (no LDS);
//  - each code bit is one wave-wide compare; a lane appends its bit to a
//    per-plane word with one add-with-carry, so a lane ends with the three
//    bit planes of its d/4 coordinates, already in the pool's layout
//    (plane p: bit i <-> coordinate i, least significant bit first).
//
// Numerics. Every float step follows the codec definition operation by
// operation (binary32, round to nearest even, no contraction - the library is
// built with -ffp-contract=off): the butterfly runs its stages in ascending
// order, the sum of squares is the pairwise tree over natural index order,
// and a cross-lane butterfly step computes fma(own, +-1, partner), which is
// exactly partner + own or partner - own. Hence codes and scales are
// bit-identical to a scalar implementation of the same definition. Decoding
// runs the butterfly on the stored levels, which sit on a 2^-15 grid: every
// partial sum is a multiple of 2^-15 below 2^9 and is exact in binary32, so
// the only roundings are the final product with s/sqrt(d) and the bf16
// conversion.
#include "codebook.h"
#include "kernels_common.h"
#include "launch.h"
#include "layout.h"

#include <atomic>
#include <chrono>
#include <cstdlib>
#include <mutex>
#include <random>
#include <utility>

// Encode workspace held by the library for kvpool_encode_noalloc (callers
// that cannot allocate). A module variable exists once per GPU, at its own
// address on each; it starts zeroed and keeps what the last call left.
static __device__ __align__(256) uint32_t scratch[kvc::kNoAllocScratchBytes / 4];

namespace kvc {
namespace {

// 1/sqrt(d) rounded to binary32
template <int D>
__device__ constexpr float inv_sqrt_d() {
    return D == 64 ? 0.125f : 0x1.6a09e6p-4f;
}

struct EncodeParams {
    const uint16_t* k;
    const uint16_t* v;
    uint8_t* pool;
    uint32_t* ws;           // workspace, see the slot helpers below
    int32_t* status;        // device status word or nullptr
    uint32_t L, H, T, nb;   // nb = 16-token blocks per head
    uint32_t blocks_per_layer;  // H * nb
    uint32_t layers_per_round;  // single-pass encode: whole layers per round
    uint64_t n_waves;           // L * H * nb
    uint64_t poll_ticks;        // single-pass encode: bound on the wait for other workgroups' maxima
    uint32_t absmax_groups;     // layered encode: key-maximum workgroups per layer
    uint32_t encode_groups;     // layered encode: encode workgroups per layer
    uint64_t call;              // this call's number (tags its exchange words)
    PoolLayout lay;
};

// Encode workspace (u32 words): 64 head words, then kWsWordsPerLayer words
// per layer. Both encode paths exchange 64-bit words that one workgroup
// publishes and others read, some before it is written: the single pass one
// per (layer, workgroup), the layered encode one per (layer, key-maximum
// workgroup) and then one per layer. Each call tags the words it writes with a call number of its
// own (48 bits, from a host counter of the library instance that starts at
// a random point and skips 0): a word is (call << 16) | 0x8000 | maximum
// bits (15 bits), and it counts only if it carries this call's number, so
// words left by earlier calls of either path (or zeros) are not taken for
// this call's, and nothing needs clearing between calls. The workspace must
// hold zeros before its first encode (zero never matches a call number).
// Head words [2..3]: the number of a call whose wait gave up (64 bits).
constexpr uint32_t kWsHead = 64;              // words
constexpr uint32_t kWsWordsPerLayer = 1024;  // = encode_workspace_words(L) / L, less the head
constexpr uint32_t kWsGaveUp = 2;             // u64 at words 2..3
constexpr int32_t kDevTimeout = 8;            // KVC_DEV_ENCODE_TIMEOUT



struct DecodeParams {
    const uint8_t* pool;
    int32_t* status;
    uint32_t L, H, T, nb;
    uint32_t l0, n_out;
    uint64_t n_waves;  // (l1 - l0) * H * nb
    PoolLayout lay;
    uint16_t* k_out[kMaxAgents];
    uint16_t* v_out[kMaxAgents];
};

// ---------------------------------------------------------------- helpers

// Unnormalised Walsh-Hadamard transform of d = 4*C values spread over the
// quad (C per lane, lane m holds block m): stages h = 1 .. C/2 in the lane,
// then h = C (partner lane m^1) and h = 2C (partner lane m^2), each
// cross-lane step one v_fmac with a DPP source: stored = own + s * partner.
// Lanes whose butterfly output is partner - own get own - partner instead,
// so after both steps lane m holds sign_m * (the transform) with
// sign_m = (-1)^popcount(m); the caller folds sign_m into its scale. Every
// non-zero value is exactly +-(the ascending-order binary32 butterfly's
// value) since rounding to nearest is symmetric; zeros may differ in sign.
template <int C>
__device__ __forceinline__ void fwht_quad(float (&y)[C], uint32_t m) {
#pragma unroll
    for (int h = 1; h < C; h *= 2) {
#pragma unroll
        for (int i = 0; i < C; i += 2 * h) {
#pragma unroll
            for (int j = i; j < i + h; ++j) {
                const float a = y[j], b = y[j + h];
                y[j] = a + b;
                y[j + h] = a - b;
            }
        }
    }
    const float s1 = (m & 1u) ? -1.0f : 1.0f;
#pragma unroll
    for (int j = 0; j < C; j += 8) fmac_dpp8_xor1(y + j, s1);
    // after the first step lane m carries sign (-1)^(m&1); the second step's
    // multiplier sign_own * sign_partner (lower half) or its negation (upper
    // half) works out to -1 exactly on the upper half
    const float s2 = (m & 2u) ? -1.0f : 1.0f;
#pragma unroll
    for (int j = 0; j < C; j += 8) fmac_dpp8_xor2(y + j, s2);
}

// Sign (+1 / -1) that fwht_quad leaves on lane m's outputs.
__device__ __forceinline__ float fwht_quad_sign(uint32_t m) {
    return (__builtin_popcount(m & 3u) & 1) ? -1.0f : 1.0f;
}

// Maximum of r over the wave, as a wave-uniform (scalar) value; every lane
// must be active. DPP folds each quad (lane xor 1, xor 2), then each 16-lane
// row (rotations by 4 and 8), so every lane holds its row's maximum; the
// four rows' are read into scalar registers and folded there.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t r) {
    const uint32_t t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)r, CTRL, 0xF, 0xF, false);
    return t > r ? t : r;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t r) {
    r = dpp_max_step<0xB1>(r);   // quad_perm [1,0,3,2]
    r = dpp_max_step<0x4E>(r);   // quad_perm [2,3,0,1]
    r = dpp_max_step<0x124>(r);  // row_ror:4
    r = dpp_max_step<0x128>(r);  // row_ror:8
    const uint32_t a = __builtin_amdgcn_readlane(r, 0), b = __builtin_amdgcn_readlane(r, 16);
    const uint32_t c = __builtin_amdgcn_readlane(r, 32), d = __builtin_amdgcn_readlane(r, 48);
    const uint32_t ab = a > b ? a : b, cd = c > d ? c : d;
    return ab > cd ? ab : cd;
}

// Header (64 B) and every padding byte of the pool; run by workgroup 0.
__device__ void pool_header_and_padding(const EncodeParams& p, uint32_t d, uint32_t tid) {
    uint8_t* pool = p.pool;
    const PoolLayout& lay = p.lay;
    if (tid < 16) {
        const uint64_t offs[5] = {lay.k_scale, lay.k_codes, lay.v_scale, lay.v_codes, lay.total};
        uint32_t val;
        switch (tid) {
            case 0: val = kPoolMagic; break;
            case 1: val = 1u | (1u << 16); break;  // version 1, kind 1
            case 2: val = p.L; break;
            case 3: val = p.H; break;
            case 4: val = p.T; break;
            case 5: val = d; break;
            default: {
                const uint64_t o = offs[(tid - 6) / 2];
                val = (tid & 1) ? (uint32_t)(o >> 32) : (uint32_t)o;
            }
        }
        reinterpret_cast<uint32_t*>(pool)[tid] = val;
    }
    const uint64_t vecs = (uint64_t)p.L * p.H * p.T;
    const uint64_t ends[5] = {kPoolHeaderBytes, lay.k_scale + 4ull * p.L, lay.k_codes + vecs * d,
                              lay.v_scale + 2ull * vecs,
                              lay.v_codes + vecs * pool_code_bytes(d)};
    const uint64_t starts[5] = {lay.k_scale, lay.k_codes, lay.v_scale, lay.v_codes, lay.total};
#pragma unroll
    for (int r = 0; r < 5; ++r)
        for (uint64_t i = ends[r] + tid; i < starts[r]; i += kBlockThreads) pool[i] = 0;
}

// ---------------------------------------------------------------- kernels

// Coordinate I of the lane: code = number of thresholds <= z, found bit by
// bit (binary search over the 7 sorted thresholds); each bit is appended to
// its plane word. Slots run from the last coordinate down so that
// coordinate i lands in bit i.
template <int C, int I>
__device__ __forceinline__ void code_slot(const float (&y)[C], float r, uint32_t (&pl)[3]) {
    const float z = y[I] * r;
    const bool b2 = z >= 0.0f;
    const float t1 = b2 ? kTh6 : -kTh6;
    const bool b1 = z >= t1;
    const float a0 = (b1 == b2) ? kTh7 : kTh5;
    const float t0 = b2 ? a0 : -a0;
    pl[0] = shift_in_bit(pl[0], __builtin_amdgcn_ballot_w64(z >= t0));
    pl[1] = shift_in_bit(pl[1], __builtin_amdgcn_ballot_w64(b1));
    pl[2] = shift_in_bit(pl[2], __builtin_amdgcn_ballot_w64(b2));
}

template <int C, int... Is>
__device__ __forceinline__ void code_all(const float (&y)[C], float r, uint32_t (&pl)[3],
                                         std::integer_sequence<int, Is...>) {
    (code_slot<C, C - 1 - Is>(y, r, pl), ...);
}

// Per-wave LDS staging for the encode outputs: the wave's K codes (16
// tokens x d bytes) and V code planes (16 tokens x 3d/8 bytes), written to
// HBM with every store instruction covering one contiguous span.
template <int D>
struct EncodeStage {
    uint4 k[kBlockTokens * D / 16];
    uint32_t v[kBlockTokens * 3 * D / 32];
};

// Geometry of one wave's block: 16 tokens of one (layer, head).
struct BlockPos {
    uint32_t l, bidx, m, nv;  // layer, block within the layer, lane's quarter, valid tokens
    uint64_t vec0, vec;       // first token of the block, this lane's token
    uint64_t elem;            // element offset this lane loads from
    bool valid;               // this lane's token exists
};

template <int D>
__device__ __forceinline__ BlockPos block_pos(const EncodeParams& p, uint32_t l, uint32_t bidx, uint32_t lane) {
    BlockPos b;
    b.l = l;
    b.bidx = bidx;
    b.m = lane & 3u;
    const uint32_t h = bidx / p.nb, t0 = (bidx % p.nb) * kBlockTokens;
    b.nv = (p.T - t0 < kBlockTokens) ? p.T - t0 : kBlockTokens;
    b.vec0 = ((uint64_t)l * p.H + h) * p.T + t0;
    b.vec = b.vec0 + (lane >> 2);
    b.valid = t0 + (lane >> 2) < p.T;
    // lanes past the end of the tokens load the block's first vector and are
    // masked at the key max and at every store
    b.elem = (b.valid ? b.vec : b.vec0) * D + (uint64_t)b.m * (D / 4);
    return b;
}

template <int D>
__device__ __forceinline__ void load_lane(const uint16_t* base, uint64_t elem, uint4 (&raw)[D / 32]) {
    const uint4* src = reinterpret_cast<const uint4*>(base + elem);
#pragma unroll
    for (int i = 0; i < D / 32; ++i) raw[i] = src[i];
}

// Values of one block: RMS scale, rotation, 3-bit codes; writes the scales
// and the code planes (PolyKV 2.B item 2).
template <int D>
__device__ __forceinline__ void encode_values(const EncodeParams& p, const BlockPos& b, const uint4 (&vraw)[D / 32],
                                              EncodeStage<D>& stg, uint32_t lane) {
    constexpr int C = D / 4;  // channels per lane
    const uint32_t m = b.m;
    float y[C];
    {
        const uint32_t* w = reinterpret_cast<const uint32_t*>(vraw);
#pragma unroll
        for (int j = 0; j < C / 2; ++j) {
            y[2 * j] = bf16_lo(w[j]);
            y[2 * j + 1] = bf16_hi(w[j]);
        }
    }
    // sum of squares: pairwise tree, left to right, lanes in block order
    float sq[C];
#pragma unroll
    for (int j = 0; j < C; ++j) sq[j] = y[j] * y[j];
#pragma unroll
    for (int w = C / 2; w >= 1; w /= 2)
#pragma unroll
        for (int j = 0; j < w; ++j) sq[j] = sq[2 * j] + sq[2 * j + 1];
    float ss = sq[0];
    ss = ss + dpp_xor1(ss);
    ss = ss + dpp_xor2(ss);
    const float rms = __builtin_sqrtf(ss * (1.0f / D));
    const _Float16 sh16 = (_Float16)__builtin_fminf(rms, 65504.0f);
    const float sc = (float)sh16;
    // scale, with the sign fwht_quad leaves on this lane folded in
    const float r = ((sc == 0.0f) ? 0.0f : inv_sqrt_d<D>() / sc) * fwht_quad_sign(m);
    if (b.valid && m == 0)
        reinterpret_cast<uint16_t*>(p.pool + p.lay.v_scale)[b.vec] = __builtin_bit_cast(uint16_t, sh16);

    fwht_quad<C>(y, m);

    uint32_t pl[3] = {0, 0, 0};
    code_all<C>(y, r, pl, std::make_integer_sequence<int, C>{});
    // stage the wave's code planes (token t: 3 planes of d/8 bytes), then
    // store them with each instruction covering a contiguous span
    const uint32_t t = lane >> 2;
    if (D == 128) {
#pragma unroll
        for (int q = 0; q < 3; ++q) stg.v[t * 12 + 4 * q + m] = pl[q];
    } else {
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            const uint32_t word = pl[q] | (dpp_xor1_u(pl[q]) << 16);
            if ((m & 1u) == 0) stg.v[t * 6 + 2 * q + (m >> 1)] = word;
        }
    }
    constexpr int VW = 3 * D / 8 / 4;  // code dwords per token
    uint32_t* dst = reinterpret_cast<uint32_t*>(p.pool + p.lay.v_codes + b.vec0 * pool_code_bytes(D));
#pragma unroll
    for (int j = 0; j < (kBlockTokens * VW + 63) / 64; ++j) {
        const uint32_t idx = 64 * j + lane;
        if (idx < kBlockTokens * VW) {
            const uint32_t wv = stg.v[idx];
            if (idx / VW < b.nv) st_stream(dst + idx, wv);
        }
    }
}

// Keys of one block given the layer's max m (as bf16 magnitude bits)
// (PolyKV 2.B item 1): q = rint(x * (127 / m)). |x * inv| <= 127 (1 + 2^-23),
// so q never leaves [-127, 127]. Rounding adds 1.5*2^23: the low byte of the
// sum is the two's-complement integer (ties to even). The maximum is taken
// on the sign-cleared bit patterns, so an Inf or NaN key makes it
// non-finite; such a layer gets a NaN scale and all-zero codes.
template <int D>
__device__ __forceinline__ void quantize_keys(const EncodeParams& p, const BlockPos& b, const uint4 (&kraw)[D / 32],
                                              uint32_t mbits, EncodeStage<D>& stg, uint32_t lane) {
    constexpr int C = D / 4;
    mbits = wave_uniform(mbits);  // the same for every lane: one scalar branch below
    const float mk = __uint_as_float(mbits << 16);
    const bool finite = mbits < 0x7F80u;
    const float inv = (mk == 0.0f) ? 0.0f : 127.0f / mk;
    const uint32_t* w = reinterpret_cast<const uint32_t*>(kraw);
    uint32_t out[C / 4];
    if (finite) {
#pragma unroll
        for (int j = 0; j < C / 4; ++j) {
            const uint32_t w0 = w[2 * j], w1 = w[2 * j + 1];
            const float q0 = bf16_lo(w0) * inv + 12582912.0f;
            const float q1 = bf16_hi(w0) * inv + 12582912.0f;
            const float q2 = bf16_lo(w1) * inv + 12582912.0f;
            const float q3 = bf16_hi(w1) * inv + 12582912.0f;
            const uint32_t ab = __builtin_amdgcn_perm(__float_as_uint(q1), __float_as_uint(q0), 0x0c0c0400u);
            const uint32_t cd = __builtin_amdgcn_perm(__float_as_uint(q3), __float_as_uint(q2), 0x04000c0cu);
            out[j] = ab | cd;
        }
    } else {
#pragma unroll
        for (int j = 0; j < C / 4; ++j) out[j] = 0;
    }
    constexpr int KC = C / 16;  // 16-byte chunks of codes per lane
#pragma unroll
    for (int c = 0; c < KC; ++c)
        stg.k[stage_slot<KC>(lane, c)] = make_uint4(out[4 * c], out[4 * c + 1], out[4 * c + 2], out[4 * c + 3]);
    uint4* dst = reinterpret_cast<uint4*>(p.pool + p.lay.k_codes + b.vec0 * D);
#pragma unroll
    for (int j = 0; j < KC; ++j) {
        const uint4 chunk16 = stg.k[stage_pos<KC>(64 * j + lane)];
        if ((64 * j + lane) / (D / 16) < b.nv) st_stream(dst + 64 * j + lane, chunk16);
    }
    if (b.bidx == 0 && lane == 0)
        reinterpret_cast<uint32_t*>(p.pool + p.lay.k_scale)[b.l] =
            finite ? __float_as_uint((mk == 0.0f) ? 0.0f : mk / 127.0f) : 0x7FC00000u;
}

// ---------------------------------------------------------------- single-pass encode
//
// The key scale of a layer needs every key of the layer before any key is
// quantised. Here K is read once and parked in LDS: a
// persistent grid (one workgroup per CU at this LDS size) walks the layers
// in rounds of whole layers. A workgroup owns 8 block slots per round (one
// 16-token block each at d = 128, two at d = 64) and splits the work by
// role, so that a SIMD holds three or four waves and the value transform's
// VALU stream is not the only work it can issue:
//
// Value wave (8, one per slot): load round r+1's values, encode round r's
// (scale, rotation, codes, stores). It never waits on another wave.
// Key wave (4, two slots each), iteration r:
//   a. issue the key loads of round r+1;
//   b. park round r's keys in LDS, fold their maxima into the workgroup's
//      (LDS atomics) and count itself done;
//   c. wait (in LDS) until the coordinator has the layer maxima of round
//      r-3, then quantise the keys parked in round r-3 (kQuantLag rounds of
//      work between a workgroup's publication and its need of everyone's:
//      a lag of 2 measured 3-4 us slower on the Llama 4K pool).
// Coordinator wave, round r: when the key waves are done with r, publish
// the workgroup's maxima of r as flag|max words (one per layer and
// workgroup; one plain device-scope store each, no returning atomic), then
// read every workgroup's words of round r-1 until all are flagged, reduce
// them to the layer maxima and hand those to the key waves in LDS. Only the
// coordinator waits on device-scope memory, so no load counter waits for a
// poll, and a round of work separates each publication from the wait for
// it.
//
// The grid is an ordinary launch: nothing guarantees that every workgroup
// is resident at once (another kernel may hold CUs). A coordinator that has
// not seen every workgroup's word for a layer within poll_ticks computes
// the layer's maximum itself from the keys in HBM. Both routes give the same
// exact maximum, so residency decides only the speed; no wait depends on a
// workgroup that may not be running.
constexpr int kFusedSlots = 8;     // block slots per workgroup and round
constexpr int kFusedKeyWaves = 4;    // key waves, kSlotsPerKeyWave slots each
constexpr int kSlotsPerKeyWave = kFusedSlots / kFusedKeyWaves;
constexpr int kFusedThreads = (kFusedSlots + kFusedKeyWaves + 1) * kWave;
constexpr int kQuantLag = 3;                // rounds between parking keys and quantising them
constexpr int kHoldRounds = kQuantLag + 1;  // LDS key buffers and handshake entries
constexpr uint32_t kMaxRoundLayers = 32;
constexpr uint32_t kMaxFusedGrid = 1024;  // bound on the grid (the launch keeps it below 960); sizes the poll registers
constexpr uint64_t kWordFlag = 0x8000u;
constexpr uint32_t kLayeredMaxGroups = 256;  // layered encode: bound on the key-maximum workgroups per layer
static_assert(2 * (kLayeredMaxGroups + 1) <= kWsWordsPerLayer, "layered encode words exceed the workspace");
// Spin limit of the waits inside a workgroup (key waves for their
// coordinator, coordinator for its key waves), in ticks of the 100 MHz
// constant clock: 0.5 s. These waits depend only on the workgroup's own
// waves, so the limit is a guard against a hang, never expected to trip.
constexpr uint64_t kWaitTicks = 50000000ull;

// Flag words of layer l, one per workgroup of a G-workgroup grid.
__device__ __forceinline__ uint64_t* round_flags(uint32_t* ws, uint32_t G, uint32_t l) {
    return reinterpret_cast<uint64_t*>(ws + kWsHead) + (uint64_t)l * G;
}

template <int D>
struct FusedLds {
    static constexpr int kBpw = 128 / D;  // blocks per slot and round: 4 KiB of keys
    uint4 hold[kHoldRounds][kFusedSlots][kBpw][D / 32][kWave];  // [round % 4][slot][block][chunk][lane]
    EncodeStage<D> stage[kFusedSlots];  // per slot: .v by its value wave, .k by its key wave
    // By round % 4: a key wave reaches round r only after its wait in round
    // r-1 saw the maxima of round r-4 ready, i.e. after the coordinator has
    // consumed and cleared the round-(r-4) entries that round r reuses.
    uint32_t wg_max[kHoldRounds][kMaxRoundLayers];     // this workgroup's key maxima
    uint32_t layer_max[kHoldRounds][kMaxRoundLayers];  // every workgroup's, per layer
    uint32_t done[kHoldRounds];                        // key waves done with the round
    uint32_t ready;                                    // rounds whose maxima are in layer_max
    uint32_t gave_up;                                  // a wave of this workgroup recorded a wait that gave up
};

// Largest bf16 magnitude (as bits) among a lane's raw words.
template <int N>
__device__ __forceinline__ uint32_t lane_absmax_bits(const uint4 (&raw)[N]) {
    typedef unsigned short us2 __attribute__((ext_vector_type(2)));
    us2 mx = {0, 0};
#pragma unroll
    for (int i = 0; i < N; ++i) {
        mx = __builtin_elementwise_max(mx, __builtin_bit_cast(us2, raw[i].x & 0x7FFF7FFFu));
        mx = __builtin_elementwise_max(mx, __builtin_bit_cast(us2, raw[i].y & 0x7FFF7FFFu));
        mx = __builtin_elementwise_max(mx, __builtin_bit_cast(us2, raw[i].z & 0x7FFF7FFFu));
        mx = __builtin_elementwise_max(mx, __builtin_bit_cast(us2, raw[i].w & 0x7FFF7FFFu));
    }
    return mx.x > mx.y ? mx.x : mx.y;
}

// Largest key magnitude (bf16 bits) of layer l, read from the keys in HBM
// by one wave: the same exact value that the workgroups' published maxima
// reduce to. Used by a coordinator whose wait for those maxima ran out.
template <int D>
__device__ uint32_t layer_absmax_direct(const EncodeParams& p, uint32_t l, uint32_t lane) {
    const uint64_t n = (uint64_t)p.H * p.T * (D / 8);  // uint4 per layer
    const uint4* src = reinterpret_cast<const uint4*>(p.k) + (uint64_t)l * n;
    uint32_t m = 0;
    for (uint64_t i = lane; i < n; i += 4 * kWave) {
        uint4 raw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint64_t idx = i + (uint64_t)j * kWave;
            raw[j] = idx < n ? src[idx] : make_uint4(0, 0, 0, 0);
        }
        const uint32_t x = lane_absmax_bits<4>(raw);
        m = x > m ? x : m;
    }
    return wave_max_u32(m);
}

struct Round {
    uint32_t l0, nl, nblk;  // first layer, layers, blocks
};

__device__ __forceinline__ Round round_of(const EncodeParams& p, uint32_t r) {
    Round q;
    q.l0 = r * p.layers_per_round;
    q.nl = (p.L - q.l0 < p.layers_per_round) ? p.L - q.l0 : p.layers_per_round;
    q.nblk = q.nl * p.blocks_per_layer;
    return q;
}

__device__ __forceinline__ uint32_t lds_load(const uint32_t* a) {
    return __hip_atomic_load(a, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Record that a wait inside the workgroup gave up (never expected). The
// wait for all of the wave's memory operations makes the flag performed
// before the wave's later work (the end-of-kernel checks below read it).
// (Waiting here, inside the rare branch, rather than on a returned value
// keeps the common path free of a full wait that would drain the
// prefetched loads.)
__device__ __forceinline__ void note_gave_up(const EncodeParams& p, uint32_t* lds_gave_up) {
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p.ws + kWsGaveUp), p.call, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    if (p.status) atomicOr(p.status, kDevTimeout);
    __builtin_amdgcn_s_waitcnt(0);
    *lds_gave_up = 1;
}

// Block bi of every round: its layer within the round, its block within the
// layer, head and first token. The same in every round (only the layer,
// l0 + lr, moves), so a wave works it out once, not at every use.
struct SlotBlock {
    uint32_t lr, bidx, h, t0;
};

__device__ __forceinline__ SlotBlock slot_block(const EncodeParams& p, uint32_t bi) {
    SlotBlock g;
    g.lr = bi / p.blocks_per_layer;
    g.bidx = bi % p.blocks_per_layer;
    g.h = g.bidx / p.nb;
    g.t0 = (g.bidx % p.nb) * kBlockTokens;
    return g;
}

// block_pos for a block whose head and first token are known
template <int D>
__device__ __forceinline__ BlockPos block_pos_at(const EncodeParams& p, uint32_t l, const SlotBlock& g, uint32_t lane) {
    BlockPos b;
    b.l = l;
    b.bidx = g.bidx;
    b.m = lane & 3u;
    b.nv = (p.T - g.t0 < kBlockTokens) ? p.T - g.t0 : kBlockTokens;
    b.vec0 = ((uint64_t)l * p.H + g.h) * p.T + g.t0;
    b.vec = b.vec0 + (lane >> 2);
    b.valid = g.t0 + (lane >> 2) < p.T;
    b.elem = (b.valid ? b.vec : b.vec0) * D + (uint64_t)b.m * (D / 4);
    return b;
}

// Block g in round r (clamped: a block past the round's end, or a round past
// the last, is block 0 of layer 0, loaded and never used). Block bi is in
// round r's range exactly when its layer lr is below the round's layers.
template <int D>
__device__ __forceinline__ BlockPos fused_block(const EncodeParams& p, uint32_t r, uint32_t nrounds, const SlotBlock& g,
                                                uint32_t lane) {
    const bool live_round = r < nrounds;
    const Round q = round_of(p, live_round ? r : 0);
    const bool live = live_round && g.lr < q.nl;
    const SlotBlock z = {0u, 0u, 0u, 0u};
    return block_pos_at<D>(p, live ? q.l0 + g.lr : 0u, live ? g : z, lane);
}

// Logical workgroup of the single-pass encode's block mapping. Workgroups
// are dealt to the 8 XCDs in turn; read this way each XCD covers a
// contiguous eighth of every round's blocks (when the grid divides by 8),
// so its L2 sees neighbouring blocks (1.5-3.5 us on the Llama 4K pool). The
// exchange words stay indexed by the physical workgroup.
__device__ __forceinline__ uint32_t fused_wg() {
    return (gridDim.x % 8u == 0) ? (blockIdx.x % 8u) * (gridDim.x / 8u) + blockIdx.x / 8u : blockIdx.x;
}

template <int D>
struct ValueRaw {
    uint4 v[FusedLds<D>::kBpw][D / 32];
};

template <int D>
struct KeyRaw {
    uint4 k[kSlotsPerKeyWave][FusedLds<D>::kBpw][D / 32];
};

// Value wave: slot vw's values, round after round, one round of loads in
// flight; no wait on any other wave.
template <int D>
__device__ __forceinline__ void value_round(const EncodeParams& p, FusedLds<D>& sm, uint32_t vw, uint32_t lane,
                                            uint32_t r, uint32_t nrounds, const SlotBlock (&g)[FusedLds<D>::kBpw],
                                            ValueRaw<D>& cur, ValueRaw<D>& fill) {
#pragma unroll
    for (int j = 0; j < FusedLds<D>::kBpw; ++j)
        load_lane<D>(p.v, fused_block<D>(p, r + 1, nrounds, g[j], lane).elem, fill.v[j]);
    const Round q = round_of(p, r);
#pragma unroll
    for (int j = 0; j < FusedLds<D>::kBpw; ++j) {
        if (g[j].lr < q.nl) {
            const BlockPos b = block_pos_at<D>(p, q.l0 + g[j].lr, g[j], lane);
            encode_values<D>(p, b, cur.v[j], sm.stage[vw], lane);
        }
    }
}

template <int D>
__device__ __forceinline__ void fused_value_wave(const EncodeParams& p, FusedLds<D>& sm, uint32_t vw, uint32_t lane,
                                                 uint32_t nrounds) {
    const uint32_t NW = gridDim.x * kFusedSlots;
    const uint32_t gw = fused_wg() * kFusedSlots + vw;
    SlotBlock g[FusedLds<D>::kBpw];
#pragma unroll
    for (int j = 0; j < FusedLds<D>::kBpw; ++j) g[j] = slot_block(p, gw + (uint32_t)j * NW);
    ValueRaw<D> a, b;
#pragma unroll
    for (int j = 0; j < FusedLds<D>::kBpw; ++j)
        load_lane<D>(p.v, fused_block<D>(p, 0, nrounds, g[j], lane).elem, a.v[j]);
    for (uint32_t r = 0; r < nrounds; r += 2) {
        value_round<D>(p, sm, vw, lane, r, nrounds, g, a, b);
        if (r + 1 < nrounds) value_round<D>(p, sm, vw, lane, r + 1, nrounds, g, b, a);
    }
}

// Key wave kw, iteration r: round r+1's key loads go out first, then
// round r's keys are parked and their maxima folded in, then round r-3's
// keys are quantised: a round of work separates the wave's count for a
// round from its wait for that round's maxima.
template <int D>
__device__ __forceinline__ void key_round(const EncodeParams& p, FusedLds<D>& sm, uint32_t kw, uint32_t lane,
                                          uint32_t r, uint32_t nrounds,
                                          const SlotBlock (&g)[kSlotsPerKeyWave][FusedLds<D>::kBpw], KeyRaw<D>& cur,
                                          KeyRaw<D>& fill) {
    constexpr int BPW = FusedLds<D>::kBpw;
#pragma unroll
    for (int i = 0; i < kSlotsPerKeyWave; ++i)
#pragma unroll
        for (int j = 0; j < BPW; ++j) load_lane<D>(p.k, fused_block<D>(p, r + 1, nrounds, g[i][j], lane).elem, fill.k[i][j]);
    if (r < nrounds) {
        const Round q = round_of(p, r);
#pragma unroll
        for (int i = 0; i < kSlotsPerKeyWave; ++i) {
            const uint32_t slot = kw * kSlotsPerKeyWave + i;
#pragma unroll
            for (int j = 0; j < BPW; ++j) {
                if (g[i][j].lr < q.nl) {
                    const uint32_t lr = g[i][j].lr;
                    const BlockPos b = block_pos_at<D>(p, q.l0 + lr, g[i][j], lane);
                    const uint32_t m = wave_max_u32(b.valid ? lane_absmax_bits<D / 32>(cur.k[i][j]) : 0u);
#pragma unroll
                    for (int c = 0; c < D / 32; ++c) sm.hold[r % kHoldRounds][slot][j][c][lane] = cur.k[i][j][c];
                    if (lane == 0)
                        __hip_atomic_fetch_max(&sm.wg_max[r % kHoldRounds][lr], m, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_WORKGROUP);
                }
            }
        }
        // LDS operations of a wave complete in order: the maxima above land
        // before the count
        if (lane == 0) __hip_atomic_fetch_add(&sm.done[r % kHoldRounds], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (r >= (uint32_t)kQuantLag) {
        const uint32_t rq = r - kQuantLag;
        const uint64_t start = wall_clock64();
        while (lds_load(&sm.ready) < rq + 1) {
            if (wall_clock64() - start > kWaitTicks) {
                note_gave_up(p, &sm.gave_up);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        const Round q = round_of(p, rq);
#pragma unroll
        for (int i = 0; i < kSlotsPerKeyWave; ++i) {
            const uint32_t slot = kw * kSlotsPerKeyWave + i;
#pragma unroll
            for (int j = 0; j < BPW; ++j) {
                if (g[i][j].lr < q.nl) {
                    const uint32_t lr = g[i][j].lr;
                    const BlockPos b = block_pos_at<D>(p, q.l0 + lr, g[i][j], lane);
                    uint4 kr[D / 32];
#pragma unroll
                    for (int c = 0; c < D / 32; ++c) kr[c] = sm.hold[rq % kHoldRounds][slot][j][c][lane];
                    quantize_keys<D>(p, b, kr, lds_load(&sm.layer_max[rq % kHoldRounds][lr]), sm.stage[slot], lane);
                }
            }
        }
    }
}

template <int D>
__device__ __forceinline__ void fused_key_wave(const EncodeParams& p, FusedLds<D>& sm, uint32_t kw, uint32_t lane,
                                               uint32_t nrounds) {
    // two register sets, alternating, one round of loads in flight (the loop
    // is unrolled by two so that both stay in registers)
    const uint32_t NW = gridDim.x * kFusedSlots;
    SlotBlock g[kSlotsPerKeyWave][FusedLds<D>::kBpw];
#pragma unroll
    for (int i = 0; i < kSlotsPerKeyWave; ++i)
#pragma unroll
        for (int j = 0; j < FusedLds<D>::kBpw; ++j)
            g[i][j] = slot_block(p, fused_wg() * kFusedSlots + kw * kSlotsPerKeyWave + i + (uint32_t)j * NW);
    KeyRaw<D> a, b;
#pragma unroll
    for (int i = 0; i < kSlotsPerKeyWave; ++i)
#pragma unroll
        for (int j = 0; j < FusedLds<D>::kBpw; ++j) load_lane<D>(p.k, fused_block<D>(p, 0, nrounds, g[i][j], lane).elem, a.k[i][j]);
    for (uint32_t r = 0; r < nrounds + kQuantLag; r += 2) {
        key_round<D>(p, sm, kw, lane, r, nrounds, g, a, b);
        if (r + 1 < nrounds + kQuantLag) key_round<D>(p, sm, kw, lane, r + 1, nrounds, g, b, a);
    }
}

template <int D>
__device__ __forceinline__ void fused_coordinator(const EncodeParams& p, FusedLds<D>& sm, uint32_t lane,
                                                  uint32_t nrounds) {
    const uint32_t G = gridDim.x;
    for (uint32_t r = 0; r <= nrounds; ++r) {
        if (r < nrounds) {
            // the key waves' round r, then this workgroup's maxima of it, published
            const Round q = round_of(p, r);
            const uint64_t start = wall_clock64();
            while (lds_load(&sm.done[r % kHoldRounds]) < (uint32_t)kFusedKeyWaves) {
                if (wall_clock64() - start > kWaitTicks) {
                    note_gave_up(p, &sm.gave_up);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            uint32_t m = 0;
            if (lane < q.nl) m = lds_load(&sm.wg_max[r % kHoldRounds][lane]);
            if (lane < kMaxRoundLayers) sm.wg_max[r % kHoldRounds][lane] = 0;  // reused in round r + 4
            if (lane == 0) sm.done[r % kHoldRounds] = 0;
            if (lane < q.nl)
                __hip_atomic_store(round_flags(p.ws, gridDim.x, q.l0 + lane) + blockIdx.x,
                                   (p.call << 16) | kWordFlag | m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (r >= 1) {
            // every workgroup's maxima of round r-1, reduced per layer
            const uint32_t rq = r - 1;
            const Round q = round_of(p, rq);
            for (uint32_t lr = 0; lr < q.nl; ++lr) {
                const uint64_t* f = round_flags(p.ws, gridDim.x, q.l0 + lr);
                const uint64_t tag = (p.call << 16) | kWordFlag;  // this call's words: (word & ~0x7FFF) == tag
                // all of the layer's words at once (lane + 64 i), then again
                // for those not yet flagged
                constexpr int kPer = kMaxFusedGrid / kWave;
                uint64_t v[kPer];
#pragma unroll
                for (int i = 0; i < kPer; ++i) {
                    const uint32_t g = lane + (uint32_t)i * kWave;
                    v[i] = g < G ? __hip_atomic_load(f + g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : tag;
                }
                const uint64_t start = wall_clock64();
                bool all_flagged = false;
                for (;;) {
                    bool all = true;
#pragma unroll
                    for (int i = 0; i < kPer; ++i) all = all && ((v[i] & ~0x7FFFull) == tag);
                    if (p.poll_ticks != 0 && __builtin_amdgcn_ballot_w64(!all) == 0) {
                        all_flagged = true;
                        break;
                    }
                    if (wall_clock64() - start >= p.poll_ticks) break;
                    __builtin_amdgcn_s_sleep(1);
#pragma unroll
                    for (int i = 0; i < kPer; ++i) {
                        const uint32_t g = lane + (uint32_t)i * kWave;
                        if ((v[i] & ~0x7FFFull) != tag)
                            v[i] = __hip_atomic_load(f + g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
                uint32_t mx = 0;
                if (all_flagged) {
#pragma unroll
                    for (int i = 0; i < kPer; ++i) {
                        const uint32_t x = (uint32_t)(v[i] & 0x7FFFu);
                        mx = x > mx ? x : mx;
                    }
                    mx = wave_max_u32(mx);
                } else {
                    // some workgroup has not published (not resident yet, or
                    // slow): the layer's maximum from its keys instead
                    mx = layer_absmax_direct<D>(p, q.l0 + lr, lane);
                }
                if (lane == 0) sm.layer_max[rq % kHoldRounds][lr] = mx;
            }
            if (lane == 0)
                __hip_atomic_store(&sm.ready, rq + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    }
}

template <int D>
__global__ __launch_bounds__(kFusedThreads) void pool_encode_fused_kernel(EncodeParams p) {
    __shared__ FusedLds<D> sm;
    const uint32_t lane = lane_id();
    const uint32_t w = wave_uniform(threadIdx.x / kWave);
    const uint32_t nrounds = (p.L + p.layers_per_round - 1) / p.layers_per_round;
    if (threadIdx.x < kHoldRounds * kMaxRoundLayers) (&sm.wg_max[0][0])[threadIdx.x] = 0;
    if (threadIdx.x < kHoldRounds) sm.done[threadIdx.x] = 0;
    if (threadIdx.x == 0) sm.ready = 0;
    if (threadIdx.x == 0) sm.gave_up = 0;
    __syncthreads();
    if (w < (uint32_t)kFusedSlots)
        fused_value_wave<D>(p, sm, w, lane, nrounds);
    else if (w < (uint32_t)(kFusedSlots + kFusedKeyWaves))
        fused_key_wave<D>(p, sm, w - kFusedSlots, lane, nrounds);
    else
        fused_coordinator<D>(p, sm, lane, nrounds);
    // Header and padding last, by workgroup 0. A wait that gave up anywhere
    // leaves the header's magic word zero (decode then refuses the pool): a
    // workgroup whose wait gave up records this call's number in the head
    // and zeroes the magic at its end, after a device-scope fence;
    // workgroup 0 reads the head after writing the header and a fence.
    // Either workgroup 0 sees the record, or the other workgroup's zero
    // lands after the header. (Other workgroups that see the record zero
    // the magic too; only these two sides need the fences.)
    __syncthreads();
    if (blockIdx.x == 0 && threadIdx.x < kBlockThreads) {
        pool_header_and_padding(p, D, threadIdx.x);
        __threadfence();
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        if (blockIdx.x == 0 || sm.gave_up) __threadfence();
        if (__hip_atomic_load(reinterpret_cast<const uint64_t*>(p.ws + kWsGaveUp), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT) == p.call)
            __hip_atomic_store(reinterpret_cast<uint32_t*>(p.pool), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// The pool's header as kvpool_encode writes it (magic, version 1 kind 1,
// shape, total bytes).
__device__ __forceinline__ bool pool_header_valid(const uint8_t* pool, uint32_t L, uint32_t H, uint32_t T, uint32_t D,
                                                  uint64_t total) {
    const uint32_t* hd = reinterpret_cast<const uint32_t*>(pool);
    const uint64_t t = (uint64_t)hd[14] | ((uint64_t)hd[15] << 32);
    return hd[0] == kPoolMagic && hd[1] == (1u | (1u << 16)) && hd[2] == L && hd[3] == H && hd[4] == T &&
           hd[5] == D && t == total;
}

// KEEP: plain stores (a fan-out copy reads the output back at once); else
// non-temporal. A template argument, not a runtime flag: the compiler
// merges two otherwise identical store branches and drops the hint.
template <int D, bool KEEP>
__global__ __launch_bounds__(kBlockThreads) void pool_decode_kernel(DecodeParams p) {
    constexpr int C = D / 4;
    const uint32_t lane = lane_id();
    const uint64_t wave = (uint64_t)blockIdx.x * (kBlockThreads / kWave) + wave_uniform(threadIdx.x / kWave);
    if (wave >= p.n_waves) return;

    uint64_t lh_rel, lq;
    uint32_t blk, hr;
    divmod_u64(wave, p.nb, lh_rel, blk);
    const uint64_t lh = (uint64_t)p.l0 * p.H + lh_rel;
    divmod_u64(lh, p.H, lq, hr);
    const uint32_t l = (uint32_t)lq;
    const uint32_t t0 = blk * kBlockTokens;
    const uint32_t m = lane & 3u;
    // lanes past the head's last token read the block's first vector (their
    // outputs are never stored)
    const bool valid = t0 + (lane >> 2) < p.T;
    const uint64_t vec = lh * p.T + (valid ? t0 + (lane >> 2) : t0);

    // The pool loads go out first; the header is checked while they are in
    // flight (nothing is written before it has passed).
    uint4 kraw[C / 16];
    {
        const uint4* src = reinterpret_cast<const uint4*>(p.pool + p.lay.k_codes + vec * D + (uint64_t)m * C);
#pragma unroll
        for (int i = 0; i < C / 16; ++i) kraw[i] = src[i];
    }
    uint32_t pw[3];
    {
        const uint8_t* codes = p.pool + p.lay.v_codes + vec * pool_code_bytes(D);
        if (D == 128) {
#pragma unroll
            for (int q = 0; q < 3; ++q) pw[q] = reinterpret_cast<const uint32_t*>(codes + 16 * q)[m];
        } else {
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                const uint32_t w = reinterpret_cast<const uint32_t*>(codes + 8 * q)[m >> 1];
                pw[q] = (m & 1u) ? (w & 0xFFFF0000u) : (w << 16);  // this lane's 16 bits on top
            }
        }
    }
    const uint16_t sbits = reinterpret_cast<const uint16_t*>(p.pool + p.lay.v_scale)[vec];
    const float ks = reinterpret_cast<const float*>(p.pool + p.lay.k_scale)[l];

    if (!pool_header_valid(p.pool, p.L, p.H, p.T, D, p.lay.total)) {
        if (lane == 0 && p.status) atomicOr(p.status, 1 /* KVC_DEV_BAD_HEADER */);
        return;
    }

    // Outputs are staged per wave in LDS (the lane-major 64-byte chunks form
    // the wave's contiguous 16-token output image) and stored so that each
    // store instruction covers one contiguous span across the wave: stores
    // where every lane writes its own 64-byte piece run at about half the
    // write bandwidth of coalesced ones.
    constexpr int CH = C / 8;  // 16-byte chunks per lane
    __shared__ uint4 stage[kBlockThreads / kWave][kWave * CH];
    uint4* st = stage[threadIdx.x / kWave];
    const uint32_t nv = (p.T - t0 < kBlockTokens) ? p.T - t0 : kBlockTokens;  // valid tokens of the block
    const uint64_t out_base = (lh_rel * p.T + t0) * D / 8;  // in 16-byte chunks

    // ---- keys: bf16(q * scale)
    {
        const uint32_t* w = reinterpret_cast<const uint32_t*>(kraw);
        uint32_t o[C / 2];
#pragma unroll
        for (int j = 0; j < C / 4; ++j) {
            const uint32_t q = w[j];
            const float f0 = (float)(int32_t)(int8_t)(q & 0xFF) * ks;
            const float f1 = (float)(int32_t)(int8_t)((q >> 8) & 0xFF) * ks;
            const float f2 = (float)(int32_t)(int8_t)((q >> 16) & 0xFF) * ks;
            const float f3 = (float)(int32_t)(int8_t)(q >> 24) * ks;
            o[2 * j] = pack_bf16x2(f0, f1);
            o[2 * j + 1] = pack_bf16x2(f2, f3);
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) st[stage_slot<CH>(lane, c)] = make_uint4(o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]);
    }
    uint4 kc[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) kc[j] = st[stage_pos<CH>(64 * j + lane)];

    // ---- values: level lookup by the code bits of this lane, then the
    // butterfly, then * (s / sqrt(d)).
    float c0 = kLv0, c1 = kLv1, c2 = kLv2, c3 = kLv3;
    asm volatile("" : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3));
    float y[C];
#pragma unroll
    for (int i = C - 1; i >= 0; --i) {
        const uint64_t w0 = shift_out_bit(pw[0]);
        const uint64_t w1 = shift_out_bit(pw[1]);
        const uint64_t w2 = shift_out_bit(pw[2]);
        // level index within the half: (b1, b0) for b2 = 1, complemented for b2 = 0
        const uint64_t m1 = ~(w1 ^ w2), m0 = ~(w0 ^ w2);
        const float lo = select_by_mask(m0, c0, c1);
        const float hi = select_by_mask(m0, c2, c3);
        const float mag = select_by_mask(m1, lo, hi);
        y[i] = signed_by_mask(w2, mag);
    }
    fwht_quad<C>(y, m);
    {
        const float a = (float)__builtin_bit_cast(_Float16, sbits) * inv_sqrt_d<D>() * fwht_quad_sign(m);
        uint32_t o[C / 2];
#pragma unroll
        for (int j = 0; j < C / 2; ++j) o[j] = pack_bf16x2(y[2 * j] * a, y[2 * j + 1] * a);
#pragma unroll
        for (int c = 0; c < CH; ++c) st[stage_slot<CH>(lane, c)] = make_uint4(o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]);
    }
    uint4 vc[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) vc[j] = st[stage_pos<CH>(64 * j + lane)];

    // chunk 64*j + lane of the image belongs to token (64*j + lane) / (4*CH).
    // (Writing each agent's spans back to back instead of interleaving the
    // agents per chunk measured about 1% slower.)
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        if ((64 * j + lane) / (4 * CH) < nv) {
            const uint4 kj = kc[j], vj = vc[j];
            for (uint32_t ag = 0; ag < p.n_out; ++ag) {
                uint4* kd = reinterpret_cast<uint4*>(p.k_out[ag]) + out_base + 64 * j + lane;
                uint4* vd = reinterpret_cast<uint4*>(p.v_out[ag]) + out_base + 64 * j + lane;
                if (KEEP) {
                    *kd = kj;
                    *vd = vj;
                } else {
                    st_stream(kd, kj);
                    st_stream(vd, vj);
                }
            }
        }
    }
}

// Fan-out (PolyKV 2.A: every agent injects the same decoded layers into its
// own cache). With many agents, the decode writes agent 0 only and this
// kernel copies agent 0's K and V to agents 1..n-1. Writing 2n streams from
// one wave measured 5.4-5.8 TB/s, while workgroups that each write one
// 4 KiB chunk of one stream, the streams taken in turn, reach 6-7 TB/s. So
// here a workgroup copies one 4 KiB chunk (one 16-byte load and store per
// thread) of one destination stream, and the grid is ordered so that each
// XCD (workgroups are dealt to the 8 XCDs round-robin) walks its share of
// the chunks in windows of kFanoutWindow chunks, every stream in turn per
// window: the window's source chunks come from HBM once and from that XCD's
// L2 for the other streams. (The mapping is only a performance assumption;
// any placement copies the same bytes.)
constexpr uint32_t kXcds = 8;
// 4 KiB chunks per XCD window: 1 MiB of source per XCD and stream turn
// (measured on 15 agents: 64: 1421 us, 128: 1380, 192-384: 1333-1338, 512: 2115)
constexpr uint32_t kFanoutWindow = 256;
constexpr uint32_t kFanoutMinAgents = 8;  // below this the decode writes every agent itself (measured: fused wins at 4, fan-out at 8 and 15)

struct FanoutParams {
    const uint8_t* pool;  // header re-checked: nothing is copied after a refused decode
    uint32_t L, H, T, D;
    uint64_t total;
    const uint4* src[2];                // agent 0's K and V
    uint4* dst[2 * (kMaxAgents - 1)];   // stream 2 (a - 1) + kv for agent a
    uint64_t n16;                       // 16-byte units per stream
    uint64_t per_xcd;                   // chunks per XCD share
    uint32_t streams, window;
};

__global__ __launch_bounds__(kBlockThreads) void fanout_copy_kernel(FanoutParams p) {
    const uint32_t xcd = blockIdx.x % kXcds;
    const uint32_t i = blockIdx.x / kXcds;  // the grid has fewer than 2^31 workgroups
    const uint32_t ci = i % p.window, t = i / p.window;
    const uint32_t s = t % p.streams;
    const uint64_t local = (uint64_t)(t / p.streams) * p.window + ci;
    if (local >= p.per_xcd) return;
    const uint64_t e = ((uint64_t)xcd * p.per_xcd + local) * kBlockThreads + threadIdx.x;
    if (e >= p.n16) return;
    // load first, check the header while the load is in flight
    const uint4 x = p.src[s & 1u][e];
    if (!pool_header_valid(p.pool, p.L, p.H, p.T, p.D, p.total)) return;
    st_stream(p.dst[s] + e, x);
}

// ---------------------------------------------------------------- layered encode
//
// Shapes whose layer does not fit a round of the single pass (long contexts:
// a Llama 32K layer holds 67 MB of keys) still read each key once from HBM.
// One ordinary launch lays its workgroups out in layer order,
//     [max 0] [max 1][encode 0] [max 2][encode 1] ... [max L-1][encode L-2] [encode L-1],
// A workgroups of each "max" segment, E of each "encode" segment. A "max l"
// workgroup reads its share of layer l's keys and publishes the share's
// largest magnitude as a tagged word, (call << 16) | 0x8000 | bits, one per
// (layer, workgroup). The segment's last workgroup then reads the layer's A
// words until all carry this call's number and publishes their maximum as
// one more tagged word, the layer's. An "encode l" workgroup (one 16-token
// block per wave) issues its key and value loads, reads the layer's word
// until it carries this call's number, quantises the keys and encodes the
// values. Measured on the Llama 32K pool: 1226 us against 1377 us for a
// key-maximum pass over all layers followed by the encode (the keys read
// twice from HBM), bit-identical; one word per layer rather than the A
// share words read by every encode wave: fewer instructions per block.
// Workgroups are dispatched in order on each XCD, so a wave waits only on
// workgroups dispatched before it (the layer's word: about one segment
// earlier); and the keys it re-reads were read by the max workgroups one
// period before, with the period's other traffic (one layer's values, pool
// and the next layer's keys) in between, within the 256 MB Infinity Cache.
// A wait that runs past the poll bound reads the layer's keys itself (an
// encode wave) or publishes nothing (the last max workgroup): the maximum
// is exact either way, residency decides only the speed.
__device__ __forceinline__ uint64_t* layered_words(uint32_t* ws, uint32_t A, uint32_t l) {
    return reinterpret_cast<uint64_t*>(ws + kWsHead) + (uint64_t)l * A;
}
// The layer's word, after all layers' share words.
__device__ __forceinline__ uint64_t* layered_layer_word(uint32_t* ws, uint32_t A, uint32_t L, uint32_t l) {
    return reinterpret_cast<uint64_t*>(ws + kWsHead) + (uint64_t)L * A + l;
}

template <int D>
__global__ __launch_bounds__(kBlockThreads) void pool_encode_layered_kernel(EncodeParams p) {
    constexpr int WPB = kBlockThreads / kWave;
    __shared__ EncodeStage<D> stage_all[WPB];
    __shared__ uint32_t red[WPB];
    const uint32_t lane = lane_id();
    const uint32_t wib = wave_uniform(threadIdx.x / kWave);
    if (blockIdx.x == 0) pool_header_and_padding(p, D, threadIdx.x);
    const uint32_t A = p.absmax_groups, E = p.encode_groups;
    // this workgroup's role, layer and index within its segment
    bool is_max;
    uint32_t layer, idx;
    {
        const uint64_t b = blockIdx.x, per = (uint64_t)A + E;
        if (b < A) {
            is_max = true;
            layer = 0;
            idx = (uint32_t)b;
        } else if (b - A < (uint64_t)(p.L - 1) * per) {
            const uint64_t q = (b - A) / per, m = (b - A) % per;
            is_max = m < A;
            layer = is_max ? (uint32_t)q + 1 : (uint32_t)q;
            idx = is_max ? (uint32_t)m : (uint32_t)(m - A);
        } else {
            is_max = false;
            layer = p.L - 1;
            idx = (uint32_t)(b - A - (uint64_t)(p.L - 1) * per);
        }
    }
    const uint64_t tag = (p.call << 16) | kWordFlag;
    if (is_max) {
        // share idx of the layer's keys (16-byte units), 8 loads in flight per thread
        const uint64_t n = (uint64_t)p.H * p.T * (D / 8);
        const uint64_t per_g = (n + A - 1) / A;
        const uint64_t lo = (uint64_t)idx * per_g, hi = lo + per_g < n ? lo + per_g : n;
        const uint4* src = reinterpret_cast<const uint4*>(p.k) + (uint64_t)layer * n;
        uint32_t m = 0;
        for (uint64_t i0 = lo + threadIdx.x; i0 < hi; i0 += 8 * kBlockThreads) {
            uint4 w[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint64_t i = i0 + (uint64_t)j * kBlockThreads;
                w[j] = src[i < hi ? i : hi - 1];  // past the share: its last unit again (max is idempotent)
            }
            const uint32_t x = lane_absmax_bits<8>(w);
            m = x > m ? x : m;
        }
        m = wave_max_u32(m);
        if (lane == 0) red[wib] = m;
        __syncthreads();
        if (threadIdx.x == 0) {
#pragma unroll
            for (int w = 1; w < WPB; ++w) m = red[w] > m ? red[w] : m;
            __hip_atomic_store(layered_words(p.ws, A, layer) + idx, tag | m, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
        if (idx != A - 1 || wib != 0 || p.poll_ticks == 0) return;
        // the segment's last workgroup, one wave: the layer's word from the
        // A share words (lane i reads words i, i + 64, ...)
        constexpr int kPer = kLayeredMaxGroups / kWave;
        const uint64_t* f = layered_words(p.ws, A, layer);
        const uint64_t start = wall_clock64();
        for (;;) {
            bool all = true;
            uint32_t mx = 0;
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const uint32_t g = lane + (uint32_t)i * kWave;
                const uint64_t w = g < A ? __hip_atomic_load(f + g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : tag;
                all = all && ((w & ~0x7FFFull) == tag);
                const uint32_t x = (uint32_t)(w & 0x7FFFu);
                mx = x > mx ? x : mx;
            }
            if (__builtin_amdgcn_ballot_w64(!all) == 0) {
                mx = wave_max_u32(mx);
                if (lane == 0)
                    __hip_atomic_store(layered_layer_word(p.ws, A, p.L, layer), tag | mx, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                return;
            }
            if (wall_clock64() - start >= p.poll_ticks) return;
            __builtin_amdgcn_s_sleep(1);
        }
    }
    const uint32_t blk = idx * WPB + wib;
    if (blk >= p.blocks_per_layer) return;
    const BlockPos b = block_pos<D>(p, layer, blk, lane);
    uint4 kraw[D / 32], vraw[D / 32];
    load_lane<D>(p.k, b.elem, kraw);
    load_lane<D>(p.v, b.elem, vraw);
    // the layer's word (one address for the wave), again until it carries
    // this call's number or the poll bound runs out
    const uint64_t* f = layered_layer_word(p.ws, A, p.L, layer);
    const uint64_t start = wall_clock64();
    uint32_t mx = 0;
    bool flagged = false;
    if (p.poll_ticks != 0) {
        for (;;) {
            const uint64_t w = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t lo = wave_uniform((uint32_t)w), hi = wave_uniform((uint32_t)(w >> 32));
            if ((((uint64_t)hi << 32 | lo) & ~0x7FFFull) == tag) {
                mx = lo & 0x7FFFu;
                flagged = true;
                break;
            }
            if (wall_clock64() - start >= p.poll_ticks) break;
            __builtin_amdgcn_s_sleep(1);
        }
    }
    if (!flagged) mx = layer_absmax_direct<D>(p, layer, lane);
    // keys first: their registers are free before the value transform's
    quantize_keys<D>(p, b, kraw, mx, stage_all[wib], lane);
    encode_values<D>(p, b, vraw, stage_all[wib], lane);
}

// Bound on a coordinator's wait for the other workgroups' key maxima, in
// ticks of the 100 MHz constant clock. Default 200 us: a resident grid
// publishes a round within a few microseconds, so the bound trips only for
// a workgroup that is not running. KVC_ENCODE_POLL_US overrides it; 0 makes
// every coordinator compute each layer's maximum itself (tests use it).
// Values above kMaxPollUs are ignored: a round of up to kMaxRoundLayers
// layers, each waited for this long and then read directly (a few hundred
// microseconds), must stay well inside the 0.5 s guard of the key waves'
// wait for their coordinator.
constexpr uint64_t kMaxPollUs = 5000;

// Call numbers of the single-pass encode (the tags of its exchange words):
// consecutive within one instance of the library, 48 bits, never 0 (a
// zeroed workspace word never matches). Each instance starts at a random
// point, so a workspace used by one instance and then by another holds no
// word carrying the other's current tag, bar a 2^-48 coincidence.
static uint64_t first_call_number() {
    uint64_t x = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
    try {
        std::random_device rd;
        x ^= ((uint64_t)rd() << 32) ^ (uint64_t)rd();
    } catch (...) {
    }
    return x;
}
uint64_t next_call_number() {
    static std::atomic<uint64_t> counter{first_call_number()};
    for (;;) {
        const uint64_t c = counter.fetch_add(1, std::memory_order_relaxed) & 0xFFFFFFFFFFFFull;
        if (c != 0) return c;
    }
}
uint64_t encode_poll_ticks() {
    uint64_t us = 200;
    if (const char* e = std::getenv("KVC_ENCODE_POLL_US")) {
        char* end = nullptr;
        const unsigned long long v = std::strtoull(e, &end, 10);
        if (end != e && *end == '\0' && v <= kMaxPollUs) us = v;
    }
    return us * 100;
}

}  // namespace

// Device address of `scratch` on the current device, looked up once per
// device with that device current (in host code the array's name is only a
// stand-in for the symbol, not a device address).
hipError_t noalloc_scratch(uint32_t** out) {
    constexpr int kMaxDevices = 64;
    static std::atomic<uint32_t*> ptrs[kMaxDevices];
    static std::mutex mu;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    uint32_t* p = ptrs[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(mu);
        p = ptrs[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            void* addr = nullptr;
            e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            p = static_cast<uint32_t*>(addr);
            ptrs[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

hipError_t launch_pool_encode(const Shape& s, const void* k, const void* v, void* pool, uint32_t* ws,
                              int32_t* dev_status, hipStream_t stream) {
    EncodeParams p;
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.pool = static_cast<uint8_t*>(pool);
    p.ws = ws;
    p.status = dev_status;
    p.L = s.L;
    p.H = s.H;
    p.T = s.T;
    p.nb = pool_blocks_per_head(s.T);
    p.blocks_per_layer = s.H * p.nb;
    p.layers_per_round = 0;
    p.n_waves = (uint64_t)s.L * p.blocks_per_layer;
    p.poll_ticks = encode_poll_ticks();
    p.absmax_groups = 0;
    p.encode_groups = 0;
    p.call = next_call_number();
    p.lay = pool_layout(s.L, s.H, s.T, s.d);

    // Single pass when a round of whole layers fits the LDS of a grid of one
    // workgroup per CU; otherwise the layered encode. Both are ordinary
    // launches whose waits never depend on a workgroup dispatched after the
    // waiting one (see the kernels). The single pass's exchange words (two
    // u32 words per layer and workgroup) must fit each layer's share.
    const void* fused = s.d == 64 ? reinterpret_cast<const void*>(pool_encode_fused_kernel<64>)
                                  : reinterpret_cast<const void*>(pool_encode_fused_kernel<128>);
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fused, kFusedThreads, 0) == hipSuccess && per_cu > 0 &&
        2 * (uint64_t)cus * (uint64_t)per_cu <= kWsWordsPerLayer &&
        (uint64_t)cus * (uint64_t)per_cu <= kMaxFusedGrid) {
        const uint64_t grid = (uint64_t)cus * (uint64_t)per_cu;
        const uint64_t per_round = grid * kFusedSlots * (128u / s.d);  // blocks a round can hold
        uint64_t lpr = per_round / p.blocks_per_layer;
        if (lpr > kMaxRoundLayers) lpr = kMaxRoundLayers;
        if (lpr > s.L) lpr = s.L;
        if (lpr >= 1) {
            p.layers_per_round = (uint32_t)lpr;
            void* argv[] = {&p};
            return report_launch(hipLaunchKernel(fused, dim3((uint32_t)grid), dim3(kFusedThreads), argv, 0, stream),
                                 "pool_encode_fused_kernel");
        }
    }
    // Layered: per layer, A key-maximum workgroups (each 16 16-byte units
    // per thread or more, at most kLayeredMaxGroups) and the encode
    // workgroups, in layer order in one launch.
    const uint64_t per_layer_u4 = (uint64_t)s.H * s.T * s.d / 8;
    uint64_t A = (per_layer_u4 + 16 * kBlockThreads - 1) / (16 * kBlockThreads);
    if (A > kLayeredMaxGroups) A = kLayeredMaxGroups;
    if (A == 0) A = 1;
    const uint64_t E = (p.blocks_per_layer + kBlockThreads / kWave - 1) / (kBlockThreads / kWave);
    p.absmax_groups = (uint32_t)A;
    p.encode_groups = (uint32_t)E;
    const uint64_t nblocks = (uint64_t)s.L * (A + E);
    if (nblocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
    return launch_kernel(s.d == 64 ? pool_encode_layered_kernel<64> : pool_encode_layered_kernel<128>,
                         dim3((uint32_t)nblocks), dim3(kBlockThreads), stream, p);
}

hipError_t launch_pool_decode(const Shape& s, const void* pool, uint32_t l0, uint32_t l1,
                              void* const* k_out, void* const* v_out, uint32_t n_out,
                              int32_t* dev_status, hipStream_t stream) {
    DecodeParams p;
    p.pool = static_cast<const uint8_t*>(pool);
    p.status = dev_status;
    p.L = s.L;
    p.H = s.H;
    p.T = s.T;
    p.nb = pool_blocks_per_head(s.T);
    p.l0 = l0;
    p.n_waves = (uint64_t)(l1 - l0) * s.H * p.nb;
    p.lay = pool_layout(s.L, s.H, s.T, s.d);

    // fan-out copy plan (see fanout_copy_kernel)
    FanoutParams f{};
    f.n16 = (uint64_t)(l1 - l0) * s.H * s.T * s.d * 2 / 16;
    const uint64_t chunks = (f.n16 + kBlockThreads - 1) / kBlockThreads;
    f.per_xcd = (chunks + kXcds - 1) / kXcds;
    f.window = (uint32_t)(f.per_xcd < kFanoutWindow ? f.per_xcd : kFanoutWindow);
    f.streams = 2 * (n_out - 1);
    const uint64_t fgrid = (uint64_t)kXcds * ((f.per_xcd + f.window - 1) / f.window) * f.streams * f.window;
    const bool fanout = n_out >= kFanoutMinAgents && fgrid <= 0x7FFFFFFFull;

    p.n_out = fanout ? 1 : n_out;
    for (uint32_t a = 0; a < (uint32_t)kMaxAgents; ++a) {
        p.k_out[a] = a < p.n_out ? static_cast<uint16_t*>(k_out[a]) : nullptr;
        p.v_out[a] = a < p.n_out ? static_cast<uint16_t*>(v_out[a]) : nullptr;
    }
    const uint64_t nblocks = (p.n_waves + 3) / 4;
    // agent 0's output is read back at once by the fan-out copy: plain
    // stores leave it in the caches for that (15 agents: 1378 -> 1350 us);
    // without a fan-out the non-temporal hint is faster (one agent:
    // 131 -> 107 us)
    void (*kernel)(DecodeParams) =
        s.d == 64 ? (fanout ? pool_decode_kernel<64, true> : pool_decode_kernel<64, false>)
                  : (fanout ? pool_decode_kernel<128, true> : pool_decode_kernel<128, false>);
    hipError_t e = launch_kernel(kernel,
                                 dim3((uint32_t)nblocks), dim3(kBlockThreads), stream, p);
    if (e != hipSuccess || !fanout) return e;

    f.pool = p.pool;
    f.L = s.L;
    f.H = s.H;
    f.T = s.T;
    f.D = s.d;
    f.total = p.lay.total;
    f.src[0] = static_cast<const uint4*>(k_out[0]);
    f.src[1] = static_cast<const uint4*>(v_out[0]);
    for (uint32_t a = 1; a < n_out; ++a) {
        f.dst[2 * (a - 1)] = static_cast<uint4*>(k_out[a]);
        f.dst[2 * (a - 1) + 1] = static_cast<uint4*>(v_out[a]);
    }
    return launch_kernel(fanout_copy_kernel, dim3((uint32_t)fgrid), dim3(kBlockThreads), stream, f);
}

}  // namespace kvc
