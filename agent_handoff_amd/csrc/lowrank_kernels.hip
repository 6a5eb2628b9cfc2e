// lowrank_kernels.hip - low-rank anchor materialisation for gfx950 (MFMA).
//
// KVCMAS (cache reuse across agents), "low-rank anchor" storage: a stored
// cache matrix Z (T tokens x D = H*d channels of one layer's K or V) is kept
// as the truncated SVD factors A = U_r S_r (T x r) and R = R_r (D x r),
// Z ~ A R^T, and a reused cache is corrected by a similarity-weighted sum
// of stored anchors. This kernel materialises, for every matrix m,
//
//     out = bf16( src + sum_v w_v * (A_v R_v^T) )
//
// with src and out in the cache layout [H][T][d] and A_v R_v^T a dense
// contraction over r, done on the matrix cores: v_mfma_f32_16x16x32_bf16
// (bf16 operands, binary32 accumulation). Each anchor's product is reduced
// over r on its own, then scaled by its binary32 weight and added in
// binary32 (fmaf), anchors in index order; src is added last and the sum is
// rounded once to bf16, ties to even.
//
// Work mapping. A workgroup owns one head of one matrix over a chunk of
// token tiles (at Llama-3-8B sizes a chunk is the whole sequence, one
// workgroup per CU): its source and output are one contiguous block of
// [H][T][d]. The anchors' R rows for that head (V x d x r bf16) are staged
// once into LDS in MFMA-fragment order, so every operand read is a
// lane-contiguous ds_read_b128. A wave owns NJ token blocks of 16 tokens
// per tile and all d channels, computed transposed: out^T block = R_block
// (16 channels x r) * A_block^T (r x 16 tokens). At r = 32, where the LDS
// has room, a workgroup runs 12 waves (three per SIMD): 8 compute waves own
// one block each (128-token tiles) and hand each finished block, through a
// double-buffered LDS staging area and a pair of flags, to one of 4 store
// waves, which write it out with non-temporal stores. The compute waves
// then never wait behind their own output stores (a wave's memory counter
// retires in order, so a store in flight delays the wait for the next A
// fragments). Otherwise 8 waves own two blocks each and store their own
// output (256-token tiles, two waves per SIMD, each R fragment read from
// LDS serving two blocks). MFMA row i of channel block cb is channel
// (d/4)(i/4) + 4cb + i%4, which leaves lane l holding token l%16 and the
// d/4 consecutive channels from (d/4)(l/16) on, so source loads are 16-byte
// accesses. The (tile, anchor) steps of a chunk form one pipeline: A
// fragments are requested five steps ahead (at r = 32), a tile's source at
// the last step of the tile before, its output staged (and, without store
// waves, stored) at its last. Matrices are dealt to XCDs (workgroup b runs
// on XCD b % 8) so that the 8 heads sharing one matrix's A factors run on
// one XCD and re-read them from its L2.
#include "kernels_common.h"
#include "launch.h"

namespace kvc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kXcds = 8;
constexpr uint64_t kLdsBytes = 160 * 1024;
// third word of a raw buffer resource on the gfx9 family: 32-bit data
// format, no swizzle, bounds checked against the record count in bytes
constexpr int kBufferWord3 = 0x00020000;
constexpr uint64_t kLowrankTargetGroups = 256;  // one workgroup per CU

struct LowrankParams {
    const uint16_t* src;  // [M][H][T][d]
    const uint16_t* a;    // [M][V][T][r]
    const uint16_t* rf;   // [M][V][H*d][r]
    const float* w;       // [M][V]
    uint16_t* out;        // [M][H][T][d]
    uint32_t M, H, T, V, r;
    uint32_t tiles;       // ceil(T / tile tokens)
    uint32_t chunks;      // token chunks per (matrix, head)
    uint32_t chunk_tiles; // tiles per chunk
    uint32_t stage_row;   // 16-byte chunks between token rows of the output staging
};

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// waves per workgroup with NJ token blocks per wave
constexpr int lr_waves(int nj) { return nj == 2 ? 8 : 12; }
// the store-wave split at one token block per wave: 8 waves compute, 4
// write the output
constexpr int kSwCompute = 8, kSwStore = 4;
constexpr uint64_t kFlagWaitTicks = 50000000;  // 0.5 s
static_assert(kSwCompute + kSwStore == lr_waves(1) && kSwCompute == 2 * kSwStore, "store waves serve two compute waves each");

template <int D, int KC, int NJ, bool SW = false>
__global__ __launch_bounds__(lr_waves(NJ) * kWave) void lowrank_materialize_kernel(LowrankParams p) {
    constexpr int W = lr_waves(NJ);
    constexpr int THR = W * kWave;
    constexpr int WC = SW ? kSwCompute : W;   // compute waves
    constexpr int TT = WC * NJ * 16;  // tile tokens
    constexpr int NCB = D / 16;   // channel blocks of 16
    constexpr int CPL = D / 4;    // channels per lane in the output layout
    constexpr int SQ = CPL / 8;   // 16-byte source chunks per lane and token
    extern __shared__ u32x4 frag[];  // [V][r/32][NCB][64 lanes], then the waves' output staging

    // workgroup -> (matrix, token chunk, head), matrices grouped by XCD
    const uint32_t b = blockIdx.x;
    const uint32_t per_matrix = p.chunks * p.H;
    const uint32_t m = b % kXcds + kXcds * ((b / kXcds) / per_matrix);
    if (m >= p.M) return;
    const uint32_t rem = (b / kXcds) % per_matrix;
    const uint32_t chunk = rem / p.H, h = rem % p.H;
    const uint32_t tile0 = chunk * p.chunk_tiles;
    if (tile0 >= p.tiles) return;
    const uint32_t n_tiles = min(p.chunk_tiles, p.tiles - tile0);
    const uint64_t HD = (uint64_t)p.H * D;

    // stage R rows h*d .. h*d + d - 1 of every anchor into fragment order:
    // fragment (v, kc, cb), lane i + 16 g holds channel (d/4)(i/4) + 4cb + i%4,
    // k = 32 kc + 8 g .. + 7
    {
        const uint32_t per_anchor = D * p.r / 8;  // 16-byte chunks
        const uint32_t total = p.V * per_anchor;
        const uint32_t qpr = p.r / 8;             // chunks per row
        for (uint32_t c0 = 0; c0 < total; c0 += 8 * THR) {
            u32x4 x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint32_t c = min(c0 + u * THR + threadIdx.x, total - 1);
                const uint32_t v = c / per_anchor, rest = c % per_anchor;
                const uint32_t row = rest / qpr, q = rest % qpr;
                x[u] = ld16(p.rf + (((uint64_t)m * p.V + v) * HD + (uint64_t)h * D + row) * p.r + q * 8);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint32_t c = c0 + u * THR + threadIdx.x;
                if (c < total) {
                    const uint32_t v = c / per_anchor, rest = c % per_anchor;
                    const uint32_t row = rest / qpr, q = rest % qpr;
                    const uint32_t kc = q / 4, g = q % 4;
                    const uint32_t i = 4 * (row / CPL) + row % 4, cb = (row % CPL) / 4;
                    frag[((v * KC + kc) * NCB + cb) * kWave + i + 16 * g] = x[u];
                }
            }
        }
    }
    if (SW) {
        uint32_t* fl = reinterpret_cast<uint32_t*>(frag + p.V * KC * NCB * kWave + WC * 2 * 16 * p.stage_row);
        if (threadIdx.x < 4 * WC) fl[threadIdx.x] = 0;
    }
    __syncthreads();

    const uint32_t lane = lane_id();
    const uint32_t wave = wave_uniform(threadIdx.x / kWave);
    const uint32_t g = lane / 16;
    const uint32_t row_in_tile = wave * 16 * NJ + lane % 16;  // + 16 j
    const uint16_t* src = p.src + ((uint64_t)m * p.H + h) * p.T * D;
    uint16_t* out = p.out + ((uint64_t)m * p.H + h) * p.T * D;
    const uint16_t* a = p.a + (uint64_t)m * p.V * p.T * p.r;
    const uint32_t S = n_tiles * p.V;  // pipeline steps

    // A fragments of step s (tile s / V, anchor s % V): token row of the
    // block, k = 32 kc + 8 g .. + 7; rows past T (and steps past the end)
    // are clamped to valid ones and their results discarded
    // A of one step as a buffer (scalar registers): it starts at the step's
    // tile of the step's anchor and holds the rows from there to T (at most
    // T x r bf16, under 2^31 bytes, checked at the call); this lane's row and
    // k are a constant vector offset, so an address costs no vector
    // instructions. Rows past T fall past the buffer's end, which the range
    // check on the vector offset turns into zeros; their results are never
    // stored.
    uint32_t a_off[NJ][KC];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) a_off[j][kc] = ((row_in_tile + 16 * j) * p.r + 32 * kc + 8 * g) * 2;
    auto load_a = [&](uint32_t s, u32x4 (&x)[NJ][KC]) {
        s = min(s, S - 1);
        const uint32_t tile = tile0 + s / p.V, v = s % p.V;
        const uint32_t row0 = tile * TT;  // below T: s is clamped to the last step
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a + ((uint64_t)v * p.T + row0) * p.r), (short)0,
                                              (int)((p.T - row0) * p.r * 2), kBufferWord3);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
                x[j][kc] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)a_off[j][kc], 0, 0);
    };
    u32x4 rc[KC][NCB];
    auto load_r = [&](uint32_t v) {
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) rc[kc][cb] = frag[((v * KC + kc) * NCB + cb) * kWave + lane];
    };
    // source chunks of a tile, requested at the last step of the tile before
    // it (as soon as that tile's own are consumed, and ahead of its output
    // stores, which later waits would otherwise also wait for) and used at
    // its last; at r = 64 the registers hold operands, and the source is
    // read at the last step
    constexpr bool kEarlySrc = KC == 1;
    u32x4 sv[NJ][SQ];
    auto load_src_block = [&](uint32_t tile, int j) {
        const uint32_t t = min(tile * TT + row_in_tile + 16 * j, p.T - 1);
#pragma unroll
        for (int q = 0; q < SQ; ++q) sv[j][q] = ld16(src + (uint64_t)t * D + g * CPL + 8 * q);
    };
    auto load_src = [&](uint32_t tile) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) load_src_block(tile, j);
    };

    float acc[NJ][NCB][4];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[j][cb][e] = 0.0f;

    // lane holds token t, channels (d/4) g + 4cb + e: add the source, round
    // once. The 16 tokens of a block are one contiguous 16 x d image of the
    // output; it goes through the wave's LDS staging (token rows p.stage_row
    // chunks apart: one chunk more than a row where the LDS has room, so that
    // the writers - 16 tokens, one chunk each - fall in different banks) and
    // out with each store covering a contiguous 1 KiB. Stores where every
    // lane writes its own d/2-byte piece ran at about half the write
    // bandwidth.
    constexpr uint32_t CR = D / 8;  // 16-byte chunks per token row
    constexpr uint32_t TPS = kWave / CR;  // token rows per store instruction
    const uint32_t SR = p.stage_row;
    u32x4* stage_base = frag + p.V * KC * NCB * kWave;
    u32x4* stg = stage_base + wave * 16 * SR;
    u32x4* stg_w = stg + (lane % 16) * SR + g * SQ;       // this lane's chunks
    u32x4* stg_r = stg + (lane / CR) * SR + lane % CR;    // chunk lane of rows 0, TPS, ...
    // With store waves: compute wave c stages the k-th tile of its chunk in
    // buffer k % 2 and sets f_ready[c][k % 2] = k + 1; its store wave writes
    // the block out and sets f_done[c][k % 2] = k + 1, after which the buffer
    // may take tile k + 2. Both flags only grow. Every wait is bounded
    // (kFlagWaitTicks of the 100 MHz clock, far beyond any tile's time), so
    // the grid drains whatever happens.
    uint32_t* flags = reinterpret_cast<uint32_t*>(stage_base + (SW ? WC * 2 : 0) * 16 * SR);
    uint32_t* f_ready = flags;            // [WC][2]
    uint32_t* f_done = flags + 2 * WC;    // [WC][2]
    if (SW && wave >= (uint32_t)WC) {
        // store wave sw serves compute waves 2 sw and 2 sw + 1, tile after tile
        const uint32_t sw = wave - WC;
        for (uint32_t k = 0; k < n_tiles; ++k) {
            const uint32_t tile = tile0 + k, buf = k & 1;
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const uint32_t c = 2 * sw + cc;
                const uint64_t t0c = wall_clock64();
                while (__hip_atomic_load(&f_ready[c * 2 + buf], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < k + 1) {
                    if (wall_clock64() - t0c > kFlagWaitTicks) break;
                    __builtin_amdgcn_s_sleep(1);
                }
                const u32x4* sr = stage_base + (c * 2 + buf) * 16 * SR + (lane / CR) * SR + lane % CR;
                u32x4 x[SQ];
#pragma unroll
                for (int u = 0; u < SQ; ++u) x[u] = sr[u * TPS * SR];
                const uint32_t tb = tile * TT + c * 16;
                u32x4* dst = reinterpret_cast<u32x4*>(out + (uint64_t)tb * D) + lane;
#pragma unroll
                for (int u = 0; u < SQ; ++u)
                    if (tb + (kWave * u + lane) / CR < p.T) __builtin_nontemporal_store(x[u], dst + kWave * u);
                // the staging reads are complete before the buffer is handed back
                // (the clobber keeps the flag store below the wait)
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                if (lane == 0) __hip_atomic_store(&f_done[c * 2 + buf], k + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
        return;
    }
    auto store_tile = [&](uint32_t tile) {
        if (SW) {
            const uint32_t k = tile - tile0, buf = k & 1;
            u32x4* sb = stage_base + (wave * 2 + buf) * 16 * SR + (lane % 16) * SR + g * SQ;
            if (k >= 2) {
                const uint64_t t0c = wall_clock64();
                while (__hip_atomic_load(&f_done[wave * 2 + buf], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < k - 1) {
                    if (wall_clock64() - t0c > kFlagWaitTicks) break;
                    __builtin_amdgcn_s_sleep(1);
                }
            }
#pragma unroll
            for (int q = 0; q < SQ; ++q) {
                const uint32_t sw[4] = {sv[0][q].x, sv[0][q].y, sv[0][q].z, sv[0][q].w};
                uint32_t o[4];
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const int cb = 2 * q + e2 / 2, e = 2 * (e2 % 2);
                    o[e2] = pack_bf16x2(bf16_lo(sw[e2]) + acc[0][cb][e], bf16_hi(sw[e2]) + acc[0][cb][e + 1]);
                }
                sb[q] = u32x4{o[0], o[1], o[2], o[3]};
            }
            if (kEarlySrc) load_src_block(tile + 1, 0);
            // the staged rows are in LDS before the flag says so
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (lane == 0) __hip_atomic_store(&f_ready[wave * 2 + buf], k + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[0][cb][e] = 0.0f;
            return;
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const uint32_t tb = tile * TT + wave * 16 * NJ + 16 * j;  // the block's first token
#pragma unroll
            for (int q = 0; q < SQ; ++q) {
                const uint32_t sw[4] = {sv[j][q].x, sv[j][q].y, sv[j][q].z, sv[j][q].w};
                uint32_t o[4];
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const int cb = 2 * q + e2 / 2, e = 2 * (e2 % 2);
                    o[e2] = pack_bf16x2(bf16_lo(sw[e2]) + acc[j][cb][e], bf16_hi(sw[e2]) + acc[j][cb][e + 1]);
                }
                stg_w[q] = u32x4{o[0], o[1], o[2], o[3]};
            }
            if (kEarlySrc) load_src_block(tile + 1, j);
            __builtin_amdgcn_wave_barrier();
            u32x4 x[SQ];
#pragma unroll
            for (int u = 0; u < SQ; ++u) x[u] = stg_r[u * TPS * SR];
            u32x4* dst = reinterpret_cast<u32x4*>(out + (uint64_t)tb * D) + lane;
#pragma unroll
            for (int u = 0; u < SQ; ++u)
                if (tb + (kWave * u + lane) / CR < p.T) dst[kWave * u] = x[u];
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[j][cb][e] = 0.0f;
        }
    };

    // weights: lane v holds w_v; each is moved to a scalar register in turn
    const float wl = p.w[(uint64_t)m * p.V + min(lane, p.V - 1)];

    // NSET register sets of A fragments in a ring: step s computes with set
    // s % NSET and requests step s + NSET - 1 into the set step s - 1 used.
    // The loop is unrolled by NSET so that the set index is a constant. The
    // first sets pass through an empty asm so that the compiler keeps the
    // loop-carried sets in registers (it would otherwise merge the loads
    // feeding one into a single load at the loop head, just before its use).
    constexpr int NSET = KC == 1 ? 6 : 2;
    u32x4 set[NSET][NJ][KC];
#pragma unroll
    for (int u = 0; u + 1 < NSET; ++u) load_a(u, set[u]);
    load_r(0);
    if (kEarlySrc) load_src(tile0);
#pragma unroll
    for (int u = 0; u + 1 < NSET; ++u)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) asm volatile("" : "+v"(set[u][j][kc]));
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) asm volatile("" : "+v"(rc[kc][cb]));

    auto step = [&](uint32_t s, const u32x4 (&ca)[NJ][KC], u32x4 (&na)[NJ][KC]) {
        const uint32_t tile = tile0 + s / p.V, v = s % p.V;
        load_a(s + NSET - 1, na);
        f32x4 t[NJ][NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                t[j][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, rc[0][cb]),
                                                                   __builtin_bit_cast(bf16x8, ca[j][0]),
                                                                   f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
                for (int kc = 1; kc < KC; ++kc)
                    t[j][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, rc[kc][cb]),
                                                                       __builtin_bit_cast(bf16x8, ca[j][kc]),
                                                                       t[j][cb], 0, 0, 0);
            }
        load_r(v + 1 == p.V ? 0 : v + 1);
        const float wv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), v));
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[j][cb][e] = fmaf(wv, t[j][cb][e], acc[j][cb][e]);
        if (v + 1 == p.V) {
            if (!kEarlySrc) load_src(tile);
            store_tile(tile);
        }
    };
    // whole rounds of NSET steps, then the remainder (fewer than NSET), so
    // that no step inside the loop is conditional
    uint32_t s = 0;
    for (; s + NSET <= S; s += NSET) {
#pragma unroll
        for (int u = 0; u < NSET; ++u) step(s + u, set[u], set[(u + NSET - 1) % NSET]);
    }
#pragma unroll
    for (int u = 0; u + 1 < NSET; ++u)
        if (s + u < S) step(s + u, set[u], set[(u + NSET - 1) % NSET]);
}

}  // namespace

uint64_t lowrank_lds_bytes(uint32_t d, uint32_t V, uint32_t r) { return (uint64_t)V * d * r * 2; }

// the output staging beside the R fragments, per buffer 16 token rows of
// row_chunks 16-byte chunks each (d / 8, or one more where it fits)
static uint64_t lowrank_stage_bytes(uint32_t row_chunks, uint32_t buffers) { return (uint64_t)buffers * 16 * row_chunks * 16; }

hipError_t launch_lowrank_materialize(uint32_t M, uint32_t H, uint32_t T, uint32_t d, uint32_t V, uint32_t r,
                                      const void* src, const void* a, const void* rf, const float* w, void* out,
                                      hipStream_t stream) {
    LowrankParams p{};
    p.src = static_cast<const uint16_t*>(src);
    p.a = static_cast<const uint16_t*>(a);
    p.rf = static_cast<const uint16_t*>(rf);
    p.w = w;
    p.out = static_cast<uint16_t*>(out);
    p.M = M;
    p.H = H;
    p.T = T;
    p.V = V;
    p.r = r;
    // at r = 32, where the double-buffered staging of the 8 compute waves
    // and the flags fit beside the R fragments, one token block per compute
    // wave and 4 store waves; else two blocks per wave (8 waves, each
    // staging and storing its own output)
    const uint64_t rb = lowrank_lds_bytes(d, V, r);
    const uint64_t flag_bytes = 4 * sizeof(uint32_t) * kSwCompute;
    const bool nj1 = r == 32 && rb + lowrank_stage_bytes(d / 8, 2 * kSwCompute) + flag_bytes <= kLdsBytes;
    const uint32_t waves = lr_waves(nj1 ? 1 : 2), tt = (nj1 ? kSwCompute : waves * 2) * 16;
    p.tiles = (T + tt - 1) / tt;
    // enough (matrix, head, chunk) items to give every CU one workgroup
    const uint64_t mh = (uint64_t)M * H;
    const uint64_t per_mh = (kLowrankTargetGroups + mh - 1) / mh;
    const uint32_t want = (uint32_t)(per_mh < p.tiles ? per_mh : p.tiles);
    p.chunk_tiles = (p.tiles + want - 1) / want;
    p.chunks = (p.tiles + p.chunk_tiles - 1) / p.chunk_tiles;
    const uint64_t groups = (M + kXcds - 1) / kXcds;
    const uint64_t nblocks = groups * kXcds * p.chunks * H;
    if (nblocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
    const uint32_t stage_buffers = nj1 ? 2 * kSwCompute : waves;
    const uint64_t fb = nj1 ? flag_bytes : 0;
    p.stage_row = rb + lowrank_stage_bytes(d / 8 + 1, stage_buffers) + fb <= kLdsBytes ? d / 8 + 1 : d / 8;
    const uint32_t lds = (uint32_t)(rb + lowrank_stage_bytes(p.stage_row, stage_buffers) + fb);
    void (*kernel)(LowrankParams) =
        d == 64 ? (r == 64 ? lowrank_materialize_kernel<64, 2, 2> : (nj1 ? lowrank_materialize_kernel<64, 1, 1, true> : lowrank_materialize_kernel<64, 1, 2>))
                : (r == 64 ? lowrank_materialize_kernel<128, 2, 2> : (nj1 ? lowrank_materialize_kernel<128, 1, 1, true> : lowrank_materialize_kernel<128, 1, 2>));
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return report_launch(e, "lowrank_materialize (LDS attribute)");
    void* argv[] = {&p};
    return report_launch(hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3((uint32_t)nblocks),
                                         dim3(waves * kWave), argv, lds, stream),
                         "lowrank_materialize");
}

}  // namespace kvc
