// kernels_common.h - device helpers shared by the pool and CacheCard kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

namespace kvc {

// Wave64: lanes 4t..4t+3 handle one head vector (token t of a 16-token
// block); quad-local exchanges use DPP quad permutes.
constexpr int kWave = 64;
constexpr int kBlockThreads = 256;  // 4 waves per workgroup

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

// DPP quad_perm selectors: xor-1 = [1,0,3,2], xor-2 = [2,3,0,1]
__device__ __forceinline__ float dpp_xor1(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_xor2(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
}
__device__ __forceinline__ uint32_t dpp_xor1_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 r;
    r.x = (__bf16)lo;
    r.y = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}

// Per-lane select from a wave-uniform 64-bit lane mask: bit `lane` of mask
// set -> b, clear -> a.
__device__ __forceinline__ float select_by_mask(uint64_t mask, float a, float b) {
    float r;
    asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(mask));
    return r;
}
// bit set -> +m, clear -> -m
__device__ __forceinline__ float signed_by_mask(uint64_t mask, float m) {
    float r;
    asm("v_cndmask_b32_e64 %0, -%1, %1, %2" : "=v"(r) : "v"(m), "s"(mask));
    return r;
}

// acc * 2 + (bit `lane` of mask): appends one code bit per lane (the mask is
// a wave-wide compare result) in a single add-with-carry.
__device__ __forceinline__ uint32_t shift_in_bit(uint32_t acc, uint64_t mask) {
    uint32_t r;
    uint64_t carry_out;
    asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(carry_out) : "v"(acc), "s"(mask));
    return r;
}

// w * 2, returning the lanes' former top bits as a wave mask (carry out).
__device__ __forceinline__ uint64_t shift_out_bit(uint32_t& w) {
    uint32_t r;
    uint64_t mask;
    asm("v_add_co_u32_e64 %0, %1, %2, %2" : "=v"(r), "=s"(mask) : "v"(w));
    w = r;
    return mask;
}

// Cross-lane butterfly step on 8 registers in one instruction each:
// y[i] <- partner(y[i]) * s + y[i] with the partner read through DPP
// (v_fmac_f32 with a DPP source). With s = -1 this yields own - partner,
// the negation of the butterfly's partner - own; callers track that sign
// per lane. The leading s_nop covers the DPP read-after-VALU-write hazard
// for registers written just before the block; within the block no
// register is read through DPP within two instructions of its write.
#define KVC_FMAC_DPP8(NAME, PERM)                                                                     \
    __device__ __forceinline__ void NAME(float* y, float s) {                                         \
        asm("s_nop 1\n"                                                                               \
            "v_fmac_f32_dpp %0, %0, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n"               \
            "v_fmac_f32_dpp %1, %1, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n"               \
            "v_fmac_f32_dpp %2, %2, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n"               \
            "v_fmac_f32_dpp %3, %3, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n"               \
            "v_fmac_f32_dpp %4, %4, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n"               \
            "v_fmac_f32_dpp %5, %5, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n"               \
            "v_fmac_f32_dpp %6, %6, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n"               \
            "v_fmac_f32_dpp %7, %7, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf"                  \
            : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3]), "+v"(y[4]), "+v"(y[5]), "+v"(y[6]),   \
              "+v"(y[7])                                                                              \
            : "v"(s));                                                                                \
    }
KVC_FMAC_DPP8(fmac_dpp8_xor1, "[1,0,3,2]")
KVC_FMAC_DPP8(fmac_dpp8_xor2, "[2,3,0,1]")
#undef KVC_FMAC_DPP8

// Launch and return this launch's own status (hipGetLastError would also
// report errors left behind by unrelated earlier runtime calls).
// With KVC_DEBUG set in the environment a failing launch prints the HIP
// error text to stderr.
inline hipError_t report_launch(hipError_t e, const char* what) {
    if (e != hipSuccess && getenv("KVC_DEBUG"))
        fprintf(stderr, "kvcodec: launch of %s failed: %s (%d)\n", what, hipGetErrorString(e), (int)e);
    return e;
}

template <typename... Args>
inline hipError_t launch_kernel(void (*kernel)(Args...), dim3 grid, dim3 block, hipStream_t stream,
                                Args... args) {
    void* argv[] = {static_cast<void*>(&args)...};
    return report_launch(hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, stream),
                         "kernel");
}

__device__ __forceinline__ uint32_t wave_uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// Swizzled per-wave LDS staging of an output image of 64 * N 16-byte chunks,
// where lane l produces chunks l*N .. l*N + N - 1 and lane i later reads
// chunks 64j + i. Chunk c of lane l goes to slot (c + l / (16 / N)) mod N of
// the lane's N slots: without it the lanes of one 16-lane LDS cycle write at
// a stride of N chunks and meet in the same banks (N-way conflicts); with it
// they cover all 64 banks, and the reads stay within one 256-byte run.
template <int N>
__device__ __forceinline__ uint32_t stage_slot(uint32_t l, uint32_t c) {
    constexpr uint32_t S = N == 4 ? 2 : (N == 2 ? 3 : 4);
    return l * N + ((c + (l >> S)) & (N - 1));
}
template <int N>
__device__ __forceinline__ uint32_t stage_pos(uint32_t p) {
    return stage_slot<N>(p / N, p % N);
}

// Stores of the big outputs (written once, not read again by the same
// kernel) carry the non-temporal hint. Measured on MI355X over the codec
// step: encode 194 -> 170 us, card pack 192 -> 153 us, one-agent decode
// 130 -> 108 us. The same hint on loads made every kernel slower (the
// fan-out copy, which re-reads agent 0's freshly written output, 1.8x), so
// loads are plain.
typedef uint32_t kvc_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st_stream(uint4* p, const uint4& x) {
    __builtin_nontemporal_store(kvc_u32x4{x.x, x.y, x.z, x.w}, reinterpret_cast<kvc_u32x4*>(p));
}
__device__ __forceinline__ void st_stream(uint32_t* p, uint32_t x) { __builtin_nontemporal_store(x, p); }

// q = x / d and r = x % d for a wave-uniform x: 32-bit arithmetic when x
// fits (the case in practice), 64-bit otherwise.
__device__ __forceinline__ void divmod_u64(uint64_t x, uint32_t d, uint64_t& q, uint32_t& r) {
    if (x <= 0xFFFFFFFFull) {
        q = (uint32_t)x / d;
        r = (uint32_t)x % d;
    } else {
        q = x / d;
        r = (uint32_t)(x % d);
    }
}

}  // namespace kvc
