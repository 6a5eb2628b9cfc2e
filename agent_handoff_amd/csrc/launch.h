// launch.h - internal launchers behind the C ABI (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

struct Shape {
    uint32_t L, H, T, d;
};

constexpr int kMaxAgents = 64;

// Pool encode: ws is the encode workspace (encode_workspace_words(L) u32
// words, zero before its first use, written by each call with words tagged
// by that call's number).
hipError_t launch_pool_encode(const Shape& s, const void* k, const void* v, void* pool, uint32_t* ws,
                              int32_t* dev_status, hipStream_t stream);

// kvpool_encode_noalloc: the library's per-GPU encode workspace (1 MiB,
// enough for kvpool_workspace_bytes of up to 255 layers) and its device
// address on the current device.
constexpr uint64_t kNoAllocScratchBytes = 1ull << 20;
hipError_t noalloc_scratch(uint32_t** out);

hipError_t launch_pool_decode(const Shape& s, const void* pool, uint32_t l0, uint32_t l1,
                              void* const* k_out, void* const* v_out, uint32_t n_out,
                              int32_t* dev_status, hipStream_t stream);

// CacheCard workspace: 256-byte info block {u64 S, u64 total, u32 flags},
// then u64 record offsets[T + 1], rounded up to 256 bytes. The transcode
// uses two of these (input card, output card).
constexpr uint64_t kCardInfoBytes = 256;
inline uint64_t card_workspace_half(uint32_t T) { return (kCardInfoBytes + 8ull * ((uint64_t)T + 1) + 255) & ~255ull; }

struct CardMetaDev {
    char model_id[64];
    int64_t position_offset;
};

hipError_t launch_card_pack(const Shape& s, const void* k, const void* v, const uint8_t* widths,
                            const CardMetaDev& meta, void* card, uint64_t capacity,
                            uint64_t* dev_card_bytes, int32_t* dev_status, void* ws,
                            hipStream_t stream);

hipError_t launch_card_unpack(const Shape& s, const void* card, uint64_t card_bytes, void* k_out,
                              void* v_out, int32_t* dev_status, void* ws, hipStream_t stream);

hipError_t launch_card_transcode(const Shape& s, const void* card_in, uint64_t card_in_bytes,
                                 const uint8_t* new_widths, void* card_out, uint64_t capacity,
                                 uint64_t* dev_card_bytes, int32_t* dev_status, void* ws, hipStream_t stream);

// Key re-alignment: at most 64 channel pairs (d <= 128); inv_freq is a host
// array of d/2 inverse frequencies, delta the positions to move by.
constexpr int kMaxRealignPairs = 64;
hipError_t launch_realign_keys(const Shape& s, const void* k_in, void* k_out, int64_t delta, const float* inv_freq,
                               uint32_t pairing, hipStream_t stream);

// Low-rank anchor materialisation over M matrices of T x (H*d); r is 32 or
// 64, V <= 32 (the weights sit one per lane), and V anchors' R rows for one
// head (V*d*r*2 bytes) must fit in the LDS budget.
constexpr uint64_t kLowrankMaxLds = 128 * 1024;
constexpr uint32_t kLowrankMaxAnchors = 32;
uint64_t lowrank_lds_bytes(uint32_t d, uint32_t V, uint32_t r);
hipError_t launch_lowrank_materialize(uint32_t M, uint32_t H, uint32_t T, uint32_t d, uint32_t V, uint32_t r,
                                      const void* src, const void* a, const void* rf, const float* w, void* out,
                                      hipStream_t stream);

// Rank-32 truncated SVD of M matrices T x (H*d) (randomized range finder,
// 48-column Gaussian sketch supplied by the caller). Workspace offsets in
// bytes (256-aligned) and total.
constexpr uint32_t kLowrankSketch = 48;
struct LowrankFactorWs {
    uint64_t y, w, part, rinv, gpart, ua, ur, sigma, total;
};
LowrankFactorWs lowrank_factor_ws(uint32_t M, uint32_t H, uint32_t T, uint32_t d);
hipError_t launch_lowrank_factor(uint32_t M, uint32_t H, uint32_t T, uint32_t d, const void* z, const float* omega,
                                 void* a_out, uint64_t a_stride, void* r_out, uint64_t r_stride, float* sigma_out,
                                 void* ws, hipStream_t stream);

}  // namespace kvc
