// layout.h - byte layouts of the pool and the CacheCard, shared by the host
// entry points and the kernels of libkvcodec (see include/kvcodec.h for the
// format description).
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define KVC_HD __host__ __device__ inline
#else
#define KVC_HD inline
#endif

namespace kvc {

constexpr uint32_t kPoolMagic = 0x4C50564Bu;  // "KVPL"
constexpr uint32_t kCardMagic = 0x43564B51u;  // "QKVC"
constexpr uint32_t kPoolHeaderBytes = 64;
constexpr uint32_t kCardHeaderBytes = 256;
constexpr uint32_t kCardGroup = 32;
constexpr uint32_t kBlockTokens = 16;  // tokens per wave in the pool kernels (4 lanes per vector)

KVC_HD uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

struct PoolLayout {
    uint64_t k_scale, k_codes, v_scale, v_codes, total;
};

KVC_HD bool pool_shape_ok(uint32_t L, uint32_t H, uint32_t T, uint32_t d) {
    return L >= 1 && H >= 1 && T >= 1 && (d == 64 || d == 128) && L <= (1u << 16) &&
           H <= (1u << 16) && T <= (1u << 26);
}

KVC_HD uint32_t pool_blocks_per_head(uint32_t T) { return (T + kBlockTokens - 1) / kBlockTokens; }

// value-code bytes of one vector: 3 bit planes of d bits
KVC_HD uint32_t pool_code_bytes(uint32_t d) { return 3u * d / 8u; }

KVC_HD PoolLayout pool_layout(uint32_t L, uint32_t H, uint32_t T, uint32_t d) {
    PoolLayout p;
    const uint64_t vecs = (uint64_t)L * H * T;
    p.k_scale = 256;
    p.k_codes = align_up(p.k_scale + 4ull * L, 256);
    p.v_scale = align_up(p.k_codes + vecs * d, 256);
    p.v_codes = align_up(p.v_scale + 2ull * vecs, 256);
    p.total = align_up(p.v_codes + vecs * pool_code_bytes(d), 256);
    return p;
}

// kvpool_encode workspace: 64 head words, then 1024 words per layer for the
// 64-bit exchange words of one path per call: one per workgroup of the
// single-pass encode (at most 512), or one per key-maximum workgroup of the
// layered encode (at most 256).
KVC_HD uint64_t encode_workspace_words(uint32_t L) { return 64u + (uint64_t)L * 1024u; }

KVC_HD bool card_shape_ok(uint32_t L, uint32_t H, uint32_t T, uint32_t d) {
    return L >= 1 && H >= 1 && T >= 1 && (d == 64 || d == 128) && L <= (1u << 16) &&
           H <= (1u << 16) && T <= (1u << 26);
}

// record bytes of one vector at width b; 0 for an invalid width
KVC_HD uint32_t card_record_bytes(uint32_t d, uint32_t b) {
    if (b == 16) return 2u * d;
    if (b != 2 && b != 4 && b != 8) return 0;
    const uint32_t raw = 4u * (d / kCardGroup) + d * b / 8u;
    return (raw + 15u) & ~15u;
}

KVC_HD uint64_t card_payload_offset(uint32_t T) { return align_up(kCardHeaderBytes + (uint64_t)T, 256); }

}  // namespace kvc
