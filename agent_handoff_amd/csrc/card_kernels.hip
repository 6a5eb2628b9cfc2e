// card_kernels.hip - CacheCard pack / unpack for gfx950.
//
// QKVShare (gist.science/ko/paper/2605.03884), method items 1-3: every token
// has a bit-width in {2, 4, 8, FP16}; the CacheCard carries the quantised KV
// groups, the widths and metadata; the receiver rebuilds full-width
// past_key_values. Groups here are 32 consecutive channels quantised with
// min-max (asymmetric) steps; width 16 keeps the bf16 input.
//
// Offsets. Records are variable-sized, so token t's record starts at the sum
// of the record sizes of tokens 0..t-1 (the same in every stream, since the
// width is per token). For cards of up to kInGridTokens tokens every pack /
// unpack workgroup sums the record sizes before its own tokens from the
// widths itself (workgroup 0 writes the header and widths); longer cards,
// and the transcode, take them from a single-workgroup scan kernel that
// writes them once into the workspace. The pack / unpack kernels place one
// record per (layer, K/V, head, token).
//
// Work mapping: one lane per 32-channel group (d/32 lanes per token, so 16
// tokens per wave at d = 128); a lane loads its 64 input bytes, finds the
// group's min and max in registers, and places its scale, minimum and codes
// in the wave's LDS image of its records, which the wave then stores as one
// contiguous span. All lanes of a token share its width, so a wave branches
// once per distinct width it holds (widths come in runs).
#include "kernels_common.h"
#include "launch.h"
#include "layout.h"

namespace kvc {
namespace {

constexpr uint32_t kFlagBadHeader = 1, kFlagBadWidth = 2, kFlagCapacity = 4;
constexpr uint32_t kStatusBits = kFlagBadHeader | kFlagBadWidth | kFlagCapacity;

// Workgroups are dealt to the 8 XCDs in turn, so consecutive token blocks
// of a stream would land on different XCDs (their L2s each fetching the
// cache lines that neighbouring spans share, their writes scattered). The
// pack and unpack grids are instead read in an order that gives each XCD
// runs of C consecutive logical workgroups: XCD x's r-th workgroup is
// logical workgroup ((r / C) * 8 + x) * C + r % C, a bijection onto
// [0, gridDim) for a grid padded to a multiple of 8 C (workgroups past the
// work exit). Measured on the Llama 4K card with the configs' width mix:
// unpack 151 -> 132 us with C = 64 (one stream of 4096 tokens per run; 16:
// 134, 128: 136), pack 144 -> 135 us with C = 16, transcode 130 -> 126 us
// with C = 64. The transcode runs one wave per workgroup: a workgroup's LDS
// is released only when its slowest wave ends, and the transcode's waves
// differ in length with their widths (99.1 -> 92.3 us; pack and unpack,
// shorter and alike, run slower that way: 134 -> 139, 128 -> 134 us).
constexpr uint32_t kXcdCount = 8;
constexpr uint32_t kUnpackXcdRun = 64;
constexpr uint32_t kPackXcdRun = 16;
constexpr uint32_t kTranscodeXcdRun = 256;  // one-wave workgroups: one stream per run
constexpr int kTranscodeThreads = kWave;

template <uint32_t C>
__device__ __forceinline__ uint64_t xcd_run_block(uint32_t b) {
    const uint32_t r = b / kXcdCount;
    return ((uint64_t)(r / C) * kXcdCount + b % kXcdCount) * C + r % C;
}

template <uint32_t C>
inline uint32_t xcd_run_grid(uint64_t workgroups) {
    const uint64_t pad = (uint64_t)kXcdCount * C;
    return (uint32_t)((workgroups + pad - 1) / pad * pad);
}
constexpr int kScanThreads = 1024;
constexpr int kScanItems = 8;

struct ScanParams {
    const uint8_t* widths;     // pack: input widths; unpack: card + 256
    uint8_t* card_out;         // pack: card to receive header and widths; unpack: null
    const uint8_t* card_in;    // unpack: card whose header is checked; pack: null
    uint64_t* info;            // ws: S, total, flags
    uint64_t* off;             // ws: record offsets [T + 1]
    uint64_t limit;            // pack: capacity; unpack: card bytes
    uint64_t* dev_card_bytes;  // pack, nullable
    int32_t* status;           // nullable
    uint32_t L, H, T, d;
    CardMetaDev meta;
    const uint8_t* meta_src;   // transcode: card whose model ID and position offset are carried over
};

// One scan per workgroup: a transcode scans its input and its output card
// in one launch of two workgroups.
struct ScanLaunch {
    ScanParams s[2];
};

struct CardParams {
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* k_out;
    uint16_t* v_out;
    const uint8_t* widths;  // device widths (pack input or card + 256)
    uint8_t* card;          // pack: output card
    const uint8_t* card_in; // unpack: input card
    const uint64_t* info;
    const uint64_t* off;
    uint32_t L, H, T, nbk;  // nbk = token blocks per stream
    uint64_t payload;
    uint64_t n_waves;
    // offsets computed in the grid (see ingrid_scan): what the scan kernel
    // would otherwise check and write
    uint64_t limit;            // pack: capacity; unpack: card bytes
    uint64_t* dev_card_bytes;  // pack, nullable
    int32_t* status;           // nullable
    CardMetaDev meta;          // pack
};

// Word i (< 64) of a card's 256-byte header.
__device__ __forceinline__ uint32_t card_header_word(uint32_t i, uint32_t L, uint32_t H, uint32_t T, uint32_t d,
                                                     uint64_t payload, uint64_t S, uint64_t total,
                                                     const CardMetaDev& meta, const uint8_t* meta_src) {
    uint32_t val = 0;
    switch (i) {
        case 0: val = kCardMagic; break;
        case 1: val = 1u | (2u << 16); break;  // version 1, kind 2
        case 2: val = L; break;
        case 3: val = H; break;
        case 4: val = T; break;
        case 5: val = d; break;
        case 6: val = kCardGroup; break;
        case 8: val = (uint32_t)(uint64_t)meta.position_offset; break;
        case 9: val = (uint32_t)((uint64_t)meta.position_offset >> 32); break;
        case 10: val = kCardHeaderBytes; break;
        case 12: val = (uint32_t)payload; break;
        case 13: val = (uint32_t)(payload >> 32); break;
        case 14: val = (uint32_t)S; break;
        case 15: val = (uint32_t)(S >> 32); break;
        case 16: val = (uint32_t)total; break;
        case 17: val = (uint32_t)(total >> 32); break;
        default:
            if (i >= 18 && i < 34) {
                const int c = (int)(i - 18) * 4;
                val = (uint32_t)(uint8_t)meta.model_id[c] | ((uint32_t)(uint8_t)meta.model_id[c + 1] << 8) |
                      ((uint32_t)(uint8_t)meta.model_id[c + 2] << 16) |
                      ((uint32_t)(uint8_t)meta.model_id[c + 3] << 24);
            }
    }
    if (meta_src && (i == 8 || i == 9 || (i >= 18 && i < 34))) {
        val = reinterpret_cast<const uint32_t*>(meta_src)[i];
        if (i == 33) val &= 0x00FFFFFFu;  // at most 63 characters, NUL-terminated
    }
    return val;
}

// Whether a card's header matches the shape and the sizes its widths give.
__device__ __forceinline__ bool card_header_ok(const uint8_t* card, uint32_t L, uint32_t H, uint32_t T, uint32_t d,
                                               uint64_t payload, uint64_t S, uint64_t total, uint64_t limit) {
    const uint32_t* h = reinterpret_cast<const uint32_t*>(card);
    const uint64_t* h64 = reinterpret_cast<const uint64_t*>(card);
    return h[0] == kCardMagic && h[1] == (1u | (2u << 16)) && h[2] == L && h[3] == H && h[4] == T && h[5] == d &&
           h[6] == kCardGroup && h64[5] == kCardHeaderBytes && h64[6] == payload && h64[7] == S && h64[8] == total &&
           total <= limit;
}

// card_record_bytes as selects (the scan takes it for 8 tokens per thread;
// the branches of the general form cost a divergent region per token)
__device__ __forceinline__ uint32_t record_bytes_sel(uint32_t d, uint32_t b) {
    const uint32_t q = (4u * (d / kCardGroup) + d * b / 8u + 15u) & ~15u;
    const bool quant = (b == 2) | (b == 4) | (b == 8);
    return b == 16 ? 2u * d : (quant ? q : 0u);
}

// Inclusive sum over the wave's lanes in lane order, by DPP: partial sums
// within each row of 16 lanes (row_shr 1, 2, 4, 8; lanes whose source lies
// before the row take 0), then row 0's total into rows 1-3 and row 1's into
// rows 2-3 (row_bcast 15 and 31, rows selected by the row mask).
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

// The scan is one workgroup's chain of dependent steps (widths in, offsets
// out) ahead of the pack / unpack grid, so it is kept short: every thread
// works out the flags itself (no barrier to publish them), an invalid width
// travels with the waves' totals (bit 31) instead of through a shared flag
// that would need clearing first, and widths and offsets move 8 and 16 bytes
// per access.
__global__ __launch_bounds__(kScanThreads) void card_scan_kernel(ScanLaunch sl) {
    constexpr int kScanWaves = kScanThreads / kWave;
    constexpr uint32_t kBadBit = 0x80000000u;
    const ScanParams& p = sl.s[blockIdx.x];
    __shared__ uint32_t wave_tot[kScanWaves];
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid % kWave, w = tid / kWave;
    // The input card's header words (unpack and transcode), loaded first so
    // that their trip to memory overlaps the widths'.
    uint32_t hw[7] = {};
    uint64_t hq[4] = {};
    if (!p.card_out && tid == 0) {
        const uint32_t* h = reinterpret_cast<const uint32_t*>(p.card_in);
        const uint64_t* h64 = reinterpret_cast<const uint64_t*>(p.card_in);
#pragma unroll
        for (int i = 0; i < 7; ++i) hw[i] = h[i];
#pragma unroll
        for (int i = 0; i < 4; ++i) hq[i] = h64[5 + i];
    }
    // With at most one chunk of tokens (the common case) each thread keeps
    // its widths, which the pack then copies into the card from registers.
    const bool one_chunk = p.T <= (uint64_t)kScanThreads * kScanItems;
    const bool vec = ((uintptr_t)p.widths & 7) == 0;
    uint8_t wv[kScanItems] = {};
    // Chunks of kScanThreads * kScanItems tokens: each thread sums its
    // tokens' record sizes, the wave scans the sums with lane shifts, and the
    // waves' totals go through LDS. A chunk's bytes fit 31 bits (at most 8192
    // records of at most 512 bytes).
    uint64_t carry = 0;
    bool bad = false;
    for (uint64_t base = 0; base < p.T; base += (uint64_t)kScanThreads * kScanItems) {
        const uint64_t t0 = base + (uint64_t)tid * kScanItems;
        const bool whole = t0 + kScanItems <= p.T;
        if (vec && whole) {
            const uint2 u = *reinterpret_cast<const uint2*>(p.widths + t0);
#pragma unroll
            for (int i = 0; i < kScanItems; ++i) wv[i] = (uint8_t)((i < 4 ? u.x : u.y) >> (8 * (i % 4)));
        } else {
#pragma unroll
            for (int i = 0; i < kScanItems; ++i) wv[i] = t0 + i < p.T ? p.widths[t0 + i] : 0;
        }
        uint32_t rs[kScanItems];
        uint32_t local = 0;
        bool my_bad = false;
#pragma unroll
        for (int i = 0; i < kScanItems; ++i) {
            const bool in = t0 + i < p.T;
            const uint32_t r = record_bytes_sel(p.d, wv[i]);
            my_bad |= in & (r == 0);
            rs[i] = in ? r : 0u;
            local += rs[i];
        }
        const uint32_t inc = wave_inclusive_sum(local);
        const bool wave_bad = __builtin_amdgcn_ballot_w64(my_bad) != 0;
        if (lane == kWave - 1) wave_tot[w] = inc | (wave_bad ? kBadBit : 0u);
        __syncthreads();
        uint32_t before = 0, chunk = 0, bad_bits = 0;
#pragma unroll
        for (int k = 0; k < kScanWaves; ++k) {
            const uint32_t v = wave_tot[k];
            bad_bits |= v;
            before += (uint32_t)k < w ? (v & ~kBadBit) : 0u;
            chunk += v & ~kBadBit;
        }
        bad |= (bad_bits & kBadBit) != 0;
        uint64_t run = carry + before + inc - local;  // exclusive prefix of this thread
        uint64_t o[kScanItems];
#pragma unroll
        for (int i = 0; i < kScanItems; ++i) {
            o[i] = run;
            run += rs[i];
        }
        if (whole) {
            // 16-byte stores: off is 16-byte aligned and t0 a multiple of 8
#pragma unroll
            for (int i = 0; i < kScanItems; i += 2)
                *reinterpret_cast<ulonglong2*>(p.off + t0 + i) = make_ulonglong2(o[i], o[i + 1]);
        } else {
#pragma unroll
            for (int i = 0; i < kScanItems; ++i)
                if (t0 + i < p.T) p.off[t0 + i] = o[i];
        }
        carry += chunk;
        if (base + (uint64_t)kScanThreads * kScanItems < p.T) __syncthreads();  // wave_tot is reused
    }
    const uint64_t S = align_up(carry, 256);
    const uint64_t payload = card_payload_offset(p.T);
    const uint64_t total = payload + 2ull * p.L * p.H * S;
    uint32_t flags = bad ? kFlagBadWidth : 0u;
    if (p.card_out && total > p.limit) flags |= kFlagCapacity;
    if (tid == 0) {
        p.off[p.T] = carry;
        if (p.card_out) {
            if (p.dev_card_bytes) *p.dev_card_bytes = total;
            // a card that will not be written gets a zero magic word (the
            // buffer holds at least a header), so that nothing it held before
            // can pass for this call's output
            if (flags) reinterpret_cast<uint32_t*>(p.card_out)[0] = 0;
        } else {
            const bool ok = hw[0] == kCardMagic && hw[1] == (1u | (2u << 16)) && hw[2] == p.L && hw[3] == p.H &&
                            hw[4] == p.T && hw[5] == p.d && hw[6] == kCardGroup && hq[0] == kCardHeaderBytes &&
                            hq[1] == payload && hq[2] == S && hq[3] == total && total <= p.limit;
            if (!ok) flags |= kFlagBadHeader;
        }
        p.info[0] = S;
        p.info[1] = total;
        p.info[2] = flags;
        if ((flags & kStatusBits) && p.status) atomicOr(p.status, (int)(flags & kStatusBits));
    }
    if (!p.card_out || flags) return;
    // header (256 B) + widths + zero padding up to the payload
    uint32_t* hdr = reinterpret_cast<uint32_t*>(p.card_out);
    if (tid < 64) hdr[tid] = card_header_word(tid, p.L, p.H, p.T, p.d, payload, S, total, p.meta, p.meta_src);
    if (one_chunk) {
        const uint64_t t0 = (uint64_t)tid * kScanItems;
        if (t0 + kScanItems <= p.T) {
            // card + 256 + t0 is 8-byte aligned
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                lo |= (uint32_t)wv[i] << (8 * i);
                hi |= (uint32_t)wv[4 + i] << (8 * i);
            }
            *reinterpret_cast<uint2*>(p.card_out + kCardHeaderBytes + t0) = make_uint2(lo, hi);
        } else {
#pragma unroll
            for (int i = 0; i < kScanItems; ++i)
                if (t0 + i < p.T) p.card_out[kCardHeaderBytes + t0 + i] = wv[i];
        }
        for (uint64_t i = p.T + tid; i < payload - kCardHeaderBytes; i += kScanThreads)
            p.card_out[kCardHeaderBytes + i] = 0;
    } else {
        for (uint64_t i = tid; i < payload - kCardHeaderBytes; i += kScanThreads)
            p.card_out[kCardHeaderBytes + i] = i < p.T ? p.widths[i] : 0;
    }
}

// Codes of one group as bytes, in the order that makes narrowing them to
// b-bit fields cheap at every width: code j = 16w + 4k + r (w < 2, k < 4,
// r < 4) goes to byte k of by[4w + r]. Code j is rne(min((x_j - mn) * inv,
// qmax)), which equals min(rne((x_j - mn) * inv), qmax) as qmax is an
// integer; the rounding, the clamp at 255 and the placement in a byte are one
// v_cvt_pk_u8_f32 (round to nearest even, saturating; checked against rintf
// on the GPU for a million values). Without Clamp the min with qmax is left
// out: the caller has shown that no code reaches it.
template <bool Clamp>
__device__ __forceinline__ void codes_to_bytes(const float (&x)[32], float mn, float inv, float qmax,
                                               uint32_t (&by)[8]) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        uint32_t acc = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int j = 16 * (m / 4) + 4 * k + (m % 4);
            float y = (x[j] - mn) * inv;
            if (Clamp) y = __builtin_fminf(y, qmax);
            acc = __builtin_amdgcn_cvt_pk_u8_f32(y, (uint32_t)k, acc);
        }
        by[m] = acc;
    }
}

// One 32-channel group at a per-lane width b (2, 4 or 8): scale and minimum
// bits and the codes as bytes (codes_to_bytes order). The arithmetic is the
// same at every width but for qmax, so a wave whose tokens mix widths runs it
// once; only the narrowing of the bytes to b-bit fields (narrow_codes)
// depends on the width.
//
// The clamp at qmax. Rounding and multiplication by inv >= 0 are monotone,
// so every (x_j - mn) * inv is at most (mx - mn) * inv, the same operations
// on the maximum. While that is below qmax + 1/2 every code rounds to at most
// qmax and min(y, qmax) changes no code; the usual case (the fp16 scale is
// within 2^-11 of the exact step). A subnormal or saturated fp16 scale, or a
// non-finite range, can break it, and a NaN group needs the clamp for its
// codes: if any lane of the wave has either, the wave takes the clamped
// form.
__device__ __forceinline__ void quant_group(const float (&x)[32], uint32_t b, uint16_t& sbits, uint16_t& mbits,
                                            uint32_t (&by)[8]) {
    // IEEE 754-2019 minimum and maximum (v_minimum3_f32, v_maximum3_f32):
    // a NaN anywhere in the group, quiet or signalling, makes both NaN, and
    // such a group takes the quiet NaN 0x7FC0 for its minimum and maximum
    // (its scale then saturates at 65504, each code is qmax through the
    // clamp, and the group decodes to NaN).
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int j = 1; j < 32; ++j) {
        mn = __builtin_elementwise_minimum(mn, x[j]);
        mx = __builtin_elementwise_maximum(mx, x[j]);
    }
    const bool nan_in_wave = __builtin_amdgcn_ballot_w64(mx != mx) != 0;
    if (nan_in_wave && mx != mx) mn = mx = __uint_as_float(0x7FC00000u);
    mn = mn + 0.0f;
    mx = mx + 0.0f;
    const float qmax = (float)((1u << b) - 1u);
    // s = (mx - mn) / qmax correctly rounded, from RN(1/qmax): z = RN(d y),
    // the remainder d - z qmax exactly by an fma, and one fma to correct.
    // Checked against the IEEE quotient for every finite d >= 0 (subnormals
    // included) at qmax = 3, 15 and 255. A non-finite d gives NaN here and
    // infinity or NaN in the quotient; the min with 65504 below makes both
    // 65504.
    const float d = mx - mn;
    const float yq = b == 2 ? 1.0f / 3.0f : (b == 4 ? 1.0f / 15.0f : 1.0f / 255.0f);
    const float z = d * yq;
    const float s = __builtin_fmaf(__builtin_fmaf(-z, qmax, d), yq, z);
    const _Float16 s16 = (_Float16)__builtin_fminf(s, 65504.0f);
    const float sf = (float)s16;
    // inv = RN(1/sf) from v_rcp_f32 (r0 = (1 + e)/sf, |e| <= 2^-23) and one
    // Newton step: 1 - sf r0 = -e exactly (an fma), and RN(r0 - e r0) =
    // RN((1 - e^2)/sf). An 11-bit sf keeps 1/sf at least 2^-35 (relative)
    // from every midpoint between binary32 neighbours, far beyond e^2 <=
    // 2^-46, so the step lands on RN(1/sf).
    const float r0 = __builtin_amdgcn_rcpf(sf);
    const float inv = (sf == 0.0f) ? 0.0f : __builtin_fmaf(__builtin_fmaf(-sf, r0, 1.0f), r0, r0);
    const bool clamp = !((mx - mn) * inv < qmax + 0.5f);
    if (!nan_in_wave && __builtin_amdgcn_ballot_w64(clamp) == 0)
        codes_to_bytes<false>(x, mn, inv, qmax, by);
    else
        codes_to_bytes<true>(x, mn, inv, qmax, by);
    sbits = __builtin_bit_cast(uint16_t, s16);
    mbits = (uint16_t)(__float_as_uint(mn) >> 16);
}

// Byte codes (each below 2^B, codes_to_bytes order) -> B-bit fields, 32
// codes in B dwords, code i of dword w at bits B*i (out[0 .. B-1]).
// __builtin_amdgcn_perm(hi, lo, sel): byte n of the result is byte sel_n of
// the 8 bytes lo (0-3), hi (4-7).
template <int B>
__device__ __forceinline__ void narrow_codes(const uint32_t (&by)[8], uint32_t (&out)[8]) {
    if (B == 8) {
        // out[4w + k] byte r = by[4w + r] byte k: a 4 x 4 byte transpose
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const uint32_t* d = by + 4 * w;
            const uint32_t p0 = __builtin_amdgcn_perm(d[1], d[0], 0x06020400u);  // d0.0 d1.0 d0.2 d1.2
            const uint32_t p1 = __builtin_amdgcn_perm(d[1], d[0], 0x07030501u);  // d0.1 d1.1 d0.3 d1.3
            const uint32_t p2 = __builtin_amdgcn_perm(d[3], d[2], 0x06020400u);
            const uint32_t p3 = __builtin_amdgcn_perm(d[3], d[2], 0x07030501u);
            out[4 * w + 0] = __builtin_amdgcn_perm(p2, p0, 0x05040100u);
            out[4 * w + 1] = __builtin_amdgcn_perm(p3, p1, 0x05040100u);
            out[4 * w + 2] = __builtin_amdgcn_perm(p2, p0, 0x07060302u);
            out[4 * w + 3] = __builtin_amdgcn_perm(p3, p1, 0x07060302u);
        }
    } else if (B == 4) {
        // e_s byte k = code 16w+4k+s | code 16w+4k+s+1 << 4 (s = 0, 2); dword
        // 2w + a takes bytes 2a, 2a+1 of e_0 and e_2 alternately
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const uint32_t e0 = by[4 * w] | (by[4 * w + 1] << 4);
            const uint32_t e2 = by[4 * w + 2] | (by[4 * w + 3] << 4);
            out[2 * w] = __builtin_amdgcn_perm(e2, e0, 0x05010400u);
            out[2 * w + 1] = __builtin_amdgcn_perm(e2, e0, 0x07030602u);
        }
    } else {
        // by[4w + r] byte k = code 16w + 4k + r, which belongs at bit 8k + 2r
#pragma unroll
        for (int w = 0; w < 2; ++w)
            out[w] = by[4 * w] | (by[4 * w + 1] << 2) | (by[4 * w + 2] << 4) | (by[4 * w + 3] << 6);
    }
}

template <int B>
__device__ __forceinline__ void store_group(uint8_t* rec, uint32_t G, uint32_t g, uint16_t sb, uint16_t mb,
                                            const uint32_t (&codes)[8]) {
    reinterpret_cast<uint16_t*>(rec)[g] = sb;
    reinterpret_cast<uint16_t*>(rec)[G + g] = mb;
    // codes start 8-byte aligned (4*G is a multiple of 8, records 16-aligned)
    uint2* dst = reinterpret_cast<uint2*>(rec + 4 * G + g * 4 * B);
#pragma unroll
    for (int i = 0; i < B / 2; ++i) dst[i] = make_uint2(codes[2 * i], codes[2 * i + 1]);
}

// Quantise one group at width b in {2, 4, 8} into its record.
__device__ __forceinline__ void quant_store_group(const float (&x)[32], uint32_t b, uint8_t* rec, uint32_t G,
                                                  uint32_t g) {
    uint16_t sb, mb;
    uint32_t by[8], codes[8];
    quant_group(x, b, sb, mb, by);
    if (b == 2) {
        narrow_codes<2>(by, codes);
        store_group<2>(rec, G, g, sb, mb, codes);
    } else if (b == 4) {
        narrow_codes<4>(by, codes);
        store_group<4>(rec, G, g, sb, mb, codes);
    } else {
        narrow_codes<8>(by, codes);
        store_group<8>(rec, G, g, sb, mb, codes);
    }
}

// Per-wave LDS image of the wave's records: its tokens are consecutive, so
// their records form one contiguous span of the stream (at most TPW records
// of at most 2d bytes: 4 KiB), 16-byte aligned at both ends.
constexpr uint32_t kSpanChunks = 256;  // 16-byte chunks

// ---------------------------------------------------------------- record offsets in the grid
//
// Cards of up to kInGridTokens tokens skip the scan kernel and the launch
// gap behind it: every pack or unpack workgroup computes the record offsets
// itself from the widths (at most 8 KiB, read from L2 after the first
// workgroups), 32 per thread. Per dword x of four widths: v_sad_u8 sums
// them, v_sad_u8 of (x >> 4) & 0x01010101 counts the 16s (a valid width has
// bit 4 only when it is 16), and x & 0xE1E1E1E1, the borrow bits of
// x - 0x01010101 and x & (x - 0x01010101) are all zero exactly when each
// byte is 2, 4, 8 or 16 (one set bit among bits 1-4, no zero byte). A record
// is 16 + (d/8) w bytes, and 2d = 16 + (d/8) 16 - 16 at w = 16, so a block
// of n tokens takes 16 n + (d/8) sum(w) - 16 n16 bytes. A workgroup scan of
// the block sums gives every block's offset; a wave scan gives each token's
// within its block. Tails and unaligned widths take the bytes one by one.
constexpr uint32_t kInGridTokens = 8192;
constexpr uint32_t kInGridBlocks = 512;  // 16-token blocks at d = 128 (256 of 32 at d = 64)
constexpr uint32_t kInGridBytes = 32;    // widths per thread

struct InGridLds {
    uint32_t pref[kInGridBlocks + 1];  // record bytes before each block; [nbk] = the stream's
    uint32_t wtot[kBlockThreads / kWave];
};

// Fills sh.pref[0 .. nbk]; all threads return the stream's record bytes and
// whether any width is invalid. wreg: the thread's 32 widths when it loaded
// them whole (w_whole), for the card copy.
template <int D>
__device__ __forceinline__ void ingrid_scan(const uint8_t* widths, uint32_t T, uint32_t nbk, InGridLds& sh,
                                            uint32_t& total, bool& bad, uint4 (&wreg)[2], bool& w_whole) {
    constexpr uint32_t TPW = kWave / (D / kCardGroup);             // tokens per block
    constexpr uint32_t BPT = kInGridBytes / TPW;                    // blocks per thread: 2 or 1
    constexpr uint32_t DPB = TPW / 4;                               // dwords per block
    static_assert(kInGridTokens / TPW <= kInGridBlocks && BPT * kBlockThreads * TPW == kInGridTokens, "layout");
    const uint32_t tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
    const uint32_t t0 = tid * kInGridBytes;
    w_whole = ((uintptr_t)widths & 15) == 0 && t0 + kInGridBytes <= T;
    uint32_t bs[BPT];
    uint32_t badbits = 0;
    wreg[0] = make_uint4(0, 0, 0, 0);
    wreg[1] = make_uint4(0, 0, 0, 0);
    if (w_whole) {
        wreg[0] = *reinterpret_cast<const uint4*>(widths + t0);
        wreg[1] = *reinterpret_cast<const uint4*>(widths + t0 + 16);
        const uint32_t x[8] = {wreg[0].x, wreg[0].y, wreg[0].z, wreg[0].w, wreg[1].x, wreg[1].y, wreg[1].z, wreg[1].w};
#pragma unroll
        for (uint32_t j = 0; j < BPT; ++j) {
            uint32_t sw = 0, n16 = 0;
#pragma unroll
            for (uint32_t q = 0; q < DPB; ++q) {
                const uint32_t v = x[j * DPB + q];
                sw = __builtin_amdgcn_sad_u8(v, 0u, sw);
                n16 = __builtin_amdgcn_sad_u8((v >> 4) & 0x01010101u, 0u, n16);
                const uint32_t t = v - 0x01010101u;
                badbits |= (v & 0xE1E1E1E1u) | (t & 0x80808080u) | (v & t);
            }
            bs[j] = 16u * TPW + (uint32_t)(D / 8) * sw - 16u * n16;
        }
    } else {
#pragma unroll
        for (uint32_t j = 0; j < BPT; ++j) {
            uint32_t r = 0;
            for (uint32_t i = 0; i < TPW && t0 + j * TPW < T; ++i) {
                const uint32_t t = t0 + j * TPW + i;
                if (t < T) {
                    const uint32_t rb = record_bytes_sel(D, widths[t]);
                    badbits |= rb == 0 ? 1u : 0u;
                    r += rb;
                }
            }
            bs[j] = r;
        }
    }
    uint32_t local = 0;
#pragma unroll
    for (uint32_t j = 0; j < BPT; ++j) local += bs[j];
    const uint32_t inc = wave_inclusive_sum(local);
    const bool wave_bad = __builtin_amdgcn_ballot_w64(badbits != 0) != 0;
    // at most 8192 records of at most 256 bytes: bit 31 is free for the flag
    if (lane == kWave - 1) sh.wtot[w] = inc | (wave_bad ? 0x80000000u : 0u);
    __syncthreads();
    uint32_t before = 0, tot = 0, flag = 0;
#pragma unroll
    for (int k = 0; k < kBlockThreads / kWave; ++k) {
        const uint32_t v = sh.wtot[k];
        flag |= v;
        before += (uint32_t)k < w ? (v & 0x7FFFFFFFu) : 0u;
        tot += v & 0x7FFFFFFFu;
    }
    uint32_t run = before + inc - local;
#pragma unroll
    for (uint32_t j = 0; j < BPT; ++j) {
        const uint32_t b = tid * BPT + j;
        if (b < nbk) sh.pref[b] = run;
        run += bs[j];
    }
    if (tid == 0) sh.pref[nbk] = tot;
    total = tot;
    bad = (flag & 0x80000000u) != 0;
    __syncthreads();
}

// Offset of this lane's token within its wave's block (tokens in lane order,
// G lanes per token): exclusive sum of the record bytes of the tokens before
// it, from one wave scan over the first lane of each token.
__device__ __forceinline__ uint32_t token_offset_in_block(uint32_t rec, uint32_t g) {
    return wave_inclusive_sum(g == 0 ? rec : 0u) - rec;
}

template <int D, bool InGrid>
__global__ __launch_bounds__(kBlockThreads) void card_pack_kernel(CardParams p) {
    constexpr uint32_t G = D / kCardGroup;  // lanes per token
    constexpr uint32_t TPW = kWave / G;     // tokens per wave
    static_assert(TPW * 2 * D <= 16 * kSpanChunks, "span exceeds the stage");
    const uint32_t lane = lane_id();
    const uint64_t wave_id = xcd_run_block<kPackXcdRun>(blockIdx.x) * (kBlockThreads / kWave) + wave_uniform(threadIdx.x / kWave);
    // with offsets computed in the grid every wave takes part in its
    // workgroup's scan; a wave past the end does nothing else
    const bool active = wave_id < p.n_waves;
    if (!InGrid && !active) return;
    const uint64_t wave = active ? wave_id : 0;
    const uint64_t s = wave / p.nbk;
    const uint32_t blk = (uint32_t)(wave % p.nbk);
    const uint32_t t0 = blk * TPW;
    const uint32_t tok = t0 + lane / G;
    const uint32_t g = lane % G;
    const bool valid = tok < p.T;
    const uint32_t nv = (p.T - t0 < TPW) ? p.T - t0 : TPW;
    const uint32_t h = (uint32_t)(s % p.H);
    const uint32_t kv = (uint32_t)((s / p.H) & 1);
    const uint32_t l = (uint32_t)(s / (2ull * p.H));
    // The input loads go out first: they depend on nothing the scan wrote
    // (lanes past the last token load the wave's first token), so their
    // latency overlaps that of the offsets below.
    uint4 raw[4] = {};
    if (active) {
        const uint16_t* src =
            (kv ? p.v : p.k) + (((uint64_t)l * p.H + h) * p.T + (valid ? tok : t0)) * D + g * kCardGroup;
#pragma unroll
        for (int i = 0; i < 4; ++i) raw[i] = reinterpret_cast<const uint4*>(src)[i];
    }
    const uint32_t width = p.widths[valid ? tok : t0];
    uint64_t S, span0, span1, my_off;
    if (InGrid) {
        __shared__ InGridLds sh;
        uint32_t tot;
        bool bad, w_whole;
        uint4 wreg[2];
        ingrid_scan<D>(p.widths, p.T, p.nbk, sh, tot, bad, wreg, w_whole);
        S = align_up(tot, 256);
        const uint64_t total = p.payload + 2ull * p.L * p.H * S;
        const uint32_t flags = (bad ? kFlagBadWidth : 0u) | (total > p.limit ? kFlagCapacity : 0u);
        if (blockIdx.x == 0) {
            // the card's header, widths and padding (what the scan kernel writes)
            const uint32_t tid = threadIdx.x;
            if (tid == 0) {
                if (p.dev_card_bytes) *p.dev_card_bytes = total;
                if (flags && p.status) atomicOr(p.status, (int)flags);
                // a card that will not be written gets a zero magic word
                if (flags) reinterpret_cast<uint32_t*>(p.card)[0] = 0;
            }
            if (!flags) {
                if (tid < 64)
                    reinterpret_cast<uint32_t*>(p.card)[tid] =
                        card_header_word(tid, p.L, p.H, p.T, D, p.payload, S, total, p.meta, nullptr);
                const uint64_t w0 = (uint64_t)tid * kInGridBytes;
                uint8_t* cw = p.card + kCardHeaderBytes;
                if (w_whole) {
                    reinterpret_cast<uint4*>(cw + w0)[0] = wreg[0];
                    reinterpret_cast<uint4*>(cw + w0)[1] = wreg[1];
                } else {
                    for (uint64_t i = w0; i < w0 + kInGridBytes && i < p.T; ++i) cw[i] = p.widths[i];
                }
                for (uint64_t i = p.T + tid; i < p.payload - kCardHeaderBytes; i += kBlockThreads) cw[i] = 0;
            }
        }
        if (flags || !active) return;
        span0 = sh.pref[blk];
        span1 = sh.pref[blk + 1];
        my_off = span0 + token_offset_in_block(valid ? record_bytes_sel(D, width) : 0u, g);
    } else {
        const uint64_t flags = p.info[2];
        S = p.info[0];
        span0 = p.off[t0];
        span1 = p.off[t0 + nv];
        my_off = p.off[valid ? tok : t0];
        if (flags != 0) return;
    }
    uint8_t* stream = p.card + p.payload + s * S;

    __shared__ uint4 stage[kBlockThreads / kWave][kSpanChunks];
    uint8_t* st = reinterpret_cast<uint8_t*>(stage[threadIdx.x / kWave]);
    if (valid) {
        uint8_t* rec = st + (uint32_t)(my_off - span0);
        if (width == 16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) reinterpret_cast<uint4*>(rec + 64 * g)[i] = raw[i];
        } else {
            const uint32_t* w = reinterpret_cast<const uint32_t*>(raw);
            float x[32];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                x[2 * j] = bf16_lo(w[j]);
                x[2 * j + 1] = bf16_hi(w[j]);
            }
            quant_store_group(x, width, rec, G, g);
            // zero the record's tail padding (present for d = 64)
            const uint32_t used = 4 * G + D * width / 8;
            const uint32_t R = card_record_bytes(D, width);
            if (g == 0)
                for (uint32_t i = used; i < R; i += 8) *reinterpret_cast<uint2*>(rec + i) = make_uint2(0, 0);
        }
    }
    // the span, 16 bytes per lane per store
    const uint32_t n16 = (uint32_t)((span1 - span0) / 16);
    uint4* dst = reinterpret_cast<uint4*>(stream + span0);
    const uint4* img = stage[threadIdx.x / kWave];
#pragma unroll
    for (uint32_t j = 0; j < kSpanChunks / kWave; ++j) {
        const uint32_t idx = kWave * j + lane;
        if (idx < n16) st_stream(dst + idx, img[idx]);
    }
    // zero the stream's tail padding after the last record
    if (t0 + nv == p.T && lane == 0)
        for (uint64_t i = span1; i < S; i += 16) *reinterpret_cast<uint4*>(stream + i) = make_uint4(0, 0, 0, 0);
}

// The codes of one group at a per-lane width b (2, 4 or 8) from its record,
// two per dword in channel order (channel 2i in the low half of h[i], 2i + 1
// in the high half), each left where masking its record bits puts it: at
// bit e = 0, 2, 4 or 6 of its half's low byte, e depending on the channel's
// place in its byte (e = 0 at b = 8; 0, 4 at b = 4; 0, 2, 4, 6 at b = 2). A
// half read as an f16 is then the subnormal code * 2^(e - 24) (below 2^-14,
// exact; the kernels keep f16 subnormals), and sc[j % 4] = sf * 2^(24 - e)
// (a power-of-two scaling of an f16 value, exact in binary32) makes the
// product of the two code * sf exactly.
__device__ __forceinline__ void code_halves(const uint8_t* rec, uint32_t G, uint32_t g, uint32_t b, float sf,
                                            uint32_t (&h)[16], float (&sc)[4]) {
    // codes start 8-byte aligned (4*G is a multiple of 8, records 16-aligned)
    const uint2* src = reinterpret_cast<const uint2*>(rec + 4 * G + g * 4 * b);
    const float s24 = sf * 16777216.0f;
    if (b == 8) {
        // dword m: codes 4m .. 4m+3, one per byte
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint2 v = src[i];
            const uint32_t c[2] = {v.x, v.y};
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int m = 2 * i + u;
                h[2 * m] = __builtin_amdgcn_perm(0u, c[u], 0x0C010C00u);
                h[2 * m + 1] = __builtin_amdgcn_perm(0u, c[u], 0x0C030C02u);
            }
        }
        sc[0] = sc[1] = sc[2] = sc[3] = s24;
    } else if (b == 4) {
        // dword m: codes 8m + 2k (low nibble) and 8m + 2k + 1 (high) in byte k
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint2 v = src[i];
            const uint32_t c[2] = {v.x, v.y};
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int m = 2 * i + u;
                const uint32_t lo = c[u] & 0x0F0F0F0Fu, hi = c[u] & 0xF0F0F0F0u;
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    h[4 * m + k] = __builtin_amdgcn_perm(hi, lo, 0x0C000C00u | (uint32_t)k | ((uint32_t)(4 + k) << 16));
            }
        }
        sc[0] = sc[2] = s24;
        sc[1] = sc[3] = s24 * 0.0625f;
    } else {
        // dword m: code 16m + 4k + r at bits 2r of byte k
        const uint2 v = src[0];
        const uint32_t c[2] = {v.x, v.y};
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const uint32_t q0 = c[m] & 0x03030303u, q1 = c[m] & 0x0C0C0C0Cu;
            const uint32_t q2 = c[m] & 0x30303030u, q3 = c[m] & 0xC0C0C0C0u;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t sel = 0x0C040C00u | (uint32_t)k | ((uint32_t)k << 16);
                h[8 * m + 2 * k] = __builtin_amdgcn_perm(q1, q0, sel);
                h[8 * m + 2 * k + 1] = __builtin_amdgcn_perm(q3, q2, sel);
            }
        }
        sc[0] = s24;
        sc[1] = s24 * 0.25f;
        sc[2] = s24 * 0.0625f;
        sc[3] = s24 * 0.015625f;
    }
}

// One group at width b in {2, 4, 8} back to 32 binary32 values y_j = q_j*s +
// mn with one rounding (q_j*s alone is exact), which the caller rounds to
// bf16. Only the extraction of the codes depends on the width: a wave whose
// tokens mix widths runs the rest once.
__device__ __forceinline__ void dequant_group(const uint8_t* rec, uint32_t G, uint32_t g, uint32_t b,
                                              float (&y)[32]) {
    const float sf = (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(rec)[g]);
    const float mn = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(rec)[G + g] << 16);
    uint32_t h[16];
    float sc[4];
    code_halves(rec, G, g, b, sf, h, sc);
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const uint16_t bits = (uint16_t)(j % 2 ? h[j / 2] >> 16 : h[j / 2]);
        y[j] = __builtin_fmaf((float)__builtin_bit_cast(_Float16, bits), sc[j % 4], mn);
    }
}

// y rounded to bf16 (round to nearest even), as a binary32 value: the
// rounded bits land in the high half of v_cvt_pk_bf16_f32(0, y), the low
// half is zero. (Written out: the compiler builds the same pair from a
// conversion into the low half and a v_perm, two instructions.)
__device__ __forceinline__ float round_bf16(float y) {
    uint32_t r;
    asm("v_cvt_pk_bf16_f32 %0, 0, %1" : "=v"(r) : "v"(y));
    return __uint_as_float(r);
}

template <int D, bool InGrid>
__global__ __launch_bounds__(kBlockThreads) void card_unpack_kernel(CardParams p) {
    constexpr uint32_t G = D / kCardGroup;
    constexpr uint32_t TPW = kWave / G;  // the wave's tokens: 4 KiB of bf16 output
    const uint32_t lane = lane_id();
    const uint64_t wave_id = xcd_run_block<kUnpackXcdRun>(blockIdx.x) * (kBlockThreads / kWave) + wave_uniform(threadIdx.x / kWave);
    // with offsets computed in the grid every wave takes part in its
    // workgroup's scan; a wave past the end does nothing else
    const bool active = wave_id < p.n_waves;
    if (!InGrid && !active) return;
    const uint64_t wave = active ? wave_id : 0;
    const uint64_t s = wave / p.nbk;
    const uint32_t b = (uint32_t)(wave % p.nbk);
    const uint32_t t0 = b * TPW;
    const uint32_t tok = t0 + lane / G;
    const uint32_t g = lane % G;
    const bool valid = tok < p.T;
    const uint32_t tc = valid ? tok : t0;
    const uint32_t nv = (p.T - t0 < TPW) ? p.T - t0 : TPW;
    const uint32_t h = (uint32_t)(s % p.H);
    const uint32_t kv = (uint32_t)((s / p.H) & 1);
    const uint32_t l = (uint32_t)(s / (2ull * p.H));
    uint64_t S, span0, span1, my_off;
    const uint32_t width = p.widths[tc];
    if (InGrid) {
        __shared__ InGridLds sh;
        uint32_t tot;
        bool bad, w_whole;
        uint4 wreg[2];
        ingrid_scan<D>(p.widths, p.T, p.nbk, sh, tot, bad, wreg, w_whole);
        S = align_up(tot, 256);
        const uint64_t total = p.payload + 2ull * p.L * p.H * S;
        // every wave checks the header itself (uniform addresses: scalar
        // loads); the widths say how large the card must be, and a card
        // shorter than that is refused before any record is read
        uint32_t flags = bad ? kFlagBadWidth : 0u;
        if (!card_header_ok(p.card_in, p.L, p.H, p.T, D, p.payload, S, total, p.limit)) flags |= kFlagBadHeader;
        if (blockIdx.x == 0 && threadIdx.x == 0 && flags && p.status) atomicOr(p.status, (int)flags);
        if (flags || !active) return;
        span0 = sh.pref[b];
        span1 = sh.pref[b + 1];
        my_off = span0 + token_offset_in_block(valid ? record_bytes_sel(D, width) : 0u, g);
    } else {
        // Everything the scan wrote that this wave needs, in one round of loads
        // (none depends on another), before the status check: a short-lived
        // wave pays each dependent round trip in full.
        const uint64_t flags = p.info[2];
        S = p.info[0];
        span0 = p.off[t0];
        span1 = p.off[t0 + nv];
        my_off = p.off[tc];
        if (flags != 0) return;
    }
    // The wave's records are one contiguous span of the stream: load it with
    // 16-byte coalesced loads into LDS, then decode each group from there.
    __shared__ uint4 stage[kBlockThreads / kWave][kSpanChunks];
    uint4* st = stage[threadIdx.x / kWave];
    {
        const uint32_t n16 = (uint32_t)((span1 - span0) / 16);
        const uint4* src = reinterpret_cast<const uint4*>(p.card_in + p.payload + s * S + span0);
        uint4 c[kSpanChunks / kWave];
#pragma unroll
        for (uint32_t j = 0; j < kSpanChunks / kWave; ++j) {
            const uint32_t idx = kWave * j + lane;
            c[j] = idx < n16 ? src[idx] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (uint32_t j = 0; j < kSpanChunks / kWave; ++j) st[kWave * j + lane] = c[j];
    }
    uint32_t o[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = 0;
    if (valid) {
        const uint8_t* rec = reinterpret_cast<const uint8_t*>(st) + (uint32_t)(my_off - span0);
        if (width == 16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) reinterpret_cast<uint4*>(o)[i] = reinterpret_cast<const uint4*>(rec + 64 * g)[i];
        } else {
            float y[32];
            dequant_group(rec, G, g, width, y);
#pragma unroll
            for (int j = 0; j < 16; ++j) o[j] = pack_bf16x2(y[2 * j], y[2 * j + 1]);
        }
    }
    // Stage the wave's contiguous output image in LDS (over the records,
    // which every lane has read by now), then store it with each instruction
    // covering a contiguous span (lane-strided 64-byte stores run at about
    // half the write bandwidth).
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int c = 0; c < 4; ++c) st[stage_slot<4>(lane, c)] = make_uint4(o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]);
    uint4* dst = reinterpret_cast<uint4*>((kv ? p.v_out : p.k_out) + (((uint64_t)l * p.H + h) * p.T + t0) * D);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint4 chunk = st[stage_pos<4>(64 * j + lane)];
        if ((64 * j + lane) / (2 * D / 16) < nv) st_stream(dst + 64 * j + lane, chunk);
    }
}

// ---------------------------------------------------------------- hop transcode
//
// One hop of a handoff chain: card_in re-encoded at new per-token widths
// into card_out, equal byte for byte to unpacking it and packing the bf16
// result again (the same exactly rounded values, then the same
// quantisation), without the bf16 round trip through HBM. A wave takes one
// token block of one stream, as in unpack: the input records' span comes
// into LDS with coalesced loads, each lane rebuilds its group's 32 values
// and quantises them at the new width into the output span in LDS, which
// then goes out with coalesced stores.
struct TranscodeParams {
    const uint8_t* card_in;
    uint8_t* card_out;
    const uint8_t* w_in;   // card_in + 256
    const uint8_t* w_out;  // new widths
    const uint64_t* info_in;
    const uint64_t* off_in;
    const uint64_t* info_out;
    const uint64_t* off_out;
    uint32_t L, H, T, nbk;
    uint64_t payload;  // the same for both cards (it depends on T only)
    uint64_t n_waves;
};

template <int D>
__global__ __launch_bounds__(kTranscodeThreads) void card_transcode_kernel(TranscodeParams p) {
    constexpr uint32_t G = D / kCardGroup;  // lanes per token
    constexpr uint32_t TPW = kWave / G;     // tokens per wave
    const uint32_t lane = lane_id();
    const uint64_t wave = xcd_run_block<kTranscodeXcdRun>(blockIdx.x) * (kTranscodeThreads / kWave) + wave_uniform(threadIdx.x / kWave);
    if (wave >= p.n_waves) return;
    const uint64_t s = wave / p.nbk;
    const uint32_t t0 = (uint32_t)(wave % p.nbk) * TPW;
    const uint32_t tok = t0 + lane / G;
    const uint32_t g = lane % G;
    const bool valid = tok < p.T;
    const uint32_t tc = valid ? tok : t0;
    const uint32_t nv = (p.T - t0 < TPW) ? p.T - t0 : TPW;
    const uint64_t f_in = p.info_in[2], f_out = p.info_out[2];
    const uint64_t S_in = p.info_in[0], S_out = p.info_out[0];
    const uint64_t a0 = p.off_in[t0], a1 = p.off_in[t0 + nv], my_a = p.off_in[tc];
    const uint64_t b0 = p.off_out[t0], b1 = p.off_out[t0 + nv], my_b = p.off_out[tc];
    const uint32_t w_in = p.w_in[tc], w_out = p.w_out[tc];
    if ((f_in | f_out) != 0) {
        // A refused output card already has a zero magic word. A refused
        // input (reported by its scan, which ran beside the output's) leaves
        // an output whose header was written: its magic is zeroed here, so
        // that it cannot pass for a transcode of the input.
        if (f_in != 0 && f_out == 0 && wave == 0 && lane == 0) reinterpret_cast<uint32_t*>(p.card_out)[0] = 0;
        return;
    }

    // One LDS image per wave holds the input span, then the output span: every
    // lane's group reads (in the rebuild below, whatever its width) are issued
    // before any lane's group writes, and a wave's LDS operations complete in
    // order. (A second image doubled the LDS of a workgroup and halved the
    // waves a CU can hold.)
    __shared__ uint4 stage[kTranscodeThreads / kWave][kSpanChunks];
    uint4* si = stage[threadIdx.x / kWave];
    uint4* so = si;
    {
        const uint32_t n16 = (uint32_t)((a1 - a0) / 16);
        const uint4* src = reinterpret_cast<const uint4*>(p.card_in + p.payload + s * S_in + a0);
        uint4 c[kSpanChunks / kWave];
#pragma unroll
        for (uint32_t j = 0; j < kSpanChunks / kWave; ++j) {
            const uint32_t idx = kWave * j + lane;
            c[j] = idx < n16 ? src[idx] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (uint32_t j = 0; j < kSpanChunks / kWave; ++j) si[kWave * j + lane] = c[j];
    }
    if (valid) {
        // rebuild the group (as unpack does: binary32 values rounded to bf16) ...
        float x[32];
        const uint8_t* rin = reinterpret_cast<const uint8_t*>(si) + (uint32_t)(my_a - a0);
        if (w_in == 16) {
            uint32_t o[16];
#pragma unroll
            for (int i = 0; i < 4; ++i) reinterpret_cast<uint4*>(o)[i] = reinterpret_cast<const uint4*>(rin + 64 * g)[i];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                x[2 * j] = bf16_lo(o[j]);
                x[2 * j + 1] = bf16_hi(o[j]);
            }
        } else {
            float y[32];
            dequant_group(rin, G, g, w_in, y);
#pragma unroll
            for (int j = 0; j < 32; ++j) x[j] = round_bf16(y[j]);
        }

        // ... and quantise it at the new width (as pack does); the barrier
        // keeps every lane's reads above ahead of the writes below
        __builtin_amdgcn_wave_barrier();
        uint8_t* rout = reinterpret_cast<uint8_t*>(so) + (uint32_t)(my_b - b0);
        if (w_out == 16) {
            // the bf16 bits of the rebuilt values, pairs in channel order
            uint32_t o[16];
#pragma unroll
            for (int j = 0; j < 16; ++j)
                o[j] = __builtin_amdgcn_perm(__float_as_uint(x[2 * j + 1]), __float_as_uint(x[2 * j]), 0x07060302u);
#pragma unroll
            for (int i = 0; i < 4; ++i) reinterpret_cast<uint4*>(rout + 64 * g)[i] = reinterpret_cast<const uint4*>(o)[i];
        } else {
            quant_store_group(x, w_out, rout, G, g);
            // zero the record's tail padding (present for d = 64)
            const uint32_t used = 4 * G + D * w_out / 8;
            const uint32_t R = card_record_bytes(D, w_out);
            if (g == 0)
                for (uint32_t i = used; i < R; i += 8) *reinterpret_cast<uint2*>(rout + i) = make_uint2(0, 0);
        }
    }
    // the output span, 16 bytes per lane per store
    uint8_t* stream = p.card_out + p.payload + s * S_out;
    const uint32_t n16 = (uint32_t)((b1 - b0) / 16);
    uint4* dst = reinterpret_cast<uint4*>(stream + b0);
#pragma unroll
    for (uint32_t j = 0; j < kSpanChunks / kWave; ++j) {
        const uint32_t idx = kWave * j + lane;
        if (idx < n16) st_stream(dst + idx, so[idx]);
    }
    // zero the stream's tail padding after the last record
    if (t0 + nv == p.T && lane == 0)
        for (uint64_t i = p.off_out[p.T]; i < S_out; i += 16)
            *reinterpret_cast<uint4*>(stream + i) = make_uint4(0, 0, 0, 0);
}

}  // namespace

static CardParams card_params(const Shape& s, const void* ws) {
    CardParams p{};
    constexpr uint32_t kTPW128 = kWave / (128 / kCardGroup), kTPW64 = kWave / (64 / kCardGroup);
    const uint32_t tpw = s.d == 128 ? kTPW128 : kTPW64;
    p.L = s.L;
    p.H = s.H;
    p.T = s.T;
    p.nbk = (s.T + tpw - 1) / tpw;
    p.payload = card_payload_offset(s.T);
    p.n_waves = 2ull * s.L * s.H * p.nbk;
    p.info = static_cast<const uint64_t*>(ws);
    p.off = reinterpret_cast<const uint64_t*>(static_cast<const uint8_t*>(ws) + kCardInfoBytes);
    return p;
}

hipError_t launch_card_pack(const Shape& s, const void* k, const void* v, const uint8_t* widths,
                            const CardMetaDev& meta, void* card, uint64_t capacity,
                            uint64_t* dev_card_bytes, int32_t* dev_status, void* ws,
                            hipStream_t stream) {
    ScanLaunch sl{};
    ScanParams& sp = sl.s[0];
    sp.widths = widths;
    sp.card_out = static_cast<uint8_t*>(card);
    sp.card_in = nullptr;
    sp.info = static_cast<uint64_t*>(ws);
    sp.off = reinterpret_cast<uint64_t*>(static_cast<uint8_t*>(ws) + kCardInfoBytes);
    sp.limit = capacity;
    sp.dev_card_bytes = dev_card_bytes;
    sp.status = dev_status;
    sp.L = s.L;
    sp.H = s.H;
    sp.T = s.T;
    sp.d = s.d;
    sp.meta = meta;
    CardParams p = card_params(s, ws);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.widths = widths;
    p.card = static_cast<uint8_t*>(card);
    p.limit = capacity;
    p.dev_card_bytes = dev_card_bytes;
    p.status = dev_status;
    p.meta = meta;
    const uint32_t nblocks = xcd_run_grid<kPackXcdRun>((p.n_waves + 3) / 4);
    // cards of up to kInGridTokens tokens: offsets computed in the grid
    if (s.T <= kInGridTokens)
        return launch_kernel(s.d == 64 ? card_pack_kernel<64, true> : card_pack_kernel<128, true>, dim3(nblocks),
                             dim3(kBlockThreads), stream, p);
    hipError_t e = launch_kernel(card_scan_kernel, dim3(1), dim3(kScanThreads), stream, sl);
    if (e != hipSuccess) return e;
    return launch_kernel(s.d == 64 ? card_pack_kernel<64, false> : card_pack_kernel<128, false>, dim3(nblocks),
                         dim3(kBlockThreads), stream, p);
}

hipError_t launch_card_unpack(const Shape& s, const void* card, uint64_t card_bytes, void* k_out,
                              void* v_out, int32_t* dev_status, void* ws, hipStream_t stream) {
    ScanLaunch sl{};
    ScanParams& sp = sl.s[0];
    sp.widths = static_cast<const uint8_t*>(card) + kCardHeaderBytes;
    sp.card_out = nullptr;
    sp.card_in = static_cast<const uint8_t*>(card);
    sp.info = static_cast<uint64_t*>(ws);
    sp.off = reinterpret_cast<uint64_t*>(static_cast<uint8_t*>(ws) + kCardInfoBytes);
    sp.limit = card_bytes;
    sp.dev_card_bytes = nullptr;
    sp.status = dev_status;
    sp.L = s.L;
    sp.H = s.H;
    sp.T = s.T;
    sp.d = s.d;
    CardParams p = card_params(s, ws);
    p.k_out = static_cast<uint16_t*>(k_out);
    p.v_out = static_cast<uint16_t*>(v_out);
    p.widths = sp.widths;
    p.card_in = static_cast<const uint8_t*>(card);
    p.limit = card_bytes;
    p.status = dev_status;
    const uint32_t nblocks = xcd_run_grid<kUnpackXcdRun>((p.n_waves + 3) / 4);
    // cards of up to kInGridTokens tokens: offsets computed in the grid
    if (s.T <= kInGridTokens)
        return launch_kernel(s.d == 64 ? card_unpack_kernel<64, true> : card_unpack_kernel<128, true>,
                             dim3(nblocks), dim3(kBlockThreads), stream, p);
    hipError_t e = launch_kernel(card_scan_kernel, dim3(1), dim3(kScanThreads), stream, sl);
    if (e != hipSuccess) return e;
    return launch_kernel(s.d == 64 ? card_unpack_kernel<64, false> : card_unpack_kernel<128, false>,
                         dim3(nblocks), dim3(kBlockThreads), stream, p);
}

hipError_t launch_card_transcode(const Shape& s, const void* card_in, uint64_t card_in_bytes,
                                 const uint8_t* new_widths, void* card_out, uint64_t capacity,
                                 uint64_t* dev_card_bytes, int32_t* dev_status, void* ws, hipStream_t stream) {
    uint8_t* ws_in = static_cast<uint8_t*>(ws);
    uint8_t* ws_out = ws_in + card_workspace_half(s.T);
    // offsets of the input records (and a check of its header), and of the
    // output's, whose header and widths are written with the input's model ID
    // and position offset: two workgroups of one launch
    ScanLaunch sl{};
    ScanParams& a = sl.s[0];
    a.widths = static_cast<const uint8_t*>(card_in) + kCardHeaderBytes;
    a.card_in = static_cast<const uint8_t*>(card_in);
    a.info = reinterpret_cast<uint64_t*>(ws_in);
    a.off = reinterpret_cast<uint64_t*>(ws_in + kCardInfoBytes);
    a.limit = card_in_bytes;
    a.status = dev_status;
    a.L = s.L;
    a.H = s.H;
    a.T = s.T;
    a.d = s.d;
    ScanParams& b = sl.s[1];
    b.widths = new_widths;
    b.card_out = static_cast<uint8_t*>(card_out);
    b.info = reinterpret_cast<uint64_t*>(ws_out);
    b.off = reinterpret_cast<uint64_t*>(ws_out + kCardInfoBytes);
    b.limit = capacity;
    b.dev_card_bytes = dev_card_bytes;
    b.status = dev_status;
    b.L = s.L;
    b.H = s.H;
    b.T = s.T;
    b.d = s.d;
    b.meta_src = static_cast<const uint8_t*>(card_in);
    hipError_t e = launch_kernel(card_scan_kernel, dim3(2), dim3(kScanThreads), stream, sl);
    if (e != hipSuccess) return e;
    const CardParams cp = card_params(s, ws);
    TranscodeParams p{};
    p.card_in = static_cast<const uint8_t*>(card_in);
    p.card_out = static_cast<uint8_t*>(card_out);
    p.w_in = a.widths;
    p.w_out = new_widths;
    p.info_in = a.info;
    p.off_in = a.off;
    p.info_out = b.info;
    p.off_out = b.off;
    p.L = s.L;
    p.H = s.H;
    p.T = s.T;
    p.nbk = cp.nbk;
    p.payload = cp.payload;
    p.n_waves = cp.n_waves;
    const uint32_t nblocks = xcd_run_grid<kTranscodeXcdRun>(p.n_waves);
    return launch_kernel(s.d == 64 ? card_transcode_kernel<64> : card_transcode_kernel<128>, dim3(nblocks),
                         dim3(kTranscodeThreads), stream, p);
}

}  // namespace kvc
