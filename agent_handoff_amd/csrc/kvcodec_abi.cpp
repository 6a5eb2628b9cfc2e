// kvcodec_abi.cpp - the C ABI of libkvcodec: host-side validation, size
// queries, header parsing and kernel launches (declared in include/kvcodec.h).
//
// Nothing here touches the GPU except the launch calls, so every size query,
// kvc_parse_header and every argument error path runs on a host without a
// GPU.
#include "kvcodec.h"

#include <math.h>
#include <string.h>

#include "codebook.h"
#include "launch.h"
#include "layout.h"

namespace {

using kvc::align_up;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
    if (na == 0 || nb == 0) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

bool pool_shape(const kvc_shape* s) {
    return s && kvc::pool_shape_ok(s->num_layers, s->num_kv_heads, s->num_tokens, s->head_dim);
}

bool card_shape(const kvc_shape* s) {
    return s && kvc::card_shape_ok(s->num_layers, s->num_kv_heads, s->num_tokens, s->head_dim);
}

uint64_t kv_bytes(const kvc_shape* s) {
    return (uint64_t)s->num_layers * s->num_kv_heads * s->num_tokens * s->head_dim * 2;
}

kvc::Shape to_shape(const kvc_shape* s) {
    return kvc::Shape{s->num_layers, s->num_kv_heads, s->num_tokens, s->head_dim};
}

uint64_t card_ws_bytes(const kvc_shape* s) { return kvc::card_workspace_half(s->num_tokens); }

uint32_t rd32(const uint8_t* p) { return (uint32_t)p[0] | (uint32_t)p[1] << 8 | (uint32_t)p[2] << 16 | (uint32_t)p[3] << 24; }
uint64_t rd64(const uint8_t* p) { return (uint64_t)rd32(p) | (uint64_t)rd32(p + 4) << 32; }

}  // namespace

extern "C" {

size_t kvpool_bytes(const kvc_shape* shape) {
    if (!pool_shape(shape)) return 0;
    return (size_t)kvc::pool_layout(shape->num_layers, shape->num_kv_heads, shape->num_tokens, shape->head_dim).total;
}

size_t kvpool_workspace_bytes(const kvc_shape* shape) {
    if (!pool_shape(shape)) return 0;
    return (size_t)align_up(
        4ull * kvc::encode_workspace_words(shape->num_layers), 256);
}

int kvpool_encode(const kvc_shape* shape, const void* k, const void* v, void* pool, size_t pool_bytes,
                  void* ws, size_t ws_bytes, int32_t* dev_status, hipStream_t stream) {
    if (!shape || !k || !v || !pool || !ws) return KVC_E_NULL;
    if (!pool_shape(shape)) return KVC_E_SHAPE;
    const uint64_t need = kvpool_bytes(shape), ws_need = kvpool_workspace_bytes(shape);
    if (pool_bytes < need || ws_bytes < ws_need) return KVC_E_SIZE;
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(pool, 256) || !aligned(ws, 16) ||
        (dev_status && !aligned(dev_status, 4)))
        return KVC_E_ALIGN;
    const uint64_t kvb = kv_bytes(shape);
    const void* outs[3] = {pool, ws, dev_status};
    const uint64_t outn[3] = {need, ws_need, dev_status ? 4u : 0u};
    for (int i = 0; i < 3; ++i) {
        if (overlap(outs[i], outn[i], k, kvb) || overlap(outs[i], outn[i], v, kvb)) return KVC_E_ALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], outn[i], outs[j], outn[j])) return KVC_E_ALIAS;
    }
    const hipError_t e = kvc::launch_pool_encode(to_shape(shape), k, v, pool, static_cast<uint32_t*>(ws), dev_status,
                                                 stream);
    return e == hipSuccess ? KVC_OK : KVC_E_HIP;
}

int kvpool_encode_noalloc(const kvc_shape* shape, const void* k, const void* v, void* pool, size_t pool_bytes,
                          int32_t* dev_status, hipStream_t stream) {
    if (!shape || !k || !v || !pool) return KVC_E_NULL;
    if (!pool_shape(shape)) return KVC_E_SHAPE;
    const uint64_t need = kvpool_bytes(shape);
    if (pool_bytes < need) return KVC_E_SIZE;
    if (kvpool_workspace_bytes(shape) > kvc::kNoAllocScratchBytes) return KVC_E_SCRATCH;
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(pool, 256) || (dev_status && !aligned(dev_status, 4)))
        return KVC_E_ALIGN;
    const uint64_t kvb = kv_bytes(shape);
    if (overlap(pool, need, k, kvb) || overlap(pool, need, v, kvb)) return KVC_E_ALIAS;
    if (dev_status && (overlap(dev_status, 4, k, kvb) || overlap(dev_status, 4, v, kvb) ||
                       overlap(dev_status, 4, pool, need)))
        return KVC_E_ALIAS;
    uint32_t* ws = nullptr;
    if (kvc::noalloc_scratch(&ws) != hipSuccess) return KVC_E_HIP;
    // the scratch starts zeroed when the library is loaded; each call tags
    // the words it writes with its own call number, so nothing an earlier
    // call left there is taken for this call's
    const hipError_t e = kvc::launch_pool_encode(to_shape(shape), k, v, pool, ws, dev_status, stream);
    return e == hipSuccess ? KVC_OK : KVC_E_HIP;
}

int kvpool_decode(const kvc_shape* shape, const void* pool, size_t pool_bytes, uint32_t layer_begin,
                  uint32_t layer_end, void* const* k_out, void* const* v_out, uint32_t n_out,
                  int32_t* dev_status, hipStream_t stream) {
    if (!shape || !pool || !k_out || !v_out) return KVC_E_NULL;
    if (!pool_shape(shape)) return KVC_E_SHAPE;
    if (layer_begin > layer_end || layer_end > shape->num_layers) return KVC_E_RANGE;
    if (n_out < 1 || n_out > KVC_MAX_AGENTS) return KVC_E_RANGE;
    for (uint32_t a = 0; a < n_out; ++a)
        if (!k_out[a] || !v_out[a]) return KVC_E_NULL;
    const uint64_t need = kvpool_bytes(shape);
    if (pool_bytes < need) return KVC_E_SIZE;
    if (!aligned(pool, 256) || (dev_status && !aligned(dev_status, 4))) return KVC_E_ALIGN;
    for (uint32_t a = 0; a < n_out; ++a)
        if (!aligned(k_out[a], 16) || !aligned(v_out[a], 16)) return KVC_E_ALIGN;
    const uint64_t ob = (uint64_t)(layer_end - layer_begin) * shape->num_kv_heads * shape->num_tokens *
                        shape->head_dim * 2;
    for (uint32_t a = 0; a < n_out; ++a) {
        if (overlap(k_out[a], ob, pool, need) || overlap(v_out[a], ob, pool, need) ||
            overlap(k_out[a], ob, v_out[a], ob))
            return KVC_E_ALIAS;
        if (dev_status && (overlap(dev_status, 4, k_out[a], ob) || overlap(dev_status, 4, v_out[a], ob)))
            return KVC_E_ALIAS;
        for (uint32_t b = a + 1; b < n_out; ++b)
            if (overlap(k_out[a], ob, k_out[b], ob) || overlap(k_out[a], ob, v_out[b], ob) ||
                overlap(v_out[a], ob, k_out[b], ob) || overlap(v_out[a], ob, v_out[b], ob))
                return KVC_E_ALIAS;
    }
    if (dev_status && overlap(dev_status, 4, pool, need)) return KVC_E_ALIAS;
    if (layer_begin == layer_end) return KVC_OK;
    const hipError_t e = kvc::launch_pool_decode(to_shape(shape), pool, layer_begin, layer_end, k_out, v_out,
                                                 n_out, dev_status, stream);
    return e == hipSuccess ? KVC_OK : KVC_E_HIP;
}

size_t cachecard_record_bytes(uint32_t head_dim, uint32_t bits) {
    if (head_dim != 64 && head_dim != 128) return 0;
    return kvc::card_record_bytes(head_dim, bits);
}

size_t cachecard_max_bytes(const kvc_shape* shape) {
    if (!card_shape(shape)) return 0;
    const uint64_t S = align_up((uint64_t)shape->num_tokens * 2 * shape->head_dim, 256);
    return (size_t)(kvc::card_payload_offset(shape->num_tokens) +
                    2ull * shape->num_layers * shape->num_kv_heads * S);
}

size_t cachecard_bytes_host(const kvc_shape* shape, const uint8_t* widths_host) {
    if (!card_shape(shape) || !widths_host) return 0;
    uint64_t sum = 0;
    for (uint32_t t = 0; t < shape->num_tokens; ++t) {
        const uint32_t r = kvc::card_record_bytes(shape->head_dim, widths_host[t]);
        if (r == 0) return 0;
        sum += r;
    }
    return (size_t)(kvc::card_payload_offset(shape->num_tokens) +
                    2ull * shape->num_layers * shape->num_kv_heads * align_up(sum, 256));
}

size_t cachecard_workspace_bytes(const kvc_shape* shape) {
    if (!card_shape(shape)) return 0;
    return (size_t)card_ws_bytes(shape);
}

int cachecard_pack(const kvc_shape* shape, const void* k, const void* v, const uint8_t* widths,
                   const kvc_card_meta* meta, void* card, size_t card_capacity, uint64_t* dev_card_bytes,
                   int32_t* dev_status, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!shape || !k || !v || !widths || !meta || !card || !ws) return KVC_E_NULL;
    if (!card_shape(shape)) return KVC_E_SHAPE;
    if (meta->group_size != 0 && meta->group_size != 32) return KVC_E_RANGE;
    const uint64_t ws_need = card_ws_bytes(shape);
    if (ws_bytes < ws_need || card_capacity < kvc::card_payload_offset(shape->num_tokens)) return KVC_E_SIZE;
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(card, 256) || !aligned(ws, 16) ||
        (dev_card_bytes && !aligned(dev_card_bytes, 8)) || (dev_status && !aligned(dev_status, 4)))
        return KVC_E_ALIGN;
    const uint64_t kvb = kv_bytes(shape), T = shape->num_tokens;
    const void* outs[4] = {card, ws, dev_card_bytes, dev_status};
    const uint64_t outn[4] = {card_capacity, ws_need, dev_card_bytes ? 8u : 0u, dev_status ? 4u : 0u};
    for (int i = 0; i < 4; ++i) {
        if (overlap(outs[i], outn[i], k, kvb) || overlap(outs[i], outn[i], v, kvb) ||
            overlap(outs[i], outn[i], widths, T))
            return KVC_E_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outn[i], outs[j], outn[j])) return KVC_E_ALIAS;
    }
    kvc::CardMetaDev m;
    memset(&m, 0, sizeof(m));
    size_t n = strnlen(meta->model_id, sizeof(meta->model_id));
    if (n > 63) n = 63;
    memcpy(m.model_id, meta->model_id, n);
    m.position_offset = meta->position_offset;
    const hipError_t e = kvc::launch_card_pack(to_shape(shape), k, v, widths, m, card, card_capacity,
                                               dev_card_bytes, dev_status, ws, stream);
    return e == hipSuccess ? KVC_OK : KVC_E_HIP;
}

int kvc_realign_keys(const kvc_shape* shape, const void* k_in, void* k_out, int64_t delta, const float* inv_freq,
                     uint32_t pairing, hipStream_t stream) {
    if (!shape || !k_in || !k_out || !inv_freq) return KVC_E_NULL;
    if (!pool_shape(shape)) return KVC_E_SHAPE;
    if (pairing > 1) return KVC_E_RANGE;
    if (!aligned(k_in, 16) || !aligned(k_out, 16)) return KVC_E_ALIGN;
    const uint64_t kb = kv_bytes(shape);
    if (k_in != k_out && overlap(k_in, kb, k_out, kb)) return KVC_E_ALIAS;
    const hipError_t e = kvc::launch_realign_keys(to_shape(shape), k_in, k_out, delta, inv_freq, pairing, stream);
    return e == hipSuccess ? KVC_OK : KVC_E_HIP;
}

int kvc_lowrank_materialize(const kvc_shape* shape, uint32_t rank, uint32_t n_anchors, const void* src,
                            const void* a, const void* r, const float* weights, void* out, hipStream_t stream) {
    if (!shape || !src || !a || !r || !weights || !out) return KVC_E_NULL;
    if (!pool_shape(shape)) return KVC_E_SHAPE;
    const uint32_t L = shape->num_layers, H = shape->num_kv_heads, T = shape->num_tokens, d = shape->head_dim;
    if ((rank != 32 && rank != 64) || n_anchors < 1 || n_anchors > kvc::kLowrankMaxAnchors ||
        kvc::lowrank_lds_bytes(d, n_anchors, rank) > kvc::kLowrankMaxLds)
        return KVC_E_RANGE;
    const uint64_t tiles = ((uint64_t)T + 191) / 192, groups = ((uint64_t)L + 7) / 8;  // the smaller tile
    if (groups * 8 * tiles * H > 0x7FFFFFFFull) return KVC_E_SHAPE;
    if ((uint64_t)T * rank * 2 > 0x7FFFFFFFull) return KVC_E_SHAPE;  // one anchor's A rows as a buffer
    if (!aligned(src, 16) || !aligned(a, 16) || !aligned(r, 16) || !aligned(out, 16) || !aligned(weights, 4))
        return KVC_E_ALIGN;
    const uint64_t kb = kv_bytes(shape);
    const uint64_t ab = (uint64_t)L * n_anchors * T * rank * 2, rb = (uint64_t)L * n_anchors * H * d * rank * 2;
    const uint64_t wb = (uint64_t)L * n_anchors * 4;
    if ((out != src && overlap(out, kb, src, kb)) || overlap(out, kb, a, ab) || overlap(out, kb, r, rb) ||
        overlap(out, kb, weights, wb))
        return KVC_E_ALIAS;
    const hipError_t e = kvc::launch_lowrank_materialize(L, H, T, d, n_anchors, rank, src, a, r, weights, out, stream);
    return e == hipSuccess ? KVC_OK : KVC_E_HIP;
}

size_t kvc_lowrank_factor_workspace_bytes(const kvc_shape* shape, uint32_t rank) {
    if (!pool_shape(shape) || rank != 32) return 0;
    return (size_t)kvc::lowrank_factor_ws(shape->num_layers, shape->num_kv_heads, shape->num_tokens, shape->head_dim)
        .total;
}

int kvc_lowrank_factor(const kvc_shape* shape, uint32_t rank, const void* z, const float* omega, void* a_out,
                       uint64_t a_stride, void* r_out, uint64_t r_stride, float* sigma_out, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
    if (!shape || !z || !omega || !a_out || !r_out || !ws) return KVC_E_NULL;
    if (!pool_shape(shape)) return KVC_E_SHAPE;
    const uint32_t L = shape->num_layers, H = shape->num_kv_heads, T = shape->num_tokens, d = shape->head_dim;
    if ((uint64_t)L * H > 65535 || L > 65535) return KVC_E_SHAPE;
    if (rank != 32) return KVC_E_RANGE;
    const uint64_t Dt = (uint64_t)H * d;
    if (a_stride < (uint64_t)T * rank || r_stride < Dt * rank) return KVC_E_RANGE;
    const uint64_t need = kvc::lowrank_factor_ws(L, H, T, d).total;
    if (ws_bytes < need) return KVC_E_SIZE;
    if (!aligned(z, 16) || !aligned(omega, 16) || !aligned(a_out, 16) || !aligned(r_out, 16) || !aligned(ws, 256) ||
        a_stride % 8 != 0 || r_stride % 8 != 0 || (sigma_out && !aligned(sigma_out, 4)))
        return KVC_E_ALIGN;
    const uint64_t zb = kv_bytes(shape), ob = Dt * kvc::kLowrankSketch * 4;
    const uint64_t ab = ((uint64_t)(L - 1) * a_stride + (uint64_t)T * rank) * 2;
    const uint64_t rb = ((uint64_t)(L - 1) * r_stride + Dt * rank) * 2, sb = sigma_out ? (uint64_t)L * rank * 4 : 0;
    const void* outs[4] = {a_out, r_out, ws, sigma_out};
    const uint64_t outn[4] = {ab, rb, need, sb};
    for (int i = 0; i < 4; ++i) {
        if (overlap(outs[i], outn[i], z, zb) || overlap(outs[i], outn[i], omega, ob)) return KVC_E_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outn[i], outs[j], outn[j])) return KVC_E_ALIAS;
    }
    const hipError_t e = kvc::launch_lowrank_factor(L, H, T, d, z, omega, a_out, a_stride, r_out, r_stride, sigma_out,
                                                    ws, stream);
    return e == hipSuccess ? KVC_OK : KVC_E_HIP;
}

size_t cachecard_transcode_workspace_bytes(const kvc_shape* shape) {
    if (!card_shape(shape)) return 0;
    return (size_t)(2 * card_ws_bytes(shape));
}

int cachecard_transcode(const kvc_shape* shape, const void* card_in, size_t card_in_bytes,
                        const uint8_t* new_widths, void* card_out, size_t card_capacity, uint64_t* dev_card_bytes,
                        int32_t* dev_status, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!shape || !card_in || !new_widths || !card_out || !ws) return KVC_E_NULL;
    if (!card_shape(shape)) return KVC_E_SHAPE;
    const uint64_t ws_need = 2 * card_ws_bytes(shape), T = shape->num_tokens;
    const uint64_t head = kvc::card_payload_offset(shape->num_tokens);
    if (ws_bytes < ws_need || card_in_bytes < head || card_capacity < head) return KVC_E_SIZE;
    if (!aligned(card_in, 256) || !aligned(card_out, 256) || !aligned(ws, 16) ||
        (dev_card_bytes && !aligned(dev_card_bytes, 8)) || (dev_status && !aligned(dev_status, 4)))
        return KVC_E_ALIGN;
    const void* outs[4] = {card_out, ws, dev_card_bytes, dev_status};
    const uint64_t outn[4] = {card_capacity, ws_need, dev_card_bytes ? 8u : 0u, dev_status ? 4u : 0u};
    for (int i = 0; i < 4; ++i) {
        if (overlap(outs[i], outn[i], card_in, card_in_bytes) || overlap(outs[i], outn[i], new_widths, T))
            return KVC_E_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outn[i], outs[j], outn[j])) return KVC_E_ALIAS;
    }
    const hipError_t e = kvc::launch_card_transcode(to_shape(shape), card_in, card_in_bytes, new_widths, card_out,
                                                    card_capacity, dev_card_bytes, dev_status, ws, stream);
    return e == hipSuccess ? KVC_OK : KVC_E_HIP;
}

int cachecard_unpack(const kvc_shape* shape, const void* card, size_t card_bytes, void* k_out, void* v_out,
                     int32_t* dev_status, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!shape || !card || !k_out || !v_out || !ws) return KVC_E_NULL;
    if (!card_shape(shape)) return KVC_E_SHAPE;
    const uint64_t ws_need = card_ws_bytes(shape);
    if (ws_bytes < ws_need || card_bytes < kvc::card_payload_offset(shape->num_tokens)) return KVC_E_SIZE;
    if (!aligned(k_out, 16) || !aligned(v_out, 16) || !aligned(card, 256) || !aligned(ws, 16) ||
        (dev_status && !aligned(dev_status, 4)))
        return KVC_E_ALIGN;
    const uint64_t kvb = kv_bytes(shape);
    const void* outs[4] = {k_out, v_out, ws, dev_status};
    const uint64_t outn[4] = {kvb, kvb, ws_need, dev_status ? 4u : 0u};
    for (int i = 0; i < 4; ++i) {
        if (overlap(outs[i], outn[i], card, card_bytes)) return KVC_E_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outn[i], outs[j], outn[j])) return KVC_E_ALIAS;
    }
    const hipError_t e = kvc::launch_card_unpack(to_shape(shape), card, card_bytes, k_out, v_out, dev_status, ws,
                                                 stream);
    return e == hipSuccess ? KVC_OK : KVC_E_HIP;
}

int kvc_parse_header(const void* host_bytes, size_t n, kvc_shape* shape_out, uint32_t* kind_out) {
    if (!host_bytes || !shape_out || !kind_out) return KVC_E_NULL;
    const uint8_t* b = static_cast<const uint8_t*>(host_bytes);
    if (n < kvc::kPoolHeaderBytes) return KVC_E_SIZE;
    const uint32_t magic = rd32(b), ver = rd32(b + 4);
    kvc_shape s{rd32(b + 8), rd32(b + 12), rd32(b + 16), rd32(b + 20)};
    if (magic == kvc::kPoolMagic) {
        if (ver != (1u | (1u << 16)) || !pool_shape(&s)) return KVC_E_FORMAT;
        const kvc::PoolLayout lay = kvc::pool_layout(s.num_layers, s.num_kv_heads, s.num_tokens, s.head_dim);
        if (rd64(b + 24) != lay.k_scale || rd64(b + 32) != lay.k_codes || rd64(b + 40) != lay.v_scale ||
            rd64(b + 48) != lay.v_codes || rd64(b + 56) != lay.total)
            return KVC_E_FORMAT;
        *shape_out = s;
        *kind_out = 1;
        return KVC_OK;
    }
    if (magic == kvc::kCardMagic) {
        if (n < kvc::kCardHeaderBytes) return KVC_E_SIZE;
        if (ver != (1u | (2u << 16)) || !card_shape(&s) || rd32(b + 24) != kvc::kCardGroup ||
            rd64(b + 40) != kvc::kCardHeaderBytes || rd64(b + 48) != kvc::card_payload_offset(s.num_tokens))
            return KVC_E_FORMAT;
        const uint64_t S = rd64(b + 56), total = rd64(b + 64);
        if (S % 256 != 0 || total != rd64(b + 48) + 2ull * s.num_layers * s.num_kv_heads * S) return KVC_E_FORMAT;
        *shape_out = s;
        *kind_out = 2;
        return KVC_OK;
    }
    return KVC_E_FORMAT;
}

const char* kvc_strerror(int code) {
    switch (code) {
        case KVC_OK: return "ok";
        case KVC_E_NULL: return "a required pointer is NULL";
        case KVC_E_SHAPE: return "shape out of range (head_dim must be 64 or 128, sizes >= 1)";
        case KVC_E_SIZE: return "a buffer is smaller than required";
        case KVC_E_ALIGN: return "a pointer is not aligned as required";
        case KVC_E_ALIAS: return "an output overlaps an input or another output";
        case KVC_E_FORMAT: return "malformed pool or card header";
        case KVC_E_RANGE: return "argument out of range (layer range, agent count, pairing, rank or anchors)";
        case KVC_E_HIP: return "kernel launch failed";
        case KVC_E_SCRATCH: return "the shape needs more workspace than the library's allocation-free scratch holds";
        default: return "unknown error";
    }
}

void kvc_codebook(float levels[8], float thresholds[7]) {
    const float pos[4] = {kvc::kLv0, kvc::kLv1, kvc::kLv2, kvc::kLv3};
    for (int i = 0; i < 4; ++i) {
        levels[4 + i] = pos[i];
        levels[3 - i] = -pos[i];
    }
    const float th[3] = {kvc::kTh5, kvc::kTh6, kvc::kTh7};
    thresholds[3] = 0.0f;
    for (int i = 0; i < 3; ++i) {
        thresholds[4 + i] = th[i];
        thresholds[2 - i] = -th[i];
    }
}

}  // extern "C"
