/*
 * kvcodec.h - compressed KV-cache codec for multi-agent handoff, AMD Instinct
 * MI355X (gfx950). C ABI; every entry point is extern "C".
 *
 * Two modes, both write-once / read-many:
 *
 *  Pool mode - PolyKV, "A Shared Asymmetrically-Compressed KV Cache Pool for
 *  Multi-Agent LLM Inference" (gist.science/ko/paper/2604.24971):
 *    section 2.A (SharedKVPool, PooledAgent): the whole KV state of a shared
 *    document is compressed once into one object; every agent decompresses
 *    it layer by layer into its own cache;
 *    section 2.B item 1: keys become int8 with one linear scale per tensor
 *    (here: per layer, over all heads, tokens and channels);
 *    section 2.B item 2: values are rotated by the fast Walsh-Hadamard
 *    transform, each coordinate is mapped to a 3-bit Lloyd-Max level for
 *    N(0,1) (after division by a per-vector fp16 RMS scale), and decoding
 *    looks the levels up and applies the inverse transform.
 *
 *  CacheCard mode - QKVShare, "Quantized KV-Cache Handoff for Multi-Agent
 *  On-Device LLMs" (gist.science/ko/paper/2605.03884), method items 1-3: each
 *  token carries a bit-width from {2, 4, 8, FP16}; the CacheCard holds the
 *  quantised KV groups (here: 32 consecutive channels, min-max), the token
 *  widths and metadata (sequence length, model ID, position offset); the
 *  receiver rebuilds full-width past_key_values before its forward pass.
 *
 * Conventions for every call:
 *  - Tensors are bf16 [L][H][T][d] (layer, kv-head, token, channel), dense,
 *    row = one head vector; d is 64 or 128.
 *  - Pointers are device memory unless marked "host". Device pointers must
 *    be 16-byte aligned (pools and cards 256-byte aligned).
 *  - The caller owns every buffer; size queries give every buffer size. The
 *    library allocates and frees nothing (kvpool_encode_noalloc's per-GPU
 *    array is part of the library's device image). Between calls it keeps
 *    only the encode's call counter and the addresses of those arrays.
 *  - Device work is enqueued on `stream` and is asynchronous: synchronise
 *    before reading outputs, byte counts or status words on the host.
 *  - Host-detectable errors return a negative KVC_E_* code before anything is
 *    enqueued. Data errors found on the device (bad header, bad width, card
 *    too large for its buffer) set bits of *dev_status (when not NULL); the
 *    affected outputs are then unspecified.
 *  - Outputs must not overlap inputs (checked on address ranges).
 *  - Pools and cards are never written by decode/unpack, so any number of
 *    decodes of one pool may run concurrently on any streams. Two encodes
 *    sharing one workspace must not overlap.
 */
#ifndef KVCODEC_H
#define KVCODEC_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kvc_shape {
    uint32_t num_layers;   /* L >= 1 */
    uint32_t num_kv_heads; /* H >= 1 */
    uint32_t num_tokens;   /* T >= 1 */
    uint32_t head_dim;     /* d: 64 or 128 */
} kvc_shape;

/* CacheCard metadata besides the sequence length (QKVShare method item 2). */
typedef struct kvc_card_meta {
    char model_id[64];       /* NUL-terminated, at most 63 characters kept */
    int64_t position_offset; /* position of token 0 in the sender's sequence */
    uint32_t group_size;     /* channels per quantisation group: 32, the only
                                size (0 is taken as 32; others are refused) */
} kvc_card_meta;

enum {
    KVC_OK = 0,
    KVC_E_NULL = -1,   /* a required pointer is NULL */
    KVC_E_SHAPE = -2,  /* shape out of range (d not 64/128, zero sizes) */
    KVC_E_SIZE = -3,   /* a buffer is smaller than required */
    KVC_E_ALIGN = -4,  /* a pointer is not aligned as required */
    KVC_E_ALIAS = -5,  /* an output overlaps an input or another output */
    KVC_E_FORMAT = -6, /* malformed header bytes */
    KVC_E_RANGE = -7,  /* argument out of range (layer range, agent count, ...) */
    KVC_E_HIP = -8,    /* a kernel launch failed */
    KVC_E_SCRATCH = -9 /* needs more workspace than kvpool_encode_noalloc's scratch */
};

/* Bits set in *dev_status by device-side checks. */
enum {
    KVC_DEV_BAD_HEADER = 1, /* pool/card header does not match the shape */
    KVC_DEV_BAD_WIDTH = 2,  /* a token width is not 2, 4, 8 or 16 */
    KVC_DEV_CAPACITY = 4,   /* the card does not fit card_capacity */
    KVC_DEV_ENCODE_TIMEOUT = 8 /* an internal wait of the encode gave up */
};

#define KVC_MAX_AGENTS 64

/* ---------------------------------------------------------------- pool mode */

/* Exact size in bytes of the pool for `shape` (PolyKV 2.A: one object,
 * independent of the number of agents); 0 if the shape is invalid.
 * Layout (little-endian, sections on 256-byte boundaries):
 *   header 64 B: "KVPL", u16 version 1, u16 kind 1, u32 L, H, T, d,
 *                u64 offsets of k_scale, k_codes, v_scale, v_codes, u64 total
 *   k_scale f32[L]           per-layer key step m_l / 127
 *   k_codes i8[L][H][T][d]   round(x * 127 / m_l)
 *   v_scale f16[L][H][T]     RMS of each value vector
 *   v_codes u8[L][H][T][3][d/8]  3 bit planes per vector: bit m of byte j
 *           of plane p is bit p of the 3-bit code of coordinate 8j+m
 * Payload ratio against bf16 K+V: 16 / 5.5 (PolyKV 2.B, compression ratio). */
size_t kvpool_bytes(const kvc_shape* shape);

/* Workspace bytes needed by kvpool_encode (per-layer reductions). The
 * workspace must hold zeros before its first encode (e.g. one hipMemset
 * after allocation) and must not be written by anything else afterwards;
 * it then serves any number of encodes in sequence, of any shapes, with no
 * clearing in between (each call tags the words it writes with a number of
 * its own, and ignores words that carry another; the numbers run on from a
 * random start in each loaded instance of the library, so a workspace may
 * also pass from one instance to another). */
size_t kvpool_workspace_bytes(const kvc_shape* shape);

/* Compress bf16 K and V ([L][H][T][d]) into `pool` (PolyKV 2.B items 1-2).
 *   k, v       device, bf16, 16-byte aligned, read only
 *   pool       device, >= kvpool_bytes(shape), 256-byte aligned; fully written
 *              (header, sections and zero padding)
 *   ws         device workspace of >= kvpool_workspace_bytes(shape) bytes,
 *              16-byte aligned, zeroed before its first use (see above)
 *   dev_status device int32 or NULL: KVC_DEV_ENCODE_TIMEOUT if an internal
 *              wait gave up (never expected); the pool's magic word is then
 *              zero and decode refuses it
 * Keys: m_l = max |K[l]| over the layer; codes clamp(rint(x*(127/m_l))).
 * Inputs are expected finite. The maximum is taken on the bf16 bit patterns
 * with the sign cleared (NaN ranks above Inf), so a layer holding an Inf or
 * NaN key gets a NaN scale and all-zero codes (its keys decode to NaN); a
 * value vector holding Inf or NaN gets the scale 65504 and codes from the
 * comparisons of its (non-finite) rotated coordinates (NaN: code 0).
 * Values: per vector, s = fp16(sqrt(sum x^2 / d)), y = H x (Sylvester
 * order), z = y / (sqrt(d) s), code = number of Lloyd-Max thresholds <= z.
 * Execution: one kernel, which reads each key once from memory. Where a
 * round of whole layers fits the LDS of one workgroup per CU, keys wait in
 * LDS for their layer's maximum; otherwise (long contexts) workgroups that
 * take a layer's maximum run one layer ahead of those that encode it, which
 * re-read the keys shortly after (from the GPU's cache, not HBM). Both are
 * ordinary launches: a wave that has not received every workgroup's key
 * maximum for a layer within a bound (200 us by default; environment
 * variable KVC_ENCODE_POLL_US, read at each call, 0 = always) reads the
 * layer's keys itself (values above 5000 are ignored). The pool is the
 * same either way; only the time differs.
 * Errors: KVC_E_NULL, KVC_E_SHAPE, KVC_E_SIZE, KVC_E_ALIGN, KVC_E_ALIAS,
 * KVC_E_HIP. */
int kvpool_encode(const kvc_shape* shape, const void* k, const void* v, void* pool,
                  size_t pool_bytes, void* ws, size_t ws_bytes, int32_t* dev_status,
                  hipStream_t stream);

/* kvpool_encode without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc). The
 * workspace is a 1 MiB array inside the library, one per GPU (the current
 * device's is used; `stream` must belong to that device), which each GPU
 * holds until the process ends: shapes whose kvpool_workspace_bytes exceeds
 * 1 MiB (more than 255 layers) are refused with KVC_E_SCRATCH. Every call on
 * a GPU uses that GPU's one array, so calls that overlap in time on one GPU
 * (other streams, other threads) race and must not be issued; calls in
 * sequence on one stream are fine. The array is zero when the library is
 * loaded and needs no clearing between calls. Arguments, output, status bits and the
 * remaining errors are those of kvpool_encode (without the workspace
 * checks); the pool is byte-identical to kvpool_encode's. */
int kvpool_encode_noalloc(const kvc_shape* shape, const void* k, const void* v, void* pool,
                          size_t pool_bytes, int32_t* dev_status, hipStream_t stream);

/* Decompress layers [layer_begin, layer_end) of `pool` into the caches of
 * n_out agents (PolyKV 2.A, PooledAgent: layer-wise injection into each
 * agent's own cache; 2.B item 2: level lookup, then inverse transform).
 * The pool is read once; every agent receives the same bf16 values.
 *   pool          device, as written by kvpool_encode, read only
 *   k_out, v_out  host arrays of n_out (1..KVC_MAX_AGENTS) device pointers,
 *                 each bf16 [layer_end-layer_begin][H][T][d], 16-byte aligned
 *   dev_status    device int32 or NULL; KVC_DEV_BAD_HEADER if the pool's
 *                 header does not match `shape`
 * Calling it with (l, l+1) for l = 0..L-1 in order streams the cache layer
 * by layer. An empty range enqueues nothing and returns KVC_OK.
 * Errors: KVC_E_NULL, KVC_E_SHAPE, KVC_E_SIZE, KVC_E_ALIGN, KVC_E_ALIAS,
 * KVC_E_RANGE, KVC_E_HIP. */
int kvpool_decode(const kvc_shape* shape, const void* pool, size_t pool_bytes,
                  uint32_t layer_begin, uint32_t layer_end, void* const* k_out,
                  void* const* v_out, uint32_t n_out, int32_t* dev_status,
                  hipStream_t stream);

/* ------------------------------------------------------------ CacheCard mode */

/* Record bytes of one head vector at width b (QKVShare item 1 widths):
 * b in {2,4,8}: f16 scale[d/32], bf16 min[d/32], then d codes of b bits,
 * least significant bit first, padded to 16 bytes; b = 16: the d bf16
 * inputs unchanged. 0 for any other b. For d = 128: 48, 80, 144, 256. */
size_t cachecard_record_bytes(uint32_t head_dim, uint32_t bits);

/* Upper bound on the card size (every token at width 16). */
size_t cachecard_max_bytes(const kvc_shape* shape);

/* Exact card size for host-resident widths (u8[T]); 0 if a width or the
 * shape is invalid. Layout (little-endian):
 *   header 256 B: "QKVC", u16 version 1, u16 kind 2, u32 L, H, T, d,
 *     u32 group size 32, u32 0, i64 position offset, u64 widths offset (256),
 *     u64 payload offset, u64 stream bytes S, u64 total, char model_id[64]
 *   widths u8[T] at 256, zero padding to a 256-byte boundary
 *   payload: 2*L*H streams of S bytes; stream (l, kv, h) at index
 *     (2*l + kv)*H + h (kv 0 = K, 1 = V); token t's record starts at the sum
 *     of the record sizes of tokens 0..t-1; S rounds that sum up to 256. */
size_t cachecard_bytes_host(const kvc_shape* shape, const uint8_t* widths_host);

/* Workspace bytes needed by cachecard_pack / cachecard_unpack (record
 * offsets; cards of up to 8192 tokens compute them inside the pack / unpack
 * grid and leave the workspace untouched, but the argument is checked the
 * same way for every T). */
size_t cachecard_workspace_bytes(const kvc_shape* shape);

/* Package K and V into a CacheCard (QKVShare item 2).
 *   k, v            device bf16 [L][H][T][d]; d a multiple of 32 (64 or 128)
 *   widths          device u8[T], each 2, 4, 8 or 16; one width per token,
 *                   shared by every layer, head, K and V
 *   meta            host; model_id and position_offset copied into the header;
 *                   group_size 32 (or 0)
 *   card            device, card_capacity bytes, 256-byte aligned
 *   dev_card_bytes  device u64 or NULL; receives the card's exact size
 *   dev_status      device int32 or NULL; KVC_DEV_BAD_WIDTH, KVC_DEV_CAPACITY
 *                   (then the card's magic word is zero and unpack refuses it)
 *   ws              device workspace, >= cachecard_workspace_bytes(shape)
 * Per group of 32 channels at width b < 16: mn, mx = group min and max,
 * s = fp16((mx - mn) / (2^b - 1)), q = min(rint((x - mn) / s), 2^b - 1).
 * Errors: KVC_E_NULL, KVC_E_SHAPE, KVC_E_RANGE (group_size), KVC_E_SIZE,
 * KVC_E_ALIGN, KVC_E_ALIAS, KVC_E_HIP. */
int cachecard_pack(const kvc_shape* shape, const void* k, const void* v, const uint8_t* widths,
                   const kvc_card_meta* meta, void* card, size_t card_capacity,
                   uint64_t* dev_card_bytes, int32_t* dev_status, void* ws, size_t ws_bytes,
                   hipStream_t stream);

/* Rebuild bf16 K and V from a CacheCard (QKVShare item 3: full-width
 * past_key_values for the receiver): x = bf16(fmaf(q, s, mn)), the binary32
 * value rounded to nearest even; width 16 copies.
 *   card        device, card_bytes valid bytes, read only
 *   k_out, v_out device bf16 [L][H][T][d]
 *   dev_status  device int32 or NULL; KVC_DEV_BAD_HEADER, KVC_DEV_BAD_WIDTH
 * The header is checked against the shape and against the sizes the widths
 * give (payload offset, stream bytes S, total, card_bytes); a card whose
 * widths were altered without changing any of those sizes is decoded as it
 * stands (the format carries no checksum).
 * Errors: KVC_E_NULL, KVC_E_SHAPE, KVC_E_SIZE, KVC_E_ALIGN, KVC_E_ALIAS,
 * KVC_E_HIP. */
int cachecard_unpack(const kvc_shape* shape, const void* card, size_t card_bytes, void* k_out,
                     void* v_out, int32_t* dev_status, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/* Workspace bytes needed by cachecard_transcode (two sets of record
 * offsets: the input card's and the output card's). */
size_t cachecard_transcode_workspace_bytes(const kvc_shape* shape);

/* One hop of a handoff chain (QKVShare: each agent forwards the cache as a
 * card at its own per-token widths; the pages call for a fused card-to-card
 * path): card_in re-encoded at new_widths into card_out without bf16 K/V
 * in between. The result equals, byte for byte, cachecard_unpack followed
 * by cachecard_pack at new_widths, with card_in's model ID and position
 * offset carried into the new header.
 *   card_in         device, card_in_bytes valid bytes, 256-byte aligned, read
 *                   only; its header must match shape
 *   new_widths      device u8[T], each 2, 4, 8 or 16
 *   card_out        device, card_capacity bytes, 256-byte aligned; header,
 *                   widths and payload written (cachecard_bytes_host of
 *                   new_widths gives the exact size)
 *   dev_card_bytes  device u64 or NULL; receives card_out's exact size
 *   dev_status      device int32 or NULL; KVC_DEV_BAD_HEADER (card_in),
 *                   KVC_DEV_BAD_WIDTH (either card), KVC_DEV_CAPACITY; on a
 *                   nonzero status card_out's magic word is zero (unpack and
 *                   later hops refuse it) and the rest is unspecified
 *   ws              device workspace, >= cachecard_transcode_workspace_bytes
 * Errors: KVC_E_NULL, KVC_E_SHAPE, KVC_E_SIZE, KVC_E_ALIGN, KVC_E_ALIAS,
 * KVC_E_HIP. */
int cachecard_transcode(const kvc_shape* shape, const void* card_in, size_t card_in_bytes,
                        const uint8_t* new_widths, void* card_out, size_t card_capacity,
                        uint64_t* dev_card_bytes, int32_t* dev_status, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* ------------------------------------------------------- key re-alignment */

/* Pairing of rotary channels: pair j is (j, j + d/2) or (2j, 2j + 1). */
#define KVC_ROPE_HALVES 0u
#define KVC_ROPE_ADJACENT 1u

/* Re-align the positions of rotary keys (KVCMAS, procedure: the key
 * positions of a shared segment are re-aligned to the target agent's before
 * reuse; a CacheCard carries the source position offset, QKVShare item 2).
 * Keys at position p hold channel pair j rotated by p * inv_freq[j];
 * re-aligning by delta rotates every pair j of every key vector by
 * delta * inv_freq[j] more.
 *   k_in, k_out  device bf16 [L][H][T][d], d = 64 or 128, 16-byte aligned;
 *                k_out == k_in re-aligns in place, any other overlap is an
 *                error
 *   delta        target position minus source position
 *   inv_freq     host, d/2 floats: the model's rotary inverse frequencies
 *   pairing      KVC_ROPE_HALVES or KVC_ROPE_ADJACENT
 * cos and sin of delta * inv_freq[j] (the product in binary64) are taken in
 * binary64 on the device; each rotated value is a*c - b*s or a*s + b*c in
 * binary64 (two products, then the sum), rounded once to bf16, ties to even.
 * Errors: KVC_E_NULL, KVC_E_SHAPE, KVC_E_RANGE (pairing), KVC_E_ALIGN,
 * KVC_E_ALIAS, KVC_E_HIP. */
int kvc_realign_keys(const kvc_shape* shape, const void* k_in, void* k_out, int64_t delta,
                     const float* inv_freq, uint32_t pairing, hipStream_t stream);

/* ------------------------------------------------------ low-rank anchors */

/* Materialise a cache from a source cache and low-rank anchors (KVCMAS,
 * low-rank anchor storage: a cache matrix Z of T tokens by D = H*d channels
 * is stored as truncated-SVD factors A = U_r S_r (T x r) and R = R_r
 * (D x r), Z ~ A R^T; a reused cache is corrected by a similarity-weighted
 * sum of stored anchors). For each of the L matrices (layers of one of K
 * or V) and every token t, head h and channel c:
 *     out[l][h][t][c] = bf16( src[l][h][t][c]
 *                      + sum_v w[l][v] * sum_k A[l][v][t][k] * R[l][v][h*d + c][k] )
 * The inner sum runs on the matrix cores with bf16 operands and binary32
 * accumulation; each anchor's sum is scaled by its weight and added in
 * binary32 (fused multiply-add, anchors in index order), src is added last
 * and the total rounded once to bf16, ties to even. Against the binary64
 * value rounded once, the result is within 1 bf16 ulp plus the binary32
 * error, at most (2r + V + 1) * 2^-24 * (|src| + sum_v |w_v| sum_k |A R|)
 * to first order (the products of bf16 operands are exact in binary32; 2r
 * covers r - 1 additions inside the matrix core even if they truncate).
 *   shape      L (matrices), H, T, d (64 or 128); T * r * 2 < 2^31
 *   rank       r: 32 or 64
 *   n_anchors  V: 1 .. 32, and V * d * r * 2 <= 131072 (at d = 128, r = 32:
 *              V <= 16)
 *   src, out   device bf16 [L][H][T][d], 16-byte aligned; out == src
 *              materialises in place, any other overlap is an error
 *   a          device bf16 [L][V][T][r] (row-major A factors), 16-byte aligned
 *   r          device bf16 [L][V][H*d][r] (row-major R factors), 16-byte aligned
 *   weights    device f32 [L][V]
 * Errors: KVC_E_NULL, KVC_E_SHAPE, KVC_E_RANGE (rank, n_anchors), KVC_E_ALIGN,
 * KVC_E_ALIAS, KVC_E_HIP. */
int kvc_lowrank_materialize(const kvc_shape* shape, uint32_t rank, uint32_t n_anchors, const void* src,
                            const void* a, const void* r, const float* weights, void* out, hipStream_t stream);

/* Workspace bytes for kvc_lowrank_factor (0 if the shape or rank is invalid). */
size_t kvc_lowrank_factor_workspace_bytes(const kvc_shape* shape, uint32_t rank);

/* Rank-r truncated SVD of cache matrices (KVCMAS, "what differs": the base
 * caches and delta corrections an anchor stores are kept as truncated SVDs
 * Z ~ U_r S_r R_r^T, A = U_r S_r, R = R_r). Matrix l is the T x (H*d) view of
 * z[l] (row t, column h*d + c = element [l][h][t][c]). The page does not fix
 * the algorithm; this is the randomized range finder with one power
 * iteration (Halko, Martinsson and Tropp, 2011) on a caller-supplied
 * Gaussian sketch, CholeskyQR in binary64 for the orthonormalisations, and
 * a binary64 Jacobi eigensolver for the 48 x 48 projected problem; the
 * matrix products run in binary32. Where the spectrum has a gap at r
 * (sigma_r clearly above sigma_{r+1}) the result agrees with the exact
 * truncated SVD up to the bf16 rounding of the factors; otherwise A R^T is
 * a rank-r approximation whose error is within a few percent of the
 * optimal one.
 *   shape       L matrices, H, T, d (64 or 128); L * H <= 65535
 *   rank        r: 32
 *   z           device bf16 [L][H][T][d], 16-byte aligned
 *   omega       device f32 [H*d][48], row-major: independent N(0, 1) draws
 *               (the sketch; the caller owns the random numbers)
 *   a_out       device bf16: A of matrix l at a_out + l * a_stride, T x r
 *               row-major; a_stride >= T * r, a multiple of 8 (so anchor v
 *               of a [L][V][T][r] array is a_out = base + v*T*r,
 *               a_stride = V*T*r)
 *   r_out       device bf16: R of matrix l at r_out + l * r_stride, (H*d) x r
 *               row-major; r_stride >= H*d*r, a multiple of 8
 *   sigma_out   device f32 [L][r] or NULL: singular values, descending
 *   ws          device workspace, 256-byte aligned,
 *               >= kvc_lowrank_factor_workspace_bytes
 * Singular values equal to 0 give zero columns in A and R.
 * Errors: KVC_E_NULL, KVC_E_SHAPE, KVC_E_RANGE (rank, strides), KVC_E_SIZE,
 * KVC_E_ALIGN, KVC_E_ALIAS, KVC_E_HIP. */
int kvc_lowrank_factor(const kvc_shape* shape, uint32_t rank, const void* z, const float* omega, void* a_out,
                       uint64_t a_stride, void* r_out, uint64_t r_stride, float* sigma_out, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* --------------------------------------------------------------- host utils */

/* Parse a pool or card header from host bytes; *kind = 1 (pool) or 2
 * (card). KVC_E_FORMAT on bad magic, version, kind or field values,
 * KVC_E_SIZE if n is shorter than the header. No device work. */
int kvc_parse_header(const void* host_bytes, size_t n, kvc_shape* shape_out, uint32_t* kind_out);

/* Static text for a KVC_E_* code. */
const char* kvc_strerror(int code);

/* The library's 3-bit level table (ascending, 8 values) and its 7 decision
 * thresholds, as used by the kernels. Host only. */
void kvc_codebook(float levels[8], float thresholds[7]);

#ifdef __cplusplus
}
#endif

#endif /* KVCODEC_H */
