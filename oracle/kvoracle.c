/*
 * kvoracle.c - plain, slow CPU reference of the compressed KV-cache codec.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library. It shares no code, header,
 * table or generator with the GPU library; the level table is passed in by the
 * caller (derived by oracle/codebook.py).
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -fPIC -shared.
 * Every float operation below is one IEEE-754 binary32 or binary64 operation
 * with round-to-nearest-even; nothing is fused or reassociated.
 *
 * Sources followed (the four pages on multi-agent KV sharing):
 *  - PolyKV (gist.science/ko/paper/2604.24971), section 2.A: one shared pool,
 *    written once and read by every agent, which decompresses layer by layer
 *    into its own cache.
 *  - PolyKV section 2.B item 1: keys quantised to int8 with one linear scale
 *    per tensor.
 *  - PolyKV section 2.B item 2: values rotated by the fast Walsh-Hadamard
 *    transform, mapped to Lloyd-Max levels for N(0,1); dequantisation looks
 *    the levels up and applies the inverse transform.
 *  - PolyKV section 2.B, compression ratio: 16 / ((8 + 3) / 2).
 *  - QKVShare (gist.science/ko/paper/2605.03884), method items 1-3: per-token
 *    bit-widths from {2, 4, 8, FP16}; the CacheCard carries quantised KV
 *    groups, the token widths and metadata (sequence length, model ID,
 *    position offset); the receiver rebuilds full-width past_key_values.
 *
 * Readings where the pages are silent (listed with reasons in the design
 * notes): keys use one scale per layer; each value vector gets an fp16 RMS
 * scale; the level table sits on a 2^-15 grid; CacheCard groups are 32
 * consecutive channels with min-max (asymmetric) quantisation; the "FP16"
 * width stores the bf16 input unchanged; the byte layouts below are this
 * codec's own.
 *
 * Precision: where a float decides an integer or a stored bit pattern (an
 * int8 code, a 3-bit code, an fp16 scale, a group minimum) the decision is
 * taken in binary32, the precision of the device kernels, in the operation
 * order written here. Reconstructions (decode) are computed in binary64 and
 * rounded once to bf16.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Thread count of the OpenMP loops below (timing only). */
void or_set_threads(int n) { omp_set_num_threads(n); }
int or_max_threads(void) { return omp_get_max_threads(); }

#define OR_OK 0
#define OR_E_ARG (-1)
#define OR_E_FORMAT (-2)

/* ------------------------------------------------------------------ */
/* number formats                                                      */
/* ------------------------------------------------------------------ */

float or_bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round a binary64 value to the nearest bf16 (8 significant bits, the
 * binary32 exponent range), ties to even. Exact value in, one rounding out. */
uint16_t or_f64_to_bf16(double x) {
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double ax = fabs(x);
    if (isnan(x)) return 0x7FC0u;
    if (ax == 0.0) return sign;
    int e;
    frexp(ax, &e);               /* ax = f * 2^e, f in [0.5, 1) */
    int lead = e - 1;            /* weight of the leading bit is 2^lead */
    if (lead < -126) lead = -126;/* below the normal range the quantum is fixed */
    double quantum = ldexp(1.0, lead - 7);
    double r = nearbyint(ax / quantum) * quantum;
    if (r > 3.3895313892515355e38) return (uint16_t)(sign | 0x7F80u); /* overflow */
    float f = (float)r;          /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | (u >> 16));
}

/* Round a binary32 value to the nearest IEEE binary16, ties to even;
 * overflow gives infinity. */
uint16_t or_f32_to_f16(float xf) {
    double x = xf;
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double ax = fabs(x);
    if (isnan(x)) return 0x7E00u;
    if (ax == 0.0) return sign;
    int e;
    frexp(ax, &e);
    int lead = e - 1;
    if (lead < -14) lead = -14;
    double quantum = ldexp(1.0, lead - 10);
    double r = nearbyint(ax / quantum) * quantum;
    if (r > 65504.0) return (uint16_t)(sign | 0x7C00u);
    if (r < ldexp(1.0, -14)) {                    /* subnormal */
        uint32_t m = (uint32_t)(r / ldexp(1.0, -24));
        return (uint16_t)(sign | m);
    }
    frexp(r, &e);
    int ex = e - 1;                               /* r in [2^ex, 2^(ex+1)) */
    uint32_t mant = (uint32_t)((r / ldexp(1.0, ex) - 1.0) * 1024.0);
    return (uint16_t)(sign | ((uint32_t)(ex + 15) << 10) | mant);
}

float or_f16_to_f32(uint16_t h) {
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 31;
    int mant = h & 1023;
    double v;
    if (ex == 0) v = ldexp((double)mant, -24);
    else if (ex == 31) v = mant ? NAN : INFINITY;
    else v = ldexp(1024.0 + mant, ex - 25);
    return (float)(sign ? -v : v);
}

static void put_u16(uint8_t* p, uint16_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static uint16_t get_u16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void put_u32(uint8_t* p, uint32_t v) { for (int i = 0; i < 4; ++i) p[i] = (uint8_t)(v >> (8 * i)); }
static uint32_t get_u32(const uint8_t* p) {
    uint32_t v = 0;
    for (int i = 0; i < 4; ++i) v |= (uint32_t)p[i] << (8 * i);
    return v;
}
static void put_u64(uint8_t* p, uint64_t v) { for (int i = 0; i < 8; ++i) p[i] = (uint8_t)(v >> (8 * i)); }
static uint64_t get_u64(const uint8_t* p) {
    uint64_t v = 0;
    for (int i = 0; i < 8; ++i) v |= (uint64_t)p[i] << (8 * i);
    return v;
}
static void put_f32(uint8_t* p, float f) { uint32_t u; memcpy(&u, &f, 4); put_u32(p, u); }
static float get_f32(const uint8_t* p) { uint32_t u = get_u32(p); float f; memcpy(&f, &u, 4); return f; }

static uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

/* ------------------------------------------------------------------ */
/* shared pool layout (PolyKV 2.A: one object for all agents)          */
/*                                                                     */
/*   0   header, 64 bytes: "KVPL", u16 version 1, u16 kind 1,          */
/*       u32 L, H, T, d, u64 offsets of the four sections, u64 total   */
/*   k_scale  f32[L]                                                   */
/*   k_codes  i8[L][H][T][d]                                           */
/*   v_scale  f16[L][H][T]                                             */
/*   v_codes  u8[L][H][T][3][d/8]: 3 bit planes per vector            */
/* Sections start on 256-byte boundaries; the total is a multiple of   */
/* 256.                                                                */
/*                                                                     */
/* v_codes: plane p of a vector holds bit p of the 3-bit code of each  */
/* coordinate, in coordinate order, least significant bit first: bit m */
/* of byte j of plane p belongs to coordinate 8*j + m.                 */
/* ------------------------------------------------------------------ */

#define POOL_HEADER 64u
#define POOL_MAGIC 0x4C50564Bu /* bytes 'K','V','P','L' */

static int shape_ok(uint32_t L, uint32_t H, uint32_t T, uint32_t d) {
    return L > 0 && H > 0 && T > 0 && (d == 64 || d == 128);
}

/* off[0..4] = k_scale, k_codes, v_scale, v_codes, total */
int or_pool_layout(uint32_t L, uint32_t H, uint32_t T, uint32_t d, uint64_t off[5]) {
    if (!shape_ok(L, H, T, d)) return OR_E_ARG;
    uint64_t n_vec = (uint64_t)L * H * T;
    off[0] = 256;
    off[1] = round_up(off[0] + 4ull * L, 256);
    off[2] = round_up(off[1] + n_vec * d, 256);
    off[3] = round_up(off[2] + 2ull * n_vec, 256);
    off[4] = round_up(off[3] + n_vec * 3ull * (d / 8), 256);
    return OR_OK;
}

uint64_t or_pool_bytes(uint32_t L, uint32_t H, uint32_t T, uint32_t d) {
    uint64_t off[5];
    if (or_pool_layout(L, H, T, d, off)) return 0;
    return off[4];
}

/* Sum of squares by pairwise summation (split at the midpoint, left half
 * first), binary32. */
static float pairwise_sum_of_squares(const float* x, int n) {
    if (n == 1) return x[0] * x[0];
    int h = n / 2;
    return pairwise_sum_of_squares(x, h) + pairwise_sum_of_squares(x + h, n - h);
}

/* Unnormalised Walsh-Hadamard transform in Sylvester (natural) order:
 * butterfly stages h = 1, 2, 4, ..., n/2, in that order (PolyKV 2.B item 2). */
static void fwht_f32(float* y, int n) {
    for (int h = 1; h < n; h *= 2)
        for (int i = 0; i < n; i += 2 * h)
            for (int j = i; j < i + h; ++j) {
                float a = y[j], b = y[j + h];
                y[j] = a + b;
                y[j + h] = a - b;
            }
}

static void fwht_f64(double* y, int n) {
    for (int h = 1; h < n; h *= 2)
        for (int i = 0; i < n; i += 2 * h)
            for (int j = i; j < i + h; ++j) {
                double a = y[j], b = y[j + h];
                y[j] = a + b;
                y[j + h] = a - b;
            }
}

static float inv_sqrt_d(uint32_t d) { return (float)(1.0 / sqrt((double)d)); }

/* One value vector -> fp16 scale bits and 3-bit codes (PolyKV 2.B item 2).
 *   rms  = sqrt(sum x^2 / d)               (binary32, pairwise sum)
 *   s    = fp16(min(rms, 65504))
 *   y    = H x                             (binary32 butterfly, ascending)
 *   z_i  = y_i * (d^-1/2 / s)              (r = 0 when s = 0)
 *   code = number of thresholds b_k with z_i >= b_k
 * Since H / sqrt(d) is orthonormal, z has unit mean square when s = rms. */
static void v_normalised(const uint16_t* v, uint32_t d, float* z, uint16_t* scale_bits) {
    float x[128], y[128];
    for (uint32_t i = 0; i < d; ++i) x[i] = y[i] = or_bf16_to_f32(v[i]);
    float ss = pairwise_sum_of_squares(x, (int)d);
    float rms = sqrtf(ss * (1.0f / (float)d));
    uint16_t sh = or_f32_to_f16(fminf(rms, 65504.0f));
    float s = or_f16_to_f32(sh);
    fwht_f32(y, (int)d);
    float r = (s == 0.0f) ? 0.0f : inv_sqrt_d(d) / s;
    for (uint32_t i = 0; i < d; ++i) z[i] = y[i] * r;
    *scale_bits = sh;
}

void or_v_encode_vector(const uint16_t* v, uint32_t d, const float thr[7],
                        uint16_t* scale_bits, uint8_t* codes) {
    float z[128];
    v_normalised(v, d, z, scale_bits);
    for (uint32_t i = 0; i < d; ++i) {
        uint8_t c = 0;
        for (int k = 0; k < 7; ++k)
            if (z[i] >= thr[k]) c++;
        codes[i] = c;
    }
}

/* Reconstruction of one value vector, binary64:
 *   out = bf16( (s / sqrt(d)) * H [level(code_i)]_i ) */
void or_v_decode_vector(const uint8_t* codes, uint16_t scale_bits, uint32_t d,
                        const float levels[8], uint16_t* out) {
    double w[128];
    for (uint32_t i = 0; i < d; ++i) w[i] = (double)levels[codes[i]];
    fwht_f64(w, (int)d);
    double a = (double)or_f16_to_f32(scale_bits) / sqrt((double)d);
    for (uint32_t i = 0; i < d; ++i) out[i] = or_f64_to_bf16(w[i] * a);
}

/* Per-layer key scale (PolyKV 2.B item 1, one linear scale per tensor; the
 * tensor is one layer's K, all heads, tokens and channels). The maximum
 * magnitude is taken on the bf16 bit patterns with the sign cleared, as
 * unsigned integers: for finite values that is the order of |x|; an
 * infinity ranks above every finite value and a NaN above an infinity (the
 * pages define the codec on finite values only; this fixes what a layer
 * holding Inf or NaN gives, see or_pool_encode). */
float or_k_layer_absmax(const uint16_t* k_layer, uint64_t n) {
    uint16_t m = 0;
    for (uint64_t i = 0; i < n; ++i) {
        uint16_t a = (uint16_t)(k_layer[i] & 0x7FFFu);
        if (a > m) m = a;
    }
    return or_bf16_to_f32(m);
}

/* q = clamp(rint(x * (127 / m)), -127, 127); scale = m / 127 (binary32). */
static int8_t k_quantize(float x, float inv) {
    float u = x * inv;
    if (u > 127.0f) u = 127.0f;
    if (u < -127.0f) u = -127.0f;
    return (int8_t)rintf(u);
}

/* codes[d] -> 3 planes of d/8 bytes (coordinate i: byte i/8, bit i%8). */
static void v_pack_planes(const uint8_t* codes, uint32_t d, uint8_t* out) {
    memset(out, 0, 3u * (d / 8));
    for (uint32_t i = 0; i < d; ++i)
        for (uint32_t p = 0; p < 3; ++p)
            if ((codes[i] >> p) & 1u) out[p * (d / 8) + i / 8] |= (uint8_t)(1u << (i % 8));
}

static void v_unpack_planes(const uint8_t* in, uint32_t d, uint8_t* codes) {
    for (uint32_t i = 0; i < d; ++i) {
        uint8_t c = 0;
        for (uint32_t p = 0; p < 3; ++p) c |= (uint8_t)(((in[p * (d / 8) + i / 8] >> (i % 8)) & 1u) << p);
        codes[i] = c;
    }
}

/* How many values sit near a decision of the encoder, for the tolerance
 * report: out[0] counts keys whose x * (127 / m) (binary32) lies within eps
 * of a half-integer (the rounding decision), out[1] value coordinates whose
 * normalised rotated value z lies within eps of one of the 7 thresholds.
 * Same operations and order as or_pool_encode. */
int or_pool_near_boundary(uint32_t L, uint32_t H, uint32_t T, uint32_t d, const uint16_t* k,
                          const uint16_t* v, const float thr[7], double eps, uint64_t out[2]) {
    if (d != 64 && d != 128) return OR_E_ARG;
    uint64_t per_layer = (uint64_t)H * T * d, nk = 0, nv = 0;
    for (uint32_t l = 0; l < L; ++l) {
        const uint16_t* kl = k + l * per_layer;
        float m = or_k_layer_absmax(kl, per_layer);
        if (!isfinite(m) || m == 0.0f) continue;
        float inv = 127.0f / m;
        #pragma omp parallel for schedule(static) reduction(+ : nk)
        for (int64_t i = 0; i < (int64_t)per_layer; ++i) {
            double u = fabs((double)(or_bf16_to_f32(kl[i]) * inv));
            if (fabs(u - floor(u) - 0.5) < eps) nk++;
        }
    }
    int64_t n_vec = (int64_t)L * H * T;
    #pragma omp parallel for schedule(static) reduction(+ : nv)
    for (int64_t vec = 0; vec < n_vec; ++vec) {
        float z[128];
        uint16_t sh;
        v_normalised(v + (uint64_t)vec * d, d, z, &sh);
        for (uint32_t i = 0; i < d; ++i) {
            int near = 0;
            for (int t = 0; t < 7; ++t)
                if (fabs((double)z[i] - (double)thr[t]) < eps) near = 1;
            nv += (uint64_t)near;
        }
    }
    out[0] = nk;
    out[1] = nv;
    return OR_OK;
}

/* Encode K and V (bf16 [L][H][T][d], raw bits) into a pool (PolyKV 2.A/2.B). */
int or_pool_encode(uint32_t L, uint32_t H, uint32_t T, uint32_t d,
                   const uint16_t* k, const uint16_t* v, const float thr[7], uint8_t* pool) {
    uint64_t off[5];
    if (or_pool_layout(L, H, T, d, off)) return OR_E_ARG;
    memset(pool, 0, off[4]);
    put_u32(pool + 0, POOL_MAGIC);
    put_u16(pool + 4, 1);
    put_u16(pool + 6, 1);
    put_u32(pool + 8, L);
    put_u32(pool + 12, H);
    put_u32(pool + 16, T);
    put_u32(pool + 20, d);
    for (int i = 0; i < 5; ++i) put_u64(pool + 24 + 8 * i, off[i]);

    uint64_t per_layer = (uint64_t)H * T * d;
    for (uint32_t l = 0; l < L; ++l) {
        const uint16_t* kl = k + l * per_layer;
        float m = or_k_layer_absmax(kl, per_layer);
        int8_t* kc = (int8_t*)(pool + off[1]) + l * per_layer;
        if (!isfinite(m)) {
            /* a layer holding Inf or NaN keys: scale NaN (bits 0x7FC00000),
             * every code 0, so its keys decode to NaN */
            put_u32(pool + off[0] + 4ull * l, 0x7FC00000u);
            memset(kc, 0, per_layer);
            continue;
        }
        float scale = (m == 0.0f) ? 0.0f : m / 127.0f;
        float inv = (m == 0.0f) ? 0.0f : 127.0f / m;
        put_f32(pool + off[0] + 4ull * l, scale);
        #pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < (int64_t)per_layer; ++i)
            kc[i] = k_quantize(or_bf16_to_f32(kl[i]), inv);
    }

    int64_t n_vec = (int64_t)L * H * T;
    #pragma omp parallel for schedule(static)
    for (int64_t vec = 0; vec < n_vec; ++vec) {
        uint8_t codes[128];
        uint16_t sh;
        or_v_encode_vector(v + (uint64_t)vec * d, d, thr, &sh, codes);
        put_u16(pool + off[2] + 2 * (uint64_t)vec, sh);
        v_pack_planes(codes, d, pool + off[3] + (uint64_t)vec * 3u * (d / 8));
    }
    return OR_OK;
}

static int pool_header_ok(const uint8_t* pool, uint64_t n, uint32_t L, uint32_t H, uint32_t T,
                          uint32_t d, uint64_t off[5]) {
    if (or_pool_layout(L, H, T, d, off)) return 0;
    if (n < off[4]) return 0;
    if (get_u32(pool) != POOL_MAGIC || get_u16(pool + 4) != 1 || get_u16(pool + 6) != 1) return 0;
    if (get_u32(pool + 8) != L || get_u32(pool + 12) != H || get_u32(pool + 16) != T ||
        get_u32(pool + 20) != d)
        return 0;
    for (int i = 0; i < 5; ++i)
        if (get_u64(pool + 24 + 8 * i) != off[i]) return 0;
    return 1;
}

/* Decode layers [l0, l1) of a pool into bf16 K and V ([l1-l0][H][T][d]).
 * One decode serves every agent: each agent's buffer receives the same
 * values (PolyKV 2.A, per-agent layer-wise decompression). */
int or_pool_decode(uint32_t L, uint32_t H, uint32_t T, uint32_t d, const uint8_t* pool,
                   uint64_t pool_bytes, uint32_t l0, uint32_t l1, const float levels[8],
                   uint16_t* k_out, uint16_t* v_out) {
    uint64_t off[5];
    if (!pool_header_ok(pool, pool_bytes, L, H, T, d, off)) return OR_E_FORMAT;
    if (l0 > l1 || l1 > L) return OR_E_ARG;
    uint64_t per_layer = (uint64_t)H * T * d;
    for (uint32_t l = l0; l < l1; ++l) {
        double scale = (double)get_f32(pool + off[0] + 4ull * l);
        const int8_t* kc = (const int8_t*)(pool + off[1]) + l * per_layer;
        uint16_t* ko = k_out + (uint64_t)(l - l0) * per_layer;
        #pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < (int64_t)per_layer; ++i)
            ko[i] = or_f64_to_bf16((double)kc[i] * scale);
    }
    int64_t nv = (int64_t)(l1 - l0) * H * T;
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < nv; ++j) {
        uint64_t vec = (uint64_t)l0 * H * T + (uint64_t)j;
        uint8_t codes[128];
        v_unpack_planes(pool + off[3] + vec * 3u * (d / 8), d, codes);
        uint16_t sh = get_u16(pool + off[2] + 2 * vec);
        or_v_decode_vector(codes, sh, d, levels, v_out + (uint64_t)j * d);
    }
    return OR_OK;
}

/* Codes of every value vector, unpacked ([L][H][T][d] bytes) - for tests. */
int or_pool_v_codes(uint32_t L, uint32_t H, uint32_t T, uint32_t d, const uint8_t* pool,
                    uint64_t pool_bytes, uint8_t* codes_out) {
    uint64_t off[5];
    if (!pool_header_ok(pool, pool_bytes, L, H, T, d, off)) return OR_E_FORMAT;
    uint64_t nv = (uint64_t)L * H * T;
    for (uint64_t vec = 0; vec < nv; ++vec)
        v_unpack_planes(pool + off[3] + vec * 3u * (d / 8), d, codes_out + vec * d);
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* CacheCard (QKVShare method item 2)                                   */
/*                                                                     */
/*   0    header, 256 bytes: "QKVC", u16 version 1, u16 kind 2,        */
/*        u32 L, H, T, d, u32 group size (32), u32 0,                  */
/*        i64 position offset, u64 widths offset (256),                */
/*        u64 payload offset, u64 stream bytes S, u64 total,           */
/*        char model_id[64] at byte 72, rest zero                      */
/*   256  u8 widths[T] (one per token, shared by all layers, heads,    */
/*        K and V), zero-padded to a 256-byte boundary                 */
/*   payload: 2*L*H streams of S bytes, stream (l, kv, h) at index     */
/*        (2*l + kv)*H + h (kv 0 = K, 1 = V); S = round_up(sum of      */
/*        record sizes, 256); token t's record at sum_{s<t} R(w_s).    */
/*                                                                     */
/* Record for width b in {2,4,8}: f16 scale[G], bf16 min[G], then the  */
/* codes of coordinates 0..d-1, b bits each, least significant bit     */
/* first, group after group (G = d/32); padded to 16 bytes.            */
/* Record for width 16: the d bf16 inputs unchanged.                   */
/* ------------------------------------------------------------------ */

#define CARD_HEADER 256u
#define CARD_MAGIC 0x43564B51u /* bytes 'Q','K','V','C' */
#define CARD_GROUP 32u

uint32_t or_card_record_bytes(uint32_t d, uint32_t b) {
    if (b == 16) return 2 * d;
    if (b != 2 && b != 4 && b != 8) return 0;
    uint32_t g = d / CARD_GROUP;
    return (uint32_t)round_up(4u * g + d * b / 8u, 16);
}

static int card_shape_ok(uint32_t L, uint32_t H, uint32_t T, uint32_t d) {
    return L > 0 && H > 0 && T > 0 && d > 0 && d % CARD_GROUP == 0 && d <= 256;
}

/* off[0..2] = payload offset, stream bytes S, total; also checks widths. */
int or_card_layout(uint32_t L, uint32_t H, uint32_t T, uint32_t d, const uint8_t* widths,
                   uint64_t off[3]) {
    if (!card_shape_ok(L, H, T, d)) return OR_E_ARG;
    uint64_t s = 0;
    for (uint32_t t = 0; t < T; ++t) {
        uint32_t r = or_card_record_bytes(d, widths[t]);
        if (r == 0) return OR_E_FORMAT;
        s += r;
    }
    off[0] = round_up(CARD_HEADER + (uint64_t)T, 256);
    off[1] = round_up(s, 256);
    off[2] = off[0] + 2ull * L * H * off[1];
    return OR_OK;
}

uint64_t or_card_bytes(uint32_t L, uint32_t H, uint32_t T, uint32_t d, const uint8_t* widths) {
    uint64_t off[3];
    if (or_card_layout(L, H, T, d, widths, off)) return 0;
    return off[2];
}

/* One group of 32 bf16 values at width b (QKVShare item 2, min-max):
 *   mn, mx = min, max of the group (both canonicalised: -0 becomes +0)
 *   s      = fp16(min((mx - mn) / (2^b - 1), 65504))   (binary32, then RNE)
 *   q_j    = min(rint((x_j - mn) * (1 / s)), 2^b - 1), q = 0 when s = 0
 * NaN (the pages give no rule; this is the reading both sides implement):
 * a group holding a NaN, quiet or signalling, has the quiet NaN 0x7FC0 for
 * its minimum and maximum (IEEE 754-2019 minimum / maximum propagate it).
 * Its scale is then 65504 (the min above) and each code min(NaN, 2^b - 1)
 * = 2^b - 1 (fminf returns the number), so the group decodes to NaN. */
static void card_quant_group(const uint16_t* x, uint32_t b, uint16_t* s_bits, uint16_t* mn_bits,
                             uint8_t* q) {
    float mn = INFINITY, mx = -INFINITY;
    int has_nan = 0;
    for (uint32_t j = 0; j < CARD_GROUP; ++j) {
        float f = or_bf16_to_f32(x[j]);
        if (isnan(f)) {
            has_nan = 1;
            continue;
        }
        if (f < mn) mn = f;
        if (f > mx) mx = f;
    }
    if (has_nan) mn = mx = or_bf16_to_f32(0x7FC0u);
    mn = mn + 0.0f;
    mx = mx + 0.0f;
    float qmax = (float)((1u << b) - 1u);
    float s = (mx - mn) / qmax;
    uint16_t sb = or_f32_to_f16(fminf(s, 65504.0f));
    float sf = or_f16_to_f32(sb);
    float inv = (sf == 0.0f) ? 0.0f : 1.0f / sf;
    for (uint32_t j = 0; j < CARD_GROUP; ++j) {
        float u = fminf(rintf((or_bf16_to_f32(x[j]) - mn) * inv), qmax);
        q[j] = (uint8_t)u;
    }
    *s_bits = sb;
    uint32_t mu;
    memcpy(&mu, &mn, 4);
    *mn_bits = (uint16_t)(mu >> 16); /* exact: mn is a bf16 value */
}

static void card_pack_record(const uint16_t* x, uint32_t d, uint32_t b, uint8_t* rec) {
    uint32_t R = or_card_record_bytes(d, b);
    memset(rec, 0, R);
    if (b == 16) {
        for (uint32_t i = 0; i < d; ++i) put_u16(rec + 2 * i, x[i]);
        return;
    }
    uint32_t G = d / CARD_GROUP;
    uint8_t* codes = rec + 4 * G;
    for (uint32_t g = 0; g < G; ++g) {
        uint16_t sb, mb;
        uint8_t q[CARD_GROUP];
        card_quant_group(x + g * CARD_GROUP, b, &sb, &mb, q);
        put_u16(rec + 2 * g, sb);
        put_u16(rec + 2 * G + 2 * g, mb);
        for (uint32_t j = 0; j < CARD_GROUP; ++j) {
            uint64_t bitpos = (uint64_t)(g * CARD_GROUP + j) * b;
            for (uint32_t u = 0; u < b; ++u)
                if ((q[j] >> u) & 1u) codes[(bitpos + u) / 8] |= (uint8_t)(1u << ((bitpos + u) % 8));
        }
    }
}

/* One dequantised card value (QKVShare method item 3, the receiver
 * rebuilding full-width values from a group's scale and minimum): q*s + mn
 * computed in binary32 with one rounding (fmaf; q*s alone is exact, at most
 * 8 + 11 significant bits), then stored as bf16, round to nearest even. */
uint16_t or_card_dequant(uint32_t q, uint16_t scale_f16, uint16_t min_bf16) {
    float r = fmaf((float)q, or_f16_to_f32(scale_f16), or_bf16_to_f32(min_bf16));
    return or_f64_to_bf16((double)r);
}

/* One record back to d bf16 values: width 16 copies the stored bf16, other
 * widths read each code LSB-first and dequantise it with its group's scale
 * and minimum. */
static void card_unpack_record(const uint8_t* rec, uint32_t d, uint32_t b, uint16_t* out) {
    if (b == 16) {
        for (uint32_t i = 0; i < d; ++i) out[i] = get_u16(rec + 2 * i);
        return;
    }
    uint32_t G = d / CARD_GROUP;
    const uint8_t* codes = rec + 4 * G;
    for (uint32_t g = 0; g < G; ++g) {
        uint16_t s = get_u16(rec + 2 * g);
        uint16_t mn = get_u16(rec + 2 * G + 2 * g);
        for (uint32_t j = 0; j < CARD_GROUP; ++j) {
            uint64_t bitpos = (uint64_t)(g * CARD_GROUP + j) * b;
            uint32_t q = 0;
            for (uint32_t u = 0; u < b; ++u)
                q |= (uint32_t)((codes[(bitpos + u) / 8] >> ((bitpos + u) % 8)) & 1u) << u;
            out[g * CARD_GROUP + j] = or_card_dequant(q, s, mn);
        }
    }
}

int or_card_pack(uint32_t L, uint32_t H, uint32_t T, uint32_t d, const uint16_t* k,
                 const uint16_t* v, const uint8_t* widths, const char* model_id,
                 int64_t position_offset, uint8_t* card) {
    uint64_t off[3];
    int rc = or_card_layout(L, H, T, d, widths, off);
    if (rc) return rc;
    memset(card, 0, off[2]);
    put_u32(card + 0, CARD_MAGIC);
    put_u16(card + 4, 1);
    put_u16(card + 6, 2);
    put_u32(card + 8, L);
    put_u32(card + 12, H);
    put_u32(card + 16, T);
    put_u32(card + 20, d);
    put_u32(card + 24, CARD_GROUP);
    put_u64(card + 32, (uint64_t)position_offset);
    put_u64(card + 40, CARD_HEADER);
    put_u64(card + 48, off[0]);
    put_u64(card + 56, off[1]);
    put_u64(card + 64, off[2]);
    if (model_id) {
        size_t n = strlen(model_id);
        if (n > 63) n = 63;
        memcpy(card + 72, model_id, n);
    }
    memcpy(card + CARD_HEADER, widths, T);

    uint64_t* rec_off = (uint64_t*)malloc(sizeof(uint64_t) * T);
    if (!rec_off) return OR_E_ARG;
    uint64_t acc = 0;
    for (uint32_t t = 0; t < T; ++t) {
        rec_off[t] = acc;
        acc += or_card_record_bytes(d, widths[t]);
    }
    int64_t nstreams = 2ll * L * H;
    #pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < nstreams; ++s) {
        uint32_t h = (uint32_t)(s % H);
        uint32_t kv = (uint32_t)((s / H) % 2);
        uint32_t l = (uint32_t)(s / (2ll * H));
        const uint16_t* src = (kv == 0 ? k : v) + ((uint64_t)l * H + h) * T * d;
        uint8_t* base = card + off[0] + (uint64_t)s * off[1];
        for (uint32_t t = 0; t < T; ++t)
            card_pack_record(src + (uint64_t)t * d, d, widths[t], base + rec_off[t]);
    }
    free(rec_off);
    return OR_OK;
}

int or_card_unpack(uint32_t L, uint32_t H, uint32_t T, uint32_t d, const uint8_t* card,
                   uint64_t card_bytes, uint16_t* k_out, uint16_t* v_out) {
    if (card_bytes < CARD_HEADER) return OR_E_FORMAT;
    if (get_u32(card) != CARD_MAGIC || get_u16(card + 4) != 1 || get_u16(card + 6) != 2)
        return OR_E_FORMAT;
    if (get_u32(card + 8) != L || get_u32(card + 12) != H || get_u32(card + 16) != T ||
        get_u32(card + 20) != d || get_u32(card + 24) != CARD_GROUP)
        return OR_E_FORMAT;
    if (card_bytes < CARD_HEADER + (uint64_t)T) return OR_E_FORMAT;
    const uint8_t* widths = card + CARD_HEADER;
    uint64_t off[3];
    if (or_card_layout(L, H, T, d, widths, off)) return OR_E_FORMAT;
    if (card_bytes < off[2] || get_u64(card + 48) != off[0] || get_u64(card + 56) != off[1] ||
        get_u64(card + 64) != off[2])
        return OR_E_FORMAT;
    uint64_t* rec_off = (uint64_t*)malloc(sizeof(uint64_t) * T);
    if (!rec_off) return OR_E_ARG;
    uint64_t acc = 0;
    for (uint32_t t = 0; t < T; ++t) {
        rec_off[t] = acc;
        acc += or_card_record_bytes(d, widths[t]);
    }
    int64_t nstreams = 2ll * L * H;
    #pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < nstreams; ++s) {
        uint32_t h = (uint32_t)(s % H);
        uint32_t kv = (uint32_t)((s / H) % 2);
        uint32_t l = (uint32_t)(s / (2ll * H));
        uint16_t* dst = (kv == 0 ? k_out : v_out) + ((uint64_t)l * H + h) * T * d;
        const uint8_t* base = card + off[0] + (uint64_t)s * off[1];
        for (uint32_t t = 0; t < T; ++t)
            card_unpack_record(base + rec_off[t], d, widths[t], dst + (uint64_t)t * d);
    }
    free(rec_off);
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* Key position re-alignment (KVCMAS procedure: a shared segment's key  */
/* positions are re-aligned to the target's before reuse; the card      */
/* carries the source position offset, QKVShare item 2). Rotary keys at */
/* position p hold each channel pair rotated by p * f_j; moving them by */
/* delta positions rotates pair j by delta * f_j more. Pairs are        */
/* (j, j + d/2) (pairing 0, halves) or (2j, 2j + 1) (pairing 1,         */
/* adjacent); f_j are the model's inverse frequencies (an input).       */
/* Computed in binary64, rounded once to bf16.                          */
/* ------------------------------------------------------------------ */
int or_realign_keys(uint32_t L, uint32_t H, uint32_t T, uint32_t d, const uint16_t* k_in, uint16_t* k_out,
                    int64_t delta, const float* inv_freq, uint32_t pairing) {
    if (d == 0 || d % 2 || pairing > 1) return OR_E_ARG;
    uint32_t half = d / 2;
    double* c = (double*)malloc(sizeof(double) * half);
    double* s = (double*)malloc(sizeof(double) * half);
    if (!c || !s) {
        free(c);
        free(s);
        return OR_E_ARG;
    }
    for (uint32_t j = 0; j < half; ++j) {
        double phi = (double)delta * (double)inv_freq[j];
        c[j] = cos(phi);
        s[j] = sin(phi);
    }
    int64_t vecs = (int64_t)L * H * T;
    #pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < vecs; ++v) {
        const uint16_t* x = k_in + (uint64_t)v * d;
        uint16_t* y = k_out + (uint64_t)v * d;
        uint16_t tmp[256];
        for (uint32_t j = 0; j < half; ++j) {
            uint32_t ia = pairing == 0 ? j : 2 * j, ib = pairing == 0 ? j + half : 2 * j + 1;
            double a = (double)or_bf16_to_f32(x[ia]), b = (double)or_bf16_to_f32(x[ib]);
            tmp[ia] = or_f64_to_bf16(a * c[j] - b * s[j]);
            tmp[ib] = or_f64_to_bf16(a * s[j] + b * c[j]);
        }
        memcpy(y, tmp, sizeof(uint16_t) * d);
    }
    free(c);
    free(s);
    return OR_OK;
}
