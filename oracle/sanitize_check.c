/* sanitize_check.c - runs every entry point of the CPU oracle on small
 * shapes (ragged token counts, both head sizes, every card width, corrupted
 * headers) so that it can be built and run under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitizers.py). Test
 * infrastructure, like the rest of oracle/.
 *
 * The level table is passed on the command line as 15 hexadecimal floats
 * (8 levels, then 7 thresholds), as the Python side derives it. Exit status
 * 0 means every call returned what it must and every check held. */
#include "kvoracle.c"

#include <stdio.h>

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static uint64_t next_u64(void) {
    /* xorshift64* */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 0x2545F4914F6CDD1Dull;
}

/* a value in (-4, 4) with a random binary exponent offset, as bf16 bits;
 * every 37th value is an exact zero of either sign */
static uint16_t rand_bf16(void) {
    uint64_t r = next_u64();
    if (r % 37 == 0) return (r & 64) ? 0x8000 : 0;
    double u = ((double)(r >> 11) / 9007199254740992.0) * 8.0 - 4.0;
    int e = (int)((r >> 3) % 9) - 4;
    return or_f64_to_bf16(ldexp(u, e));
}

static int failures = 0;
#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                 \
        }                                                               \
    } while (0)

static void run_shape(uint32_t L, uint32_t H, uint32_t T, uint32_t d, const float levels[8],
                      const float thr[7]) {
    uint64_t n = (uint64_t)L * H * T * d;
    uint16_t* k = malloc(2 * n);
    uint16_t* v = malloc(2 * n);
    uint16_t* ko = malloc(2 * n);
    uint16_t* vo = malloc(2 * n);
    for (uint64_t i = 0; i < n; ++i) {
        k[i] = rand_bf16();
        v[i] = rand_bf16();
    }
    /* pool */
    uint64_t pb = or_pool_bytes(L, H, T, d);
    uint8_t* pool = malloc(pb);
    CHECK(or_pool_encode(L, H, T, d, k, v, thr, pool) == OR_OK);
    CHECK(or_pool_decode(L, H, T, d, pool, pb, 0, L, levels, ko, vo) == OR_OK);
    CHECK(or_pool_decode(L, H, T, d, pool, pb, L - 1, L, levels, ko, vo) == OR_OK);
    CHECK(or_pool_decode(L, H, T, d, pool, pb, 0, L + 1, levels, ko, vo) == OR_E_ARG);
    CHECK(or_pool_decode(L, H, T, d, pool, pb - 1, 0, L, levels, ko, vo) == OR_E_FORMAT);
    uint8_t* codes = malloc(n);
    CHECK(or_pool_v_codes(L, H, T, d, pool, pb, codes) == OR_OK);
    for (uint64_t i = 0; i < n; ++i) CHECK(codes[i] < 8);
    pool[9] ^= 1; /* layer count */
    CHECK(or_pool_decode(L, H, T, d, pool, pb, 0, L, levels, ko, vo) == OR_E_FORMAT);
    free(codes);
    free(pool);

    /* card: every width, then random widths */
    uint8_t* widths = malloc(T);
    const uint8_t ws[4] = {2, 4, 8, 16};
    for (int pass = 0; pass < 5; ++pass) {
        for (uint32_t t = 0; t < T; ++t) widths[t] = pass < 4 ? ws[pass] : ws[next_u64() % 4];
        uint64_t cb = or_card_bytes(L, H, T, d, widths);
        CHECK(cb > 0);
        uint8_t* card = malloc(cb);
        CHECK(or_card_pack(L, H, T, d, k, v, widths, "sanitize", -7, card) == OR_OK);
        CHECK(or_card_unpack(L, H, T, d, card, cb, ko, vo) == OR_OK);
        for (uint64_t i = 0; i < n; ++i) {
            uint64_t t = (i / d) % T;
            if (widths[t] == 16) CHECK(ko[i] == k[i] && vo[i] == v[i]);
        }
        CHECK(or_card_unpack(L, H, T, d, card, cb - 1, ko, vo) == OR_E_FORMAT);
        card[CARD_HEADER] = 5; /* an invalid width */
        CHECK(or_card_unpack(L, H, T, d, card, cb, ko, vo) != OR_OK);
        card[0] ^= 0xFF;
        CHECK(or_card_unpack(L, H, T, d, card, cb, ko, vo) == OR_E_FORMAT);
        free(card);
    }
    widths[T - 1] = 3;
    CHECK(or_card_bytes(L, H, T, d, widths) == 0);
    free(widths);

    /* key re-alignment, both pairings, and in place */
    float inv_freq[64];
    for (uint32_t j = 0; j < d / 2; ++j) inv_freq[j] = (float)pow(500000.0, -2.0 * j / d);
    CHECK(or_realign_keys(L, H, T, d, k, ko, 4096, inv_freq, 0) == OR_OK);
    CHECK(or_realign_keys(L, H, T, d, k, ko, -3, inv_freq, 1) == OR_OK);
    CHECK(or_realign_keys(L, H, T, d, ko, ko, 17, inv_freq, 0) == OR_OK);
    CHECK(or_realign_keys(L, H, T, d, k, ko, 1, inv_freq, 2) == OR_E_ARG);

    free(k);
    free(v);
    free(ko);
    free(vo);
}

int main(int argc, char** argv) {
    if (argc != 16) {
        fprintf(stderr, "usage: %s 8 levels then 7 thresholds (hex floats)\n", argv[0]);
        return 2;
    }
    float levels[8], thr[7];
    for (int i = 0; i < 8; ++i) levels[i] = strtof(argv[1 + i], NULL);
    for (int i = 0; i < 7; ++i) thr[i] = strtof(argv[9 + i], NULL);

    /* scalar conversions at their edges */
    const double edge[] = {0.0, -0.0, 1e-45, -1e-40, 65504.0, 65520.0, 1e38, 3.5e38, -3.5e38, INFINITY, NAN};
    for (unsigned i = 0; i < sizeof(edge) / sizeof(edge[0]); ++i) {
        (void)or_f64_to_bf16(edge[i]);
        (void)or_f32_to_f16((float)edge[i]);
    }
    for (uint32_t h = 0; h < 65536; h += 7) {
        (void)or_f16_to_f32((uint16_t)h);
        (void)or_bf16_to_f32((uint16_t)h);
    }
    for (uint32_t q = 0; q < 256; ++q) (void)or_card_dequant(q, 0x3C00, 0xBF80);

    const uint32_t shapes[][4] = {{1, 1, 1, 64}, {2, 3, 37, 128}, {1, 2, 5, 64}, {3, 1, 17, 128}, {1, 4, 64, 64}};
    for (unsigned s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s)
        run_shape(shapes[s][0], shapes[s][1], shapes[s][2], shapes[s][3], levels, thr);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer run ok\n");
    return 0;
}
