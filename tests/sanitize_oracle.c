/* Drives the C oracle under AddressSanitizer and UndefinedBehaviorSanitizer:
 * pack, offset check, unpack and GEMM on random small matrices, then with
 * corrupted width codes and tile offsets, which the oracle must reject with a
 * status before it reads the payload out of bounds. Built and run by
 * tests/test_sanitizers.py; exit status 0 when every check holds. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_pack_sizes(uint32_t n, uint32_t k, const uint8_t *bits, uint64_t out[5]);
int oracle_pack(uint32_t n, uint32_t k, const uint8_t *bits, const int8_t *codes, const uint16_t *scales,
                uint8_t *widths_out, uint16_t *scales_out, uint32_t *tile_offsets_out, uint8_t *payload_out,
                uint64_t payload_capacity);
int oracle_check_offsets(uint32_t n, uint32_t k, const uint8_t *widths, const uint32_t *tile_offsets,
                         uint64_t payload_bytes);
int oracle_unpack(uint32_t n, uint32_t k, const uint8_t *widths, const uint32_t *tile_offsets,
                  const uint8_t *payload, uint64_t payload_bytes, int8_t *codes_out);
int oracle_gemm(uint32_t n, uint32_t k, const uint8_t *widths, const uint16_t *scales, const uint32_t *tile_offsets,
                const uint8_t *payload, uint64_t payload_bytes, const uint16_t *x, uint32_t m, double *y,
                uint32_t row_begin, uint32_t row_end);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint64_t next(void)   /* splitmix64 */
{
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static int g_fail = 0;

static void check(int ok, const char *what, int it)
{
    if (!ok) {
        ++g_fail;
        fprintf(stderr, "iteration %d: %s\n", it, what);
    }
}

int main(int argc, char **argv)
{
    int iters = argc > 1 ? atoi(argv[1]) : 60;
    for (int it = 0; it < iters; ++it) {
        uint32_t n = 1 + (uint32_t)(next() % 120), G = 1 + (uint32_t)(next() % 10), k = 64 * G;
        uint64_t groups = (uint64_t)n * G, sz[5];
        uint8_t *bits = malloc(groups);
        int8_t *codes = malloc((size_t)n * k);
        uint16_t *scales = malloc(2 * groups);
        for (uint64_t t = 0; t < groups; ++t) {
            static const uint8_t w[4] = {1, 2, 4, 8};
            int b = w[next() % 4];
            bits[t] = (uint8_t)b;
            scales[t] = (uint16_t)(next() % 0x7C00);
            for (int i = 0; i < 64; ++i) {
                int lim = (1 << (b - 1)) - 1;
                codes[t * 64 + i] = (int8_t)(b == 1 ? ((next() & 1) ? 1 : -1) : (int)(next() % (2 * lim + 1)) - lim);
            }
        }
        check(oracle_pack_sizes(n, k, bits, sz) == 0, "pack sizes", it);
        uint8_t *widths = calloc(sz[0] + 1, 1), *payload = calloc(sz[3] + 1, 1);
        uint16_t *sc = calloc(sz[1] / 2 + 1, 2);
        uint32_t *offs = calloc(sz[2] / 4, 4);
        check(oracle_pack(n, k, bits, codes, scales, widths, sc, offs, payload, sz[3]) == 0, "pack", it);
        check(oracle_check_offsets(n, k, widths, offs, sz[3]) == 0, "offsets of a packed matrix", it);
        int8_t *out = malloc((size_t)n * k);
        check(oracle_unpack(n, k, widths, offs, payload, sz[3], out) == 0 && memcmp(out, codes, (size_t)n * k) == 0,
              "unpack round trip", it);
        uint32_t m = 1 + (uint32_t)(next() % 3);
        uint16_t *x = malloc(2 * (size_t)m * k);
        for (uint64_t i = 0; i < (uint64_t)m * k; ++i) x[i] = (uint16_t)(next() % 0x7C00) | (uint16_t)((next() & 1) << 15);
        double *y = malloc(sizeof(double) * m * n);
        check(oracle_gemm(n, k, widths, sc, offs, payload, sz[3], x, m, y, 0, n) == 0, "gemm", it);
        /* damage: a width code or a tile offset; the oracle must say so and stay in bounds */
        for (int t = 0; t < 8; ++t) {
            uint8_t *w2 = malloc(sz[0] + 1);
            uint32_t *o2 = malloc(sz[2]);
            memcpy(w2, widths, sz[0] + 1);
            memcpy(o2, offs, sz[2]);
            if (t & 1)
                w2[next() % sz[0]] ^= (uint8_t)(1u << (next() % 8));
            else
                o2[next() % (sz[2] / 4)] += 1 + (uint32_t)(next() % 100000);
            int st = oracle_check_offsets(n, k, w2, o2, sz[3]);
            int su = oracle_unpack(n, k, w2, o2, payload, sz[3], out);
            int sg = oracle_gemm(n, k, w2, sc, o2, payload, sz[3], x, m, y, 0, n);
            check((st != 0) == (su != 0) && (su != 0) == (sg != 0), "check, unpack and gemm disagree", it);
            free(w2);
            free(o2);
        }
        free(bits); free(codes); free(scales); free(widths); free(payload); free(sc); free(offs); free(out);
        free(x); free(y);
    }
    printf("oracle sanitizer run: %d failures\n", g_fail);
    return g_fail ? 1 : 0;
}
