/*
 * VBQ packed-weight CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it. It shares no code, header, table or helper with the
 * HIP library: it has its own binary16 decoder, its own field reader and its
 * own packer, all written from the definitions below.
 *
 * Method: "Variable Bit-width Quantization: Learning Per-Group Precision for
 * 'Bigger-but-Smaller' Language Models" (arXiv 2607.02893).
 *   - §3.1, Eq. (1): a weight matrix is cut into contiguous groups of
 *     G = 64 weights; each group g has its own bit width b_g and scale s_g,
 *     and the dequantised weight is w_hat = s_g * q with an integer code q
 *     on the symmetric grid |q| <= 2^(b-1) - 1; the 1-bit case is
 *     sign * scale, q in {-1, +1}.
 *   - §6 ("Fused kernels over packed weights", "Granularity is
 *     deployment-friendly"): widths are drawn from {1, 2, 4, 8}, groups
 *     pack into whole bytes, and decode computes y = W x from the packed
 *     groups without forming the dense matrix.
 *
 * Packed layout (the pages fix only the items above; every other choice is
 * a stated reading, listed with the design notes):
 *   W is N x K row-major, K % 64 == 0, G = K / 64; group (n, j) covers
 *   W[n][64j .. 64j+63].
 *   Tiles                 the groups are cut into tiles of 64 rows x 4
 *                         groups (edge tiles are smaller); tile (a, c)
 *                         holds rows [64a, 64a+64) and groups [4c, 4c+4);
 *                         tiles are numbered a * ceil(G/4) + c.
 *   metadata index        group (n, j) in tile (a, c) = (n/64, j/4), with
 *                         R = rows of row tile a and C = groups of tile
 *                         (a, c), has index t = 64*a*G + R*4*c
 *                         + (n - 64a)*C + (j - 4c): tiles in order, each
 *                         tile row-major.
 *   widths[ceil(N*G/4)]   width code c_t = (widths[t/4] >> 2*(t%4)) & 3,
 *                         b_t = 1 << c_t.
 *   scales[N*G]           IEEE binary16 bit pattern of s_t.
 *   tile_offsets[T+1]     exclusive prefix sum of the tiles' payload sizes
 *                         (each the sum of 8*b over the tile's groups).
 *   payload               tile by tile; inside a tile, bucketed by width
 *                         (1, 2, 4, then 8 bits); inside a bucket, groups in
 *                         column-major order (group index j ascending, then
 *                         row ascending). Each group holds 8*b bytes, so its
 *                         offset is the exclusive prefix sum of 8*b over the
 *                         groups stored before it.
 *   inside a group        element i (weight W[n][64j+i]) is a b-bit field:
 *                         b = 1: bit i (byte i/8, bit i%8);
 *                         b = 8: byte i;
 *                         b = 2: in little-endian 32-bit word i/16, field
 *                                m = e/2 + 8*(e%2) with e = i%16, bits 2m..2m+1;
 *                         b = 4: in little-endian 32-bit word i/8, field
 *                                m = e/2 + 4*(e%2) with e = i%8, bits 4m..4m+3.
 *   field f -> code q     b == 1: f is a sign bit, q = +1 (f = 0) or -1
 *                         (f = 1). b >= 2: two's complement; the pattern
 *                         -2^(b-1) lies outside the grid and is rejected by
 *                         the packer (a decoder still reads it as -2^(b-1)).
 *
 * Results: y[m][n] = sum_j s_{n,j} * sum_i q_{n,j,i} * x[m][64 j + i],
 * accumulated in double precision in that order. Every fp16 value and every
 * product q*x is exact in double, so the only rounding is the summation.
 */
#include <stddef.h>
#include <stdint.h>
#include <math.h>
#include <stdlib.h>

enum {
    OR_OK = 0,
    OR_ERR_NULL = 1,
    OR_ERR_SHAPE = 2,
    OR_ERR_WIDTH = 3,
    OR_ERR_CODE = 4,
    OR_ERR_SCALE = 5,
    OR_ERR_CAPACITY = 6,
    OR_ERR_OFFSETS = 7
};

/* IEEE 754 binary16 -> double: sign, 5-bit exponent (bias 15), 10-bit
 * fraction; exponent 0 is zero / subnormal, exponent 31 is inf / NaN. */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 31;
    int frac = h & 1023;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25);
    return sign ? -v : v;
}

#define TILE_ROWS 64u
#define TILE_GROUPS 4u

static uint64_t tile_count(uint32_t n, uint32_t G)
{
    return (uint64_t)((n + TILE_ROWS - 1) / TILE_ROWS) * ((G + TILE_GROUPS - 1) / TILE_GROUPS);
}

/* Metadata index of group (r, j): tiles in order, each tile row-major. */
static uint64_t meta_index(uint32_t n, uint32_t G, uint32_t r, uint32_t j)
{
    uint32_t a = r / TILE_ROWS, c = j / TILE_GROUPS;
    uint32_t rows = n - a * TILE_ROWS < TILE_ROWS ? n - a * TILE_ROWS : TILE_ROWS;
    uint32_t cols = G - c * TILE_GROUPS < TILE_GROUPS ? G - c * TILE_GROUPS : TILE_GROUPS;
    return (uint64_t)TILE_ROWS * a * G + (uint64_t)rows * TILE_GROUPS * c +
           (uint64_t)(r - a * TILE_ROWS) * cols + (j - c * TILE_GROUPS);
}

/* Bit position of element i inside a b-bit group's byte string. */
static unsigned field_bit(int b, int i)
{
    if (b == 2) {
        int e = i % 16, m = e / 2 + 8 * (e % 2);
        return 32u * (unsigned)(i / 16) + 2u * (unsigned)m;
    }
    if (b == 4) {
        int e = i % 8, m = e / 2 + 4 * (e % 2);
        return 32u * (unsigned)(i / 8) + 4u * (unsigned)m;
    }
    return (unsigned)(b * i); /* b = 1: bit i; b = 8: byte i */
}

/* Walk the storage order: off[t] receives the payload byte offset of group
 * t = n*G + j, tile_offsets (T+1 entries, optional) the tile starts.
 * bits[t] is the width of group t. Returns the payload size. */
static uint64_t locate_groups(uint32_t n, uint32_t G, const uint8_t *bits, uint64_t *off,
                              uint32_t *tile_offsets)
{
    uint64_t pos = 0, tile = 0;
    for (uint32_t r0 = 0; r0 < n; r0 += TILE_ROWS) {
        uint32_t r1 = r0 + TILE_ROWS < n ? r0 + TILE_ROWS : n;
        for (uint32_t j0 = 0; j0 < G; j0 += TILE_GROUPS) {
            uint32_t j1 = j0 + TILE_GROUPS < G ? j0 + TILE_GROUPS : G;
            if (tile_offsets)
                tile_offsets[tile] = (uint32_t)pos;
            for (int b = 1; b <= 8; b *= 2)
                for (uint32_t j = j0; j < j1; ++j)
                    for (uint32_t r = r0; r < r1; ++r) {
                        uint64_t t = (uint64_t)r * G + j;
                        if (bits[t] == b) {
                            if (off)
                                off[t] = pos;
                            pos += 8u * b;
                        }
                    }
            ++tile;
        }
    }
    if (tile_offsets)
        tile_offsets[tile] = (uint32_t)pos;
    return pos;
}

/* width code stored at metadata index t */
static int group_width(const uint8_t *widths, uint64_t t)
{
    int c = (widths[t / 4] >> (2 * (t % 4))) & 3;
    return 1 << c;
}

/* widths the format allows (§6: {1, 2, 4, 8}) */
static int width_is_valid(int b)
{
    return b == 1 || b == 2 || b == 4 || b == 8;
}

static int code_is_on_grid(int b, int q)
{
    if (b == 1)
        return q == 1 || q == -1;
    int lim = (1 << (b - 1)) - 1;
    return q >= -lim && q <= lim;
}

/* Sizes in bytes of the four packed arrays; out = {widths, scales,
 * tile_offsets, payload, total}. bits[n*G + j] is the width of group (n, j)
 * (packer inputs are in natural row-major group order). */
int oracle_pack_sizes(uint32_t n, uint32_t k, const uint8_t *bits, uint64_t out[5])
{
    if (!out || (!bits && (uint64_t)n * k != 0))
        return OR_ERR_NULL;
    if (k % 64)
        return OR_ERR_SHAPE;
    uint64_t groups = (uint64_t)n * (k / 64);
    uint64_t payload = 0;
    for (uint64_t t = 0; t < groups; ++t) {
        if (!width_is_valid(bits[t]))
            return OR_ERR_WIDTH;
        payload += 8u * bits[t];
    }
    out[0] = (groups + 3) / 4;
    out[1] = 2 * groups;
    out[2] = 4 * (tile_count(n, k / 64) + 1);
    out[3] = payload;
    out[4] = out[0] + out[1] + out[2] + out[3];
    return OR_OK;
}

/* Independent packer. codes is int8 [n][k], scales binary16 [n][G]. */
int oracle_pack(uint32_t n, uint32_t k, const uint8_t *bits, const int8_t *codes,
                const uint16_t *scales, uint8_t *widths_out, uint16_t *scales_out,
                uint32_t *tile_offsets_out, uint8_t *payload_out, uint64_t payload_capacity)
{
    uint64_t sz[5];
    int st = oracle_pack_sizes(n, k, bits, sz);
    if (st)
        return st;
    if (!tile_offsets_out || ((uint64_t)n * k != 0 && (!codes || !scales || !widths_out || !scales_out)))
        return OR_ERR_NULL;
    if (sz[3] && !payload_out)
        return OR_ERR_NULL;
    if (sz[3] > payload_capacity)
        return OR_ERR_CAPACITY;
    if (sz[3] > 0xFFFFFFFFull)
        return OR_ERR_SHAPE;
    uint32_t G = k / 64;
    uint64_t groups = (uint64_t)n * G;
    /* check everything before writing anything */
    for (uint64_t t = 0; t < groups; ++t) {
        uint16_t h = scales[t];
        if (((h >> 10) & 31) == 31)
            return OR_ERR_SCALE;
        int b = bits[t];
        for (int i = 0; i < 64; ++i)
            if (!code_is_on_grid(b, codes[t * 64 + i]))
                return OR_ERR_CODE;
    }
    uint64_t *off = malloc((groups ? groups : 1) * sizeof *off);
    if (!off)
        return OR_ERR_CAPACITY;
    locate_groups(n, G, bits, off, tile_offsets_out);
    for (uint64_t i = 0; i < sz[0]; ++i)
        widths_out[i] = 0;
    for (uint64_t i = 0; i < sz[3]; ++i)
        payload_out[i] = 0;
    for (uint64_t t = 0; t < groups; ++t) {
        int b = bits[t];
        int c = b == 1 ? 0 : b == 2 ? 1 : b == 4 ? 2 : 3;
        uint64_t m = meta_index(n, G, (uint32_t)(t / G), (uint32_t)(t % G));
        widths_out[m / 4] |= (uint8_t)(c << (2 * (m % 4)));
        scales_out[m] = scales[t];
        for (int i = 0; i < 64; ++i) {
            int q = codes[t * 64 + i];
            unsigned f;
            if (b == 1)
                f = q < 0 ? 1u : 0u;
            else
                f = (unsigned)q & ((1u << b) - 1u);
            unsigned bit = field_bit(b, i);
            payload_out[off[t] + bit / 8] |= (uint8_t)(f << (bit % 8));
        }
    }
    free(off);
    return OR_OK;
}

/* Width of group (r, j) from the packed codes. */
static int width_of(const uint8_t *widths, uint32_t n, uint32_t G, uint32_t r, uint32_t j)
{
    return group_width(widths, meta_index(n, G, r, j));
}

/* Expand the packed width codes into one width per group, natural order
 * n*G + j (caller frees). */
static uint8_t *expand_widths(const uint8_t *widths, uint32_t n, uint32_t G)
{
    uint64_t groups = (uint64_t)n * G;
    uint8_t *bits = malloc(groups ? groups : 1);
    if (!bits)
        return NULL;
    for (uint32_t r = 0; r < n; ++r)
        for (uint32_t j = 0; j < G; ++j)
            bits[(uint64_t)r * G + j] = (uint8_t)width_of(widths, n, G, r, j);
    return bits;
}

/* tile_offsets must be the exclusive prefix sum of the tile payload sizes
 * and end at payload_bytes. */
int oracle_check_offsets(uint32_t n, uint32_t k, const uint8_t *widths,
                         const uint32_t *tile_offsets, uint64_t payload_bytes)
{
    if (!tile_offsets || (!widths && (uint64_t)n * k != 0))
        return OR_ERR_NULL;
    if (k % 64)
        return OR_ERR_SHAPE;
    uint32_t G = k / 64;
    uint64_t tiles = tile_count(n, G);
    uint8_t *bits = expand_widths(widths, n, G);
    uint32_t *expect = malloc((tiles + 1) * sizeof *expect);
    int st = OR_OK;
    if (!bits || !expect) {
        st = OR_ERR_CAPACITY;
    } else {
        uint64_t total = locate_groups(n, G, bits, NULL, expect);
        for (uint64_t i = 0; i <= tiles; ++i)
            if (tile_offsets[i] != expect[i])
                st = OR_ERR_OFFSETS;
        if (total != payload_bytes)
            st = OR_ERR_OFFSETS;
    }
    free(bits);
    free(expect);
    return st;
}

/* b-bit field of element i of the group whose payload starts at byte p */
static int decode_code(const uint8_t *payload, uint64_t p, int b, int i)
{
    unsigned bit = field_bit(b, i);
    unsigned f = (payload[p + bit / 8] >> (bit % 8)) & ((1u << b) - 1u);
    if (b == 1)
        return f ? -1 : 1;
    if (f >= (1u << (b - 1)))
        return (int)f - (1 << b);
    return (int)f;
}

/* Payload offset of every group (caller frees), after checking the offsets. */
static int group_offsets(uint32_t n, uint32_t k, const uint8_t *widths, const uint32_t *tile_offsets,
                         uint64_t payload_bytes, uint64_t **off_out)
{
    int st = oracle_check_offsets(n, k, widths, tile_offsets, payload_bytes);
    if (st)
        return st;
    uint64_t groups = (uint64_t)n * (k / 64);
    uint8_t *bits = expand_widths(widths, n, k / 64);
    uint64_t *off = malloc((groups ? groups : 1) * sizeof *off);
    if (!bits || !off) {
        free(bits);
        free(off);
        return OR_ERR_CAPACITY;
    }
    locate_groups(n, k / 64, bits, off, NULL);
    free(bits);
    *off_out = off;
    return OR_OK;
}

/* Decoded codes int8 [n][k]. */
int oracle_unpack(uint32_t n, uint32_t k, const uint8_t *widths, const uint32_t *tile_offsets,
                  const uint8_t *payload, uint64_t payload_bytes, int8_t *codes_out)
{
    uint64_t *off = NULL;
    int st = group_offsets(n, k, widths, tile_offsets, payload_bytes, &off);
    if (st)
        return st;
    if ((uint64_t)n * k != 0 && (!payload || !codes_out)) {
        free(off);
        return OR_ERR_NULL;
    }
    uint32_t G = k / 64;
    for (uint32_t r = 0; r < n; ++r)
        for (uint32_t j = 0; j < G; ++j) {
            uint64_t t = (uint64_t)r * G + j;
            int b = width_of(widths, n, G, r, j);
            for (int i = 0; i < 64; ++i)
                codes_out[t * 64 + i] = (int8_t)decode_code(payload, off[t], b, i);
        }
    free(off);
    return OR_OK;
}

/* y[mm][r] for rows r in [row_begin, row_end) and all m inputs.
 * x is binary16 [m][k]; y is double [m][n] (only the selected rows are
 * written). Scalar loops in the order of the definition. */
int oracle_gemm(uint32_t n, uint32_t k, const uint8_t *widths, const uint16_t *scales,
                const uint32_t *tile_offsets, const uint8_t *payload, uint64_t payload_bytes,
                const uint16_t *x, uint32_t m, double *y, uint32_t row_begin, uint32_t row_end)
{
    if (row_begin > row_end || row_end > n)
        return OR_ERR_SHAPE;
    if ((uint64_t)m * n != 0 && !y)
        return OR_ERR_NULL;
    if ((uint64_t)n * k != 0 && (!payload || !scales || (m && !x)))
        return OR_ERR_NULL;
    uint64_t *off = NULL;
    int st = group_offsets(n, k, widths, tile_offsets, payload_bytes, &off);
    if (st)
        return st;
    uint32_t G = k / 64;
    for (uint32_t mm = 0; mm < m; ++mm) {
        const uint16_t *xm = x + (uint64_t)mm * k;
        for (uint32_t r = row_begin; r < row_end; ++r) {
            double acc = 0.0;
            for (uint32_t j = 0; j < G; ++j) {
                uint64_t t = (uint64_t)r * G + j;
                int b = width_of(widths, n, G, r, j);
                double s = oracle_half_to_double(scales[meta_index(n, G, r, j)]);
                double d = 0.0;
                for (int i = 0; i < 64; ++i)
                    d += (double)decode_code(payload, off[t], b, i) *
                         oracle_half_to_double(xm[(uint64_t)j * 64 + i]);
                acc += s * d;
            }
            y[(uint64_t)mm * n + r] = acc;
        }
    }
    free(off);
    return OR_OK;
}

/* batch-1 GEMV: y[r] for r in [row_begin, row_end) */
int oracle_gemv(uint32_t n, uint32_t k, const uint8_t *widths, const uint16_t *scales,
                const uint32_t *tile_offsets, const uint8_t *payload, uint64_t payload_bytes,
                const uint16_t *x, double *y, uint32_t row_begin, uint32_t row_end)
{
    return oracle_gemm(n, k, widths, scales, tile_offsets, payload, payload_bytes, x, 1, y,
                       row_begin, row_end);
}
