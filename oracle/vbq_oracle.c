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
 *   W is N x K row-major, K % 64 == 0, G = K / 64, flat group t = n*G + j.
 *   widths[ceil(N*G/4)]   width code c_t = (widths[t/4] >> 2*(t%4)) & 3,
 *                         b_t = 1 << c_t.
 *   scales[N*G]           IEEE binary16 bit pattern of s_t.
 *   row_offsets[N+1]      exclusive prefix sum of the group payload sizes
 *                         8*b_t, sampled at row starts.
 *   payload               group (n, j) starts at row_offsets[n] +
 *                         sum_{j'<j} 8*b_{n,j'} and holds 8*b bytes;
 *                         element i is the b-bit field at bit b*i of that
 *                         byte string, little-endian (byte b*i/8, bit
 *                         b*i%8).
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

/* width code of flat group t */
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
 * row_offsets, payload, total}. bits[n*G + j] is the width of group (n, j). */
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
    out[2] = 4 * ((uint64_t)n + 1);
    out[3] = payload;
    out[4] = out[0] + out[1] + out[2] + out[3];
    return OR_OK;
}

/* Independent packer. codes is int8 [n][k], scales binary16 [n][G]. */
int oracle_pack(uint32_t n, uint32_t k, const uint8_t *bits, const int8_t *codes,
                const uint16_t *scales, uint8_t *widths_out, uint16_t *scales_out,
                uint32_t *row_offsets_out, uint8_t *payload_out, uint64_t payload_capacity)
{
    uint64_t sz[5];
    int st = oracle_pack_sizes(n, k, bits, sz);
    if (st)
        return st;
    if (!row_offsets_out || ((uint64_t)n * k != 0 && (!codes || !scales || !widths_out || !scales_out)))
        return OR_ERR_NULL;
    if (sz[3] && !payload_out)
        return OR_ERR_NULL;
    if (sz[3] > payload_capacity)
        return OR_ERR_CAPACITY;
    if (sz[3] > 0xFFFFFFFFull)
        return OR_ERR_SHAPE;
    uint32_t G = k / 64;
    /* check everything before writing anything */
    for (uint64_t t = 0; t < (uint64_t)n * G; ++t) {
        uint16_t h = scales[t];
        if (((h >> 10) & 31) == 31)
            return OR_ERR_SCALE;
        int b = bits[t];
        for (int i = 0; i < 64; ++i)
            if (!code_is_on_grid(b, codes[t * 64 + i]))
                return OR_ERR_CODE;
    }
    for (uint64_t i = 0; i < sz[0]; ++i)
        widths_out[i] = 0;
    for (uint64_t i = 0; i < sz[3]; ++i)
        payload_out[i] = 0;
    uint64_t pos = 0;
    row_offsets_out[0] = 0;
    for (uint32_t r = 0; r < n; ++r) {
        for (uint32_t j = 0; j < G; ++j) {
            uint64_t t = (uint64_t)r * G + j;
            int b = bits[t];
            int c = b == 1 ? 0 : b == 2 ? 1 : b == 4 ? 2 : 3;
            widths_out[t / 4] |= (uint8_t)(c << (2 * (t % 4)));
            scales_out[t] = scales[t];
            for (int i = 0; i < 64; ++i) {
                int q = codes[t * 64 + i];
                unsigned f;
                if (b == 1)
                    f = q < 0 ? 1u : 0u;
                else
                    f = (unsigned)q & ((1u << b) - 1u);
                unsigned bitpos = (unsigned)(b * i);
                payload_out[pos + bitpos / 8] |= (uint8_t)(f << (bitpos % 8));
            }
            pos += 8u * b;
        }
        row_offsets_out[r + 1] = (uint32_t)pos;
    }
    return OR_OK;
}

/* row_offsets must be the exclusive prefix sum of 8*b at row starts and end
 * at payload_bytes. */
int oracle_check_offsets(uint32_t n, uint32_t k, const uint8_t *widths,
                         const uint32_t *row_offsets, uint64_t payload_bytes)
{
    if (!row_offsets || (!widths && (uint64_t)n * k != 0))
        return OR_ERR_NULL;
    if (k % 64)
        return OR_ERR_SHAPE;
    uint32_t G = k / 64;
    uint64_t pos = 0;
    if (row_offsets[0] != 0)
        return OR_ERR_OFFSETS;
    for (uint32_t r = 0; r < n; ++r) {
        for (uint32_t j = 0; j < G; ++j)
            pos += 8u * group_width(widths, (uint64_t)r * G + j);
        if (row_offsets[r + 1] != pos)
            return OR_ERR_OFFSETS;
    }
    return pos == payload_bytes ? OR_OK : OR_ERR_OFFSETS;
}

/* b-bit field i of the group whose payload starts at byte p */
static int decode_code(const uint8_t *payload, uint64_t p, int b, int i)
{
    unsigned bitpos = (unsigned)(b * i);
    unsigned f = (payload[p + bitpos / 8] >> (bitpos % 8)) & ((1u << b) - 1u);
    if (b == 1)
        return f ? -1 : 1;
    if (f >= (1u << (b - 1)))
        return (int)f - (1 << b);
    return (int)f;
}

/* Decoded codes int8 [n][k]. */
int oracle_unpack(uint32_t n, uint32_t k, const uint8_t *widths, const uint32_t *row_offsets,
                  const uint8_t *payload, uint64_t payload_bytes, int8_t *codes_out)
{
    int st = oracle_check_offsets(n, k, widths, row_offsets, payload_bytes);
    if (st)
        return st;
    if ((uint64_t)n * k != 0 && (!payload || !codes_out))
        return OR_ERR_NULL;
    uint32_t G = k / 64;
    for (uint32_t r = 0; r < n; ++r) {
        uint64_t p = row_offsets[r];
        for (uint32_t j = 0; j < G; ++j) {
            uint64_t t = (uint64_t)r * G + j;
            int b = group_width(widths, t);
            for (int i = 0; i < 64; ++i)
                codes_out[t * 64 + i] = (int8_t)decode_code(payload, p, b, i);
            p += 8u * b;
        }
    }
    return OR_OK;
}

/* y[mm][r] for rows r in [row_begin, row_end) and all m inputs.
 * x is binary16 [m][k]; y is double [m][n] (only the selected rows are
 * written). Scalar loops in the order of the definition. */
int oracle_gemm(uint32_t n, uint32_t k, const uint8_t *widths, const uint16_t *scales,
                const uint32_t *row_offsets, const uint8_t *payload, uint64_t payload_bytes,
                const uint16_t *x, uint32_t m, double *y, uint32_t row_begin, uint32_t row_end)
{
    int st = oracle_check_offsets(n, k, widths, row_offsets, payload_bytes);
    if (st)
        return st;
    if (row_begin > row_end || row_end > n)
        return OR_ERR_SHAPE;
    if ((uint64_t)m * n != 0 && !y)
        return OR_ERR_NULL;
    if ((uint64_t)n * k != 0 && (!payload || !scales || (m && !x)))
        return OR_ERR_NULL;
    uint32_t G = k / 64;
    for (uint32_t mm = 0; mm < m; ++mm) {
        const uint16_t *xm = x + (uint64_t)mm * k;
        for (uint32_t r = row_begin; r < row_end; ++r) {
            uint64_t p = row_offsets[r];
            double acc = 0.0;
            for (uint32_t j = 0; j < G; ++j) {
                uint64_t t = (uint64_t)r * G + j;
                int b = group_width(widths, t);
                double s = oracle_half_to_double(scales[t]);
                double d = 0.0;
                for (int i = 0; i < 64; ++i)
                    d += (double)decode_code(payload, p, b, i) *
                         oracle_half_to_double(xm[(uint64_t)j * 64 + i]);
                acc += s * d;
                p += 8u * b;
            }
            y[(uint64_t)mm * n + r] = acc;
        }
    }
    return OR_OK;
}

/* batch-1 GEMV: y[r] for r in [row_begin, row_end) */
int oracle_gemv(uint32_t n, uint32_t k, const uint8_t *widths, const uint16_t *scales,
                const uint32_t *row_offsets, const uint8_t *payload, uint64_t payload_bytes,
                const uint16_t *x, double *y, uint32_t row_begin, uint32_t row_end)
{
    return oracle_gemm(n, k, widths, scales, row_offsets, payload, payload_bytes, x, 1, y,
                       row_begin, row_end);
}
