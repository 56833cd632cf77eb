/*
 * vbq.h - C ABI of the VBQ packed-weight decode library for AMD MI355X (gfx950).
 *
 * Method: "Variable Bit-width Quantization: Learning Per-Group Precision for
 * 'Bigger-but-Smaller' Language Models" (arXiv 2607.02893).
 *   §3.1, Eq. (1): weights are quantised in contiguous groups of 64 along the
 *     contracted dimension; group g has a width b_g and a scale s_g, and the
 *     dequantised weight is s_g * q with q on the symmetric integer grid
 *     |q| <= 2^(b-1) - 1; the 1-bit case is sign * scale (q in {-1, +1}).
 *   §6, "Fused kernels over packed weights": decode reads each group's packed
 *     bytes, expands them in registers with the group's scale and accumulates
 *     y = W x without writing a dense matrix; "Granularity is
 *     deployment-friendly": widths come from {1, 2, 4, 8} and groups pack into
 *     whole bytes.
 *
 * Packed layout (what the paper leaves open is fixed here):
 *   W is n x k, row-major, k % 64 == 0, G = k / 64 groups per row; group
 *   (r, j) covers W[r][64j .. 64j+63].
 *   tiles        groups are cut into tiles of VBQ_TILE_ROWS = 64 rows by
 *                VBQ_TILE_GROUPS = 4 groups (edge tiles are smaller); tile
 *                (a, c) holds rows [64a, 64a+64) and groups [4c, 4c+4) and is
 *                numbered a * ceil(G/4) + c.
 *   metadata slot of group (r, j), in tile order: with r0 = 64a, j0 = 4c and
 *                the tile's R rows and C groups,
 *                  m = r0*G + R*j0 + (r - r0)*C + (j - j0),
 *                i.e. tiles one after the other, each tile row-major, so the
 *                metadata of one tile is one contiguous run of R*C slots.
 *   widths       uint8 [ceil(n*G/4)]  2-bit code c = (widths[m/4] >> 2*(m%4)) & 3,
 *                                     width b = 1 << c in {1, 2, 4, 8}.
 *   scales       uint16 [n*G]         scales[m] = IEEE binary16 bit pattern of s.
 *   tile_offsets uint32 [tiles+1]     exclusive prefix sum of the tile payload
 *                                     sizes (each the sum of 8*b over its
 *                                     groups); tile_offsets[tiles] = payload size.
 *   payload      uint8                tile after tile; inside a tile the groups
 *                                     are bucketed by width (1, 2, 4 then 8
 *                                     bits) and ordered column-major inside a
 *                                     bucket (j ascending, then r ascending);
 *                                     each group holds 8*b bytes, so its offset
 *                                     is the exclusive prefix sum of 8*b over
 *                                     the groups stored before it.
 *   inside a group, element i (weight W[r][64j+i]) is a b-bit field:
 *     b = 1: bit i (byte i/8, bit i%8) - a sign bit: 0 -> +1, 1 -> -1;
 *     b = 8: byte i, two's complement;
 *     b = 2: in little-endian 32-bit word i/16, field m = e/2 + 8*(e%2) with
 *            e = i%16, bits 2m..2m+1, two's complement;
 *     b = 4: in little-endian 32-bit word i/8, field m = e/2 + 4*(e%2) with
 *            e = i%8, bits 4m..4m+3, two's complement.
 *   The two's complement pattern -2^(b-1) is off the grid: vbq_pack rejects
 *   it (kernels read it as -2^(b-1)).
 *   Result: y[m][r] = sum_j s_{r,j} * sum_i q_{r,j,i} * x[m][64j+i]; codes are
 *   exact in fp16, products and sums are fp32, the scale is applied in fp32
 *   once per group, y is fp32 (fp16 from vbq_gemv_multi_f16, and
 *   fp16(silu(g) * u) from vbq_gemv_swiglu).
 *   The export side fills this layout: vbq_quantize (§3.1 Eq. (1) on the
 *   device), the §3.4 recipe's widths, vbq_pack, vbq_check_padding and the
 *   container; vbq_soft_quantize is the §3.2 training-time mixture.
 *
 * Conventions for every entry point:
 *   - All buffers belong to the caller. Host entry points (vbq_pack*,
 *     vbq_validate_host, vbq_check_padding, vbq_uniform_width, vbq_container_*,
 *     vbq_recipe_head_*) take host pointers and run synchronously. Device
 *     entry points take device pointers inside vbq_matrix and as arguments,
 *     enqueue work on `stream` (a hipStream_t passed as void*, NULL = the
 *     null stream) and return without waiting; results are visible after the
 *     stream is synchronised.
 *   - A non-VBQ_OK status means nothing was written and nothing was enqueued;
 *     vbq_last_error() then holds a one-line description (thread-local).
 *     No C++ exception leaves the library: a failed host allocation returns
 *     VBQ_ERR_NOMEM.
 *   - Device entry points trust the metadata (use vbq_validate_host on the
 *     host copy once after packing); they check shapes, pointers, alignment
 *     and the ABI version.
 *   - Alignment: x, y and every vbq_matrix array 16-byte aligned (device
 *     allocators return 256-byte aligned memory).
 */
#ifndef VBQ_H
#define VBQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Only the entry points below are exported from the shared library. */
#define VBQ_API __attribute__((visibility("default")))

#define VBQ_ABI_VERSION 3u
#define VBQ_GROUP 64u
#define VBQ_TILE_ROWS 64u
#define VBQ_TILE_GROUPS 4u
#define VBQ_MAX_K 65536u      /* k limit of the device entry points */
#define VBQ_MAX_BATCH 64u     /* m limit of vbq_gemm_smallbatch */
#define VBQ_MAX_MULTI 32u     /* matrices per vbq_gemv_multi call */

typedef enum vbq_status {
    VBQ_OK = 0,
    VBQ_ERR_NULL = 1,       /* a required pointer is NULL */
    VBQ_ERR_SHAPE = 2,      /* k % 64 != 0, k > VBQ_MAX_K (device), m == 0 or m > VBQ_MAX_BATCH */
    VBQ_ERR_WIDTH = 3,      /* a width is not 1, 2, 4 or 8 */
    VBQ_ERR_CODE = 4,       /* a code is off its width's grid */
    VBQ_ERR_SCALE = 5,      /* a scale is inf or NaN */
    VBQ_ERR_CAPACITY = 6,   /* payload_capacity is smaller than the packed payload */
    VBQ_ERR_OFFSETS = 7,    /* tile_offsets / payload_bytes disagree with the widths */
    VBQ_ERR_ALIGN = 8,      /* a device pointer is not 16-byte aligned */
    VBQ_ERR_TOO_LARGE = 9,  /* payload would not fit 32-bit offsets */
    VBQ_ERR_HIP = 10,       /* the HIP runtime refused a launch */
    VBQ_ERR_ABI = 11,       /* vbq_matrix.abi_version != VBQ_ABI_VERSION */
    VBQ_ERR_PADDING = 12,   /* a padded row or column does not dequantize to zero */
    VBQ_ERR_FORMAT = 13,    /* a container's header, sizes or checksum is wrong */
    VBQ_ERR_NOMEM = 14,     /* a host allocation inside the library failed */
    VBQ_ERR_INTERNAL = 15   /* any other C++ exception inside the library (none is expected) */
} vbq_status;

/* Byte sizes of the four packed arrays. */
typedef struct vbq_sizes {
    uint64_t widths_bytes;
    uint64_t scales_bytes;
    uint64_t offsets_bytes;     /* tile_offsets: 4 * (tiles + 1) */
    uint64_t payload_bytes;
    uint64_t total_bytes;   /* = sum of the four; the bytes one GEMV must stream for W */
} vbq_sizes;

/* Non-owning view of one packed matrix. The struct itself lives in host
 * memory; the array pointers are host pointers for host entry points and
 * device pointers for device entry points. Device kernels read the payload
 * through bounds-checked buffer descriptors: no read leaves
 * [payload, payload + payload_bytes), even with a corrupt tile_offsets. */
typedef struct vbq_matrix {
    uint32_t abi_version;          /* VBQ_ABI_VERSION */
    uint32_t n;                    /* rows (outputs) */
    uint32_t k;                    /* columns (inputs), multiple of 64 */
    uint32_t payload_bytes;        /* == tile_offsets[tiles] */
    const uint8_t *widths;
    const uint16_t *scales;
    const uint32_t *tile_offsets;
    const uint8_t *payload;
    /* 0, or b in {1, 2, 4, 8} when every group has width b (the deployed
     * recipe of VBQ §3.4 stores whole projections at one width; §6 notes a
     * kernel then handles one width per projection). Device entry points
     * given a launch whose matrices all carry the same b run the
     * uniform-width kernels, which read neither the width codes nor
     * tile_offsets. vbq_uniform_width computes it from a host view;
     * vbq_validate_host checks it; device entry points check only that
     * payload_bytes == 8 * b * n * k / 64 (OFFSETS otherwise). */
    uint32_t uniform_bits;
    /* NULL, or the matrix's stream index (derived data, device memory,
     * 16-byte aligned, vbq_stream_index_bytes bytes; vbq_build_stream_index
     * writes it): for tile t, bytes [256 t, 256 t + 256) list the tile's
     * groups in payload order (width buckets 1, 2, 4, 8 bits, column-major
     * inside a bucket, as the layout above stores them), one byte each,
     * (j - j0) * 64 + (r - r0); unused bytes of smaller tiles are 0. After
     * all tiles' lists, at 256 * tiles + 8 t: the tile's group counts per
     * width code 0..3 as four uint16. The mixed-width GEMV kernels then read
     * the index instead of the width codes and skip deriving the counts and
     * the list per tile and call. It belongs to the widths it was built
     * from: rebuild it when they change. */
    const uint8_t *stream_index;
} vbq_matrix;

/* Library ABI version (compare with VBQ_ABI_VERSION). Plumbing: the pages
 * define no such call. */
VBQ_API uint32_t vbq_abi_version(void);

/* Bytes of an n x k matrix's stream index: 264 per tile (host). The pages
 * are silent: the index is a decode-side acceleration of the layout above
 * (VBQ §6, "Fused kernels over packed weights": the kernel walks each width
 * bucket; the index says in advance which group each bucket entry is).
 * Errors: NULL, SHAPE (k % 64). */
VBQ_API vbq_status vbq_stream_index_bytes(uint32_t n, uint32_t k, uint64_t *bytes_out);

/* Write w's stream index (layout at vbq_matrix.stream_index) to the device
 * buffer index_out of vbq_stream_index_bytes(w->n, w->k) bytes, 16-byte
 * aligned: one wave per tile counts its widths and lists its groups, the
 * same derivation the mixed-width kernels (VBQ §6, "Fused kernels over
 * packed weights") otherwise repeat per tile and call; the pages are silent
 * on such an index. w->stream_index is not read (but must be NULL or
 * aligned). Asynchronous on `stream`. Errors: NULL, ABI, SHAPE, ALIGN,
 * OFFSETS, HIP. */
VBQ_API vbq_status vbq_build_stream_index(const vbq_matrix *w, uint8_t *index_out, void *stream);

/* Sizes of the packed arrays for an n x k matrix with per-group widths
 * bits[n*(k/64)] (host). Errors: NULL, SHAPE (k % 64), WIDTH, TOO_LARGE.
 * Layout: §3.1 (groups of 64) and §6 (whole-byte groups of {1,2,4,8} bits). */
VBQ_API vbq_status vbq_pack_sizes(uint32_t n, uint32_t k, const uint8_t *bits, vbq_sizes *out);

/* Pack integer codes into the layout above (host, single-threaded,
 * deterministic). Inputs are in natural order, group (r, j) at r*G + j:
 * bits: [n*G] widths; codes: int8 [n][k] on each group's grid (§3.1 Eq. (1):
 * |q| <= 2^(b-1)-1, b = 1: q = +-1); scales: binary16 [n*G], finite. Outputs
 * widths_out and scales_out are in metadata-slot (tile) order. Output arrays sized by vbq_pack_sizes; payload_capacity is the size
 * of payload_out in bytes. Every input is checked before anything is written:
 * NULL, SHAPE, WIDTH, CODE, SCALE, CAPACITY, TOO_LARGE. */
VBQ_API vbq_status vbq_pack(uint32_t n, uint32_t k, const uint8_t *bits, const int8_t *codes,
                    const uint16_t *scales, uint8_t *widths_out, uint16_t *scales_out,
                    uint32_t *tile_offsets_out, uint8_t *payload_out, uint64_t payload_capacity);

/* Number of tiles of an n x k matrix: ceil(n/64) * ceil(k/256). Plumbing of
 * the layout above (the pages fix no tiling). */
VBQ_API uint64_t vbq_tile_count(uint32_t n, uint32_t k);

/* Check a packed matrix held in host memory: k % 64, tile_offsets equal to
 * the prefix sum of the tile payload sizes, payload_bytes == tile_offsets[tiles],
 * every field on its grid, every scale finite. This is the export-time check
 * of the packed contract that VBQ §6, "Granularity is deployment-friendly",
 * calls for; the device entry points do not repeat it.
 * Errors: NULL, ABI, SHAPE, OFFSETS, CODE, SCALE, NOMEM. */
VBQ_API vbq_status vbq_validate_host(const vbq_matrix *host_view);

/* y = W x for one fp16 vector (§6 fused decode at batch 1).
 * w: device view; x: device binary16 [k]; y: device fp32 [n] (overwritten).
 * Asynchronous on `stream`. Errors: NULL, ABI, SHAPE (k > VBQ_MAX_K), ALIGN,
 * OFFSETS (payload_bytes below 8 per group: no packed matrix has that; the
 * device views are not otherwise re-validated), HIP. n == 0 enqueues
 * nothing; k == 0 writes y = 0. */
VBQ_API vbq_status vbq_gemv(const vbq_matrix *w, const uint16_t *x, float *y, void *stream);

/* Several independent batch-1 GEMVs in one launch (VBQ §6, "Fused kernels
 * over packed weights", for each matrix): ys[i] = W_i xs[i] for
 * i < count <= VBQ_MAX_MULTI. ws, xs and ys are host arrays of count entries
 * (the matrix views and x / y pointers as for vbq_gemv). Matrices that read
 * the same activation (q/k/v, gate/up) or a whole layer's projections run as
 * one dispatch. When every matrix declares a width (uniform_bits), the
 * uniform-width kernels run, also when the declared widths differ. Asynchronous on `stream`. Errors: NULL, ABI, SHAPE (count),
 * ALIGN, OFFSETS, HIP.
 * Scratch: launches that split a row tile across workgroups (large k, small
 * n) and the gated epilogue use a library-owned device buffer per (device,
 * stream): partial sums and self-resetting arrival counters. It is
 * allocated (hipMalloc, then a clearing kernel on `stream`) the first time a
 * call on that stream needs it, and enlarged when a later call needs more;
 * a superseded buffer is kept, not freed, because a graph captured earlier
 * may still use it. Every buffer is held until the process ends. While
 * `stream` is being captured into a graph the library never allocates: a
 * call that would need a new or larger buffer returns VBQ_ERR_HIP (make one
 * call of the same shapes on that stream before capturing). A captured graph
 * uses the scratch of the stream it was captured on. Calls that overlap on
 * the same stream handle (including replays of such a graph on another
 * stream) race on the scratch and are not allowed. vbq_gemv_multi_noalloc is
 * the variant that never allocates. */
VBQ_API vbq_status vbq_gemv_multi(const vbq_matrix *const *ws, const uint16_t *const *xs, float *const *ys,
                                  uint32_t count, void *stream);

/* vbq_gemv_multi with fp16 outputs (VBQ §6, "Fused kernels over packed
 * weights", with the decode step's fp16 activations handed to the next
 * projection): ys[i] is device binary16 [n_i], each
 * value the fp32 result vbq_gemv_multi computes, rounded to nearest even
 * (beyond the fp16 range: +-inf), so a projection feeds the next layer's
 * fp16 input without a conversion launch. Same arguments, errors and
 * scratch as vbq_gemv_multi otherwise. */
VBQ_API vbq_status vbq_gemv_multi_f16(const vbq_matrix *const *ws, const uint16_t *const *xs, uint16_t *const *ys,
                                      uint32_t count, void *stream);

/* Gated-MLP front half in one launch (VBQ §6, "Granularity is
 * deployment-friendly", states the gated form silu(g) * u of the MLP
 * intermediates): g = gate x and u = up x exactly as vbq_gemv computes them
 * (fp32, same order of sums), then h[r] = fp16(g[r] * u[r] / (1 + e^-g[r])),
 * rounded to nearest even (beyond the fp16 range: +-inf). The launch writes
 * h itself; g and u stay in the library's scratch. h is the fp16 input of
 * the down projection's vbq_gemv.
 * gate, up: device views of one shape n x k. x: device binary16 [k]; h:
 * device binary16 [n]; both 16-byte aligned; the caller owns them. k == 0
 * writes h = 0. Scratch as for vbq_gemv_multi. Asynchronous on `stream`.
 * Errors: NULL, ABI, SHAPE (the shapes differ, k > VBQ_MAX_K), ALIGN,
 * OFFSETS, HIP. */
VBQ_API vbq_status vbq_gemv_swiglu(const vbq_matrix *gate, const vbq_matrix *up, const uint16_t *x, uint16_t *h,
                                   void *stream);

/* Y = X W^T for m <= VBQ_MAX_BATCH fp16 vectors (small-batch decode). The
 * pages run decode at batch 1 only (VBQ §6, "Fused kernels over packed
 * weights": every generated token streams every weight once) and are
 * silent on batches; this call is the same per-group arithmetic (§3.1
 * Eq. (1), w_hat = s * q) applied to m activation rows, with each group
 * decoded once for all rows on the matrix-core path.
 * x: device binary16 [m][k] row-major; y: device fp32 [m][n] row-major
 * (overwritten). Runs on the matrix cores (each group's codes decoded once,
 * 16x16x32 fp16 products, fp32 accumulation) when m > 16, or when m >= 4 and
 * m * m times the matrix's tile count (64x256 weights per tile) is at least
 * 85000; otherwise on the vector units as GEMVs in one launch: one row of X
 * per wave, or, at m = 2 on a matrix of at least 2048 tiles, both rows per
 * wave (each tile decoded once for both); the faster choices, measured.
 * Scratch as for vbq_gemv_multi.
 * Asynchronous on `stream`. Errors: NULL, ABI, SHAPE, ALIGN, OFFSETS, HIP. */
VBQ_API vbq_status vbq_gemm_smallbatch(const vbq_matrix *w, const uint16_t *x, uint32_t m, float *y,
                               void *stream);

/* Small-batch products of several matrices that read the same m rows of X
 * (VBQ §6, "Fused kernels over packed weights", batched: q, k and v, or gate
 * and up, at one decode step of m sequences; the pages are silent on
 * batches): ys[i] = X W_i^T. x: device binary16 [m][k] shared by all
 * matrices (every ws[i] has the same k); ys[i]: device fp32 [m][n_i]. The
 * small-batch rule is applied to the matrices together (their tile counts
 * summed): on the matrix cores they share launches of up to 8 matrices,
 * whose latency they then pay once; otherwise each runs as GEMVs of one row
 * of X per wave (both rows at m = 2 when the matrices have at least 2048
 * tiles together), and those share launches of up to VBQ_MAX_MULTI
 * (matrix, rows) entries, so a layer's projections at batch 8 take as many
 * launches as at batch 1. The
 * results agree with vbq_gemm_smallbatch on each matrix within the GEMV
 * tolerance (the two may take different paths). Asynchronous on `stream`;
 * scratch as for vbq_gemv_multi. Errors: NULL, ABI, SHAPE (m, or the k's
 * differ), ALIGN, OFFSETS, HIP. */
VBQ_API vbq_status vbq_gemm_smallbatch_multi(const vbq_matrix *const *ws, const uint16_t *x, uint32_t m,
                                             float *const *ys, uint32_t count, void *stream);

/* vbq_gemv_multi for callers that cannot allocate device memory: code under
 * graph capture, serving loops and harnesses that forbid hipMalloc. Same
 * arguments, kernels, launch shapes and results (bit for bit) as
 * vbq_gemv_multi, but the split-K partial sums and arrival counters live in
 * a fixed array in the library's device memory (VBQ_NOALLOC_SCRATCH_BYTES per
 * GPU, the first VBQ_NOALLOC_COUNTER_BYTES of it counters that are zero
 * between calls), so the call never allocates, frees or synchronizes. Each
 * GPU the library runs on holds its own copy of the array until the process
 * ends; the first call on a GPU clears its counters with a kernel on
 * `stream`. Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (on any streams, graph replays included) race and are
 * not allowed. Errors: those of vbq_gemv_multi, and CAPACITY when the
 * launch needs more than the array holds (more split 64-row tiles than
 * VBQ_NOALLOC_COUNTER_BYTES / 128, each tile's arrival counter on a
 * 128-byte line of its own, or more partial sums than the rest of the
 * array). */
#define VBQ_NOALLOC_SCRATCH_BYTES (4u << 20)
#define VBQ_NOALLOC_COUNTER_BYTES (64u << 10)
VBQ_API vbq_status vbq_gemv_multi_noalloc(const vbq_matrix *const *ws, const uint16_t *const *xs, float *const *ys,
                                          uint32_t count, void *stream);

/* Decoded integer codes int8 [n][k] of a device matrix, produced with the
 * same in-register field decoding the GEMV and GEMM kernels use (a test and
 * inspection hook; §3.1 Eq. (1) grid). Asynchronous. Errors: NULL, ABI,
 * SHAPE, ALIGN, OFFSETS, HIP. */
VBQ_API vbq_status vbq_unpack_codes(const vbq_matrix *w, int8_t *codes_out, void *stream);

/* Quantize fp32 weights group by group into the codes and scales vbq_pack
 * takes (VBQ §3.1 Eq. (1); device, asynchronous on `stream`).
 * w: device fp32 [n][k] row-major, 16-byte aligned, finite.
 * bits: device uint8 [n*(k/64)], each group's width in {1, 2, 4, 8} (a group
 *   with any other value gets scale 0 and codes 0).
 * codes_out: device int8 [n][k] (4-byte aligned); scales_out: device
 *   binary16 bit patterns [n*(k/64)] (2-byte aligned).
 * b >= 2: s = max|w| / (2^(b-1) - 1) in fp32, stored as binary16 (nearest
 *   even, saturated at 65504); q = clip(round(w / s), +-(2^(b-1) - 1)) with
 *   the stored s, ties away from zero, and q = 0 if the stored s is 0.
 * b = 1: s = the mean of |w| (summed in fp64, rounded once to binary16);
 *   q = -1 for w < 0, else +1.
 * The caller owns every buffer. Errors: SHAPE (k % 64, or more groups than
 * one launch takes), NULL, ALIGN, HIP. */
VBQ_API vbq_status vbq_quantize(uint32_t n, uint32_t k, const float *w, const uint8_t *bits, int8_t *codes_out,
                                uint16_t *scales_out, void *stream);

/* Training-side soft quantizer (VBQ §3.2, "Differentiable bit selection";
 * device, asynchronous on `stream`). Per group g of w (fp32 [n][k], 16-byte
 * aligned): pi_g = softmax((logits_g + gumbel_g) / tau) over the widths
 * (1, 2, 4, 8), w_soft = sum_k pi_g,k * w_hat^(B_k) with w_hat^(b) Eq. (1)
 * at width b with an fp32 scale (no binary16 rounding; fp32 division and
 * ties away from zero as in vbq_quantize, the 1-bit mean summed in fp64),
 * group_bits[g] = sum_k pi_g,k * B_k, and *mean_bits = the mean of
 * group_bits over the groups, summed in fp64 in a fixed order (0 when there
 * is no group). logits, gumbel, pi: fp32 [n*k/64][4] (the Gumbel noise is
 * the caller's draw); w_soft fp32 [n][k]; group_bits fp32 [n*k/64];
 * mean_bits one double. w, w_soft, logits, gumbel and pi 16-byte aligned,
 * group_bits 4, mean_bits 8; the caller owns every buffer. The mean uses an
 * 8 KiB library-owned device buffer per (device, stream), allocated on the
 * first call on that stream and held until the process ends; that first call
 * must not be made while the stream is being captured (VBQ_ERR_HIP); calls
 * that overlap on one stream handle are not allowed. Errors: SHAPE
 * (k % 64, tau not positive and finite, too many groups), NULL, ALIGN, HIP. */
VBQ_API vbq_status vbq_soft_quantize(uint32_t n, uint32_t k, const float *w, const float *logits,
                                     const float *gumbel, float tau, float *w_soft, float *pi, float *group_bits,
                                     double *mean_bits, void *stream);

/* The fixed recipe's head widths (VBQ §3.4, host): one width per vocabulary
 * row from its token frequency freq[rows]. Rows are ranked by descending
 * frequency (ties: lower row first); with N rows, the first round(0.005 N)
 * ranks get 8 bits, ranks up to round(0.02 N) 4 bits, up to round(0.12 N)
 * 2 bits, the rest 1 bit (round = half up; a 32000-row head averages 1.18
 * bits). Every group of row r then has width bits_out[r]. The projection
 * recipe of the same section needs no call: first-block MLP projections
 * (gate, up, down) at 4 bits, all other attention and MLP projections at 2.
 * Errors: NULL (rows > 0 and a NULL pointer). */
VBQ_API vbq_status vbq_recipe_head_bits(uint32_t rows, const uint64_t *freq, uint8_t *bits_out);

/* The same ranking (VBQ §3.4, frequency-tiered head) as vocabulary rows
 * (host): order_out[i] = the row of
 * rank i (descending frequency, ties to the lower row). The recipe's tiers
 * are then the rank ranges [0, round(0.005 N)), [.., round(0.02 N)),
 * [.., round(0.12 N)), [.., N): a head stored as four one-width matrices
 * over those ranges runs as one launch of vbq_gemv_multi (each matrix
 * declaring its width), and its outputs, concatenated, are the logits in
 * rank order. Errors: NULL (rows > 0 and a NULL pointer). */
VBQ_API vbq_status vbq_recipe_head_order(uint32_t rows, const uint64_t *freq, uint32_t *order_out);

/* The frequency-grouped head as row blocks (VBQ §3.4, "From discovery to a
 * fixed recipe": the head's widths are tiered by token frequency; §6,
 * "Fused kernels over packed weights": the head runs as frequency-grouped
 * row buckets). order_out[rows] = the rows in rank order as
 * vbq_recipe_head_order gives them; tier_rows_out[4] = how many ranks fall in
 * the 8-, 4-, 2- and 1-bit tiers, so tier t holds the ranks from the sum of
 * the earlier counts on. Packing each non-empty tier's rows (in rank order)
 * as one one-width matrix gives the grouped head. Errors: NULL (a NULL
 * pointer with rows > 0, or tier_rows_out NULL), NOMEM. */
VBQ_API vbq_status vbq_recipe_head_tiers(uint32_t rows, const uint64_t *freq, uint32_t *order_out,
                                         uint32_t *tier_rows_out);

/* The frequency-grouped head in one launch, its logits in vocabulary order
 * (VBQ §6, "Fused kernels over packed weights": the head runs as
 * frequency-grouped row buckets; §3.4, "From discovery to a fixed recipe",
 * for the tiers). tiers[0..count) are the head's row blocks in rank order,
 * tier t holding the ranks s_t .. s_t + n_t - 1 (s_0 = 0, s_{t+1} = s_t +
 * n_t; the blocks vbq_recipe_head_tiers describes, each usually declaring
 * its width), all with the same k, count <= VBQ_MAX_MULTI. row_map: device
 * uint32 [sum of n_t], the vocabulary row of each rank (the order_out of
 * vbq_recipe_head_tiers). The call computes (tier x)[r] exactly as
 * vbq_gemv_multi computes it for these tiers and stores it at
 * y[row_map[s_t + r]]; map values >= y_rows are skipped, and rows of y that
 * no rank maps to are left unchanged. Distinct ranks must map to distinct
 * rows (two ranks on one row race). x: device binary16 [k]; y: device fp32
 * [y_rows]; x, row_map and y 16-byte aligned, owned by the caller. k == 0
 * stores 0 at every mapped row. Scratch as for vbq_gemv_multi.
 * Asynchronous on `stream`. Errors: NULL, ABI, SHAPE (count, the k's
 * differ, k > VBQ_MAX_K), ALIGN, OFFSETS, HIP. */
VBQ_API vbq_status vbq_gemv_head_grouped(const vbq_matrix *const *tiers, uint32_t count, const uint16_t *x,
                                         const uint32_t *row_map, float *y, uint32_t y_rows, void *stream);

/* Export-time check of the padding contract (VBQ §6, "Granularity is
 * deployment-friendly": MLP intermediates are zero-padded so the contracted
 * dimension is a multiple of 512; padded channels are inert because
 * silu(0) * u = 0). Host pointers. Passes when the matrix validates
 * (vbq_validate_host), k is a multiple of k_multiple, n_real <= n,
 * k_real <= k, and every weight in a padded row (r >= n_real) or padded
 * column (c >= k_real) dequantizes to exactly zero: its group's scale is
 * +-0, or its code is 0 (so a 1-bit group touching the padding needs scale
 * 0). Errors: those of vbq_validate_host; SHAPE (k_multiple == 0, k not a
 * multiple of it, n_real > n or k_real > k); PADDING (the first non-zero
 * padded weight is named by vbq_last_error). */
VBQ_API vbq_status vbq_check_padding(const vbq_matrix *host_view, uint32_t n_real, uint32_t k_real,
                                     uint32_t k_multiple);

/* Versioned container: one packed matrix as one byte image (a file's
 * contents), little-endian.
 *   bytes 0-7    magic "VBQPACK" and a zero byte
 *   8  u32 format version (VBQ_CONTAINER_VERSION)
 *   12 u32 header bytes (128)
 *   16 u32 n, 20 u32 k, 24 u32 group size (64), 28 u32 tile rows (64),
 *   32 u32 tile groups (4), 36 u32 payload_bytes
 *   40 u64 widths offset, 48 u64 scales offset, 56 u64 tile_offsets offset,
 *   64 u64 payload offset, 72 u64 total bytes
 *   80 u32 CRC-32 (IEEE 802.3) of bytes [128, total), 84 u32 CRC-32 of
 *   bytes [0, 84); the rest of the header is zero.
 * The four arrays follow at 256-byte aligned offsets, in that order, with
 * zero bytes between them, so one contiguous upload keeps every array
 * aligned for the device entry points. */
#define VBQ_CONTAINER_VERSION 1u
#define VBQ_CONTAINER_HEADER 128u

/* Bytes the container of w takes. Host pointers are not read. Errors: NULL,
 * ABI, SHAPE (k % 64). The container is the file form of the export step
 * (VBQ §6, "Granularity is deployment-friendly": packed groups produced at
 * export and checked there); its byte format is this library's own. */
VBQ_API vbq_status vbq_container_size(const vbq_matrix *host_view, uint64_t *bytes_out);

/* Write w (host pointers, validated first, as the export-time check of
 * VBQ §6, "Granularity is deployment-friendly", asks) into out[0, capacity); the
 * caller owns out. *written = the container size. Errors: those of
 * vbq_validate_host; NULL; CAPACITY (capacity below the container size). */
VBQ_API vbq_status vbq_container_write(const vbq_matrix *host_view, uint8_t *out, uint64_t capacity,
                                       uint64_t *written);

/* Check a container image buf[0, len) and fill *view_out with pointers into
 * buf (no copy; buf must outlive the view); the load side of the export
 * step of VBQ §6, "Granularity is deployment-friendly". Checks the magic, version,
 * layout constants, that every array lies inside buf at its aligned offset
 * with the sizes n and k give, both checksums, then runs vbq_validate_host
 * on the view and sets its uniform_bits (vbq_uniform_width). Errors: NULL; FORMAT (header, sizes or
 * checksum); those of vbq_validate_host. */
VBQ_API vbq_status vbq_container_open(const uint8_t *buf, uint64_t len, vbq_matrix *view_out);

/* One width per projection (VBQ §3.4, "From discovery to a fixed recipe",
 * and §6, one bucket per projection): *bits_out = b when every group of the
 * host view has width b, else 0
 * (also for n == 0 or k == 0). Reads the width codes only. Errors: NULL,
 * ABI, SHAPE (k % 64). */
VBQ_API vbq_status vbq_uniform_width(const vbq_matrix *host_view, uint32_t *bits_out);

/* ---- measurement: what the packed GEMV is compared with (not its path) ---- */

/* Read bytes of device memory at buf once with 16-byte loads and keep nothing
 * (device, asynchronous on `stream`): the HBM read rate a streaming launch of
 * that size reaches on this GPU, ramp and drain included, i.e. the practical
 * ceiling of the packed GEMV's launches. Plumbing of the measurement: the
 * pages define no such call. buf and bytes are multiples of 16; blocks
 * (1..2^20) workgroups of 256 threads; sink: device uint32 [blocks * 256],
 * written only for a value the buffer's XOR practically never takes.
 * Errors: NULL, ALIGN, SHAPE, HIP. */
VBQ_API vbq_status vbq_probe_stream_read(const void *buf, uint64_t bytes, uint32_t *sink, uint32_t blocks,
                                         void *stream);

/* y = W x for a dense fp16 W [n][k] row-major, fp16 x [k], fp32 y [n] (device,
 * asynchronous on `stream`): the dense baseline VBQ §6 compares packed decode
 * with (Figure 5 and the Table 2 caption: the same weights dequantized to
 * dense FP16). fp16 products, fp32 sums. w and x 16-byte aligned; k a
 * multiple of 64 up to 16384. Errors: NULL, ALIGN, SHAPE, HIP. */
VBQ_API vbq_status vbq_probe_dense_gemv(const uint16_t *w, const uint16_t *x, float *y, uint32_t n, uint32_t k,
                                        void *stream);

/* Static English name of a status. Plumbing: the pages define no such call. */
VBQ_API const char *vbq_status_string(vbq_status s);

/* Detail of the last failure on the calling thread ("" if none). Plumbing:
 * the pages define no such call. */
VBQ_API const char *vbq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VBQ_H */
