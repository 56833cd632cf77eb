// Device half of the VBQ library (gfx950): launches and kernels.
//
// VBQ paper (arXiv 2607.02893) §6, "Fused kernels over packed weights": each
// group's packed bytes are read once, expanded in registers and combined with
// the group's fp16 scale while y = W x accumulates; no dense weight matrix is
// written. Grid and scale: §3.1 Eq. (1). The payload is the width-bucketed
// tile stream described in vbq.h.
//
// Work decomposition. A wave owns one tile (64 rows x 4 groups) at a time:
//   1. lane r reads the four width codes and scales of row r; per column a
//      DPP prefix sum of one-hot width counters gives each row its rank
//      among the rows of its width and the per-width counts, which fix where
//      each width's bucket starts, so the payload loads are issued now;
//   2. while they travel, it stages the tile's 256 activations in LDS, once
//      as fp16 pairs and once as a 4-bit lookup table (16 partial sums per 4
//      activations), and writes one list of the tile's groups in the
//      stream's order (buckets by width, column-major inside a bucket);
//   3. for each width the wave walks its bucket with one group (or a 16-byte
//      slice of a group) per lane, so every instruction runs a single width's
//      unpack; the bucket is contiguous, so loads are coalesced (and go
//      through a buffer descriptor: the hardware bounds-checks them);
//   4. each group's fp32 dot product is parked in LDS; each row's lane
//      scales its groups once and sums them in a fixed order, so results are
//      bitwise repeatable.
// A workgroup of 4, 8 or 16 waves shares one row tile and splits its column
// tiles; when a row tile is further split across workgroups (small n, large
// k), the partial sums go to a scratch buffer and the last workgroup to
// arrive adds them in a fixed order. The host picks the workgroup size and
// the split count per launch from a cost model (gemv_plan).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "vbq_internal.h"

using vbq::fail;

namespace {

constexpr uint32_t kWave = 64;
constexpr uint32_t kTileRows = VBQ_TILE_ROWS;     // 64
constexpr uint32_t kTileGroups = VBQ_TILE_GROUPS; // 4
constexpr uint32_t kXStride = 36;                 // dwords per staged column (32 used, padded)
// Arrival counters (split row tiles, gate/up pairs) sit one per 128-byte line: device-scope atomics on
// one line serialize, and a launch's workgroups bump their counters at about the same time (9B o and
// down launches: 6.6 -> 6.2 and 8.8 -> 8.5 us; 1.0B set 532 -> 525 us a pass).
constexpr uint32_t kCounterStride = 32;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

// A constant the compiler treats as an unknown register value: lets a mask
// and an OR constant share one v_bitop3_b32 instead of a literal v_or_b32.
__device__ __forceinline__ uint32_t opaque(uint32_t c) {
    uint32_t r;
    asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
    return r;
}

// x ^ c computed where written (not folded into later mask-and-or steps)
__device__ __forceinline__ uint32_t xor_opaque(uint32_t x, uint32_t c) {
    uint32_t r;
    asm("v_xor_b32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(c));
    return r;
}

// Cross-lane moves on the VALU (DPP): quad permutes and rotations inside a row of 16 lanes.
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kRowRor1 = 0x121, kRowRor2 = 0x122, kRowRor4 = 0x124, kRowRor8 = 0x128;

// sum over the 16 lanes of a row, in every lane of the row
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp<kRowRor8>(v);
    v += dpp<kRowRor4>(v);
    v += dpp<kRowRor2>(v);
    v += dpp<kRowRor1>(v);
    return v;
}

__device__ __forceinline__ float half_to_float(uint32_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// Buffer descriptors (raw, 32-bit data format). The hardware checks every
// read against the descriptor's byte count and returns zeros past it, so a
// lane with nothing to read needs no clamped address and a read can never
// leave the array.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes), kRsrcWord3);
}
__device__ __forceinline__ uint2 buf_load8(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(off), 0, 0));
}
__device__ __forceinline__ uint4 buf_load16x(rsrc_t r, uint32_t off) {   // one 128-bit load
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0));
}
__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, uint32_t off) {
    return static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, 0));
}

// A tile's payload: from its first byte to the payload's end (nothing if the
// offset is past it; the saturating subtract is a vector instruction, so its
// result is moved back to a scalar register).
__device__ __forceinline__ rsrc_t tile_rsrc(const uint8_t *payload, uint32_t payload_bytes, uint32_t off) {
    const uint32_t left = __builtin_amdgcn_readfirstlane(payload_bytes - min(off, payload_bytes));
    return make_rsrc(payload + off, left);
}

// ---------------------------------------------------------------- per-width unpack
// Each helper turns one little-endian 32-bit word of a group into fp16 pairs
// whose bit patterns are f * u, u = q + 2^(b-1) the offset-binary code and f
// the field's power-of-two position factor: fp16 subnormals of value
// f * u * 2^-24, exact. The pairs come out in natural element order (2i,
// 2i+1) thanks to the in-group field layout and multiply fp16 activation
// pairs with v_dot2, which keeps fp16 subnormal inputs, so each product is
// exact in fp32; the group's sum is scaled by 2^24 / f and the offset
// 2^(b-1) * (sum of the group's activations) is taken off once per group.

// 8-bit: elements 4w..4w+3 -> pairs (0,1), (2,3); factor 1
__device__ __forceinline__ void unpack8(uint32_t v, uint32_t &p0, uint32_t &p1) {
    v ^= 0x80808080u;
    p0 = __builtin_amdgcn_perm(0u, v, 0x0C010C00u);   // bytes {v0, 0, v1, 0}
    p1 = __builtin_amdgcn_perm(0u, v, 0x0C030C02u);   // bytes {v2, 0, v3, 0}
}

// 4-bit: elements 8w..8w+7 -> pairs (0,1) x1, (2,3) x16, (4,5) x1, (6,7) x16: one mask each
__device__ __forceinline__ void unpack4(uint32_t v, uint32_t p[4]) {
    v = xor_opaque(v, 0x88888888u);
    const uint32_t h = v >> 8;
    p[0] = v & 0x000F000Fu;
    p[1] = v & 0x00F000F0u;
    p[2] = h & 0x000F000Fu;
    p[3] = h & 0x00F000F0u;
}

// 2-bit: elements 16w..16w+15 -> pairs m = 0..7 with factors 1,4,16,64,256,1,4,16
__device__ __forceinline__ void unpack2(uint32_t v, uint32_t p[8]) {
    v = xor_opaque(v, 0xAAAAAAAAu);
    const uint32_t h = v >> 10;
    p[0] = v & 0x00030003u;
    p[1] = v & 0x000C000Cu;
    p[2] = v & 0x00300030u;
    p[3] = v & 0x00C000C0u;
    p[4] = v & 0x03000300u;
    p[5] = h & 0x00030003u;
    p[6] = h & 0x000C000Cu;
    p[7] = h & 0x00300030u;
}

// 1-bit: bit i is the sign of element i; pair k = (2k, 2k+1) as fp16 +-1
__device__ __forceinline__ uint32_t unpack1_pair(uint32_t lo16, uint32_t hi16) {
    // lo16/hi16: the two sign bits already in bit positions 15 and 31
    return ((lo16 & 0x00008000u) | (hi16 & 0x80000000u)) | 0x3C003C00u;
}

// ---------------------------------------------------------------- tiles and lists

struct MatArgs {
    const uint8_t *widths;
    const uint16_t *scales;
    const uint32_t *tile_offsets;
    const uint8_t *payload;
    const uint16_t *x;
    float *y;
    float *partial;       // [splits][n] when splits > 1
    uint32_t *counters;   // [row tiles x kCounterStride] arrival counters when splits > 1 (self-resetting)
    uint32_t n, groups, col_tiles, splits, blocks;   // blocks = row tiles x splits
    uint32_t units;   // work units along K: column tiles, or groups of one chunk for uniform 8- and lean 4-bit
    uint32_t payload_bytes;
    uint32_t ubits;   // the matrix's declared single width, or 0
    uint16_t *y16;    // when set, y is stored here as fp16 (nearest even) instead of fp32 to y
    const uint8_t *index;   // the matrix's stream index (gemv_tiles<..., kIndexed = true>), else NULL
};


// Launched as a 2D grid: blockIdx.y picks the matrix, so a block loads its
// matrix's arguments with one scalar load and no search.
struct Batch {
    MatArgs m[VBQ_MAX_MULTI];
    // 1D launches (matrices of different declared widths): matrix i owns workgroups
    // [first_block[i], first_block[i + 1]); entries past the last matrix hold the total
    uint32_t first_block[VBQ_MAX_MULTI + 1];
    // Gated-MLP epilogue, when h is set: matrix 0 is gate and matrix 1 is up
    // (same n), and instead of y the launch writes h = fp16(silu(g) * u).
    uint16_t *h;
    float *pair;              // [2][n]: each row tile's finished g and u values
    uint32_t *pair_counters;  // [row tiles x kCounterStride] arrival counters (self-resetting)
    // Grouped head: when row_map is set, the matrices are row blocks of one head, matrix i holding the
    // ranks after those of matrices 0..i-1, and row r of matrix i is stored at y[row_map[rank]] (every
    // matrix's y is the head's y); map values at or past y_rows are not stored.
    const uint32_t *row_map;
    uint32_t y_rows;
};
static_assert(sizeof(Batch) <= 4096, "a launch's kernel arguments fit 4 KiB");

// 4992 bytes per wave: eight 4-wave, four 8-wave or two 16-wave workgroups
// fit one CU's 160 KiB. 64-byte aligned: the lookup table's addresses are
// formed with XORs below 64.
//
// Lookup table layout: table k (activations 4k..4k+3 of a column, k < 16) of
// column jl is the 64 bytes at 256 k + 64 jl, and its entry u (the sum of the
// activations picked by the set bits of u) sits at word u ^ 4 sw(k) with
// sw(k) = (k >> 1) & 3. One k's tables of the four columns then lie in four
// different groups of 16 banks (reads by lanes of different columns do not
// collide), and the 16 lanes that build one column's tables write their four
// 16-byte pieces to different banks.
struct alignas(64) WaveLds {
    union {
        float lut[16 * kTileGroups * 16];     // [nibble position][column][4-bit index, swizzled]
        float part[kTileGroups * kTileRows];  // group dot products (unscaled) at column * 64 + row, once
                                              // the 1-bit groups are done
    };
    uint32_t xs[kTileGroups * kXStride];     // fp16 activation pairs per column
    float corr[kTileGroups];                 // per column: the sum of its 64 activations
    uint8_t list[kTileRows * kTileGroups];   // the tile's groups in stream order, 1-bit bucket first:
                                             // column * 64 + row
};

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Lane index, recomputed at each use: kept live across a tile loop, every
// value derived from it would be hoisted too and the loop would run out of
// registers.
__device__ __forceinline__ uint32_t lane_id() {
    uint32_t r;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(r));
    return r;
}

// A copy of a kept lane index that the compiler cannot see through: one
// move per use instead of two instructions, and still nothing derived from
// it is hoisted.
__device__ __forceinline__ uint32_t relane(uint32_t lane) {
    uint32_t r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(lane));
    return r;
}

// Inputs of one tile that need no payload: read in one round trip and
// prefetched one tile ahead.
struct TileMeta {
    uint32_t off;     // payload byte offset of the tile (uniform)
    uint2 xv;         // activations 4k..4k+3 of column lane/16 (k = lane%16)
    uint32_t codes;   // width codes of row `lane`, groups j0..j0+3
    uint32_t s01;     // scales of row `lane`, groups j0, j0+1
    uint32_t s23;     // scales of row `lane`, groups j0+2, j0+3
};

template <bool kAligned, class Args>
__device__ __forceinline__ TileMeta load_meta(const Args &M, uint32_t a, uint32_t ct, uint32_t lane,
                                              bool with_x, bool with_codes = true) {
    TileMeta t;
    const uint32_t r0 = a * kTileRows, rows = min(kTileRows, M.n - r0);
    // kAligned: the group count is a multiple of 4, so every tile has four columns
    const uint32_t j0 = ct * kTileGroups, cn = kAligned ? kTileGroups : min(kTileGroups, M.groups - j0);
    // The tile offset is uniform: a scalar load (constant address space), so
    // moving it into a scalar register waits on the scalar counter only and
    // not on the payload loads issued before it.
    typedef const __attribute__((address_space(4))) uint32_t *const_u32p;
    t.off = ((const_u32p)(reinterpret_cast<uintptr_t>(M.tile_offsets)))[a * M.col_tiles + ct];
    // Loads are unconditional (lanes past the tile read a valid neighbour and
    // their values are never used), so the compiler can count them and wait
    // for exactly these, not for loads issued after them.
    // Byte offsets are 32-bit: a matrix has fewer than 2^29 groups (each group
    // has at least 8 payload bytes and the payload fits 32-bit offsets, which
    // the launch checks), so they address from a scalar base register.
    const uint32_t jl = min(lane >> 4, cn - 1), k = lane & 15;
    t.xv = make_uint2(0u, 0u);
    const uint32_t xoff = 128u * (j0 + jl) + 8u * k;
    if (with_x) t.xv = *reinterpret_cast<const uint2 *>(reinterpret_cast<const char *>(M.x) + xoff);
    t.codes = t.s01 = t.s23 = 0u;
    {
        // the tile's metadata is one contiguous run of rows*cn slots, row-major
        const uint32_t base = r0 * M.groups + rows * j0;
        const uint32_t lr = min(lane, rows - 1);
        if (kAligned || cn == kTileGroups) {
            // base is a multiple of 4: one width byte and one 8-byte scale load per row
            if (with_codes) t.codes = M.widths[(base >> 2) + lr];
            const uint2 sv =
                *reinterpret_cast<const uint2 *>(reinterpret_cast<const char *>(M.scales) + 2u * (base + 4u * lr));
            t.s01 = sv.x;
            t.s23 = sv.y;
        } else {
            const uint64_t g = base + static_cast<uint64_t>(lr) * cn;
            if (with_codes) {
                const uint64_t wbytes = (static_cast<uint64_t>(M.n) * M.groups + 3) >> 2;
                uint32_t two = M.widths[g >> 2];
                if ((g >> 2) + 1 < wbytes) two |= static_cast<uint32_t>(M.widths[(g >> 2) + 1]) << 8;
                t.codes = (two >> (2 * (g & 3))) & ((1u << (2 * cn)) - 1u);
            }
            uint32_t sc[4] = {0u, 0u, 0u, 0u};
            for (uint32_t q = 0; q < cn; ++q) sc[q] = M.scales[g + q];
            t.s01 = sc[0] | (sc[1] << 16);
            t.s23 = sc[2] | (sc[3] << 16);
        }
    }
    return t;
}

typedef __attribute__((address_space(3))) char lds_char;

// LDS byte address of a workgroup-shared object
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_char *)p));
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void lds_store16(uint32_t byte_addr, f32x4_t v) {
    *reinterpret_cast<__attribute__((address_space(3))) f32x4_t *>(byte_addr) = v;
}

// Stage the tile's activations: fp16 pairs, the 4-bit lookup table (sums of
// the activations selected by the set bits of a 4-bit index) and each
// column's activation sum (the offset of the unpack paths).
template <bool kLut = true>
__device__ __forceinline__ void stage_x_at(float *lut, uint32_t *xs, float *corr, uint2 xv, uint32_t lane) {
    const uint32_t jl = lane >> 4, k = lane & 15;
    xs[jl * kXStride + 2 * k] = xv.x;
    xs[jl * kXStride + 2 * k + 1] = xv.y;
    const float x0 = half_to_float(xv.x & 0xFFFFu), x1 = half_to_float(xv.x >> 16);
    const float x2 = half_to_float(xv.y & 0xFFFFu), x3 = half_to_float(xv.y >> 16);
    const float a01 = x0 + x1, t5 = x2 + x0, t6 = x2 + x1, t7 = x2 + a01;
    if (kLut) {
        // piece c of table (k, jl) at byte 256 k + 64 jl + 16 (c ^ sw(k)): the table is 64-byte
        // aligned, so the four addresses are one base and three XORs
        const uint32_t base = lds_addr(lut) + 256u * k + 64u * jl + 16u * ((k >> 1) & 3u);
        lds_store16(base, f32x4_t{0.f, x0, x1, a01});
        lds_store16(base ^ 16u, f32x4_t{x2, t5, t6, t7});
        lds_store16(base ^ 32u, f32x4_t{x3, x3 + x0, x3 + x1, x3 + a01});
        lds_store16(base ^ 48u, f32x4_t{x3 + x2, x3 + t5, x3 + t6, x3 + t7});
    }
    const float xsum = row16_sum(a01 + (x2 + x3));
    if (k == 0) corr[jl] = xsum;
}

template <bool kLut = true>
__device__ __forceinline__ void stage_x(WaveLds &L, uint2 xv, uint32_t lane) {
    stage_x_at<kLut>(L.lut, L.xs, L.corr, xv, lane);
}

// Inclusive prefix sum over the 64 lanes (DPP: row shifts, then row broadcasts).
__device__ __forceinline__ uint32_t wave_scan(uint32_t v) {
    v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x111, 0xF, 0xF, true));  // row_shr:1
    v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x112, 0xF, 0xF, true));  // row_shr:2
    v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x114, 0xF, 0xF, true));  // row_shr:4
    v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x118, 0xF, 0xF, true));  // row_shr:8
    v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x142, 0xA, 0xF, false)); // row_bcast:15
    v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x143, 0xC, 0xF, false)); // row_bcast:31
    return v;
}

// Per column, each lane's width code as a one-hot byte counter (byte c = 1
// for code c) and its inclusive prefix sum over the rows: byte c of the
// exclusive sum is the row's rank among the rows of its width in that column,
// byte c of lane 63's sum is the column's count of width c.
struct TileScan {
    uint32_t incl[kTileGroups];   // per lane
    uint32_t cols[kTileGroups];   // column counts, four bytes (uniform)
};

__device__ __forceinline__ TileScan tile_scan(const TileMeta &t, uint32_t rows, uint32_t cn, uint32_t lane,
                                              uint32_t cnt[4]) {
    TileScan T;
    const bool valid = lane < rows;
#pragma unroll
    for (uint32_t jl = 0; jl < kTileGroups; ++jl) {
        const uint32_t c = (t.codes >> (2 * jl)) & 3u;
        const uint32_t one = (valid && jl < cn) ? 1u << (8 * c) : 0u;
        T.incl[jl] = wave_scan(one);
        T.cols[jl] = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(T.incl[jl]), kWave - 1));
    }
    // tile totals per width (up to 256: summed outside the byte fields)
    uint32_t c0 = 0, c1 = 0, c2 = 0, c3 = 0;
#pragma unroll
    for (uint32_t jl = 0; jl < kTileGroups; ++jl) {
        c0 += T.cols[jl] & 0xFFu;
        c1 += (T.cols[jl] >> 8) & 0xFFu;
        c2 += (T.cols[jl] >> 16) & 0xFFu;
        c3 += T.cols[jl] >> 24;
    }
    cnt[0] = c0;
    cnt[1] = c1;
    cnt[2] = c2;
    cnt[3] = c3;
    return T;
}

// Lane r = row r of the tile: put each of its groups into the list at its
// place in the stream's order (buckets by width, column-major inside a bucket).
template <class Lds>
__device__ __forceinline__ void build_lists(Lds &L, const TileMeta &t, const TileScan &T, const uint32_t cnt[4],
                                            uint32_t rows, uint32_t cn, uint32_t lane) {
    const bool valid = lane < rows;
    // bucket starts, then the groups of each width in earlier columns, 16 bits per width (uniform)
    uint64_t before = (static_cast<uint64_t>(cnt[0]) << 16) | (static_cast<uint64_t>(cnt[0] + cnt[1]) << 32) |
                      (static_cast<uint64_t>(cnt[0] + cnt[1] + cnt[2]) << 48);
#pragma unroll
    for (uint32_t jl = 0; jl < kTileGroups; ++jl) {
        if (jl >= cn) break;
        const uint32_t c = (t.codes >> (2 * jl)) & 3u;
        const uint32_t excl = T.incl[jl] - (1u << (8 * c));
        const uint32_t slot = static_cast<uint32_t>((before >> (16 * c)) & 0xFFFFu) + ((excl >> (8 * c)) & 0xFFu);
        if (valid) L.list[slot] = static_cast<uint8_t>(jl * kTileRows + lane);
        const uint32_t cc = T.cols[jl];
        before += static_cast<uint64_t>(cc & 0xFFu) | (static_cast<uint64_t>((cc >> 8) & 0xFFu) << 16) |
                  (static_cast<uint64_t>((cc >> 16) & 0xFFu) << 32) | (static_cast<uint64_t>(cc >> 24) << 48);
    }
}


// Sum of the split partials p[0], p[stride], ... in split order. The coherent
// loads go out eight at a time (clamped addresses, no branches) so their round
// trips overlap instead of following one another.
__device__ __forceinline__ float sum_partials(const float *p, uint64_t stride, uint32_t splits) {
    float tot = 0.f;
    for (uint32_t s0 = 0; s0 < splits; s0 += 8) {
        float v[8];
#pragma unroll
        for (uint32_t i = 0; i < 8; ++i) {
            const uint32_t s = min(s0 + i, splits - 1);
            v[i] = __hip_atomic_load(p + s * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (uint32_t i = 0; i < 8; ++i)
            if (s0 + i < splits) tot += v[i];
    }
    return tot;
}

// ---- one group (or slice) per lane, per width; results to L.part[column * 64 + row]
// A list entry is that index (so the column is bits 6-7). The products are
// stored unscaled: the row's lane applies its own scales when it adds them.

__device__ __forceinline__ void store_part(WaveLds &L, uint32_t info, float v) { L.part[info] = v; }

// The two constants of the 1-bit lookup addresses, held in registers for a whole kernel
struct LutKeys {
    uint32_t mask, swz;
};
__device__ __forceinline__ LutKeys lut_keys() { return LutKeys{opaque(0x3c3c3c3cu), opaque(0x30201000u)}; }

// returns the product: L.part shares its bytes with the lookup table, so it
// is stored once every 1-bit group of the tile is done
__device__ __forceinline__ float group1(WaveLds &L, uint32_t info, uint2 v, LutKeys keys) {
    const uint32_t jl = info >> 6;
    // table k of column jl at byte 256 k + 64 jl, entry u at byte 4 u ^ 16 sw(k). Bytes t of lo / hi hold
    // 4 * (nibble 2t / 2t+1) of each word; nibble positions k = 8q + 2t and 8q + 2t + 1 both have
    // sw(k) = t, so one mask-then-XOR (v_bitop3, truth table 0x6a = (a & b) ^ c) serves both
    const char *lut = reinterpret_cast<const char *>(L.lut + jl * 16u);
    const uint32_t mask = keys.mask, swz = keys.swz;
    const uint32_t w[2] = {v.x, v.y};
    float acc[4];
#pragma unroll
    for (uint32_t q = 0; q < 2; ++q) {
        uint32_t lo, hi;
        asm("v_lshlrev_b32 %0, 2, %1\n\tv_bitop3_b32 %0, %0, %2, %3 bitop3:0x6a"
            : "=&v"(lo) : "v"(w[q]), "v"(mask), "v"(swz));
        asm("v_lshrrev_b32 %0, 2, %1\n\tv_bitop3_b32 %0, %0, %2, %3 bitop3:0x6a"
            : "=&v"(hi) : "v"(w[q]), "v"(mask), "v"(swz));
#pragma unroll
        for (uint32_t t = 0; t < 4; ++t) {
            const uint32_t k = 8 * q + 2 * t;
            const float a = *reinterpret_cast<const float *>(lut + 256u * k + ((lo >> (8 * t)) & 0xFFu));
            const float b = *reinterpret_cast<const float *>(lut + 256u * (k + 1) + ((hi >> (8 * t)) & 0xFFu));
            acc[t] = q == 0 ? a + b : acc[t] + (a + b);
        }
    }
    const float sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    return L.corr[jl] - 2.f * sum;
}

// unscaled product of one 2-bit group of column jl: pair m holds 4^m u (4^(m-5) u for m >= 5) as
// subnormals, so sum u x = 2^24 (a1 + a4 / 4 + ...), and q = u - 2
__device__ __forceinline__ float dot2bit(WaveLds &L, uint32_t jl, uint2 va, uint2 vb) {
    const uint32_t w[4] = {va.x, va.y, vb.x, vb.y};
    const uint4 *xp = reinterpret_cast<const uint4 *>(L.xs + jl * kXStride);
    float a1 = 0.f, a4 = 0.f, a16 = 0.f, a64 = 0.f, a256 = 0.f;
#pragma unroll
    for (uint32_t q = 0; q < 4; ++q) {
        uint32_t p[8];
        unpack2(w[q], p);
        const uint4 xa = xp[2 * q], xb = xp[2 * q + 1];
        a1 = dot2(p[0], xa.x, a1);
        a4 = dot2(p[1], xa.y, a4);
        a16 = dot2(p[2], xa.z, a16);
        a64 = dot2(p[3], xa.w, a64);
        a256 = dot2(p[4], xb.x, a256);
        a1 = dot2(p[5], xb.y, a1);
        a4 = dot2(p[6], xb.z, a4);
        a16 = dot2(p[7], xb.w, a16);
    }
    // explicit fma: the mixed and the one-width kernels inline this and must round it alike
    const float ux = fmaf(0x1p16f, a256, fmaf(0x1p18f, a64, fmaf(0x1p20f, a16, fmaf(0x1p22f, a4, 0x1p24f * a1))));
    return fmaf(-2.f, L.corr[jl], ux);
}

__device__ __forceinline__ void group2(WaveLds &L, uint32_t info, uint2 va, uint2 vb) {
    store_part(L, info, dot2bit(L, info >> 6, va, vb));
}

// 4-bit: a 16-byte half group (h = 0, 1) of column jl: sum u x / 2^24 over its 32 elements
__device__ __forceinline__ float half4bit(WaveLds &L, uint32_t jl, uint32_t h, uint2 va, uint2 vb) {
    const uint32_t w[4] = {va.x, va.y, vb.x, vb.y};
    const uint4 *xp = reinterpret_cast<const uint4 *>(L.xs + jl * kXStride + 16u * h);
    float a1 = 0.f, a16 = 0.f;
#pragma unroll
    for (uint32_t q = 0; q < 4; ++q) {
        uint32_t p[4];
        unpack4(w[q], p);
        const uint4 xa = xp[q];
        a1 = dot2(p[0], xa.x, a1);
        a16 = dot2(p[1], xa.y, a16);
        a1 = dot2(p[2], xa.z, a1);
        a16 = dot2(p[3], xa.w, a16);
    }
    return fmaf(0.0625f, a16, a1);
}

// the group's product from its two halves' sums (q = u - 8)
__device__ __forceinline__ float finish4bit(WaveLds &L, uint32_t jl, float halves) {
    return fmaf(-8.f, L.corr[jl], 0x1p24f * halves);
}

// 4-bit: lane pairs add their halves (h = lane & 1)
__device__ __forceinline__ void task4(WaveLds &L, uint32_t info, uint32_t h, uint2 va, uint2 vb) {
    const uint32_t jl = info >> 6;
    float part = half4bit(L, jl, h, va, vb);
    part += dpp<kQuadXor1>(part);
    if (h == 0) store_part(L, info, finish4bit(L, jl, part));
}

// 8-bit: a 16-byte quarter group (qd = 0..3) of column jl: sum u x / 2^24 over its 16 elements
__device__ __forceinline__ float quarter8bit(WaveLds &L, uint32_t jl, uint32_t qd, uint2 va, uint2 vb) {
    const uint32_t w[4] = {va.x, va.y, vb.x, vb.y};
    const uint4 *xp = reinterpret_cast<const uint4 *>(L.xs + jl * kXStride + 8u * qd);
    float a = 0.f;
#pragma unroll
    for (uint32_t q = 0; q < 2; ++q) {
        const uint4 xa = xp[q];
        uint32_t p0, p1, p2, p3;
        unpack8(w[2 * q], p0, p1);
        unpack8(w[2 * q + 1], p2, p3);
        a = dot2(p0, xa.x, a);
        a = dot2(p1, xa.y, a);
        a = dot2(p2, xa.z, a);
        a = dot2(p3, xa.w, a);
    }
    return a;
}

// the group's product from its quarters' sum (q = u - 128)
__device__ __forceinline__ float finish8bit(WaveLds &L, uint32_t jl, float quarters) {
    return fmaf(-128.f, L.corr[jl], 0x1p24f * quarters);
}

// 8-bit: lane quads add their quarters (qd = lane & 3)
__device__ __forceinline__ void task8(WaveLds &L, uint32_t info, uint32_t qd, uint2 va, uint2 vb) {
    const uint32_t jl = info >> 6;
    float a = quarter8bit(L, jl, qd, va, vb);
    a += dpp<kQuadXor1>(a);
    a += dpp<kQuadXor2>(a);
    if (qd == 0) store_part(L, info, finish8bit(L, jl, a));
}

// A width that is rare in a tile (a few 2- or 4-bit groups among 1-bit
// ones, as in a head tiered by frequency) leaves most lanes of its round
// idle, and the round costs the same instructions whatever the number of
// active lanes. Such a bucket is spread over more lanes per group: a 2-bit
// group over 2 lanes (two words each) or 4 (one word each), a 4-bit group
// over 4 (two words each), which cuts the round's instructions by about
// the same factor. The per-lane partials are added across the lanes with
// DPP quad permutes; the per-tile choice is uniform over the wave.

// 2-bit: the partial u x sum of kWords consecutive words from word w0 of a group of column jl
template <uint32_t kWords>
__device__ __forceinline__ float part2bit(WaveLds &L, uint32_t jl, uint32_t w0, const uint32_t w[kWords]) {
    const uint4 *xp = reinterpret_cast<const uint4 *>(L.xs + jl * kXStride) + 2u * w0;
    float a1 = 0.f, a4 = 0.f, a16 = 0.f, a64 = 0.f, a256 = 0.f;
#pragma unroll
    for (uint32_t q = 0; q < kWords; ++q) {
        uint32_t p[8];
        unpack2(w[q], p);
        const uint4 xa = xp[2 * q], xb = xp[2 * q + 1];
        a1 = dot2(p[0], xa.x, a1);
        a4 = dot2(p[1], xa.y, a4);
        a16 = dot2(p[2], xa.z, a16);
        a64 = dot2(p[3], xa.w, a64);
        a256 = dot2(p[4], xb.x, a256);
        a1 = dot2(p[5], xb.y, a1);
        a4 = dot2(p[6], xb.z, a4);
        a16 = dot2(p[7], xb.w, a16);
    }
    return fmaf(0x1p16f, a256, fmaf(0x1p18f, a64, fmaf(0x1p20f, a16, fmaf(0x1p22f, a4, 0x1p24f * a1))));
}

// 2-bit over two lanes: lane half h holds words 2h, 2h+1 (v)
__device__ __forceinline__ void task2h(WaveLds &L, uint32_t info, uint32_t h, uint2 v) {
    const uint32_t jl = info >> 6;
    const uint32_t w[2] = {v.x, v.y};
    float ux = part2bit<2>(L, jl, 2u * h, w);
    ux += dpp<kQuadXor1>(ux);
    if (h == 0) store_part(L, info, fmaf(-2.f, L.corr[jl], ux));
}

// 2-bit over four lanes: lane quarter qd holds word qd (v)
__device__ __forceinline__ void task2q(WaveLds &L, uint32_t info, uint32_t qd, uint32_t v) {
    const uint32_t jl = info >> 6;
    const uint32_t w[1] = {v};
    float ux = part2bit<1>(L, jl, qd, w);
    ux += dpp<kQuadXor1>(ux);
    ux += dpp<kQuadXor2>(ux);
    if (qd == 0) store_part(L, info, fmaf(-2.f, L.corr[jl], ux));
}

// 4-bit over four lanes: lane quarter qd holds words 2qd, 2qd+1 (elements 16qd .. 16qd+15)
__device__ __forceinline__ void task4q(WaveLds &L, uint32_t info, uint32_t qd, uint2 v) {
    const uint32_t jl = info >> 6;
    const uint32_t w[2] = {v.x, v.y};
    const uint4 *xp = reinterpret_cast<const uint4 *>(L.xs + jl * kXStride + 8u * qd);
    float a1 = 0.f, a16 = 0.f;
#pragma unroll
    for (uint32_t q = 0; q < 2; ++q) {
        uint32_t p[4];
        unpack4(w[q], p);
        const uint4 xa = xp[q];
        a1 = dot2(p[0], xa.x, a1);
        a16 = dot2(p[1], xa.y, a16);
        a1 = dot2(p[2], xa.z, a1);
        a16 = dot2(p[3], xa.w, a16);
    }
    float part = fmaf(0.0625f, a16, a1);
    part += dpp<kQuadXor1>(part);
    part += dpp<kQuadXor2>(part);
    if (qd == 0) store_part(L, info, finish4bit(L, jl, part));
}

// Lanes per group of a tile's 2-bit and 4-bit buckets, as shifts: 2 bits take 1, 2 or 4 lanes (s2 = 0,
// 1, 2), 4 bits 2 or 4 (s4 = 0, 1); a bucket that fits one round at the wider spread takes it.
struct Spread {
    uint32_t s2, s4;
};
__device__ __forceinline__ Spread tile_spread(const uint32_t cnt[4]) {
    return Spread{cnt[1] <= kWave / 4 ? 2u : cnt[1] <= kWave / 2 ? 1u : 0u, cnt[2] <= kWave / 4 ? 1u : 0u};
}

// Payload of the first 256 one-bit groups and of the first 64 slices of
// each wider bucket, loaded before any of it is used. A tile has at most
// 256 groups, so only the wider buckets can need more rounds. The addresses
// need only the per-width counts, so the loads leave before the lists exist.
struct Staged {
    uint2 p1[4];
    uint2 p2a, p2b, p4a, p4b, p8a, p8b;
};

// Every staged load is issued unconditionally through the tile's descriptor
// (base at the tile, bytes to the payload's end): a lane without a task
// reads later buckets or tiles, or zeros past the payload, and ignores them.
// With a fixed number of loads the compiler waits for exactly these and not
// for the next tile's metadata issued after them.
__device__ __forceinline__ void stage_payload(rsrc_t tile, const uint32_t cnt[4], uint32_t lane, Staged &S) {
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i) S.p1[i] = buf_load8(tile, 8u * lane + 8u * kWave * i);
    const uint32_t o2 = 8u * cnt[0], o4 = o2 + 16u * cnt[1], o8 = o4 + 32u * cnt[2];
    S.p2a = buf_load8(tile, o2 + 16u * lane);
    S.p2b = buf_load8(tile, o2 + 16u * lane + 8u);
    S.p4a = buf_load8(tile, o4 + 16u * lane);
    S.p4b = buf_load8(tile, o4 + 16u * lane + 8u);
    S.p8a = buf_load8(tile, o8 + 16u * lane);
    S.p8b = buf_load8(tile, o8 + 16u * lane + 8u);
}

// stage_payload with the 2- and 4-bit buckets read at their spread (tile_spread): a lane's bytes of
// a 2-bit bucket start at 16, 8 or 4 bytes per lane, of a 4-bit bucket at 16 or 8 (the same loads
// every time; the second 8 bytes are used only at the one-lane and two-lane spreads)
__device__ __forceinline__ void stage_payload_spread(rsrc_t tile, const uint32_t cnt[4], Spread sp, uint32_t lane,
                                                     Staged &S) {
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i) S.p1[i] = buf_load8(tile, 8u * lane + 8u * kWave * i);
    const uint32_t o2 = 8u * cnt[0], o4 = o2 + 16u * cnt[1], o8 = o4 + 32u * cnt[2];
    const uint32_t a2 = o2 + ((16u * lane) >> sp.s2), a4 = o4 + ((16u * lane) >> sp.s4);
    S.p2a = buf_load8(tile, a2);
    S.p2b = buf_load8(tile, a2 + 8u);
    S.p4a = buf_load8(tile, a4);
    S.p4b = buf_load8(tile, a4 + 8u);
    S.p8a = buf_load8(tile, o8 + 16u * lane);
    S.p8b = buf_load8(tile, o8 + 16u * lane + 8u);
}

// Staged work first, then the rounds that load their own bytes (rare: more than 64 two-bit groups or 64
// slices of a wider width in one tile); the 2- and 4-bit rounds at the tile's spread (a spread bucket
// fits its one staged round).
__device__ __forceinline__ void tile_products(WaveLds &L, const Staged &S, rsrc_t tile, const uint32_t cnt[4],
                                              Spread sp, uint32_t lane, LutKeys keys) {
    // A lane without a group in a round parks its (unused) result in a spare
    // slot past L.part, so the deferred stores need no branches.
    uint32_t info1[4];
    float v1[4];
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i) {
        const bool on = lane + kWave * i < cnt[0];
        const uint32_t e = L.list[lane + kWave * i];
        info1[i] = on ? e : kTileGroups * kTileRows + lane;
        v1[i] = 0.f;
        if (on) v1[i] = group1(L, e, S.p1[i], keys);
    }
    // the lookup table is dead from here: its bytes take the products
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i) store_part(L, info1[i], v1[i]);
    const uint32_t o2 = 8u * cnt[0], o4 = o2 + 16u * cnt[1], o8 = o4 + 32u * cnt[2];
    const uint8_t *l2 = L.list + cnt[0], *l4 = l2 + cnt[1], *l8 = l4 + cnt[2];
    if (sp.s2 == 2) {
        if (lane < 4u * cnt[1]) task2q(L, l2[lane >> 2], lane & 3u, S.p2a.x);
    } else if (sp.s2 == 1) {
        if (lane < 2u * cnt[1]) task2h(L, l2[lane >> 1], lane & 1u, S.p2a);
    } else {
        if (lane < cnt[1]) group2(L, l2[lane], S.p2a, S.p2b);
        for (uint32_t e = lane + kWave; e < cnt[1]; e += kWave)
            group2(L, l2[e], buf_load8(tile, o2 + 16u * e), buf_load8(tile, o2 + 16u * e + 8u));
    }
    if (sp.s4 == 1) {
        if (lane < 4u * cnt[2]) task4q(L, l4[lane >> 2], lane & 3u, S.p4a);
    } else {
        if (lane < 2u * cnt[2]) task4(L, l4[lane >> 1], lane & 1u, S.p4a, S.p4b);
        for (uint32_t e = lane + kWave; e < 2u * cnt[2]; e += kWave)
            task4(L, l4[e >> 1], e & 1u, buf_load8(tile, o4 + 16u * e), buf_load8(tile, o4 + 16u * e + 8u));
    }
    if (lane < 4u * cnt[3]) task8(L, l8[lane >> 2], lane & 3u, S.p8a, S.p8b);
    for (uint32_t e = lane + kWave; e < 4u * cnt[3]; e += kWave)
        task8(L, l8[e >> 2], e & 3u, buf_load8(tile, o8 + 16u * e), buf_load8(tile, o8 + 16u * e + 8u));
}

// fp16 bits of silu(g) * u = g * u / (1 + e^-g), rounded to nearest even (beyond the fp16 range: +-inf)
__device__ __forceinline__ uint16_t swiglu_half(float g, float u) {
    const float v = g * u / (1.f + expf(-g));
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}

// Gated-MLP epilogue of one finished row tile (wave 0 of the tile's last
// workgroup; which = 0 for gate, 1 for up): publish the tile's values, count
// arrivals per row tile; the second of the two tiles reads the other's values
// and writes h, then resets the counter. Same publication protocol as the
// split-K partial sums.
__device__ __forceinline__ void swiglu_pair(const Batch &B, uint32_t which, uint32_t a, uint32_t row, bool live,
                                            uint32_t n, uint32_t lane, float v) {
    if (live) __hip_atomic_store(&B.pair[static_cast<uint64_t>(which) * n + row], v, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    uint32_t arrived = 0;
    if (lane == 0) arrived = __hip_atomic_fetch_add(&B.pair_counters[a * kCounterStride], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    arrived = __shfl(arrived, 0, kWave);
    if (arrived != 1) return;
    if (live) {
        const float o = __hip_atomic_load(&B.pair[static_cast<uint64_t>(1 - which) * n + row], __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
        B.h[row] = which == 0 ? swiglu_half(v, o) : swiglu_half(o, v);
    }
    if (lane == 0) __hip_atomic_store(&B.pair_counters[a * kCounterStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The workgroup's row sums (waves added in wave order), the split-K
// reduction when the row tile is split, then y or the gated-MLP epilogue.
template <uint32_t kWaves>
__device__ __forceinline__ void finish_row_tile(const Batch &B, const MatArgs &M, uint32_t which, WaveLds *lds,
                                                uint32_t wave, bool spare, uint32_t a, uint32_t split, uint32_t r0,
                                                uint32_t rows, uint32_t lane, float acc) {
    // a grouped head's output row, requested before the barrier so that the load's trip overlaps it
    uint32_t out_row = r0 + lane;
    if (B.row_map && wave == 0) {
        uint32_t rank0 = 0;
        for (uint32_t j = 0; j < which; ++j) rank0 += B.m[j].n;
        out_row = B.row_map[rank0 + r0 + min(lane, rows - 1)];
    }
    lds[wave].part[lane] = acc;   // the wave's row sums, in its own (now idle) LDS
    __syncthreads();
    if (wave != 0 || spare) return;
    float sum = lds[0].part[lane];
#pragma unroll
    for (uint32_t w = 1; w < kWaves; ++w) sum += lds[w].part[lane];   // in wave order
    if (M.splits > 1) {
        // Split row tile: publish the partial sums with device-scope stores, wait
        // until they have completed, then count arrivals; the last workgroup reads
        // them with device-scope loads, adds them in split order and resets the
        // counter for the next call. No cache holds an older copy of another
        // split's partials: each line is written only by its split in this launch
        // and read only by the last arriver, and caches are invalidated between
        // launches. (Agent-scope release/acquire fences would write back and
        // invalidate a whole L2 per workgroup: about 4 us per split launch.)
        if (lane < rows)
            __hip_atomic_store(&M.partial[static_cast<uint64_t>(split) * M.n + r0 + lane], sum, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        uint32_t arrived = 0;
        if (lane == 0)
            arrived = __hip_atomic_fetch_add(&M.counters[a * kCounterStride], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        arrived = __shfl(arrived, 0, kWave);
        if (arrived != M.splits - 1) return;
        if (lane < rows) sum = sum_partials(M.partial + r0 + lane, M.n, M.splits);
        if (lane == 0) __hip_atomic_store(&M.counters[a * kCounterStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!B.h) {
        if (lane < rows) {
            if (B.row_map) {
                if (out_row < B.y_rows) M.y[out_row] = sum;
            } else if (M.y16) {
                M.y16[r0 + lane] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(sum));
            } else {
                M.y[r0 + lane] = sum;
            }
        }
        return;
    }
    swiglu_pair(B, which, a, r0 + lane, lane < rows, M.n, lane, sum);
}

// A tile's entry in the stream index: the list bytes 4 lane .. 4 lane + 3 and
// the per-width counts (uniform, a scalar load like the tile offset).
struct TileIndex {
    uint32_t list4;
    uint32_t c01, c23;   // counts of width codes 0 | 1 << 16, 2 | 3 << 16
};

__device__ __forceinline__ TileIndex load_index(const MatArgs &M, uint32_t tile, uint32_t lane) {
    TileIndex t;
    t.list4 = reinterpret_cast<const uint32_t *>(M.index + 256ull * tile)[lane];
    const uint64_t tiles = static_cast<uint64_t>((M.n + kTileRows - 1) / kTileRows) * M.col_tiles;
    typedef const __attribute__((address_space(4))) uint32_t *const_u32p;
    const const_u32p c = (const_u32p)(reinterpret_cast<uintptr_t>(M.index + 256ull * tiles));
    t.c01 = c[2ull * tile];
    t.c23 = c[2ull * tile + 1];
    return t;
}

// The counts of an index entry, each held to what is left of the tile's 256
// groups, so that a damaged index cannot move a bucket past the list.
__device__ __forceinline__ void index_counts(const TileIndex &t, uint32_t cnt[4]) {
    const uint32_t c0 = min(t.c01 & 0xFFFFu, 256u);
    const uint32_t c1 = min(t.c01 >> 16, 256u - c0);
    const uint32_t c2 = min(t.c23 & 0xFFFFu, 256u - c0 - c1);
    cnt[0] = c0;
    cnt[1] = c1;
    cnt[2] = c2;
    cnt[3] = min(t.c23 >> 16, 256u - c0 - c1 - c2);
}

// kWaves waves per workgroup (4, 8 or 16) share one row tile; the LDS
// (4992 B per wave) allows 8, 4 or 2 such workgroups per CU, eight waves
// per SIMD, and the registers are held to the 64 that allow the same.
// kExit: the launch's matrices differ in size, so workgroups past a smaller matrix's end leave at once
// (all seven 9B-layer matrices in one launch: 32.9 -> 23.7 us); launches of equal matrices have none and
// skip the test, which would put a dependent load ahead of the others (about 0.7 us a step).
// kIndexed: every matrix of the launch has a stream index; a tile's counts and list are read from it
// instead of being derived from the width codes (the scan and list build, about 80 VALU per tile).
template <bool kAligned, uint32_t kWaves, bool kExit, bool kIndexed>
__global__ __launch_bounds__(kWaves * kWave) __attribute__((amdgpu_waves_per_eu(8, 8))) void gemv_tiles(Batch B) {
    __shared__ WaveLds lds[kWaves];
    // which matrix, row tile and split this block serves (uniform)
    const MatArgs M = B.m[blockIdx.y];   // by value: loaded into scalar registers once
    // The grid is as wide as the largest matrix of the launch. A block past
    // its matrix's end repeats the matrix's last block and stores nothing:
    // testing first would put a dependent load ahead of the others.
    if (kExit && blockIdx.x >= M.blocks) return;
    const bool spare = !kExit && blockIdx.x >= M.blocks;
    const uint32_t bx = spare ? M.blocks - 1 : blockIdx.x;
    const uint32_t a = bx / M.splits, split = bx % M.splits;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x) / kWave;   // uniform
    const uint32_t r0 = a * kTileRows;
    const uint32_t rows = min(kTileRows, M.n - r0);
    const uint32_t c_lo = (split * M.col_tiles) / M.splits, c_hi = ((split + 1) * M.col_tiles) / M.splits;
    WaveLds &L = lds[wave];
    float acc = 0.f;
    const uint32_t lane0 = lane_id();
    const LutKeys keys = lut_keys();
    uint32_t ct = c_lo + wave;
    // metadata loads are unconditional (a wave without a next tile reloads its
    // own): a conditional load would make its result a branch merge, and the
    // merge copy would wait for the load
    const uint32_t ct0 = ct < c_hi ? ct : c_lo;
    TileMeta cur = load_meta<kAligned>(M, a, ct0, relane(lane0), true, !kIndexed);
    TileIndex cix{};
    if constexpr (kIndexed) cix = load_index(M, a * M.col_tiles + ct0, relane(lane0));
    for (; ct < c_hi; ct += kWaves) {
        const uint32_t cn = kAligned ? kTileGroups : min(kTileGroups, M.groups - ct * kTileGroups);
        // counts first: the payload loads leave before the tables and lists are built
        uint32_t cnt[4];
        TileScan P;
        if constexpr (kIndexed)
            index_counts(cix, cnt);
        else
            P = tile_scan(cur, rows, cn, relane(lane0), cnt);
        const rsrc_t tp = tile_rsrc(M.payload, M.payload_bytes, cur.off);
        const Spread sp = tile_spread(cnt);
        Staged S;
        stage_payload_spread(tp, cnt, sp, relane(lane0), S);
        // the next tile's metadata travels while this tile computes
        const uint32_t cnx = ct + kWaves < c_hi ? ct + kWaves : ct;
        const TileMeta nxt = load_meta<kAligned>(M, a, cnx, relane(lane0), true, !kIndexed);
        TileIndex nix{};
        if constexpr (kIndexed) nix = load_index(M, a * M.col_tiles + cnx, relane(lane0));
        stage_x(L, cur.xv, relane(lane0));
        if constexpr (kIndexed)
            reinterpret_cast<uint32_t *>(L.list)[relane(lane0)] = cix.list4;
        else
            build_lists(L, cur, P, cnt, rows, cn, relane(lane0));
        wave_lds_sync();
        tile_products(L, S, tp, cnt, sp, relane(lane0), keys);
        wave_lds_sync();
        const uint32_t lane = relane(lane0);
        if (lane < rows)
            for (uint32_t jl = 0; jl < cn; ++jl) {
                const uint32_t sb = (jl < 2 ? cur.s01 >> (16 * jl) : cur.s23 >> (16 * (jl - 2))) & 0xFFFFu;
                acc = fmaf(half_to_float(sb), L.part[jl * kTileRows + lane], acc);
            }
        wave_lds_sync();
        cur = nxt;
        if constexpr (kIndexed) cix = nix;
    }
    finish_row_tile<kWaves>(B, M, blockIdx.y, lds, wave, spare, a, split, r0, rows, relane(lane0), acc);
}

// ---------------------------------------------------------------- several rows of X
// Small batches: a wave decodes each tile once and multiplies it by kR = 2
// rows of X, so the per-tile work that does not depend on x (metadata,
// counts, list, payload loads, field masks, the 1-bit lookup addresses) is
// shared by the rows. Each row has its own staged activations, lookup table
// and products in LDS (the single-row layout, kR times), and per row the
// arithmetic is the single-row kernel's, in the same order. x row r is at
// x + r k and y row r at y + r n.
template <uint32_t kR>
struct alignas(64) RowsLds {
    union {
        float lut[kR][16 * kTileGroups * 16];             // per row: the single-row table layout
        float part[kR][kTileGroups * kTileRows + kWave];  // per row: products, then one spare slot per lane
    };
    uint32_t xs[kR][kTileGroups * kXStride];
    float corr[kR][kTileGroups];
    uint8_t list[kTileRows * kTileGroups];
};

// Activations 4k..4k+3 of column lane/16 (k = lane % 16) of each row, as load_meta loads one row's
template <bool kAligned, uint32_t kR>
__device__ __forceinline__ void load_x_rows(const MatArgs &M, uint32_t ct, uint32_t lane, uint2 xv[kR]) {
    const uint32_t j0 = ct * kTileGroups, cn = kAligned ? kTileGroups : min(kTileGroups, M.groups - j0);
    const uint32_t jl = min(lane >> 4, cn - 1), k = lane & 15;
    const uint32_t xoff = 128u * (j0 + jl) + 8u * k;
    const uint64_t row_bytes = 128ull * M.groups;
#pragma unroll
    for (uint32_t r = 0; r < kR; ++r)
        xv[r] = *reinterpret_cast<const uint2 *>(reinterpret_cast<const char *>(M.x) + r * row_bytes + xoff);
}

// 1-bit group of column info >> 6 for every row: the table offsets are formed once (as in group1) and
// each row reads its own table, 4 KiB further on
template <uint32_t kR>
__device__ __forceinline__ void group1_rows(RowsLds<kR> &L, uint32_t info, uint2 v, LutKeys keys, float out[kR]) {
    const uint32_t jl = info >> 6;
    const char *lut = reinterpret_cast<const char *>(L.lut[0] + jl * 16u);
    const uint32_t w[2] = {v.x, v.y};
    float acc[kR][4];
#pragma unroll
    for (uint32_t q = 0; q < 2; ++q) {
        uint32_t lo, hi;
        asm("v_lshlrev_b32 %0, 2, %1\n\tv_bitop3_b32 %0, %0, %2, %3 bitop3:0x6a"
            : "=&v"(lo) : "v"(w[q]), "v"(keys.mask), "v"(keys.swz));
        asm("v_lshrrev_b32 %0, 2, %1\n\tv_bitop3_b32 %0, %0, %2, %3 bitop3:0x6a"
            : "=&v"(hi) : "v"(w[q]), "v"(keys.mask), "v"(keys.swz));
#pragma unroll
        for (uint32_t t = 0; t < 4; ++t) {
            const uint32_t k = 8 * q + 2 * t;
            const char *pa = lut + 256u * k + ((lo >> (8 * t)) & 0xFFu);
            const char *pb = lut + 256u * (k + 1) + ((hi >> (8 * t)) & 0xFFu);
#pragma unroll
            for (uint32_t r = 0; r < kR; ++r) {
                const float a = *reinterpret_cast<const float *>(pa + sizeof(L.lut[0]) * r);
                const float b = *reinterpret_cast<const float *>(pb + sizeof(L.lut[0]) * r);
                acc[r][t] = q == 0 ? a + b : acc[r][t] + (a + b);
            }
        }
    }
#pragma unroll
    for (uint32_t r = 0; r < kR; ++r) {
        const float sum = (acc[r][0] + acc[r][1]) + (acc[r][2] + acc[r][3]);
        out[r] = L.corr[r][jl] - 2.f * sum;
    }
}

// 2-bit group: each word unpacked once, then dotted with every row (dot2bit's order per row)
template <uint32_t kR>
__device__ __forceinline__ void group2_rows(RowsLds<kR> &L, uint32_t info, uint2 va, uint2 vb) {
    const uint32_t jl = info >> 6;
    const uint32_t w[4] = {va.x, va.y, vb.x, vb.y};
    float a1[kR], a4[kR], a16[kR], a64[kR], a256[kR];
#pragma unroll
    for (uint32_t r = 0; r < kR; ++r) a1[r] = a4[r] = a16[r] = a64[r] = a256[r] = 0.f;
#pragma unroll
    for (uint32_t q = 0; q < 4; ++q) {
        uint32_t p[8];
        unpack2(w[q], p);
#pragma unroll
        for (uint32_t r = 0; r < kR; ++r) {
            const uint4 *xp = reinterpret_cast<const uint4 *>(L.xs[r] + jl * kXStride);
            const uint4 xa = xp[2 * q], xb = xp[2 * q + 1];
            a1[r] = dot2(p[0], xa.x, a1[r]);
            a4[r] = dot2(p[1], xa.y, a4[r]);
            a16[r] = dot2(p[2], xa.z, a16[r]);
            a64[r] = dot2(p[3], xa.w, a64[r]);
            a256[r] = dot2(p[4], xb.x, a256[r]);
            a1[r] = dot2(p[5], xb.y, a1[r]);
            a4[r] = dot2(p[6], xb.z, a4[r]);
            a16[r] = dot2(p[7], xb.w, a16[r]);
        }
    }
#pragma unroll
    for (uint32_t r = 0; r < kR; ++r) {
        const float ux = fmaf(0x1p16f, a256[r],
                              fmaf(0x1p18f, a64[r], fmaf(0x1p20f, a16[r], fmaf(0x1p22f, a4[r], 0x1p24f * a1[r]))));
        L.part[r][info] = fmaf(-2.f, L.corr[r][jl], ux);
    }
}

// 4-bit half group h of every row; lane pairs add their halves (task4's order per row)
template <uint32_t kR>
__device__ __forceinline__ void task4_rows(RowsLds<kR> &L, uint32_t info, uint32_t h, uint2 va, uint2 vb) {
    const uint32_t jl = info >> 6;
    const uint32_t w[4] = {va.x, va.y, vb.x, vb.y};
    float a1[kR], a16[kR];
#pragma unroll
    for (uint32_t r = 0; r < kR; ++r) a1[r] = a16[r] = 0.f;
#pragma unroll
    for (uint32_t q = 0; q < 4; ++q) {
        uint32_t p[4];
        unpack4(w[q], p);
#pragma unroll
        for (uint32_t r = 0; r < kR; ++r) {
            const uint4 xa = reinterpret_cast<const uint4 *>(L.xs[r] + jl * kXStride + 16u * h)[q];
            a1[r] = dot2(p[0], xa.x, a1[r]);
            a16[r] = dot2(p[1], xa.y, a16[r]);
            a1[r] = dot2(p[2], xa.z, a1[r]);
            a16[r] = dot2(p[3], xa.w, a16[r]);
        }
    }
#pragma unroll
    for (uint32_t r = 0; r < kR; ++r) {
        float part = fmaf(0.0625f, a16[r], a1[r]);
        part += dpp<kQuadXor1>(part);
        if (h == 0) L.part[r][info] = fmaf(-8.f, L.corr[r][jl], 0x1p24f * part);
    }
}

// 8-bit quarter group qd of every row; lane quads add their quarters (task8's order per row)
template <uint32_t kR>
__device__ __forceinline__ void task8_rows(RowsLds<kR> &L, uint32_t info, uint32_t qd, uint2 va, uint2 vb) {
    const uint32_t jl = info >> 6;
    const uint32_t w[4] = {va.x, va.y, vb.x, vb.y};
    float a[kR];
#pragma unroll
    for (uint32_t r = 0; r < kR; ++r) a[r] = 0.f;
#pragma unroll
    for (uint32_t q = 0; q < 2; ++q) {
        uint32_t p0, p1, p2, p3;
        unpack8(w[2 * q], p0, p1);
        unpack8(w[2 * q + 1], p2, p3);
#pragma unroll
        for (uint32_t r = 0; r < kR; ++r) {
            const uint4 xa = reinterpret_cast<const uint4 *>(L.xs[r] + jl * kXStride + 8u * qd)[q];
            a[r] = dot2(p0, xa.x, a[r]);
            a[r] = dot2(p1, xa.y, a[r]);
            a[r] = dot2(p2, xa.z, a[r]);
            a[r] = dot2(p3, xa.w, a[r]);
        }
    }
#pragma unroll
    for (uint32_t r = 0; r < kR; ++r) {
        float v = a[r];
        v += dpp<kQuadXor1>(v);
        v += dpp<kQuadXor2>(v);
        if (qd == 0) L.part[r][info] = fmaf(-128.f, L.corr[r][jl], 0x1p24f * v);
    }
}

// tile_products for kR rows: the same rounds and the same staged loads
template <uint32_t kR>
__device__ __forceinline__ void tile_products_rows(RowsLds<kR> &L, const Staged &S, rsrc_t tile, const uint32_t cnt[4],
                                                   uint32_t lane, LutKeys keys) {
    uint32_t info1[4];
    float v1[4][kR];
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i) {
        const bool on = lane + kWave * i < cnt[0];
        const uint32_t e = L.list[lane + kWave * i];
        info1[i] = on ? e : kTileGroups * kTileRows + lane;
#pragma unroll
        for (uint32_t r = 0; r < kR; ++r) v1[i][r] = 0.f;
        if (on) group1_rows<kR>(L, e, S.p1[i], keys, v1[i]);
    }
    // the lookup tables are dead from here: their bytes take the products
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i)
#pragma unroll
        for (uint32_t r = 0; r < kR; ++r) L.part[r][info1[i]] = v1[i][r];
    const uint32_t o2 = 8u * cnt[0], o4 = o2 + 16u * cnt[1], o8 = o4 + 32u * cnt[2];
    const uint8_t *l2 = L.list + cnt[0], *l4 = l2 + cnt[1], *l8 = l4 + cnt[2];
    if (lane < cnt[1]) group2_rows<kR>(L, l2[lane], S.p2a, S.p2b);
    if (lane < 2u * cnt[2]) task4_rows<kR>(L, l4[lane >> 1], lane & 1u, S.p4a, S.p4b);
    if (lane < 4u * cnt[3]) task8_rows<kR>(L, l8[lane >> 2], lane & 3u, S.p8a, S.p8b);
    for (uint32_t e = lane + kWave; e < cnt[1]; e += kWave)
        group2_rows<kR>(L, l2[e], buf_load8(tile, o2 + 16u * e), buf_load8(tile, o2 + 16u * e + 8u));
    for (uint32_t e = lane + kWave; e < 2u * cnt[2]; e += kWave)
        task4_rows<kR>(L, l4[e >> 1], e & 1u, buf_load8(tile, o4 + 16u * e), buf_load8(tile, o4 + 16u * e + 8u));
    for (uint32_t e = lane + kWave; e < 4u * cnt[3]; e += kWave)
        task8_rows<kR>(L, l8[e >> 2], e & 3u, buf_load8(tile, o8 + 16u * e), buf_load8(tile, o8 + 16u * e + 8u));
}

// The workgroup's row sums per row of X (waves in wave order), the split-K
// reduction (one arrival count per row tile for all the rows; partial sums
// of row r and split s at partial[(r * splits + s) * n]), then y.
template <uint32_t kWaves, uint32_t kR>
__device__ __forceinline__ void finish_rows(const MatArgs &M, RowsLds<kR> *lds, uint32_t wave, uint32_t a,
                                            uint32_t split, uint32_t r0, uint32_t rows, uint32_t lane,
                                            const float acc[kR]) {
#pragma unroll
    for (uint32_t r = 0; r < kR; ++r) lds[wave].part[r][lane] = acc[r];
    __syncthreads();
    if (wave != 0) return;
    float sum[kR];
#pragma unroll
    for (uint32_t r = 0; r < kR; ++r) {
        sum[r] = lds[0].part[r][lane];
#pragma unroll
        for (uint32_t w = 1; w < kWaves; ++w) sum[r] += lds[w].part[r][lane];   // in wave order
    }
    if (M.splits > 1) {
        // the split-K publication protocol of finish_row_tile, for every row of X
        if (lane < rows) {
#pragma unroll
            for (uint32_t r = 0; r < kR; ++r)
                __hip_atomic_store(&M.partial[(static_cast<uint64_t>(r) * M.splits + split) * M.n + r0 + lane],
                                   sum[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        uint32_t arrived = 0;
        if (lane == 0)
            arrived = __hip_atomic_fetch_add(&M.counters[a * kCounterStride], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        arrived = __shfl(arrived, 0, kWave);
        if (arrived != M.splits - 1) return;
        if (lane < rows) {
#pragma unroll
            for (uint32_t r = 0; r < kR; ++r)
                sum[r] = sum_partials(M.partial + static_cast<uint64_t>(r) * M.splits * M.n + r0 + lane, M.n,
                                      M.splits);
        }
        if (lane == 0) __hip_atomic_store(&M.counters[a * kCounterStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (lane < rows) {
#pragma unroll
        for (uint32_t r = 0; r < kR; ++r) M.y[static_cast<uint64_t>(r) * M.n + r0 + lane] = sum[r];
    }
}

// kR rows of X per wave. The LDS (kR times the single-row layout) allows
// 8 / kR waves per SIMD, so the registers may grow to match. Workgroups past
// their matrix's end leave at once.
template <bool kAligned, uint32_t kWaves, uint32_t kR>
__global__ __launch_bounds__(kWaves * kWave) __attribute__((amdgpu_waves_per_eu(8 / kR, 8 / kR))) void gemv_rows(
    Batch B) {
    __shared__ RowsLds<kR> lds[kWaves];
    const MatArgs M = B.m[blockIdx.y];
    if (blockIdx.x >= M.blocks) return;
    const uint32_t a = blockIdx.x / M.splits, split = blockIdx.x % M.splits;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x) / kWave;
    const uint32_t r0 = a * kTileRows;
    const uint32_t rows = min(kTileRows, M.n - r0);
    const uint32_t c_lo = (split * M.col_tiles) / M.splits, c_hi = ((split + 1) * M.col_tiles) / M.splits;
    RowsLds<kR> &L = lds[wave];
    float acc[kR];
#pragma unroll
    for (uint32_t r = 0; r < kR; ++r) acc[r] = 0.f;
    const uint32_t lane0 = lane_id();
    const LutKeys keys = lut_keys();
    uint32_t ct = c_lo + wave;
    TileMeta cur = load_meta<kAligned>(M, a, ct < c_hi ? ct : c_lo, relane(lane0), false);
    uint2 xc[kR];
    load_x_rows<kAligned, kR>(M, ct < c_hi ? ct : c_lo, relane(lane0), xc);
    for (; ct < c_hi; ct += kWaves) {
        const uint32_t cn = kAligned ? kTileGroups : min(kTileGroups, M.groups - ct * kTileGroups);
        uint32_t cnt[4];
        const TileScan P = tile_scan(cur, rows, cn, relane(lane0), cnt);
        const rsrc_t tp = tile_rsrc(M.payload, M.payload_bytes, cur.off);
        Staged S;
        stage_payload(tp, cnt, relane(lane0), S);
        const uint32_t cnx = ct + kWaves < c_hi ? ct + kWaves : ct;
        const TileMeta nxt = load_meta<kAligned>(M, a, cnx, relane(lane0), false);
        uint2 xn[kR];
        load_x_rows<kAligned, kR>(M, cnx, relane(lane0), xn);
#pragma unroll
        for (uint32_t r = 0; r < kR; ++r) stage_x_at(L.lut[r], L.xs[r], L.corr[r], xc[r], relane(lane0));
        build_lists(L, cur, P, cnt, rows, cn, relane(lane0));
        wave_lds_sync();
        tile_products_rows<kR>(L, S, tp, cnt, relane(lane0), keys);
        wave_lds_sync();
        const uint32_t lane = relane(lane0);
        if (lane < rows)
            for (uint32_t jl = 0; jl < cn; ++jl) {
                const uint32_t sb = (jl < 2 ? cur.s01 >> (16 * jl) : cur.s23 >> (16 * (jl - 2))) & 0xFFFFu;
#pragma unroll
                for (uint32_t r = 0; r < kR; ++r)
                    acc[r] = fmaf(half_to_float(sb), L.part[r][jl * kTileRows + lane], acc[r]);
            }
        wave_lds_sync();
        cur = nxt;
#pragma unroll
        for (uint32_t r = 0; r < kR; ++r) xc[r] = xn[r];
    }
    finish_rows<kWaves, kR>(M, lds, wave, a, split, r0, rows, relane(lane0), acc);
}

// ---------------------------------------------------------------- uniform width
// Every group of the matrix has width kBits (the deployed recipe stores whole
// projections at one width). A tile is then a single bucket: group (jl, r)
// sits (jl * rows + r) * 8 * kBits bytes into its tile, and the tile sits at
// 8 * kBits * (r0 * G + rows * 4 * ct). No width codes, offset table, scan or
// lists are needed. A lane owns its row: it loads the row's groups of the
// tile, forms each product with the mixed kernel's decoders and adds it,
// scaled, into its own row sum.
template <uint32_t kBits>
struct RowGroups {
    uint4 v[kBits == 1 ? 1 : kBits / 2];   // 8 * kBits bytes (1 bit: the low 8 bytes)
};

template <uint32_t kBits>
__device__ __forceinline__ RowGroups<kBits> load_row_group(rsrc_t tile, uint32_t off) {
    RowGroups<kBits> g;
    if (kBits == 1) {
        const uint2 v = buf_load8(tile, off);
        g.v[0] = make_uint4(v.x, v.y, 0u, 0u);
    } else {
#pragma unroll
        for (uint32_t i = 0; i < kBits / 2; ++i) g.v[i] = buf_load16x(tile, off + 16u * i);
    }
    return g;
}

template <uint32_t kBits>
__device__ __forceinline__ float row_group_dot(WaveLds &L, uint32_t jl, const RowGroups<kBits> &g, LutKeys keys) {
    if constexpr (kBits == 1) return group1(L, jl << 6, make_uint2(g.v[0].x, g.v[0].y), keys);
    else if constexpr (kBits == 2) return dot2bit(L, jl, make_uint2(g.v[0].x, g.v[0].y), make_uint2(g.v[0].z, g.v[0].w));
    else if constexpr (kBits == 4)
        return finish4bit(L, jl, half4bit(L, jl, 0, make_uint2(g.v[0].x, g.v[0].y), make_uint2(g.v[0].z, g.v[0].w)) +
                                     half4bit(L, jl, 1, make_uint2(g.v[1].x, g.v[1].y), make_uint2(g.v[1].z, g.v[1].w)));
    else {
        // quarters added as the mixed kernel's lane quads add them, so both kernels give the same bits
        float q[4];
#pragma unroll
        for (uint32_t i = 0; i < 4; ++i)
            q[i] = quarter8bit(L, jl, i, make_uint2(g.v[i].x, g.v[i].y), make_uint2(g.v[i].z, g.v[i].w));
        return finish8bit(L, jl, (q[0] + q[1]) + (q[2] + q[3]));
    }
}

// kLean: hold two 4-bit groups of a row at once instead of four (the per-matrix-width kernel, whose
// register budget is the largest of its four paths plus the dispatch). kChunkUnits: a wave's unit of
// work along K is the groups it holds at once (the per-matrix-width kernel), else a whole tile.
template <uint32_t kBits, bool kAligned, uint32_t kWaves, bool kLean = false, bool kChunkUnits = false>
__device__ __forceinline__ void uniform_tiles(const Batch &B, const MatArgs &M, uint32_t which, uint32_t bx,
                                              WaveLds *lds) {
    // A workgroup past its matrix's end leaves at once: with matrices of very different sizes in one
    // launch (a head grouped by width) repeating the last row tile would multiply the work.
    if (bx >= M.blocks) return;
    const bool spare = false;
    const uint32_t a = bx / M.splits, split = bx % M.splits;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x) / kWave;
    const uint32_t r0 = a * kTileRows;
    const uint32_t rows = min(kTileRows, M.n - r0);
    WaveLds &L = lds[wave];
    float acc = 0.f;
    const uint32_t lane0 = lane_id();
    const LutKeys keys = lut_keys();
    constexpr uint32_t kChunk = kBits == 8 ? 1 : (kBits == 4 && kLean) ? 2 : kTileGroups;   // groups held at once
    // A wave's unit of work: a whole tile, or with kChunkUnits the groups it holds at once (8 bits: one,
    // lean 4 bits: two), so that it waits for its payload once per unit; M.units counts them along K.
    constexpr uint32_t kUnit = kChunkUnits ? kChunk : kTileGroups;
    const uint32_t u_lo = (split * M.units) / M.splits, u_hi = ((split + 1) * M.units) / M.splits;
    uint32_t u = u_lo + wave;
    TileMeta cur = load_meta<kAligned>(M, a, (u < u_hi ? u : u_lo) * kUnit / kTileGroups, relane(lane0), true);
    for (; u < u_hi; u += kWaves) {
        const uint32_t ct = u * kUnit / kTileGroups, g0 = u * kUnit % kTileGroups;   // tile, first group
        const uint32_t cn = kAligned ? kTileGroups : min(kTileGroups, M.groups - ct * kTileGroups);
        const uint32_t lr = min(relane(lane0), rows - 1);
        const uint32_t tile_off = 8u * kBits * (r0 * M.groups + rows * kTileGroups * ct);
        const rsrc_t tp = tile_rsrc(M.payload, M.payload_bytes, tile_off);
        RowGroups<kBits> g[kChunk];
#pragma unroll
        for (uint32_t jl = 0; jl < kChunk; ++jl)
            g[jl] = load_row_group<kBits>(tp, (min(g0 + jl, cn - 1) * rows + lr) * 8u * kBits);
        const TileMeta nxt = load_meta<kAligned>(
            M, a, (u + kWaves < u_hi ? u + kWaves : u) * kUnit / kTileGroups, relane(lane0), true);
        stage_x<kBits == 1>(L, cur.xv, relane(lane0));
        wave_lds_sync();
        const uint32_t lane = relane(lane0);
#pragma unroll
        for (uint32_t c0 = 0; c0 < kUnit; c0 += kChunk) {
            if (c0 > 0) {
#pragma unroll
                for (uint32_t jl = 0; jl < kChunk; ++jl)
                    g[jl] = load_row_group<kBits>(tp, (min(g0 + c0 + jl, cn - 1) * rows + lr) * 8u * kBits);
            }
#pragma unroll
            for (uint32_t jl = 0; jl < kChunk; ++jl) {
                const uint32_t j = g0 + c0 + jl;
                const uint32_t sb = (j < 2 ? cur.s01 >> (16 * j) : cur.s23 >> (16 * (j - 2))) & 0xFFFFu;
                const float d = row_group_dot<kBits>(L, j, g[jl], keys);
                if (lane < rows && j < cn) acc = fmaf(half_to_float(sb), d, acc);
            }
        }
        wave_lds_sync();
        cur = nxt;
    }
    finish_row_tile<kWaves>(B, M, which, lds, wave, spare, a, split, r0, rows, relane(lane0), acc);
}

template <uint32_t kBits, bool kAligned, uint32_t kWaves>
__global__ __launch_bounds__(kWaves * kWave) __attribute__((amdgpu_waves_per_eu(8, 8))) void gemv_uniform(Batch B) {
    __shared__ WaveLds lds[kWaves];
    const MatArgs M = B.m[blockIdx.y];   // by value: loaded into scalar registers once
    uniform_tiles<kBits, kAligned, kWaves>(B, M, blockIdx.y, blockIdx.x, lds);
}

// One-width matrices of different widths in one launch (e.g. a head whose rows
// are grouped by width): each workgroup takes its matrix's width, uniform over
// the workgroup, so there is no divergence. The grid is 1D, the matrices'
// workgroups one after the other, so no workgroup is launched only to leave:
// such workgroups hold a CU slot (and 78 KiB of LDS) for the latency of their
// argument load, and with a few large matrices among small ones they delayed
// the large matrix's workgroups by microseconds.
template <bool kAligned, uint32_t kWaves>
__global__ __launch_bounds__(kWaves * kWave) __attribute__((amdgpu_waves_per_eu(8, 8))) void gemv_uniform_mixed(
    Batch B) {
    __shared__ WaveLds lds[kWaves];
    uint32_t which = 0;
#pragma unroll
    for (uint32_t i = 1; i < VBQ_MAX_MULTI; ++i) which += blockIdx.x >= B.first_block[i] ? 1u : 0u;
    const uint32_t bx = blockIdx.x - B.first_block[which];
    const MatArgs M = B.m[which];
    switch (M.ubits) {
        case 1: uniform_tiles<1, kAligned, kWaves>(B, M, which, bx, lds); break;
        case 2: uniform_tiles<2, kAligned, kWaves>(B, M, which, bx, lds); break;
        case 4: uniform_tiles<4, kAligned, kWaves, true, true>(B, M, which, bx, lds); break;
        default: uniform_tiles<8, kAligned, kWaves, false, true>(B, M, which, bx, lds); break;
    }
}

// Decoded codes of every group, written at its natural position; the same
// field decoders as the GEMV kernels (fp16 pairs whose halves are the
// subnormals f u 2^-24, then exact integer recovery) plus the sign bits of
// 1-bit groups.
template <bool kAligned>
__global__ __launch_bounds__(64) void unpack_tiles(MatArgs M, int8_t *__restrict__ codes) {
    __shared__ WaveLds L;
    const uint32_t lane = threadIdx.x;
    const uint32_t a = blockIdx.x / M.col_tiles, ct = blockIdx.x % M.col_tiles;
    const uint32_t r0 = a * kTileRows, rows = min(kTileRows, M.n - r0);
    const uint32_t j0 = ct * kTileGroups, cn = min(kTileGroups, M.groups - j0);
    const TileMeta t = load_meta<kAligned>(M, a, ct, lane, false);
    const rsrc_t tp = tile_rsrc(M.payload, M.payload_bytes, t.off);
    const uint64_t k = static_cast<uint64_t>(M.groups) * 64u;
    uint32_t cnt[4];
    const TileScan P = tile_scan(t, rows, cn, lane, cnt);
    build_lists(L, t, P, cnt, rows, cn, lane);
    wave_lds_sync();
    uint32_t base = 0;    // byte offset of the bucket in the tile
    uint32_t first = 0;   // list index of the bucket's first group
    for (uint32_t wsel = 0; wsel < 4; ++wsel) {
        const uint32_t b = 1u << wsel;
        for (uint32_t e = lane; e < cnt[wsel]; e += kWave) {
            const uint32_t info = L.list[first + e];
            const uint32_t r = info % kTileRows, jl = info / kTileRows;
            const uint32_t src = base + 8u * b * e;
            uint32_t *dst = reinterpret_cast<uint32_t *>(codes + (r0 + r) * k + 64u * (j0 + jl));
            for (uint32_t wd = 0; wd < 2 * b; ++wd) {
                const uint32_t v = buf_load4(tp, src + 4u * wd);
                if (b == 1) {
                    // 32 sign bits -> 32 codes of +-1
                    for (uint32_t o = 0; o < 8; ++o) {
                        uint32_t out = 0;
                        for (uint32_t i = 0; i < 4; ++i) {
                            const uint32_t bit = (v >> (4 * o + i)) & 1u;
                            const uint32_t pair = unpack1_pair(bit << 15, 0u);
                            const int q = static_cast<int>(half_to_float(pair & 0xFFFFu));
                            out |= (static_cast<uint32_t>(q) & 0xFFu) << (8 * i);
                        }
                        dst[wd * 8 + o] = out;
                    }
                } else if (b == 2) {
                    uint32_t p[8];
                    unpack2(v, p);
                    const float f[8] = {1.f, 4.f, 16.f, 64.f, 256.f, 1.f, 4.f, 16.f};
                    uint32_t outw[4] = {0, 0, 0, 0};
                    for (uint32_t m = 0; m < 8; ++m) {
                        // a pair half is the subnormal f u 2^-24: exact after scaling back
                        const int qa = static_cast<int>(half_to_float(p[m] & 0xFFFFu) * 0x1p24f / f[m]) - 2;
                        const int qb = static_cast<int>(half_to_float(p[m] >> 16) * 0x1p24f / f[m]) - 2;
                        const uint32_t e0 = 2 * m, e1 = 2 * m + 1;
                        outw[e0 >> 2] |= (static_cast<uint32_t>(qa) & 0xFFu) << (8 * (e0 & 3));
                        outw[e1 >> 2] |= (static_cast<uint32_t>(qb) & 0xFFu) << (8 * (e1 & 3));
                    }
                    for (uint32_t o = 0; o < 4; ++o) dst[wd * 4 + o] = outw[o];
                } else if (b == 4) {
                    uint32_t p[4];
                    unpack4(v, p);
                    uint32_t outw[2] = {0, 0};
                    for (uint32_t m = 0; m < 4; ++m) {
                        const float f = (m & 1) ? 16.f : 1.f;
                        const int qa = static_cast<int>(half_to_float(p[m] & 0xFFFFu) * 0x1p24f / f) - 8;
                        const int qb = static_cast<int>(half_to_float(p[m] >> 16) * 0x1p24f / f) - 8;
                        const uint32_t e0 = 2 * m, e1 = 2 * m + 1;
                        outw[e0 >> 2] |= (static_cast<uint32_t>(qa) & 0xFFu) << (8 * (e0 & 3));
                        outw[e1 >> 2] |= (static_cast<uint32_t>(qb) & 0xFFu) << (8 * (e1 & 3));
                    }
                    dst[wd * 2] = outw[0];
                    dst[wd * 2 + 1] = outw[1];
                } else {
                    uint32_t p0, p1;
                    unpack8(v, p0, p1);
                    const int q0 = static_cast<int>(half_to_float(p0 & 0xFFFFu) * 0x1p24f) - 128;
                    const int q1 = static_cast<int>(half_to_float(p0 >> 16) * 0x1p24f) - 128;
                    const int q2 = static_cast<int>(half_to_float(p1 & 0xFFFFu) * 0x1p24f) - 128;
                    const int q3 = static_cast<int>(half_to_float(p1 >> 16) * 0x1p24f) - 128;
                    dst[wd] = (static_cast<uint32_t>(q0) & 0xFFu) | ((static_cast<uint32_t>(q1) & 0xFFu) << 8) |
                              ((static_cast<uint32_t>(q2) & 0xFFu) << 16) | ((static_cast<uint32_t>(q3) & 0xFFu) << 24);
                }
            }
        }
        base += 8u * b * cnt[wsel];
        first += cnt[wsel];
    }
}

// The stream index (layout in vbq.h): one wave per tile derives the tile's
// per-width counts and its list of groups in payload order with the mixed
// kernel's own tile_scan and build_lists, and stores them.
template <bool kAligned>
__global__ __launch_bounds__(64) void stream_index_tiles(MatArgs M, uint8_t *__restrict__ index, uint64_t tiles) {
    __shared__ WaveLds L;
    const uint32_t lane = threadIdx.x;
    const uint32_t a = blockIdx.x / M.col_tiles, ct = blockIdx.x % M.col_tiles;
    const uint32_t rows = min(kTileRows, M.n - a * kTileRows);
    const uint32_t cn = min(kTileGroups, M.groups - ct * kTileGroups);
    const TileMeta t = load_meta<kAligned>(M, a, ct, lane, false);
    uint32_t cnt[4];
    const TileScan P = tile_scan(t, rows, cn, lane, cnt);
    reinterpret_cast<uint32_t *>(L.list)[lane] = 0u;   // a smaller tile's unused entries stay 0
    wave_lds_sync();
    build_lists(L, t, P, cnt, rows, cn, lane);
    wave_lds_sync();
    reinterpret_cast<uint32_t *>(index + 256ull * blockIdx.x)[lane] = reinterpret_cast<const uint32_t *>(L.list)[lane];
    if (lane == 0) {
        uint2 c;
        c.x = cnt[0] | (cnt[1] << 16);
        c.y = cnt[2] | (cnt[3] << 16);
        reinterpret_cast<uint2 *>(index + 256ull * tiles)[blockIdx.x] = c;
    }
}

__global__ void fill_zero(float *__restrict__ y, uint64_t count) {
    const uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < count) y[i] = 0.f;
}

// y[row_map[r]] = 0 for r < rows, skipping map values at or past y_rows (a grouped head with k = 0)
__global__ void scatter_zero(float *y, const uint32_t *row_map, uint64_t rows, uint32_t y_rows) {
    const uint64_t r = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (r < rows && row_map[r] < y_rows) y[row_map[r]] = 0.f;
}

__global__ void fill_zero_u16(uint16_t *__restrict__ h, uint64_t count) {
    const uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < count) h[i] = 0;
}

// ---------------------------------------------------------------- small batch on the matrix cores
// Y[m][r] = sum_j s[r,j] * sum_i q[r,j,i] * X[m][64j+i] for up to 64 rows of X
// (VBQ paper §6 fused decode, batched; grid and scale §3.1 Eq. (1)).
// A wave owns one tile at a time, two columns per pass: it decodes every
// group of the two columns into exact fp16 codes in LDS (natural row order,
// one width per instruction, from the same bucket lists as the GEMV), then
// multiplies 16-row blocks of codes with 16-row blocks of X on the matrix
// cores (v_mfma_f32_16x16x32_f16, 32 k per instruction). Each column's fp32
// product is scaled by the group scale once and added to the accumulators.
// The four waves of a workgroup take a row tile's column tiles round robin
// and add their accumulators in a fixed order at the end.

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint16_t ushort2_t __attribute__((ext_vector_type(2)));

// When the matrix cores run a small batch (measured on MI355X, graph-replayed,
// standard width mix): the matrix-core kernel costs about the same for any m up
// to 16, with a floor of 7-12 us on small matrices (one tile per wave, a long
// dependent chain per tile), while m GEMVs in one launch cost more with every
// row. The crossover row count falls with the tile count roughly as
// 1/sqrt(tiles): the matrix cores win from m = 4 rows when m^2 x tiles reaches
// 85000 (32000x4096, 8000 tiles: m = 3 25.0 us as GEMVs vs 26.6, m = 4 25.6 vs
// 31.6 as GEMVs; 4096x4096: m = 8 10.7 as GEMVs vs 11.5, m = 12 12.0 vs 14.9 as
// GEMVs; 5632x2048: m = 8 9.1 as GEMVs vs 9.8, m = 12 10.0 vs 13.0 as GEMVs;
// 2048x2048 and smaller: GEMVs up to 16 rows), and always beyond 16 rows.
constexpr uint32_t kGemmMinBatch = 4;
constexpr uint32_t kGemmAlwaysBatch = 16;   // beyond this many rows of X, always the matrix cores
constexpr uint64_t kGemmMinWork = 85000;   // rows of X squared times tiles of W

struct GemmArgs {
    const uint8_t *widths;
    const uint16_t *scales;
    const uint32_t *tile_offsets;
    const uint8_t *payload;
    const uint16_t *x;    // [m][k] fp16
    float *y;             // [m][n] fp32
    float *partial;       // [splits][m][n] when splits > 1
    uint32_t *counters;   // [row tiles] when splits > 1 (self-resetting)
    uint32_t n, groups, col_tiles, splits, m, k;
    uint32_t payload_bytes;
};

// Up to kGemmMulti matrices that read the same X in one launch (gate and up, at a few rows of X): a 1D
// grid, matrix i owning workgroups [first_block[i], first_block[i + 1]); entries past the last hold the
// total.
constexpr uint32_t kGemmMulti = 8;
struct GemmBatch {
    GemmArgs g[kGemmMulti];
    uint32_t first_block[kGemmMulti + 1];
};

__device__ __forceinline__ uint32_t half2_fma(uint32_t v, uint32_t mul, uint32_t add) {
    const half2_t r = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, v), __builtin_bit_cast(half2_t, mul),
                                                __builtin_bit_cast(half2_t, add));
    return __builtin_bit_cast(uint32_t, r);
}

// How many groups of each width come before each column (16 bits per width),
// from the per-column counts of the tile scan; entry 4 holds the tile totals.
__device__ __forceinline__ void column_starts(const TileScan &T, uint64_t colstart[kTileGroups + 1]) {
    uint64_t before = 0;
#pragma unroll
    for (uint32_t jl = 0; jl < kTileGroups; ++jl) {
        colstart[jl] = before;
        const uint32_t cc = T.cols[jl];
        before += static_cast<uint64_t>(cc & 0xFFu) | (static_cast<uint64_t>((cc >> 8) & 0xFFu) << 16) |
                  (static_cast<uint64_t>((cc >> 16) & 0xFFu) << 32) | (static_cast<uint64_t>(cc >> 24) << 48);
    }
    colstart[kTileGroups] = before;
}

__device__ __forceinline__ uint32_t field16(uint64_t v, uint32_t w) {
    return static_cast<uint32_t>((v >> (16 * w)) & 0xFFFFu);
}

// ---------------------------------------------------------------- small-batch GEMM, A fragments decoded in registers
//
// One wave owns one 64x256 tile at a time and multiplies it with the m rows
// of X on v_mfma_f32_16x16x32_f16, one group (64 codes) per two instructions,
// then scales the group's products by its fp32 scale. The A operand of a
// 16-row block is decoded by the lanes straight from the payload into the
// fragment registers, with no round trip through LDS: lane (i, q) holds codes
// 8q..8q+7 (first instruction) and 32+8q..32+8q+7 (second) of row 16rb+i's
// group, which are whole bytes of that group at places fixed by its width
// (1 bit: byte 4h+q; 2 bits: the word 2h+q/2; 4 bits: the word 4h+q; 8 bits:
// bytes 32h+8q..32h+8q+7, h the instruction). The rows of one block may have
// different widths. A block whose 16 rows are all 1-bit in the column (most
// blocks of a head dominated by 1-bit rows) runs the 1-bit decoder; any other
// runs one width-generic decoder whose per-lane constants come from a table: for pair p (codes 2p, 2p+1), t = perm(hi, lo, sel0 + p dsel) brings
// the pair's bytes into the 16-bit halves, a packed shift by sh0 + p dsh moves
// each field to its place, (t & A) ^ B keeps the field, flips its top bit
// (two's complement to offset binary) and sets the fp16 exponent of 1024, and
// an fp16 fma (mul, add) maps 1024 + 2^s u to the code, exactly.

struct FragParams {
    uint32_t sel0, dsel, sh0, dsh, A, B, mul, add;
};

// constants of width code c (1, 2, 4, 8 bits) for lanes of quarter q
__device__ __forceinline__ FragParams frag_params(uint32_t c, uint32_t q) {
    switch (c) {
        case 0:   // byte q into the high byte of both halves; bit 8+2p (8+2p+1) down to bit 1; 1 - 2f = 1025 - v
            return FragParams{0x000C000Cu | (q << 8) | (q << 24), 0u, 7u | (8u << 16), 0x00020002u, 0x00020002u,
                              0x64006400u, 0xBC00BC00u, 0x64016401u};
        case 1:   // fields 4(q&1)+p and 12+4(q&1)+p of the word: bits 8(q&1)+2p of each half; q = v - 1026
            return FragParams{0x03020100u, 0u, (8u * (q & 1u)) * 0x00010001u, 0x00020002u, 0x00030003u,
                              0x64026402u, 0x3C003C00u, 0xE402E402u};
        case 2:   // nibbles p and 4+p of the word: bits 4p of each half; q = v - 1032
            return FragParams{0x03020100u, 0u, 0u, 0x00040004u, 0x000F000Fu, 0x64086408u, 0x3C003C00u, 0xE408E408u};
        default:  // bytes 2p, 2p+1 of the eight into the low byte of each half; q = v - 1152
            return FragParams{0x0C010C00u, 0x00020002u, 0u, 0u, 0x00FF00FFu, 0x64806480u, 0x3C003C00u, 0xE480E480u};
    }
}

// (t & a) ^ b in one instruction (v_bitop3_b32, truth table 0x6a)
__device__ __forceinline__ uint32_t and_xor(uint32_t t, uint32_t a, uint32_t b) {
    uint32_t r;
    asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x6a" : "=v"(r) : "v"(t), "v"(a), "v"(b));
    return r;
}

__device__ __forceinline__ uint32_t shr16x2(uint32_t v, uint32_t s) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(ushort2_t, v) >> __builtin_bit_cast(ushort2_t, s));
}

__device__ __forceinline__ half8_t frag_of(uint32_t o0, uint32_t o1, uint32_t o2, uint32_t o3) {
    return __builtin_bit_cast(half8_t, make_uint4(o0, o1, o2, o3));
}

// both fragment halves, pair by pair (one selector and one shift live at a time)
__device__ __forceinline__ void frag_generic(uint2 w0, uint2 w1, const FragParams &P, half8_t &a0, half8_t &a1) {
    uint32_t o0[4], o1[4];
    uint32_t sel = P.sel0, sh = P.sh0;
#pragma unroll
    for (uint32_t p = 0; p < 4; ++p) {
        if (p > 0) {
            sel += P.dsel;
            sh += P.dsh;
        }
        o0[p] = half2_fma(and_xor(shr16x2(__builtin_amdgcn_perm(w0.y, w0.x, sel), sh), P.A, P.B), P.mul, P.add);
        o1[p] = half2_fma(and_xor(shr16x2(__builtin_amdgcn_perm(w1.y, w1.x, sel), sh), P.A, P.B), P.mul, P.add);
    }
    a0 = frag_of(o0[0], o0[1], o0[2], o0[3]);
    a1 = frag_of(o1[0], o1[1], o1[2], o1[3]);
}

// The lane's payload bytes of one column of the tile: for each 16-row block, eight bytes per fragment half
struct FragCol {
    uint2 w[4][2];
};

struct alignas(16) FragTables {
    uint32_t where[kTileGroups][kTileRows];   // group byte offset in the tile | width code (0 past the rows)
    float scale[kTileGroups][kTileRows];      // group scale as fp32 (0 past the rows)
    uint32_t hscale[kTileGroups][kTileRows];  // 17 to 32 rows of X: the scale's fp16 bits in both halves (0 past the rows)
};
constexpr uint32_t kRedStride = kTileRows + 4;   // floats per parked activation row (spreads the banks)

template <uint32_t MB, uint32_t kWaves>
union alignas(16) FragLds {
    struct {
        FragParams params[16];   // [width code][quarter]
        uint2 nib1[16];          // 1-bit nibble n -> its four codes +-1 as two fp16 pairs
        FragTables tab[kWaves];
    } run;
    float red[kWaves][16 * MB * kRedStride];   // each wave's sums, [activation row][tile row]
};

// Lane r = row r: the byte offset and width of each of its groups, and its scales as fp32. Returns
// (uniform) bit 4 jl + rb set when every row of 16-row block rb is 1-bit in column jl. kScaled: also
// the scales' fp16 bits, and bit 16 + 4 jl + rb set when every row of the block is 1- or 2-bit in
// column jl with a scale s that is zero or normal and below 2^15 (then s q is an exact fp16 value, normal
// or zero, for each code q in [-2, 1]).
template <bool kScaled>
__device__ __forceinline__ uint32_t frag_tables(FragTables &T, const TileMeta &t, const TileScan &S,
                                                const uint64_t colstart[kTileGroups + 1], const uint32_t cnt[4],
                                                uint32_t rows, uint32_t cn, uint32_t lane) {
    const bool valid = lane < rows;
    const uint32_t b1 = 8u * cnt[0], b2 = b1 + 16u * cnt[1], b3 = b2 + 32u * cnt[2];   // bucket starts
    uint32_t ones = 0;
#pragma unroll
    for (uint32_t jl = 0; jl < kTileGroups; ++jl) {
        const uint32_t c = (t.codes >> (2 * jl)) & 3u;
        const uint32_t excl = S.incl[jl] - (1u << (8 * c));
        const uint32_t slot = field16(colstart[jl], c) + ((excl >> (8 * c)) & 0xFFu);
        const uint32_t base = c == 0 ? 0u : c == 1 ? b1 : c == 2 ? b2 : b3;
        const bool ok = valid && jl < cn;
        T.where[jl][lane] = ok ? ((base + (8u << c) * slot) | c) : 0u;
        const uint32_t sb = (jl < 2 ? (t.s01 >> (16 * jl)) : (t.s23 >> (16 * (jl - 2)))) & 0xFFFFu;
        T.scale[jl][lane] = ok ? half_to_float(sb) : 0.f;
        const uint64_t wide = __builtin_amdgcn_ballot_w64(ok && c != 0);   // rows with a wider group
#pragma unroll
        for (uint32_t rb = 0; rb < 4; ++rb)
            ones |= (((wide >> (16 * rb)) & 0xFFFFu) == 0 ? 1u : 0u) << (4 * jl + rb);
        if constexpr (kScaled) {
            T.hscale[jl][lane] = ok ? sb * 0x00010001u : 0u;
            const uint32_t e = (sb >> 10) & 0x1Fu;
            const bool fits = (e >= 1 && e <= 29) || (sb & 0x7FFFu) == 0;
            const uint64_t unfit = __builtin_amdgcn_ballot_w64(ok && (c > 1 || !fits));
#pragma unroll
            for (uint32_t rb = 0; rb < 4; ++rb)
                ones |= (((unfit >> (16 * rb)) & 0xFFFFu) == 0 ? 1u : 0u) << (16 + 4 * jl + rb);
        }
    }
    return ones;
}

// Activations of the tile's column jl: lane holds X[16mb + lane%16][64(j0 + jl) + 32h + 8q .. +7], from
// xp[mb] = the lane's row at 64 j0 + 8q. Rows past m read row m-1: a matrix-core output column depends
// only on its own input column, and those outputs are not stored.
template <uint32_t MB>
__device__ __forceinline__ void frag_x_rows(const GemmArgs &G, uint32_t j0, const uint16_t *xp[MB]) {
    const uint32_t lane = lane_id(), q = lane >> 4, mr = lane & 15u;
#pragma unroll
    for (uint32_t mb = 0; mb < MB; ++mb)
        xp[mb] = G.x + static_cast<uint64_t>(min(16 * mb + mr, G.m - 1)) * G.k + 64u * j0 + 8u * q;
}

template <uint32_t MB>
__device__ __forceinline__ void frag_load_x(const uint16_t *const xp[MB], uint32_t jl, half8_t bx[2][MB]) {
#pragma unroll
    for (uint32_t h = 0; h < 2; ++h)
#pragma unroll
        for (uint32_t mb = 0; mb < MB; ++mb)
            bx[h][mb] = __builtin_bit_cast(half8_t, *reinterpret_cast<const uint4 *>(xp[mb] + 64u * jl + 32u * h));
}

// A 1-bit block's lanes read their group's eight bytes once (both halves); other blocks read eight bytes
// per half at the width's places.
__device__ __forceinline__ FragCol frag_col_load(const FragTables &T, rsrc_t tile, uint32_t jl, uint32_t ones,
                                                 uint32_t q, uint32_t i) {
    FragCol B;
#pragma unroll
    for (uint32_t rb = 0; rb < 4; ++rb) {
        const uint32_t where = T.where[jl][16 * rb + i];
        if ((ones >> (4 * jl + rb)) & 1u) {
            B.w[rb][0] = buf_load8(tile, where);   // width code 0: where is the offset
        } else {
            const uint32_t qoff = ((4u * (q >> 1)) << 8) | ((4u * q) << 16) | ((8u * q) << 24);   // byte c: width c
            const uint32_t c = where & 3u;
            const uint32_t o0 = (where & ~7u) + ((qoff >> (8 * c)) & 0xFFu);
            B.w[rb][0] = buf_load8(tile, o0);
            B.w[rb][1] = buf_load8(tile, o0 + (4u << c));
        }
    }
    return B;
}

// kMulti: the launch holds several matrices, and a workgroup finds its own from the block prefix (one
// more dependent scalar load, about half a microsecond, so single-matrix launches skip it).
// The workgroup's sums (each wave's acc over its tiles of row tile a) added in wave order through LDS, then
// stored, or, for a split row tile, published as partials and added in split order by the last arriver.
template <uint32_t MB, uint32_t kWaves>
__device__ __forceinline__ void frag_finish(FragLds<MB, kWaves> &S, const GemmArgs &G, uint32_t wave, uint32_t a,
                                            uint32_t split, uint32_t r0, uint32_t rows, const float4_t acc[4][MB],
                                            uint32_t &arrived_s) {
    // Workgroup sum in wave order: each wave parks its sums as fp32 [activation row][tile row]
    __syncthreads();
    {
        float *red = S.red[wave];
        const uint32_t lane = lane_id(), q = lane >> 4, mr = lane & 15u;
#pragma unroll
        for (uint32_t rb = 0; rb < 4; ++rb)
#pragma unroll
            for (uint32_t mb = 0; mb < MB; ++mb)
                *reinterpret_cast<float4_t *>(&red[(16 * mb + mr) * kRedStride + 16 * rb + 4 * q]) = acc[rb][mb];
    }
    __syncthreads();
    const uint32_t outs = G.m * kTileRows;
    constexpr uint32_t kThreads = kWaves * kWave;
    auto wg_sum = [&](uint32_t i) {
        const uint32_t at = (i / kTileRows) * kRedStride + i % kTileRows;
        float t = S.red[0][at];
#pragma unroll
        for (uint32_t w = 1; w < kWaves; ++w) t += S.red[w][at];
        return t;
    };
    if (G.splits == 1) {
        for (uint32_t i = threadIdx.x; i < outs; i += kThreads) {
            const uint32_t m = i / kTileRows, row = i % kTileRows;
            if (row < rows) G.y[static_cast<uint64_t>(m) * G.n + r0 + row] = wg_sum(i);
        }
        return;
    }
    // split row tile: publish partial sums, count arrivals, the last workgroup adds them in split order
    for (uint32_t i = threadIdx.x; i < outs; i += kThreads) {
        const uint32_t m = i / kTileRows, row = i % kTileRows;
        if (row < rows)
            __hip_atomic_store(&G.partial[(static_cast<uint64_t>(split) * G.m + m) * G.n + r0 + row], wg_sum(i),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0)
        arrived_s = __hip_atomic_fetch_add(&G.counters[a * kCounterStride], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (arrived_s != G.splits - 1) return;
    // every output's partials are requested before any is added (clamped
    // addresses for outputs past m x rows, which are not stored)
    constexpr uint32_t kPerThread = (VBQ_MAX_BATCH * kTileRows) / kThreads;
    const uint64_t stride = static_cast<uint64_t>(G.m) * G.n;
    for (uint32_t s0 = 0; s0 < G.splits; s0 += 2) {
        float v[kPerThread][2];
#pragma unroll
        for (uint32_t j = 0; j < kPerThread; ++j) {
            const uint32_t i = min(threadIdx.x + j * kThreads, outs - 1);
            const uint32_t m = i / kTileRows, row = min(i % kTileRows, rows - 1);
            const float *p = G.partial + static_cast<uint64_t>(m) * G.n + r0 + row;
#pragma unroll
            for (uint32_t h = 0; h < 2; ++h)
                v[j][h] = __hip_atomic_load(p + min(s0 + h, G.splits - 1) * stride, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (uint32_t j = 0; j < kPerThread; ++j) {
            const uint32_t i = threadIdx.x + j * kThreads;
            if (i >= outs) break;
            const uint32_t m = i / kTileRows, row = i % kTileRows;
            float *y = G.y + static_cast<uint64_t>(m) * G.n + r0 + row;
            if (row < rows) {
                float t = s0 == 0 ? 0.f : *y;
                t += v[j][0];
                if (s0 + 1 < G.splits) t += v[j][1];
                *y = t;
            }
        }
    }
    if (threadIdx.x == 0) __hip_atomic_store(&G.counters[a * kCounterStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One 16-row block rb of column jl: decode the lane's A fragments (codes 8q..+7 and 32+8q..+7 of row
// 16rb + i; a block whose rows are all 1-bit by the nibble table, any other by the width-generic
// decoder), multiply with the activations on the matrix cores and add into acc (rows 16rb + 4q .. +3,
// activation row mr). At 17 to 32 rows of X a scaled block (every row 1- or 2-bit, scales that keep s q
// exact in fp16) carries s q in its fragments, so the matrix cores add straight into acc; any other
// block's products are scaled by each row's fp32 group scale and then added. (Beyond 32 rows the same
// folding measured slower, with the accumulators in matrix-core registers or in VGPRs: every block is
// scaled after its products there.)
template <uint32_t MB>
__device__ __forceinline__ void frag_block(const FragParams *params, const uint2 *nib, const FragTables &T,
                                           uint32_t jl, uint32_t rb, uint32_t kind, const uint2 w[2],
                                           const half8_t bx[2][MB], uint32_t q, uint32_t i, float4_t acc[MB]) {
    const bool one_bit = (kind & 1u) != 0;
    half8_t a0, a1;
    if (one_bit) {
        const uint32_t w0 = w[0].x, w1 = w[0].y;
        const uint2 p00 = nib[__builtin_amdgcn_ubfe(w0, 8 * q, 4)], p01 = nib[__builtin_amdgcn_ubfe(w0, 8 * q + 4, 4)];
        const uint2 p10 = nib[__builtin_amdgcn_ubfe(w1, 8 * q, 4)], p11 = nib[__builtin_amdgcn_ubfe(w1, 8 * q + 4, 4)];
        a0 = frag_of(p00.x, p00.y, p01.x, p01.y);
        a1 = frag_of(p10.x, p10.y, p11.x, p11.y);
    } else {
        const uint32_t c = T.where[jl][16 * rb + i] & 3u;
        frag_generic(w[0], w[1], params[4 * c + q], a0, a1);
    }
    if constexpr (MB == 2) {
        if (kind & 2u) {
            const uint32_t hs = T.hscale[jl][16 * rb + i];
            if (one_bit) {   // +-1 -> +-s: the codes' sign bits onto the scale's
                const uint32_t k = hs ^ 0x3C003C00u;
                const uint4 u0 = __builtin_bit_cast(uint4, a0), u1 = __builtin_bit_cast(uint4, a1);
                a0 = frag_of(u0.x ^ k, u0.y ^ k, u0.z ^ k, u0.w ^ k);
                a1 = frag_of(u1.x ^ k, u1.y ^ k, u1.z ^ k, u1.w ^ k);
            } else {
                const half8_t s8 = __builtin_bit_cast(half8_t, make_uint4(hs, hs, hs, hs));
                a0 *= s8;
                a1 *= s8;
            }
#pragma unroll
            for (uint32_t mb = 0; mb < MB; ++mb) acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bx[0][mb], acc[mb], 0, 0, 0);
#pragma unroll
            for (uint32_t mb = 0; mb < MB; ++mb) acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bx[1][mb], acc[mb], 0, 0, 0);
            return;
        }
    }
    float4_t d[MB];
#pragma unroll
    for (uint32_t mb = 0; mb < MB; ++mb)
        d[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bx[0][mb], float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
    for (uint32_t mb = 0; mb < MB; ++mb) d[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bx[1][mb], d[mb], 0, 0, 0);
    const float4_t s = *static_cast<const float4_t *>(__builtin_assume_aligned(&T.scale[jl][16 * rb + 4 * q], 16));
#pragma unroll
    for (uint32_t mb = 0; mb < MB; ++mb) acc[mb] += s * d[mb];
}

// frag_block's kind from frag_tables' masks: bit 0 all 1-bit, bit 1 scaled
__device__ __forceinline__ uint32_t block_kind(uint32_t masks, uint32_t jl, uint32_t rb) {
    return ((masks >> (4 * jl + rb)) & 1u) | (((masks >> (16 + 4 * jl + rb)) & 1u) << 1);
}

// The small-batch kernel: one wave per 64x256 tile at a time, MB blocks of 16 rows of X. At 33 to 48
// rows (MB = 3) three waves per SIMD fit without spills (146 + 36 -> 158 registers: LM head m = 48
// 38.7 -> 38.1 us, 9B layer at batch 48 129.8 -> 127.4 us).
template <uint32_t MB, uint32_t kWaves, bool kAligned, bool kMulti>
__global__ __launch_bounds__(kWaves * kWave) __attribute__((amdgpu_waves_per_eu(MB == 3 ? 3 : 1))) void gemm_frag(
    GemmBatch B) {
    __shared__ FragLds<MB, kWaves> S;
    __shared__ uint32_t arrived_s;
    uint32_t which = 0;
    if constexpr (kMulti) {
#pragma unroll
        for (uint32_t i = 1; i < kGemmMulti; ++i) which += blockIdx.x >= B.first_block[i] ? 1u : 0u;
    }
    const GemmArgs G = B.g[which];   // by value: scalar registers
    const uint32_t bx = kMulti ? blockIdx.x - B.first_block[which] : blockIdx.x;
    const uint32_t a = bx / G.splits, split = bx % G.splits;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x) / kWave;
    const uint32_t r0 = a * kTileRows;
    const uint32_t rows = min(kTileRows, G.n - r0);
    const uint32_t c_lo = (split * G.col_tiles) / G.splits, c_hi = ((split + 1) * G.col_tiles) / G.splits;
    if (threadIdx.x < 16) {
        S.run.params[threadIdx.x] = frag_params(threadIdx.x >> 2, threadIdx.x & 3u);
        const uint32_t n = threadIdx.x;   // bit t set: code 4..+t is -1
        auto pm = [](uint32_t bit) { return bit ? 0xBC00u : 0x3C00u; };
        S.run.nib1[n] = make_uint2(pm(n & 1u) | (pm(n & 2u) << 16), pm(n & 4u) | (pm(n & 8u) << 16));
    }
    __syncthreads();
    FragTables &T = S.run.tab[wave];

    float4_t acc[4][MB];
#pragma unroll
    for (uint32_t rb = 0; rb < 4; ++rb)
#pragma unroll
        for (uint32_t mb = 0; mb < MB; ++mb) acc[rb][mb] = float4_t{0.f, 0.f, 0.f, 0.f};

    // (a wave usually owns one or two tiles, and the other waves of the CU cover its metadata wait: no
    // prefetch of the next tile's metadata, whose registers would be held across the whole tile)
    uint32_t ct = c_lo + wave;
    TileMeta meta = load_meta<kAligned>(G, a, ct < c_hi ? ct : c_lo, lane_id(), false);
    for (; ct < c_hi; ct += kWaves) {
        const uint32_t j0 = ct * kTileGroups, cn = kAligned ? kTileGroups : min(kTileGroups, G.groups - j0);
        uint32_t cnt[4];
        const TileScan sc = tile_scan(meta, rows, cn, lane_id(), cnt);
        uint64_t colstart[kTileGroups + 1];
        column_starts(sc, colstart);
        const uint32_t ones = frag_tables<(MB == 2)>(T, meta, sc, colstart, cnt, rows, cn, lane_id());
        const rsrc_t tile = tile_rsrc(G.payload, G.payload_bytes, meta.off);
        const uint16_t *xp[MB];
        frag_x_rows<MB>(G, j0, xp);
        const uint32_t lane = lane_id(), q = lane >> 4, i = lane & 15u;
        wave_lds_sync();
        if constexpr (MB != 2) {
            // the next tile's metadata travels while this tile computes
            meta = load_meta<kAligned>(G, a, ct + kWaves < c_hi ? ct + kWaves : ct, lane_id(), false);
            // one column at a time: the other waves of the SIMD cover the loads' latency (LM head, head
            // mix, against the two-stage pipeline below: m = 16 22.9 -> 21.7 us, m = 48 42.2 -> 38.3,
            // m = 64 alike; at m = 17..32 the pipeline is faster, 28.8 against 30.8 us at m = 24)
#pragma unroll 1
            for (uint32_t jl = 0; jl < kTileGroups; ++jl) {
                if (jl >= cn) break;
                const FragCol col = frag_col_load(T, tile, jl, ones, q, i);
                half8_t bx[2][MB];
                frag_load_x<MB>(xp, jl, bx);
#pragma unroll
                for (uint32_t rb = 0; rb < 4; ++rb)
                    frag_block<MB>(S.run.params, S.run.nib1, T, jl, rb, block_kind(ones, jl, rb), col.w[rb], bx,
                                   q, i, acc[rb]);
            }
            wave_lds_sync();
            continue;
        }
        // two-stage pipeline over the columns: the next column's payload bytes are requested before this
        // column is decoded, so a wave waits for memory about once per tile
        FragCol cur = frag_col_load(T, tile, 0, ones, q, i);
        half8_t bx[2][MB];
        frag_load_x<MB>(xp, 0, bx);
        // the next tile's metadata travels while this tile computes
        meta = load_meta<kAligned>(G, a, ct + kWaves < c_hi ? ct + kWaves : ct, lane_id(), false);
        // (a rolled loop: unrolled, the compiler hoists every column's loads and runs out of registers)
#pragma unroll 1
        for (uint32_t jl = 0; jl < kTileGroups; ++jl) {
            if (jl >= cn) break;
            FragCol nxt;
            if (jl + 1 < cn) nxt = frag_col_load(T, tile, jl + 1, ones, q, i);
            if (jl > 0) frag_load_x<MB>(xp, jl, bx);
#pragma unroll
            for (uint32_t rb = 0; rb < 4; ++rb) {
                frag_block<MB>(S.run.params, S.run.nib1, T, jl, rb, block_kind(ones, jl, rb), cur.w[rb], bx, q, i,
                               acc[rb]);
            }
            cur = nxt;
        }
        wave_lds_sync();
    }

    frag_finish<MB, kWaves>(S, G, wave, a, split, r0, rows, acc, arrived_s);
}

// ---------------------------------------------------------------- host side

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline uint32_t ceil_div(uint32_t a, uint32_t b) { return (a + b - 1) / b; }

vbq_status check_matrix(const char *who, const vbq_matrix *w) {
    if (!w) return fail(VBQ_ERR_NULL, "%s: matrix view is NULL", who);
    if (w->abi_version != VBQ_ABI_VERSION)
        return fail(VBQ_ERR_ABI, "%s: abi_version %u, library %u", who, w->abi_version, VBQ_ABI_VERSION);
    if (w->k % VBQ_GROUP) return fail(VBQ_ERR_SHAPE, "%s: k=%u is not a multiple of 64", who, w->k);
    if (w->k > VBQ_MAX_K) return fail(VBQ_ERR_SHAPE, "%s: k=%u exceeds %u", who, w->k, VBQ_MAX_K);
    if (w->n == 0 || w->k == 0) return VBQ_OK;
    // every group has at least 8 payload bytes; the kernels rely on it for 32-bit metadata offsets
    if (static_cast<uint64_t>(w->n) * (w->k / VBQ_GROUP) * 8u > w->payload_bytes)
        return fail(VBQ_ERR_OFFSETS, "%s: payload_bytes=%u is below 8 bytes per group (n=%u, k=%u)", who,
                    w->payload_bytes, w->n, w->k);
    if (!w->tile_offsets || !w->widths || !w->scales || !w->payload)
        return fail(VBQ_ERR_NULL, "%s: widths, scales, tile_offsets or payload is NULL", who);
    if (!aligned16(w->tile_offsets) || !aligned16(w->widths) || !aligned16(w->scales) || !aligned16(w->payload) ||
        !aligned16(w->stream_index))
        return fail(VBQ_ERR_ALIGN, "%s: a matrix array is not 16-byte aligned", who);
    const uint32_t b = w->uniform_bits;
    if (b != 0 && b != 1 && b != 2 && b != 4 && b != 8)
        return fail(VBQ_ERR_WIDTH, "%s: uniform_bits=%u is not 0, 1, 2, 4 or 8", who, b);
    if (b && static_cast<uint64_t>(w->n) * (w->k / VBQ_GROUP) * 8u * b != w->payload_bytes)
        return fail(VBQ_ERR_OFFSETS, "%s: payload_bytes=%u is not 8*%u bytes per group", who, w->payload_bytes, b);
    return VBQ_OK;
}

vbq_status launched(const char *who) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(VBQ_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
    return VBQ_OK;
}

// Scratch for split row tiles and the gated epilogue: one buffer per
// (device, stream), enlarged on demand. The buffer starts with a region that
// only ever holds arrival counters: it is zeroed when allocated and every
// counter is reset to zero by the last workgroup of its row tile, so the
// region is all zeros between calls however the next call lays out its
// matrices. Partial sums follow it. A superseded buffer is never freed (a
// graph captured earlier may still hold its address), and nothing is
// allocated while the caller's stream is being captured.
struct Scratch {
    void *ptr = nullptr;
    size_t counter_bytes = 0;
    size_t partial_bytes = 0;
};

std::mutex g_scratch_mu;
std::unordered_map<uint64_t, Scratch> g_scratch;
std::vector<void *> g_retired;   // superseded scratch buffers, held until the process ends

vbq_status scratch_for(const char *who, hipStream_t stream, size_t counters, size_t partials, uint32_t **ctr_out,
                       char **part_out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(VBQ_ERR_HIP, "%s: hipGetDevice failed", who);
    const uint64_t key = (static_cast<uint64_t>(dev) << 56) ^ reinterpret_cast<uintptr_t>(stream);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    Scratch &s = g_scratch[key];
    if (s.counter_bytes < counters || s.partial_bytes < partials) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &cs) != hipSuccess)
            return fail(VBQ_ERR_HIP, "%s: could not query the stream's capture state", who);
        if (cs != hipStreamCaptureStatusNone)
            return fail(VBQ_ERR_HIP,
                        "%s: needs %zu B of scratch on a stream that is being captured (the library does not "
                        "allocate during capture; make one call of the same shapes on this stream first)",
                        who, counters + partials);
        g_retired.reserve(g_retired.size() + 1);   // may throw before anything changes
        const size_t cb = std::max<size_t>(counters, std::max<size_t>(s.counter_bytes, 64u << 10));
        const size_t pb = std::max<size_t>(partials, std::max<size_t>(s.partial_bytes, 1u << 20));
        void *fresh = nullptr;
        if (hipMalloc(&fresh, cb + pb) != hipSuccess) return fail(VBQ_ERR_HIP, "%s: scratch hipMalloc failed", who);
        // zero the counter region on the caller's stream, ahead of the launches that use it (a memset on
        // the null stream is not ordered with non-blocking streams)
        const uint64_t words = cb / 4;
        hipLaunchKernelGGL(fill_zero, dim3(static_cast<uint32_t>((words + 255) / 256)), dim3(256), 0, stream,
                           static_cast<float *>(fresh), words);
        if (hipGetLastError() != hipSuccess) {
            g_retired.push_back(fresh);
            return fail(VBQ_ERR_HIP, "%s: scratch clear failed", who);
        }
        if (s.ptr) g_retired.push_back(s.ptr);
        s.ptr = fresh;
        s.counter_bytes = cb;
        s.partial_bytes = pb;
    }
    *ctr_out = static_cast<uint32_t *>(s.ptr);
    *part_out = static_cast<char *>(s.ptr) + s.counter_bytes;
    return VBQ_OK;
}

// Scratch of vbq_gemv_multi_noalloc: a fixed array in the library's device
// memory (one copy per GPU, zero-initialised when the code object loads).
// Host code never uses the name `scratch` as an address: the device address
// of each GPU's copy comes from hipGetSymbolAddress, taken once per device
// with that device current, and only that address reaches kernels.
static __device__ __align__(256) uint8_t scratch[VBQ_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void *g_static_ptr[kMaxDevices] = {};

vbq_status static_scratch(const char *who, hipStream_t stream, size_t counters, size_t partials, uint32_t **ctr_out,
                          char **part_out) {
    if (counters > VBQ_NOALLOC_COUNTER_BYTES || partials > VBQ_NOALLOC_SCRATCH_BYTES - VBQ_NOALLOC_COUNTER_BYTES)
        return fail(VBQ_ERR_CAPACITY,
                    "%s: the launch needs %zu B of counters and %zu B of partial sums; the fixed scratch holds %u "
                    "and %u",
                    who, counters, partials, VBQ_NOALLOC_COUNTER_BYTES,
                    VBQ_NOALLOC_SCRATCH_BYTES - VBQ_NOALLOC_COUNTER_BYTES);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(VBQ_ERR_HIP, "%s: hipGetDevice failed", who);
    if (dev < 0 || dev >= kMaxDevices) return fail(VBQ_ERR_HIP, "%s: device %d beyond %d", who, dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_static_mu);
    if (!g_static_ptr[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(VBQ_ERR_HIP, "%s: hipGetSymbolAddress of the scratch array failed: %s", who,
                        hipGetErrorString(e));
        // the counters are zero at load and every call leaves them zero; clear them once anyway, with a
        // kernel (not a memset) so a first call under graph capture records nothing a replay mishandles
        const uint64_t words = VBQ_NOALLOC_COUNTER_BYTES / 4;
        hipLaunchKernelGGL(fill_zero, dim3(static_cast<uint32_t>((words + 255) / 256)), dim3(256), 0, stream,
                           static_cast<float *>(ptr), words);
        if (hipGetLastError() != hipSuccess) return fail(VBQ_ERR_HIP, "%s: scratch clear failed", who);
        g_static_ptr[dev] = ptr;
    }
    *ctr_out = static_cast<uint32_t *>(g_static_ptr[dev]);
    *part_out = static_cast<char *>(g_static_ptr[dev]) + VBQ_NOALLOC_COUNTER_BYTES;
    return VBQ_OK;
}

inline size_t partial_bytes(uint32_t splits, uint32_t n) {
    return (static_cast<size_t>(splits) * n * 4 + 255) / 256 * 256;
}

// Launch shape of one batched GEMV launch: waves per workgroup and splits
// per row tile. The cost model was fitted to graph-replayed launch times on
// MI355X over the shapes of every decode workload (4096- to 14336-wide
// layers, the 1.0B and 131M sets, the 32000-row head) and a 131072x4096
// matrix, 13 shapes, every waves/splits choice: time ~ 1.1 per tile slot of
// a SIMD (tiles per wave x waves per SIMD, averaged over the CUs a launch
// occupies) + 2.5 per tile a wave handles after its first and per extra
// round of workgroups + the split tail (1.4 + 0.23 per split: partial
// stores, the arrival count and the last arriver's sum, three dependent
// round trips to memory). It picks the fastest measured shape for all 13.
struct GemvPlan {
    uint32_t waves, splits;
};

// Cost of a tile in gemv_rows (two rows of X) relative to the single-row
// kernel, from the kernels' instruction counts per tile.
constexpr double kRowsCost2 = 1.15;

// Rows of X a GEMV wave takes in the small-batch GEMV route. Two rows per
// decoded tile pay off only at m = 2 and where the launch is bound by issue
// rate, from kRowsMinTiles tiles in the call (9B q+k+v 11.2 -> 10.1 us,
// 14336x4096 gate+up 19.1 -> 16.8, LM head 19.9 -> 17.2). Smaller launches are
// bound by each wave's latency, and halving their waves costs more than the
// shared decoding saves (1.0B q+k+v, 768 tiles: 5.8 -> 6.8 us); at m = 3 and 4
// one row per wave keeps more waves in flight and wins (LM head m = 3: 26.5
// against 28.7 with pairs). Four rows per wave (211 VGPRs, two waves per
// SIMD) lost everywhere the matrix cores do not already win.
constexpr uint64_t kRowsMinTiles = 2048;
inline uint32_t rows_per_wave(uint32_t m, uint64_t tiles) { return m == 2 && tiles >= kRowsMinTiles ? 2u : 1u; }

// rows: rows of X per wave (gemv_rows); its LDS per wave is that many times
// larger, so fewer workgroups are resident, and a tile costs more to handle.
GemvPlan gemv_plan(uint32_t row_tiles, uint32_t col_tiles, uint32_t rows = 1) {
    constexpr uint32_t kCUs = 256;
    constexpr uint32_t kLdsPerCu = 160u * 1024u;
    const uint32_t waves[3] = {4, 8, 16};
    const uint32_t lds_per_wave = rows == 1 ? sizeof(WaveLds) : sizeof(RowsLds<2>);
    const double tile_cost = rows == 1 ? 1.1 : 1.1 * kRowsCost2;
    GemvPlan best{4, 1};
    double best_cost = 1e300;
    for (uint32_t w = 0; w < 3; ++w) {
        const uint32_t gw = waves[w];
        const uint32_t per_cu = kLdsPerCu / (gw * lds_per_wave);   // resident workgroups per CU (LDS bound)
        if (per_cu == 0) continue;
        for (uint32_t s = 1; s <= ceil_div(col_tiles, gw); ++s) {
            const double wgs = static_cast<double>(row_tiles) * s;
            const uint32_t ct_per = ceil_div(col_tiles, s);              // column tiles of a workgroup (at most)
            const uint32_t active = std::min(gw, ct_per);                // waves with a tile
            const uint32_t tpw = ceil_div(ct_per, gw);                   // tiles per wave (at most)
            const double cu_load = std::max(1.0, wgs / kCUs);            // workgroups per occupied CU
            const double rounds = std::ceil(cu_load / per_cu);
            const double slots = tpw * (active / 4.0) * cu_load;
            const double cost =
                tile_cost * slots + 2.5 * ((tpw - 1) + (rounds - 1)) + (s > 1 ? 1.4 + 0.23 * s : 0.0);
            if (cost < best_cost) {
                best_cost = cost;
                best = GemvPlan{gw, s};
            }
        }
    }
    return best;
}

template <uint32_t kBits, uint32_t kWaves>
void gemv_dispatch_uniform(bool aligned, uint32_t blocks, uint32_t used, const Batch &B, hipStream_t stream) {
    if (aligned)
        hipLaunchKernelGGL((gemv_uniform<kBits, true, kWaves>), dim3(blocks, used), dim3(kWaves * kWave), 0, stream,
                           B);
    else
        hipLaunchKernelGGL((gemv_uniform<kBits, false, kWaves>), dim3(blocks, used), dim3(kWaves * kWave), 0, stream,
                           B);
}

// ubits: the width every matrix of the launch has; kPerMatrix when each matrix declares a width but
// they differ; 0 when some matrix declares none (the mixed-width kernel)
constexpr uint32_t kPerMatrix = 0xFFu;

template <uint32_t kWaves, bool kIndexed>
void gemv_dispatch_mixed(bool aligned, bool ragged, dim3 grid, const Batch &B, hipStream_t stream) {
    const dim3 block(kWaves * kWave);
    if (aligned && ragged)
        hipLaunchKernelGGL((gemv_tiles<true, kWaves, true, kIndexed>), grid, block, 0, stream, B);
    else if (aligned)
        hipLaunchKernelGGL((gemv_tiles<true, kWaves, false, kIndexed>), grid, block, 0, stream, B);
    else if (ragged)
        hipLaunchKernelGGL((gemv_tiles<false, kWaves, true, kIndexed>), grid, block, 0, stream, B);
    else
        hipLaunchKernelGGL((gemv_tiles<false, kWaves, false, kIndexed>), grid, block, 0, stream, B);
}

// indexed: the mixed-width kernel reads every matrix's stream index
template <uint32_t kWaves>
void gemv_dispatch(bool aligned, bool ragged, bool indexed, uint32_t ubits, uint32_t blocks, uint32_t used,
                   const Batch &B, hipStream_t stream) {
    if (ubits == kPerMatrix) {   // 1D grid: every matrix's workgroups, back to back
        const uint32_t total = B.first_block[VBQ_MAX_MULTI];
        if (aligned)
            hipLaunchKernelGGL((gemv_uniform_mixed<true, kWaves>), dim3(total), dim3(kWaves * kWave), 0, stream, B);
        else
            hipLaunchKernelGGL((gemv_uniform_mixed<false, kWaves>), dim3(total), dim3(kWaves * kWave), 0, stream, B);
        return;
    }
    switch (ubits) {
        case 1: gemv_dispatch_uniform<1, kWaves>(aligned, blocks, used, B, stream); return;
        case 2: gemv_dispatch_uniform<2, kWaves>(aligned, blocks, used, B, stream); return;
        case 4: gemv_dispatch_uniform<4, kWaves>(aligned, blocks, used, B, stream); return;
        case 8: gemv_dispatch_uniform<8, kWaves>(aligned, blocks, used, B, stream); return;
        default: break;
    }
    if (indexed)
        gemv_dispatch_mixed<kWaves, true>(aligned, ragged, dim3(blocks, used), B, stream);
    else
        gemv_dispatch_mixed<kWaves, false>(aligned, ragged, dim3(blocks, used), B, stream);
}

template <uint32_t kWaves, uint32_t kR>
void gemv_rows_dispatch(bool aligned, uint32_t blocks, uint32_t used, const Batch &B, hipStream_t stream) {
    const dim3 grid(blocks, used), block(kWaves * kWave);
    if (aligned)
        hipLaunchKernelGGL((gemv_rows<true, kWaves, kR>), grid, block, 0, stream, B);
    else
        hipLaunchKernelGGL((gemv_rows<false, kWaves, kR>), grid, block, 0, stream, B);
}

// One launch for up to VBQ_MAX_MULTI independent GEMVs; with h set, the two
// matrices are gate and up (same shape, k > 0) and the launch writes
// h = fp16(silu(gate x) * (up x)) instead of y.
// no_alloc: the split scratch comes from the fixed array (vbq_gemv_multi_noalloc), never from hipMalloc.
// rows = 2: every entry is two rows of X (row r at xs[i] + r k) against ws[i], written to ys[i] + r n,
// by gemv_rows (no h, no fp16 y).
// row_map, y_rows: a grouped head (Batch::row_map); the matrices are its row blocks in rank order.
vbq_status gemv_launch(const char *who, const vbq_matrix *const *ws, const uint16_t *const *xs, float *const *ys,
                       uint32_t count, hipStream_t stream, uint16_t *h = nullptr, uint16_t *const *ys16 = nullptr,
                       bool no_alloc = false, uint32_t rows = 1, const uint32_t *row_map = nullptr,
                       uint32_t y_rows = 0) {
    Batch B{};
    B.row_map = row_map;
    B.y_rows = y_rows;
    uint32_t blocks = 0, total_row_tiles = 0, max_col_tiles = 0;
    bool aligned = true;
    for (uint32_t i = 0; i < count; ++i) {
        const vbq_matrix *w = ws[i];
        if (w->n == 0 || w->k == 0) continue;
        total_row_tiles += ceil_div(w->n, kTileRows);
        max_col_tiles = std::max(max_col_tiles, ceil_div(w->k / VBQ_GROUP, kTileGroups));
    }
    const GemvPlan plan = total_row_tiles ? gemv_plan(total_row_tiles, max_col_tiles, rows) : GemvPlan{4, 1};
    size_t counter_slots = 0, partial_total = 0;
    uint32_t used = 0;
    bool any_launch = false;
    // the uniform-width kernels run when every matrix launched declares a width: one kernel per width
    // when they agree, the per-matrix dispatch when they differ
    uint32_t ubits = 0;
    bool first = true;
    for (uint32_t i = 0; i < count && rows == 1; ++i) {
        if (ws[i]->n == 0 || ws[i]->k == 0) continue;
        const uint32_t b = ws[i]->uniform_bits;
        if (first || b == 0 || ubits == 0)
            ubits = first || ubits != 0 ? b : 0u;
        else if (b != ubits)
            ubits = kPerMatrix;
        first = false;
    }
    for (uint32_t i = 0; i < count; ++i) {
        const vbq_matrix *w = ws[i];
        if (w->n == 0 || w->k == 0) continue;
        MatArgs &M = B.m[used++];
        M.widths = w->widths;
        M.scales = w->scales;
        M.tile_offsets = w->tile_offsets;
        M.payload = w->payload;
        M.payload_bytes = w->payload_bytes;
        M.ubits = w->uniform_bits;
        M.x = xs[i];
        M.y = ys ? ys[i] : nullptr;
        M.y16 = ys16 ? ys16[i] : nullptr;
        M.index = w->stream_index;
        M.n = w->n;
        M.groups = w->k / VBQ_GROUP;
        M.col_tiles = ceil_div(M.groups, kTileGroups);
        const uint32_t row_tiles = ceil_div(M.n, kTileRows);
        // a wave's unit along K (see uniform_tiles): a tile, or in the per-matrix-width kernel one group of
        // an 8-bit matrix and two of a 4-bit one, with up to that many times the plan's splits, so that a
        // small such matrix (the 8-bit tier of a grouped head) waits for its payload once per wave
        const uint32_t ub = ubits == kPerMatrix ? w->uniform_bits : 0u;
        const uint32_t unit = ub == 8 ? 1u : ub == 4 ? 2u : kTileGroups;
        M.units = unit == kTileGroups ? M.col_tiles : ceil_div(M.groups, unit);
        M.splits = std::max(1u, std::min(ceil_div(M.units, plan.waves), plan.splits * (kTileGroups / unit)));
        M.blocks = row_tiles * M.splits;
        blocks = std::max(blocks, M.blocks);
        if (M.groups % 4) aligned = false;
    }
    if (ubits == kPerMatrix) {
        // The per-matrix-width kernel multiplies the splits of 8- and 4-bit matrices (above). Where that
        // pushes the grid past one round of resident workgroups, the last ones would start only when
        // others leave and add a whole workgroup's time (the grouped 32000-row head: 518 workgroups of 16
        // waves for 512 places); the multipliers are then halved, matrix by matrix, until the grid fits
        // or none is left.
        const uint32_t room =
            256u * std::max(1u, (160u * 1024u) / (plan.waves * static_cast<uint32_t>(sizeof(WaveLds))));
        auto total_blocks = [&]() {
            uint32_t t = 0;
            for (uint32_t i = 0; i < used; ++i) t += B.m[i].blocks;
            return t;
        };
        for (uint32_t pass = 0; pass < 4 && total_blocks() > room; ++pass) {
            bool changed = false;
            for (uint32_t i = 0; i < used && total_blocks() > room; ++i) {
                MatArgs &M = B.m[i];
                const uint32_t floor_splits = std::max(1u, std::min(ceil_div(M.units, plan.waves), plan.splits));
                if (M.ubits < 4 || M.splits <= floor_splits) continue;
                M.splits = std::max(floor_splits, M.splits / 2);
                M.blocks = ceil_div(M.n, kTileRows) * M.splits;
                changed = true;
            }
            if (!changed) break;
        }
        blocks = 0;
        for (uint32_t i = 0; i < used; ++i) blocks = std::max(blocks, B.m[i].blocks);
    }
    for (uint32_t i = 0; i < used; ++i) {
        const MatArgs &M = B.m[i];
        if (M.splits > 1) {
            counter_slots += ceil_div(M.n, kTileRows) * kCounterStride;
            partial_total += partial_bytes(M.splits * rows, M.n);
        }
    }
    if (h && used) {   // the pair region follows the split regions
        counter_slots += ceil_div(B.m[0].n, kTileRows) * kCounterStride;
        partial_total += partial_bytes(2, B.m[0].n);
    }
    if (counter_slots) {
        uint32_t *ctr = nullptr;
        char *part = nullptr;
        vbq_status st = no_alloc ? static_scratch(who, stream, counter_slots * 4, partial_total, &ctr, &part)
                                 : scratch_for(who, stream, counter_slots * 4, partial_total, &ctr, &part);
        if (st != VBQ_OK) return st;
        for (uint32_t i = 0; i < used; ++i) {
            MatArgs &M = B.m[i];
            if (M.splits == 1) continue;
            M.counters = ctr;
            ctr += ceil_div(M.n, kTileRows) * kCounterStride;
            M.partial = reinterpret_cast<float *>(part);
            part += partial_bytes(M.splits * rows, M.n);
        }
        if (h) {
            B.h = h;
            B.pair_counters = ctr;
            B.pair = reinterpret_cast<float *>(part);
        }
    }
    // only now that nothing can fail: k == 0 matrices get y = 0
    for (uint32_t i = 0; i < count; ++i) {
        const vbq_matrix *w = ws[i];
        if (w->n == 0 || w->k != 0) continue;
        const uint64_t cnt = static_cast<uint64_t>(w->n) * rows;
        if (ys16)
            hipLaunchKernelGGL(fill_zero_u16, dim3(static_cast<uint32_t>((cnt + 255) / 256)), dim3(256), 0, stream,
                               ys16[i], cnt);
        else
            hipLaunchKernelGGL(fill_zero, dim3(static_cast<uint32_t>((cnt + 255) / 256)), dim3(256), 0, stream,
                               ys[i], cnt);
        any_launch = true;
    }
    if (used == 0) return any_launch ? launched(who) : VBQ_OK;
    bool ragged = false;   // some matrix has fewer workgroups than the grid is wide
    for (uint32_t i = 0; i < used; ++i) ragged = ragged || B.m[i].blocks != blocks;
    bool indexed = rows == 1;   // the mixed-width kernel reads stream indexes when every matrix has one
    for (uint32_t i = 0; i < used; ++i) indexed = indexed && B.m[i].index != nullptr;
    uint32_t acc = 0;
    for (uint32_t i = 0; i <= VBQ_MAX_MULTI; ++i) {
        B.first_block[i] = acc;
        if (i < used) acc += B.m[i].blocks;
    }
    if (rows == 2) {
        if (plan.waves == 16)
            gemv_rows_dispatch<16, 2>(aligned, blocks, used, B, stream);
        else if (plan.waves == 8)
            gemv_rows_dispatch<8, 2>(aligned, blocks, used, B, stream);
        else
            gemv_rows_dispatch<4, 2>(aligned, blocks, used, B, stream);
    } else if (plan.waves == 16)
        gemv_dispatch<16>(aligned, ragged, indexed, ubits, blocks, used, B, stream);
    else if (plan.waves == 8)
        gemv_dispatch<8>(aligned, ragged, indexed, ubits, blocks, used, B, stream);
    else
        gemv_dispatch<4>(aligned, ragged, indexed, ubits, blocks, used, B, stream);
    return launched(who);
}

template <bool kAligned, bool kMulti>
void gemm_frag_dispatch(uint32_t mb, uint32_t waves, dim3 grid, const GemmBatch &G, hipStream_t stream) {
    if (mb == 1 && waves == 8)
        hipLaunchKernelGGL((gemm_frag<1, 8, kAligned, kMulti>), grid, dim3(8 * kWave), 0, stream, G);
    else if (mb == 1)
        hipLaunchKernelGGL((gemm_frag<1, 4, kAligned, kMulti>), grid, dim3(4 * kWave), 0, stream, G);
    else if (mb == 2 && waves == 8)
        hipLaunchKernelGGL((gemm_frag<2, 8, kAligned, kMulti>), grid, dim3(8 * kWave), 0, stream, G);
    else if (mb == 2)
        hipLaunchKernelGGL((gemm_frag<2, 4, kAligned, kMulti>), grid, dim3(4 * kWave), 0, stream, G);
    else if (mb == 3)
        hipLaunchKernelGGL((gemm_frag<3, 4, kAligned, kMulti>), grid, dim3(4 * kWave), 0, stream, G);
    else
        hipLaunchKernelGGL((gemm_frag<4, 4, kAligned, kMulti>), grid, dim3(4 * kWave), 0, stream, G);
}

// Small-batch GEMM on the matrix cores: one launch for up to 64 rows of X and up to kGemmMulti matrices
// that read them (same k, n > 0, k > 0).
vbq_status gemm_launch(const char *who, const vbq_matrix *const *ws, float *const *ys, uint32_t count,
                       const uint16_t *x, uint32_t m, hipStream_t stream) {
    GemmBatch B{};
    const uint32_t k = ws[0]->k, groups = k / VBQ_GROUP, col_tiles = ceil_div(groups, kTileGroups);
    // a wave per column tile of the row tile: 8 waves for up to 32 activation rows, 4 beyond (the
    // workgroup's sum buffer is at most 68 KiB); no more waves than column tiles need
    const uint32_t mb = ceil_div(m, 16);
    uint32_t waves = mb <= 2 ? 8u : 4u;
    while (waves > 4 && waves / 2 >= col_tiles) waves /= 2;
    uint32_t total_row_tiles = 0;
    for (uint32_t i = 0; i < count; ++i) total_row_tiles += ceil_div(ws[i]->n, kTileRows);
    // two workgroups per CU are resident (LDS): split the column tiles only
    // while the row tiles alone leave CUs idle
    const uint32_t splits = std::max(1u, std::min(ceil_div(col_tiles, waves), 512u / total_row_tiles));
    uint32_t *ctr = nullptr;
    char *part = nullptr;
    if (splits > 1) {
        size_t partials = 0;
        for (uint32_t i = 0; i < count; ++i)
            partials += (static_cast<size_t>(splits) * m * ws[i]->n * 4 + 255) / 256 * 256;
        vbq_status st =
            scratch_for(who, stream, static_cast<size_t>(total_row_tiles) * 4 * kCounterStride, partials, &ctr, &part);
        if (st != VBQ_OK) return st;
    }
    uint32_t blocks = 0;
    for (uint32_t i = 0; i <= kGemmMulti; ++i) {
        B.first_block[i] = blocks;
        if (i >= count) continue;
        const vbq_matrix *w = ws[i];
        GemmArgs &G = B.g[i];
        G.widths = w->widths;
        G.scales = w->scales;
        G.tile_offsets = w->tile_offsets;
        G.payload = w->payload;
        G.payload_bytes = w->payload_bytes;
        G.x = x;
        G.y = ys[i];
        G.n = w->n;
        G.groups = groups;
        G.col_tiles = col_tiles;
        G.m = m;
        G.k = k;
        G.splits = splits;
        const uint32_t row_tiles = ceil_div(G.n, kTileRows);
        if (splits > 1) {
            G.counters = ctr;
            ctr += row_tiles * kCounterStride;
            G.partial = reinterpret_cast<float *>(part);
            part += (static_cast<size_t>(splits) * m * G.n * 4 + 255) / 256 * 256;
        }
        blocks += row_tiles * splits;
    }
    const dim3 grid(blocks);
    if (groups % kTileGroups == 0) {
        if (count > 1)
            gemm_frag_dispatch<true, true>(mb, waves, grid, B, stream);
        else
            gemm_frag_dispatch<true, false>(mb, waves, grid, B, stream);
    } else {
        if (count > 1)
            gemm_frag_dispatch<false, true>(mb, waves, grid, B, stream);
        else
            gemm_frag_dispatch<false, false>(mb, waves, grid, B, stream);
    }
    return launched(who);
}

// The small-batch rule: matrix cores for m > 16 rows of X, or from 4 rows when m^2 x tiles reaches
// kGemmMinWork; one GEMV per row otherwise (measured, see kGemmMinWork)
uint64_t tile_count(const vbq_matrix *w) {
    return static_cast<uint64_t>(ceil_div(w->n, kTileRows)) * ceil_div(w->k / VBQ_GROUP, kTileGroups);
}

// tiles: of one matrix, or of all the matrices one launch would hold (their products share the launch's
// latency, so the matrix cores pay off at fewer rows)
bool uses_matrix_cores(uint64_t tiles, uint32_t m) {
    return m > kGemmAlwaysBatch || (m >= kGemmMinBatch && static_cast<uint64_t>(m) * m * tiles >= kGemmMinWork);
}

vbq_status check_vectors(const char *who, const vbq_matrix *w, const void *x, const void *y) {
    if (w->n == 0) return VBQ_OK;
    if (!y || (w->k && !x)) return fail(VBQ_ERR_NULL, "%s: x or y is NULL", who);
    if (!aligned16(y) || (w->k && !aligned16(x))) return fail(VBQ_ERR_ALIGN, "%s: x or y is not 16-byte aligned", who);
    return VBQ_OK;
}

}  // namespace

extern "C" vbq_status vbq_gemv_multi(const vbq_matrix *const *ws, const uint16_t *const *xs, float *const *ys,
                                     uint32_t count, void *stream) {
    return vbq::guarded("vbq_gemv_multi", [&]() -> vbq_status {
        vbq::clear_error();
        const char *who = "vbq_gemv_multi";
        if (count > VBQ_MAX_MULTI) return fail(VBQ_ERR_SHAPE, "%s: count=%u exceeds %u", who, count, VBQ_MAX_MULTI);
        if (count == 0) return VBQ_OK;
        if (!ws || !xs || !ys) return fail(VBQ_ERR_NULL, "%s: ws, xs or ys is NULL", who);
        for (uint32_t i = 0; i < count; ++i) {
            vbq_status st = check_matrix(who, ws[i]);
            if (st != VBQ_OK) return st;
            st = check_vectors(who, ws[i], xs[i], ys[i]);
            if (st != VBQ_OK) return st;
        }
        (void)hipGetLastError();
        return gemv_launch(who, ws, xs, ys, count, static_cast<hipStream_t>(stream));
    });
}

extern "C" vbq_status vbq_gemv_multi_noalloc(const vbq_matrix *const *ws, const uint16_t *const *xs,
                                             float *const *ys, uint32_t count, void *stream) {
    return vbq::guarded("vbq_gemv_multi_noalloc", [&]() -> vbq_status {
        vbq::clear_error();
        const char *who = "vbq_gemv_multi_noalloc";
        if (count > VBQ_MAX_MULTI) return fail(VBQ_ERR_SHAPE, "%s: count=%u exceeds %u", who, count, VBQ_MAX_MULTI);
        if (count == 0) return VBQ_OK;
        if (!ws || !xs || !ys) return fail(VBQ_ERR_NULL, "%s: ws, xs or ys is NULL", who);
        for (uint32_t i = 0; i < count; ++i) {
            vbq_status st = check_matrix(who, ws[i]);
            if (st != VBQ_OK) return st;
            st = check_vectors(who, ws[i], xs[i], ys[i]);
            if (st != VBQ_OK) return st;
        }
        (void)hipGetLastError();
        return gemv_launch(who, ws, xs, ys, count, static_cast<hipStream_t>(stream), nullptr, nullptr, true);
    });
}

extern "C" vbq_status vbq_gemv_swiglu(const vbq_matrix *gate, const vbq_matrix *up, const uint16_t *x, uint16_t *h,
                                      void *stream) {
    return vbq::guarded("vbq_gemv_swiglu", [&]() -> vbq_status {
        vbq::clear_error();
        const char *who = "vbq_gemv_swiglu";
        vbq_status st = check_matrix(who, gate);
        if (st != VBQ_OK) return st;
        st = check_matrix(who, up);
        if (st != VBQ_OK) return st;
        if (gate->n != up->n || gate->k != up->k)
            return fail(VBQ_ERR_SHAPE, "%s: gate is %ux%u, up is %ux%u", who, gate->n, gate->k, up->n, up->k);
        if (gate->n == 0) return VBQ_OK;
        if (!h || (gate->k && !x)) return fail(VBQ_ERR_NULL, "%s: x or h is NULL", who);
        if (!aligned16(h) || (gate->k && !aligned16(x)))
            return fail(VBQ_ERR_ALIGN, "%s: x or h is not 16-byte aligned", who);
        (void)hipGetLastError();
        const hipStream_t s = static_cast<hipStream_t>(stream);
        if (gate->k == 0) {   // g = u = 0, so h = silu(0) * 0 = 0
            hipLaunchKernelGGL(fill_zero_u16, dim3((gate->n + 255) / 256), dim3(256), 0, s, h, uint64_t(gate->n));
            return launched(who);
        }
        const vbq_matrix *ws[2] = {gate, up};
        const uint16_t *xs[2] = {x, x};
        float *ys[2] = {nullptr, nullptr};
        return gemv_launch(who, ws, xs, ys, 2, s, h);
    });
}

extern "C" vbq_status vbq_gemv_head_grouped(const vbq_matrix *const *tiers, uint32_t count, const uint16_t *x,
                                            const uint32_t *row_map, float *y, uint32_t y_rows, void *stream) {
    return vbq::guarded("vbq_gemv_head_grouped", [&]() -> vbq_status {
        vbq::clear_error();
        const char *who = "vbq_gemv_head_grouped";
        if (count > VBQ_MAX_MULTI) return fail(VBQ_ERR_SHAPE, "%s: count=%u exceeds %u", who, count, VBQ_MAX_MULTI);
        if (count == 0) return VBQ_OK;
        if (!tiers) return fail(VBQ_ERR_NULL, "%s: tiers is NULL", who);
        uint64_t ranks = 0;
        for (uint32_t i = 0; i < count; ++i) {
            vbq_status st = check_matrix(who, tiers[i]);
            if (st != VBQ_OK) return st;
            if (tiers[i]->k != tiers[0]->k)
                return fail(VBQ_ERR_SHAPE, "%s: tier %u has k=%u, tier 0 k=%u (they share x)", who, i, tiers[i]->k,
                            tiers[0]->k);
            ranks += tiers[i]->n;
        }
        if (ranks == 0) return VBQ_OK;
        if (ranks > 0xFFFFFFFFull) return fail(VBQ_ERR_SHAPE, "%s: %llu ranks exceed 32 bits", who,
                                               static_cast<unsigned long long>(ranks));
        if (!row_map || !y || (tiers[0]->k && !x)) return fail(VBQ_ERR_NULL, "%s: x, row_map or y is NULL", who);
        if (!aligned16(row_map) || !aligned16(y) || (tiers[0]->k && !aligned16(x)))
            return fail(VBQ_ERR_ALIGN, "%s: x, row_map or y is not 16-byte aligned", who);
        (void)hipGetLastError();
        const hipStream_t s = static_cast<hipStream_t>(stream);
        if (tiers[0]->k == 0) {   // every logit is 0
            hipLaunchKernelGGL(scatter_zero, dim3(static_cast<uint32_t>((ranks + 255) / 256)), dim3(256), 0, s, y,
                               row_map, ranks, y_rows);
            return launched(who);
        }
        const uint16_t *xs[VBQ_MAX_MULTI];
        float *ys[VBQ_MAX_MULTI];
        for (uint32_t i = 0; i < count; ++i) {
            xs[i] = x;
            ys[i] = y;
        }
        return gemv_launch(who, tiers, xs, ys, count, s, nullptr, nullptr, false, 1, row_map, y_rows);
    });
}

extern "C" vbq_status vbq_gemv_multi_f16(const vbq_matrix *const *ws, const uint16_t *const *xs, uint16_t *const *ys,
                                         uint32_t count, void *stream) {
    return vbq::guarded("vbq_gemv_multi_f16", [&]() -> vbq_status {
        vbq::clear_error();
        const char *who = "vbq_gemv_multi_f16";
        if (count > VBQ_MAX_MULTI) return fail(VBQ_ERR_SHAPE, "%s: count=%u exceeds %u", who, count, VBQ_MAX_MULTI);
        if (count == 0) return VBQ_OK;
        if (!ws || !xs || !ys) return fail(VBQ_ERR_NULL, "%s: ws, xs or ys is NULL", who);
        for (uint32_t i = 0; i < count; ++i) {
            vbq_status st = check_matrix(who, ws[i]);
            if (st != VBQ_OK) return st;
            st = check_vectors(who, ws[i], xs[i], ys[i]);
            if (st != VBQ_OK) return st;
        }
        (void)hipGetLastError();
        return gemv_launch(who, ws, xs, nullptr, count, static_cast<hipStream_t>(stream), nullptr, ys);
    });
}

extern "C" vbq_status vbq_gemv(const vbq_matrix *w, const uint16_t *x, float *y, void *stream) {
    return vbq::guarded("vbq_gemv", [&]() -> vbq_status {
        vbq::clear_error();
        const char *who = "vbq_gemv";
        vbq_status st = check_matrix(who, w);
        if (st != VBQ_OK) return st;
        st = check_vectors(who, w, x, y);
        if (st != VBQ_OK) return st;
        (void)hipGetLastError();
        return gemv_launch(who, &w, &x, &y, 1, static_cast<hipStream_t>(stream));
    });
}

extern "C" vbq_status vbq_gemm_smallbatch(const vbq_matrix *w, const uint16_t *x, uint32_t m, float *y,
                                          void *stream) {
    return vbq::guarded("vbq_gemm_smallbatch", [&]() -> vbq_status {
        vbq::clear_error();
        const char *who = "vbq_gemm_smallbatch";
        if (m == 0 || m > VBQ_MAX_BATCH) return fail(VBQ_ERR_SHAPE, "%s: m=%u outside [1, %u]", who, m, VBQ_MAX_BATCH);
        vbq_status st = check_matrix(who, w);
        if (st != VBQ_OK) return st;
        st = check_vectors(who, w, x, y);
        if (st != VBQ_OK) return st;
        if (w->n == 0) return VBQ_OK;
        (void)hipGetLastError();
        hipStream_t s = static_cast<hipStream_t>(stream);
        if (uses_matrix_cores(tile_count(w), m)) {
            if (w->k == 0) {
                const uint64_t cnt = static_cast<uint64_t>(m) * w->n;
                hipLaunchKernelGGL(fill_zero, dim3(static_cast<uint32_t>((cnt + 255) / 256)), dim3(256), 0, s, y, cnt);
                return launched(who);
            }
            return gemm_launch(who, &w, &y, 1, x, m, s);
        }
        // GEMV launches whose waves take rows_per_wave rows of X each
        const uint32_t rw = rows_per_wave(m, tile_count(w));
        const vbq_matrix *ws[VBQ_MAX_MULTI];
        const uint16_t *xs[VBQ_MAX_MULTI];
        float *ys[VBQ_MAX_MULTI];
        uint32_t cnt = 0;
        for (uint32_t r0 = 0; r0 < m; r0 += rw) {
            ws[cnt] = w;
            xs[cnt] = x + static_cast<uint64_t>(r0) * w->k;
            ys[cnt] = y + static_cast<uint64_t>(r0) * w->n;
            if (++cnt == VBQ_MAX_MULTI || r0 + rw >= m) {
                st = gemv_launch(who, ws, xs, ys, cnt, s, nullptr, nullptr, false, rw);
                if (st != VBQ_OK) return st;
                cnt = 0;
            }
        }
        return VBQ_OK;
    });
}

// Small-batch products of several matrices that read the same rows of X
// (q, k, v; gate, up). The small-batch rule is applied to all of them
// together: on the matrix cores they share launches of up to kGemmMulti
// matrices (the launch's latency is paid once), otherwise each becomes
// GEMVs of one or two rows of X per wave (rows_per_wave, on the tiles of
// all of them), and those share launches of up to VBQ_MAX_MULTI entries,
// matrix by matrix and row by row.
extern "C" vbq_status vbq_gemm_smallbatch_multi(const vbq_matrix *const *ws, const uint16_t *x, uint32_t m,
                                                float *const *ys, uint32_t count, void *stream) {
    return vbq::guarded("vbq_gemm_smallbatch_multi", [&]() -> vbq_status {
        vbq::clear_error();
        const char *who = "vbq_gemm_smallbatch_multi";
        if (m == 0 || m > VBQ_MAX_BATCH) return fail(VBQ_ERR_SHAPE, "%s: m=%u outside [1, %u]", who, m, VBQ_MAX_BATCH);
        if (count == 0) return VBQ_OK;
        if (!ws || !ys) return fail(VBQ_ERR_NULL, "%s: ws or ys is NULL", who);
        for (uint32_t i = 0; i < count; ++i) {
            vbq_status st = check_matrix(who, ws[i]);
            if (st != VBQ_OK) return st;
            if (ws[i]->k != ws[0]->k)
                return fail(VBQ_ERR_SHAPE, "%s: matrix %u has k=%u, matrix 0 k=%u (they share X)", who, i, ws[i]->k,
                            ws[0]->k);
            st = check_vectors(who, ws[i], x, ys[i]);
            if (st != VBQ_OK) return st;
        }
        (void)hipGetLastError();
        hipStream_t s = static_cast<hipStream_t>(stream);
        const uint32_t k = ws[0]->k;
        uint64_t tiles = 0;
        for (uint32_t i = 0; i < count; ++i) tiles += tile_count(ws[i]);
        const uint32_t rw = rows_per_wave(m, tiles);
        const vbq_matrix *gw[VBQ_MAX_MULTI];
        const uint16_t *gx[VBQ_MAX_MULTI];
        float *gy[VBQ_MAX_MULTI];
        uint32_t pending = 0;
        auto flush = [&]() -> vbq_status {
            const vbq_status st = pending ? gemv_launch(who, gw, gx, gy, pending, s, nullptr, nullptr, false, rw) : VBQ_OK;
            pending = 0;
            return st;
        };
        // the rule on all the matrices together: on the matrix cores they share one launch
        if (uses_matrix_cores(tiles, m)) {
            const vbq_matrix *mw[kGemmMulti];
            float *my[kGemmMulti];
            uint32_t held = 0;
            for (uint32_t i = 0; i < count; ++i) {
                const vbq_matrix *w = ws[i];
                if (w->n == 0) continue;
                if (k == 0) {
                    const uint64_t cnt = static_cast<uint64_t>(m) * w->n;
                    hipLaunchKernelGGL(fill_zero, dim3(static_cast<uint32_t>((cnt + 255) / 256)), dim3(256), 0, s,
                                       ys[i], cnt);
                    const vbq_status st = launched(who);
                    if (st != VBQ_OK) return st;
                    continue;
                }
                mw[held] = w;
                my[held] = ys[i];
                if (++held == kGemmMulti || i + 1 == count) {
                    const vbq_status st = gemm_launch(who, mw, my, held, x, m, s);
                    if (st != VBQ_OK) return st;
                    held = 0;
                }
            }
            return held ? gemm_launch(who, mw, my, held, x, m, s) : VBQ_OK;
        }
        for (uint32_t i = 0; i < count; ++i) {
            const vbq_matrix *w = ws[i];
            if (w->n == 0) continue;
            for (uint32_t r = 0; r < m; r += rw) {
                gw[pending] = w;
                gx[pending] = x + static_cast<uint64_t>(r) * k;
                gy[pending] = ys[i] + static_cast<uint64_t>(r) * w->n;
                if (++pending == VBQ_MAX_MULTI) {
                    const vbq_status st = flush();
                    if (st != VBQ_OK) return st;
                }
            }
        }
        return flush();
    });
}

extern "C" vbq_status vbq_build_stream_index(const vbq_matrix *w, uint8_t *index_out, void *stream) {
    return vbq::guarded("vbq_build_stream_index", [&]() -> vbq_status {
        vbq::clear_error();
        const char *who = "vbq_build_stream_index";
        vbq_status st = check_matrix(who, w);
        if (st != VBQ_OK) return st;
        if (w->n == 0 || w->k == 0) return VBQ_OK;
        if (!index_out) return fail(VBQ_ERR_NULL, "%s: index_out is NULL", who);
        if (!aligned16(index_out)) return fail(VBQ_ERR_ALIGN, "%s: index_out is not 16-byte aligned", who);
        (void)hipGetLastError();
        MatArgs M{};
        M.payload_bytes = w->payload_bytes;
        M.widths = w->widths;
        M.scales = w->scales;
        M.tile_offsets = w->tile_offsets;
        M.payload = w->payload;
        M.n = w->n;
        M.groups = w->k / VBQ_GROUP;
        M.col_tiles = ceil_div(M.groups, kTileGroups);
        M.splits = 1;
        // fewer than 2^29 groups (the payload fits 32-bit offsets at 8 bytes or more a group), so the tile
        // count fits the grid
        const uint32_t tiles = ceil_div(M.n, kTileRows) * M.col_tiles;
        hipStream_t s = static_cast<hipStream_t>(stream);
        if (M.groups % 4 == 0)
            hipLaunchKernelGGL(stream_index_tiles<true>, dim3(tiles), dim3(64), 0, s, M, index_out, uint64_t(tiles));
        else
            hipLaunchKernelGGL(stream_index_tiles<false>, dim3(tiles), dim3(64), 0, s, M, index_out, uint64_t(tiles));
        return launched(who);
    });
}

extern "C" vbq_status vbq_unpack_codes(const vbq_matrix *w, int8_t *codes_out, void *stream) {
    return vbq::guarded("vbq_unpack_codes", [&]() -> vbq_status {
        vbq::clear_error();
        vbq_status st = check_matrix("vbq_unpack_codes", w);
        if (st != VBQ_OK) return st;
        if (w->n == 0 || w->k == 0) return VBQ_OK;
        if (!codes_out) return fail(VBQ_ERR_NULL, "vbq_unpack_codes: codes_out is NULL");
        if (!aligned16(codes_out)) return fail(VBQ_ERR_ALIGN, "vbq_unpack_codes: codes_out is not 16-byte aligned");
        (void)hipGetLastError();
        MatArgs M{};
        M.payload_bytes = w->payload_bytes;
        M.widths = w->widths;
        M.scales = w->scales;
        M.tile_offsets = w->tile_offsets;
        M.payload = w->payload;
        M.n = w->n;
        M.groups = w->k / VBQ_GROUP;
        M.col_tiles = ceil_div(M.groups, kTileGroups);
        M.splits = 1;
        const uint32_t tiles = ceil_div(M.n, kTileRows) * M.col_tiles;
        hipStream_t s = static_cast<hipStream_t>(stream);
        if (M.groups % 4 == 0)
            hipLaunchKernelGGL(unpack_tiles<true>, dim3(tiles), dim3(64), 0, s, M, codes_out);
        else
            hipLaunchKernelGGL(unpack_tiles<false>, dim3(tiles), dim3(64), 0, s, M, codes_out);
        return launched("vbq_unpack_codes");
    });
}
