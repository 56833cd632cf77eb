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

#include "vbq_internal.h"

using vbq::fail;

namespace {

constexpr uint32_t kWave = 64;
constexpr uint32_t kTileRows = VBQ_TILE_ROWS;     // 64
constexpr uint32_t kTileGroups = VBQ_TILE_GROUPS; // 4
constexpr uint32_t kWavesPerBlock = 4;
constexpr uint32_t kXStride = 36;                 // dwords per staged column (32 used, padded)
constexpr uint32_t kMagic = 0x64006400u;          // two fp16 1024.0

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
// (1024 + 2^s * u) where u = q + 2^(b-1) is the offset-binary code; the pairs
// come out in natural element order (2i, 2i+1) thanks to the in-group field
// layout, and multiply fp16 activation pairs with v_dot2.

// 8-bit: elements 4w..4w+3 -> pairs (0,1), (2,3); factor 1
__device__ __forceinline__ void unpack8(uint32_t v, uint32_t &p0, uint32_t &p1) {
    v ^= 0x80808080u;
    p0 = __builtin_amdgcn_perm(0x64646464u, v, 0x04010400u);   // bytes {v0, 64, v1, 64}
    p1 = __builtin_amdgcn_perm(0x64646464u, v, 0x04030402u);   // bytes {v2, 64, v3, 64}
}

// 4-bit: elements 8w..8w+7 -> pairs (0,1) x1, (2,3) x16, (4,5) x1, (6,7) x16.
// magic holds kMagic in a register so each pair is one mask-and-or.
__device__ __forceinline__ void unpack4(uint32_t v, uint32_t magic, uint32_t p[4]) {
    v = xor_opaque(v, 0x88888888u);
    const uint32_t h = v >> 8;
    p[0] = (v & 0x000F000Fu) | magic;
    p[1] = (v & 0x00F000F0u) | magic;
    p[2] = (h & 0x000F000Fu) | magic;
    p[3] = (h & 0x00F000F0u) | magic;
}

// 2-bit: elements 16w..16w+15 -> pairs m = 0..7 with factors 1,4,16,64,256,1,4,16
__device__ __forceinline__ void unpack2(uint32_t v, uint32_t magic, uint32_t p[8]) {
    v = xor_opaque(v, 0xAAAAAAAAu);
    const uint32_t h = v >> 10;
    p[0] = (v & 0x00030003u) | magic;
    p[1] = (v & 0x000C000Cu) | magic;
    p[2] = (v & 0x00300030u) | magic;
    p[3] = (v & 0x00C000C0u) | magic;
    p[4] = (v & 0x03000300u) | magic;
    p[5] = (h & 0x00030003u) | magic;
    p[6] = (h & 0x000C000Cu) | magic;
    p[7] = (h & 0x00300030u) | magic;
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
    uint32_t *counters;   // [row tiles] arrival counters when splits > 1 (self-resetting)
    uint32_t n, groups, col_tiles, splits, blocks;   // blocks = row tiles x splits
    uint32_t payload_bytes;
    uint32_t ubits;   // the matrix's declared single width, or 0
    uint16_t *y16;    // when set, y is stored here as fp16 (nearest even) instead of fp32 to y
};


// Launched as a 2D grid: blockIdx.y picks the matrix, so a block loads its
// matrix's arguments with one scalar load and no search.
struct Batch {
    MatArgs m[VBQ_MAX_MULTI];
    // Gated-MLP epilogue, when h is set: matrix 0 is gate and matrix 1 is up
    // (same n), and instead of y the launch writes h = fp16(silu(g) * u).
    uint16_t *h;
    float *pair;              // [2][n]: each row tile's finished g and u values
    uint32_t *pair_counters;  // [row tiles] arrival counters (self-resetting)
};

// 4992 bytes per wave: eight 4-wave, four 8-wave or two 16-wave workgroups
// fit one CU's 160 KiB.
struct alignas(16) WaveLds {
    union {
        float lut[kTileGroups * 16 * 16];     // [column][nibble position][4-bit index]
        float part[kTileGroups * kTileRows];  // group dot products (unscaled) at column * 64 + row, once
                                              // the 1-bit groups are done
    };
    uint32_t xs[kTileGroups * kXStride];     // fp16 activation pairs per column
    float corr[kTileGroups][4];              // per column: sum x, 2-bit and 4-bit bias terms
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
                                              bool with_x) {
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
            t.codes = M.widths[(base >> 2) + lr];
            const uint2 sv =
                *reinterpret_cast<const uint2 *>(reinterpret_cast<const char *>(M.scales) + 2u * (base + 4u * lr));
            t.s01 = sv.x;
            t.s23 = sv.y;
        } else {
            const uint64_t g = base + static_cast<uint64_t>(lr) * cn;
            const uint64_t wbytes = (static_cast<uint64_t>(M.n) * M.groups + 3) >> 2;
            uint32_t two = M.widths[g >> 2];
            if ((g >> 2) + 1 < wbytes) two |= static_cast<uint32_t>(M.widths[(g >> 2) + 1]) << 8;
            t.codes = (two >> (2 * (g & 3))) & ((1u << (2 * cn)) - 1u);
            uint32_t sc[4] = {0u, 0u, 0u, 0u};
            for (uint32_t q = 0; q < cn; ++q) sc[q] = M.scales[g + q];
            t.s01 = sc[0] | (sc[1] << 16);
            t.s23 = sc[2] | (sc[3] << 16);
        }
    }
    return t;
}

// Stage the tile's activations: fp16 pairs, the 4-bit lookup table (sums of
// the activations selected by the set bits of a 4-bit index) and the
// per-column bias terms of the unpack paths.
template <bool kLut = true>
__device__ __forceinline__ void stage_x(WaveLds &L, uint2 xv, uint32_t lane, float wa, float wb) {
    const uint32_t jl = lane >> 4, k = lane & 15;
    L.xs[jl * kXStride + 2 * k] = xv.x;
    L.xs[jl * kXStride + 2 * k + 1] = xv.y;
    const float x0 = half_to_float(xv.x & 0xFFFFu), x1 = half_to_float(xv.x >> 16);
    const float x2 = half_to_float(xv.y & 0xFFFFu), x3 = half_to_float(xv.y >> 16);
    const float a01 = x0 + x1, t5 = x2 + x0, t6 = x2 + x1, t7 = x2 + a01;
    if (kLut) {
        float4 *t = reinterpret_cast<float4 *>(L.lut + lane * 16);
        t[0] = make_float4(0.f, x0, x1, a01);
        t[1] = make_float4(x2, t5, t6, t7);
        t[2] = make_float4(x3, x3 + x0, x3 + x1, x3 + a01);
        t[3] = make_float4(x3 + x2, x3 + t5, x3 + t6, x3 + t7);
    }
    // bias terms. 4-bit: element pairs alternate factor 1 / 16 -> weights 1032 / 72.
    // 2-bit: pair factors 1,4,16,64,256,1,4,16 -> weights 1024/f + 2.
    const float a23 = x2 + x3;
    float xsum = a01 + a23;
    // explicit fma: every kernel that stages x rounds these the same way, whatever the compiler
    // would contract in its own context
    float c4 = fmaf(1032.f, a01, 72.f * a23);
    float c2 = fmaf(wa, a01, wb * a23);
    xsum = row16_sum(xsum);
    c2 = row16_sum(c2);
    c4 = row16_sum(c4);
    if (k == 0) {
        L.corr[jl][0] = xsum;
        L.corr[jl][1] = c2;
        L.corr[jl][2] = c4;
    }
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
__device__ __forceinline__ void build_lists(WaveLds &L, const TileMeta &t, const TileScan &T, const uint32_t cnt[4],
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

// returns the product: L.part shares its bytes with the lookup table, so it
// is stored once every 1-bit group of the tile is done
__device__ __forceinline__ float group1(WaveLds &L, uint32_t info, uint2 v) {
    const uint32_t jl = info >> 6;
    // table k (one per 4 activations) starts at byte 64k; the entry for nibble u is at +4u.
    // Bytes of lo/hi hold 4 * (nibble 2t / 2t+1) of each word.
    const char *lut = reinterpret_cast<const char *>(L.lut + jl * 256u);
    const uint32_t w[2] = {v.x, v.y};
    float acc[4];
#pragma unroll
    for (uint32_t q = 0; q < 2; ++q) {
        uint32_t lo, hi;
        asm("v_lshlrev_b32 %0, 2, %1\n\tv_and_b32 %0, 0x3c3c3c3c, %0" : "=&v"(lo) : "v"(w[q]));
        asm("v_lshrrev_b32 %0, 2, %1\n\tv_and_b32 %0, 0x3c3c3c3c, %0" : "=&v"(hi) : "v"(w[q]));
#pragma unroll
        for (uint32_t t = 0; t < 4; ++t) {
            const uint32_t k = 8 * q + 2 * t;
            const float a = *reinterpret_cast<const float *>(lut + 64u * k + ((lo >> (8 * t)) & 0xFFu));
            const float b = *reinterpret_cast<const float *>(lut + 64u * (k + 1) + ((hi >> (8 * t)) & 0xFFu));
            acc[t] = q == 0 ? a + b : acc[t] + (a + b);
        }
    }
    const float sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    return L.corr[jl][0] - 2.f * sum;
}

// unscaled product of one 2-bit group of column jl
__device__ __forceinline__ float dot2bit(WaveLds &L, uint32_t jl, uint2 va, uint2 vb) {
    const uint32_t w[4] = {va.x, va.y, vb.x, vb.y};
    const uint4 *xp = reinterpret_cast<const uint4 *>(L.xs + jl * kXStride);
    const uint32_t magic = opaque(kMagic);
    float a1 = 0.f, a4 = 0.f, a16 = 0.f, a64 = 0.f, a256 = 0.f;
#pragma unroll
    for (uint32_t q = 0; q < 4; ++q) {
        uint32_t p[8];
        unpack2(w[q], magic, p);
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
    return a1 + 0.25f * a4 + 0.0625f * a16 + 0.015625f * a64 + 0.00390625f * a256 - L.corr[jl][1];
}

__device__ __forceinline__ void group2(WaveLds &L, uint32_t info, uint2 va, uint2 vb) {
    store_part(L, info, dot2bit(L, info >> 6, va, vb));
}

// 4-bit: a 16-byte half group (h = task & 1); lane pairs add their halves
// 4-bit: a 16-byte half group (h = 0, 1) of column jl, without the bias term
__device__ __forceinline__ float half4bit(WaveLds &L, uint32_t jl, uint32_t h, uint2 va, uint2 vb) {
    const uint32_t w[4] = {va.x, va.y, vb.x, vb.y};
    const uint4 *xp = reinterpret_cast<const uint4 *>(L.xs + jl * kXStride + 16u * h);
    const uint32_t magic = opaque(kMagic);
    float a1 = 0.f, a16 = 0.f;
#pragma unroll
    for (uint32_t q = 0; q < 4; ++q) {
        uint32_t p[4];
        unpack4(w[q], magic, p);
        const uint4 xa = xp[q];
        a1 = dot2(p[0], xa.x, a1);
        a16 = dot2(p[1], xa.y, a16);
        a1 = dot2(p[2], xa.z, a1);
        a16 = dot2(p[3], xa.w, a16);
    }
    return a1 + 0.0625f * a16;
}

__device__ __forceinline__ void task4(WaveLds &L, uint32_t info, uint32_t h, uint2 va, uint2 vb) {
    const uint32_t jl = info >> 6;
    float part = half4bit(L, jl, h, va, vb);
    part += dpp<kQuadXor1>(part);
    if (h == 0) store_part(L, info, part - L.corr[jl][2]);
}

// 8-bit: a 16-byte quarter group (qd = task & 3); lane quads add their quarters
// 8-bit: a 16-byte quarter group (qd = 0..3) of column jl, without the bias term
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

__device__ __forceinline__ void task8(WaveLds &L, uint32_t info, uint32_t qd, uint2 va, uint2 vb) {
    const uint32_t jl = info >> 6;
    float a = quarter8bit(L, jl, qd, va, vb);
    a += dpp<kQuadXor1>(a);
    a += dpp<kQuadXor2>(a);
    if (qd == 0) store_part(L, info, fmaf(-1152.f, L.corr[jl][0], a));
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

// Staged work first, then the rounds that load their own bytes (rare: more
// than 64 two-bit groups or 64 slices of a wider width in one tile).
__device__ __forceinline__ void tile_products(WaveLds &L, const Staged &S, rsrc_t tile, const uint32_t cnt[4],
                                              uint32_t lane) {
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
        if (on) v1[i] = group1(L, e, S.p1[i]);
    }
    // the lookup table is dead from here: its bytes take the products
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i) store_part(L, info1[i], v1[i]);
    const uint32_t o2 = 8u * cnt[0], o4 = o2 + 16u * cnt[1], o8 = o4 + 32u * cnt[2];
    const uint8_t *l2 = L.list + cnt[0], *l4 = l2 + cnt[1], *l8 = l4 + cnt[2];
    if (lane < cnt[1]) group2(L, l2[lane], S.p2a, S.p2b);
    if (lane < 2u * cnt[2]) task4(L, l4[lane >> 1], lane & 1u, S.p4a, S.p4b);
    if (lane < 4u * cnt[3]) task8(L, l8[lane >> 2], lane & 3u, S.p8a, S.p8b);
    for (uint32_t e = lane + kWave; e < cnt[1]; e += kWave)
        group2(L, l2[e], buf_load8(tile, o2 + 16u * e), buf_load8(tile, o2 + 16u * e + 8u));
    for (uint32_t e = lane + kWave; e < 2u * cnt[2]; e += kWave)
        task4(L, l4[e >> 1], e & 1u, buf_load8(tile, o4 + 16u * e), buf_load8(tile, o4 + 16u * e + 8u));
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
    if (lane == 0) arrived = __hip_atomic_fetch_add(&B.pair_counters[a], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    arrived = __shfl(arrived, 0, kWave);
    if (arrived != 1) return;
    if (live) {
        const float o = __hip_atomic_load(&B.pair[static_cast<uint64_t>(1 - which) * n + row], __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
        B.h[row] = which == 0 ? swiglu_half(v, o) : swiglu_half(o, v);
    }
    if (lane == 0) __hip_atomic_store(&B.pair_counters[a], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The workgroup's row sums (waves added in wave order), the split-K
// reduction when the row tile is split, then y or the gated-MLP epilogue.
template <uint32_t kWaves>
__device__ __forceinline__ void finish_row_tile(const Batch &B, const MatArgs &M, uint32_t which, WaveLds *lds,
                                                uint32_t wave, bool spare, uint32_t a, uint32_t split, uint32_t r0,
                                                uint32_t rows, uint32_t lane, float acc) {
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
            arrived = __hip_atomic_fetch_add(&M.counters[a], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        arrived = __shfl(arrived, 0, kWave);
        if (arrived != M.splits - 1) return;
        if (lane < rows) sum = sum_partials(M.partial + r0 + lane, M.n, M.splits);
        if (lane == 0) __hip_atomic_store(&M.counters[a], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!B.h) {
        if (lane < rows) {
            if (M.y16)
                M.y16[r0 + lane] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(sum));
            else
                M.y[r0 + lane] = sum;
        }
        return;
    }
    swiglu_pair(B, which, a, r0 + lane, lane < rows, M.n, lane, sum);
}

// kWaves waves per workgroup (4, 8 or 16) share one row tile; the LDS
// (4992 B per wave) allows 8, 4 or 2 such workgroups per CU, eight waves
// per SIMD, and the registers are held to the 64 that allow the same.
// kExit: the launch's matrices differ in size, so workgroups past a smaller matrix's end leave at once
// (all seven 9B-layer matrices in one launch: 32.9 -> 23.7 us); launches of equal matrices have none and
// skip the test, which would put a dependent load ahead of the others (about 0.7 us a step).
template <bool kAligned, uint32_t kWaves, bool kExit>
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
    // 2-bit bias weights of this lane's activation pairs (pair factors 1,4,16,64,256,1,4,16: 1024/f + 2)
    const uint32_t km = lane0 & 3u;
    const float wa = km == 0 ? 1026.f : km == 1 ? 66.f : km == 2 ? 6.f : 258.f;
    const float wb = km == 0 ? 258.f : km == 1 ? 18.f : km == 2 ? 1026.f : 66.f;
    uint32_t ct = c_lo + wave;
    // metadata loads are unconditional (a wave without a next tile reloads its
    // own): a conditional load would make its result a branch merge, and the
    // merge copy would wait for the load
    TileMeta cur = load_meta<kAligned>(M, a, ct < c_hi ? ct : c_lo, relane(lane0), true);
    for (; ct < c_hi; ct += kWaves) {
        const uint32_t cn = kAligned ? kTileGroups : min(kTileGroups, M.groups - ct * kTileGroups);
        // counts first: the payload loads leave before the tables and lists are built
        uint32_t cnt[4];
        const TileScan P = tile_scan(cur, rows, cn, relane(lane0), cnt);
        const rsrc_t tp = tile_rsrc(M.payload, M.payload_bytes, cur.off);
        Staged S;
        stage_payload(tp, cnt, relane(lane0), S);
        // the next tile's metadata travels while this tile computes
        const TileMeta nxt =
            load_meta<kAligned>(M, a, ct + kWaves < c_hi ? ct + kWaves : ct, relane(lane0), true);
        stage_x(L, cur.xv, relane(lane0), wa, wb);
        build_lists(L, cur, P, cnt, rows, cn, relane(lane0));
        wave_lds_sync();
        tile_products(L, S, tp, cnt, relane(lane0));
        wave_lds_sync();
        const uint32_t lane = relane(lane0);
        if (lane < rows)
            for (uint32_t jl = 0; jl < cn; ++jl) {
                const uint32_t sb = (jl < 2 ? cur.s01 >> (16 * jl) : cur.s23 >> (16 * (jl - 2))) & 0xFFFFu;
                acc = fmaf(half_to_float(sb), L.part[jl * kTileRows + lane], acc);
            }
        wave_lds_sync();
        cur = nxt;
    }
    finish_row_tile<kWaves>(B, M, blockIdx.y, lds, wave, spare, a, split, r0, rows, relane(lane0), acc);
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
__device__ __forceinline__ float row_group_dot(WaveLds &L, uint32_t jl, const RowGroups<kBits> &g) {
    if (kBits == 1) return group1(L, jl << 6, make_uint2(g.v[0].x, g.v[0].y));
    if (kBits == 2) return dot2bit(L, jl, make_uint2(g.v[0].x, g.v[0].y), make_uint2(g.v[0].z, g.v[0].w));
    if (kBits == 4)
        return (half4bit(L, jl, 0, make_uint2(g.v[0].x, g.v[0].y), make_uint2(g.v[0].z, g.v[0].w)) +
                half4bit(L, jl, 1, make_uint2(g.v[1].x, g.v[1].y), make_uint2(g.v[1].z, g.v[1].w))) -
               L.corr[jl][2];
    // quarters added as the mixed kernel's lane quads add them, so both kernels give the same bits
    float q[4];
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i)
        q[i] = quarter8bit(L, jl, i, make_uint2(g.v[i & (kBits / 2 - 1)].x, g.v[i & (kBits / 2 - 1)].y),
                           make_uint2(g.v[i & (kBits / 2 - 1)].z, g.v[i & (kBits / 2 - 1)].w));
    return fmaf(-1152.f, L.corr[jl][0], (q[0] + q[1]) + (q[2] + q[3]));
}

// kLean: hold two 4-bit groups of a row at once instead of four (the per-matrix-width kernel, whose
// register budget is the largest of its four paths plus the dispatch)
template <uint32_t kBits, bool kAligned, uint32_t kWaves, bool kLean = false>
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
    const uint32_t c_lo = (split * M.col_tiles) / M.splits, c_hi = ((split + 1) * M.col_tiles) / M.splits;
    WaveLds &L = lds[wave];
    float acc = 0.f;
    const uint32_t lane0 = lane_id();
    const uint32_t km = lane0 & 3u;
    const float wa = km == 0 ? 1026.f : km == 1 ? 66.f : km == 2 ? 6.f : 258.f;
    const float wb = km == 0 ? 258.f : km == 1 ? 18.f : km == 2 ? 1026.f : 66.f;
    constexpr uint32_t kChunk = kBits == 8 ? 1 : (kBits == 4 && kLean) ? 2 : kTileGroups;   // groups held at once
    uint32_t ct = c_lo + wave;
    TileMeta cur = load_meta<kAligned>(M, a, ct < c_hi ? ct : c_lo, relane(lane0), true);
    for (; ct < c_hi; ct += kWaves) {
        const uint32_t cn = kAligned ? kTileGroups : min(kTileGroups, M.groups - ct * kTileGroups);
        const uint32_t lr = min(relane(lane0), rows - 1);
        const uint32_t tile_off = 8u * kBits * (r0 * M.groups + rows * kTileGroups * ct);
        const rsrc_t tp = tile_rsrc(M.payload, M.payload_bytes, tile_off);
        RowGroups<kBits> g[kChunk];
#pragma unroll
        for (uint32_t jl = 0; jl < kChunk; ++jl)
            g[jl] = load_row_group<kBits>(tp, (min(jl, cn - 1) * rows + lr) * 8u * kBits);
        const TileMeta nxt =
            load_meta<kAligned>(M, a, ct + kWaves < c_hi ? ct + kWaves : ct, relane(lane0), true);
        stage_x<kBits == 1>(L, cur.xv, relane(lane0), wa, wb);
        wave_lds_sync();
        const uint32_t lane = relane(lane0);
#pragma unroll
        for (uint32_t c0 = 0; c0 < kTileGroups; c0 += kChunk) {
            if (c0 > 0) {
#pragma unroll
                for (uint32_t jl = 0; jl < kChunk; ++jl)
                    g[jl] = load_row_group<kBits>(tp, (min(c0 + jl, cn - 1) * rows + lr) * 8u * kBits);
            }
#pragma unroll
            for (uint32_t jl = 0; jl < kChunk; ++jl) {
                const uint32_t j = c0 + jl;
                const uint32_t sb = (j < 2 ? cur.s01 >> (16 * j) : cur.s23 >> (16 * (j - 2))) & 0xFFFFu;
                const float d = row_group_dot<kBits>(L, j, g[jl]);
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
// the workgroup, so there is no divergence.
template <bool kAligned, uint32_t kWaves>
__global__ __launch_bounds__(kWaves * kWave) __attribute__((amdgpu_waves_per_eu(8, 8))) void gemv_uniform_mixed(
    Batch B) {
    __shared__ WaveLds lds[kWaves];
    const uint32_t which = blockIdx.y, bx = blockIdx.x;
    const MatArgs M = B.m[which];
    switch (M.ubits) {
        case 1: uniform_tiles<1, kAligned, kWaves>(B, M, which, bx, lds); break;
        case 2: uniform_tiles<2, kAligned, kWaves>(B, M, which, bx, lds); break;
        case 4: uniform_tiles<4, kAligned, kWaves, true>(B, M, which, bx, lds); break;
        default: uniform_tiles<8, kAligned, kWaves>(B, M, which, bx, lds); break;
    }
}

// Decoded codes of every group, written at its natural position; the same
// field decoders as the product kernels (fp16 pairs 1024 + 2^s*u, then exact
// integer recovery) plus the sign bits of 1-bit groups.
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
                    unpack2(v, opaque(kMagic), p);
                    const float f[8] = {1.f, 4.f, 16.f, 64.f, 256.f, 1.f, 4.f, 16.f};
                    uint32_t outw[4] = {0, 0, 0, 0};
                    for (uint32_t m = 0; m < 8; ++m) {
                        const int qa = static_cast<int>((half_to_float(p[m] & 0xFFFFu) - 1024.f) / f[m]) - 2;
                        const int qb = static_cast<int>((half_to_float(p[m] >> 16) - 1024.f) / f[m]) - 2;
                        const uint32_t e0 = 2 * m, e1 = 2 * m + 1;
                        outw[e0 >> 2] |= (static_cast<uint32_t>(qa) & 0xFFu) << (8 * (e0 & 3));
                        outw[e1 >> 2] |= (static_cast<uint32_t>(qb) & 0xFFu) << (8 * (e1 & 3));
                    }
                    for (uint32_t o = 0; o < 4; ++o) dst[wd * 4 + o] = outw[o];
                } else if (b == 4) {
                    uint32_t p[4];
                    unpack4(v, opaque(kMagic), p);
                    uint32_t outw[2] = {0, 0};
                    for (uint32_t m = 0; m < 4; ++m) {
                        const float f = (m & 1) ? 16.f : 1.f;
                        const int qa = static_cast<int>((half_to_float(p[m] & 0xFFFFu) - 1024.f) / f) - 8;
                        const int qb = static_cast<int>((half_to_float(p[m] >> 16) - 1024.f) / f) - 8;
                        const uint32_t e0 = 2 * m, e1 = 2 * m + 1;
                        outw[e0 >> 2] |= (static_cast<uint32_t>(qa) & 0xFFu) << (8 * (e0 & 3));
                        outw[e1 >> 2] |= (static_cast<uint32_t>(qb) & 0xFFu) << (8 * (e1 & 3));
                    }
                    dst[wd * 2] = outw[0];
                    dst[wd * 2 + 1] = outw[1];
                } else {
                    uint32_t p0, p1;
                    unpack8(v, p0, p1);
                    const int q0 = static_cast<int>(half_to_float(p0 & 0xFFFFu)) - 1152;
                    const int q1 = static_cast<int>(half_to_float(p0 >> 16)) - 1152;
                    const int q2 = static_cast<int>(half_to_float(p1 & 0xFFFFu)) - 1152;
                    const int q3 = static_cast<int>(half_to_float(p1 >> 16)) - 1152;
                    dst[wd] = (static_cast<uint32_t>(q0) & 0xFFu) | ((static_cast<uint32_t>(q1) & 0xFFu) << 8) |
                              ((static_cast<uint32_t>(q2) & 0xFFu) << 16) | ((static_cast<uint32_t>(q3) & 0xFFu) << 24);
                }
            }
        }
        base += 8u * b * cnt[wsel];
        first += cnt[wsel];
    }
}

__global__ void fill_zero(float *__restrict__ y, uint64_t count) {
    const uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < count) y[i] = 0.f;
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

// When the matrix cores run a small batch (measured on MI355X, graph-replayed):
// the matrix-core kernel costs about the same for any m up to 16, while m
// GEMVs in one launch cost more with every row, less so on small matrices
// whose launches leave the chip idle. The crossover row count falls with the
// tile count roughly as 1/sqrt(tiles): the matrix cores win from m = 4 rows
// when m^2 x tiles reaches 85000 (LM head 32000x4096, 8000 tiles: m = 3 24.9
// vs 27.6 us as GEMVs, m = 4 27.4 vs 31.3 on the matrix cores; 14336x4096:
// m = 4 19.2 vs 20.0 as GEMVs, m = 6 20.4 vs 25.7; 4096x4096: m = 8 11.1 vs
// 12.2 as GEMVs, m = 12 12.7 vs 15.6), and always beyond the 16 rows one GEMV
// launch takes.
constexpr uint32_t kGemmMinBatch = 4;
constexpr uint64_t kGemmMinWork = 85000;   // rows of X squared times tiles of W
constexpr uint32_t kAStride = 136;   // fp16 per staged row: two columns of 64 codes + 8 pad (272 B)

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

struct alignas(16) GemmWaveLds {
    uint16_t a[kTileRows * kAStride];            // decoded codes of two columns, exact fp16, row-major
    float scale[kTileGroups][kTileRows];         // group scales as fp32 [column][row]
    uint8_t list[4][kTileRows * kTileGroups];    // per width: row | column << 6, in bucket order
};

__device__ __forceinline__ uint32_t half2_fma(uint32_t v, uint32_t mul, uint32_t add) {
    const half2_t r = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, v), __builtin_bit_cast(half2_t, mul),
                                                __builtin_bit_cast(half2_t, add));
    return __builtin_bit_cast(uint32_t, r);
}

// fp16 pair constants: (mul, add) turn 1024 + f*u into u - bias exactly
constexpr uint32_t h2(uint32_t h) { return h | (h << 16); }

// 1-bit group (8 payload bytes) -> 64 codes +-1 at dst
__device__ __forceinline__ void decode1(uint2 v, uint16_t *dst) {
    const uint32_t ones = opaque(0x3C003C00u);
#pragma unroll
    for (uint32_t t = 0; t < 8; ++t) {
        const uint32_t w = t < 4 ? v.x : v.y;
        const uint32_t sel = (t & 3u) | 0x0C000000u | 0x00000C00u | ((t & 3u) << 16);
        const uint32_t d = __builtin_amdgcn_perm(0u, w, sel);          // {byte t, 0, byte t, 0}
        uint32_t o[4];
#pragma unroll
        for (uint32_t p = 0; p < 4; ++p) {
            const ushort2_t sh = {static_cast<uint16_t>(15 - 2 * p), static_cast<uint16_t>(14 - 2 * p)};
            const uint32_t s = __builtin_bit_cast(uint32_t, __builtin_bit_cast(ushort2_t, d) << sh);
            o[p] = (s & 0x80008000u) | ones;                           // sign bits 2p, 2p+1 -> fp16 +-1
        }
        *reinterpret_cast<uint4 *>(dst + 8 * t) = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// 2-bit group (16 payload bytes) -> 64 codes at dst
__device__ __forceinline__ void decode2(uint4 v, uint16_t *dst) {
    // offset binary: u = q + 2 in every field
    const uint32_t w[4] = {xor_opaque(v.x, 0xAAAAAAAAu), xor_opaque(v.y, 0xAAAAAAAAu), xor_opaque(v.z, 0xAAAAAAAAu),
                           xor_opaque(v.w, 0xAAAAAAAAu)};
    const uint32_t magic = opaque(kMagic);
    // pair p = fields p, p+8 -> 1024 + 4^p u (p < 5) or, from word >> 10, 1024 + 4^(p-5) u
    constexpr uint32_t mul[5] = {h2(0x3C00), h2(0x3400), h2(0x2C00), h2(0x2400), h2(0x1C00)};   // 4^-p
    constexpr uint32_t add[5] = {h2(0xE402), h2(0xDC08), h2(0xD420), h2(0xCC80), h2(0xC600)};   // -(1024/4^p + 2)
#pragma unroll
    for (uint32_t q = 0; q < 4; ++q) {
        const uint32_t lo = w[q], hi = w[q] >> 10;
        uint32_t o[8];
#pragma unroll
        for (uint32_t p = 0; p < 8; ++p) {
            const uint32_t src = p < 5 ? lo : hi, c = p < 5 ? p : p - 5;
            const uint32_t f = (src & (0x00030003u << (2 * c))) | magic;
            o[p] = half2_fma(f, mul[c], add[c]);
        }
        *reinterpret_cast<uint4 *>(dst + 16 * q) = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4 *>(dst + 16 * q + 8) = make_uint4(o[4], o[5], o[6], o[7]);
    }
}

// 16 payload bytes of a 4-bit group (32 elements) -> 32 codes at dst
__device__ __forceinline__ void decode4(uint4 v, uint16_t *dst) {
    // offset binary: u = q + 8 in every field
    const uint32_t w[4] = {xor_opaque(v.x, 0x88888888u), xor_opaque(v.y, 0x88888888u), xor_opaque(v.z, 0x88888888u),
                           xor_opaque(v.w, 0x88888888u)};
    const uint32_t magic = opaque(kMagic);
    constexpr uint32_t m1 = h2(0x3C00), a1 = h2(0xE408);    // 1, -(1024 + 8)
    constexpr uint32_t m16 = h2(0x2C00), a16 = h2(0xD480);  // 1/16, -(64 + 8)
#pragma unroll
    for (uint32_t q = 0; q < 4; ++q) {
        const uint32_t lo = w[q], hi = w[q] >> 8;
        const uint32_t o0 = half2_fma((lo & 0x000F000Fu) | magic, m1, a1);
        const uint32_t o1 = half2_fma((lo & 0x00F000F0u) | magic, m16, a16);
        const uint32_t o2 = half2_fma((hi & 0x000F000Fu) | magic, m1, a1);
        const uint32_t o3 = half2_fma((hi & 0x00F000F0u) | magic, m16, a16);
        *reinterpret_cast<uint4 *>(dst + 8 * q) = make_uint4(o0, o1, o2, o3);
    }
}

// 16 payload bytes of an 8-bit group (16 elements) -> 16 codes at dst
__device__ __forceinline__ void decode8(uint4 v, uint16_t *dst) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    constexpr uint32_t one = h2(0x3C00), a8 = h2(0xE480);   // 1, -(1024 + 128)
    uint32_t o[8];
#pragma unroll
    for (uint32_t q = 0; q < 4; ++q) {
        uint32_t p0, p1;
        unpack8(w[q], p0, p1);
        o[2 * q] = half2_fma(p0, one, a8);
        o[2 * q + 1] = half2_fma(p1, one, a8);
    }
    *reinterpret_cast<uint4 *>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<uint4 *>(dst + 8) = make_uint4(o[4], o[5], o[6], o[7]);
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

// Per-width lists of one tile (bucket order) from the tile scan, and the
// scales of the tile as fp32.
__device__ __forceinline__ void gemm_lists(GemmWaveLds &L, const TileMeta &t, const TileScan &T,
                                           const uint64_t colstart[kTileGroups + 1], uint32_t rows, uint32_t cn,
                                           uint32_t lane) {
    const bool valid = lane < rows;
#pragma unroll
    for (uint32_t jl = 0; jl < kTileGroups; ++jl) {
        if (jl >= cn) break;
        const uint32_t c = (t.codes >> (2 * jl)) & 3u;
        const uint32_t excl = T.incl[jl] - (1u << (8 * c));
        const uint32_t slot = field16(colstart[jl], c) + ((excl >> (8 * c)) & 0xFFu);
        if (valid) {
            L.list[c][slot] = static_cast<uint8_t>(lane | (jl << 6));
            const uint32_t sb = (jl < 2 ? (t.s01 >> (16 * jl)) : (t.s23 >> (16 * (jl - 2)))) & 0xFFFFu;
            L.scale[jl][lane] = half_to_float(sb);
        }
    }
}

// 16 payload bytes at an 8-byte aligned offset (buckets start at multiples of 8)
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t off) {
    const uint2 lo = buf_load8(r, off), hi = buf_load8(r, off + 8u);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
}


// Payload of one pass (two columns of a tile): the first 128 one-bit groups
// and the first 64 tasks of each wider width, loaded before any is decoded.
struct PassStage {
    uint2 p1[2];
    uint4 p2, p4, p8;
};

// List range [e0, e1) of width wi for the columns of `pass`, and the byte
// offset of that width's bucket in the tile.
__device__ __forceinline__ void pass_range(const uint64_t colstart[kTileGroups + 1], uint32_t pass, uint32_t cn,
                                           uint32_t wi, uint32_t &e0, uint32_t &e1, uint32_t &base) {
    const uint32_t c_end = min(2 * pass + 2, cn);
    e0 = field16(colstart[2 * pass], wi);
    e1 = field16(colstart[c_end], wi);
    const uint64_t total = colstart[kTileGroups];
    base = 0;
    for (uint32_t w = 0; w < wi; ++w) base += (8u << w) * field16(total, w);
}

__device__ __forceinline__ PassStage gemm_stage_pass(rsrc_t tile, const uint64_t colstart[kTileGroups + 1],
                                                     uint32_t pass, uint32_t cn) {
    const uint32_t lane = lane_id();
    // unconditional loads through the tile's descriptor (a lane without a task
    // reads later bytes, or zeros past the payload, and ignores them), so the
    // compiler counts them
    PassStage S;
    uint32_t e0, e1, base;
    pass_range(colstart, pass, cn, 0, e0, e1, base);
    S.p1[0] = buf_load8(tile, base + 8u * (e0 + lane));
    S.p1[1] = buf_load8(tile, base + 8u * (e0 + lane + kWave));
    pass_range(colstart, pass, cn, 1, e0, e1, base);
    S.p2 = buf_load16(tile, base + 16u * (e0 + lane));
    pass_range(colstart, pass, cn, 2, e0, e1, base);
    S.p4 = buf_load16(tile, base + 32u * e0 + 16u * lane);
    pass_range(colstart, pass, cn, 3, e0, e1, base);
    S.p8 = buf_load16(tile, base + 64u * e0 + 16u * lane);
    return S;
}

// Decode columns 2*pass and 2*pass+1 of the tile into L.a; tasks past the
// staged ones load their bytes here.
__device__ __forceinline__ void gemm_decode_pass(GemmWaveLds &L, const PassStage &S, rsrc_t tile,
                                                 const uint64_t colstart[kTileGroups + 1], uint32_t pass, uint32_t cn) {
    const uint32_t lane = lane_id();
#pragma unroll
    for (uint32_t wi = 0; wi < 4; ++wi) {
        const uint32_t b = 1u << wi;
        uint32_t e0, e1, base;
        pass_range(colstart, pass, cn, wi, e0, e1, base);
        const uint32_t tpg = wi < 2 ? 1u : (b >> 1);           // tasks per group: 1, 1, 2, 4
        const uint32_t tasks = (e1 - e0) * tpg;
        uint32_t round = 0;
        for (uint32_t t = lane; t < tasks; t += kWave, ++round) {
            const uint32_t e = e0 + t / tpg, sl = t % tpg;
            const uint32_t info = L.list[wi][e];
            const uint32_t r = info & 63u, jj = (info >> 6) - 2 * pass;
            uint16_t *dst = L.a + r * kAStride + 64u * jj;
            const uint32_t src = base + 8u * b * e;   // the group's byte offset in the tile
            if (wi == 0) {
                decode1(round == 0 ? S.p1[0] : round == 1 ? S.p1[1] : buf_load8(tile, src), dst);
            } else if (wi == 1) {
                decode2(round == 0 ? S.p2 : buf_load16(tile, src), dst);
            } else if (wi == 2) {
                decode4(round == 0 ? S.p4 : buf_load16(tile, src + 16u * sl), dst + 32u * sl);
            } else {
                decode8(round == 0 ? S.p8 : buf_load16(tile, src + 16u * sl), dst + 16u * sl);
            }
        }
    }
}

// Activations of one pass: lane holds X[16mb + lane%16][k .. k+7] for each
// column jj and half h of the pass. Rows past m and columns past the tile
// load a valid neighbour instead: the products they feed are never stored
// (a matrix-core output column depends on its own input column only) or
// never computed, and branch-free loads are waited for exactly.
template <uint32_t MB>
__device__ __forceinline__ void load_bx(const GemmArgs &G, uint32_t j0, uint32_t pass, uint32_t cn,
                                        half8_t bx[2][2][MB]) {
    const uint32_t lane = lane_id(), q = lane >> 4, mr = lane & 15u;
#pragma unroll
    for (uint32_t jj = 0; jj < 2; ++jj)
#pragma unroll
        for (uint32_t h = 0; h < 2; ++h)
#pragma unroll
            for (uint32_t mb = 0; mb < MB; ++mb) {
                const uint32_t m = min(16 * mb + mr, G.m - 1), jl = min(2 * pass + jj, cn - 1);
                const uint4 v = *reinterpret_cast<const uint4 *>(G.x + static_cast<uint64_t>(m) * G.k +
                                                                 64u * (j0 + jl) + 32u * h + 8u * q);
                bx[jj][h][mb] = __builtin_bit_cast(half8_t, v);
            }
}

// Codes of the pass (L.a) times activations, scaled per group, into acc.
template <uint32_t MB>
__device__ __forceinline__ void mfma_pass(const GemmWaveLds &L, const half8_t bx[2][2][MB], uint32_t pass,
                                          uint32_t cn, float4_t acc[4][MB]) {
    const uint32_t lane = lane_id(), q = lane >> 4, mr = lane & 15u;
#pragma unroll
    for (uint32_t jj = 0; jj < 2; ++jj) {
        const uint32_t jl = 2 * pass + jj;
        if (jl >= cn) break;
#pragma unroll
        for (uint32_t rb = 0; rb < 4; ++rb) {
            const uint16_t *arow = L.a + (16 * rb + mr) * kAStride + 64u * jj + 8u * q;
            const half8_t a0 = *reinterpret_cast<const half8_t *>(arow);
            const half8_t a1 = *reinterpret_cast<const half8_t *>(arow + 32);
            float4_t d[MB];
#pragma unroll
            for (uint32_t mb = 0; mb < MB; ++mb)
                d[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bx[jj][0][mb], float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0,
                                                               0);
#pragma unroll
            for (uint32_t mb = 0; mb < MB; ++mb)
                d[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bx[jj][1][mb], d[mb], 0, 0, 0);
            // rows 16rb + 4q .. +3 of this column
            const float4_t sc = *reinterpret_cast<const float4_t *>(&L.scale[jl][16 * rb + 4 * q]);
#pragma unroll
            for (uint32_t mb = 0; mb < MB; ++mb) acc[rb][mb] += sc * d[mb];
        }
    }
}

template <uint32_t MB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MB <= 2 ? 2 : 1, 8))) void gemm_tiles(GemmArgs G) {
    __shared__ GemmWaveLds lds[kWavesPerBlock];
    __shared__ uint32_t arrived_s;
    const uint32_t a = blockIdx.x / G.splits, split = blockIdx.x % G.splits;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x) / kWave;
    const uint32_t r0 = a * kTileRows;
    const uint32_t rows = min(kTileRows, G.n - r0);
    const uint32_t c_lo = (split * G.col_tiles) / G.splits, c_hi = ((split + 1) * G.col_tiles) / G.splits;
    GemmWaveLds &L = lds[wave];

    float4_t acc[4][MB];
#pragma unroll
    for (uint32_t rb = 0; rb < 4; ++rb)
#pragma unroll
        for (uint32_t mb = 0; mb < MB; ++mb) acc[rb][mb] = float4_t{0.f, 0.f, 0.f, 0.f};

    uint32_t ct = c_lo + wave;
    TileMeta cur = load_meta<false>(G, a, ct < c_hi ? ct : c_lo, lane_id(), false);
    for (; ct < c_hi; ct += kWavesPerBlock) {
        const uint32_t j0 = ct * kTileGroups, cn = min(kTileGroups, G.groups - j0);
        // counts first: every payload byte of the tile is requested before the lists are built
        uint32_t cnt[4];
        const TileScan T = tile_scan(cur, rows, cn, lane_id(), cnt);
        uint64_t colstart[kTileGroups + 1];
        column_starts(T, colstart);
        const rsrc_t tile = tile_rsrc(G.payload, G.payload_bytes, cur.off);
        const PassStage s0 = gemm_stage_pass(tile, colstart, 0, cn);
        const PassStage s1 = gemm_stage_pass(tile, colstart, cn > 2 ? 1 : 0, cn);
        half8_t bx[2][2][MB], bx1[2][2][MB];
        load_bx<MB>(G, j0, 0, cn, bx);
        if (MB <= 2) load_bx<MB>(G, j0, cn > 2 ? 1 : 0, cn, bx1);   // both passes' activations up front
        // the next tile's metadata travels while this tile computes
        const TileMeta nxt = load_meta<false>(G, a, ct + kWavesPerBlock < c_hi ? ct + kWavesPerBlock : ct,
                                              lane_id(), false);
        gemm_lists(L, cur, T, colstart, rows, cn, lane_id());
        wave_lds_sync();
        gemm_decode_pass(L, s0, tile, colstart, 0, cn);
        wave_lds_sync();
        mfma_pass<MB>(L, bx, 0, cn, acc);
        if (cn > 2) {
            wave_lds_sync();
            gemm_decode_pass(L, s1, tile, colstart, 1, cn);
            // (issued after the decode: its own loads of later rounds would otherwise wait for these)
            if (MB > 2) load_bx<MB>(G, j0, 1, cn, bx1);
            wave_lds_sync();
            mfma_pass<MB>(L, bx1, 1, cn, acc);
        }
        wave_lds_sync();
        cur = nxt;
    }

    // Workgroup sum in wave order: each wave parks its accumulators as fp32 [m][row]
    {
        float *red = reinterpret_cast<float *>(L.a);
        const uint32_t lane = lane_id(), q = lane >> 4, mr = lane & 15u;
#pragma unroll
        for (uint32_t rb = 0; rb < 4; ++rb)
#pragma unroll
            for (uint32_t mb = 0; mb < MB; ++mb)
#pragma unroll
                for (uint32_t v = 0; v < 4; ++v) red[(16 * mb + mr) * kTileRows + 16 * rb + 4 * q + v] = acc[rb][mb][v];
    }
    __syncthreads();
    // output i = m * 64 + row; thread t owns outputs t, t + 256, ... (at most 16)
    const uint32_t outs = G.m * kTileRows;
    const float *r0p = reinterpret_cast<const float *>(lds[0].a), *r1p = reinterpret_cast<const float *>(lds[1].a);
    const float *r2p = reinterpret_cast<const float *>(lds[2].a), *r3p = reinterpret_cast<const float *>(lds[3].a);
    constexpr uint32_t kPerThread = (VBQ_MAX_BATCH * kTileRows) / (kWavesPerBlock * kWave);   // 16
    if (G.splits == 1) {
        for (uint32_t i = threadIdx.x; i < outs; i += blockDim.x) {
            const uint32_t m = i / kTileRows, row = i % kTileRows;
            if (row < rows) G.y[static_cast<uint64_t>(m) * G.n + r0 + row] = ((r0p[i] + r1p[i]) + r2p[i]) + r3p[i];
        }
        return;
    }
    // split row tile: publish partial sums, count arrivals, the last workgroup adds them in split order
    for (uint32_t i = threadIdx.x; i < outs; i += blockDim.x) {
        const uint32_t m = i / kTileRows, row = i % kTileRows;
        if (row < rows)
            __hip_atomic_store(&G.partial[(static_cast<uint64_t>(split) * G.m + m) * G.n + r0 + row],
                               ((r0p[i] + r1p[i]) + r2p[i]) + r3p[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0)
        arrived_s = __hip_atomic_fetch_add(&G.counters[a], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (arrived_s != G.splits - 1) return;
    // every output's partials are requested before any is added (clamped
    // addresses for outputs past m x rows, which are not stored)
    const uint64_t stride = static_cast<uint64_t>(G.m) * G.n;
    for (uint32_t s0 = 0; s0 < G.splits; s0 += 2) {
        float v[kPerThread][2];
#pragma unroll
        for (uint32_t j = 0; j < kPerThread; ++j) {
            const uint32_t i = min(threadIdx.x + j * blockDim.x, outs - 1);
            const uint32_t m = i / kTileRows, row = min(i % kTileRows, rows - 1);
            const float *p = G.partial + static_cast<uint64_t>(m) * G.n + r0 + row;
#pragma unroll
            for (uint32_t h = 0; h < 2; ++h)
                v[j][h] = __hip_atomic_load(p + min(s0 + h, G.splits - 1) * stride, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (uint32_t j = 0; j < kPerThread; ++j) {
            const uint32_t i = threadIdx.x + j * blockDim.x;
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
    if (threadIdx.x == 0) __hip_atomic_store(&G.counters[a], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    if (!aligned16(w->tile_offsets) || !aligned16(w->widths) || !aligned16(w->scales) || !aligned16(w->payload))
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

// Scratch for split row tiles: one buffer per (device, stream), grown on demand.
// The buffer starts with a region that only ever holds arrival counters: it is
// zeroed when allocated and every counter is reset to zero by the last
// workgroup of its row tile, so the region is all zeros between calls however
// the next call lays out its matrices. Partial sums follow it.
struct Scratch {
    void *ptr = nullptr;
    size_t counter_bytes = 0;
    size_t partial_bytes = 0;
};

std::mutex g_scratch_mu;
std::unordered_map<uint64_t, Scratch> g_scratch;

vbq_status scratch_for(const char *who, hipStream_t stream, size_t counters, size_t partials, uint32_t **ctr_out,
                       char **part_out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(VBQ_ERR_HIP, "%s: hipGetDevice failed", who);
    const uint64_t key = (static_cast<uint64_t>(dev) << 56) ^ reinterpret_cast<uintptr_t>(stream);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    Scratch &s = g_scratch[key];
    if (s.counter_bytes < counters || s.partial_bytes < partials) {
        if (s.ptr) {
            if (hipStreamSynchronize(stream) != hipSuccess || hipFree(s.ptr) != hipSuccess)
                return fail(VBQ_ERR_HIP, "%s: could not release the old scratch buffer", who);
            s.ptr = nullptr;
        }
        const size_t cb = std::max<size_t>(counters, std::max<size_t>(s.counter_bytes, 64u << 10));
        const size_t pb = std::max<size_t>(partials, std::max<size_t>(s.partial_bytes, 1u << 20));
        if (hipMalloc(&s.ptr, cb + pb) != hipSuccess) return fail(VBQ_ERR_HIP, "%s: scratch hipMalloc failed", who);
        // zero the counter region on the caller's stream, ahead of the launches that use it (a memset on
        // the null stream is not ordered with non-blocking streams)
        const uint64_t words = cb / 4;
        hipLaunchKernelGGL(fill_zero, dim3(static_cast<uint32_t>((words + 255) / 256)), dim3(256), 0, stream,
                           static_cast<float *>(s.ptr), words);
        if (hipGetLastError() != hipSuccess) return fail(VBQ_ERR_HIP, "%s: scratch clear failed", who);
        s.counter_bytes = cb;
        s.partial_bytes = pb;
    }
    *ctr_out = static_cast<uint32_t *>(s.ptr);
    *part_out = static_cast<char *>(s.ptr) + s.counter_bytes;
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

GemvPlan gemv_plan(uint32_t row_tiles, uint32_t col_tiles) {
    constexpr uint32_t kCUs = 256;
    const uint32_t waves[3] = {4, 8, 16}, per_cu[3] = {8, 4, 2};   // resident workgroups per CU (LDS bound)
    GemvPlan best{4, 1};
    double best_cost = 1e300;
    for (uint32_t w = 0; w < 3; ++w) {
        const uint32_t gw = waves[w];
        for (uint32_t s = 1; s <= ceil_div(col_tiles, gw); ++s) {
            const double wgs = static_cast<double>(row_tiles) * s;
            const uint32_t ct_per = ceil_div(col_tiles, s);              // column tiles of a workgroup (at most)
            const uint32_t active = std::min(gw, ct_per);                // waves with a tile
            const uint32_t tpw = ceil_div(ct_per, gw);                   // tiles per wave (at most)
            const double cu_load = std::max(1.0, wgs / kCUs);            // workgroups per occupied CU
            const double rounds = std::ceil(cu_load / per_cu[w]);
            const double slots = tpw * (active / 4.0) * cu_load;
            const double cost = 1.1 * slots + 2.5 * ((tpw - 1) + (rounds - 1)) + (s > 1 ? 1.4 + 0.23 * s : 0.0);
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

template <uint32_t kWaves>
void gemv_dispatch(bool aligned, bool ragged, uint32_t ubits, uint32_t blocks, uint32_t used, const Batch &B,
                   hipStream_t stream) {
    if (ubits == kPerMatrix) {
        if (aligned)
            hipLaunchKernelGGL((gemv_uniform_mixed<true, kWaves>), dim3(blocks, used), dim3(kWaves * kWave), 0,
                               stream, B);
        else
            hipLaunchKernelGGL((gemv_uniform_mixed<false, kWaves>), dim3(blocks, used), dim3(kWaves * kWave), 0,
                               stream, B);
        return;
    }
    switch (ubits) {
        case 1: gemv_dispatch_uniform<1, kWaves>(aligned, blocks, used, B, stream); return;
        case 2: gemv_dispatch_uniform<2, kWaves>(aligned, blocks, used, B, stream); return;
        case 4: gemv_dispatch_uniform<4, kWaves>(aligned, blocks, used, B, stream); return;
        case 8: gemv_dispatch_uniform<8, kWaves>(aligned, blocks, used, B, stream); return;
        default: break;
    }
    const dim3 grid(blocks, used), block(kWaves * kWave);
    if (aligned && ragged)
        hipLaunchKernelGGL((gemv_tiles<true, kWaves, true>), grid, block, 0, stream, B);
    else if (aligned)
        hipLaunchKernelGGL((gemv_tiles<true, kWaves, false>), grid, block, 0, stream, B);
    else if (ragged)
        hipLaunchKernelGGL((gemv_tiles<false, kWaves, true>), grid, block, 0, stream, B);
    else
        hipLaunchKernelGGL((gemv_tiles<false, kWaves, false>), grid, block, 0, stream, B);
}

// One launch for up to VBQ_MAX_MULTI independent GEMVs; with h set, the two
// matrices are gate and up (same shape, k > 0) and the launch writes
// h = fp16(silu(gate x) * (up x)) instead of y.
vbq_status gemv_launch(const char *who, const vbq_matrix *const *ws, const uint16_t *const *xs, float *const *ys,
                       uint32_t count, hipStream_t stream, uint16_t *h = nullptr, uint16_t *const *ys16 = nullptr) {
    Batch B{};
    uint32_t blocks = 0, total_row_tiles = 0, max_col_tiles = 0;
    bool aligned = true;
    for (uint32_t i = 0; i < count; ++i) {
        const vbq_matrix *w = ws[i];
        if (w->n == 0 || w->k == 0) continue;
        total_row_tiles += ceil_div(w->n, kTileRows);
        max_col_tiles = std::max(max_col_tiles, ceil_div(w->k / VBQ_GROUP, kTileGroups));
    }
    const GemvPlan plan = total_row_tiles ? gemv_plan(total_row_tiles, max_col_tiles) : GemvPlan{4, 1};
    size_t counter_slots = 0, partial_total = 0;
    uint32_t used = 0;
    bool any_launch = false;
    // the uniform-width kernels run when every matrix launched declares a width: one kernel per width
    // when they agree, the per-matrix dispatch when they differ
    uint32_t ubits = 0;
    bool first = true;
    for (uint32_t i = 0; i < count; ++i) {
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
        if (w->n == 0) continue;
        if (w->k == 0) {
            const uint64_t cnt = w->n;
            if (ys16)
                hipLaunchKernelGGL(fill_zero_u16, dim3(static_cast<uint32_t>((cnt + 255) / 256)), dim3(256), 0, stream,
                                   ys16[i], cnt);
            else
                hipLaunchKernelGGL(fill_zero, dim3(static_cast<uint32_t>((cnt + 255) / 256)), dim3(256), 0, stream,
                                   ys[i], cnt);
            any_launch = true;
            continue;
        }
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
        M.n = w->n;
        M.groups = w->k / VBQ_GROUP;
        M.col_tiles = ceil_div(M.groups, kTileGroups);
        const uint32_t row_tiles = ceil_div(M.n, kTileRows);
        M.splits = std::max(1u, std::min(ceil_div(M.col_tiles, plan.waves), plan.splits));
        M.blocks = row_tiles * M.splits;
        blocks = std::max(blocks, M.blocks);
        if (M.groups % 4) aligned = false;
        if (M.splits > 1) {
            counter_slots += row_tiles;
            partial_total += partial_bytes(M.splits, M.n);
        }
    }
    if (used == 0) return any_launch ? launched(who) : VBQ_OK;
    if (h) {   // the pair region follows the split regions
        counter_slots += ceil_div(B.m[0].n, kTileRows);
        partial_total += partial_bytes(2, B.m[0].n);
    }
    if (counter_slots) {
        uint32_t *ctr = nullptr;
        char *part = nullptr;
        vbq_status st = scratch_for(who, stream, counter_slots * 4, partial_total, &ctr, &part);
        if (st != VBQ_OK) return st;
        for (uint32_t i = 0; i < used; ++i) {
            MatArgs &M = B.m[i];
            if (M.splits == 1) continue;
            M.counters = ctr;
            ctr += ceil_div(M.n, kTileRows);
            M.partial = reinterpret_cast<float *>(part);
            part += partial_bytes(M.splits, M.n);
        }
        if (h) {
            B.h = h;
            B.pair_counters = ctr;
            B.pair = reinterpret_cast<float *>(part);
        }
    }
    bool ragged = false;   // some matrix has fewer workgroups than the grid is wide
    for (uint32_t i = 0; i < used; ++i) ragged = ragged || B.m[i].blocks != blocks;
    if (plan.waves == 16)
        gemv_dispatch<16>(aligned, ragged, ubits, blocks, used, B, stream);
    else if (plan.waves == 8)
        gemv_dispatch<8>(aligned, ragged, ubits, blocks, used, B, stream);
    else
        gemv_dispatch<4>(aligned, ragged, ubits, blocks, used, B, stream);
    return launched(who);
}

// Small-batch GEMM on the matrix cores: one launch for up to 64 rows of X.
vbq_status gemm_launch(const char *who, const vbq_matrix *w, const uint16_t *x, uint32_t m, float *y,
                       hipStream_t stream) {
    GemmArgs G{};
    G.widths = w->widths;
    G.scales = w->scales;
    G.tile_offsets = w->tile_offsets;
    G.payload = w->payload;
    G.payload_bytes = w->payload_bytes;
    G.x = x;
    G.y = y;
    G.n = w->n;
    G.groups = w->k / VBQ_GROUP;
    G.col_tiles = ceil_div(G.groups, kTileGroups);
    G.m = m;
    G.k = w->k;
    const uint32_t row_tiles = ceil_div(G.n, kTileRows);
    // two workgroups per CU are resident (LDS): split the column tiles only
    // while the row tiles alone leave CUs idle
    const uint32_t want_blocks = 512;
    G.splits = std::max(1u, std::min(ceil_div(G.col_tiles, kWavesPerBlock), want_blocks / row_tiles));
    if (G.splits > 1) {
        uint32_t *ctr = nullptr;
        char *part = nullptr;
        const size_t partials = (static_cast<size_t>(G.splits) * m * G.n * 4 + 255) / 256 * 256;
        vbq_status st = scratch_for(who, stream, static_cast<size_t>(row_tiles) * 4, partials, &ctr, &part);
        if (st != VBQ_OK) return st;
        G.counters = ctr;
        G.partial = reinterpret_cast<float *>(part);
    }
    const dim3 grid(row_tiles * G.splits), block(kWavesPerBlock * kWave);
    switch (ceil_div(m, 16)) {
        case 1: hipLaunchKernelGGL(gemm_tiles<1>, grid, block, 0, stream, G); break;
        case 2: hipLaunchKernelGGL(gemm_tiles<2>, grid, block, 0, stream, G); break;
        case 3: hipLaunchKernelGGL(gemm_tiles<3>, grid, block, 0, stream, G); break;
        default: hipLaunchKernelGGL(gemm_tiles<4>, grid, block, 0, stream, G); break;
    }
    return launched(who);
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
}

extern "C" vbq_status vbq_gemv_swiglu(const vbq_matrix *gate, const vbq_matrix *up, const uint16_t *x, uint16_t *h,
                                      void *stream) {
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
}

extern "C" vbq_status vbq_gemv_multi_f16(const vbq_matrix *const *ws, const uint16_t *const *xs, uint16_t *const *ys,
                                         uint32_t count, void *stream) {
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
}

extern "C" vbq_status vbq_gemv(const vbq_matrix *w, const uint16_t *x, float *y, void *stream) {
    vbq::clear_error();
    const char *who = "vbq_gemv";
    vbq_status st = check_matrix(who, w);
    if (st != VBQ_OK) return st;
    st = check_vectors(who, w, x, y);
    if (st != VBQ_OK) return st;
    (void)hipGetLastError();
    return gemv_launch(who, &w, &x, &y, 1, static_cast<hipStream_t>(stream));
}

extern "C" vbq_status vbq_gemm_smallbatch(const vbq_matrix *w, const uint16_t *x, uint32_t m, float *y,
                                          void *stream) {
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
    const uint64_t tiles = static_cast<uint64_t>(ceil_div(w->n, kTileRows)) * ceil_div(w->k / VBQ_GROUP, kTileGroups);
    if (m > VBQ_MAX_MULTI || (m >= kGemmMinBatch && static_cast<uint64_t>(m) * m * tiles >= kGemmMinWork)) {
        if (w->k == 0) {
            const uint64_t cnt = static_cast<uint64_t>(m) * w->n;
            hipLaunchKernelGGL(fill_zero, dim3(static_cast<uint32_t>((cnt + 255) / 256)), dim3(256), 0, s, y, cnt);
            return launched(who);
        }
        return gemm_launch(who, w, x, m, y, s);
    }
    // each input row as its own GEMV of one batched launch
    const vbq_matrix *ws[VBQ_MAX_MULTI];
    const uint16_t *xs[VBQ_MAX_MULTI];
    float *ys[VBQ_MAX_MULTI];
    for (uint32_t m0 = 0; m0 < m; m0 += VBQ_MAX_MULTI) {
        const uint32_t cnt = std::min(VBQ_MAX_MULTI, m - m0);
        for (uint32_t i = 0; i < cnt; ++i) {
            ws[i] = w;
            xs[i] = x + static_cast<uint64_t>(m0 + i) * w->k;
            ys[i] = y + static_cast<uint64_t>(m0 + i) * w->n;
        }
        st = gemv_launch(who, ws, xs, ys, cnt, s);
        if (st != VBQ_OK) return st;
    }
    return VBQ_OK;
}

extern "C" vbq_status vbq_unpack_codes(const vbq_matrix *w, int8_t *codes_out, void *stream) {
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
}
