// Host half of the VBQ library: packing, validation and error reporting.
//
// Layout and grid: VBQ paper (arXiv 2607.02893) §3.1 Eq. (1) and §6
// "Granularity is deployment-friendly"; the byte-level choices are spelled out
// in include/vbq.h. Everything here runs on the host and is deterministic.
#include "vbq_internal.h"

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <string>
#include <vector>

namespace {

// fixed size so that recording an error never allocates (and so never throws)
thread_local char g_last_error[512];

inline bool valid_width(uint8_t b) { return b == 1 || b == 2 || b == 4 || b == 8; }

inline uint8_t width_code(uint8_t b) { return b == 1 ? 0 : b == 2 ? 1 : b == 4 ? 2 : 3; }

inline bool half_is_finite(uint16_t h) { return ((h >> 10) & 0x1F) != 0x1F; }

// b-bit field for code q (two's complement for b >= 2, sign bit for b = 1)
inline uint32_t encode_field(int q, uint32_t b) {
    if (b == 1) return q < 0 ? 1u : 0u;
    return static_cast<uint32_t>(q) & ((1u << b) - 1u);
}

inline bool on_grid(int q, uint32_t b) {
    if (b == 1) return q == 1 || q == -1;
    const int lim = (1 << (b - 1)) - 1;
    return q >= -lim && q <= lim;
}

}  // namespace

namespace vbq {

vbq_status fail(vbq_status st, const char *fmt, ...) noexcept {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

void clear_error() noexcept { g_last_error[0] = '\0'; }

}  // namespace vbq

using vbq::fail;

extern "C" uint32_t vbq_abi_version(void) { return VBQ_ABI_VERSION; }

extern "C" const char *vbq_status_string(vbq_status s) {
    switch (s) {
        case VBQ_OK: return "ok";
        case VBQ_ERR_NULL: return "null pointer";
        case VBQ_ERR_SHAPE: return "bad shape";
        case VBQ_ERR_WIDTH: return "width not in {1,2,4,8}";
        case VBQ_ERR_CODE: return "code off its width's grid";
        case VBQ_ERR_SCALE: return "non-finite scale";
        case VBQ_ERR_CAPACITY: return "payload capacity too small";
        case VBQ_ERR_OFFSETS: return "tile offsets inconsistent with widths";
        case VBQ_ERR_ALIGN: return "pointer not 16-byte aligned";
        case VBQ_ERR_TOO_LARGE: return "payload exceeds 32-bit offsets";
        case VBQ_ERR_HIP: return "HIP runtime error";
        case VBQ_ERR_ABI: return "ABI version mismatch";
        case VBQ_ERR_PADDING: return "padding not inert";
        case VBQ_ERR_FORMAT: return "bad container";
        case VBQ_ERR_NOMEM: return "host memory exhausted";
        case VBQ_ERR_INTERNAL: return "internal error";
    }
    return "unknown status";
}

extern "C" const char *vbq_last_error(void) { return g_last_error; }

namespace {

// bit position of element i inside a b-bit group (see the layout in vbq.h)
inline uint32_t field_pos(uint32_t b, uint32_t i) {
    switch (b) {
        case 1: return i;
        case 2: { const uint32_t e = i & 15; return 32 * (i >> 4) + 2 * ((e >> 1) | ((e & 1) << 3)); }
        case 4: { const uint32_t e = i & 7; return 32 * (i >> 3) + 4 * ((e >> 1) | ((e & 1) << 2)); }
        default: return 8 * i;
    }
}

inline uint32_t width_slot(uint32_t b) { return b == 1 ? 0 : b == 2 ? 1 : b == 4 ? 2 : 3; }

uint64_t tiles_of(uint32_t n, uint32_t G) {
    return uint64_t((n + VBQ_TILE_ROWS - 1) / VBQ_TILE_ROWS) * ((G + VBQ_TILE_GROUPS - 1) / VBQ_TILE_GROUPS);
}

// Slot of group (r, j) in the width-code and scale arrays: tiles one after the
// other (row tile major), the groups of a tile row-major inside it. A full
// row tile holds 64*G slots; a tile of R rows and C groups holds R*C.
inline uint64_t meta_slot(uint32_t n, uint32_t G, uint32_t r, uint32_t j) {
    const uint32_t r0 = r / VBQ_TILE_ROWS * VBQ_TILE_ROWS, j0 = j / VBQ_TILE_GROUPS * VBQ_TILE_GROUPS;
    const uint32_t R = std::min<uint32_t>(VBQ_TILE_ROWS, n - r0), C = std::min<uint32_t>(VBQ_TILE_GROUPS, G - j0);
    return uint64_t(r0) * G + uint64_t(R) * j0 + uint64_t(r - r0) * C + (j - j0);
}

// Payload offset of every group, plus the tile offsets, for per-group widths
// given by width(r, j). Inside a tile the four width buckets follow each other;
// a group's place in its bucket is its column-major rank among same-width
// groups of the tile.
template <class WidthFn>
uint64_t place_groups(uint32_t n, uint32_t G, WidthFn width, uint64_t *group_off, uint32_t *tile_off) {
    uint64_t pos = 0, tile = 0;
    for (uint32_t r0 = 0; r0 < n; r0 += VBQ_TILE_ROWS) {
        const uint32_t r1 = std::min(n, r0 + VBQ_TILE_ROWS);
        for (uint32_t j0 = 0; j0 < G; j0 += VBQ_TILE_GROUPS) {
            const uint32_t j1 = std::min(G, j0 + VBQ_TILE_GROUPS);
            uint64_t bucket_bytes[4] = {0, 0, 0, 0};
            for (uint32_t j = j0; j < j1; ++j)
                for (uint32_t r = r0; r < r1; ++r) {
                    const uint32_t b = width(r, j);
                    bucket_bytes[width_slot(b)] += 8u * b;
                }
            uint64_t next[4];
            next[0] = pos;
            for (int i = 1; i < 4; ++i) next[i] = next[i - 1] + bucket_bytes[i - 1];
            if (tile_off) tile_off[tile] = uint32_t(pos);
            for (uint32_t j = j0; j < j1; ++j)
                for (uint32_t r = r0; r < r1; ++r) {
                    const uint64_t t = uint64_t(r) * G + j;
                    const uint32_t b = width(r, j);
                    if (group_off) group_off[t] = next[width_slot(b)];
                    next[width_slot(b)] += 8u * b;
                }
            pos = next[3];
            ++tile;
        }
    }
    if (tile_off) tile_off[tile] = uint32_t(pos);
    return pos;
}

}  // namespace

extern "C" uint64_t vbq_tile_count(uint32_t n, uint32_t k) { return tiles_of(n, k / VBQ_GROUP); }

// 256 list bytes and 8 count bytes per tile
extern "C" vbq_status vbq_stream_index_bytes(uint32_t n, uint32_t k, uint64_t *bytes_out) {
    return vbq::guarded("vbq_stream_index_bytes", [&]() -> vbq_status {
        vbq::clear_error();
        if (!bytes_out) return fail(VBQ_ERR_NULL, "vbq_stream_index_bytes: bytes_out is NULL");
        if (k % VBQ_GROUP) return fail(VBQ_ERR_SHAPE, "vbq_stream_index_bytes: k=%u is not a multiple of 64", k);
        *bytes_out = 264u * tiles_of(n, k / VBQ_GROUP);
        return VBQ_OK;
    });
}

extern "C" vbq_status vbq_pack_sizes(uint32_t n, uint32_t k, const uint8_t *bits, vbq_sizes *out) {
    return vbq::guarded("vbq_pack_sizes", [&]() -> vbq_status {
        vbq::clear_error();
        if (!out) return fail(VBQ_ERR_NULL, "vbq_pack_sizes: out is NULL");
        if (k % VBQ_GROUP) return fail(VBQ_ERR_SHAPE, "vbq_pack_sizes: k=%u is not a multiple of 64", k);
        const uint64_t groups = uint64_t(n) * (k / VBQ_GROUP);
        if (groups && !bits) return fail(VBQ_ERR_NULL, "vbq_pack_sizes: bits is NULL");
        uint64_t payload = 0;
        for (uint64_t t = 0; t < groups; ++t) {
            if (!valid_width(bits[t]))
                return fail(VBQ_ERR_WIDTH, "vbq_pack_sizes: group %llu has width %u", (unsigned long long)t, bits[t]);
            payload += 8u * bits[t];
        }
        if (payload > 0xFFFFFFFFull)
            return fail(VBQ_ERR_TOO_LARGE, "vbq_pack_sizes: payload %llu B exceeds 32-bit offsets",
                        (unsigned long long)payload);
        out->widths_bytes = (groups + 3) / 4;
        out->scales_bytes = 2 * groups;
        out->offsets_bytes = 4 * (tiles_of(n, k / VBQ_GROUP) + 1);
        out->payload_bytes = payload;
        out->total_bytes = out->widths_bytes + out->scales_bytes + out->offsets_bytes + out->payload_bytes;
        return VBQ_OK;
    });
}

extern "C" vbq_status vbq_pack(uint32_t n, uint32_t k, const uint8_t *bits, const int8_t *codes,
                               const uint16_t *scales, uint8_t *widths_out, uint16_t *scales_out,
                               uint32_t *tile_offsets_out, uint8_t *payload_out, uint64_t payload_capacity) {
    return vbq::guarded("vbq_pack", [&]() -> vbq_status {
        vbq_sizes sz;
        vbq_status st = vbq_pack_sizes(n, k, bits, &sz);
        if (st != VBQ_OK) return st;
        const uint32_t G = k / VBQ_GROUP;
        const uint64_t groups = uint64_t(n) * G;
        if (!tile_offsets_out) return fail(VBQ_ERR_NULL, "vbq_pack: tile_offsets_out is NULL");
        if (groups && (!codes || !scales || !widths_out || !scales_out))
            return fail(VBQ_ERR_NULL, "vbq_pack: codes, scales, widths_out or scales_out is NULL");
        if (sz.payload_bytes && !payload_out) return fail(VBQ_ERR_NULL, "vbq_pack: payload_out is NULL");
        if (sz.payload_bytes > payload_capacity)
            return fail(VBQ_ERR_CAPACITY, "vbq_pack: payload needs %llu B, capacity %llu B",
                        (unsigned long long)sz.payload_bytes, (unsigned long long)payload_capacity);
        // validate everything before the first write
        for (uint64_t t = 0; t < groups; ++t) {
            if (!half_is_finite(scales[t]))
                return fail(VBQ_ERR_SCALE, "vbq_pack: scale of group %llu is 0x%04x (not finite)",
                            (unsigned long long)t, scales[t]);
            const int8_t *q = codes + t * VBQ_GROUP;
            for (uint32_t i = 0; i < VBQ_GROUP; ++i)
                if (!on_grid(q[i], bits[t]))
                    return fail(VBQ_ERR_CODE, "vbq_pack: code %d at group %llu element %u is off the %u-bit grid",
                                q[i], (unsigned long long)t, i, bits[t]);
        }
        std::vector<uint64_t> off(groups);
        place_groups(n, G, [&](uint32_t r, uint32_t j) { return uint32_t(bits[uint64_t(r) * G + j]); }, off.data(),
                     tile_offsets_out);
        if (sz.widths_bytes) std::memset(widths_out, 0, sz.widths_bytes);
        if (sz.payload_bytes) std::memset(payload_out, 0, sz.payload_bytes);
        for (uint64_t t = 0; t < groups; ++t) {
            const uint32_t b = bits[t];
            const uint64_t m = meta_slot(n, G, uint32_t(t / G), uint32_t(t % G));
            widths_out[m >> 2] |= uint8_t(width_code(uint8_t(b)) << (2 * (m & 3)));
            scales_out[m] = scales[t];
            const int8_t *q = codes + t * VBQ_GROUP;
            uint8_t *dst = payload_out + off[t];
            // fields never straddle a byte: b divides 8 and every field starts at a multiple of b
            for (uint32_t i = 0; i < VBQ_GROUP; ++i) {
                const uint32_t bit = field_pos(b, i);
                dst[bit >> 3] |= uint8_t(encode_field(q[i], b) << (bit & 7));
            }
        }
        return VBQ_OK;
    });
}

extern "C" vbq_status vbq_validate_host(const vbq_matrix *w) {
    return vbq::guarded("vbq_validate_host", [&]() -> vbq_status {
        vbq::clear_error();
        if (!w) return fail(VBQ_ERR_NULL, "vbq_validate_host: view is NULL");
        if (w->abi_version != VBQ_ABI_VERSION)
            return fail(VBQ_ERR_ABI, "vbq_validate_host: abi_version %u, library %u", w->abi_version, VBQ_ABI_VERSION);
        if (w->k % VBQ_GROUP) return fail(VBQ_ERR_SHAPE, "vbq_validate_host: k=%u is not a multiple of 64", w->k);
        const uint32_t G = w->k / VBQ_GROUP;
        const uint64_t groups = uint64_t(w->n) * G;
        const uint64_t tiles = tiles_of(w->n, G);
        if (!w->tile_offsets) return fail(VBQ_ERR_NULL, "vbq_validate_host: tile_offsets is NULL");
        if (groups && (!w->widths || !w->scales || !w->payload))
            return fail(VBQ_ERR_NULL, "vbq_validate_host: widths, scales or payload is NULL");
        auto width = [&](uint32_t r, uint32_t j) {
            const uint64_t m = meta_slot(w->n, G, r, j);
            return 1u << ((w->widths[m >> 2] >> (2 * (m & 3))) & 3u);
        };
        std::vector<uint64_t> off(groups);
        std::vector<uint32_t> expect(tiles + 1);
        const uint64_t total = place_groups(w->n, G, width, off.data(), expect.data());
        for (uint64_t i = 0; i <= tiles; ++i)
            if (w->tile_offsets[i] != expect[i])
                return fail(VBQ_ERR_OFFSETS, "vbq_validate_host: tile_offsets[%llu]=%u, widths give %u",
                            (unsigned long long)i, w->tile_offsets[i], expect[i]);
        if (total != w->payload_bytes)
            return fail(VBQ_ERR_OFFSETS, "vbq_validate_host: payload_bytes=%u, widths give %llu", w->payload_bytes,
                        (unsigned long long)total);
        if (w->uniform_bits) {
            const uint32_t ub = w->uniform_bits;
            if (ub != 1 && ub != 2 && ub != 4 && ub != 8)
                return fail(VBQ_ERR_WIDTH, "vbq_validate_host: uniform_bits=%u is not 0, 1, 2, 4 or 8", ub);
            for (uint32_t r = 0; r < w->n; ++r)
                for (uint32_t j = 0; j < G; ++j)
                    if (width(r, j) != ub)
                        return fail(VBQ_ERR_WIDTH, "vbq_validate_host: group (%u, %u) has width %u, uniform_bits=%u", r,
                                    j, width(r, j), ub);
        }
        for (uint64_t t = 0; t < groups; ++t) {
            if (!half_is_finite(w->scales[t]))
                return fail(VBQ_ERR_SCALE, "vbq_validate_host: scale slot %llu not finite", (unsigned long long)t);
            const uint32_t b = width(uint32_t(t / G), uint32_t(t % G));
            if (b == 1) continue;
            const uint8_t *src = w->payload + off[t];
            for (uint32_t i = 0; i < VBQ_GROUP; ++i) {
                const uint32_t bit = field_pos(b, i);
                const uint32_t f = (src[bit >> 3] >> (bit & 7)) & ((1u << b) - 1u);
                if (f == (1u << (b - 1)))
                    return fail(VBQ_ERR_CODE, "vbq_validate_host: reserved pattern at group %llu element %u",
                                (unsigned long long)t, i);
            }
        }
        return VBQ_OK;
    });
}

// VBQ §3.4, the frequency-tiered head: rank rows by descending frequency (ties
// to the lower row), then cut the ranking at half-up roundings of 0.5%, 2% and
// 12% of the rows into the 8-, 4- and 2-bit tiers; the rest get 1 bit.
extern "C" vbq_status vbq_recipe_head_order(uint32_t rows, const uint64_t *freq, uint32_t *order) {
    return vbq::guarded("vbq_recipe_head_order", [&]() -> vbq_status {
        vbq::clear_error();
        if (rows == 0) return VBQ_OK;
        if (!freq || !order) return fail(VBQ_ERR_NULL, "vbq_recipe_head_order: a pointer is NULL");
        for (uint32_t r = 0; r < rows; ++r) order[r] = r;
        std::stable_sort(order, order + rows, [&](uint32_t a, uint32_t b) { return freq[a] > freq[b]; });
        return VBQ_OK;
    });
}

extern "C" vbq_status vbq_recipe_head_bits(uint32_t rows, const uint64_t *freq, uint8_t *bits_out) {
    return vbq::guarded("vbq_recipe_head_bits", [&]() -> vbq_status {
        vbq::clear_error();
        if (rows == 0) return VBQ_OK;
        if (!freq || !bits_out) return fail(VBQ_ERR_NULL, "vbq_recipe_head_bits: a pointer is NULL");
        std::vector<uint32_t> order(rows);
        vbq_recipe_head_order(rows, freq, order.data());
        const uint64_t cut8 = (5ull * rows + 500) / 1000, cut4 = (20ull * rows + 500) / 1000,
                       cut2 = (120ull * rows + 500) / 1000;
        for (uint64_t rank = 0; rank < rows; ++rank)
            bits_out[order[rank]] = rank < cut8 ? 8 : rank < cut4 ? 4 : rank < cut2 ? 2 : 1;
        return VBQ_OK;
    });
}

extern "C" vbq_status vbq_recipe_head_tiers(uint32_t rows, const uint64_t *freq, uint32_t *order_out,
                                            uint32_t *tier_rows_out) {
    return vbq::guarded("vbq_recipe_head_tiers", [&]() -> vbq_status {
        vbq::clear_error();
        if (!tier_rows_out) return fail(VBQ_ERR_NULL, "vbq_recipe_head_tiers: tier_rows_out is NULL");
        for (int t = 0; t < 4; ++t) tier_rows_out[t] = 0;
        if (rows == 0) return VBQ_OK;
        if (!freq || !order_out) return fail(VBQ_ERR_NULL, "vbq_recipe_head_tiers: a pointer is NULL");
        std::vector<uint8_t> bits(rows);
        vbq_status st = vbq_recipe_head_order(rows, freq, order_out);
        if (st != VBQ_OK) return st;
        st = vbq_recipe_head_bits(rows, freq, bits.data());
        if (st != VBQ_OK) return st;
        // the ranking is monotone in width (8, 4, 2, then 1 bit), so each tier is one contiguous run of ranks
        for (uint32_t rank = 0; rank < rows; ++rank) ++tier_rows_out[3 - width_code(bits[order_out[rank]])];
        return VBQ_OK;
    });
}

namespace {

// Code of element i of a group from its packed bytes: b = 1 gives +-1, b >= 2 two's complement.
int32_t packed_code(uint32_t b, const uint8_t *src, uint32_t i) {
    const uint32_t bit = field_pos(b, i);
    const uint32_t f = (src[bit >> 3] >> (bit & 7)) & ((1u << b) - 1u);
    if (b == 1) return f ? -1 : 1;
    return f >= (1u << (b - 1)) ? int32_t(f) - int32_t(1u << b) : int32_t(f);
}

}  // namespace

// VBQ §6, "Granularity is deployment-friendly": padded MLP channels must be
// inert, i.e. every padded weight dequantizes to exactly zero.
extern "C" vbq_status vbq_check_padding(const vbq_matrix *w, uint32_t n_real, uint32_t k_real, uint32_t k_multiple) {
    return vbq::guarded("vbq_check_padding", [&]() -> vbq_status {
        const vbq_status st = vbq_validate_host(w);
        if (st != VBQ_OK) return st;
        if (k_multiple == 0) return fail(VBQ_ERR_SHAPE, "vbq_check_padding: k_multiple is 0");
        if (w->k % k_multiple)
            return fail(VBQ_ERR_SHAPE, "vbq_check_padding: k=%u is not a multiple of %u", w->k, k_multiple);
        if (n_real > w->n || k_real > w->k)
            return fail(VBQ_ERR_SHAPE, "vbq_check_padding: real %ux%u exceeds the packed %ux%u", n_real, k_real, w->n,
                        w->k);
        const uint32_t G = w->k / VBQ_GROUP;
        std::vector<uint64_t> off(uint64_t(w->n) * G);
        auto width = [&](uint32_t r, uint32_t j) {
            const uint64_t m = meta_slot(w->n, G, r, j);
            return 1u << ((w->widths[m >> 2] >> (2 * (m & 3))) & 3u);
        };
        place_groups(w->n, G, width, off.data(), nullptr);
        for (uint32_t r = 0; r < w->n; ++r)
            for (uint32_t j = 0; j < G; ++j) {
                if (r < n_real && (j + 1) * VBQ_GROUP <= k_real) continue;   // no padded weight in this group
                const uint64_t m = meta_slot(w->n, G, r, j);
                if ((w->scales[m] & 0x7FFFu) == 0) continue;                   // scale +-0: the whole group is zero
                const uint32_t b = width(r, j);
                for (uint32_t i = 0; i < VBQ_GROUP; ++i) {
                    const uint32_t c = j * VBQ_GROUP + i;
                    if (r < n_real && c < k_real) continue;
                    if (packed_code(b, w->payload + off[uint64_t(r) * G + j], i) != 0)
                        return fail(VBQ_ERR_PADDING, "vbq_check_padding: weight (%u, %u) is padding but not zero", r, c);
                }
            }
        return VBQ_OK;
    });
}

// ------------------------------------------------------------------ container

namespace {

constexpr char kMagic[8] = {'V', 'B', 'Q', 'P', 'A', 'C', 'K', '\0'};
constexpr uint64_t kAlign = 256;

uint64_t align_up(uint64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// CRC-32 of IEEE 802.3 (reflected polynomial 0xEDB88320, initial and final complement).
uint32_t crc32(const uint8_t *p, uint64_t len) {
    static uint32_t table[256];
    static const bool ready = [] {
        for (uint32_t i = 0; i < 256; ++i) {
            uint32_t c = i;
            for (int k = 0; k < 8; ++k) c = (c & 1) ? 0xEDB88320u ^ (c >> 1) : c >> 1;
            table[i] = c;
        }
        return true;
    }();
    (void)ready;
    uint32_t c = 0xFFFFFFFFu;
    for (uint64_t i = 0; i < len; ++i) c = table[(c ^ p[i]) & 0xFFu] ^ (c >> 8);
    return c ^ 0xFFFFFFFFu;
}

struct Layout {
    uint64_t widths, scales, offsets, payload, total;   // offsets into the image
    uint64_t widths_bytes, scales_bytes, offsets_bytes, payload_bytes;
};

Layout layout_of(uint32_t n, uint32_t k, uint64_t payload_bytes) {
    const uint64_t groups = uint64_t(n) * (k / VBQ_GROUP);
    Layout L{};
    L.widths_bytes = (groups + 3) / 4;
    L.scales_bytes = 2 * groups;
    L.offsets_bytes = 4 * (tiles_of(n, k / VBQ_GROUP) + 1);
    L.payload_bytes = payload_bytes;
    L.widths = align_up(VBQ_CONTAINER_HEADER);
    L.scales = align_up(L.widths + L.widths_bytes);
    L.offsets = align_up(L.scales + L.scales_bytes);
    L.payload = align_up(L.offsets + L.offsets_bytes);
    L.total = L.payload + L.payload_bytes;
    return L;
}

template <class T> void put(uint8_t *h, uint32_t at, T v) { std::memcpy(h + at, &v, sizeof v); }
template <class T> T get(const uint8_t *h, uint32_t at) { T v; std::memcpy(&v, h + at, sizeof v); return v; }

}  // namespace

extern "C" vbq_status vbq_container_size(const vbq_matrix *w, uint64_t *bytes_out) {
    return vbq::guarded("vbq_container_size", [&]() -> vbq_status {
        vbq::clear_error();
        if (!w || !bytes_out) return fail(VBQ_ERR_NULL, "vbq_container_size: a pointer is NULL");
        if (w->abi_version != VBQ_ABI_VERSION)
            return fail(VBQ_ERR_ABI, "vbq_container_size: abi_version %u, library %u", w->abi_version, VBQ_ABI_VERSION);
        if (w->k % VBQ_GROUP) return fail(VBQ_ERR_SHAPE, "vbq_container_size: k=%u is not a multiple of 64", w->k);
        *bytes_out = layout_of(w->n, w->k, w->payload_bytes).total;
        return VBQ_OK;
    });
}

extern "C" vbq_status vbq_container_write(const vbq_matrix *w, uint8_t *out, uint64_t capacity, uint64_t *written) {
    return vbq::guarded("vbq_container_write", [&]() -> vbq_status {
        const vbq_status st = vbq_validate_host(w);
        if (st != VBQ_OK) return st;
        if (!out || !written) return fail(VBQ_ERR_NULL, "vbq_container_write: a pointer is NULL");
        const Layout L = layout_of(w->n, w->k, w->payload_bytes);
        if (capacity < L.total)
            return fail(VBQ_ERR_CAPACITY, "vbq_container_write: needs %llu bytes, capacity %llu",
                        (unsigned long long)L.total, (unsigned long long)capacity);
        std::memset(out, 0, L.total);
        std::memcpy(out, kMagic, 8);
        put<uint32_t>(out, 8, VBQ_CONTAINER_VERSION);
        put<uint32_t>(out, 12, VBQ_CONTAINER_HEADER);
        put<uint32_t>(out, 16, w->n);
        put<uint32_t>(out, 20, w->k);
        put<uint32_t>(out, 24, VBQ_GROUP);
        put<uint32_t>(out, 28, VBQ_TILE_ROWS);
        put<uint32_t>(out, 32, VBQ_TILE_GROUPS);
        put<uint32_t>(out, 36, w->payload_bytes);
        put<uint64_t>(out, 40, L.widths);
        put<uint64_t>(out, 48, L.scales);
        put<uint64_t>(out, 56, L.offsets);
        put<uint64_t>(out, 64, L.payload);
        put<uint64_t>(out, 72, L.total);
        if (L.widths_bytes) std::memcpy(out + L.widths, w->widths, L.widths_bytes);
        if (L.scales_bytes) std::memcpy(out + L.scales, w->scales, L.scales_bytes);
        std::memcpy(out + L.offsets, w->tile_offsets, L.offsets_bytes);
        if (L.payload_bytes) std::memcpy(out + L.payload, w->payload, L.payload_bytes);
        put<uint32_t>(out, 80, crc32(out + VBQ_CONTAINER_HEADER, L.total - VBQ_CONTAINER_HEADER));
        put<uint32_t>(out, 84, crc32(out, 84));
        *written = L.total;
        return VBQ_OK;
    });
}

extern "C" vbq_status vbq_container_open(const uint8_t *buf, uint64_t len, vbq_matrix *view) {
    return vbq::guarded("vbq_container_open", [&]() -> vbq_status {
        vbq::clear_error();
        if (!buf || !view) return fail(VBQ_ERR_NULL, "vbq_container_open: a pointer is NULL");
        if (len < VBQ_CONTAINER_HEADER)
            return fail(VBQ_ERR_FORMAT, "vbq_container_open: %llu bytes, shorter than the header",
                        (unsigned long long)len);
        if (std::memcmp(buf, kMagic, 8) != 0) return fail(VBQ_ERR_FORMAT, "vbq_container_open: bad magic");
        if (crc32(buf, 84) != get<uint32_t>(buf, 84)) return fail(VBQ_ERR_FORMAT, "vbq_container_open: header checksum");
        if (get<uint32_t>(buf, 8) != VBQ_CONTAINER_VERSION)
            return fail(VBQ_ERR_FORMAT, "vbq_container_open: format version %u, library reads %u", get<uint32_t>(buf, 8),
                        VBQ_CONTAINER_VERSION);
        const uint32_t n = get<uint32_t>(buf, 16), k = get<uint32_t>(buf, 20);
        if (get<uint32_t>(buf, 12) != VBQ_CONTAINER_HEADER || get<uint32_t>(buf, 24) != VBQ_GROUP ||
            get<uint32_t>(buf, 28) != VBQ_TILE_ROWS || get<uint32_t>(buf, 32) != VBQ_TILE_GROUPS || k % VBQ_GROUP)
            return fail(VBQ_ERR_FORMAT, "vbq_container_open: layout constants or k=%u differ from the library's", k);
        const Layout L = layout_of(n, k, get<uint32_t>(buf, 36));
        if (get<uint64_t>(buf, 40) != L.widths || get<uint64_t>(buf, 48) != L.scales ||
            get<uint64_t>(buf, 56) != L.offsets || get<uint64_t>(buf, 64) != L.payload || get<uint64_t>(buf, 72) != L.total)
            return fail(VBQ_ERR_FORMAT, "vbq_container_open: array offsets disagree with n=%u, k=%u", n, k);
        if (L.total > len)
            return fail(VBQ_ERR_FORMAT, "vbq_container_open: needs %llu bytes, image has %llu",
                        (unsigned long long)L.total, (unsigned long long)len);
        if (crc32(buf + VBQ_CONTAINER_HEADER, L.total - VBQ_CONTAINER_HEADER) != get<uint32_t>(buf, 80))
            return fail(VBQ_ERR_FORMAT, "vbq_container_open: body checksum");
        vbq_matrix v{};
        v.abi_version = VBQ_ABI_VERSION;
        v.n = n;
        v.k = k;
        v.payload_bytes = uint32_t(L.payload_bytes);
        v.widths = L.widths_bytes ? buf + L.widths : nullptr;
        v.scales = L.scales_bytes ? reinterpret_cast<const uint16_t *>(buf + L.scales) : nullptr;
        v.tile_offsets = reinterpret_cast<const uint32_t *>(buf + L.offsets);
        v.payload = L.payload_bytes ? buf + L.payload : nullptr;
        vbq_status st = vbq_validate_host(&v);
        if (st != VBQ_OK) return st;
        st = vbq_uniform_width(&v, &v.uniform_bits);
        if (st != VBQ_OK) return st;
        *view = v;
        return VBQ_OK;
    });
}

extern "C" vbq_status vbq_uniform_width(const vbq_matrix *w, uint32_t *bits_out) {
    return vbq::guarded("vbq_uniform_width", [&]() -> vbq_status {
        vbq::clear_error();
        if (!w || !bits_out) return fail(VBQ_ERR_NULL, "vbq_uniform_width: a pointer is NULL");
        if (w->abi_version != VBQ_ABI_VERSION)
            return fail(VBQ_ERR_ABI, "vbq_uniform_width: abi_version %u, library %u", w->abi_version, VBQ_ABI_VERSION);
        if (w->k % VBQ_GROUP) return fail(VBQ_ERR_SHAPE, "vbq_uniform_width: k=%u is not a multiple of 64", w->k);
        const uint64_t groups = uint64_t(w->n) * (w->k / VBQ_GROUP);
        *bits_out = 0;
        if (groups == 0) return VBQ_OK;
        if (!w->widths) return fail(VBQ_ERR_NULL, "vbq_uniform_width: widths is NULL");
        // four codes a byte: a uniform matrix has every full byte equal to c * 0x55
        const uint32_t c = w->widths[0] & 3u;
        const uint8_t full = uint8_t(c * 0x55u);
        for (uint64_t i = 0; i < groups / 4; ++i)
            if (w->widths[i] != full) return VBQ_OK;
        for (uint64_t t = groups / 4 * 4; t < groups; ++t)
            if (((w->widths[t >> 2] >> (2 * (t & 3))) & 3u) != c) return VBQ_OK;
        *bits_out = 1u << c;
        return VBQ_OK;
    });
}
