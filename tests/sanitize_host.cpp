// Drives the library's host entry points (packer, validator, padding check,
// container, head recipe) under AddressSanitizer and UndefinedBehaviorSanitizer:
// valid inputs, then truncated and corrupted container images and corrupted
// packed arrays, which must be rejected with a status and never read or write
// out of bounds. Built and run by tests/test_sanitizers.py (host code only; no
// device code is compiled). Exit status 0 when every check holds.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "vbq.h"

namespace {

int g_fail = 0;

void check(bool ok, const char *what, int iter) {
    if (!ok) {
        ++g_fail;
        std::fprintf(stderr, "iteration %d: %s (%s)\n", iter, what, vbq_last_error());
    }
}

struct Packed {
    uint32_t n = 0, k = 0;
    std::vector<uint8_t> widths, payload;
    std::vector<uint16_t> scales;
    std::vector<uint32_t> offsets;
    vbq_matrix view() const {
        vbq_matrix v{};
        v.abi_version = VBQ_ABI_VERSION;
        v.n = n;
        v.k = k;
        v.payload_bytes = static_cast<uint32_t>(payload.size());
        v.widths = widths.empty() ? nullptr : widths.data();
        v.scales = scales.empty() ? nullptr : scales.data();
        v.tile_offsets = offsets.data();
        v.payload = payload.empty() ? nullptr : payload.data();
        return v;
    }
};

uint16_t random_finite_half(std::mt19937_64 &rng) {
    for (;;) {
        const uint16_t h = static_cast<uint16_t>(rng());
        if (((h >> 10) & 0x1F) != 0x1F) return h;
    }
}

bool make(std::mt19937_64 &rng, uint32_t n, uint32_t k, Packed &p) {
    const uint32_t G = k / VBQ_GROUP;
    const uint64_t groups = uint64_t(n) * G;
    std::vector<uint8_t> bits(groups);
    std::vector<int8_t> codes(uint64_t(n) * k);
    std::vector<uint16_t> scales(groups);
    static const uint8_t widths[4] = {1, 2, 4, 8};
    for (uint64_t t = 0; t < groups; ++t) {
        const uint8_t b = widths[rng() % 4];
        bits[t] = b;
        scales[t] = random_finite_half(rng);
        for (uint32_t i = 0; i < VBQ_GROUP; ++i) {
            int q;
            if (b == 1) {
                q = (rng() & 1) ? 1 : -1;
            } else {
                const int lim = (1 << (b - 1)) - 1;
                q = static_cast<int>(rng() % (2 * lim + 1)) - lim;
            }
            codes[t * VBQ_GROUP + i] = static_cast<int8_t>(q);
        }
    }
    vbq_sizes sz{};
    if (vbq_pack_sizes(n, k, bits.data(), &sz) != VBQ_OK) return false;
    p.n = n;
    p.k = k;
    p.widths.assign(sz.widths_bytes, 0);
    p.scales.assign(sz.scales_bytes / 2, 0);
    p.offsets.assign(sz.offsets_bytes / 4, 0);
    p.payload.assign(sz.payload_bytes, 0);
    return vbq_pack(n, k, bits.data(), codes.data(), scales.data(), p.widths.data(), p.scales.data(),
                    p.offsets.data(), p.payload.data(), p.payload.size()) == VBQ_OK;
}

void put32(std::vector<uint8_t> &img, size_t at, uint32_t v) { std::memcpy(img.data() + at, &v, 4); }

// CRC-32 (IEEE 802.3, reflected 0xEDB88320), to forge images whose checksums hold
uint32_t crc32(const uint8_t *p, size_t len) {
    uint32_t c = 0xFFFFFFFFu;
    for (size_t i = 0; i < len; ++i) {
        c ^= p[i];
        for (int b = 0; b < 8; ++b) c = (c & 1) ? 0xEDB88320u ^ (c >> 1) : c >> 1;
    }
    return c ^ 0xFFFFFFFFu;
}

void reseal_header(std::vector<uint8_t> &img) { put32(img, 84, crc32(img.data(), 84)); }

}  // namespace

int main(int argc, char **argv) {
    const int iters = argc > 1 ? std::atoi(argv[1]) : 60;
    std::mt19937_64 rng(20261203);
    for (int it = 0; it < iters; ++it) {
        const uint32_t n = static_cast<uint32_t>(rng() % 150);
        const uint32_t k = 64u * static_cast<uint32_t>(rng() % 12);
        Packed p;
        check(make(rng, n, k, p), "pack", it);
        vbq_matrix v = p.view();
        check(vbq_validate_host(&v) == VBQ_OK, "validate packed", it);
        uint32_t ub = 0;
        check(vbq_uniform_width(&v, &ub) == VBQ_OK, "uniform width", it);
        (void)vbq_check_padding(&v, n ? static_cast<uint32_t>(rng() % (n + 1)) : 0,
                                k ? static_cast<uint32_t>(rng() % (k + 1)) : 0, (rng() & 1) ? 64 : 512);

        // container round trip, then every kind of damage
        uint64_t size = 0, written = 0;
        check(vbq_container_size(&v, &size) == VBQ_OK, "container size", it);
        std::vector<uint8_t> img(size);
        check(vbq_container_write(&v, img.data(), img.size(), &written) == VBQ_OK && written == size,
              "container write", it);
        vbq_matrix back{};
        check(vbq_container_open(img.data(), img.size(), &back) == VBQ_OK && back.n == n && back.k == k,
              "container open", it);
        for (int t = 0; t < 8; ++t) {   // truncated images: copies holding only the first len bytes
            const size_t len = size ? static_cast<size_t>(rng() % size) : 0;
            std::vector<uint8_t> cut(img.begin(), img.begin() + static_cast<long>(len));
            check(vbq_container_open(cut.data(), cut.size(), &back) != VBQ_OK, "truncated image accepted", it);
        }
        for (int t = 0; t < 16; ++t) {  // flipped bytes anywhere
            std::vector<uint8_t> bad = img;
            const size_t at = static_cast<size_t>(rng() % bad.size());
            bad[at] ^= static_cast<uint8_t>(1u << (rng() % 8));
            (void)vbq_container_open(bad.data(), bad.size(), &back);
        }
        if (k) {   // a header claiming a huge n, with its checksum made to hold (with k = 0 any n is valid)
            std::vector<uint8_t> bad = img;
            put32(bad, 16, 0x7FFFFFFFu);
            reseal_header(bad);
            check(vbq_container_open(bad.data(), bad.size(), &back) == VBQ_ERR_FORMAT, "huge n accepted", it);
        }
        if (n == 0 || k == 0) continue;
        // corrupted packed arrays handed to the validator directly
        for (int t = 0; t < 6; ++t) {
            Packed q = p;
            switch (t % 3) {
                case 0: q.widths[rng() % q.widths.size()] ^= static_cast<uint8_t>(1u << (rng() % 8)); break;
                case 1: q.offsets[rng() % q.offsets.size()] += static_cast<uint32_t>(1 + rng() % 4096); break;
                default:
                    if (!q.payload.empty()) q.payload[rng() % q.payload.size()] ^= 0xFF;
                    break;
            }
            vbq_matrix qv = q.view();
            (void)vbq_validate_host(&qv);
            (void)vbq_check_padding(&qv, n, k, 64);
        }
    }
    // packer rejections
    {
        uint8_t bits[2] = {2, 3};
        vbq_sizes sz{};
        check(vbq_pack_sizes(1, 128, bits, &sz) == VBQ_ERR_WIDTH, "width 3 accepted", -1);
        check(vbq_pack_sizes(1, 100, bits, &sz) == VBQ_ERR_SHAPE, "k % 64 accepted", -1);
    }
    // head recipe on random frequencies (ties included), and on no rows
    for (int it = 0; it < 20; ++it) {
        const uint32_t rows = static_cast<uint32_t>(rng() % 3000);
        std::vector<uint64_t> freq(rows);
        for (auto &f : freq) f = rng() % 50;
        std::vector<uint8_t> bits(rows);
        std::vector<uint32_t> order(rows);
        uint32_t tiers[4];
        check(vbq_recipe_head_bits(rows, freq.data(), bits.data()) == VBQ_OK, "head bits", it);
        check(vbq_recipe_head_order(rows, freq.data(), order.data()) == VBQ_OK, "head order", it);
        check(vbq_recipe_head_tiers(rows, freq.data(), order.data(), tiers) == VBQ_OK &&
                  tiers[0] + tiers[1] + tiers[2] + tiers[3] == rows,
              "head tiers", it);
    }
    std::printf("host sanitizer run: %d failures\n", g_fail);
    return g_fail ? 1 : 0;
}
