"""Planted-mistake check for the oracle's pins (CPU only).

Each case copies ``oracle/vbq_oracle.c``, plants one plausible mistake (a
flipped sign, a wrong bit order, a dropped term, a transposed index...),
compiles the copy into a temporary library and runs the pin checks against
it. A pin set that lets any of these mutants through would not be pinning the
oracle, so every mutant must fail at least one check.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W
from oracle.build import SRC, build

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "vectors.json")

MUTANTS = {
    "one_bit_sign": ("return f ? -1 : 1;", "return f ? 1 : -1;"),
    "twos_complement_threshold": ("if (f >= (1u << (b - 1)))", "if (f > (1u << (b - 1)))"),
    "field_bit_order_msb_first": ("unsigned f = (payload[p + bit / 8] >> (bit % 8))",
                                  "unsigned f = (payload[p + bit / 8] >> (8 - b - bit % 8))"),
    "two_bit_fields_not_interleaved": ("int e = i % 16, m = e / 2 + 8 * (e % 2);", "int e = i % 16, m = e;"),
    "four_bit_fields_not_interleaved": ("int e = i % 8, m = e / 2 + 4 * (e % 2);", "int e = i % 8, m = e;"),
    "dropped_scale": ("acc += s * d;", "acc += d;"),
    "dropped_product_terms": ("d += (double)decode_code", "d = (double)decode_code"),
    "x_reversed_in_group": ("xm[(uint64_t)j * 64 + i]", "xm[(uint64_t)j * 64 + (63 - i)]"),
    "width_code_msb_first": ("int c = (widths[t / 4] >> (2 * (t % 4))) & 3;",
                             "int c = (widths[t / 4] >> (2 * (3 - t % 4))) & 3;"),
    "buckets_descending": ("for (int b = 1; b <= 8; b *= 2)", "for (int b = 8; b >= 1; b /= 2)"),
    "bucket_row_major": ("for (uint32_t j = j0; j < j1; ++j)\n                    for (uint32_t r = r0; r < r1; ++r) {",
                         "for (uint32_t r = r0; r < r1; ++r)\n                    for (uint32_t j = j0; j < j1; ++j) {"),
    "tile_rows_32": ("#define TILE_ROWS 64u", "#define TILE_ROWS 32u"),
    "tile_groups_8": ("#define TILE_GROUPS 4u", "#define TILE_GROUPS 8u"),
    "half_subnormal_exponent": ("v = ldexp((double)frac, -24);", "v = ldexp((double)frac, -25);"),
    "half_bias": ("v = ldexp((double)(1024 + frac), expo - 25);", "v = ldexp((double)(1024 + frac), expo - 24);"),
    "half_implicit_bit": ("v = ldexp((double)(1024 + frac), expo - 25);", "v = ldexp((double)frac, expo - 25);"),
    "scale_natural_order": ("double s = oracle_half_to_double(scales[meta_index(n, G, r, j)]);",
                            "double s = oracle_half_to_double(scales[t]);"),
    "metadata_natural_order": ("    return (uint64_t)TILE_ROWS * a * G + (uint64_t)rows * TILE_GROUPS * c +",
                               "    return (uint64_t)r * G + j;\n    return (uint64_t)TILE_ROWS * a * G + (uint64_t)rows * TILE_GROUPS * c +"),
    "packer_sign": ("f = q < 0 ? 1u : 0u;", "f = q > 0 ? 1u : 0u;"),
    "packer_width_code": ("int c = b == 1 ? 0 : b == 2 ? 1 : b == 4 ? 2 : 3;",
                          "int c = b == 1 ? 0 : b == 2 ? 2 : b == 4 ? 1 : 3;"),
    "tile_offsets_shifted": ("tile_offsets[tile] = (uint32_t)pos;\n            for",
                             "tile_offsets[tile] = (uint32_t)(tile ? pos + 8 : pos);\n            for"),
    "gemm_output_transposed": ("y[(uint64_t)mm * n + r] = acc;",
                               "y[((uint64_t)r * m + mm) < (uint64_t)m * n ? ((uint64_t)r * m + mm) : 0] = acc;"),
    "grid_too_wide": ("int lim = (1 << (b - 1)) - 1;", "int lim = (1 << (b - 1));"),
}


def dense(bits, codes, scales):
    n, g = bits.shape
    s = scales.view(np.float16).astype(np.float64)
    return (codes.astype(np.float64).reshape(n, g, 64) * s[:, :, None]).reshape(n, g * 64)


def failed_pins(lib):
    """Names of the pin checks this library fails (empty = passes all)."""
    bad = []
    # binary16 decoding vs numpy
    pats = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([lib.oracle_half_to_double(int(p)) for p in pats])
    fin = np.isfinite(ref)
    if not np.array_equal(got[fin], ref[fin]):
        bad.append("half")
    # golden vectors
    for v in json.load(open(GOLDEN)):
        n, k = v["n"], v["k"]
        bits = np.array(v["bits"], np.uint8).reshape(n, k // 64)
        codes = np.array(v["codes"], np.int8).reshape(n, k)
        scales = np.array([int(h, 16) for h in v["scales_hex"]], np.uint16).reshape(n, k // 64)
        try:
            p = oracle.pack(n, k, bits, codes, scales, lib=lib)
            ok = (p.payload.tobytes().hex() == v["payload_hex"] and p.widths.tobytes().hex() == v["widths_hex"]
                  and p.scales.tobytes().hex() == v.get("packed_scales_hex", p.scales.tobytes().hex())
                  and p.tile_offsets.tolist() == v["tile_offsets"]
                  and oracle.gemv(p, np.array(v["x"], np.float16).view(np.uint16), lib=lib).tolist() == v["y"])
        except oracle.OracleError:
            ok = False
        if not ok:
            bad.append("golden:" + v["id"])
    # dense float64 products from the drawn inputs, several inputs at once
    for seed, (n, k) in enumerate(((5, 320), (3, 128))):
        bits, codes, scales = W.draw_random_matrix((seed, 99), n, k, W.FIRST_MLP_MIX)
        try:
            p = oracle.pack(n, k, bits, codes, scales, lib=lib)
            x = W.draw_x((seed, 98), k, 3)
            y = oracle.gemm(p, x, lib=lib)
            ref = x.view(np.float16).astype(np.float64) @ dense(bits, codes, scales).T
            if not np.allclose(y, ref, rtol=1e-12, atol=1e-12):
                bad.append(f"dense:{n}x{k}")
            if not np.array_equal(oracle.unpack(p, lib=lib), codes):
                bad.append(f"roundtrip:{n}x{k}")
        except oracle.OracleError:
            bad.append(f"dense:{n}x{k}:error")
    # the reserved two's complement pattern -2^(b-1) decodes as -2^(b-1)
    for b, c in ((2, 1), (4, 2), (8, 3)):
        bitstr = np.zeros(64 * b, np.uint8)
        bitstr[b - 1::b] = 1
        p = oracle.Packed(1, 64, np.array([c], np.uint8), np.array([0x3C00], np.uint16),
                          np.array([0, 8 * b], np.uint32), np.packbits(bitstr, bitorder="little"))
        try:
            if not np.all(oracle.unpack(p, lib=lib) == -(1 << (b - 1))):
                bad.append(f"reserved:{b}")
        except oracle.OracleError:
            bad.append(f"reserved:{b}:error")
    # grid: a code just outside the grid must be rejected
    for b, lim in ((2, 1), (4, 7), (8, 127)):
        codes = np.zeros((1, 64), np.int8)
        codes[0, 3] = -lim - 1
        try:
            oracle.pack(1, 64, np.full((1, 1), b, np.uint8), codes, np.full((1, 1), 0x3C00, np.uint16), lib=lib)
            bad.append(f"grid:{b}")
        except oracle.OracleError:
            pass
    return bad


def test_unmutated_oracle_passes_every_pin():
    assert failed_pins(oracle.load()) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new, 1))
    lib_path = str(tmp_path / "libmutant.so")
    build(str(mutated), lib_path)
    lib = oracle.load(lib_path)
    assert failed_pins(lib), f"mutant {name} passed every pin"
