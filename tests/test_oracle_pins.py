"""Pins for the CPU oracle: checks against facts fixed outside the oracle itself.

Each test compares the oracle with something it does not share code with:
numpy's own binary16 conversion, hand-derived golden vectors, dense float64
products built straight from the drawn codes (never from the oracle's
unpacking), exact rational arithmetic, and invariants of the method (VBQ paper,
arXiv 2607.02893, §3.1 Eq. (1): w_hat = s * q on the symmetric grid, 1-bit =
sign * scale; §6: per-group decode of packed {1,2,4,8}-bit groups).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "vectors.json")


def dense_from_inputs(bits, codes, scales):
    """float64 dense W = s * q straight from the drawn inputs (no packing involved)."""
    n, g = bits.shape
    s = scales.view(np.float16).astype(np.float64)
    return (codes.astype(np.float64).reshape(n, g, 64) * s[:, :, None]).reshape(n, g * 64)


def xf(x):
    return np.asarray(x, dtype=np.uint16).view(np.float16).astype(np.float64)


# ---------------------------------------------------------------- binary16 decoding

def test_half_to_double_all_patterns(oracle_lib):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([oracle_lib.oracle_half_to_double(int(p)) for p in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


# ---------------------------------------------------------------- golden vectors

def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("v", _golden(), ids=lambda v: v["id"])
def test_golden_vector(v):
    n, k = v["n"], v["k"]
    bits = np.array(v["bits"], dtype=np.uint8).reshape(n, k // 64)
    codes = np.array(v["codes"], dtype=np.int8).reshape(n, k)
    scales = np.array([int(h, 16) for h in v["scales_hex"]], dtype=np.uint16).reshape(n, k // 64)
    p = oracle.pack(n, k, bits, codes, scales)
    assert p.widths.tobytes().hex() == v["widths_hex"]
    assert p.tile_offsets.tolist() == v["tile_offsets"]
    assert p.payload.tobytes().hex() == v["payload_hex"]
    if "packed_scales_hex" in v:
        assert p.scales.tobytes().hex() == v["packed_scales_hex"]
    assert np.array_equal(oracle.unpack(p), codes)
    x = np.array(v["x"], dtype=np.float16).view(np.uint16)
    y = oracle.gemv(p, x)
    assert y.tolist() == v["y"]          # exact: every golden sum is exactly representable


# ---------------------------------------------------------------- invariants of the layout

shapes = st.tuples(st.integers(1, 9), st.integers(0, 12).map(lambda g: 64 * g))


@settings(max_examples=40, deadline=None)
@given(shapes, st.integers(0, 2**31 - 1), st.sampled_from(["std", "first", "head", "u1", "u2", "u4", "u8"]))
def test_pack_size_and_roundtrip(shape, seed, mixname):
    n, k = shape
    mix = {"std": W.STD_MIX, "first": W.FIRST_MLP_MIX, "head": W.HEAD_MIX,
           "u1": {1: 1.0}, "u2": {2: 1.0}, "u4": {4: 1.0}, "u8": {8: 1.0}}[mixname]
    bits, codes, scales = W.draw_random_matrix(seed, n, k, mix)
    p = oracle.pack(n, k, bits, codes, scales)
    g = n * (k // 64)
    payload = int((8 * bits.astype(np.int64)).sum())
    assert p.payload_bytes == payload
    tiles_r, tiles_c = -(-n // 64), -(-(k // 64) // 4)
    assert p.total_bytes == payload + (g + 3) // 4 + 2 * g + 4 * (tiles_r * tiles_c + 1)
    # tile offsets = exclusive prefix sum of the tiles' payload sizes (64 rows x 4 groups per tile)
    sizes = [int((8 * bits[64 * a:64 * a + 64, 4 * c:4 * c + 4].astype(np.int64)).sum())
             for a in range(tiles_r) for c in range(tiles_c)]
    assert p.tile_offsets.tolist() == np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64).tolist()
    assert oracle.check_offsets(p) == 0
    assert np.array_equal(oracle.unpack(p), codes)
    assert sorted(p.scales.tolist()) == sorted(scales.reshape(-1).tolist())   # same scales, tile order


def test_all_8bit_is_int8_times_scale():
    n, k = 6, 320
    bits, codes, scales = W.draw_random_matrix(11, n, k, {8: 1.0})
    p = oracle.pack(n, k, bits, codes, scales)
    # every group's 64 payload bytes are literally its int8 codes (compared as a multiset of blocks)
    blocks = sorted(p.payload.reshape(-1, 64).tobytes()[i * 64:(i + 1) * 64] for i in range(n * k // 64))
    assert blocks == sorted(codes.reshape(-1, 64)[t].tobytes() for t in range(n * k // 64))
    x = W.draw_x(12, k)
    ref = dense_from_inputs(bits, codes, scales) @ xf(x)[0]
    assert np.allclose(oracle.gemv(p, x), ref, rtol=1e-13, atol=1e-15)


def test_all_1bit_is_sign_times_scale():
    n, k = 7, 256
    bits, codes, scales = W.draw_random_matrix(13, n, k, {1: 1.0})
    p = oracle.pack(n, k, bits, codes, scales)
    # one sign bit per weight, LSB first, set for negative weights (8-byte blocks, as a multiset)
    want = sorted(np.packbits((codes.reshape(-1, 64)[t] < 0).astype(np.uint8), bitorder="little").tobytes()
                  for t in range(n * k // 64))
    assert sorted(p.payload[8 * t:8 * t + 8].tobytes() for t in range(n * k // 64)) == want
    x = W.draw_x(14, k)
    s = np.repeat(scales.view(np.float16).astype(np.float64), 64, axis=1)
    ref = (np.sign(codes.astype(np.float64)) * s) @ xf(x)[0]
    assert np.allclose(oracle.gemv(p, x), ref, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- arithmetic pins

@settings(max_examples=30, deadline=None)
@given(st.integers(1, 12), st.integers(1, 8), st.integers(1, 4), st.integers(0, 2**31 - 1))
def test_matches_dense_float64(n, g, m, seed):
    k = 64 * g
    bits, codes, scales = W.draw_random_matrix(seed, n, k, W.FIRST_MLP_MIX)
    p = oracle.pack(n, k, bits, codes, scales)
    x = W.draw_x(seed + 1, k, m)
    wd = dense_from_inputs(bits, codes, scales)
    ref = xf(x) @ wd.T
    got = oracle.gemm(p, x)
    bound = (64 + g) * 2.0**-52 * (np.abs(xf(x)) @ np.abs(wd).T) + 1e-300
    assert np.all(np.abs(got - ref) <= 2 * bound)


def test_matches_exact_rational():
    rng_seed = 77
    for n, k in ((3, 64), (2, 192), (1, 512)):
        bits, codes, scales = W.draw_random_matrix((rng_seed, n, k), n, k, W.STD_MIX)
        p = oracle.pack(n, k, bits, codes, scales)
        x = W.draw_x((rng_seed, k), k)
        got = oracle.gemv(p, x)
        xs = [Fraction(float(v)) for v in xf(x)[0]]
        ss = scales.view(np.float16).astype(np.float64)
        for r in range(n):
            exact = Fraction(0)
            mag = Fraction(0)
            for j in range(k // 64):
                s = Fraction(float(ss[r, j]))
                d = sum(int(codes[r, 64 * j + i]) * xs[64 * j + i] for i in range(64))
                exact += s * d
                mag += abs(s) * sum(abs(int(codes[r, 64 * j + i]) * xs[64 * j + i]) for i in range(64))
            err = abs(Fraction(float(got[r])) - exact)
            assert err <= (64 + k // 64) * Fraction(2) ** -52 * mag


def test_one_hot_gives_exact_column():
    n, k = 9, 448
    bits, codes, scales = W.draw_random_matrix(21, n, k, W.FIRST_MLP_MIX)
    p = oracle.pack(n, k, bits, codes, scales)
    wd = dense_from_inputs(bits, codes, scales)
    for col in (0, 1, 63, 64, 200, k - 1):
        x = np.zeros(k, dtype=np.float16)
        x[col] = 1.0
        assert np.array_equal(oracle.gemv(p, x.view(np.uint16)), wd[:, col])


def test_all_ones_gives_integer_row_sums_times_scale():
    n, k = 4, 256
    bits, codes, scales = W.draw_random_matrix(22, n, k, W.STD_MIX)
    p = oracle.pack(n, k, bits, codes, scales)
    x = np.ones(k, dtype=np.float16).view(np.uint16)
    sums = codes.astype(np.int64).reshape(n, k // 64, 64).sum(axis=2)
    ref = (sums * scales.view(np.float16).astype(np.float64)).sum(axis=1)
    assert np.array_equal(oracle.gemv(p, x), ref)


def test_zero_scales_and_zero_x():
    n, k = 3, 128
    bits, codes, _ = W.draw_random_matrix(23, n, k, W.STD_MIX)
    p = oracle.pack(n, k, bits, codes, np.zeros((n, 2), np.uint16))
    assert np.all(oracle.gemv(p, W.draw_x(1, k)) == 0)
    bits, codes, scales = W.draw_random_matrix(24, n, k, W.STD_MIX)
    p = oracle.pack(n, k, bits, codes, scales)
    assert np.all(oracle.gemv(p, np.zeros(k, np.uint16)) == 0)


def test_scaling_x_by_two_is_exact():
    n, k = 5, 320
    bits, codes, scales = W.draw_random_matrix(25, n, k, W.STD_MIX)
    p = oracle.pack(n, k, bits, codes, scales)
    x = W.draw_x(26, k)
    x2 = (xf(x) * 2).astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.gemv(p, x2), 2 * oracle.gemv(p, x))


def test_gemm_rows_are_independent_gemvs():
    n, k, m = 6, 192, 5
    bits, codes, scales = W.draw_random_matrix(27, n, k, W.STD_MIX)
    p = oracle.pack(n, k, bits, codes, scales)
    x = W.draw_x(28, k, m)
    y = oracle.gemm(p, x)
    for i in range(m):
        assert np.array_equal(y[i], oracle.gemv(p, x[i]))
    part = oracle.gemm(p, x, rows=(2, 5))
    assert np.array_equal(part[:, 2:5], y[:, 2:5])
    assert np.all(np.isnan(part[:, :2])) and np.all(np.isnan(part[:, 5:]))


def test_threaded_matches_serial():
    n, k = 37, 256
    bits, codes, scales = W.draw_random_matrix(29, n, k, W.STD_MIX)
    p = oracle.pack(n, k, bits, codes, scales)
    x = W.draw_x(30, k)
    assert np.array_equal(oracle.gemv_threaded(p, x, 3, 30, 4), oracle.gemv(p, x)[3:30])


# ---------------------------------------------------------------- degenerate shapes

def test_empty_shapes():
    p = oracle.pack(0, 128, np.zeros(0, np.uint8), np.zeros(0, np.int8), np.zeros(0, np.uint16))
    assert p.payload_bytes == 0 and p.tile_offsets.tolist() == [0]      # no tiles when n == 0
    assert oracle.gemv(p, W.draw_x(1, 128)).shape == (0,)
    p = oracle.pack(3, 0, np.zeros(0, np.uint8), np.zeros(0, np.int8), np.zeros(0, np.uint16))
    assert p.tile_offsets.tolist() == [0]      # no tiles when k == 0
    assert np.all(oracle.gemv(p, np.zeros(0, np.uint16)) == 0)


# ---------------------------------------------------------------- rejected inputs

def _ok_inputs(n=2, k=128):
    return W.draw_random_matrix(31, n, k, W.STD_MIX)


def test_rejects_bad_width():
    bits, codes, scales = _ok_inputs()
    bits = bits.copy()
    bits[1, 0] = 3
    with pytest.raises(oracle.OracleError) as e:
        oracle.pack(2, 128, bits, codes, scales)
    assert e.value.status == oracle.ERR_WIDTH


@pytest.mark.parametrize("b,bad", [(1, 0), (1, 2), (2, -2), (2, 2), (4, -8), (4, 8), (8, -128)])
def test_rejects_codes_off_grid(b, bad):
    bits = np.full((1, 1), b, np.uint8)
    codes = np.ones((1, 64), np.int8)
    codes[0, 17] = bad
    with pytest.raises(oracle.OracleError) as e:
        oracle.pack(1, 64, bits, codes, np.full((1, 1), 0x3C00, np.uint16))
    assert e.value.status == oracle.ERR_CODE


@pytest.mark.parametrize("h", [0x7C00, 0xFC00, 0x7E00])
def test_rejects_nonfinite_scale(h):
    bits, codes, scales = _ok_inputs()
    scales = scales.copy()
    scales[0, 1] = h
    with pytest.raises(oracle.OracleError) as e:
        oracle.pack(2, 128, bits, codes, scales)
    assert e.value.status == oracle.ERR_SCALE


def test_rejects_ragged_k():
    with pytest.raises(oracle.OracleError) as e:
        oracle.pack_sizes(2, 100, np.ones(4, np.uint8))
    assert e.value.status == oracle.ERR_SHAPE


def test_rejects_inconsistent_offsets():
    bits, codes, scales = _ok_inputs()
    p = oracle.pack(2, 128, bits, codes, scales)
    p.tile_offsets = p.tile_offsets.copy()
    p.tile_offsets[1] += 8
    assert oracle.check_offsets(p) == oracle.ERR_OFFSETS
    with pytest.raises(oracle.OracleError):
        oracle.gemv(p, W.draw_x(1, 128))


@pytest.mark.parametrize("b", [2, 4, 8])
def test_reserved_pattern_decodes_as_most_negative(b):
    # hand-built payload holding the reserved two's complement pattern -2^(b-1)
    f = 1 << (b - 1)
    bitstr = np.zeros(64 * b, np.uint8)
    for i in range(64):
        for t in range(b):
            bitstr[i * b + t] = (f >> t) & 1
    payload = np.packbits(bitstr, bitorder="little")
    c = {2: 1, 4: 2, 8: 3}[b]
    p = oracle.Packed(1, 64, np.array([c], np.uint8), np.array([0x3C00], np.uint16),
                      np.array([0, 8 * b], np.uint32), payload)
    assert np.all(oracle.unpack(p) == -(1 << (b - 1)))


def test_swiglu_pins():
    from scipy.special import expit
    rng = np.random.default_rng(3)
    u = rng.standard_normal(1000) * 5
    # the pages' inertness statement: silu(0) * u = 0 for every u
    assert np.all(oracle.swiglu(np.zeros(1000), u) == 0)
    g = rng.standard_normal(1000) * 8
    # g * sigmoid(g) * u through the library logistic
    assert np.allclose(oracle.swiglu(g, u), g * expit(g) * u, rtol=1e-14, atol=0)
    # closed form: silu(g) - silu(-g) = g
    one = np.ones_like(g)
    assert np.allclose(oracle.swiglu(g, one) - oracle.swiglu(-g, one), g, rtol=1e-13, atol=1e-13)
    # limits: silu(g) -> g for large g, -> 0 (not NaN) for very negative g
    assert oracle.swiglu(np.array([60.0]), np.array([2.0]))[0] == 120.0
    assert oracle.swiglu(np.array([-1000.0]), np.array([3.0]))[0] == 0.0
