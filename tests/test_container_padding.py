"""CPU checks of the export-side host entry points: the padding contract
check and the versioned container.

Padding (VBQ paper, arXiv 2607.02893, §6 "Granularity is
deployment-friendly": MLP intermediates are zero-padded so the contracted
dimension is a multiple of 512, and the padded channels are inert since
silu(0) * u = 0): the library's verdict is compared with a brute-force test
on the unpacked arrays (every padded weight s * q is zero). Container: round
trips, checksums against zlib's CRC-32, and every corruption refused.
"""
import zlib

import numpy as np
import pytest

import workloads as W


@pytest.fixture(scope="module")
def V():
    import decode_gemv_02_amd as V
    return V


def padded_matrix(seed, n_real, k_real, n, k, mix=None):
    """Codes and scales of an n_real x k_real matrix zero-padded to n x k (natural [n][G] order)."""
    bits, codes, scales = W.draw_random_matrix(seed, n, k, mix or W.STD_MIX)
    codes = codes.copy()
    scales = scales.copy()
    codes[n_real:, :] = 0
    codes[:, k_real:] = 0
    pad_groups = np.zeros(bits.shape, bool)
    pad_groups[n_real:, :] = True
    pad_groups[:, k_real // 64:] = True
    # a zero-padded group quantizes to scale 0 (and +1 codes at 1 bit, which the zero scale makes inert)
    scales[pad_groups] = 0
    codes[np.repeat(pad_groups & (bits == 1), 64, axis=1)] = 1
    return bits, codes, scales


def brute_force_inert(bits, codes, scales, n_real, k_real):
    s = np.repeat(scales.view(np.float16).astype(np.float64), 64, axis=1)
    w = codes.astype(np.float64) * s
    pad = np.zeros(w.shape, bool)
    pad[n_real:, :] = True
    pad[:, k_real:] = True
    return bool(np.all(w[pad] == 0))


@pytest.mark.parametrize("n_real, k_real, n, k", [(300, 8960, 320, 9216), (64, 448, 64, 512), (5, 512, 5, 512),
                                                  (1536, 1500, 1536, 1536)])
def test_zero_padded_matrix_passes(V, n_real, k_real, n, k):
    bits, codes, scales = padded_matrix((n, k), n_real, k_real // 64 * 64, n, k)
    k_real = k_real // 64 * 64 if k_real % 64 == 0 else k_real
    if k_real % 64:                       # a partial group: zero its padded codes at b >= 2, zero scale at 1 bit
        j = k_real // 64
        codes[:, k_real:] = 0
        one = bits[:, j] == 1
        scales[one, j] = 0
        codes[one, 64 * j:64 * j + 64] = 1
    assert brute_force_inert(bits, codes, scales, n_real, k_real)
    h = V.vbq_pack(n, k, bits, codes, scales)
    V.vbq_check_padding(h, n_real, k_real, 512)


def test_check_agrees_with_brute_force_on_planted_weights(V):
    n_real, k_real, n, k = 100, 896, 128, 1024
    base = padded_matrix((9,), n_real, k_real, n, k)
    rng = np.random.default_rng(10)
    for trial in range(60):
        bits, codes, scales = (a.copy() for a in base)
        r = int(rng.integers(0, n))
        c = int(rng.integers(k_real, k)) if trial % 2 else int(rng.integers(0, k))
        if trial % 3 == 0:
            r = int(rng.integers(n_real, n))
        j = c // 64
        b = int(bits[r, j])
        if b == 1:
            scales[r, j] = np.float16(0.01).view(np.uint16)     # a 1-bit group: a non-zero scale is never inert
        else:
            codes[r, c] = 1
            if scales[r, j] == 0:
                scales[r, j] = np.float16(0.01).view(np.uint16)
        expect = brute_force_inert(bits, codes, scales, n_real, k_real)
        h = V.vbq_pack(n, k, bits, codes, scales)
        if expect:
            V.vbq_check_padding(h, n_real, k_real, 512)
        else:
            with pytest.raises(V.VbqError) as e:
                V.vbq_check_padding(h, n_real, k_real, 512)
            assert e.value.status == V.ERR_PADDING


def test_check_padding_shape_errors(V):
    bits, codes, scales = padded_matrix((3,), 64, 448, 64, 512)
    h = V.vbq_pack(64, 512, bits, codes, scales)
    for args in [(64, 448, 0), (64, 448, 1024), (65, 448, 512), (64, 576, 512)]:
        with pytest.raises(V.VbqError) as e:
            V.vbq_check_padding(h, *args)
        assert e.value.status == V.ERR_SHAPE
    V.vbq_check_padding(h, 64, 448, 256)
    # a scale of -0 also zeroes its group
    scales2 = scales.copy()
    scales2[:, 7] = 0x8000
    codes2 = codes.copy()
    codes2[:, 7 * 64:] = np.where(bits[:, 7:8].repeat(64, axis=1) == 1, -1, 1)
    V.vbq_check_padding(V.vbq_pack(64, 512, bits, codes2, scales2), 64, 448, 512)


# ------------------------------------------------------------------ container

@pytest.mark.parametrize("n, k", [(1, 64), (65, 320), (300, 4096 + 64), (0, 128)])
def test_container_round_trip(V, tmp_path, n, k):
    bits, codes, scales = W.draw_random_matrix((n, k, 5), n, k, W.STD_MIX)
    h = V.vbq_pack(n, k, bits, codes, scales)
    img = V.vbq_container_bytes(h)
    hdr = img[:128]
    f = lambda at, dt: int(hdr[at:at + np.dtype(dt).itemsize].view(dt)[0])   # noqa: E731
    assert bytes(hdr[:8]) == b"VBQPACK\0" and f(8, np.uint32) == 1 and f(12, np.uint32) == 128
    assert (f(16, np.uint32), f(20, np.uint32), f(36, np.uint32)) == (n, k, h.payload_bytes)
    offs = [f(at, np.uint64) for at in (40, 48, 56, 64)]
    assert all(o % 256 == 0 for o in offs) and f(72, np.uint64) == img.size == offs[3] + h.payload_bytes
    assert f(80, np.uint32) == zlib.crc32(img[128:].tobytes())
    assert f(84, np.uint32) == zlib.crc32(img[:84].tobytes())
    assert np.all(hdr[88:] == 0)
    path = tmp_path / "m.vbq"
    V.vbq_save(str(path), h)
    for g in (V.vbq_container_open(img), V.vbq_load(str(path))):
        assert (g.n, g.k) == (n, k)
        for a, b in ((g.widths, h.widths), (g.scales, h.scales), (g.tile_offsets, h.tile_offsets),
                     (g.payload, h.payload)):
            assert np.array_equal(a, b)


def _refresh_crcs(img):
    img[80:84] = np.frombuffer(np.uint32(zlib.crc32(img[128:].tobytes())).tobytes(), np.uint8)
    img[84:88] = np.frombuffer(np.uint32(zlib.crc32(img[:84].tobytes())).tobytes(), np.uint8)
    return img


def test_container_refuses_corruption(V):
    n, k = 70, 384
    h = V.vbq_pack(n, k, *W.draw_random_matrix((77,), n, k, W.STD_MIX))
    good = V.vbq_container_bytes(h)
    rng = np.random.default_rng(1)

    def status(img):
        try:
            V.vbq_container_open(img)
            return V.OK
        except V.VbqError as e:
            return e.value.status if hasattr(e, "value") else e.status

    for pos in list(rng.integers(0, good.size, 40)) + [0, 8, 16, 84, 128, good.size - 1]:
        bad = good.copy()
        bad[pos] ^= 0x10
        assert status(bad) == V.ERR_FORMAT, pos
    assert status(good[:-1]) == V.ERR_FORMAT          # truncated
    assert status(good[:100]) == V.ERR_FORMAT
    bad = good.copy()
    bad[8] = 2                                         # another version, checksums made consistent
    assert status(_refresh_crcs(bad)) == V.ERR_FORMAT
    bad = good.copy()
    bad[24] = 32                                       # another group size
    assert status(_refresh_crcs(bad)) == V.ERR_FORMAT
    bad = good.copy()
    bad[16] += 64                                      # n that disagrees with the array offsets
    assert status(_refresh_crcs(bad)) == V.ERR_FORMAT
    bad = good.copy()
    bad[16] += 1                                       # same offsets, but the tile table no longer fits
    assert status(_refresh_crcs(bad)) in (V.ERR_FORMAT, V.ERR_OFFSETS)
    # a well-formed container of an invalid matrix: the validator's verdict comes through
    bad = good.copy()
    tile_off = int(bad[56:64].view(np.uint64)[0])
    bad[tile_off + 4:tile_off + 8] = np.frombuffer(np.uint32(1).tobytes(), np.uint8)
    assert status(_refresh_crcs(bad)) == V.ERR_OFFSETS
    assert status(good) == V.OK


def test_container_write_errors(V):
    import ctypes
    n, k = 4, 128
    h = V.vbq_pack(n, k, *W.draw_random_matrix((78,), n, k, W.STD_MIX))
    v = h.view()
    size = ctypes.c_uint64()
    assert V.lib.vbq_container_size(ctypes.byref(v), ctypes.byref(size)) == V.OK
    out = np.zeros(size.value, np.uint8)
    written = ctypes.c_uint64()
    assert V.lib.vbq_container_write(ctypes.byref(v), out.ctypes.data, out.size - 1, ctypes.byref(written)) \
        == V.ERR_CAPACITY
    assert V.lib.vbq_container_write(ctypes.byref(v), None, out.size, ctypes.byref(written)) == V.ERR_NULL
    assert V.lib.vbq_container_size(None, ctypes.byref(size)) == V.ERR_NULL
    assert V.lib.vbq_container_open(None, 0, None) == V.ERR_NULL
