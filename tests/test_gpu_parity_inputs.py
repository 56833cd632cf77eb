"""GPU parity on inputs the seeded workloads do not draw: activations with a
common mode, payloads that hold the reserved two's-complement pattern, and
negative scales. Every case runs through the mixed-width kernel (matrices
that do not declare their width), the one-width kernels (matrices that do)
and the small-batch paths, against the CPU oracle at the parity bar
(relative L2 <= 1e-3 and max abs <= 2e-3 * ||x||_2 * max|s| per output
vector); decoded codes are compared bit for bit.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.conftest import gpu_available
from tests.helpers import assert_within_tolerance, tolerance_report

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def V():
    import torch  # noqa: F401
    import decode_gemv_02_amd as V
    return V


def print_case(**kw):
    print("CASE", " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def run(V, dm, x_bits):
    """Y [m, n] in float64: the GEMV for m = 1, the small-batch entry point otherwise."""
    import torch
    x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.float16)).cuda()
    m = x.shape[0]
    y = torch.full((m, dm.n), float("nan"), dtype=torch.float32, device="cuda")
    if m == 1:
        V.vbq_gemv(dm, x[0], y[0])
    else:
        V.vbq_gemm_smallbatch(dm, x, y)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def both_kernels(V, host):
    """The same packed bytes as a one-width matrix (declared) and as a mixed-width one (not declared)."""
    return {"declared": V.DeviceMatrix(host), "mixed": V.DeviceMatrix(host, uniform=False)}


@pytest.mark.parametrize("mean", [1.0, 4.0, -16.0])
@pytest.mark.parametrize("mix", [{2: 1.0}, {4: 1.0}, {8: 1.0}, {1: 1.0}, W.STD_MIX])
def test_offset_activations(V, mean, mix):
    """x = mean + 0.5 N(0,1): the 2-, 4- and 8-bit paths take 2^(b-1) times the group's activation
    sum off once per group, so a large common mode must not cost precision."""
    n, k = 200, 4096 + 256
    b = max(mix) if len(mix) == 1 else 0
    bits, codes, scales = W.draw_random_matrix((110, b, int(mean) + 100), n, k, mix)
    host = V.vbq_pack(n, k, bits, codes, scales)
    p = oracle.pack(n, k, bits, codes, scales)
    for m in (1, 16, 64):
        x = W.draw_x_offset((111, b, m, int(mean) + 100), k, m, mean=mean, sigma=0.5)
        ref = oracle.gemm(p, x)
        for name, dm in both_kernels(V, host).items():
            if name == "declared" and not b:
                continue
            print_case(test="offset_x", mean=mean, b=b, m=m, kernel=name)
            got = run(V, dm, x)
            assert_within_tolerance(got, ref, x, scales, f"mean={mean} b={b} m={m} {name}")
            if m == 1:
                rel = tolerance_report(got, ref, x, scales)[0][0]
                assert rel <= 2e-5, f"mean={mean} b={b} {name}: rel L2 {rel:.2e} (cancellation?)"


def plant_reserved(payload: np.ndarray, b: int, rng, frac: float = 0.05) -> int:
    """Set about frac of the b-bit fields of a one-width payload to the reserved pattern 2^(b-1)
    (two's complement -2^(b-1)); fields never straddle a byte. Returns how many were set."""
    per_byte = 8 // b
    fields = payload.size * per_byte
    pick = np.unique(rng.integers(0, fields, size=max(1, int(frac * fields))))
    byte, slot = pick // per_byte, pick % per_byte
    shift = (slot * b).astype(np.uint8)
    mask = np.left_shift(np.uint8((1 << b) - 1), shift)
    val = np.left_shift(np.uint8(1 << (b - 1)), shift)
    np.bitwise_and.at(payload, byte, ~mask)
    np.bitwise_or.at(payload, byte, val)
    return int(pick.size)


@pytest.mark.parametrize("b", [2, 4, 8])
def test_reserved_pattern_decodes_as_the_oracle(V, b):
    """The packer never writes -2^(b-1), but a payload may hold it: the kernels read it as
    -2^(b-1), exactly as the oracle does (codes bit for bit, products at the parity bar)."""
    import torch
    n, k = 130, 1280
    bits, codes, scales = W.draw_random_matrix((112, b), n, k, {b: 1.0})
    host = V.vbq_pack(n, k, bits, codes, scales)
    p = oracle.pack(n, k, bits, codes, scales)
    assert np.array_equal(host.payload, p.payload)
    planted = plant_reserved(host.payload, b, np.random.default_rng(113 + b))
    p.payload[:] = host.payload
    assert planted > 0
    with pytest.raises(V.VbqError) as err:
        V.vbq_validate_host(host)
    assert err.value.status == V.ERR_CODE
    want = oracle.unpack(p)
    assert int((want == -(1 << (b - 1))).sum()) == planted
    for name, dm in both_kernels(V, host).items():
        print_case(test="reserved", b=b, kernel=name)
        out = torch.empty((n, k), dtype=torch.int8, device="cuda")
        V.vbq_unpack_codes(dm, out)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), want)
        for m in (1, 17, 64):
            x = W.draw_x((114, b, m), k, m)
            assert_within_tolerance(run(V, dm, x), oracle.gemm(p, x), x, scales, f"reserved b={b} m={m} {name}")


@pytest.mark.parametrize("mix", [W.STD_MIX, W.HEAD_MIX, {1: 1.0}, {8: 1.0}])
def test_negative_scales(V, mix):
    """Scales of either sign (binary16 with the sign bit set): every path multiplies by s as it is."""
    n, k = 300, 2048 + 192
    bits, codes, _ = W.draw_random_matrix((115, len(mix)), n, k, mix)
    scales = W.draw_signed_scales((116, len(mix)), n, k // 64)
    assert (scales >> 15).any() and not (scales >> 15).all()
    host = V.vbq_pack(n, k, bits, codes, scales)
    p = oracle.pack(n, k, bits, codes, scales)
    for m in (1, 5, 16, 64):
        x = W.draw_x((117, len(mix), m), k, m)
        ref = oracle.gemm(p, x)
        for name, dm in both_kernels(V, host).items():
            if name == "declared" and len(mix) > 1:
                continue
            print_case(test="negative_scales", mix=len(mix), m=m, kernel=name)
            assert_within_tolerance(run(V, dm, x), ref, x, scales, f"signed scales m={m} {name}")


def spread_modes(bits: np.ndarray) -> set:
    """The rare-width spreads the mixed kernel takes over this matrix's tiles (64 rows x 4 groups): per
    tile, 2-bit groups at 4 lanes (at most 16 in the tile), 2 lanes (at most 32) or 1; 4-bit groups at 4
    lanes (at most 16) or 2."""
    n, G = bits.shape
    modes = set()
    for r0 in range(0, n, 64):
        for j0 in range(0, G, 4):
            t = bits[r0:r0 + 64, j0:j0 + 4]
            c2, c4 = int((t == 2).sum()), int((t == 4).sum())
            if c2:
                modes.add("2bit-quarter" if c2 <= 16 else "2bit-half" if c2 <= 32 else "2bit-one")
            if c4:
                modes.add("4bit-quarter" if c4 <= 16 else "4bit-half")
    return modes


@pytest.mark.parametrize("mix, want", [
    ({1: 0.95, 2: 0.05}, {"2bit-quarter"}),
    ({1: 0.9, 2: 0.1}, {"2bit-quarter", "2bit-half", "2bit-one"}),
    ({1: 0.95, 4: 0.05}, {"4bit-quarter"}),
    ({1: 0.85, 4: 0.1, 2: 0.05}, {"4bit-quarter", "4bit-half", "2bit-quarter"}),
    ({1: 0.97, 2: 0.02, 4: 0.01}, {"2bit-quarter", "4bit-quarter"}),
])
@pytest.mark.parametrize("mean", [0.0, 4.0])
def test_rare_width_spreads(V, mix, want, mean):
    """Tiles whose 2- or 4-bit bucket is small spread each such group over two or four lanes; every
    spread (checked on the host from the widths) against the oracle, on a ragged shape, with plain and
    offset activations."""
    n, k = 300, 4160
    bits, codes, scales = W.draw_random_matrix((120, len(mix), int(100 * min(mix.values()))), n, k, mix)
    assert want <= spread_modes(bits), spread_modes(bits)
    host = V.vbq_pack(n, k, bits, codes, scales)
    p = oracle.pack(n, k, bits, codes, scales)
    x = (W.draw_x_offset((121, int(mean)), k, 1, mean=mean, sigma=0.5) if mean else W.draw_x((121, 0), k))
    print_case(test="rare_spread", mix=sorted(mix.items()), mean=mean)
    got = run(V, V.DeviceMatrix(host), x)
    assert_within_tolerance(got, oracle.gemm(p, x), x, scales, f"spread {sorted(mix.items())} mean={mean}")


def scaled_blocks(bits: np.ndarray, scales: np.ndarray) -> tuple:
    """(scaled, other) counts of 16-row blocks per group column that the matrix-core kernel runs at 17 to 32
    rows of X: a block is scaled (s q folded into its fp16 codes) when every row is 1- or 2-bit with a
    scale that is zero or normal and below 2^15; rows past n do not count."""
    e = (scales >> 10) & 0x1F
    ok = (bits <= 2) & (((e >= 1) & (e <= 29)) | ((scales & 0x7FFF) == 0))
    scaled = sum(int(ok[r:r + 16].all(axis=0).sum()) for r in range(0, bits.shape[0], 16))
    return scaled, (-(-bits.shape[0] // 16)) * bits.shape[1] - scaled


@pytest.mark.parametrize("key, mix", [(1, {1: 1.0}), (2, {2: 1.0}), (3, W.HEAD_MIX), (4, {1: 0.6, 2: 0.3, 4: 0.1})])
def test_gemm_scaled_blocks(V, key, mix):
    """At 17 to 32 rows of X the matrix-core kernel multiplies a block of 1- and 2-bit rows by its scales in
    fp16 before the matrix cores (exact for the scales it admits) and every other block in fp32 after
    them (beyond 32 rows every block is scaled after, which m = 48 and 64 check). Scales here include zeros, subnormals, values of 2^15 and above and negatives, so both kinds of
    block and each reason to fall back occur; rows with a scale of 2^15 or more are checked apart, so their
    size does not loosen the bound on the others."""
    n, k = 200, 1024 + 3 * 64
    G = k // 64
    bits, codes, _ = W.draw_random_matrix((118, key), n, k, mix)
    scales = W.draw_signed_scales((119, key), n, G)
    rng = np.random.default_rng(120 + key)
    sign = rng.integers(0, 2, size=(n, G)).astype(np.uint16) << 15
    pick = rng.random((n, G))
    scales = np.where(pick < 0.01, sign, scales)                                            # +-0
    scales = np.where((pick >= 0.01) & (pick < 0.02), sign | rng.integers(1, 0x400, size=(n, G)), scales)
    big = (pick >= 0.02) & (pick < 0.025)
    scales = np.where(big, sign | rng.integers(0x7800, 0x7C00, size=(n, G)), scales)        # 2^15 .. 65504
    scales = np.where((pick >= 0.025) & (pick < 0.03), sign | rng.integers(0x7400, 0x7800, size=(n, G)), scales)
    scales = scales.astype(np.uint16)
    scaled, other = scaled_blocks(bits, scales)
    assert scaled > 0 and other > 0, (scaled, other)
    host = V.vbq_pack(n, k, bits, codes, scales)
    p = oracle.pack(n, k, bits, codes, scales)
    huge = big.any(axis=1)
    rest = np.flatnonzero(~huge)
    for name, dm in both_kernels(V, host).items():
        if name == "declared" and len(mix) > 1:
            continue
        for m in (17, 32, 48, 64):
            print_case(test="gemm_scaled", mix=key, m=m, kernel=name, scaled=scaled, other=other)
            x = W.draw_x((121, key, m), k, m)
            y, ref = run(V, dm, x), oracle.gemm(p, x)
            assert_within_tolerance(y[:, rest], ref[:, rest], x, scales[rest], f"scaled m={m} {name}")
            if huge.any():
                rows = np.flatnonzero(huge)
                assert_within_tolerance(y[:, rows], ref[:, rows], x, scales[rows], f"scaled, big scales m={m} {name}")


def test_gemm_scaled_blocks_with_reserved_codes(V):
    """A 2-bit payload that holds the reserved pattern (q = -2) next to scales near 2^15: 2 s stays finite
    in fp16 only below 2^15, which is where the kernel stops folding the scale into the codes."""
    import torch  # noqa: F401
    n, k = 130, 1280
    G = k // 64
    bits, codes, _ = W.draw_random_matrix((122, 2), n, k, {2: 1.0})
    rng = np.random.default_rng(123)
    below = ((np.arange(n) // 16) % 2 == 0)[:, None]   # 16-row blocks alternate: below 2^15, then above
    scales = np.where(below, rng.integers(0x7400, 0x7800, size=(n, G)),
                      rng.integers(0x7800, 0x7C00, size=(n, G))).astype(np.uint16)
    scaled, other = scaled_blocks(bits, scales)
    assert scaled > 0 and other > 0, (scaled, other)
    host = V.vbq_pack(n, k, bits, codes, scales)
    p = oracle.pack(n, k, bits, codes, scales)
    assert plant_reserved(host.payload, 2, np.random.default_rng(124)) > 0
    p.payload[:] = host.payload
    for m in (17, 64):
        x = W.draw_x((125, m), k, m)
        for name, dm in both_kernels(V, host).items():
            print_case(test="gemm_scaled_reserved", m=m, kernel=name)
            assert_within_tolerance(run(V, dm, x), oracle.gemm(p, x), x, scales, f"reserved, big scales m={m} {name}")
