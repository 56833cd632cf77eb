"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bars (per output vector): relative L2 error <= 1e-3 and max abs error <=
2e-3 * ||x||_2 * max|scale|; decoded codes bit-exact. Inputs are the seeded
synthetic draws of workloads.py; the library packs with its own packer, the
oracle with its own, and the two byte streams are compared too.
"""
import os

import numpy as np
import pytest

import oracle
import workloads as W
from tests.conftest import gpu_available
from tests.helpers import assert_within_tolerance, make_case, xf64

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def V():
    import torch  # noqa: F401
    import decode_gemv_02_amd as V
    return V


@pytest.fixture(scope="module")
def torch_mod():
    import torch
    return torch


def upload(V, bits, codes, scales):
    n, k = codes.shape
    h = V.vbq_pack(n, k, bits, codes, scales)
    return h, V.DeviceMatrix(h)


def gpu_gemm(V, torch, dm, x_bits):
    x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.float16)).cuda()
    m = x.shape[0]
    y = torch.full((m, dm.n), float("nan"), dtype=torch.float32, device="cuda")
    if m == 1:
        V.vbq_gemv(dm, x[0], y[0])
    else:
        V.vbq_gemm_smallbatch(dm, x, y)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def print_case(**kw):
    print("CASE", " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


# ------------------------------------------------------------------ runtime sanity

def test_one_hip_runtime_mapped(V, torch_mod):
    torch_mod.zeros(1, device="cuda")
    maps = open("/proc/self/maps").read().splitlines()
    libs = {line.split()[-1] for line in maps if "libamdhip64" in line}
    assert len(libs) == 1, libs
    assert any(V.LIB_PATH in line for line in maps)


# ------------------------------------------------------------------ decoded codes

@pytest.mark.parametrize("n,k,mix", [(1, 64, W.STD_MIX), (7, 192, W.FIRST_MLP_MIX), (129, 768, W.STD_MIX),
                                     (33, 4160, {1: 0.25, 2: 0.25, 4: 0.25, 8: 0.25}), (5, 128, {8: 1.0}),
                                     (5, 128, {1: 1.0})])
def test_unpack_codes_bit_exact(V, torch_mod, n, k, mix):
    print_case(test="unpack", n=n, k=k)
    bits, codes, scales, p = make_case((n, k, 1), n, k, mix)
    h, dm = upload(V, bits, codes, scales)
    assert h.payload.tobytes() == p.payload.tobytes()
    out = torch_mod.full((n, k), 99, dtype=torch_mod.int8, device="cuda")
    V.vbq_unpack_codes(dm, out)
    torch_mod.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got, oracle.unpack(p))
    assert np.array_equal(got, codes)


# ------------------------------------------------------------------ GEMV / GEMM, small shapes with ragged tails

SHAPES = [(1, 64), (3, 128), (17, 768), (64, 192), (255, 1024), (1000, 448), (130, 4096 + 64), (9, 14336),
          (40, 65536)]


@pytest.mark.parametrize("n,k", SHAPES)
def test_gemv_matches_oracle(V, torch_mod, n, k):
    print_case(test="gemv", n=n, k=k)
    bits, codes, scales, p = make_case((n, k, 2), n, k, W.FIRST_MLP_MIX)
    h, dm = upload(V, bits, codes, scales)
    x = W.draw_x((n, k, 3), k)
    y = gpu_gemm(V, torch_mod, dm, x)
    assert_within_tolerance(y, oracle.gemm(p, x), x, scales, f"gemv {n}x{k}")


# Shapes that take each GEMV launch shape the host picks: 16-wave workgroups
# with no split (12288 x 4096 / 4032), 8-wave with no split (6144 x 1984),
# 16-wave split four ways (4000 x 14272), 8-wave split four ways (3000 x 6400);
# k = 4032, 1984 and 14272 leave the last column tile with three groups.
@pytest.mark.parametrize("n,k", [(12288, 4096), (12288, 4032), (6144, 1984), (4000, 14272), (3000, 6400)])
def test_gemv_launch_shapes(V, torch_mod, n, k):
    print_case(test="gemv_shapes", n=n, k=k)
    bits, codes, scales, p = make_case((n, k, 5), n, k, W.STD_MIX)
    h, dm = upload(V, bits, codes, scales)
    x = W.draw_x((n, k, 6), k)
    y = gpu_gemm(V, torch_mod, dm, x)
    assert_within_tolerance(y, oracle.gemm(p, x), x, scales, f"gemv {n}x{k}")


@pytest.mark.parametrize("m", [2, 3, 4, 5, 8, 15, 16, 17, 31, 48, 63, 64])
def test_gemm_matches_oracle(V, torch_mod, m):
    n, k = 97, 1088
    print_case(test="gemm", n=n, k=k, m=m)
    bits, codes, scales, p = make_case((m, 4), n, k, W.STD_MIX)
    h, dm = upload(V, bits, codes, scales)
    x = W.draw_x((m, 5), k, m)
    assert_within_tolerance(gpu_gemm(V, torch_mod, dm, x), oracle.gemm(p, x), x, scales, f"gemm m={m}")


# The GEMV route of the small-batch call: at m = 2 on calls of at least 2048 tiles its waves take both
# rows of X per decoded tile; otherwise (m = 3, 5, 8; 5632 x 2048 has 704 tiles) one row per wave. Shapes:
# 256 x 8 tiles, 64 x 32 (split row tiles), a ragged 2200 x 15424 (35 x 61 tiles, k % 256 != 0) and
# 8 x 256 tiles (many splits). Each result against the oracle; a second call gives the same bits; the
# y row after the m rows stays untouched.
@pytest.mark.parametrize("n,k,m", [(16384, 2048, 2), (16384, 2048, 3), (4096, 8192, 2), (4096, 8192, 5),
                                   (2200, 15424, 2), (512, 65536, 2), (5632, 2048, 2), (5632, 2048, 8)])
def test_gemv_rows_route(V, torch_mod, n, k, m):
    torch = torch_mod
    print_case(test="gemv_rows", n=n, k=k, m=m)
    bits, codes, scales, p = make_case((n, k, m, 41), n, k, W.STD_MIX)
    h, dm = upload(V, bits, codes, scales)
    x = W.draw_x((n, k, m, 42), k, m)
    xt = torch.from_numpy(np.ascontiguousarray(x).view(np.float16)).cuda()
    y = torch.full((m + 1, n), float("nan"), dtype=torch.float32, device="cuda")
    V.vbq_gemm_smallbatch(dm, xt, y[:m])
    torch.cuda.synchronize()
    first = y.cpu().numpy()
    assert np.isnan(first[m]).all()
    assert_within_tolerance(first[:m].astype(np.float64), oracle.gemm(p, x), x, scales, f"rows {n}x{k} m={m}")
    V.vbq_gemm_smallbatch(dm, xt, y[:m])
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy()[:m], first[:m])


@pytest.mark.parametrize("m", [4, 8, 12, 16])
def test_gemm_both_paths_below_17_rows(V, torch_mod, m):
    # 1280x8192 has 640 tiles: m = 12 and 16 reach the matrix cores (m * m * tiles >= 85000),
    # m = 4 and 8 run on the GEMV route (four rows of X per wave); 97x1088 (10 tiles) stays on it
    for n, k in ((1280, 8192), (97, 1088)):
        print_case(test="gemm_paths", n=n, k=k, m=m)
        bits, codes, scales, p = make_case((m, n, k, 31), n, k, W.STD_MIX)
        h, dm = upload(V, bits, codes, scales)
        x = W.draw_x((m, n, k, 32), k, m)
        assert_within_tolerance(gpu_gemm(V, torch_mod, dm, x), oracle.gemm(p, x), x, scales, f"paths {n}x{k} m={m}")


@pytest.mark.parametrize("b", [1, 2, 4, 8])
def test_single_width_matrices(V, torch_mod, b):
    n, k = 77, 960
    print_case(test="single_width", b=b)
    bits, codes, scales, p = make_case((b, 6), n, k, {b: 1.0})
    h, dm = upload(V, bits, codes, scales)
    for m in (1, 5, 16, 17):
        x = W.draw_x((b, m, 7), k, m)
        assert_within_tolerance(gpu_gemm(V, torch_mod, dm, x), oracle.gemm(p, x), x, scales, f"b={b} m={m}")


def test_one_hot_x_returns_dequantised_column(V, torch_mod):
    # s*q has at most 18 significant bits, so the product with 1.0 and the sum of zeros are exact in fp32
    n, k = 50, 512
    bits, codes, scales, p = make_case(8, n, k, W.FIRST_MLP_MIX)
    h, dm = upload(V, bits, codes, scales)
    wd = codes.astype(np.float64).reshape(n, k // 64, 64) * xf64(scales)[:, :, None]
    for col in (0, 37, 64, 511):
        x = np.zeros((1, k), np.float16)
        x[0, col] = 1.0
        y = gpu_gemm(V, torch_mod, dm, x.view(np.uint16))
        assert np.array_equal(y[0], wd.reshape(n, k)[:, col])


@pytest.mark.parametrize("m", [2, 3, 16, 37, 64])
def test_one_hot_rows_exact(V, torch_mod, m):
    # row i of X is one-hot at column c_i: Y[i] is that column of s*q, exact in fp32
    n, k = 130, 1216
    bits, codes, scales, p = make_case((m, 12), n, k, W.FIRST_MLP_MIX)
    h, dm = upload(V, bits, codes, scales)
    wd = (codes.astype(np.float64).reshape(n, k // 64, 64) * xf64(scales)[:, :, None]).reshape(n, k)
    cols = (np.arange(m) * 97 + 5) % k
    x = np.zeros((m, k), np.float16)
    x[np.arange(m), cols] = 1.0
    print_case(test="one_hot_rows", n=n, k=k, m=m)
    y = gpu_gemm(V, torch_mod, dm, x.view(np.uint16))
    assert np.array_equal(y, wd[:, cols].T)


def test_gemm_split_path_repeats_exactly(V, torch_mod):
    # few row tiles and a long k: each row tile is split across workgroups
    torch = torch_mod
    n, k, m = 100, 32768, 32
    bits, codes, scales, p = make_case(43, n, k, W.STD_MIX)
    h, dm = upload(V, bits, codes, scales)
    x = W.draw_x(44, k, m)
    print_case(test="gemm_split", n=n, k=k, m=m)
    outs = [gpu_gemm(V, torch_mod, dm, x) for _ in range(3)]
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])
    assert_within_tolerance(outs[0], oracle.gemm(p, x), x, scales, "gemm split")


def test_edge_values(V, torch_mod):
    n, k = 60, 640
    bits, codes, scales = W.draw_random_matrix(9, n, k, W.STD_MIX)
    scales = scales.copy()
    scales.reshape(-1)[::7] = 0               # zero scales
    scales.reshape(-1)[3::11] = 0x0001        # smallest subnormal
    scales.reshape(-1)[5::13] = 0x03FF        # largest subnormal
    scales.reshape(-1)[1::17] = 0x7BFF        # largest finite
    p = oracle.pack(n, k, bits, codes, scales)
    h, dm = upload(V, bits, codes, scales)
    x = W.draw_x(10, k)
    xs = x.copy()
    xs.reshape(-1)[::5] = 0x0003              # subnormal x
    xs.reshape(-1)[2::9] = 0
    for xx in (x, xs, np.zeros_like(x)):
        y = gpu_gemm(V, torch_mod, dm, xx)
        ref = oracle.gemm(p, xx)
        if not np.any(ref):
            assert np.all(y == 0)
        else:
            assert_within_tolerance(y, ref, xx, scales, "edge values")


@pytest.mark.parametrize("m", [17, 24, 32, 64])
def test_edge_values_small_batch(V, torch_mod, m):
    # 1- and 2-bit rows, so the matrix-core kernel folds most blocks' scales into the fp16 codes at 17 to
    # 32 rows: zero, subnormal and largest finite scales (the last two keep their blocks on the fp32
    # scaling), with subnormal, zero and all-zero activations
    n, k = 130, 640
    bits, codes, scales = W.draw_random_matrix(11, n, k, {1: 0.5, 2: 0.5})
    scales = scales.copy()
    scales.reshape(-1)[::7] = 0
    scales.reshape(-1)[2::9] = 0x8000         # negative zero
    scales.reshape(-1)[3::97] = 0x0001
    scales.reshape(-1)[5::101] = 0x03FF
    scales.reshape(-1)[1::103] = 0x7BFF
    p = oracle.pack(n, k, bits, codes, scales)
    h, dm = upload(V, bits, codes, scales)
    x = W.draw_x(12, k, m)
    xs = x.copy()
    xs.reshape(-1)[::5] = 0x0003
    xs.reshape(-1)[2::9] = 0
    for xx in (x, xs, np.zeros_like(x)):
        print_case(test="edge_values_small_batch", m=m)
        y = gpu_gemm(V, torch_mod, dm, xx)
        ref = oracle.gemm(p, xx)
        if not np.any(ref):
            assert np.all(y == 0)
        else:
            assert_within_tolerance(y, ref, xx, scales, f"edge values m={m}")


def test_empty_shapes(V, torch_mod):
    torch = torch_mod
    h, dm = upload(V, np.zeros((0, 2), np.uint8), np.zeros((0, 128), np.int8), np.zeros((0, 2), np.uint16))
    y = torch.zeros(4, device="cuda")
    V.vbq_gemv(dm, torch.zeros(128, dtype=torch.float16, device="cuda"), y)
    h, dm = upload(V, np.zeros((5, 0), np.uint8), np.zeros((5, 0), np.int8), np.zeros((5, 0), np.uint16))
    y = torch.full((3, 5), 7.0, device="cuda")
    V.vbq_gemm_smallbatch(dm, torch.zeros((3, 0), dtype=torch.float16, device="cuda"), y)
    torch.cuda.synchronize()
    assert torch.all(y == 0)


def test_deterministic_and_stream_aware(V, torch_mod):
    torch = torch_mod
    n, k = 2048, 4096
    bits, codes, scales, p = make_case(11, n, k, W.STD_MIX)
    h, dm = upload(V, bits, codes, scales)
    x = torch.from_numpy(W.draw_x(12, k)[0].view(np.float16)).cuda()
    y1 = torch.empty(n, device="cuda")
    y2 = torch.empty(n, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        V.vbq_gemv(dm, x, y1)
    V.vbq_gemv(dm, x, y2, stream=s)
    s.synchronize()
    assert torch.equal(y1, y2)
    assert_within_tolerance(y1.cpu().numpy(), oracle.gemv(p, W.draw_x(12, k)), W.draw_x(12, k), scales, "stream")


# ------------------------------------------------------------------ full-size workloads, sampled rows

def sample_ranges(n, width=96):
    """First, middle and last row blocks (the last one covers the ragged tail tile)."""
    mid = max(0, n // 2 - width // 2)
    spans = [(0, min(n, width)), (mid, min(n, mid + width)), (max(0, n - width), n)]
    out = []
    for b, e in sorted(spans):
        if out and b <= out[-1][1]:
            out[-1] = (out[-1][0], max(out[-1][1], e))
        else:
            out.append((b, e))
    return out


def _config_matrices(cid):
    cfg = W.config(cid)
    if cid == 2:       # layer 0 (its own MLP mix) and layer 1 cover every shape and mix
        return cfg, [m for m in cfg.matrices if m.layer in (0, 1)]
    if cid == 3:       # one layer covers every shape; the rest differ only in seeds
        return cfg, [m for m in cfg.matrices if m.layer == 0]
    return cfg, cfg.matrices


@pytest.mark.slow
@pytest.mark.parametrize("cid", W.ALL_CONFIGS)
def test_full_size_workloads(V, torch_mod, cid):
    cfg, mats = _config_matrices(cid)
    for spec in mats:
        bits, codes, scales = W.draw_matrix(spec)
        p = oracle.pack(spec.n, spec.k, bits, codes, scales)
        h, dm = upload(V, bits, codes, scales)
        assert h.payload.tobytes() == p.payload.tobytes()
        ranges = sample_ranges(spec.n)
        rows = np.concatenate([np.arange(b, e) for b, e in ranges])
        for m in cfg.batches:
            print_case(test="full", cfg=cfg.name, mat=spec.name, n=spec.n, k=spec.k, m=m)
            x = W.draw_x(W.x_seed(spec), spec.k, m)
            y = gpu_gemm(V, torch_mod, dm, x)
            ref = np.concatenate([oracle.gemm(p, x, rows=(b, e))[:, b:e] for b, e in ranges], axis=1)
            assert_within_tolerance(y[:, rows], ref, x, scales, f"{cfg.name}/{spec.name} m={m}")
        out = torch_mod.empty((spec.n, spec.k), dtype=torch_mod.int8, device="cuda")
        V.vbq_unpack_codes(dm, out)
        torch_mod.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), codes), f"{cfg.name}/{spec.name} codes"
        del dm, out


def test_gemv_multi_mixed_shapes_one_launch(V, torch_mod):
    torch = torch_mod
    shapes = [(300, 768), (64, 4096), (9, 14336), (130, 320), (1, 64), (700, 1024), (65, 4160)]
    dms, xs, ys, refs = [], [], [], []
    for i, (n, k) in enumerate(shapes):
        bits, codes, scales, p = make_case((i, 31), n, k, W.STD_MIX)
        h, dm = upload(V, bits, codes, scales)
        x = W.draw_x((i, 32), k)
        dms.append(dm)
        xs.append(torch.from_numpy(x[0].view(np.float16)).cuda())
        ys.append(torch.full((n,), float("nan"), device="cuda"))
        refs.append((oracle.gemv(p, x), x, scales))
    print_case(test="gemv_multi", count=len(shapes))
    V.vbq_gemv_multi(dms, xs, ys)
    torch.cuda.synchronize()
    for (n, k), y, (ref, x, scales) in zip(shapes, ys, refs):
        assert_within_tolerance(y.cpu().numpy(), ref, x, scales, f"multi {n}x{k}")
    # the same call again gives identical bits (the split path resets its counters)
    first = [y.clone() for y in ys]
    V.vbq_gemv_multi(dms, xs, ys)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(first, ys))


def test_split_path_repeats_exactly(V, torch_mod):
    # small n and large k split each row tile across several workgroups
    torch = torch_mod
    n, k = 100, 32768
    bits, codes, scales, p = make_case(41, n, k, W.STD_MIX)
    h, dm = upload(V, bits, codes, scales)
    x = W.draw_x(42, k)
    xt = torch.from_numpy(x[0].view(np.float16)).cuda()
    outs = []
    for _ in range(3):
        y = torch.empty(n, device="cuda")
        V.vbq_gemv(dm, xt, y)
        torch.cuda.synchronize()
        outs.append(y.cpu().numpy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])
    assert_within_tolerance(outs[0], oracle.gemv(p, x), x, scales, "split")


# ------------------------------------------------------------------ uniform-width kernels

@pytest.mark.parametrize("b", [1, 2, 4, 8])
@pytest.mark.parametrize("n, k", [(64, 256), (300, 4096 + 64), (1000, 1984), (64, 14336), (4096, 4096)])
def test_uniform_width_kernels(V, torch_mod, b, n, k):
    # a matrix at one width: the uniform-width kernel (declared width) against the oracle, and bit for
    # bit against the mixed-width kernel on the same matrix (same launch shape, same order of sums)
    torch = torch_mod
    print_case(test="uniform", b=b, n=n, k=k)
    bits, codes, scales = W.draw_random_matrix((b, n, k), n, k, {b: 1.0})
    h = V.vbq_pack(n, k, bits, codes, scales)
    assert V.vbq_uniform_width(h) == b
    fast, mixed = V.DeviceMatrix(h), V.DeviceMatrix(h, uniform=False)
    assert fast.uniform_bits == b and mixed.uniform_bits == 0
    x = W.draw_x((b, n, k, 1), k)
    xt = torch.from_numpy(x.view(np.float16)).cuda()
    ys = []
    for dm in (fast, mixed):
        y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
        V.vbq_gemv(dm, xt[0], y)
        torch.cuda.synchronize()
        ys.append(y.cpu().numpy())
    p = oracle.pack(n, k, bits, codes, scales)
    assert_within_tolerance(ys[0][None], oracle.gemv(p, x[0])[None], x, scales, f"uniform b={b}")
    assert np.array_equal(ys[0], ys[1])


def test_uniform_width_multi_and_mixed_batches(V, torch_mod):
    # q/k/v-like launch of three 2-bit matrices (uniform kernel), then a batch that mixes a uniform and
    # a mixed-width matrix (falls back to the mixed kernel for both); also gate+up epilogue at 4 bits
    torch = torch_mod
    print_case(test="uniform_multi")
    n, k = 2048, 2048
    hs, packs, dms = [], [], []
    for i, mix in enumerate([{2: 1.0}, {2: 1.0}, {2: 1.0}, W.STD_MIX]):
        bits, codes, scales = W.draw_random_matrix((70, i), n, k, mix)
        hs.append(V.vbq_pack(n, k, bits, codes, scales))
        packs.append((oracle.pack(n, k, bits, codes, scales), scales))
        dms.append(V.DeviceMatrix(hs[-1]))
    x = W.draw_x((71,), k)
    xt = torch.from_numpy(x.view(np.float16)).cuda()
    for sel in ([0, 1, 2], [0, 3], [3, 1]):
        ys = [torch.full((n,), float("nan"), dtype=torch.float32, device="cuda") for _ in sel]
        V.vbq_gemv_multi([dms[i] for i in sel], [xt[0]] * len(sel), ys)
        torch.cuda.synchronize()
        for i, y in zip(sel, ys):
            assert_within_tolerance(y.cpu().numpy()[None], oracle.gemv(packs[i][0], x[0])[None], x, packs[i][1],
                                    f"batch {sel} matrix {i}")
    gates = []
    for i in range(2):
        bits, codes, scales = W.draw_random_matrix((72, i), 3000, k, {4: 1.0})
        gates.append(V.vbq_pack(3000, k, bits, codes, scales))
    hf = torch.empty(3000, dtype=torch.float16, device="cuda")
    hm = torch.empty(3000, dtype=torch.float16, device="cuda")
    V.vbq_gemv_swiglu(V.DeviceMatrix(gates[0]), V.DeviceMatrix(gates[1]), xt[0], hf)
    V.vbq_gemv_swiglu(V.DeviceMatrix(gates[0], uniform=False), V.DeviceMatrix(gates[1], uniform=False), xt[0], hm)
    torch.cuda.synchronize()
    assert torch.equal(hf, hm)


def test_uniform_width_declaration_is_checked(V):
    n, k = 64, 512
    h = V.vbq_pack(n, k, *W.draw_random_matrix((73,), n, k, {2: 1.0}))
    dm = V.DeviceMatrix(h)
    import ctypes
    import torch
    x = torch.zeros(k, dtype=torch.float16, device="cuda")
    y = torch.zeros(n, dtype=torch.float32, device="cuda")
    bad = V.VbqMatrix.from_buffer_copy(dm.struct)
    bad.uniform_bits = 4                                   # payload_bytes says 2 bits
    assert V.lib.vbq_gemv(ctypes.byref(bad), x.data_ptr(), y.data_ptr(), None) == V.ERR_OFFSETS
    bad.uniform_bits = 3
    assert V.lib.vbq_gemv(ctypes.byref(bad), x.data_ptr(), y.data_ptr(), None) == V.ERR_WIDTH


def test_grouped_recipe_head(V, torch_mod):
    # the frequency-tiered head as four one-width row blocks in one launch (per-matrix widths): logits
    # in rank order, mapped back through the row order, against the oracle on the vocabulary-order matrix
    from oracle import quantize as Q
    torch = torch_mod
    rows, k = 4000, 1024
    print_case(test="grouped_head", rows=rows, k=k)
    freq = np.minimum(np.random.default_rng(80).zipf(1.3, rows), 10 ** 6).astype(np.uint64)
    bits = np.repeat(Q.head_bits(freq)[:, None], k // 64, axis=1)
    w = W.draw_weights((81,), rows, k)
    codes, scales = Q.quantize(w, bits)
    order, blocks = V.vbq_pack_grouped_head(freq, codes, scales)
    dms = [V.DeviceMatrix(b) for b in blocks]
    assert [d.uniform_bits for d in dms] == [8, 4, 2, 1]
    x = W.draw_x((82,), k)
    xt = torch.from_numpy(x.view(np.float16)).cuda()
    ys = [torch.full((d.n,), float("nan"), dtype=torch.float32, device="cuda") for d in dms]
    V.vbq_gemv_multi(dms, [xt[0]] * len(dms), ys)
    torch.cuda.synchronize()
    logits = np.empty(rows)
    logits[order] = np.concatenate([y.cpu().numpy() for y in ys])
    ref = oracle.gemv(oracle.pack(rows, k, bits, codes, scales), x[0])
    assert_within_tolerance(logits[None], ref[None], x, scales, "grouped head")
    # the vocabulary-order matrix on the mixed kernel agrees too, and so does a single block alone
    y = torch.empty(rows, dtype=torch.float32, device="cuda")
    V.vbq_gemv(V.DeviceMatrix(V.vbq_pack(rows, k, bits, codes, scales)), xt[0], y)
    y1 = torch.empty(dms[2].n, dtype=torch.float32, device="cuda")
    V.vbq_gemv(dms[2], xt[0], y1)
    torch.cuda.synchronize()
    assert_within_tolerance(y.cpu().numpy()[None], ref[None], x, scales, "vocabulary order")
    assert np.array_equal(y1.cpu().numpy(), ys[2].cpu().numpy())


@pytest.mark.parametrize("m, k, shapes", [
    (1, 2048, [97, 8192, 300, 64, 1000]),
    (8, 2048, [97, 8192, 300, 64, 1000]),      # 1216 tiles: 64 x 1216 < 85000, GEMV route (two 4-row entries each)
    (12, 2048, [97, 8192, 300, 64, 1000]),     # 144 x 1216 >= 85000: one matrix-core launch for all five
    (20, 2048, [97, 8192, 300, 64, 1000]),
    (20, 1088, [97, 130, 64, 300, 33, 200, 64, 1000, 70, 5]),   # ten matrices: two launches; k % 256 != 0
    (2, 4096, [4096, 4096, 4096]),             # 3072 tiles: both rows of X per GEMV wave
    (3, 4096, [97, 16384, 300]),               # 4208 tiles: one row per GEMV wave
])
def test_gemm_smallbatch_multi_matches_oracle(V, torch_mod, m, k, shapes):
    # matrices sharing the m rows of X, as q/k/v and gate/up do, with ragged row counts: the small-batch
    # rule applies to all of them together, so they share matrix-core launches (up to eight matrices
    # each) or GEMV launches (up to 32 entries of up to four rows each)
    torch = torch_mod
    print_case(test="gemm_multi", m=m, k=k, shapes=shapes)
    x = W.draw_x((90, m), k, m)
    xt = torch.from_numpy(np.ascontiguousarray(x).view(np.float16)).cuda()
    packs, dms, hs = [], [], []
    for i, n in enumerate(shapes):
        bits, codes, scales, p = make_case((91, m, k, i), n, k, W.STD_MIX)
        h, dm = upload(V, bits, codes, scales)
        hs.append(h)
        dms.append(dm)
        packs.append((p, scales))
    ys = [torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda") for n in shapes]
    V.vbq_gemm_smallbatch_multi(dms, xt, ys)
    torch.cuda.synchronize()
    for i, (y, (p, scales)) in enumerate(zip(ys, packs)):
        assert_within_tolerance(y.cpu().numpy(), oracle.gemm(p, x), x, scales, f"multi m={m} matrix {i}")


def test_split_partials_are_never_read_stale(V, torch_mod):
    # Two different matrices of one shape use the same split-K scratch slots. Alternating them many
    # times, every call must give exactly its matrix's own result: a partial sum left in a cache by
    # the other matrix's call would show as a large error. Covers the GEMV split tail, the gated-MLP
    # pair buffer and the GEMM split tail.
    torch = torch_mod
    print_case(test="split_stale")
    n, k = 128, 16384                       # few row tiles, long rows: split row tiles
    mats = [V.DeviceMatrix(V.vbq_pack(n, k, *W.draw_random_matrix((85, i), n, k, W.STD_MIX))) for i in range(2)]
    x = torch.from_numpy(W.draw_x((86,), k, 16).view(np.float16)).cuda()
    first = {}
    for it in range(24):
        i = it % 2
        y = torch.empty(n, dtype=torch.float32, device="cuda")
        V.vbq_gemv(mats[i], x[0], y)
        h = torch.empty(n, dtype=torch.float16, device="cuda")
        V.vbq_gemv_swiglu(mats[i], mats[1 - i], x[0], h)
        yg = torch.empty((16, n), dtype=torch.float32, device="cuda")
        V.vbq_gemm_smallbatch(mats[i], x, yg)
        torch.cuda.synchronize()
        got = (y.cpu().numpy(), h.cpu().numpy(), yg.cpu().numpy())
        if i not in first:
            first[i] = got
        else:
            for a, b in zip(got, first[i]):
                assert np.array_equal(a, b), f"iteration {it}: result changed between calls"
    assert not np.array_equal(first[0][0], first[1][0])


@pytest.mark.parametrize("mix", ["std", "two_bit"])
def test_fp16_outputs_are_the_rounded_fp32_outputs(V, torch_mod, mix):
    # q/k/v-like launch (mixed or uniform kernel) and a split launch (long rows): every fp16 output is
    # exactly the fp32 output of the same launch shape rounded to nearest even
    torch = torch_mod
    print_case(test="fp16_out", mix=mix)
    m = {"std": W.STD_MIX, "two_bit": {2: 1.0}}[mix]
    shapes = [(2048, 2048), (2048, 2048), (2048, 2048), (64, 14336)]
    mats = [V.DeviceMatrix(V.vbq_pack(n, k, *W.draw_random_matrix((88, i), n, k, m))) for i, (n, k) in
            enumerate(shapes)]
    xs = [torch.from_numpy(W.draw_x((89, i), k)[0].view(np.float16)).cuda() for i, (n, k) in enumerate(shapes)]
    for sel in ([0, 1, 2], [3]):
        y32 = [torch.empty(shapes[i][0], dtype=torch.float32, device="cuda") for i in sel]
        y16 = [torch.full((shapes[i][0],), float("nan"), dtype=torch.float16, device="cuda") for i in sel]
        V.vbq_gemv_multi([mats[i] for i in sel], [xs[i] for i in sel], y32)
        V.vbq_gemv_multi_f16([mats[i] for i in sel], [xs[i] for i in sel], y16)
        torch.cuda.synchronize()
        for a, b in zip(y32, y16):
            assert torch.equal(a.half(), b)


def test_multi_launch_of_unequal_matrices(V, torch_mod):
    # one launch over matrices of different row and column counts (the instance whose idle workgroups
    # leave at once), including a split matrix, a ragged one and a one-row one: each against the oracle
    torch = torch_mod
    print_case(test="ragged_multi")
    shapes = [(4096, 1024), (64, 16384), (1000, 1984), (1, 64), (300, 4160)]
    cases = []
    for i, (n, k) in enumerate(shapes):
        bits, codes, scales = W.draw_random_matrix((95, i), n, k, W.STD_MIX)
        cases.append((V.DeviceMatrix(V.vbq_pack(n, k, bits, codes, scales)), oracle.pack(n, k, bits, codes, scales),
                      scales, W.draw_x((96, i), k)))
    for _ in range(2):   # twice: the split matrix's counters must have reset
        ys = [torch.full((n,), float("nan"), dtype=torch.float32, device="cuda") for n, _ in shapes]
        xs = [torch.from_numpy(c[3].view(np.float16)).cuda()[0] for c in cases]
        V.vbq_gemv_multi([c[0] for c in cases], xs, ys)
        torch.cuda.synchronize()
        for (dm, p, scales, x), y in zip(cases, ys):
            assert_within_tolerance(y.cpu().numpy()[None], oracle.gemv(p, x[0])[None], x, scales,
                                    f"{dm.n}x{dm.k} in a launch of unequal matrices")


# Seeded random shapes across every route of the GEMV / small-batch call: n from 1 row to a few thousand,
# k any multiple of 64 (ragged column tiles included), m from 1 to 40 (single-row and two-row GEMVs,
# matrix cores), widths from a random mix per case. Each against the oracle.
def _random_cases(count=24):
    rng = np.random.default_rng(20261204)
    mixes = [W.STD_MIX, W.FIRST_MLP_MIX, W.HEAD_MIX, {1: 0.25, 2: 0.25, 4: 0.25, 8: 0.25}, {8: 0.5, 1: 0.5}]
    cases = []
    while len(cases) < count:
        n = int(rng.integers(1, 4097))
        k = 64 * int(rng.integers(1, 161))
        m = int(rng.choice([1, 1, 2, 2, 3, 5, 8, 16, 17, 40]))
        if n * k * m > 60_000_000:
            continue
        cases.append((len(cases), n, k, m, int(rng.integers(len(mixes)))))
    return cases, mixes


_CASES, _MIXES = _random_cases()


@pytest.mark.parametrize("idx,n,k,m,mix", _CASES)
def test_random_shapes_match_oracle(V, torch_mod, idx, n, k, m, mix):
    print_case(test="random_shapes", idx=idx, n=n, k=k, m=m, mix=mix)
    bits, codes, scales, p = make_case((idx, n, k, 51), n, k, _MIXES[mix])
    h, dm = upload(V, bits, codes, scales)
    x = W.draw_x((idx, n, k, 52), k, m)
    assert_within_tolerance(gpu_gemm(V, torch_mod, dm, x), oracle.gemm(p, x), x, scales, f"random {idx}")
