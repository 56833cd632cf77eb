"""The stream index (vbq_build_stream_index) on the GPU.

Its bytes are checked against the layout the packed format defines (the
payload's bucket order, derived here from the widths alone); and every GEMV
entry point gives the same bits with and without it, since the indexed
kernel reads the counts and list the scanning kernel derives.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.conftest import gpu_available
from tests.helpers import assert_within_tolerance, make_case

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


def expected_index(bits: np.ndarray, n: int, k: int) -> bytes:
    """Per tile: its groups in payload order (width buckets 1, 2, 4, 8, column-major inside a bucket) as
    (j - j0) * 64 + (r - r0), zero-padded to 256 bytes; then per tile the counts per width as uint16."""
    G = k // 64
    code = {1: 0, 2: 1, 4: 2, 8: 3}
    lists, counts = [], []
    for r0 in range(0, n, 64):
        for j0 in range(0, G, 4):
            R, C = min(64, n - r0), min(4, G - j0)
            entries, cnt = [], [0, 0, 0, 0]
            for c in range(4):
                for jl in range(C):
                    for r in range(R):
                        if code[int(bits[r0 + r, j0 + jl])] == c:
                            entries.append(jl * 64 + r)
                            cnt[c] += 1
            lists.append(bytes(entries) + bytes(256 - len(entries)))
            counts.append(np.array(cnt, np.uint16).tobytes())
    return b"".join(lists) + b"".join(counts)


@pytest.mark.parametrize("n,k,mix", [(1, 64, W.STD_MIX), (64, 256, W.STD_MIX), (130, 960, W.FIRST_MLP_MIX),
                                     (77, 320, {1: 0.25, 2: 0.25, 4: 0.25, 8: 0.25}), (200, 1088, W.HEAD_MIX),
                                     (3, 4096, {8: 1.0}), (500, 2048, W.STD_MIX)])
def test_stream_index_bytes_follow_the_layout(V, torch_mod, n, k, mix):
    print("CASE index", n, k, flush=True)
    bits, codes, scales, p = make_case((n, k, 61), n, k, mix)
    dm = V.DeviceMatrix(V.vbq_pack(n, k, bits, codes, scales), uniform=False)
    torch_mod.cuda.synchronize()
    got = dm._index.cpu().numpy().tobytes()
    assert len(got) == V.vbq_stream_index_bytes(n, k)
    assert got == expected_index(bits, n, k)


# Launch shapes of the mixed kernel: q+k+v-like (16 waves), split row tiles (long rows), ragged
# matrices in one launch, k % 256 != 0.
@pytest.mark.parametrize("shapes", [[(2048, 2048)] * 3, [(64, 14336)], [(4000, 14272)],
                                    [(97, 1088), (300, 4096), (5, 64), (1000, 1984)]])
def test_indexed_and_scanning_kernels_agree_bitwise(V, torch_mod, shapes):
    torch = torch_mod
    print("CASE agree", shapes, flush=True)
    hosts, packs, xs = [], [], []
    for i, (n, k) in enumerate(shapes):
        bits, codes, scales, p = make_case((n, k, i, 62), n, k, W.STD_MIX)
        hosts.append(V.vbq_pack(n, k, bits, codes, scales))
        packs.append((p, scales))
        xs.append(W.draw_x((n, k, i, 63), k))
    with_index = [V.DeviceMatrix(h, uniform=False) for h in hosts]
    without = [V.DeviceMatrix(h, uniform=False, stream_index=False) for h in hosts]
    assert all(d.index_bytes > 0 for d in with_index) and all(d.index_bytes == 0 for d in without)
    xt = [torch.from_numpy(x[0].view(np.float16)).cuda() for x in xs]

    def run(mats, fn):
        ys = [torch.full((n,), float("nan"), dtype=torch.float32, device="cuda") for n, _ in shapes]
        fn(mats, xt, ys)
        torch.cuda.synchronize()
        return [y.cpu().numpy() for y in ys]

    for fn in (V.vbq_gemv_multi, V.vbq_gemv_multi_noalloc):
        a, b = run(with_index, fn), run(without, fn)
        for i, (ya, yb) in enumerate(zip(a, b)):
            assert np.array_equal(ya, yb), f"{fn.__name__} matrix {i}"
            p, scales = packs[i]
            assert_within_tolerance(ya[None].astype(np.float64), oracle.gemm(p, xs[i]), xs[i], scales, "indexed")
    # fp16 outputs and the gated-MLP epilogue (two equal shapes)
    n, k = shapes[0]
    y16 = [torch.empty(n, dtype=torch.float16, device="cuda") for _ in range(2)]
    V.vbq_gemv_multi_f16([with_index[0]], [xt[0]], [y16[0]])
    V.vbq_gemv_multi_f16([without[0]], [xt[0]], [y16[1]])
    torch.cuda.synchronize()
    assert torch.equal(y16[0], y16[1])
    if len(shapes) > 1 and shapes[1] == shapes[0]:
        h = [torch.empty(n, dtype=torch.float16, device="cuda") for _ in range(2)]
        V.vbq_gemv_swiglu(with_index[0], with_index[1], xt[0], h[0])
        V.vbq_gemv_swiglu(without[0], without[1], xt[0], h[1])
        torch.cuda.synchronize()
        assert torch.equal(h[0], h[1])


def test_mixed_launch_of_indexed_and_plain_matrices(V, torch_mod):
    # a launch takes the indexed kernel only when every matrix has an index; otherwise all scan
    torch = torch_mod
    n, k = 300, 2048
    hs = [V.vbq_pack(n, k, *W.draw_random_matrix((64, i), n, k, W.STD_MIX)) for i in range(2)]
    mats = [V.DeviceMatrix(hs[0]), V.DeviceMatrix(hs[1], stream_index=False)]
    x = torch.from_numpy(W.draw_x((65,), k)[0].view(np.float16)).cuda()
    ys = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(2)]
    V.vbq_gemv_multi(mats, [x, x], ys)
    ref = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(2)]
    V.vbq_gemv_multi([V.DeviceMatrix(h) for h in hs], [x, x], ref)
    torch.cuda.synchronize()
    for a, b in zip(ys, ref):
        assert torch.equal(a, b)
