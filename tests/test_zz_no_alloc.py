"""The entry point that allocates nothing (vbq_gemv_multi_noalloc) against vbq_gemv_multi.

Both run the same kernels and launch shapes, so the outputs must agree bit for
bit; both are also held to the oracle's parity bar. Two calls in a row, the
second smaller, show that the fixed scratch array (kept between calls) is
reused correctly; the launches split row tiles, so the array's counters and
partial sums are actually used.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.conftest import gpu_available
from tests.helpers import assert_within_tolerance

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def V():
    import torch  # noqa: F401
    import decode_gemv_02_amd as V
    return V


def case(V, seed, shapes):
    import torch
    mats, packs, xs, xts, scales = [], [], [], [], []
    for i, (n, k) in enumerate(shapes):
        b, c, s = W.draw_random_matrix(seed + (i,), n, k, W.STD_MIX)
        mats.append(V.DeviceMatrix(V.vbq_pack(n, k, b, c, s)))
        packs.append(oracle.pack(n, k, b, c, s))
        x = W.draw_x(seed + (100 + i,), k)
        xs.append(x)
        xts.append(torch.from_numpy(x[0].view(np.float16)).cuda())
        scales.append(s)
    return mats, packs, xs, xts, scales


def run(V, fn, mats, xts):
    import torch
    ys = [torch.full((m.n,), float("nan"), dtype=torch.float32, device="cuda") for m in mats]
    fn(mats, xts, ys)
    torch.cuda.synchronize()
    return [y.cpu().numpy() for y in ys]


@pytest.mark.parametrize("first,second", [
    ([(512, 16384), (512, 16384), (512, 16384)], [(200, 4096)]),
    ([(4096, 14336)], [(100, 65536), (64, 768)]),
])
def test_noalloc_matches_gemv_multi(V, first, second):
    print("CASE test=noalloc first=%s second=%s" % (first, second), flush=True)
    for call, shapes in enumerate((first, second)):
        mats, packs, xs, xts, scales = case(V, (80, call, len(shapes)), shapes)
        got = run(V, V.vbq_gemv_multi_noalloc, mats, xts)
        ref = run(V, V.vbq_gemv_multi, mats, xts)
        for i, (n, k) in enumerate(shapes):
            assert np.array_equal(got[i], ref[i]), f"call {call} matrix {i}: differs from vbq_gemv_multi"
            rows = min(n, 256)
            want = oracle.gemv(packs[i], xs[i][0], rows=(0, rows))
            assert_within_tolerance(got[i][:rows], want[:rows], xs[i], scales[i], f"call {call} matrix {i}")
