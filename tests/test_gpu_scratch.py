"""GPU checks of the library's scratch contract under HIP-graph capture.

The split-K launches (large k, small n) keep partial sums and arrival
counters in a per-stream scratch buffer. The library never allocates while
the caller's stream is being captured, and a buffer it has replaced is kept
alive, so a graph captured earlier stays valid after a later call enlarges
the scratch. Results are checked against the CPU oracle at the parity bar.
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


def print_case(**kw):
    print("CASE", " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def split_case(V, seed, n, k):
    import torch
    bits, codes, scales = W.draw_random_matrix(seed, n, k, W.STD_MIX)
    dm = V.DeviceMatrix(V.vbq_pack(n, k, bits, codes, scales))
    x = W.draw_x(seed + (1,), k)
    xt = torch.from_numpy(x[0].view(np.float16)).cuda()
    ref = oracle.gemv(oracle.pack(n, k, bits, codes, scales), x[0])
    return dm, x, xt, ref, scales


def test_capture_refuses_to_allocate_scratch(V):
    """The first split launch on a fresh stream, made inside a graph capture, returns VBQ_ERR_HIP
    instead of allocating; after one eager call on that stream, the same capture works and every
    replay reproduces the eager result."""
    import torch
    print_case(test="capture_refuses_to_allocate", n=128, k=32768)
    dm, x, xt, ref, scales = split_case(V, (70, 0), 128, 32768)
    st = torch.cuda.Stream()
    y = torch.zeros(128, dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with pytest.raises(V.VbqError) as err:
        with torch.cuda.graph(g, stream=st):
            V.vbq_gemv(dm, xt, y, st)
    assert err.value.status == V.ERR_HIP
    assert "captured" in str(err.value)
    torch.cuda.synchronize()
    with torch.cuda.stream(st):
        V.vbq_gemv(dm, xt, y, st)            # eager: the stream's scratch now exists
    torch.cuda.synchronize()
    eager = y.cpu().numpy().copy()
    assert_within_tolerance(eager, ref, x, scales, "eager")
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2, stream=st):
        V.vbq_gemv(dm, xt, y, st)
    for _ in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g2.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy(), eager)


def test_graph_survives_a_larger_scratch(V):
    """Capture a split launch, then enlarge the same stream's scratch with a larger eager call (a
    small-batch GEMM whose split partial sums need several MiB), then replay: the graph still holds
    the superseded buffer, which the library keeps, so each replay matches the eager result and the
    oracle."""
    import torch
    print_case(test="graph_survives_larger_scratch", n=128, k=32768)
    dm, x, xt, ref, scales = split_case(V, (71, 0), 128, 32768)
    st = torch.cuda.Stream()
    y = torch.zeros(128, dtype=torch.float32, device="cuda")
    with torch.cuda.stream(st):
        V.vbq_gemv(dm, xt, y, st)
    torch.cuda.synchronize()
    eager = y.cpu().numpy().copy()
    assert_within_tolerance(eager, ref, x, scales, "eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        V.vbq_gemv(dm, xt, y, st)
    # a larger consumer of the same stream's scratch: m = 64 rows of X over 2048 x 16384
    nb, kb, m = 2048, 16384, 64
    bb, bc, bs = W.draw_random_matrix((71, 1), nb, kb, W.STD_MIX)
    big = V.DeviceMatrix(V.vbq_pack(nb, kb, bb, bc, bs))
    xb = W.draw_x((71, 2), kb, m)
    xbt = torch.from_numpy(xb.view(np.float16)).cuda()
    yb = torch.empty((m, nb), dtype=torch.float32, device="cuda")
    for _ in range(2):
        with torch.cuda.stream(st):
            V.vbq_gemm_smallbatch(big, xbt, yb, st)
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy(), eager)
    pb = oracle.pack(nb, kb, bb, bc, bs)
    got = yb.cpu().numpy().astype(np.float64)
    refb = oracle.gemm(pb, xb, rows=(0, 192))
    assert_within_tolerance(got[:, :192], refb[:, :192], xb, bs, "larger gemm")
