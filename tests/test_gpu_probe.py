"""GPU checks of the measurement kernels: the dense fp16 GEMV baseline computes
y = W x (fp16 products, fp32 sums) and the read probe reads without writing."""
import numpy as np
import pytest

from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def V():
    import torch  # noqa: F401
    import decode_gemv_02_amd as V
    return V


@pytest.mark.parametrize("n,k", [(1, 64), (7, 768), (130, 2048), (300, 5632), (64, 14336), (33, 16384)])
def test_dense_gemv_baseline(V, n, k):
    import torch
    print(f"CASE test=dense_gemv n={n} k={k}", flush=True)
    rng = np.random.default_rng(n * 7 + k)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float16)
    x = rng.standard_normal(k).astype(np.float16)
    y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    V.vbq_probe_dense_gemv(torch.from_numpy(w).cuda(), torch.from_numpy(x).cuda(), y)
    torch.cuda.synchronize()
    ref = w.astype(np.float64) @ x.astype(np.float64)
    got = y.cpu().numpy().astype(np.float64)
    assert np.linalg.norm(got - ref) <= 1e-5 * np.linalg.norm(ref)


def test_stream_read_writes_nothing(V):
    import torch
    print("CASE test=stream_read", flush=True)
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.full((16 * 256,), 7, dtype=torch.int32, device="cuda")
    V.vbq_probe_stream_read(buf, buf.numel(), sink, 16)
    V.vbq_probe_stream_read(buf, 4096 + 16, sink, 16)
    torch.cuda.synchronize()
    assert bool((sink == 7).all())
    with pytest.raises(V.VbqError):
        V.vbq_probe_stream_read(buf, 24, sink, 16)
