"""GPU parity of the fused gated-MLP front half, vbq_gemv_swiglu (through the
C ABI), against the CPU oracle.

h = fp16(silu(g) * u) with g = gate x, u = up x (VBQ paper, arXiv
2607.02893, §6 "Granularity is deployment-friendly", for the gated form).
Two bars: (1) against the oracle in fp64, within the fp16 rounding of h plus
the GEMV error bound carried through silu(g) * u; (2) against the library's
own unfused GEMVs: the fused g and u are the same fp32 sums, so h is within
one fp16 step of fp16(silu(g) * u) computed from vbq_gemv_multi's outputs.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.conftest import gpu_available
from tests.helpers import MAX_ABS_K, xf64

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def V():
    import torch  # noqa: F401
    import decode_gemv_02_amd as V
    return V


def print_case(**kw):
    print("CASE", " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def half_step(v):
    """Spacing of fp16 values at |v| (subnormal spacing below the normal range)."""
    a = np.maximum(np.abs(v), 2.0 ** -14)
    return 2.0 ** (np.floor(np.log2(a)) - 10)


def setup(V, seed, n, k, mix=None):
    import torch
    mats, packs = [], []
    for i in range(2):
        bits, codes, scales = W.draw_random_matrix((seed, i), n, k, mix or W.STD_MIX)
        mats.append(V.DeviceMatrix(V.vbq_pack(n, k, bits, codes, scales)))
        packs.append((oracle.pack(n, k, bits, codes, scales), scales))
    x = W.draw_x((seed, 9), k)
    xt = torch.from_numpy(x[0].view(np.float16)).cuda()
    return mats, packs, x, xt


def run_fused(V, mats, xt, n):
    import torch
    h = torch.full((n,), float("nan"), dtype=torch.float16, device="cuda")
    V.vbq_gemv_swiglu(mats[0], mats[1], xt, h)
    torch.cuda.synchronize()
    return h.cpu().numpy().astype(np.float64)


def check_against_oracle(h, packs, x, rows):
    g = oracle.gemv_threaded(packs[0][0], x[0], 0, packs[0][0].n, 8)[rows]
    u = oracle.gemv_threaded(packs[1][0], x[0], 0, packs[1][0].n, 8)[rows]
    ref = oracle.swiglu(g, u)
    xn = float(np.linalg.norm(xf64(x)[0]))
    eg = MAX_ABS_K * xn * float(np.abs(packs[0][1].view(np.float16).astype(np.float64)).max())
    eu = MAX_ABS_K * xn * float(np.abs(packs[1][1].view(np.float16).astype(np.float64)).max())
    sig = 1.0 / (1.0 + np.exp(-g))
    dsilu = np.abs(sig * (1 + g * (1 - sig)))          # |d silu / dg| <= 1.1
    bound = half_step(np.maximum(np.abs(ref), np.abs(h[rows]))) / 2 + dsilu * (np.abs(u) + eu) * eg + np.abs(oracle.swiglu(g, np.ones_like(g))) * eu
    err = np.abs(h[rows] - ref)
    worst = int(np.argmax(err - bound))
    assert np.all(err <= bound), f"row {rows[worst]}: |h - ref| = {err[worst]:.3e} > {bound[worst]:.3e}"


def check_against_unfused(V, mats, xt, h, n):
    import torch
    ys = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(2)]
    V.vbq_gemv_multi(mats, [xt, xt], ys)
    torch.cuda.synchronize()
    g, u = (y.cpu().numpy().astype(np.float64) for y in ys)
    ref = oracle.swiglu(g, u)
    assert np.all(np.abs(h - ref) <= half_step(ref)), "fused h differs from the unfused GEMVs by over one fp16 step"


@pytest.mark.parametrize("n, k", [(64, 256), (1000, 448), (5632, 2048), (64, 14336), (130, 65536), (14336, 4096)])
def test_swiglu_parity(V, n, k):
    print_case(test="swiglu", n=n, k=k)
    mats, packs, x, xt = setup(V, 61, n, k)
    h = run_fused(V, mats, xt, n)
    assert np.all(np.isfinite(h))
    rows = np.arange(n) if n <= 6000 else np.unique(np.r_[np.arange(0, n, 37), n - 1])
    check_against_oracle(h, packs, x, rows)
    check_against_unfused(V, mats, xt, h, n)


def test_swiglu_repeats_and_shares_scratch_with_split_gemvs(V):
    # split row tiles (large k, few rows) use the same per-stream scratch: run the fused call, a
    # split GEMV, and the fused call again; counters must have reset and results must repeat bitwise
    import torch
    print_case(test="swiglu_repeat")
    mats, packs, x, xt = setup(V, 62, 128, 16384)
    other, _, _, xo = setup(V, 63, 64, 32768)
    h0 = run_fused(V, mats, xt, 128)
    for _ in range(3):
        y = torch.empty(64, dtype=torch.float32, device="cuda")
        V.vbq_gemv(other[0], xo, y)
        h1 = run_fused(V, mats, xt, 128)
        assert np.array_equal(h0, h1, equal_nan=False)
    check_against_oracle(h0, packs, x, np.arange(128))


def test_swiglu_degenerate(V):
    import torch
    print_case(test="swiglu_degenerate")
    empty = V.DeviceMatrix(V.vbq_pack(3, 0, np.zeros((3, 0), np.uint8), np.zeros((3, 0), np.int8),
                                      np.zeros((3, 0), np.uint16)))
    h = torch.full((3,), float("nan"), dtype=torch.float16, device="cuda")
    V.vbq_gemv_swiglu(empty, empty, torch.empty(0, dtype=torch.float16, device="cuda"), h)
    torch.cuda.synchronize()
    assert np.all(h.cpu().numpy() == 0)
    # a gate row of zeros makes its h exactly zero whatever up holds (silu(0) * u = 0)
    n, k = 70, 512
    gb, gc, gs = W.draw_random_matrix((64, 0), n, k, W.STD_MIX)
    gs = gs.copy()
    gs[5] = 0
    gate = V.DeviceMatrix(V.vbq_pack(n, k, gb, gc, gs))
    up = V.DeviceMatrix(V.vbq_pack(n, k, *W.draw_random_matrix((64, 1), n, k, W.STD_MIX)))
    x = torch.from_numpy(W.draw_x((64, 2), k)[0].view(np.float16)).cuda()
    h = run_fused(V, [gate, up], x, n)
    assert h[5] == 0 and np.count_nonzero(h) > n // 2


def test_swiglu_graph_replay(V):
    import torch
    print_case(test="swiglu_graph")
    n, k = 3000, 4096
    mats, packs, x, xt = setup(V, 65, n, k)
    st = torch.cuda.Stream()
    h = torch.zeros(n, dtype=torch.float16, device="cuda")
    with torch.cuda.stream(st):
        V.vbq_gemv_swiglu(mats[0], mats[1], xt, h, st)    # scratch exists before capture
    torch.cuda.synchronize()
    eager = h.cpu().numpy().copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        V.vbq_gemv_swiglu(mats[0], mats[1], xt, h, st)
    for _ in range(4):
        h.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(h.cpu().numpy(), eager)
    check_against_oracle(eager.astype(np.float64), packs, x, np.arange(0, n, 7))
