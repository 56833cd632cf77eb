"""GPU parity of the frequency-grouped head with vocabulary-order logits,
vbq_gemv_head_grouped (through the C ABI).

The head's rows are tiered by a synthetic Zipf token frequency (VBQ paper,
arXiv 2607.02893, §3.4: 8/4/2/1 bits by frequency rank) and packed as one
one-width row block per tier in rank order (§6, "Fused kernels over packed
weights": the head as frequency-grouped row buckets). One launch stores each
rank's logit at its vocabulary row. Bars:
  (1) bit for bit the unmapped grouped launch (vbq_gemv_multi on the tiers),
      gathered on the host, on one-width tiers (the per-matrix-width kernel)
      and on mixed-width tiers (the mixed kernel, with and without stream
      indexes);
  (2) within the GEMV tolerance of the CPU oracle on the same rows packed in
      vocabulary order;
  (3) rows no rank maps to, and ranks whose map value is at or past y_rows,
      leave y untouched; k = 0 stores zeros at the mapped rows only.
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


def make_head(V, seed, rows, k, mixed=False, index=True):
    """Tier blocks (DeviceMatrix, rank order), the rank -> row map, and the same rows in vocabulary order
    as one oracle pack. mixed: every tier draws its widths per group from the standard mix (no declared
    width: the mixed-width kernel runs, with or without stream indexes)."""
    freq = np.minimum(np.random.default_rng(seed).zipf(1.3, rows), 10 ** 6).astype(np.uint64)
    order, tiers = V.vbq_recipe_head_tiers(freq)
    G = k // 64
    full_bits = np.zeros((rows, G), np.uint8)
    full_codes = np.zeros((rows, k), np.int8)
    full_scales = np.zeros((rows, G), np.uint16)
    blocks, start = [], 0
    for t, (b, cnt) in enumerate(zip((8, 4, 2, 1), tiers)):
        cnt = int(cnt)
        if cnt == 0:
            continue
        bb, bc, bs = W.draw_random_matrix((seed, t), cnt, k, W.STD_MIX if mixed else {b: 1.0})
        r = order[start:start + cnt]
        full_bits[r], full_codes[r], full_scales[r] = bb, bc, bs
        blocks.append(V.DeviceMatrix(V.vbq_pack(cnt, k, bb, bc, bs), stream_index=index))
        start += cnt
    ref_pack = oracle.pack(rows, k, full_bits, full_codes, full_scales) if k else None
    return blocks, order, ref_pack, full_scales


@pytest.mark.parametrize("rows, k, mixed, index", [(4000, 1024, False, True), (32000, 4096, False, True),
                                                   (777, 320, False, True), (3000, 2048, True, True),
                                                   (1500, 448, True, False)])
def test_grouped_head_vocabulary_order(V, rows, k, mixed, index):
    import torch
    print_case(test="head_grouped", rows=rows, k=k, mixed=mixed, index=index)
    blocks, order, ref_pack, scales = make_head(V, 97, rows, k, mixed, index)
    assert all(b.uniform_bits == 0 for b in blocks) if mixed else all(b.uniform_bits for b in blocks)
    x = W.draw_x((97, 1), k)
    xt = torch.from_numpy(x[0].view(np.float16)).cuda()
    row_map = torch.from_numpy(order.astype(np.int32)).cuda()
    y = torch.full((rows + 5,), -7.0, dtype=torch.float32, device="cuda")   # 5 rows no rank maps to
    V.vbq_gemv_head_grouped(blocks, xt, row_map, y)
    tier_y = [torch.empty(b.n, dtype=torch.float32, device="cuda") for b in blocks]
    V.vbq_gemv_multi(blocks, [xt] * len(blocks), tier_y)
    torch.cuda.synchronize()
    yn = y.cpu().numpy()
    ranked = torch.cat(tier_y).cpu().numpy()
    assert np.array_equal(yn[order].view(np.uint32), ranked.view(np.uint32)), "differs from the unmapped launch"
    assert np.all(yn[rows:] == -7.0), "rows no rank maps to were written"
    ref = oracle.gemv_threaded(ref_pack, x[0], 0, rows, 8)
    assert_within_tolerance(yn[:rows].astype(np.float64)[None], ref[None], x, scales, "head")


def test_grouped_head_skips_map_values_past_y(V):
    import torch
    print_case(test="head_grouped_bounds")
    rows, k = 3000, 512
    blocks, order, _, _ = make_head(V, 98, rows, k)
    x = torch.from_numpy(W.draw_x((98, 1), k)[0].view(np.float16)).cuda()
    full = torch.empty(rows, dtype=torch.float32, device="cuda")
    V.vbq_gemv_head_grouped(blocks, x, torch.from_numpy(order.astype(np.int32)).cuda(), full)
    # every third rank points past y; y holds only the first 2500 rows
    bad = order.astype(np.int64).copy()
    bad[::3] = 2500 + 7
    y_rows = 2500
    y = torch.full((y_rows,), 3.5, dtype=torch.float32, device="cuda")
    V.vbq_gemv_head_grouped(blocks, x, torch.from_numpy(bad.astype(np.int32)).cuda(), y)
    torch.cuda.synchronize()
    yn, fn = y.cpu().numpy(), full.cpu().numpy()
    written = bad[(bad < y_rows)]
    assert np.array_equal(yn[written].view(np.uint32), fn[written].view(np.uint32))
    untouched = np.setdiff1d(np.arange(y_rows), written)
    assert np.all(yn[untouched] == 3.5)


def test_grouped_head_k0_and_graph_replay(V):
    import torch
    print_case(test="head_grouped_k0_graph")
    empty = [V.DeviceMatrix(V.vbq_pack(n, 0, np.zeros((n, 0), np.uint8), np.zeros((n, 0), np.int8),
                                       np.zeros((n, 0), np.uint16))) for n in (3, 5)]
    y = torch.full((10,), 2.0, dtype=torch.float32, device="cuda")
    m = torch.tensor([9, 0, 4, 2, 7, 1, 6, 3], dtype=torch.int32, device="cuda")
    V.vbq_gemv_head_grouped(empty, torch.empty(0, dtype=torch.float16, device="cuda"), m, y)
    torch.cuda.synchronize()
    yn = y.cpu().numpy()
    assert np.all(yn[[9, 0, 4, 2, 7, 1, 6, 3]] == 0) and yn[5] == 2.0 and yn[8] == 2.0
    # replays of a captured grouped head give the eager bits each time
    rows, k = 6000, 2048
    blocks, order, _, _ = make_head(V, 99, rows, k)
    x = torch.from_numpy(W.draw_x((99, 1), k)[0].view(np.float16)).cuda()
    rm = torch.from_numpy(order.astype(np.int32)).cuda()
    st = torch.cuda.Stream()
    yg = torch.zeros(rows, dtype=torch.float32, device="cuda")
    with torch.cuda.stream(st):
        V.vbq_gemv_head_grouped(blocks, x, rm, yg, st)
    torch.cuda.synchronize()
    eager = yg.cpu().numpy().copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        V.vbq_gemv_head_grouped(blocks, x, rm, yg, st)
    for _ in range(3):
        yg.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(yg.cpu().numpy().view(np.uint32), eager.view(np.uint32))
