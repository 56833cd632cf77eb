"""Throughput of every workload of the packed-weight library on one GPU.

Prints one JSON line per (workload, batch): packed bytes streamed per pass,
microseconds per pass and GB/s of packed bytes (for batch > 1 also TFLOP/s
of useful multiply-adds, 2*m flop per weight). A pass runs every matrix of
the workload once in decode order: per layer the q/k/v GEMVs share one
launch, then o, then gate/up in one launch, then down (vbq_gemv_multi); at
batch > 1 each such group is one vbq_gemm_smallbatch_multi call (matrices on
the matrix cores launch alone, the rest share GEMV launches of up to 32
(matrix, row) products). Weights are uploaded
as enough distinct copies that one round of passes reads at least
--rotate-mb of HBM, so caches do not hold them. Timing: hipEvents on one
stream around passes replayed from a HIP graph (one graph holds one pass per
copy, at most --graph-launches launches), so the figure is the GPU's and not
the Python launch rate; eager_us_per_pass times the same passes launched one
by one from Python (for workloads of small matrices that rate is the bound).
Beside each line, the same pass on dense fp16 weights of the same shapes
(torch F.linear, i.e. rocBLAS/hipBLASLt; random values, timed the same way)
gives fp16_us_per_pass and speedup_vs_fp16.

  python bench_configs.py [--configs 1,2,3,4,5] [--passes 50] [--warmup 10] [--batches 24,32]

--batches replaces each workload's own batch sizes (1 to 64 rows of X).
"""
from __future__ import annotations

import argparse
import json
import math

import numpy as np

import workloads as W

HBM_PEAK_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--configs", default="1,2,3,4,5")
    ap.add_argument("--passes", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rotate-mb", type=float, default=640.0)
    ap.add_argument("--graph-launches", type=int, default=4096)
    ap.add_argument("--no-fp16", action="store_true")
    ap.add_argument("--batches", default="", help="comma-separated batch sizes instead of each workload's own")
    a = ap.parse_args()
    a.batches = tuple(int(m) for m in a.batches.split(",") if m)
    if any(not 1 <= m <= 64 for m in a.batches):
        ap.error("--batches: each batch size must be in 1..64")
    return a


def launch_groups(specs):
    """Indices of the matrices that share one launch, in decode order."""
    groups, cur, key = [], [], None
    for i, s in enumerate(specs):
        k = (s.layer, s.role)
        if k != key and cur:
            groups.append(cur)
            cur = []
        cur.append(i)
        key = k
    if cur:
        groups.append(cur)
    return groups


def graph_time(torch, stream, one_pass, passes_per_graph, passes):
    """Microseconds per pass: passes_per_graph passes captured once, replayed on `stream`."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(passes_per_graph):
            one_pass(i)
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, math.ceil(passes / passes_per_graph))
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(reps):
        g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    del g
    return t0.elapsed_time(t1) * 1e3 / (reps * passes_per_graph)


def main():
    args = parse()
    import torch
    import decode_gemv_02_amd as V

    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(dev)
    for cid in [int(c) for c in args.configs.split(",") if c]:
        cfg = W.config(cid)
        specs = cfg.matrices
        hosts = []
        for s in specs:
            b, c, sc = W.draw_matrix(s)
            hosts.append(V.vbq_pack(s.n, s.k, b, c, sc))
        packed = sum(h.total_bytes for h in hosts)
        copies = max(1, math.ceil(args.rotate_mb * 1e6 / packed))
        layers = [[V.DeviceMatrix(h, dev) for h in hosts] for _ in range(copies)]
        groups = launch_groups(specs)
        for m in args.batches or cfg.batches:
            xs, ys = {}, []
            for s in specs:
                key = (W.x_seed(s), m)
                if key not in xs:
                    xs[key] = torch.from_numpy(np.ascontiguousarray(W.draw_x(W.x_seed(s), s.k, m)).view(np.float16)).to(dev)
                ys.append(torch.empty((m, s.n), dtype=torch.float32, device=dev))
            xin = [xs[(W.x_seed(s), m)] for s in specs]

            def one_pass(i):
                layer = layers[i % copies]
                if m == 1:
                    for g in groups:
                        V.vbq_gemv_multi([layer[j] for j in g], [xin[j][0] for j in g], [ys[j][0] for j in g], stream)
                else:
                    for g in groups:
                        V.vbq_gemm_smallbatch_multi([layer[j] for j in g], xin[g[0]], [ys[j] for j in g], stream)

            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                for i in range(args.warmup):
                    one_pass(i)
                torch.cuda.synchronize()
                t0.record(stream)
                for i in range(args.passes):
                    one_pass(i)
                t1.record(stream)
                torch.cuda.synchronize()
                eager_us = t0.elapsed_time(t1) * 1e3 / args.passes
                # one graph: one pass per copy (the scratch buffers exist already, so nothing allocates)
                # at most one launch per matrix and row
                launches = len(groups) if m == 1 else len(specs) * m
                per_graph = max(1, min(copies, args.graph_launches // launches))
                us = graph_time(torch, stream, one_pass, per_graph, args.passes)
            gbps = packed / (us * 1e-6) / 1e9
            line = {"workload": cfg.name, "batch": m, "matrices": len(specs), "packed_bytes": packed,
                    "weights": cfg.weights, "us_per_pass": round(us, 3), "GBps": round(gbps, 2),
                    "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2), "eager_us_per_pass": round(eager_us, 3),
                    "rotated_copies": copies, "passes_per_graph": per_graph,
                    "calls_per_pass": len(groups),
                    "entry": "vbq_gemv_multi" if m == 1 else "vbq_gemm_smallbatch_multi"}
            if m > 1:
                line["TFLOPs"] = round(2.0 * m * cfg.weights / (us * 1e-6) / 1e12, 2)
            if not args.no_fp16:
                dense_bytes = 2 * cfg.weights
                dcopies = max(1, math.ceil(args.rotate_mb * 1e6 / dense_bytes))
                dense = [[(torch.randn(s.n, s.k, device=dev) * 0.02).half() for s in specs] for _ in range(dcopies)]
                xd = [xi.view(m, -1) for xi in xin]
                yd = [torch.empty((m, s.n), dtype=torch.float16, device=dev) for s in specs]

                def dense_pass(i):
                    d = dense[i % dcopies]
                    for j in range(len(specs)):
                        torch.nn.functional.linear(xd[j], d[j], out=yd[j])

                with torch.cuda.stream(stream):
                    for i in range(args.warmup):
                        dense_pass(i)
                    torch.cuda.synchronize()
                    fp16_us = graph_time(torch, stream, dense_pass, max(1, min(dcopies, args.graph_launches // len(specs))),
                                         args.passes)
                line["fp16_us_per_pass"] = round(fp16_us, 3)
                line["fp16_dense_GBps"] = round(dense_bytes / (fp16_us * 1e-6) / 1e9, 2)
                line["speedup_vs_fp16"] = round(fp16_us / us, 3)
                del dense
            print(json.dumps(line), flush=True)
        del layers


if __name__ == "__main__":
    main()
