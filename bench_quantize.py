"""Throughput of the per-group quantizer (vbq_quantize) on one GPU.

Quantizes every weight matrix of one 9B decoder layer (q, k, v, o 4096x4096,
gate, up 14336x4096, down 4096x14336) with the fixed recipe's projection
widths, plus a 32000x4096 LM head tiered by token frequency, from fp32
weights already in HBM. VBQ paper (arXiv 2607.02893) §3.1 Eq. (1) for the
arithmetic, §3.4 for the recipe (first-block MLP at 4 bits, other
projections at 2, the head at 8/4/2/1 bits by frequency rank).

Algorithmic bytes per weight: 4 (fp32 read) + 1 (int8 code written) + per
64-weight group 1 (width read) + 2 (binary16 scale written), i.e.
5 + 3/64. The kernel streams each byte once, so HBM bandwidth bounds it.
Timing: hipEvents on one stream around --passes passes over all matrices
(1.4 GB of fp32 weights, far beyond the caches). The CPU baseline times the
reference quantizer (numpy) on one 4096x4096 projection. A second leg times
the training-side soft quantizer (§3.2, vbq_soft_quantize) over the seven
layer matrices: 8 + 52/64 algorithmic bytes per weight.

  python bench_quantize.py [--passes 20] [--warmup 3] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import time

import numpy as np

import workloads as W

HBM_PEAK_GBS = 8000.0
BYTES_PER_WEIGHT = 5 + 3 / 64


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--passes", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    return ap.parse_args()


def shapes():
    layer = [(m.name.split(".")[-1], m.n, m.k) for m in W.config(4).matrices]
    return layer + [("head", 32000, 4096)]


def main():
    args = parse()
    import torch
    import decode_gemv_02_amd as V

    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(dev)
    mats = []
    for i, (name, n, k) in enumerate(shapes()):
        w = torch.from_numpy(W.draw_weights((40, i), n, k)).to(dev)
        if name == "head":
            freq = np.minimum(np.random.default_rng(41).zipf(1.3, n), 10 ** 6).astype(np.uint64)
            bits = np.repeat(V.vbq_recipe_head_bits(freq)[:, None], k // 64, axis=1)
        else:
            bits = np.full((n, k // 64), 4 if name in ("gate", "up", "down") else 2, np.uint8)
        b = torch.from_numpy(bits.reshape(-1)).to(dev)
        codes = torch.empty((n, k), dtype=torch.int8, device=dev)
        scales = torch.empty((n, k // 64), dtype=torch.int16, device=dev)
        mats.append((name, n, k, w, b, codes, scales))
    torch.cuda.synchronize()
    weights = sum(n * k for _, n, k, *_ in mats)
    alg_bytes = weights * BYTES_PER_WEIGHT

    def one_pass():
        for _, _, _, w, b, c, s in mats:
            V.vbq_quantize(w, b, c, s, stream)

    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.passes):
        one_pass()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.passes
    gbs = alg_bytes / (ms * 1e-3) / 1e9

    # per matrix: that launch alone, back to back
    per = {}
    for name, n, k, w, b, c, s in mats:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.passes):
            V.vbq_quantize(w, b, c, s, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.passes
        per[name] = {"us": round(us, 2), "GB/s": round(n * k * BYTES_PER_WEIGHT / (us * 1e-6) / 1e9, 1)}

    result = {
        "metric": "quantize_throughput", "value": round(gbs, 1), "unit": "GB/s", "ms_per_pass": round(ms, 4),
        "weights_per_pass": weights, "alg_bytes_per_weight": round(BYTES_PER_WEIGHT, 5),
        "gweights_per_s": round(weights / (ms * 1e-3) / 1e9, 2), "passes": args.passes, "warmup": args.warmup,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "9B decoder layer (q,k,v,o 4096x4096; gate,up 14336x4096; down 4096x14336) at "
                               "the recipe's 2/4 bits + 32000x4096 head tiered 8/4/2/1 by frequency, fp32 "
                               "weights N(0, 0.02) with 0.2% outliers x10-50"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4)},
        "per_matrix": per,
    }
    # training-side soft quantizer (§3.2) over the seven layer matrices: per weight 4 bytes read and 4
    # written, per 64-weight group 16 + 16 bytes of logits and noise read, 16 of pi and 4 of expected
    # bits written: 8 + 52/64 bytes per weight
    soft_bpw = 8 + 52 / 64
    soft = [m for m in mats if m[0] != "head"]
    sbufs = []
    for name, n, k, w, *_ in soft:
        g = n * (k // 64)
        gen = torch.Generator(device=dev).manual_seed(n + k)
        lg = torch.randn(g, 4, device=dev, generator=gen)
        u = torch.rand(g, 4, device=dev, generator=gen).clamp_(1e-7, 1 - 1e-7)
        sbufs.append((w, lg, -torch.log(-torch.log(u)), torch.empty_like(w), torch.empty(g, 4, device=dev),
                      torch.empty(g, device=dev), torch.empty(1, dtype=torch.float64, device=dev)))
    sweights = sum(n * k for _, n, k, *_ in soft)

    def soft_pass():
        for w, lg, gu, ws, pi, gb, mb in sbufs:
            V.vbq_soft_quantize(w, lg, gu, 1.0, ws, pi, gb, mb, stream)

    for _ in range(args.warmup):
        soft_pass()
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.passes):
        soft_pass()
    t1.record(stream)
    torch.cuda.synchronize()
    sms = t0.elapsed_time(t1) / args.passes
    result["soft_quantize"] = {"weights_per_pass": sweights, "alg_bytes_per_weight": round(soft_bpw, 5),
                               "ms_per_pass": round(sms, 4),
                               "GBps": round(sweights * soft_bpw / (sms * 1e-3) / 1e9, 1),
                               "pct_hbm_peak": round(100 * sweights * soft_bpw / (sms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                               "workload": "the seven 9B-layer matrices, tau 1.0, N(0,1) logits, Gumbel noise"}
    del sbufs
    if not args.no_cpu_baseline:
        from oracle import quantize as Q
        n, k = 4096, 4096
        w = W.draw_weights((40, 0), n, k)
        bits = np.full((n, k // 64), 2, np.uint8)
        reps, t_start = 0, time.perf_counter()
        while True:
            Q.quantize(w, bits)
            reps += 1
            dt = time.perf_counter() - t_start
            if dt >= args.cpu_seconds:
                break
        result["cpu_baseline"] = {"value": round(n * k * BYTES_PER_WEIGHT * reps / dt / 1e9, 4), "unit": "GB/s",
                                  "cores": 1, "kind": "oracle",
                                  "sample": f"numpy reference quantizer on one 4096x4096 projection at 2 bits, "
                                            f"{reps} reps in {dt:.1f} s"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    os.environ.setdefault("PYTHONUNBUFFERED", "1")
    main()
