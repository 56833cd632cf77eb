"""Benchmark: packed-weight GB/s of the fused mixed-bit GEMV at batch 1 on one MI355X.

One step = the seven batch-1 GEMVs of one 9B-shaped decoder layer (q, k, v, o
4096x4096; gate, up 14336x4096; down 4096x14336) in decode order, widths drawn
i.i.d. per 64-weight group from {1: .69, 2: .16, 4: .10, 8: .05}. Every step
reads a different copy of the packed layer (copies are rotated so that the
working set is well beyond the 256 MB Infinity Cache), so the weights come from
HBM. Throughput = packed bytes streamed (payload + widths + scales + row
offsets) per second.

Workload shapes: VBQ paper (arXiv 2607.02893) §6, Figure 5 (decode at 131M,
1.0B and 9B). Synthetic weights and activations (workloads.py).

Prints one JSON line. `--gpus N` with N > 1 exits: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "packed-weight GB/s and % HBM peak for fused mixed-bit GEMV, batch 1"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate-mb", type=float, default=640.0, help="minimum bytes of distinct weight copies")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp16-baseline", action="store_true")
    ap.add_argument("--only-timed", action="store_true", help="skip every leg except the timed loop and the roofline leg (profiling)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only copy 256 MiB device to device once (counter calibration run)")
    return ap.parse_args()


COPY_BYTES = 256 << 20
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemv_tiles_layer9b_traffic.txt")


def calibrate_copy():
    import torch
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda:0")
    a.fill_(3)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copied_bytes": COPY_BYTES}))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this path runs on a single GPU; --gpus must be 1 (multi-GPU sharding is design-only)",
              file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return

    import torch

    import decode_gemv_02_amd as V
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = W.config(4)

    # ---- pack once on the host, upload rotated copies
    hosts, specs = [], cfg.matrices
    for spec in specs:
        bits, codes, scales = W.draw_matrix(spec)
        hosts.append((V.vbq_pack(spec.n, spec.k, bits, codes, scales), bits, codes, scales))
    layer_bytes = sum(h.total_bytes for h, *_ in hosts)
    copies = max(2, math.ceil(args.rotate_mb * 1e6 / layer_bytes))
    dev_layers = [[V.DeviceMatrix(h, dev) for h, *_ in hosts] for _ in range(copies)]
    xs = {}
    for spec in specs:
        key = W.x_seed(spec)
        if key not in xs:
            xs[key] = torch.from_numpy(W.draw_x(key, spec.k)[0].view(np.float16)).to(dev)
    ys = [torch.empty(spec.n, dtype=torch.float32, device=dev) for spec in specs]
    xin = [xs[W.x_seed(spec)] for spec in specs]
    stream = torch.cuda.current_stream(dev)

    # decode order with the dependencies of a decoder layer: q,k,v read one input (one launch),
    # o reads the attention output, gate,up read one input (one launch), down reads silu(gate)*up
    groups = [[0, 1, 2], [3], [4, 5], [6]]

    def step(i):
        layer = dev_layers[i % copies]
        for g in groups:
            V.vbq_gemv_multi([layer[j] for j in g], [xin[j] for j in g], [ys[j] for j in g], stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    value = layer_bytes / (ms_per_step * 1e-3) / 1e9

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "layer_9b: q,k,v,o 4096x4096 + gate,up 14336x4096 + down 4096x14336, batch 1, "
                               "widths i.i.d. per 64-group {1:.69,2:.16,4:.10,8:.05}, fp16 scales and x, fp32 y",
                   "packed_bytes_per_step": layer_bytes, "weights_per_step": cfg.weights,
                   "rotated_copies": copies, "launches_per_step": len(groups),
                   "launch_groups": "q+k+v | o | gate+up | down (vbq_gemv_multi)"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
    }
    # ---- roofline of the dominant launch (most algorithmic bytes): that launch alone, back to back on
    # its stream, timed with one event pair (a kernel trace of --only-timed records these dispatches last)
    gbytes = [sum(hosts[j][0].total_bytes for j in g) for g in groups]
    names = ["+".join(specs[j].name.split(".")[-1] for j in g) for g in groups]
    dom = int(np.argmax(gbytes))
    g = groups[dom]
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        layer = dev_layers[i % copies]
        V.vbq_gemv_multi([layer[j] for j in g], [xin[j] for j in g], [ys[j] for j in g], stream)
    t1.record(stream)
    torch.cuda.synchronize()
    avg_ms = t0.elapsed_time(t1) / args.steps
    achieved = gbytes[dom] / (avg_ms * 1e-3) / 1e9
    import bench_counters
    traffic = bench_counters.read_traffic(TRAFFIC_SUMMARY)
    result["roofline"] = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(achieved / HBM_PEAK_GBS, 4),
                          "traffic": None if traffic is None else round(traffic[names[dom]]),
                          "kernel": f"gemv_tiles ({names[dom]} launch)", "avg_launch_us": round(avg_ms * 1e3, 3),
                          "algorithmic_bytes_per_launch": gbytes[dom]}
    if args.only_timed:
        print(json.dumps(result))
        return

    # ---- per-launch durations (events around each launch on the launch stream)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in groups]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        layer = dev_layers[i % copies]
        for gi, g in enumerate(groups):
            a, b = ev[i][gi]
            a.record(stream)
            V.vbq_gemv_multi([layer[j] for j in g], [xin[j] for j in g], [ys[j] for j in g], stream)
            b.record(stream)
    torch.cuda.synchronize()
    per = np.array([[a.elapsed_time(b) for a, b in row] for row in ev])        # ms [steps, groups]
    result["per_launch_us"] = {nm: round(float(np.mean(per[:, gi])) * 1e3, 3) for gi, nm in enumerate(names)}
    ksum = float(per.mean(axis=0).sum())
    result["launch_time_sum"] = {"us": round(ksum * 1e3, 3), "GBps": round(layer_bytes / (ksum * 1e-3) / 1e9, 2)}

    # ---- the same seven GEMVs as a single launch (no decode dependencies) and as seven launches
    def timed(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(args.steps):
            fn(args.warmup + i)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / args.steps

    one = timed(lambda i: V.vbq_gemv_multi(dev_layers[i % copies], xin, ys, stream))
    sep = timed(lambda i: [V.vbq_gemv(dev_layers[i % copies][j], xin[j], ys[j], stream) for j in range(len(specs))])
    result["other_launch_shapes"] = {
        "all_seven_one_launch": {"ms_per_step": round(one, 5), "GBps": round(layer_bytes / (one * 1e-3) / 1e9, 2)},
        "seven_launches": {"ms_per_step": round(sep, 5), "GBps": round(layer_bytes / (sep * 1e-3) / 1e9, 2)}}

    # ---- the same step with the gated-MLP epilogue fused: gate+up write h = fp16(silu(g) * u) in their
    # launch and down reads h, so the step's data flow is the decoder layer's own
    gi_gate = [s.name.split(".")[-1] for s in specs].index("gate")
    gi_up, gi_down = gi_gate + 1, gi_gate + 2
    hbuf = torch.empty(specs[gi_gate].n, dtype=torch.float16, device=dev)

    def fused_step(i):
        layer = dev_layers[i % copies]
        V.vbq_gemv_multi(layer[0:3], xin[0:3], ys[0:3], stream)
        V.vbq_gemv(layer[3], xin[3], ys[3], stream)
        V.vbq_gemv_swiglu(layer[gi_gate], layer[gi_up], xin[gi_gate], hbuf, stream)
        V.vbq_gemv(layer[gi_down], hbuf, ys[gi_down], stream)

    def torch_epilogue_step(i):
        layer = dev_layers[i % copies]
        V.vbq_gemv_multi(layer[0:3], xin[0:3], ys[0:3], stream)
        V.vbq_gemv(layer[3], xin[3], ys[3], stream)
        V.vbq_gemv_multi([layer[gi_gate], layer[gi_up]], [xin[gi_gate]] * 2, [ys[gi_gate], ys[gi_up]], stream)
        torch.mul(torch.nn.functional.silu(ys[gi_gate]), ys[gi_up], out=hbuf32)
        hbuf.copy_(hbuf32)
        V.vbq_gemv(layer[gi_down], hbuf, ys[gi_down], stream)

    hbuf32 = torch.empty(specs[gi_gate].n, dtype=torch.float32, device=dev)
    fused = timed(fused_step)
    unfused = timed(torch_epilogue_step)
    gu = timed(lambda i: V.vbq_gemv_swiglu(dev_layers[i % copies][gi_gate], dev_layers[i % copies][gi_up],
                                           xin[gi_gate], hbuf, stream))
    result["fused_mlp_step"] = {
        "launches": "q+k+v | o | gate+up -> h = fp16(silu(g)*u) (vbq_gemv_swiglu) | down(h)",
        "ms_per_step": round(fused, 5), "GBps": round(layer_bytes / (fused * 1e-3) / 1e9, 2),
        "gate_up_swiglu_alone_us": round(gu * 1e3, 3),
        "with_torch_epilogue_ms_per_step": round(unfused, 5)}

    # ---- the deployed recipe (one width per projection): a block past the first stores every projection
    # at 2 bits, the first block its MLP at 4; each matrix declares its width, so the uniform-width kernels
    # run. Same shapes, launches and rotation as the timed step.
    recipe = {}
    for name, widths in (("recipe_2bit_block", {}), ("recipe_first_block", {"gate": 4, "up": 4, "down": 4})):
        rhosts = []
        for i, spec in enumerate(specs):
            b = widths.get(spec.name.split(".")[-1], 2)
            rb, rc, rs = W.draw_random_matrix((90, i, b), spec.n, spec.k, {b: 1.0})
            rhosts.append(V.vbq_pack(spec.n, spec.k, rb, rc, rs))
        rbytes = sum(h.total_bytes for h in rhosts)
        rcopies = max(2, math.ceil(args.rotate_mb * 1e6 / rbytes))
        rlayers = [[V.DeviceMatrix(h, dev) for h in rhosts] for _ in range(rcopies)]
        assert all(m.uniform_bits for m in rlayers[0])

        def rstep(i, rl=rlayers, rc_=rcopies):
            layer = rl[i % rc_]
            for g in groups:
                V.vbq_gemv_multi([layer[j] for j in g], [xin[j] for j in g], [ys[j] for j in g], stream)

        def rfused(i, rl=rlayers, rc_=rcopies):
            layer = rl[i % rc_]
            V.vbq_gemv_multi(layer[0:3], xin[0:3], ys[0:3], stream)
            V.vbq_gemv(layer[3], xin[3], ys[3], stream)
            V.vbq_gemv_swiglu(layer[gi_gate], layer[gi_up], xin[gi_gate], hbuf, stream)
            V.vbq_gemv(layer[gi_down], hbuf, ys[gi_down], stream)

        rms = timed(rstep)
        rfms = timed(rfused)
        recipe[name] = {"packed_bytes_per_step": rbytes, "ms_per_step": round(rms, 5),
                        "GBps": round(rbytes / (rms * 1e-3) / 1e9, 2),
                        "pct_hbm_peak": round(100 * rbytes / (rms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                        "with_fused_mlp_epilogue_ms_per_step": round(rfms, 5)}
        del rlayers
    # the recipe head (32000x4096, rows tiered 8/4/2/1 bits by a Zipf frequency rank): as four one-width
    # row blocks in one launch, against the same rows in vocabulary order on the mixed-width kernel
    hrows, hk = 32000, 4096
    freq = np.minimum(np.random.default_rng(95).zipf(1.3, hrows), 10 ** 6).astype(np.uint64)
    order = V.vbq_recipe_head_order(freq)
    tier = V.vbq_recipe_head_bits(freq)[order]
    full_bits = np.zeros((hrows, hk // 64), np.uint8)
    full_codes = np.zeros((hrows, hk), np.int8)
    full_scales = np.zeros((hrows, hk // 64), np.uint16)
    blocks, start = [], 0
    for t, b in enumerate((8, 4, 2, 1)):
        cnt = int((tier == b).sum())
        bb, bc, bs = W.draw_random_matrix((95, t), cnt, hk, {b: 1.0})
        rows_t = order[start:start + cnt]
        full_bits[rows_t], full_codes[rows_t], full_scales[rows_t] = bb, bc, bs
        blocks.append(V.vbq_pack(cnt, hk, bb, bc, bs))
        start += cnt
    full = V.vbq_pack(hrows, hk, full_bits, full_codes, full_scales)
    hbytes = full.total_bytes
    hcopies = max(2, math.ceil(args.rotate_mb * 1e6 / hbytes))
    grouped = [[V.DeviceMatrix(b, dev) for b in blocks] for _ in range(hcopies)]
    vocab = [V.DeviceMatrix(full, dev) for _ in range(hcopies)]
    hx = torch.from_numpy(W.draw_x((96,), hk)[0].view(np.float16)).to(dev)
    hy = [torch.empty(b.n, dtype=torch.float32, device=dev) for b in blocks]
    hyf = torch.empty(hrows, dtype=torch.float32, device=dev)
    g_ms = timed(lambda i: V.vbq_gemv_multi(grouped[i % hcopies], [hx] * len(blocks), hy, stream))
    # the same blocks with the largest (1-bit) first: its workgroups are dispatched first
    gr_ms = timed(lambda i: V.vbq_gemv_multi(grouped[i % hcopies][::-1], [hx] * len(blocks), hy[::-1], stream))
    v_ms = timed(lambda i: V.vbq_gemv(vocab[i % hcopies], hx, hyf, stream))
    # the same four blocks without declared widths: the mixed-width kernel, one launch of unequal matrices
    gmixed = [[V.DeviceMatrix(b, dev, uniform=False) for b in blocks] for _ in range(hcopies)]
    gm_ms = timed(lambda i: V.vbq_gemv_multi(gmixed[i % hcopies], [hx] * len(blocks), hy, stream))
    del gmixed
    recipe["recipe_head_32000x4096"] = {
        "mean_bits": round(float(V.vbq_recipe_head_bits(freq).astype(np.float64).mean()), 4),
        "packed_bytes": hbytes, "grouped_one_launch_us": round(g_ms * 1e3, 3),
        "grouped_GBps": round(hbytes / (g_ms * 1e-3) / 1e9, 2),
        "grouped_largest_first_us": round(gr_ms * 1e3, 3), "grouped_mixed_kernel_us": round(gm_ms * 1e3, 3),
        "vocabulary_order_us": round(v_ms * 1e3, 3),
        "vocabulary_order_GBps": round(hbytes / (v_ms * 1e-3) / 1e9, 2)}
    del grouped, vocab
    result["deployed_recipe"] = recipe

    # ---- dense fp16 GEMV of the same shapes (torch matmul on the same stream, rotated copies)
    if not args.no_fp16_baseline:
        dense_bytes = sum(2 * s.n * s.k for s in specs)
        dcopies = max(2, math.ceil(args.rotate_mb * 1e6 / dense_bytes))
        gen = torch.Generator(device=dev).manual_seed(0)
        dense = [[torch.randn(s.n, s.k, dtype=torch.float16, device=dev, generator=gen) * 0.02 for s in specs]
                 for _ in range(dcopies)]
        outs = [torch.empty(s.n, dtype=torch.float16, device=dev) for s in specs]

        def dstep(i):
            for j in range(len(specs)):
                torch.mv(dense[i % dcopies][j], xin[j], out=outs[j])

        for i in range(args.warmup):
            dstep(i)
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(args.steps):
            dstep(i)
        t1.record(stream)
        torch.cuda.synchronize()
        dms = t0.elapsed_time(t1) / args.steps
        result["fp16_baseline"] = {"impl": "torch.mv (rocBLAS/hipBLASLt) on dense fp16 W of the same shapes",
                                   "ms_per_step": round(dms, 5), "dense_bytes_per_step": dense_bytes,
                                   "dense_GBps": round(dense_bytes / (dms * 1e-3) / 1e9, 2),
                                   "speedup_vbq_over_fp16": round(dms / ms_per_step, 3)}
        del dense

    # ---- CPU oracle on the host cores (bounded sample of the same workload)
    if not args.no_cpu_baseline:
        import oracle
        cores = len(os.sched_getaffinity(0))
        packs = [oracle.pack(s.n, s.k, b, c, sc) for s, (h, b, c, sc) in zip(specs, hosts)]
        xh = {key: W.draw_x(key, specs[[W.x_seed(s) for s in specs].index(key)].k)[0] for key in
              {W.x_seed(s) for s in specs}}
        # whole-layer passes repeated until about cpu_seconds of host time have been spent
        reps = 0
        t = time.perf_counter()
        while True:
            for s, p in zip(specs, packs):
                oracle.gemv_threaded(p, xh[W.x_seed(s)], 0, s.n, cores)
            reps += 1
            dt = time.perf_counter() - t
            if dt >= args.cpu_seconds or reps >= 200:
                break
        result["cpu_baseline"] = {"value": round(layer_bytes * reps / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
                                  "kind": "oracle",
                                  "sample": f"{reps} passes over all 7 matrices of the layer "
                                            f"({layer_bytes * reps / 1e6:.0f} MB packed), {dt:.1f} s, {cores} threads"}
    print(json.dumps(result))


if __name__ == "__main__":
    main()
