"""Benchmark: packed-weight GB/s of the fused mixed-bit GEMV at batch 1 on one MI355X.

One step = the seven batch-1 GEMVs of one 9B-shaped decoder layer (q, k, v, o
4096x4096; gate, up 14336x4096; down 4096x14336) in decode order, widths drawn
i.i.d. per 64-weight group from {1: .69, 2: .16, 4: .10, 8: .05}. Every step
reads a different copy of the packed layer (copies are rotated so that the
working set is well beyond the 256 MB Infinity Cache), so the weights come from
HBM. Throughput = packed bytes streamed (payload + widths + scales + tile
offsets) per second.

The timed steps are replayed from one HIP graph that holds exactly --steps
steps (the launches a decode loop would capture); the same steps launched one
by one from Python are reported beside them (eager). Also reported: the
dominant launch alone (roofline), each launch alone, a read-only HBM probe of
the same sizes (the achievable ceiling), a dense fp16 GEMV of the same shapes
(ours and torch.mv), the deployed recipe's one-width layers, and the CPU
oracle on the host cores.

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
PROBE_BLOCKS = 2048          # 256 CUs x 8 workgroups of 256 threads


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate-mb", type=float, default=640.0, help="minimum bytes of distinct weight copies")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp16-baseline", action="store_true")
    ap.add_argument("--only-timed", action="store_true",
                    help="only the warmup, the graph-replayed steps and the roofline leg (profiling)")
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


class Timer:
    """Graph and eager timing on one stream (torch's events are recorded on that stream)."""

    def __init__(self, torch, stream, steps, warmup):
        self.torch, self.stream, self.steps, self.warmup = torch, stream, steps, warmup

    def _events(self):
        t = self.torch
        return t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)

    def graph_ms(self, fn, count=None):
        """ms per fn(i): `warmup` eager calls (they also create the stream's scratch), then fn(0..count-1)
        captured into one graph, replayed once untimed and once timed."""
        t = self.torch
        count = count or self.steps
        with t.cuda.stream(self.stream):
            for i in range(self.warmup):
                fn(i)
        t.cuda.synchronize()
        g = t.cuda.CUDAGraph()
        with t.cuda.graph(g, stream=self.stream):
            for i in range(count):
                fn(i)
        # a replay runs on torch's current stream: make it the timed stream
        with t.cuda.stream(self.stream):
            g.replay()
            t.cuda.synchronize()
            a, b = self._events()
            a.record(self.stream)
            g.replay()
            b.record(self.stream)
        t.cuda.synchronize()
        del g
        return a.elapsed_time(b) / count

    def eager_ms(self, fn, count=None):
        """ms per fn(i), launched one by one from Python after `warmup` untimed calls."""
        t = self.torch
        count = count or self.steps
        with t.cuda.stream(self.stream):
            for i in range(self.warmup):
                fn(i)
            t.cuda.synchronize()
            a, b = self._events()
            a.record(self.stream)
            for i in range(count):
                fn(self.warmup + i)
            b.record(self.stream)
        t.cuda.synchronize()
        return a.elapsed_time(b) / count


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
    stream = torch.cuda.Stream(dev)          # default priority
    T = Timer(torch, stream, args.steps, args.warmup)

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

    # decode order with the dependencies of a decoder layer: q,k,v read one input (one launch),
    # o reads the attention output, gate,up read one input (one launch), down reads silu(gate)*up
    groups = [[0, 1, 2], [3], [4, 5], [6]]
    names = ["+".join(specs[j].name.split(".")[-1] for j in g) for g in groups]
    gbytes = [sum(hosts[j][0].total_bytes for j in g) for g in groups]
    # the stream index each matrix carries (built once at upload), read by the kernel in place of the width
    # codes: bytes beyond the packed format, not counted in the metric's bytes
    index_bytes = [sum(dev_layers[0][j].index_bytes for j in g) for g in groups]

    def launch(layer, g):
        V.vbq_gemv_multi([layer[j] for j in g], [xin[j] for j in g], [ys[j] for j in g], stream)

    def step(i):
        layer = dev_layers[i % copies]
        for g in groups:
            launch(layer, g)

    ms_per_step = T.graph_ms(step)
    value = layer_bytes / (ms_per_step * 1e-3) / 1e9
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "layer_9b: q,k,v,o 4096x4096 + gate,up 14336x4096 + down 4096x14336, batch 1, "
                               "widths i.i.d. per 64-group {1:.69,2:.16,4:.10,8:.05}, fp16 scales and x, fp32 y",
                   "packed_bytes_per_step": layer_bytes, "weights_per_step": cfg.weights,
                   "rotated_copies": copies, "launches_per_step": len(groups),
                   "launch_groups": "q+k+v | o | gate+up | down (vbq_gemv_multi)",
                   "stream_index": "built once per matrix at upload (vbq_build_stream_index); the mixed-width "
                                   "kernel reads it instead of the width codes",
                   "index_bytes_per_step": sum(index_bytes),
                   "timing": "the --steps steps captured in one HIP graph, one untimed and one timed replay"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
    }

    # ---- roofline of the dominant launch (most algorithmic bytes): that launch alone, back to back, from a
    # graph on the same stream (a kernel trace of --only-timed records these dispatches last)
    dom = int(np.argmax(gbytes))
    avg_ms = T.graph_ms(lambda i: launch(dev_layers[i % copies], groups[dom]))
    achieved = gbytes[dom] / (avg_ms * 1e-3) / 1e9
    import bench_counters
    traffic = bench_counters.read_traffic(TRAFFIC_SUMMARY)
    result["roofline"] = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(achieved / HBM_PEAK_GBS, 4),
                          "traffic": None if traffic is None else round(traffic[names[dom]]),
                          "kernel": f"gemv_tiles ({names[dom]} launch)", "avg_launch_us": round(avg_ms * 1e3, 3),
                          "algorithmic_bytes_per_launch": gbytes[dom], "index_bytes_per_launch": index_bytes[dom]}
    if args.only_timed:
        print(json.dumps(result))
        return

    # ---- the same steps launched one by one from Python
    eager = T.eager_ms(step)
    result["eager"] = {"ms_per_step": round(eager, 5), "GBps": round(layer_bytes / (eager * 1e-3) / 1e9, 2)}

    # ---- each launch alone, back to back from a graph (isolated launch time, not a partition of the step)
    per = {nm: T.graph_ms(lambda i, g=g: launch(dev_layers[i % copies], g)) for nm, g in zip(names, groups)}
    result["per_launch_graph_us"] = {nm: round(v * 1e3, 3) for nm, v in per.items()}
    result["per_launch_graph_GBps"] = {nm: round(b / (per[nm] * 1e-3) / 1e9, 1) for nm, b in zip(names, gbytes)}

    # ---- achievable ceiling: a read-only HBM stream of the same bytes, same rotation and launch order
    probe_bytes = max(int(args.rotate_mb * 1e6), 2 * layer_bytes)
    probe_buf = torch.empty(probe_bytes // 16 * 16, dtype=torch.uint8, device=dev)
    probe_buf.fill_(1)
    sink = torch.zeros(1 << 22, dtype=torch.int32, device=dev)
    sizes = [b // 16 * 16 for b in gbytes]
    windows = max(1, (probe_buf.numel() - sum(sizes)) // (sum(sizes) + 4096))

    def probe_step(i):
        off = (i % windows) * (sum(sizes) + 4096)
        for b in sizes:
            V.vbq_probe_stream_read(probe_buf[off:], b, sink, PROBE_BLOCKS, stream)
            off += b

    pstep = T.graph_ms(probe_step)
    big = probe_buf.numel() // 2 // 16 * 16
    pbig = T.graph_ms(lambda i: V.vbq_probe_stream_read(probe_buf[(i % 2) * big:], big, sink, PROBE_BLOCKS, stream),
                      count=8)
    pdom = T.graph_ms(lambda i: V.vbq_probe_stream_read(probe_buf[(i % windows) * (sizes[dom] + 4096):], sizes[dom],
                                                        sink, PROBE_BLOCKS, stream))
    step_probe_gbps = sum(sizes) / (pstep * 1e-3) / 1e9
    result["ceiling"] = {
        "kernel": "vbq_probe_stream_read (read-only, 16-byte loads, 2048 x 256 threads)",
        "probe_GBps_large": round(big / (pbig * 1e-3) / 1e9, 1), "probe_large_bytes": big,
        "probe_step_us": round(pstep * 1e3, 3), "probe_step_GBps": round(step_probe_gbps, 1),
        "value_frac_of_probe_step": round(value / step_probe_gbps, 4),
        "value_frac_of_probe_large": round(value / (big / (pbig * 1e-3) / 1e9), 4),
        "probe_dominant_launch_us": round(pdom * 1e3, 3),
        "roofline_frac_of_probe_dominant": round(achieved / (sizes[dom] / (pdom * 1e-3) / 1e9), 4)}
    del probe_buf

    # ---- the same seven GEMVs as a single launch (no decode dependencies) and as seven launches
    one = T.graph_ms(lambda i: V.vbq_gemv_multi(dev_layers[i % copies], xin, ys, stream))
    sep = T.graph_ms(lambda i: [V.vbq_gemv(dev_layers[i % copies][j], xin[j], ys[j], stream)
                                for j in range(len(specs))])
    result["other_launch_shapes"] = {
        "all_seven_one_launch": {"ms_per_step": round(one, 5), "GBps": round(layer_bytes / (one * 1e-3) / 1e9, 2)},
        "seven_launches": {"ms_per_step": round(sep, 5), "GBps": round(layer_bytes / (sep * 1e-3) / 1e9, 2)}}

    # ---- the same step with the gated-MLP epilogue fused: gate+up write h = fp16(silu(g) * u) in their
    # launch and down reads h, so the step's data flow is the decoder layer's own
    gi_gate = [s.name.split(".")[-1] for s in specs].index("gate")
    gi_up, gi_down = gi_gate + 1, gi_gate + 2
    hbuf = torch.empty(specs[gi_gate].n, dtype=torch.float16, device=dev)
    hbuf32 = torch.empty(specs[gi_gate].n, dtype=torch.float32, device=dev)

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

    fused = T.graph_ms(fused_step)
    unfused = T.graph_ms(torch_epilogue_step)
    gu = T.graph_ms(lambda i: V.vbq_gemv_swiglu(dev_layers[i % copies][gi_gate], dev_layers[i % copies][gi_up],
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

        rms = T.graph_ms(rstep)
        rfms = T.graph_ms(rfused)
        recipe[name] = {"packed_bytes_per_step": rbytes, "ms_per_step": round(rms, 5),
                        "GBps": round(rbytes / (rms * 1e-3) / 1e9, 2),
                        "pct_hbm_peak": round(100 * rbytes / (rms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                        "with_fused_mlp_epilogue_ms_per_step": round(rfms, 5)}
        del rlayers
    # the recipe head (32000x4096, rows tiered 8/4/2/1 bits by a Zipf frequency rank): as one-width row
    # blocks in one launch, against the same rows in vocabulary order on the mixed-width kernel
    hrows, hk = 32000, 4096
    freq = np.minimum(np.random.default_rng(95).zipf(1.3, hrows), 10 ** 6).astype(np.uint64)
    order, tiers = V.vbq_recipe_head_tiers(freq)
    full_bits = np.zeros((hrows, hk // 64), np.uint8)
    full_codes = np.zeros((hrows, hk), np.int8)
    full_scales = np.zeros((hrows, hk // 64), np.uint16)
    blocks, start = [], 0
    for t, (b, cnt) in enumerate(zip((8, 4, 2, 1), tiers)):
        cnt = int(cnt)
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
    g_ms = T.graph_ms(lambda i: V.vbq_gemv_multi(grouped[i % hcopies], [hx] * len(blocks), hy, stream))
    hmap = torch.from_numpy(order.astype(np.int32)).to(dev)
    gm_ms = T.graph_ms(lambda i: V.vbq_gemv_head_grouped(grouped[i % hcopies], hx, hmap, hyf, stream))
    v_ms = T.graph_ms(lambda i: V.vbq_gemv(vocab[i % hcopies], hx, hyf, stream))
    recipe["recipe_head_32000x4096"] = {
        "mean_bits": round(float(V.vbq_recipe_head_bits(freq).astype(np.float64).mean()), 4),
        "packed_bytes": hbytes, "grouped_one_launch_us": round(g_ms * 1e3, 3),
        "grouped_GBps": round(hbytes / (g_ms * 1e-3) / 1e9, 2),
        "grouped_vocabulary_order_us": round(gm_ms * 1e3, 3),
        "grouped_vocabulary_order_note": "vbq_gemv_head_grouped: the same launch storing each rank's logit at its "
                                         "vocabulary row",
        "vocabulary_order_us": round(v_ms * 1e3, 3),
        "vocabulary_order_GBps": round(hbytes / (v_ms * 1e-3) / 1e9, 2)}
    del grouped, vocab
    result["deployed_recipe"] = recipe

    # ---- dense fp16 GEMV of the same shapes (the same weights' dense size), rotated copies: our HIP kernel
    # (graph-replayed, like the packed step) and torch.mv (eager: library calls stay out of graphs here)
    if not args.no_fp16_baseline:
        dense_bytes = sum(2 * s.n * s.k for s in specs)
        dcopies = max(2, math.ceil(args.rotate_mb * 1e6 / dense_bytes))
        gen = torch.Generator(device=dev).manual_seed(0)
        dense = [[torch.randn(s.n, s.k, dtype=torch.float16, device=dev, generator=gen) * 0.02 for s in specs]
                 for _ in range(dcopies)]
        outs = [torch.empty(s.n, dtype=torch.float16, device=dev) for s in specs]

        def dstep_ours(i):
            for j in range(len(specs)):
                V.vbq_probe_dense_gemv(dense[i % dcopies][j], xin[j], ys[j], stream)

        def dstep_torch(i):
            for j in range(len(specs)):
                torch.mv(dense[i % dcopies][j], xin[j], out=outs[j])

        ours = T.graph_ms(dstep_ours)
        tms = T.eager_ms(dstep_torch)
        result["fp16_baseline"] = {
            "dense_bytes_per_step": dense_bytes,
            "hip_dense_gemv": {"impl": "vbq_probe_dense_gemv (hand-written, fp16 x fp16 -> fp32), graph-replayed",
                               "ms_per_step": round(ours, 5), "dense_GBps": round(dense_bytes / (ours * 1e-3) / 1e9, 2),
                               "speedup_vbq_over_fp16": round(ours / ms_per_step, 3)},
            "torch_mv": {"impl": "torch.mv (rocBLAS/hipBLASLt), eager", "ms_per_step": round(tms, 5),
                         "dense_GBps": round(dense_bytes / (tms * 1e-3) / 1e9, 2),
                         "speedup_vbq_over_fp16": round(tms / ms_per_step, 3)}}
        del dense

    # ---- CPU oracle on the host cores (bounded sample of the same workload)
    if not args.no_cpu_baseline:
        import oracle
        cores = len(os.sched_getaffinity(0))
        model = "unknown"
        try:
            with open("/proc/cpuinfo") as f:
                model = next(line.split(":", 1)[1].strip() for line in f if line.startswith("model name"))
        except (OSError, StopIteration):
            pass
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
        # one thread: the first 512 rows of the gate projection, repeated for about 3 s
        gs = specs[gi_gate]
        rows1 = 512
        row_bytes = hosts[gi_gate][0].total_bytes * rows1 / gs.n
        reps1 = 0
        t = time.perf_counter()
        while True:
            oracle.gemv_threaded(packs[gi_gate], xh[W.x_seed(gs)], 0, rows1, 1)
            reps1 += 1
            dt1 = time.perf_counter() - t
            if dt1 >= min(3.0, args.cpu_seconds / 4):
                break
        result["cpu_baseline"] = {"value": round(layer_bytes * reps / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
                                  "kind": "oracle", "cpu_model": model,
                                  "sample": f"{reps} passes over all 7 matrices of the layer "
                                            f"({layer_bytes * reps / 1e6:.0f} MB packed), {dt:.1f} s, {cores} threads",
                                  "one_thread_GBps": round(row_bytes * reps1 / dt1 / 1e9, 4),
                                  "one_thread_sample": f"{reps1} passes over the first {rows1} rows of gate "
                                                       f"(14336x4096), {dt1:.1f} s"}
    print(json.dumps(result))


if __name__ == "__main__":
    main()
