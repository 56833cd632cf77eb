"""Per-launch summaries of rocprofv3 runs of bench.py's timed loop.

Writes the short text summaries kept under profiles/ and reads the traffic
summary back for bench.py. Launches are told apart by dispatch order: every
step of bench.py issues the same launches in the same order (LAUNCHES), and
after the steps bench.py runs its dominant launch alone, back to back, once
per step (the roofline leg).

Kernel durations (`trace`):
  rocprofv3 --kernel-trace --stats -f csv -d <dir> -o kt -- python bench.py --steps 50 --warmup 10 --only-timed
  python bench_counters.py trace --csv <dir>/kt_kernel_trace.csv --out profiles/gemv_tiles_layer9b_kernel_trace.txt

Kernel durations by kernel name (`kernels`), for any run, e.g. the LM head:
  rocprofv3 --kernel-trace --stats -f csv -d <dir> -o kt5 -- python bench_configs.py --configs 5 --no-fp16
  python bench_counters.py kernels --csv <dir>/kt5_kernel_trace.csv --title "..." --command "..." --out <file>
or the quantizer:
  rocprofv3 --kernel-trace --stats -f csv -d <dir> -o qt -- python bench_quantize.py --passes 20 --warmup 3 --no-cpu-baseline

HBM traffic (`traffic`), one rocprofv3 run per counter:
  rocprofv3 --pmc FETCH_SIZE -d <dir> -o fetch -- python bench.py --steps 5 --warmup 2 --only-timed
  rocprofv3 --pmc WRITE_SIZE -d <dir> -o write -- python bench.py --steps 5 --warmup 2 --only-timed
  rocprofv3 --pmc FETCH_SIZE -d <dir> -o cfetch -- python bench.py --calibrate-copy
  rocprofv3 --pmc WRITE_SIZE -d <dir> -o cwrite -- python bench.py --calibrate-copy
  python bench_counters.py traffic --fetch F.db --write W.db --copy-fetch CF.db --copy-write CW.db \
      --copy-bytes 268435456 --out profiles/gemv_tiles_layer9b_traffic.txt

FETCH_SIZE and WRITE_SIZE are KiB per dispatch as the counters define them.
Each is scaled by the ratio (bytes the copy kernel moved) / (what the same
counter reads for that copy), so the reported figure is in true bytes. Both
summaries record a hash of the kernel source; bench.py reports the traffic
only while that hash still matches.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import sqlite3
import statistics

ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCE = os.path.join(ROOT, "decode_gemv_02_amd", "csrc", "vbq_device.hip")
QUANTIZE_SOURCE = os.path.join(ROOT, "decode_gemv_02_amd", "csrc", "vbq_quantize.hip")
LAUNCHES = ["q+k+v", "o", "gate+up", "down"]     # bench.py's launch order within a step
GEMV_KERNEL = "gemv_tiles"
COPY_KERNEL = "copyBuffer"


def kernel_source_sha(path: str = KERNEL_SOURCE) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _by_launch(vals: list, warmup: int, steps: int, what: str) -> tuple[dict, list]:
    """Timed step dispatches per launch name, and the dominant launch's timed back-to-back dispatches.

    bench.py --only-timed dispatches, in order: `warmup` eager steps, the graph of `steps` steps replayed
    twice (untimed, then timed), then the dominant launch alone: `warmup` eager launches and its graph of
    `steps` launches replayed twice. The timed replays are the ones kept."""
    nl = len(LAUNCHES)
    n_step = nl * (warmup + 2 * steps)
    if len(vals) != n_step + warmup + 2 * steps:
        raise SystemExit(f"{what}: {len(vals)} GEMV dispatches, expected {n_step} in the steps and "
                         f"{warmup + 2 * steps} after")
    timed = vals[n_step - nl * steps:n_step]
    return {nm: timed[i::nl] for i, nm in enumerate(LAUNCHES)}, vals[len(vals) - steps:]


def _counter_rows(db: str, counter: str):
    con = sqlite3.connect(db)
    try:
        return con.execute("select dispatch_id, kernel_name, value from counters_collection "
                           "where counter_name = ? order by dispatch_id", (counter,)).fetchall()
    finally:
        con.close()


def _copy_reading(db: str, counter: str) -> float:
    """Counter value (KiB) of the largest copy-kernel dispatch (the calibration copy)."""
    vals = [v for _, name, v in _counter_rows(db, counter) if COPY_KERNEL in name]
    if not vals:
        raise SystemExit(f"{db}: no copy kernel dispatch")
    return max(vals)


def traffic_summary(a) -> str:
    cf, cw = _copy_reading(a.copy_fetch, "FETCH_SIZE"), _copy_reading(a.copy_write, "WRITE_SIZE")
    fscale, wscale = a.copy_bytes / (cf * 1024.0), a.copy_bytes / (cw * 1024.0)
    fetch, _ = _by_launch([v for _, nm, v in _counter_rows(a.fetch, "FETCH_SIZE") if GEMV_KERNEL in nm],
                          a.warmup, a.steps, a.fetch)
    write, _ = _by_launch([v for _, nm, v in _counter_rows(a.write, "WRITE_SIZE") if GEMV_KERNEL in nm],
                          a.warmup, a.steps, a.write)
    lines = [
        "# HBM traffic per launch of gemv_tiles, layer_9b decode step (q+k+v | o | gate+up | down), batch 1",
        "# commands (repository root, one rocprofv3 run each):",
        "#   rocprofv3 --pmc FETCH_SIZE -d <dir> -o fetch -- python bench.py --steps 5 --warmup 2 --only-timed",
        "#   rocprofv3 --pmc WRITE_SIZE -d <dir> -o write -- python bench.py --steps 5 --warmup 2 --only-timed",
        "#   rocprofv3 --pmc FETCH_SIZE -d <dir> -o cfetch -- python bench.py --calibrate-copy",
        "#   rocprofv3 --pmc WRITE_SIZE -d <dir> -o cwrite -- python bench.py --calibrate-copy",
        "#   python bench_counters.py traffic --fetch ... --write ... --copy-fetch ... --copy-write ... "
        f"--copy-bytes {a.copy_bytes} --out <this file>",
        f"kernel_source_sha256: {kernel_source_sha()}",
        f"copy_calibration: bytes={a.copy_bytes} fetch_kib={cf:.2f} write_kib={cw:.2f} "
        f"fetch_scale={fscale:.4f} write_scale={wscale:.4f}",
    ]
    for nm in LAUNCHES:
        fk, wk = statistics.fmean(fetch[nm]), statistics.fmean(write[nm])
        tb = fk * 1024 * fscale + wk * 1024 * wscale
        lines.append(f"launch {nm}: dispatches={len(fetch[nm])} fetch_kib={fk:.2f} write_kib={wk:.2f} "
                     f"traffic_bytes={tb:.0f}")
    return "\n".join(lines) + "\n"


def trace_summary(a) -> str:
    with open(a.csv, newline="") as f:
        rows = [r for r in csv.DictReader(f) if GEMV_KERNEL in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]    # us
    per, b2b = _by_launch(dur, a.warmup, a.steps, a.csv)
    first = {nm: rows[i] for i, nm in enumerate(LAUNCHES)}   # each launch's first dispatch: its kernel and shape
    last = rows[-1]
    dom = [nm for nm in LAUNCHES if (first[nm]["Kernel_Name"], first[nm]["Grid_Size_X"], first[nm]["Grid_Size_Y"])
           == (last["Kernel_Name"], last["Grid_Size_X"], last["Grid_Size_Y"])]
    lines = [
        "# Kernel durations per launch of gemv_tiles, layer_9b decode step (q+k+v | o | gate+up | down), batch 1",
        "# command (repository root):",
        "#   rocprofv3 --kernel-trace --stats -f csv -d <dir> -o kt -- python bench.py --steps 50 --warmup 10 "
        "--only-timed",
        "#   python bench_counters.py trace --csv <dir>/kt_kernel_trace.csv --out <this file>",
        f"kernel_source_sha256: {kernel_source_sha()}",
        f"all launches: dispatches={len(dur)} avg_us={statistics.fmean(dur):.3f}",
    ]
    for nm in LAUNCHES:
        v, r = per[nm], first[nm]
        lines.append(f"launch {nm}: dispatches={len(v)} avg_us={statistics.fmean(v):.3f} "
                     f"median_us={statistics.median(v):.3f} min_us={min(v):.3f} max_us={max(v):.3f}")
        lines.append(f"  kernel: {r['Kernel_Name']} workgroup={r['Workgroup_Size_X']} "
                     f"grid={r['Grid_Size_X']}x{r['Grid_Size_Y']} vgpr={r['VGPR_Count']} sgpr={r['SGPR_Count']} "
                     f"lds={r['LDS_Block_Size']} scratch={r['Scratch_Size']}")
    tot = sum(statistics.fmean(per[nm]) for nm in LAUNCHES)
    lines.append(f"step: sum_of_launch_avg_us={tot:.3f}")
    lines.append(f"roofline leg ({'+'.join(dom) or '?'} alone, back to back): dispatches={len(b2b)} "
                 f"avg_us={statistics.fmean(b2b):.3f} median_us={statistics.median(b2b):.3f} "
                 f"min_us={min(b2b):.3f} max_us={max(b2b):.3f}")
    return "\n".join(lines) + "\n"


def kernels_summary(a) -> str:
    """Dispatch count and duration statistics per kernel name and grid (VBQ kernels only).

    For the quantizer every grid is one matrix shape: a workgroup of 256 lanes covers 64 groups of
    64 weights (16 in the one-group-a-team instance), and each weight costs 5 + 3/64 algorithmic bytes (fp32 read, int8 code written, one
    width byte read and one binary16 scale written per group), which gives alg_GBps. The soft
    quantizer runs 16 lanes a group and moves 8 + 52/64 bytes a weight (fp32 read and written; per
    group 32 bytes of logits and noise read, 16 of pi and 4 of expected bits written)."""
    per, meta = {}, {}
    with open(a.csv) as f:
        for row in csv.DictReader(f):
            name = row["Kernel_Name"]
            if not any(k in name for k in ("gemv_tiles", "gemv_uniform", "gemm_frag", "unpack_tiles",
                                           "quantize_groups", "chunk_sums", "mean_of_parts")):
                continue
            key = (name, row["Grid_Size_X"], row["Grid_Size_Y"])
            per.setdefault(key, []).append((int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1000.0)
            meta.setdefault(key, row)
    lines = [f"# Kernel durations by kernel and grid, {a.title}", "# command (repository root):", f"#   {a.command}",
             f"#   python bench_counters.py kernels --csv <dir>/<name>_kernel_trace.csv --out <this file>",
             f"kernel_source_sha256: {kernel_source_sha()}",
             f"quantize_source_sha256: {kernel_source_sha(QUANTIZE_SOURCE)}"]
    for key, d in per.items():
        name, r = key[0], meta[key]
        lines.append(f"kernel: {name} vgpr={r['VGPR_Count']} sgpr={r['SGPR_Count']} lds={r['LDS_Block_Size']} "
                     f"scratch={r['Scratch_Size']} grid={r['Grid_Size_X']}x{r['Grid_Size_Y']}")
        extra = ""
        if "soft_quantize_groups" in name:   # 16 lanes a group: weights = lanes * 4; 8 + 52/64 bytes a weight
            weights = int(r["Grid_Size_X"]) * 4
            extra = f" weights={weights} alg_GBps={weights * (8 + 52 / 64) / (statistics.fmean(d) * 1e3):.1f}"
        elif "quantize_groups" in name:   # 16 groups a workgroup with one group a team, else 64
            weights = int(r["Grid_Size_X"]) // 256 * (16 if "quantize_groups<1u>" in name else 64) * 64
            extra = f" weights={weights} alg_GBps={weights * (5 + 3 / 64) / (statistics.fmean(d) * 1e3):.1f}"
        lines.append(f"  dispatches={len(d)} avg_us={statistics.fmean(d):.3f} median_us={statistics.median(d):.3f} "
                     f"min_us={min(d):.3f} max_us={max(d):.3f}{extra}")
    return "\n".join(lines) + "\n"


# instruction and occupancy counters per launch (one rocprofv3 --pmc pass per line of PMC_PASSES)
PMC_PASSES = [
    "SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_LDS SQ_INSTS_SMEM SQ_INSTS_VMEM_RD SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES",
    "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_SCA SQ_ACTIVE_INST_VMEM SQ_LDS_BANK_CONFLICT "
    "SQ_LDS_IDX_ACTIVE SQ_WAIT_INST_ANY SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE",   # GRBM_GUI_ACTIVE tells the dispatches apart
]
CU_NUM = 256


def _launch_signatures(con) -> list:
    """GEMV dispatches as (dispatch_id, launch name): a launch is told apart by its kernel, workgroup
    and grid (its first appearance follows LAUNCHES' order; the roofline leg repeats gate+up's)."""
    rows = con.execute("select distinct dispatch_id, kernel_name, workgroup_size, grid_size_x, grid_size_y "
                       "from counters_collection order by dispatch_id").fetchall()
    names, out = {}, []
    for did, kn, wg, gx, gy in rows:
        if GEMV_KERNEL not in kn:
            continue
        sig = (kn, wg, gx, gy)
        if sig not in names:
            if len(names) >= len(LAUNCHES):
                raise SystemExit(f"more than {len(LAUNCHES)} distinct GEMV launches")
            names[sig] = LAUNCHES[len(names)]
        out.append((did, names[sig]))
    return out


def counters_summary(a) -> str:
    """Per launch and per wave (one wave = one 64x256 tile in these launches): instructions by kind,
    LDS bank-conflict share, VALU busy share of the CUs' cycles, mean wave lifetime."""
    totals = {nm: {} for nm in LAUNCHES}
    gui = {nm: [] for nm in LAUNCHES}
    dispatches = {}
    for db in a.db:
        con = sqlite3.connect(db)
        try:
            which = dict(_launch_signatures(con))
            for nm in LAUNCHES:
                dispatches.setdefault(nm, sum(1 for v in which.values() if v == nm))
            for did, cn, val in con.execute("select dispatch_id, counter_name, value from counters_collection "
                                            "order by dispatch_id"):
                nm = which.get(did)
                if nm is None:
                    continue
                if cn == "GRBM_GUI_ACTIVE":
                    gui[nm].append((did, val))
                    continue
                totals[nm][cn] = totals[nm].get(cn, 0.0) + val
        finally:
            con.close()
    lines = ["# Instruction and occupancy counters per launch of gemv_tiles, layer_9b decode step "
             "(q+k+v | o | gate+up | down), batch 1",
             "# commands (repository root; one rocprofv3 run per counter set):"]
    for i, pas in enumerate(PMC_PASSES):
        lines.append(f"#   rocprofv3 --pmc {pas} -d <dir> -o pmc{i} -- python bench.py --steps 5 --warmup 2 "
                     f"--only-timed --no-cpu-baseline")
    lines.append("#   python bench_counters.py counters --db <dir>/pmc0_results.db <dir>/pmc1_results.db --out <this file>")
    lines.append("# per wave: instructions issued by one wave (one tile); valu_us_per_simd: SQ_ACTIVE_INST_VALU "
                 f"(quad-cycles) x 4 / {4 * CU_NUM} SIMDs at 2.4 GHz, the mean time a SIMD issues this launch's "
                 "VALU work (compare with its kernel-trace duration); lds_conflict: SQ_LDS_BANK_CONFLICT / "
                 "(SQ_LDS_IDX_ACTIVE - SQ_LDS_BANK_CONFLICT); cycles are per wave")
    if a.title:
        lines.append(f"# {a.title}")
    lines.append(f"kernel_source_sha256: {a.kernel_sha or kernel_source_sha()}")
    for nm in LAUNCHES:
        t = totals[nm]
        waves = t.get("SQ_WAVES", 0.0)
        if not waves:
            continue
        per = {k.replace("SQ_", "").lower(): v / waves for k, v in sorted(t.items()) if k != "SQ_WAVES"}
        parts = [f"waves_per_dispatch={waves / dispatches[nm]:.0f}"]   # SQ_WAVES is in one counter set
        parts += [f"{k}={v:.1f}" for k, v in per.items() if k.startswith("insts_")]
        if "SQ_LDS_IDX_ACTIVE" in t and "SQ_LDS_BANK_CONFLICT" in t:
            c = t["SQ_LDS_BANK_CONFLICT"]
            parts.append(f"lds_conflict={c / max(1.0, t['SQ_LDS_IDX_ACTIVE'] - c):.3f}")
        if "SQ_ACTIVE_INST_VALU" in t and gui[nm]:
            cycles = 4 * t["SQ_ACTIVE_INST_VALU"] / (4 * CU_NUM) / len(set(d for d, _ in gui[nm]))
            parts.append(f"valu_us_per_simd={cycles / 2400.0:.2f}")
        if "SQ_WAVE_CYCLES" in t:
            parts.append(f"wave_lifetime_cycles={4 * t['SQ_WAVE_CYCLES'] / waves:.0f}")
        if "SQ_WAIT_INST_ANY" in t:
            parts.append(f"wait_inst_any_cycles={4 * t['SQ_WAIT_INST_ANY'] / waves:.0f}")
        lines.append(f"launch {nm}: " + " ".join(parts))
    return "\n".join(lines) + "\n"


PROBE_KERNEL = "stream_read"


def probe_summary(a) -> str:
    """The read-only stream probe of a full bench.py run, by dispatch order: the step-shaped probe (four
    launches of the step's launch sizes per step: `warmup` eager steps, then its graph of `steps` steps
    replayed twice), the large read (`warmup` eager launches, a graph of 8 replayed twice) and the probe
    of the dominant launch's size (`warmup` eager, a graph of `steps` replayed twice). Timed replays only."""
    with open(a.csv, newline="") as f:
        rows = [r for r in csv.DictReader(f) if PROBE_KERNEL in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]
    w, k, nl = a.warmup, a.steps, len(LAUNCHES)
    n_step = nl * (w + 2 * k)
    n_big = w + 2 * 8
    n_dom = w + 2 * k
    if len(dur) != n_step + n_big + n_dom:
        raise SystemExit(f"{a.csv}: {len(dur)} probe dispatches, expected {n_step + n_big + n_dom}")
    step = dur[n_step - nl * k:n_step]
    big = dur[n_step + n_big - 8:n_step + n_big]
    dom = dur[len(dur) - k:]
    lines = ["# Read-only HBM stream probe (vbq_probe_stream_read, 2048 x 256 threads, 16-byte loads), the "
             "ceiling of the layer_9b decode step's launches",
             "# command (repository root):",
             f"#   rocprofv3 --kernel-trace --stats -f csv -d <dir> -o kp -- python bench.py --steps {k} "
             f"--warmup {w} --no-cpu-baseline",
             "#   python bench_counters.py probe --csv <dir>/kp_kernel_trace.csv --out <this file>"]
    for i, nm in enumerate(LAUNCHES):
        v = step[i::nl]
        lines.append(f"probe of the {nm} launch's bytes: dispatches={len(v)} avg_us={statistics.fmean(v):.3f} "
                     f"min_us={min(v):.3f} max_us={max(v):.3f}")
    lines.append(f"probe step (four launches): sum_of_avg_us={sum(statistics.fmean(step[i::nl]) for i in range(nl)):.3f}")
    lines.append(f"large read: dispatches={len(big)} avg_us={statistics.fmean(big):.3f}")
    lines.append(f"dominant launch's bytes alone, back to back: dispatches={len(dom)} avg_us={statistics.fmean(dom):.3f}")
    return "\n".join(lines) + "\n"


# counters of the matrix-core GEMM (one rocprofv3 --pmc pass: eight SQ counters and the GPU's busy cycles)
GEMM_PMC = ("SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_VMEM_RD SQ_INSTS_SALU SQ_WAVES "
            "SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU GRBM_GUI_ACTIVE")
SIMD_NUM = 4 * CU_NUM


def kernel_counters_summary(a) -> str:
    """Per kernel and grid of the VBQ kernels in one --pmc pass: instructions by kind per wave, and the
    mean time a SIMD spends per dispatch issuing VALU work (SQ_ACTIVE_INST_VALU quad-cycles x 4) and
    with its matrix core busy (SQ_VALU_MFMA_BUSY_CYCLES), over all SIMDs at 2.4 GHz (compare with the
    kernel-trace duration)."""
    con = sqlite3.connect(a.db)
    try:
        rows = con.execute("select dispatch_id, kernel_name, grid_size_x, grid_size_y, counter_name, value "
                           "from counters_collection order by dispatch_id").fetchall()
    finally:
        con.close()
    per, disp = {}, {}
    for did, kn, gx, gy, cn, val in rows:
        if not any(k in kn for k in ("gemv_tiles", "gemv_uniform", "gemv_rows", "gemm_frag")):
            continue
        key = (kn, gx, gy)
        per.setdefault(key, {})
        per[key][cn] = per[key].get(cn, 0.0) + val
        disp.setdefault(key, set()).add(did)
    lines = [f"# Instruction counters per kernel and grid, {a.title}",
             "# commands (repository root):",
             f"#   rocprofv3 --pmc {GEMM_PMC} -d <dir> -o {a.name} -- {a.command}",
             f"#   python bench_counters.py kcounters --db <dir>/{a.name}_results.db --out <this file>",
             "# per wave: instructions issued by one wave; valu_us_per_simd / mfma_busy_us_per_simd: per "
             f"dispatch, summed over the {SIMD_NUM} SIMDs and divided by them, at 2.4 GHz",
             f"kernel_source_sha256: {kernel_source_sha()}"]
    for key, t in per.items():
        waves = t.get("SQ_WAVES", 0.0)
        if not waves:
            continue
        nd = len(disp[key])
        parts = [f"dispatches={nd}", f"waves_per_dispatch={waves / nd:.0f}"]
        parts += [f"{k.replace('SQ_', '').lower()}={v / waves:.1f}" for k, v in sorted(t.items())
                  if k.startswith("SQ_INSTS_")]
        parts.append(f"valu_us_per_simd={4 * t.get('SQ_ACTIVE_INST_VALU', 0.0) / SIMD_NUM / nd / 2400.0:.2f}")
        parts.append(f"mfma_busy_us_per_simd={t.get('SQ_VALU_MFMA_BUSY_CYCLES', 0.0) / SIMD_NUM / nd / 2400.0:.2f}")
        lines.append(f"kernel: {key[0]} grid={key[1]}x{key[2]}")
        lines.append("  " + " ".join(parts))
    return "\n".join(lines) + "\n"


def read_traffic(path: str) -> dict | None:
    """{launch: traffic bytes} from a traffic summary, or None if absent or taken on another kernel source."""
    if not os.path.exists(path):
        return None
    sha, out = None, {}
    with open(path) as f:
        for line in f:
            if line.startswith("kernel_source_sha256:"):
                sha = line.split(":", 1)[1].strip()
            elif line.startswith("launch "):
                name, rest = line[len("launch "):].split(":", 1)
                fields = dict(kv.split("=") for kv in rest.split())
                out[name] = float(fields["traffic_bytes"])
    if sha != kernel_source_sha():
        return None
    return out


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--steps", type=int, default=5)
    t.add_argument("--warmup", type=int, default=2)
    t.add_argument("--out", required=True)
    k = sub.add_parser("trace")
    k.add_argument("--csv", required=True)
    k.add_argument("--steps", type=int, default=50)
    k.add_argument("--warmup", type=int, default=10)
    k.add_argument("--out", required=True)
    n = sub.add_parser("kernels")
    n.add_argument("--csv", required=True)
    n.add_argument("--title", required=True)
    n.add_argument("--command", required=True)
    n.add_argument("--out", required=True)
    pr = sub.add_parser("probe")
    pr.add_argument("--csv", required=True)
    pr.add_argument("--steps", type=int, default=20)
    pr.add_argument("--warmup", type=int, default=5)
    pr.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--db", nargs="+", required=True)
    c.add_argument("--out", required=True)
    c.add_argument("--title", default="")
    c.add_argument("--kernel-sha", default="", help="sha256 of the kernel source the counters were taken on "
                                                     "(default: the current source)")
    kc = sub.add_parser("kcounters")
    kc.add_argument("--db", required=True)
    kc.add_argument("--name", default="gemm")
    kc.add_argument("--title", required=True)
    kc.add_argument("--command", required=True)
    kc.add_argument("--out", required=True)
    a = ap.parse_args()
    text = {"traffic": traffic_summary, "trace": trace_summary, "kernels": kernels_summary,
            "counters": counters_summary, "probe": probe_summary, "kcounters": kernel_counters_summary}[a.cmd](a)
    with open(a.out, "w") as f:
        f.write(text)
    print(text, end="")


if __name__ == "__main__":
    main()
