"""Benchmark of the blockwise ring-attention step on one MI355X.

One step = one pass of the whole hot path for one rank's share: the forward ring
(ra_ring_fwd: every ring step's tiled online softmax with the fused LSE merge,
final output rounded to bf16, LSE saved), then the backward (ra_bwd_delta, then
for every live ring step the dK/dV kernel and the dQ kernel, recomputing P from
the saved LSE).
Default workload: 16 heads x d 128, S = 131072 in the zigzag layout over p = 2,
rank 0, bf16 -- the only workload that exercises every step, forward and backward.

Inputs are synthetic (seeded, see ring_context_parallelism_amd/workloads.py) and
already resident in HBM when the timed region starts.  Timing uses HIP events on
the stream the kernels are launched on.  Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
F32_PEAK_TFLOPS = 157.3    # MI355X fp32 matrix
# Vector ALU: 256 CU x 4 SIMD x 16 lanes x 2.4 GHz = 39.3 T lane-operations/s for
# full-rate fp32 instructions without the packed forms (exp and add have none).
ALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# Vector operations the method needs per visible pair in every attention kernel: the
# scaled shift of the score (one FMA), its exponential, and one more (the row sum in
# the forward, the product P (dP - delta) in the backward).
ALU_OPS_PER_PAIR = 3
HBM_PEAK_GBS = 8000.0
CSRC = os.path.join(ROOT, "ring_context_parallelism_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
COPY_PROBE_BYTES = 1 << 30
# kernel key -> (substring of the device function's name, sources it is built from)
WARM_SECONDS = 0.5  # default untimed warmup work, seconds

KERNELS = {
    "fwd_kernel": ("fwd_bf16_kernel", ("ra_fwd.hip", "ra_internal.h")),
    "fwd_kernel_f32": ("fwd_f32_kernel", ("ra_fwd.hip", "ra_internal.h")),
    "bwd_dkdv_kernel": ("bwd_dkdv_kernel", ("ra_bwd.hip", "ra_internal.h")),
    "bwd_dq_kernel": ("bwd_dq_kernel", ("ra_bwd.hip", "ra_internal.h")),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warmup steps (default: at least 2, and enough for about "
                         f"{WARM_SECONDS} s of work, so that short workloads run at the "
                         "clock a sustained load settles at)")
    ap.add_argument("--workload", default="zigzag_fwdbwd")
    ap.add_argument("--dtype", default=None, help="override the workload dtype (f32|bf16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall time of the oracle sample")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run one device-to-device copy of BYTES (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters against a known byte count)")
    ap.add_argument("--aux", action="store_true",
                    help="time the HBM-bound helper kernels (standalone LSE merge, delta) "
                         "instead of the step and print one JSON line")
    ap.add_argument("--sq-summary", metavar="DIR", default=None,
                    help="print the markdown summary of the three SQ-counter --pmc runs under "
                         "DIR (cnt_1/, cnt_2/, cnt_3/) and exit")
    ap.add_argument("--trace-summary", metavar="DIR", default=None,
                    help="print the markdown summary of the rocprofv3 --kernel-trace --stats run "
                         "under DIR (run_kernel_stats.csv, and the bench line in DIR.log) and exit")
    ap.add_argument("--pmc-summary", metavar="DIR", default=None,
                    help="print the markdown traffic summary of the rocprofv3 --pmc runs under "
                         "DIR (pmc_fetch/, pmc_write/, pmc_copy_fetch/, pmc_copy_write/) and exit")
    return ap.parse_args()


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _logged_hashes(*logs):
    """Kernel source hashes printed by the bench runs that took a set of counters (one
    dict), or None when a log is missing or the runs disagree."""
    seen = None
    for log in logs:
        if not os.path.exists(log):
            return None
        found = None
        for line in open(log):
            if line.startswith("[bench] source hashes "):
                found = json.loads(line[len("[bench] source hashes "):])
        if found is None or (seen is not None and found != seen):
            return None
        seen = found
    return seen


def _check_workload(log, workload):
    """Refuses to summarise a run of another workload than the one named (the bench line
    in the run's log names the workload it ran)."""
    if not os.path.exists(log):
        return
    for line in open(log):
        if line.startswith("{") and '"config"' in line:
            ran = json.loads(line)["config"]["workload"]
            if ran != workload:
                raise SystemExit(f"bench.py: {log} is a run of {ran}, not {workload} "
                                 f"(pass --workload {ran})")


def _counter_kib(run_dir, counter):
    """Mean counter value (KiB) per dispatch, keyed by kernel name, from a --pmc run."""
    acc = {}
    with open(os.path.join(run_dir, "run_counter_collection.csv")) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter:
                acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def pmc_summary(root, workload):
    """Traffic per dispatch from FETCH_SIZE and WRITE_SIZE, each scaled by what the same
    counter reads for a plain device copy of COPY_PROBE_BYTES."""
    _check_workload(os.path.join(root, "pmc_fetch.log"), workload)
    fetch = _counter_kib(os.path.join(root, "pmc_fetch"), "FETCH_SIZE")
    write = _counter_kib(os.path.join(root, "pmc_write"), "WRITE_SIZE")
    cf = _counter_kib(os.path.join(root, "pmc_copy_fetch"), "FETCH_SIZE")
    cw = _counter_kib(os.path.join(root, "pmc_copy_write"), "WRITE_SIZE")
    copy_name = next(k for k in cf if "copyBuffer" in k)
    f_factor = COPY_PROBE_BYTES / (cf[copy_name][0] * 1024.0)
    w_factor = COPY_PROBE_BYTES / (cw[copy_name][0] * 1024.0)
    cmd = ("cd /tmp && timeout -s KILL 240 rocprofv3 --pmc {c} --output-format csv -d <out>/{d} "
           "-o run -- python3 <repo>/bench.py {a}")
    lines = [f"# HBM traffic per dispatch: {workload} workload", "",
             "Commands (one counter per run, on one MI355X):", "", "```"]
    for c, d, a in (("FETCH_SIZE", "pmc_fetch", f"--workload {workload} --steps 1 --warmup 0 "
                     "--no-cpu-baseline"),
                    ("WRITE_SIZE", "pmc_write", f"--workload {workload} --steps 1 --warmup 0 "
                     "--no-cpu-baseline"),
                    ("FETCH_SIZE", "pmc_copy_fetch", f"--copy-probe {COPY_PROBE_BYTES}"),
                    ("WRITE_SIZE", "pmc_copy_write", f"--copy-probe {COPY_PROBE_BYTES}")):
        lines.append(cmd.format(c=c, d=d, a=a))
    lines += ["python3 <repo>/bench.py --pmc-summary <out>", "```", "",
              f"Calibration: a {COPY_PROBE_BYTES} B device copy (`{copy_name}`) reads "
              f"FETCH_SIZE = {cf[copy_name][0]:.0f} KiB and WRITE_SIZE = {cw[copy_name][0]:.0f} KiB, "
              f"so bytes = FETCH_SIZE x 1024 x {f_factor:.3f} and WRITE_SIZE x 1024 x {w_factor:.3f}.",
              "", "| kernel | dispatches | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | fetched (GB) | "
              "written (GB) | traffic (GB) |", "|---|---|---|---|---|---|---|"]
    logged = _logged_hashes(os.path.join(root, "pmc_fetch.log"), os.path.join(root, "pmc_write.log")) or {}
    data = {"workload": workload, "fetch_factor": f_factor, "write_factor": w_factor, "kernels": {}}
    for key, (sub, files) in KERNELS.items():
        name = next((k for k in fetch if sub in k), None)
        if name is None or name not in write:
            continue
        fb = fetch[name][0] * 1024.0 * f_factor
        wb = write[name][0] * 1024.0 * w_factor
        data["kernels"][key] = {"name": name, "source_hash": logged.get(key),
                                "fetch_bytes": fb, "write_bytes": wb, "traffic_bytes": fb + wb}
        lines.append(f"| `{name[:80]}` | {fetch[name][1]} | {fetch[name][0]:.0f} | "
                     f"{write[name][0]:.0f} | {fb / 1e9:.3f} | {wb / 1e9:.3f} | "
                     f"{(fb + wb) / 1e9:.3f} |")
    lines += ["", "Source hashes (sha256 prefix of the kernel's source files, as printed by the "
              "profiled bench runs) identify the kernel build the counters were taken on; "
              "`bench.py` reports `traffic` only while they match.", "", "```json",
              json.dumps(data, indent=1), "```", ""]
    return "\n".join(lines)


SQ_PASSES = (
    "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_LDS "
    "SQ_WAIT_INST_LDS SQ_ACTIVE_INST_LDS SQ_LDS_IDX_ACTIVE",
    "SQ_LDS_BANK_CONFLICT SQ_LDS_ADDR_CONFLICT SQ_LDS_DATA_FIFO_FULL SQ_LDS_CMD_FIFO_FULL "
    "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_MISC SQ_WAIT_ANY SQ_BUSY_CU_CYCLES",
    "SQ_INSTS_VALU SQ_ACTIVE_INST_ANY SQ_WAIT_INST_ANY SQ_INST_LEVEL_LDS SQ_INSTS_SALU "
    "SQ_ACTIVE_INST_SCA SQ_INSTS_VMEM SQ_WAVES",
)


def sq_summary(root, workload, n_cu=256):
    """Per-kernel ratios from three SQ-counter passes (one launch of each kernel per step)."""
    _check_workload(os.path.join(root, "cnt_1.log"), workload)
    agg, dur = {}, {}
    for i in range(len(SQ_PASSES)):
        with open(os.path.join(root, f"cnt_{i + 1}", "run_counter_collection.csv")) as fh:
            for r in csv.DictReader(fh):
                key = next((k for k, (sub, _) in KERNELS.items() if sub in r["Kernel_Name"]), None)
                if key is None:
                    continue
                agg.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(
                    float(r["Counter_Value"]))
                dur.setdefault(key, {})[(i, r["Dispatch_Id"])] = (
                    int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    cmd = ("cd /tmp && timeout -s KILL 200 rocprofv3 --pmc {c} --output-format csv -d <out>/cnt_{i} "
           "-o run -- python3 <repo>/bench.py --workload {w} --steps 1 --warmup 0 --no-cpu-baseline")
    lines = [f"# SQ counters per kernel: {workload} workload", "",
             "Commands (three passes, at most 8 SQ counters each, on one MI355X):", "", "```"]
    lines += [cmd.format(c=c, i=i + 1, w=workload) for i, c in enumerate(SQ_PASSES)]
    lines += ["python3 <repo>/bench.py --sq-summary <out>", "```", "",
              "Cycle counters are summed over the chip (`SQ_BUSY_CU_CYCLES` over 256 CUs, "
              "`SQ_VALU_MFMA_BUSY_CYCLES` over 1024 SIMDs; the latter counts the clocks each "
              "MFMA occupies: 16 for a 16x16x32 bf16 tile, 32 for a 32x32x16 one).  Effective "
              "clock = "
              "`SQ_BUSY_CU_CYCLES` / 256 / kernel duration.  VALU instructions per SIMD-cycle = "
              "`SQ_INSTS_VALU` / (4 `SQ_BUSY_CU_CYCLES`); waves per SIMD = `SQ_WAVE_CYCLES` / "
              "`SQ_BUSY_CU_CYCLES` (`SQ_WAVE_CYCLES` counts in units of 4 cycles).", "",
              "| kernel | duration (ms, under counters) | effective clock (GHz) | MFMA busy | LDS busy "
              "| LDS bank-conflict share | VALU / MFMA | LDS / MFMA | SALU / MFMA | wait-any / wave cycles "
              "| VALU instr per SIMD-cycle | waves per SIMD |",
              "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    logged = _logged_hashes(*[os.path.join(root, f"cnt_{i + 1}.log")
                              for i in range(len(SQ_PASSES))]) or {}
    data = {"workload": workload, "kernels": {}}
    for key, c in agg.items():
        m = {k: sum(v) / len(v) for k, v in c.items()}
        t = sum(dur[key].values()) / len(dur[key])
        busy = m["SQ_BUSY_CU_CYCLES"]
        data["kernels"][key] = {
            "name": KERNELS[key][0], "source_hash": logged.get(key),
            "mfma_busy": round(m["SQ_VALU_MFMA_BUSY_CYCLES"] / (4 * busy), 4),
            "effective_clock_ghz": round(busy / n_cu / t / 1e9, 3),
            "lds_busy": round(m["SQ_LDS_IDX_ACTIVE"] / busy, 4)}
        lines.append(
            f"| `{KERNELS[key][0]}` | {t * 1e3:.2f} | {busy / n_cu / t / 1e9:.2f} | "
            f"{m['SQ_VALU_MFMA_BUSY_CYCLES'] / (4 * busy):.3f} | "
            f"{m['SQ_LDS_IDX_ACTIVE'] / busy:.3f} | "
            f"{m['SQ_LDS_BANK_CONFLICT'] / max(m['SQ_LDS_IDX_ACTIVE'], 1):.3f} | "
            f"{m['SQ_INSTS_VALU'] / m['SQ_INSTS_MFMA']:.2f} | "
            f"{m['SQ_INSTS_LDS'] / m['SQ_INSTS_MFMA']:.2f} | "
            f"{m['SQ_INSTS_SALU'] / m['SQ_INSTS_MFMA']:.2f} | "
            f"{m['SQ_WAIT_ANY'] / m['SQ_WAVE_CYCLES']:.3f} | "
            f"{m['SQ_INSTS_VALU'] / (4 * busy):.3f} | {m['SQ_WAVE_CYCLES'] / busy:.2f} |")
    lines += ["", "Read by `bench.py`, which attaches a kernel's figures to its `roofline` only "
              "while the `source_hash` printed by the profiled runs matches the current "
              "sources:", "", "```json", json.dumps(data, indent=1), "```", ""]
    return "\n".join(lines)


def trace_summary(run_dir, workload):
    """Kernel durations from a --kernel-trace --stats run, with the algorithmic FLOP rate of
    each attention kernel (forward 4d, dK/dV 8d, dQ 2d per visible pair and head)."""
    from ring_context_parallelism_amd import ra
    from ring_context_parallelism_amd.workloads import WORKLOADS, document_bounds
    w = WORKLOADS[workload]
    bounds = document_bounds(w) if w.docs else None
    prob = ra.make_problem(batch=w.batch, heads_q=w.heads_q, heads_kv=w.heads_kv,
                           head_dim=w.head_dim, head_dim_padded=w.head_dim_padded,
                           seq_total=w.seq_total, world=w.world, layout=w.layout,
                           causal=w.causal, dtype=w.dtype)
    steps = step_flops(w, prob, ra, bounds)
    pairs = sum(st["visible_pairs_per_head"] * w.batch * w.heads_q for st in steps) / len(steps)
    per_pair = {"fwd_bf16_kernel": 4, "fwd_f32_kernel": 4, "bwd_dkdv_kernel": 8,
                "bwd_dq_kernel": 2}
    peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else F32_PEAK_TFLOPS
    rows = list(csv.DictReader(open(os.path.join(run_dir, "run_kernel_stats.csv"))))
    bench_line = None
    log = run_dir.rstrip("/") + ".log"
    _check_workload(log, workload)
    if os.path.exists(log):
        for line in open(log):
            if line.startswith("{") and '"roofline"' in line:
                bench_line = json.loads(line)
    lines = [f"# Kernel durations: {workload} workload ({w.batch} x {w.heads_q} heads x "
             f"d{w.head_dim}, S={w.seq_total}, {w.layout} p={w.world}, rank {w.rank}, {w.dtype})",
             "", "Command (run from /tmp on one MI355X):", "", "```",
             "cd /tmp && timeout -k 10 300 rocprofv3 --kernel-trace --stats --output-format csv "
             "-d <out>/prof_default -o run -- python3 <repo>/bench.py --workload "
             f"{workload} --steps 3 --warmup 1 --no-cpu-baseline > <out>/prof_default.log",
             f"python3 <repo>/bench.py --workload {workload} --trace-summary <out>/prof_default",
             "```", "",
             f"{len(steps)} live ring steps per bench step; {pairs:.4g} visible (query, key) pairs "
             "per launch summed over batch and heads.  Algorithmic FLOP per launch: forward 4d, "
             "dK/dV kernel 8d (S, dP, dV, dK), dQ kernel 2d (its recomputation of S and dP is "
             "not counted) per pair.  The forward kernel's calls include the per-step "
             "timing pass that follows the timed steps (each live step launched once more "
             "on its own).", "",
             "| kernel | calls | average (ms) | min (ms) | max (ms) | share | algorithmic "
             "TFLOP/s | of peak |", "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        avg = float(r["AverageNs"]) * 1e-6
        rate = ""
        frac = ""
        for sub, k in per_pair.items():
            if sub in r["Name"]:
                tf = k * w.head_dim * pairs / (avg * 1e-3) / 1e12
                rate, frac = f"{tf:.1f}", f"{100 * tf / peak:.1f}%"
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {avg:.3f} | "
                     f"{float(r['MinNs']) * 1e-6:.3f} | {float(r['MaxNs']) * 1e-6:.3f} | "
                     f"{float(r['Percentage']):.2f}% | {rate} | {frac} |")
    if bench_line is not None:
        rf = bench_line["roofline"]
        lines += ["", "The bench line printed by the same profiled command (HIP events on the "
                  "launch stream, timed steps only; the rocprof averages include the warmup "
                  f"step): {bench_line['value']:.1f} TFLOP/s per step, forward "
                  f"{bench_line['fwd']['pct_peak']:.1f}% of peak"
                  + (f", backward {bench_line['bwd']['pct_peak']:.1f}%" if "bwd" in bench_line
                     else "")
                  + f"; roofline kernel `{rf['kernel']}` ({rf['bound']}-bound) "
                  f"{rf['avg_launch_ms']:.3f} ms per launch, {rf['achieved']:.1f} {rf['unit']}, "
                  f"frac {rf['frac']:.4f}."]
    lines.append("")
    return "\n".join(lines)


def measured_traffic(workload, key):
    """Bytes per dispatch from the committed counter summary, or None when there is none for
    this workload or the kernel's sources changed since the counters were taken."""
    path = os.path.join(PROFILES, f"pmc_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    data = json.loads(m.group(1))
    k = data["kernels"].get(key)
    if k is None or data["workload"] != workload or k["source_hash"] != source_hash(KERNELS[key][1]):
        return None
    return k["traffic_bytes"]


def measured_counters(workload, key):
    """MFMA busy, effective clock and LDS busy of one kernel from the committed SQ-counter
    summary, or None when there is none for this workload or the kernel's sources
    changed since the counters were taken."""
    path = os.path.join(PROFILES, f"sq_counters_{workload}.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    data = json.loads(m.group(1))
    k = data["kernels"].get(key)
    if k is None or data["workload"] != workload or k["source_hash"] != source_hash(KERNELS[key][1]):
        return None
    return {f: k[f] for f in ("mfma_busy", "effective_clock_ghz", "lds_busy")}


def roofline(flop, pairs, launch_ms, mfma_peak):
    """The roof a kernel sits closer to: the matrix cores (its algorithmic FLOP against
    the dense MFMA peak of its dtype) or the vector ALU (ALU_OPS_PER_PAIR per visible
    pair against ALU_PEAK_TOPS; small head dims, where the per-score softmax work
    dominates).  The other fraction is reported alongside."""
    achieved = flop / (launch_ms * 1e-3) / 1e12
    alu_ops = ALU_OPS_PER_PAIR * pairs
    alu_achieved = alu_ops / (launch_ms * 1e-3) / 1e12
    if alu_achieved / ALU_PEAK_TOPS > achieved / mfma_peak:
        return {"bound": "alu", "achieved": round(alu_achieved, 3),
                "peak": round(ALU_PEAK_TOPS, 2), "unit": "TOP/s",
                "frac": round(alu_achieved / ALU_PEAK_TOPS, 4), "ops_per_launch": alu_ops,
                "mfma_frac": round(achieved / mfma_peak, 4)}
    return {"bound": "mfma", "achieved": round(achieved, 3), "peak": mfma_peak,
            "unit": "TFLOP/s", "frac": round(achieved / mfma_peak, 4), "flop_per_launch": flop,
            "alu_frac": round(alu_achieved / ALU_PEAK_TOPS, 4)}


def step_flops(w, prob, ra, bounds=None):
    """Algorithmic FLOP per live ring step: exact visible pairs x 4d (fwd), x 10d (bwd).
    Packed workloads count pairs inside documents (summed over the batch)."""
    out = []
    for s in range(w.world):
        c = (w.rank - s) % w.world
        if bounds is None:
            pairs = ra.ra_visible_pairs(prob, w.rank, c)
            per_head = pairs * w.batch
        else:
            per_head = ra.ra_visible_pairs_packed(prob, w.rank, c, bounds)
            pairs = per_head / w.batch
        if per_head == 0:
            continue
        out.append(dict(step=s, chunk=c, visible_pairs_per_head=pairs,
                        fwd_flop=4.0 * w.head_dim * per_head * w.heads_q,
                        bwd_flop=10.0 * w.head_dim * per_head * w.heads_q))
    return out


def cpu_baseline(w, arrays, target_s):
    """The oracle, as it is, on a bounded sample of the same share (fp64, host cores)."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        blas = ",".join(sorted({p.get("internal_api", "?") for p in threadpool_info()}))
    except Exception:  # pragma: no cover - reporting only
        threads, blas = 1, "unknown"
    rows_all = oracle.positions(w.layout, w.seq_total, w.world, w.rank)
    bounds = None if arrays.get("bounds") is None else [list(map(int, e)) for e in arrays["bounds"]]
    rng = np.random.default_rng(1234)
    n = 64
    while True:
        t_idx = np.sort(rng.choice(rows_all.size, size=min(n, rows_all.size), replace=False))
        rows = rows_all[t_idx]
        t0 = time.perf_counter()
        dQ = None
        if w.backward:
            dO = arrays["do"][:, :1][:, :, rows]
            dQ, _, _ = oracle.attention_bwd(arrays["q"], arrays["k"], arrays["v"], dO, rows,
                                            w.causal, heads=[0], bounds=bounds)
        O, LSE = oracle.attention_fwd(arrays["q"], arrays["k"], arrays["v"], rows, w.causal,
                                      heads=[0], bounds=bounds)
        dt = time.perf_counter() - t0
        if dt >= 0.6 * target_s or n >= rows_all.size:
            break
        # grow the sample towards the target wall time (at most 16x per round)
        n = int(min(rows_all.size, n * min(16.0, max(2.0, target_s / max(dt, 1e-3)))))
    if bounds is None:
        pairs = float(np.sum(rows + 1)) if w.causal else float(rows.size * w.seq_total)
    else:  # keys of the row's own document (at or before it when causal), per batch element
        pairs = 0.0
        for e in bounds:
            e = np.asarray(e, dtype=np.int64)
            k = np.searchsorted(e, rows, side="right") - 1
            live = rows < e[-1]
            start, end = e[np.clip(k, 0, e.size - 1)], e[np.clip(k + 1, 0, e.size - 1)]
            cnt = np.where(w.causal, rows - start + 1, end - start)
            pairs += float(np.sum(np.where(live, cnt, 0)))
        pairs /= w.batch
    per_pair = (4.0 + (10.0 if w.backward else 0.0)) * w.head_dim
    flop = pairs * per_pair * w.batch
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{rows.size} query rows of head 0 (batch {w.batch}), "
                      f"{'forward + backward' if w.backward else 'forward'} in fp64, "
                      f"{pairs:.3e} visible pairs, {dt:.1f} s wall, BLAS {blas}",
            "seconds": dt}, (t_idx, O, LSE, dQ)


def sample_parity(w, ref, out, lse, dq):
    """The timed run's outputs on the oracle's sample rows (head 0) against the oracle."""
    import numpy as np
    t_idx, O, LSE, dQ = ref
    d = w.head_dim
    ti = torch_index(t_idx, out.device)

    def cmp(got, want):
        err = np.abs(got - want)
        den = np.linalg.norm(want)
        return {"max_abs": float(err.max()), "mean_abs": float(err.mean()),
                "rel_fro": float(np.linalg.norm(got - want) / den) if den > 0 else 0.0}

    res = {"rows": int(t_idx.size), "head": 0}
    res["o"] = cmp(out[:, :1][:, :, ti].float().cpu().numpy()[..., :d], O)
    lg = lse[:, :1][:, :, ti].cpu().numpy()
    fin = np.isfinite(LSE)
    res["lse_max_abs"] = float(np.abs(lg[fin] - LSE[fin]).max()) if fin.any() else 0.0
    res["lse_inf_rows_match"] = bool(np.array_equal(np.isneginf(lg), np.isneginf(LSE)))
    if dQ is not None and dq is not None:
        res["dq"] = cmp(dq[:, :1][:, :, ti].cpu().numpy()[..., :d], dQ)
    tol = (2e-2, 2e-3, 1e-2) if w.dtype == "bf16" else (1e-5, 1e-5, 1e-5)
    ok = all(res[k]["max_abs"] <= tol[0] and res[k]["mean_abs"] <= tol[1]
             and res[k]["rel_fro"] <= tol[2] for k in ("o", "dq") if k in res)
    res["pass"] = bool(ok and res["lse_max_abs"] <= 1e-3 and res["lse_inf_rows_match"])
    return res


def torch_index(idx, device):
    import torch
    return torch.from_numpy(idx).to(device)


def copy_probe(nbytes):
    import torch
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes}), flush=True)


def aux_bench(reps=50):
    """The HBM-bound helpers against the 8 TB/s roofline, at the llama_share and
    zigzag_fwdbwd shapes: the standalone LSE merge (rows x d fp32 partials) and the
    backward's delta = rowsum(dO * O) (bf16 inputs).  Algorithmic bytes per row:
    the merge reads both partials (2 d x 4 B) and both LSEs and writes the accumulator
    (d x 4 B) and its LSE, (3 d + 3) x 4 B in all; delta reads O and dO (2 d x 2 B)
    and writes 4 B."""
    import torch

    from ring_context_parallelism_amd import ra
    dev = torch.device("cuda:0")
    ra.lib()
    out = {"metric": "HBM-bound helper kernels, achieved GB/s", "unit": "GB/s", "kernels": []}
    stream = torch.cuda.current_stream()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    for name, rows, d in (("llama_share", 1 * 16 * 8192, 128), ("zigzag_fwdbwd", 16 * 65536, 128)):
        oa = torch.randn(rows, d, device=dev)
        op = torch.randn(rows, d, device=dev)
        la = torch.randn(rows, device=dev)
        lp = torch.randn(rows, device=dev)
        ms = timed(lambda: ra.ra_lse_merge(rows, d, oa, la, op, lp, stream=stream))
        nbytes = rows * (3 * d * 4 + 3 * 4)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out["kernels"].append({"kernel": "lse_merge_kernel", "shape": f"{name}: {rows} rows x {d}",
                               "ms": round(ms, 4), "bytes": nbytes, "achieved": round(gbs, 1),
                               "peak": HBM_PEAK_GBS, "frac": round(gbs / HBM_PEAK_GBS, 4)})
    # reference: a plain device-to-device copy of 1 GiB (read + write)
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    ms = timed(lambda: dst.copy_(src))
    gbs = 2 * src.numel() * 4 / (ms * 1e-3) / 1e9
    out["copy_reference"] = {"bytes": 2 * src.numel() * 4, "ms": round(ms, 4),
                             "achieved": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}
    del src, dst
    B, H, L, D = 1, 16, 65536, 128
    o = torch.randn(B, H, L, D, device=dev).to(torch.bfloat16)
    do = torch.randn(B, H, L, D, device=dev).to(torch.bfloat16)
    delta = torch.empty(B, H, L, device=dev)
    prob = ra.make_problem(batch=B, heads_q=H, heads_kv=H, head_dim=D, head_dim_padded=D,
                           seq_total=2 * L, world=2, layout="zigzag", causal=True, dtype="bf16")
    ms = timed(lambda: ra.ra_bwd_delta(prob, o, do, delta, stream=stream))
    nbytes = B * H * L * (2 * D * 2 + 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    out["kernels"].append({"kernel": "bwd_delta_kernel", "shape": f"zigzag_fwdbwd: {B * H * L} rows x {D}",
                           "ms": round(ms, 4), "bytes": nbytes, "achieved": round(gbs, 1),
                           "peak": HBM_PEAK_GBS, "frac": round(gbs / HBM_PEAK_GBS, 4)})
    print(json.dumps(out), flush=True)


def time_fwd_steps(ra, prob, w, share, steps, ws, stream, reps):
    """Milliseconds of each live forward step launched on its own, one array per step.

    The steps run in ring order through ra_block_attn_fwd: the first writes the fp32
    workspace, the others merge into it, as in the ring driver (whose last launch
    writes the output dtype instead).  One untimed pass comes first."""
    import numpy as np
    import torch
    lse = torch.empty((w.batch, w.heads_q, w.chunk_len), dtype=torch.float32, device=ws.device)
    n = len(steps)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(reps + 1)]
    for e in ev:
        e[0].record(stream)
        for i, st in enumerate(steps):
            c = st["chunk"]
            ra.ra_block_attn_fwd(prob, share.q, w.rank, share.k_chunks[c], share.v_chunks[c], c,
                                 ws, lse, ra.RA_WRITE if i == 0 else ra.RA_MERGE, stream=stream)
            e[i + 1].record(stream)
    torch.cuda.synchronize()
    return [np.array([e[i].elapsed_time(e[i + 1]) for e in ev[1:]]) for i in range(n)]


def main():
    args = parse()
    if args.aux:
        aux_bench()
        return
    if args.pmc_summary:
        print(pmc_summary(args.pmc_summary, args.workload))
        return
    if args.trace_summary:
        print(trace_summary(args.trace_summary, args.workload))
        return
    if args.sq_summary:
        print(sq_summary(args.sq_summary, args.workload))
        return
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU ring exchange is designed but not implemented).",
              file=sys.stderr)
        sys.exit(2)

    print("[bench] source hashes " + json.dumps({k: source_hash(f) for k, (_, f) in KERNELS.items()}),
          file=sys.stderr, flush=True)
    import numpy as np
    import torch

    from ring_context_parallelism_amd import ra, staging
    from ring_context_parallelism_amd.workloads import WORKLOADS, generate

    w = WORKLOADS[args.workload]
    if args.dtype:
        w = w.with_dtype(args.dtype)
    dev = torch.device("cuda:0")
    ra.lib()  # fail loudly if the library is missing
    print(f"[bench] workload {w.name} {w.dtype}: generating inputs", file=sys.stderr, flush=True)
    arrays = generate(w)
    share = staging.stage(w, arrays, dev)
    prob = share.prob
    steps = step_flops(w, prob, ra, arrays.get("bounds"))
    L, D = w.chunk_len, w.head_dim_padded
    stream = torch.cuda.current_stream()
    tdt = staging.torch_dtype(w)

    out = torch.empty((w.batch, w.heads_q, L, D), dtype=tdt, device=dev)
    lse = torch.empty((w.batch, w.heads_q, L), dtype=torch.float32, device=dev)
    ws = torch.empty(ra.ra_ring_workspace_size(prob) // 4, dtype=torch.float32, device=dev)
    if w.backward:
        delta = torch.empty((w.batch, w.heads_q, L), dtype=torch.float32, device=dev)
        dq = torch.empty((w.batch, w.heads_q, L, D), dtype=torch.float32, device=dev)
        dks = [torch.empty((w.batch, w.heads_kv, L, D), dtype=torch.float32, device=dev)
               for _ in range(w.world)]
        dvs = [torch.empty_like(dks[0]) for _ in range(w.world)]

    n_ev = 2 + (1 + 2 * len(steps) if w.backward else 0)

    def one_step(ev):
        ev[0].record(stream)
        ra.ra_ring_fwd(prob, w.rank, share.q, share.k_chunks, share.v_chunks, out, lse, ws,
                       stream=stream)
        ev[1].record(stream)
        if not w.backward:
            return
        ra.ra_bwd_prepare(prob, out, share.do, delta, dq, dks, dvs, stream=stream)
        ev[2].record(stream)
        for i, st in enumerate(steps):
            c = st["chunk"]
            args_ = (prob, share.q, w.rank, share.k_chunks[c], share.v_chunks[c], c, share.do, lse,
                     delta)
            ra.ra_block_attn_bwd_dkdv(*args_, dks[c], dvs[c], stream=stream)
            ev[3 + 2 * i].record(stream)
            ra.ra_block_attn_bwd_dq(*args_, dq, stream=stream)
            ev[4 + 2 * i].record(stream)

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
              for _ in range(args.steps)]
    warm = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    if args.warmup is None:
        # Default: at least 2 steps and about WARM_SECONDS of work.  The chip's clock
        # settles only under sustained load, which a few steps of a short workload
        # do not give.
        one_step(warm)  # the first step also loads the kernels: not timed
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        one_step(warm)
        torch.cuda.synchronize()
        per = max(time.perf_counter() - t0, 1e-6)
        todo = min(5000, int(WARM_SECONDS / per))
        args.warmup = 2 + todo
    else:
        todo = args.warmup
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(todo):
        one_step(warm)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t_start = time.perf_counter()
    for k in range(args.steps):
        one_step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start

    fwd_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    step_ms = np.array([e[0].elapsed_time(e[-1]) for e in events])
    fwd_flop = sum(s["fwd_flop"] for s in steps)
    bwd_flop = sum(s["bwd_flop"] for s in steps) if w.backward else 0.0
    peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else F32_PEAK_TFLOPS
    ms_per_step = float(np.mean(step_ms))
    value = (fwd_flop + bwd_flop) / (ms_per_step * 1e-3) / 1e12

    fwd_step_ms = float(np.mean(fwd_ms)) / len(steps)  # the driver launches one kernel per live step
    # Per-step forward times: the driver is timed as a whole above, so each live step
    # is launched once more on its own (ra_block_attn_fwd, WRITE then MERGE into the
    # fp32 workspace), with events around every launch, after the timed region.
    step_fwd = time_fwd_steps(ra, prob, w, share, steps, ws, stream, max(3, args.steps))
    detail = []
    for i, st in enumerate(steps):
        sm = step_fwd[i]
        d = dict(step=st["step"], chunk=st["chunk"],
                 visible_pairs_per_head=st["visible_pairs_per_head"],
                 fwd_ms=float(np.mean(sm)), fwd_ms_median=float(np.median(sm)),
                 fwd_ms_min=float(np.min(sm)),
                 fwd_tflops=st["fwd_flop"] / (float(np.mean(sm)) * 1e-3) / 1e12)
        if w.backward:
            kv_ms = np.array([e[2 + 2 * i].elapsed_time(e[3 + 2 * i]) for e in events])
            q_ms = np.array([e[3 + 2 * i].elapsed_time(e[4 + 2 * i]) for e in events])
            bms = kv_ms + q_ms
            d.update(bwd_ms=float(np.mean(bms)), bwd_ms_median=float(np.median(bms)),
                     bwd_ms_min=float(np.min(bms)),
                     bwd_dkdv_ms=float(np.mean(kv_ms)), bwd_dq_ms=float(np.mean(q_ms)),
                     bwd_tflops=st["bwd_flop"] / (float(np.mean(bms)) * 1e-3) / 1e12)
        d["fwd_pct_peak"] = 100.0 * d["fwd_tflops"] / peak
        if w.backward:
            d["bwd_pct_peak"] = 100.0 * d["bwd_tflops"] / peak
        detail.append(d)

    fwd_tflops = fwd_flop / (float(np.mean(fwd_ms)) * 1e-3) / 1e12
    res = {
        "metric": "causal-adjusted attention TFLOP/s per ring step (fwd, bwd) + % of MFMA peak",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads_q": w.heads_q,
                   "heads_kv": w.heads_kv, "head_dim": w.head_dim,
                   "head_dim_padded": w.head_dim_padded, "seq_total": w.seq_total,
                   "world": w.world, "layout": w.layout, "rank": w.rank, "causal": w.causal,
                   "passes": "fwd+bwd" if w.backward else "fwd"},
        "fwd": {"ms": round(float(np.mean(fwd_ms)), 4), "tflops": round(fwd_tflops, 3),
                "pct_peak": round(100.0 * fwd_tflops / peak, 2), "flop": fwd_flop},
        "per_step": detail,
        "wall_s": round(wall, 3),
    }
    if w.backward:
        bwd_ms_total = float(np.mean([e[2].elapsed_time(e[-1]) for e in events]))
        aux_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
        bwd_tflops = bwd_flop / (bwd_ms_total * 1e-3) / 1e12
        res["bwd"] = {"ms": round(bwd_ms_total, 4), "tflops": round(bwd_tflops, 3),
                      "pct_peak": round(100.0 * bwd_tflops / peak, 2), "flop": bwd_flop,
                      "delta_and_zero_ms": round(aux_ms, 4)}
    # Dominant kernel: the one with the largest share of the step.  Algorithmic FLOP
    # per launch count only the contractions the method needs: forward 4d per
    # visible pair (QK^T, PV); dK/dV kernel 8d (S, dP, dV, dK); dQ kernel 2d (dQ --
    # its recomputation of S and dP is not counted).
    pairs_bh = [st["visible_pairs_per_head"] * w.batch * w.heads_q for st in steps]
    fwd_key = "fwd_kernel" if w.dtype == "bf16" else "fwd_kernel_f32"
    kern = {fwd_key: (fwd_step_ms * len(steps), fwd_flop / len(steps), fwd_step_ms)}
    if w.backward:
        kv_ms = float(np.mean([sum(e[2 + 2 * i].elapsed_time(e[3 + 2 * i]) for i in range(len(steps)))
                               for e in events]))
        q_ms = float(np.mean([sum(e[3 + 2 * i].elapsed_time(e[4 + 2 * i]) for i in range(len(steps)))
                              for e in events]))
        res["bwd"]["dkdv_ms"] = round(kv_ms, 4)
        res["bwd"]["dq_ms"] = round(q_ms, 4)
        kern["bwd_dkdv_kernel"] = (kv_ms, 8.0 * w.head_dim * sum(pairs_bh) / len(steps),
                                   kv_ms / len(steps))
        kern["bwd_dq_kernel"] = (q_ms, 2.0 * w.head_dim * sum(pairs_bh) / len(steps),
                                 q_ms / len(steps))
    name = max(kern, key=lambda k: kern[k][0])
    _, per_launch_flop, launch_ms = kern[name]
    res["roofline"] = roofline(per_launch_flop, sum(pairs_bh) / len(steps), launch_ms, peak)
    res["roofline"].update({"traffic": measured_traffic(w.name, name), "kernel": name,
                            "avg_launch_ms": round(launch_ms, 4)})
    counters = measured_counters(w.name, name)
    if counters is not None:
        res["roofline"]["counters"] = counters
    if res["roofline"]["traffic"] is not None:
        res["roofline"]["traffic_gbps"] = round(res["roofline"]["traffic"] / (launch_ms * 1e-3) / 1e9, 1)
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on host cores", file=sys.stderr, flush=True)
        res["cpu_baseline"], ref = cpu_baseline(w, arrays, args.cpu_seconds)
        res["parity"] = sample_parity(w, ref, out, lse, dq if w.backward else None)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
