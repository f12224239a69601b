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
the stream the kernels are launched on.  Prints ONE JSON line: the headline share
with its roofline, parity and the oracle's CPU rate, and (default run) every other
workload -- the forward shares, and the packed-document share forward and backward --
each timed with its own parity check.
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
# full-rate fp32 instructions (a wave64 instruction occupies a SIMD for 4 cycles).
ALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# Vector work the method needs per visible (query, key) pair, in full-rate issue slots:
# the scaled shift of the score (one FMA), its exponential (v_exp_f32 occupies a SIMD
# for 8 cycles, two slots: the SQ counters' VALU cycles per instruction fit
# 4 (1 - f) + 8 f with f the transcendental share, on every profiled kernel), then
#   forward, bf16: the row-sum add and half a conversion (v_cvt_pk_bf16_f32 rounds two
#     values of P for the PV MFMA)                                   1 + 2 + 1 + 0.5
#   forward, fp32: the row-sum add and the row-max pass                1 + 2 + 1 + 1
#   dK/dV: the product P (dP - delta) and two half conversions (P, dS) 1 + 2 + 1 + 1
#   dQ: the product P (dP - delta) and half a conversion (dS)        1 + 2 + 1 + 0.5
ALU_SLOTS_PER_PAIR = {"fwd_kernel": 4.5, "fwd_kernel_f32": 5.0, "bwd_dkdv_kernel": 5.0,
                      "bwd_dq_kernel": 4.5}
HBM_PEAK_GBS = 8000.0
CSRC = os.path.join(ROOT, "ring_context_parallelism_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
COPY_PROBE_BYTES = 1 << 30
WARM_SECONDS = 0.5  # default untimed warmup work, seconds
DEFAULT_WORKLOAD = "zigzag_fwdbwd"
# The forward-only workloads the default run also times (each as one object of the
# line's "configs" list), in the order of their sizes.
OTHER_CONFIGS = ("tiny_fp32", "llama_share", "gqa_striped", "tabular_rows", "tabular_rows_bf16")
# The packed-document share (forward and backward), reported beside them.
PACKED_CONFIG = "packed_fwdbwd"

# kernel key -> (substring of the device function's name, sources it is built from)
KERNELS = {
    "fwd_kernel": ("fwd_bf16_kernel", ("ra_fwd.hip", "ra_internal.h")),
    "fwd_kernel_f32": ("fwd_f32_kernel", ("ra_fwd_f32.hip", "ra_internal.h")),
    "bwd_dkdv_kernel": ("bwd_dkdv_kernel", ("ra_bwd.hip", "ra_internal.h")),
    "bwd_dq_kernel": ("bwd_dq_kernel", ("ra_bwd.hip", "ra_internal.h")),
    "lse_merge_kernel": ("lse_merge_kernel", ("ra_misc.hip", "ra_internal.h")),
    "bwd_delta_kernel": ("bwd_delta_kernel", ("ra_misc.hip", "ra_internal.h")),
}
# Shapes the HBM-bound helpers are timed and counted at (--aux): (name, rows, head dim).
AUX_SHAPES = {"llama_share": (1 * 16 * 8192, 128), "zigzag_fwdbwd": (16 * 65536, 128)}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warmup steps (default: at least 2, and enough for about "
                         f"{WARM_SECONDS} s of work, so that short workloads run at the "
                         "clock a sustained load settles at)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--dtype", default=None, help="override the workload dtype (f32|bf16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the forward-only workloads timed after the default one")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall time of the oracle sample")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run one device-to-device copy of BYTES (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters against a known byte count)")
    ap.add_argument("--aux", action="store_true",
                    help="time the HBM-bound helper kernels (standalone LSE merge, delta) "
                         "instead of the step and print one JSON line")
    ap.add_argument("--aux-shape", default=None, choices=sorted(AUX_SHAPES),
                    help="with --aux: only this shape (one shape per counter run)")
    ap.add_argument("--sq-summary", metavar="DIR", default=None,
                    help="print the markdown summary of the four SQ-counter --pmc runs under "
                         "DIR (cnt_1/ .. cnt_4/) and exit")
    ap.add_argument("--trace-summary", metavar="DIR", default=None,
                    help="print the markdown summary of the rocprofv3 --kernel-trace --stats run "
                         "under DIR (run_kernel_stats.csv, and the bench line in DIR.log) and exit")
    ap.add_argument("--aux-summary", metavar="FILE", default=None,
                    help="print the markdown summary of a saved --aux JSON line and exit")
    ap.add_argument("--pmc-summary", metavar="DIR", default=None,
                    help="print the markdown traffic summary of the rocprofv3 --pmc runs under "
                         "DIR (pmc_fetch/, pmc_write/, pmc_copy_fetch/, pmc_copy_write/) and exit")
    return ap.parse_args()


def source_hash(files):
    """Hash of a kernel's source files and of the compiler flags they are built with
    (a flag can change the code as much as the source)."""
    from ring_context_parallelism_amd import build as _build
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
        if f.endswith(".hip"):
            h.update(" ".join(_build.FLAGS + _build.SOURCE_FLAGS.get(f, [])).encode())
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


def _profiled_args(workload):
    """bench.py arguments of a counter run: one step of the workload, or the helper
    kernels at the zig-zag share's shape for the pseudo-workload "aux"."""
    if workload == "aux":
        return "--aux --aux-shape zigzag_fwdbwd"
    return f"--workload {workload} --steps 1 --warmup 0 --no-cpu-baseline --no-configs"


def _aux_algorithmic_bytes(workload):
    """Algorithmic bytes per launch of the helper kernels of an "aux" counter run."""
    if workload != "aux":
        return {}
    rows, d = AUX_SHAPES["zigzag_fwdbwd"]
    return {"lse_merge_kernel": rows * (3 * d + 3) * 4, "bwd_delta_kernel": rows * (2 * d * 2 + 4)}


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
    run_args = _profiled_args(workload)
    title = ("the HBM-bound helper kernels (standalone LSE merge, backward delta) at the "
             "zig-zag share's shape" if workload == "aux" else f"{workload} workload")
    lines = [f"# HBM traffic per dispatch: {title}", "",
             "Commands (one counter per run, on one MI355X):", "", "```"]
    for c, d, a in (("FETCH_SIZE", "pmc_fetch", run_args),
                    ("WRITE_SIZE", "pmc_write", run_args),
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
    algo = _aux_algorithmic_bytes(workload)
    for key, (sub, files) in KERNELS.items():
        name = next((k for k in fetch if sub in k), None)
        if name is None or name not in write:
            continue
        fb = fetch[name][0] * 1024.0 * f_factor
        wb = write[name][0] * 1024.0 * w_factor
        data["kernels"][key] = {"name": name, "source_hash": logged.get(key),
                                "fetch_bytes": fb, "write_bytes": wb, "traffic_bytes": fb + wb}
        if key in algo:
            data["kernels"][key].update(algorithmic_bytes=algo[key],
                                        traffic_over_algorithmic=(fb + wb) / algo[key])
        lines.append(f"| `{name[:80]}` | {fetch[name][1]} | {fetch[name][0]:.0f} | "
                     f"{write[name][0]:.0f} | {fb / 1e9:.3f} | {wb / 1e9:.3f} | "
                     f"{(fb + wb) / 1e9:.3f} |")
    if algo:
        lines += ["", "Algorithmic bytes per launch at this shape (merge: (3 d + 3) x 4 B per "
                  "row; delta: 2 d x 2 B + 4 B per row): "
                  + "; ".join(f"`{k}` {v / 1e9:.3f} GB (measured / algorithmic = "
                              f"{data['kernels'][k]['traffic_over_algorithmic']:.3f})"
                              for k, v in algo.items() if k in data["kernels"]) + "."]
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
    "SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_VALU_FMA_F32 SQ_INSTS_VALU_ADD_F32 SQ_INSTS_VALU_MUL_F32 "
    "SQ_INSTS_VALU_CVT SQ_INSTS_VALU_INT32 SQ_VALU_MFMA_COEXEC_CYCLES SQ_BUSY_CU_CYCLES",
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
           "-o run -- python3 <repo>/bench.py {a}")
    lines = [f"# SQ counters per kernel: {workload} workload", "",
             f"Commands ({len(SQ_PASSES)} passes, at most 8 SQ counters each, on one MI355X):",
             "", "```"]
    lines += [cmd.format(c=c, i=i + 1, a=_profiled_args(workload)) for i, c in enumerate(SQ_PASSES)]
    lines += ["python3 <repo>/bench.py --sq-summary <out>", "```", "",
              "Cycle counters are summed over the chip (`SQ_BUSY_CU_CYCLES` over 256 CUs, "
              "`SQ_VALU_MFMA_BUSY_CYCLES` over 1024 SIMDs; the latter counts the clocks each "
              "MFMA occupies: 16 for a 16x16x32 bf16 tile, 32 for a 32x32x16 one).  Effective "
              "clock = "
              "`SQ_BUSY_CU_CYCLES` / 256 / kernel duration.  VALU instructions per SIMD-cycle = "
              "`SQ_INSTS_VALU` / (4 `SQ_BUSY_CU_CYCLES`); waves per SIMD = `SQ_WAVE_CYCLES` / "
              "`SQ_BUSY_CU_CYCLES` (`SQ_WAVE_CYCLES` counts in units of 4 cycles).  VALU busy = "
              "`SQ_ACTIVE_INST_VALU` / `SQ_BUSY_CU_CYCLES` (quad-cycles over the chip's 4 "
              "SIMDs per CU: the share of SIMD cycles a VALU instruction occupies, the "
              "vendor's VALUBusy); VALU cycles per instruction = 4 `SQ_ACTIVE_INST_VALU` / "
              "`SQ_INSTS_VALU` (4 for a stream of full-rate wave64 instructions).", "",
              "| kernel | duration (ms, under counters) | effective clock (GHz) | MFMA busy | LDS busy "
              "| LDS bank-conflict share | VALU / MFMA | LDS / MFMA | SALU / MFMA | wait-any / wave cycles "
              "| VALU instr per SIMD-cycle | waves per SIMD | VALU busy |",
              "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    mix_lines = ["", "VALU instruction mix (shares of `SQ_INSTS_VALU`) and VALU cycles per "
                 "instruction:", "",
                 "| kernel | transcendental f32 | FMA f32 | add f32 | mul f32 | convert | int32 | "
                 "other | VALU cycles per instruction | MFMA + VALU co-issue / MFMA busy |",
                 "|---|---|---|---|---|---|---|---|---|---|"]
    logged = _logged_hashes(*[os.path.join(root, f"cnt_{i + 1}.log")
                              for i in range(len(SQ_PASSES))]) or {}
    data = {"workload": workload, "kernels": {}}
    for key, c in agg.items():
        m = {k: sum(v) / len(v) for k, v in c.items()}
        t = sum(dur[key].values()) / len(dur[key])
        busy = m["SQ_BUSY_CU_CYCLES"]
        valu_busy = m["SQ_ACTIVE_INST_VALU"] / busy
        data["kernels"][key] = {
            "name": KERNELS[key][0], "source_hash": logged.get(key),
            "mfma_busy": round(m["SQ_VALU_MFMA_BUSY_CYCLES"] / (4 * busy), 4),
            "effective_clock_ghz": round(busy / n_cu / t / 1e9, 3),
            "lds_busy": round(m["SQ_LDS_IDX_ACTIVE"] / busy, 4),
            "valu_busy": round(valu_busy, 4)}
        if "SQ_INSTS_VALU_TRANS_F32" in m:
            n = max(m["SQ_INSTS_VALU"], 1.0)
            parts = [m[c] / n for c in ("SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_VALU_FMA_F32",
                                        "SQ_INSTS_VALU_ADD_F32", "SQ_INSTS_VALU_MUL_F32",
                                        "SQ_INSTS_VALU_CVT", "SQ_INSTS_VALU_INT32")]
            cpi = 4 * m["SQ_ACTIVE_INST_VALU"] / max(n, 1)
            coex = m["SQ_VALU_MFMA_COEXEC_CYCLES"] / max(m["SQ_VALU_MFMA_BUSY_CYCLES"] / 4, 1)
            data["kernels"][key].update(valu_trans_share=round(parts[0], 4),
                                        valu_cycles_per_instr=round(cpi, 3))
            mix_lines.append(f"| `{KERNELS[key][0]}` | " + " | ".join(f"{x:.3f}" for x in parts)
                             + f" | {max(0.0, 1 - sum(parts)):.3f} | {cpi:.2f} | {coex:.3f} |")
        per_mfma = (lambda c: f"{m[c] / m['SQ_INSTS_MFMA']:.2f}" if m["SQ_INSTS_MFMA"] > 0
                    else "-")
        lines.append(
            f"| `{KERNELS[key][0]}` | {t * 1e3:.2f} | {busy / n_cu / t / 1e9:.2f} | "
            f"{m['SQ_VALU_MFMA_BUSY_CYCLES'] / (4 * busy):.3f} | "
            f"{m['SQ_LDS_IDX_ACTIVE'] / busy:.3f} | "
            f"{m['SQ_LDS_BANK_CONFLICT'] / max(m['SQ_LDS_IDX_ACTIVE'], 1):.3f} | "
            f"{per_mfma('SQ_INSTS_VALU')} | {per_mfma('SQ_INSTS_LDS')} | "
            f"{per_mfma('SQ_INSTS_SALU')} | "
            f"{m['SQ_WAIT_ANY'] / m['SQ_WAVE_CYCLES']:.3f} | "
            f"{m['SQ_INSTS_VALU'] / (4 * busy):.3f} | {m['SQ_WAVE_CYCLES'] / busy:.2f} | "
            f"{valu_busy:.3f} |")
    if len(mix_lines) > 5:
        lines += mix_lines
    lines += ["", "Read by `bench.py`, which attaches a kernel's figures to its `roofline` only "
              "while the `source_hash` printed by the profiled runs matches the current "
              "sources:", "", "```json", json.dumps(data, indent=1), "```", ""]
    return "\n".join(lines)


def _problem_of(w, bounds=None):
    """ra_problem_t of a workload for the host-only calls (pair counts): a packed
    workload gets a stand-in boundary address, which these calls never read."""
    from ring_context_parallelism_amd import ra
    kw = {} if bounds is None else dict(seg_bounds=1 << 20, seg_count=int(bounds.shape[1]))
    return ra.make_problem(batch=w.batch, heads_q=w.heads_q, heads_kv=w.heads_kv,
                           head_dim=w.head_dim, head_dim_padded=w.head_dim_padded,
                           seq_total=w.seq_total, world=w.world, layout=w.layout,
                           causal=w.causal, dtype=w.dtype, **kw)


def _bench_line(log):
    if os.path.exists(log):
        for line in open(log):
            if line.startswith("{") and '"roofline"' in line:
                return json.loads(line)
    return None


def trace_summary(run_dir, workload):
    """Kernel durations from a --kernel-trace run, with the algorithmic FLOP rate of each
    attention kernel (forward 4d, dK/dV 8d, dQ 2d per visible pair and head) over the
    launches of the timed steps only: the warmup steps before them and the forward's
    per-step timing pass after them are left out."""
    import numpy as np

    from ring_context_parallelism_amd import ra
    from ring_context_parallelism_amd.workloads import WORKLOADS, document_bounds
    w = WORKLOADS[workload]
    bounds = document_bounds(w) if w.docs else None
    steps = step_flops(w, _problem_of(w, bounds), ra, bounds)
    n_live = len(steps)
    pairs = sum(st["visible_pairs_per_head"] * w.batch * w.heads_q for st in steps) / n_live
    per_pair = {"fwd_kernel": 4, "fwd_kernel_f32": 4, "bwd_dkdv_kernel": 8, "bwd_dq_kernel": 2}
    peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else F32_PEAK_TFLOPS
    log = run_dir.rstrip("/") + ".log"
    _check_workload(log, workload)
    bench_line = _bench_line(log)
    if bench_line is None:
        raise SystemExit(f"bench.py: no bench line in {log}")
    warm, timed = int(bench_line["warmup"]), int(bench_line["steps"])
    launches = {}
    for r in csv.DictReader(open(os.path.join(run_dir, "run_kernel_trace.csv"))):
        t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        launches.setdefault(r["Kernel_Name"], []).append((t0, (t1 - t0) * 1e-6))
    total = sum(d for xs in launches.values() for _, d in xs)
    lines = [f"# Kernel durations: {workload} workload ({w.batch} x {w.heads_q}/{w.heads_kv} heads "
             f"x d{w.head_dim}, S={w.seq_total}, {w.layout} p={w.world}, rank {w.rank}, {w.dtype}"
             f"{', packed documents' if w.docs else ''})",
             "", "Command (run from /tmp on one MI355X):", "", "```",
             "cd /tmp && timeout -k 10 300 rocprofv3 --kernel-trace --stats --output-format csv "
             "-d <out>/prof_" + workload + " -o run -- python3 <repo>/bench.py --workload "
             f"{workload} --steps {timed} --warmup {warm} --no-cpu-baseline --no-configs > "
             f"<out>/prof_{workload}.log",
             f"python3 <repo>/bench.py --workload {workload} --trace-summary <out>/prof_{workload}",
             "```", "",
             f"{n_live} live ring steps per bench step; {pairs:.4g} visible (query, key) pairs "
             "per launch (mean over the live steps) summed over batch and heads.  Algorithmic "
             "FLOP per launch: forward 4d, dK/dV kernel 8d (S, dP, dV, dK), dQ kernel 2d (its "
             "recomputation of S and dP is not counted) per pair.  The attention kernels' "
             f"figures cover the {timed} timed steps only ({timed * n_live} launches each): the "
             f"{warm} warmup step(s) before them and the forward's per-step timing pass after "
             "them are left out.  Other kernels: every launch.", "",
             "| kernel | launches (all) | timed launches | mean (ms) | median (ms) | min (ms) | "
             "max (ms) | share of GPU time | algorithmic TFLOP/s (mean) | of peak |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    data = {"workload": workload, "kernels": {}}
    for name, xs in sorted(launches.items(), key=lambda kv: -sum(d for _, d in kv[1])):
        durs = [d for _, d in sorted(xs)]
        key = next((k for k in per_pair if KERNELS[k][0] in name), None)
        sel = durs[warm * n_live:(warm + timed) * n_live] if key else durs
        if not sel:
            continue
        mean, med = float(np.mean(sel)), float(np.median(sel))
        rate = frac = ""
        if key:
            tf = per_pair[key] * w.head_dim * pairs / (mean * 1e-3) / 1e12
            rate, frac = f"{tf:.1f}", f"{100 * tf / peak:.1f}%"
            data["kernels"][key] = {"name": name, "timed_launches": len(sel), "mean_ms": mean,
                                    "median_ms": med, "tflops": tf, "frac": tf / peak}
        lines.append(f"| `{name[:90]}` | {len(durs)} | {len(sel)} | {mean:.3f} | {med:.3f} | "
                     f"{min(sel):.3f} | {max(sel):.3f} | {100 * sum(durs) / total:.2f}% | "
                     f"{rate} | {frac} |")
    rf = bench_line["roofline"]
    lines += ["", "The bench line printed by the same profiled command (HIP events on the "
              f"launch stream, the same timed steps): {bench_line['value']:.1f} TFLOP/s per "
              f"step, forward {bench_line['fwd']['pct_peak']:.1f}% of peak"
              + (f", backward {bench_line['bwd']['pct_peak']:.1f}%" if "bwd" in bench_line
                 else "")
              + f"; roofline kernel `{rf['kernel']}` ({rf['bound']}-bound) "
              f"{rf['avg_launch_ms']:.3f} ms per launch, {rf['achieved']:.1f} {rf['unit']}, "
              f"frac {rf['frac']:.4f}.", "", "```json", json.dumps(data, indent=1), "```", ""]
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
    return {f: k[f] for f in ("mfma_busy", "effective_clock_ghz", "lds_busy", "valu_busy")
            if f in k}


def roofline(flop, pairs, launch_ms, mfma_peak, alu_slots):
    """The roof a kernel sits closer to: the matrix cores (its algorithmic FLOP against
    the dense MFMA peak of its dtype) or the vector ALU (alu_slots full-rate issue slots
    per visible pair against ALU_PEAK_TOPS; small head dims, where the per-score softmax
    work dominates).  The other fraction is reported alongside."""
    achieved = flop / (launch_ms * 1e-3) / 1e12
    alu_ops = alu_slots * pairs
    alu_achieved = alu_ops / (launch_ms * 1e-3) / 1e12
    if alu_achieved / ALU_PEAK_TOPS > achieved / mfma_peak:
        return {"bound": "alu", "achieved": round(alu_achieved, 3),
                "peak": round(ALU_PEAK_TOPS, 2), "unit": "TOP/s",
                "frac": round(alu_achieved / ALU_PEAK_TOPS, 4), "ops_per_launch": alu_ops,
                "slots_per_pair": alu_slots, "mfma_frac": round(achieved / mfma_peak, 4)}
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


def _blas_name():
    try:
        from threadpoolctl import threadpool_info
        return ",".join(sorted({p.get("internal_api", "?") for p in threadpool_info()})) or "?"
    except Exception:  # pragma: no cover - reporting only
        return "unknown"


def _pairs_of_rows(w, rows, bounds):
    """Exact visible (query, key) pairs of the given global query rows, per head, summed
    over the batch (the oracle's own arithmetic is not used: this only prices its work)."""
    import numpy as np
    if bounds is None:
        per = float(np.sum(rows + 1)) if w.causal else float(rows.size * w.seq_total)
        return per * w.batch
    pairs = 0.0
    for e in bounds:
        e = np.asarray(e, dtype=np.int64)
        k = np.searchsorted(e, rows, side="right") - 1
        live = rows < e[-1]
        start, end = e[np.clip(k, 0, e.size - 1)], e[np.clip(k + 1, 0, e.size - 1)]
        cnt = np.where(w.causal, rows - start + 1, end - start)
        pairs += float(np.sum(np.where(live, cnt, 0)))
    return pairs


def cpu_baseline(w, arrays, target_s, full_bwd_max_s=120.0):
    """The oracle, as it is, on a bounded sample of the same share (fp64, host cores).

    The oracle's rows are spread over a pool of threads, one BLAS thread each
    (oracle.rows).  Forward workloads: a sample of head 0's rows, grown until it takes
    about 0.6 x target_s.  Backward workloads: the whole of head 0 forward + backward
    (dQ of every row, dK and dV of every key) when a calibration run projects it
    within full_bwd_max_s, else a row sample; then O and LSE on a row sample.
    Returns (record, reference values for sample_parity)."""
    import numpy as np

    import oracle
    from oracle.rows import attention_bwd_rows, attention_fwd_rows, default_workers
    workers = default_workers()
    rows_all = oracle.positions(w.layout, w.seq_total, w.world, w.rank)
    bounds = None if arrays.get("bounds") is None else [list(map(int, e)) for e in arrays["bounds"]]
    rng = np.random.default_rng(1234)
    d = w.head_dim
    total_s, flop, what = 0.0, 0.0, []
    ref = {"head": 0}

    def fwd(t_idx):
        t0 = time.perf_counter()
        O, LSE = attention_fwd_rows(arrays["q"], arrays["k"], arrays["v"], rows_all[t_idx],
                                    w.causal, heads=[0], bounds=bounds, workers=workers)
        return (O, LSE), time.perf_counter() - t0

    def bwd(t_idx):
        rows = rows_all[t_idx]
        t0 = time.perf_counter()
        g = attention_bwd_rows(arrays["q"], arrays["k"], arrays["v"],
                               arrays["do"][:, :1][:, :, rows], rows, w.causal, heads=[0],
                               bounds=bounds, workers=workers)
        return g, time.perf_counter() - t0

    fwd_share = 0.6
    if w.backward:
        # calibration sample, then the whole head when it fits the time bound
        b_idx = np.sort(rng.choice(rows_all.size, size=min(1024, rows_all.size), replace=False))
        grads, dt = bwd(b_idx)
        projected = dt * _pairs_of_rows(w, rows_all, bounds) / max(
            _pairs_of_rows(w, rows_all[b_idx], bounds), 1.0)
        whole = projected <= full_bwd_max_s
        if whole:
            b_idx = np.arange(rows_all.size)
            grads, dt = bwd(b_idx)
        total_s += dt
        flop += 14.0 * d * _pairs_of_rows(w, rows_all[b_idx], bounds)
        what.append(f"{'every query row' if whole else f'{b_idx.size} query rows'} of head 0, "
                    f"forward + backward ({dt:.1f} s)")
        ref.update(bwd_idx=b_idx, dQ=grads[0], dK=grads[1] if whole else None,
                   dV=grads[2] if whole else None)
        fwd_share = 0.2
    n = 64
    while True:
        t_idx = np.sort(rng.choice(rows_all.size, size=min(n, rows_all.size), replace=False))
        (O, LSE), dt = fwd(t_idx)
        budget = fwd_share * target_s
        if dt >= budget or n >= rows_all.size:
            break
        n = int(min(rows_all.size, n * min(16.0, max(2.0, budget / max(dt, 1e-3)))))
    total_s += dt
    flop += 4.0 * d * _pairs_of_rows(w, rows_all[t_idx], bounds)
    what.append(f"{t_idx.size} query rows of head 0, forward ({dt:.1f} s)")
    ref.update(fwd_idx=t_idx, O=O, LSE=LSE)
    host_cores = len(os.sched_getaffinity(0))
    rec = {"value": flop / total_s / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
           "sample": "; ".join(what) + f" in fp64 (batch {w.batch}), {flop:.3e} algorithmic "
                     f"FLOP in {total_s:.1f} s",
           "pool": f"{workers} worker threads, 1 BLAS thread each ({_blas_name()})",
           "host_cores": host_cores, "seconds": total_s}
    return rec, ref


def sample_parity(w, ref, out, lse, dq=None, dks=None, dvs=None):
    """The timed run's outputs against the oracle's: O and LSE on the sampled rows of
    head 0; dQ on the rows the oracle's backward covered; dK and dV of every key of
    every chunk for head 0's KV head when the oracle ran the whole head."""
    import numpy as np
    d = w.head_dim

    def cmp(got, want):
        err = np.abs(got - want)
        den = np.linalg.norm(want)
        return {"max_abs": float(err.max()), "mean_abs": float(err.mean()),
                "rel_fro": float(np.linalg.norm(got - want) / den) if den > 0 else 0.0}

    ti = torch_index(ref["fwd_idx"], out.device)
    res = {"rows": int(ref["fwd_idx"].size), "head": 0}
    res["o"] = cmp(out[:, :1][:, :, ti].float().cpu().numpy()[..., :d], ref["O"])
    lg = lse[:, :1][:, :, ti].cpu().numpy()
    LSE = ref["LSE"]
    fin = np.isfinite(LSE)
    res["lse_max_abs"] = float(np.abs(lg[fin] - LSE[fin]).max()) if fin.any() else 0.0
    res["lse_inf_rows_match"] = bool(np.array_equal(np.isneginf(lg), np.isneginf(LSE)))
    if ref.get("dQ") is not None and dq is not None:
        bi = torch_index(ref["bwd_idx"], dq.device)
        res["bwd_rows"] = int(ref["bwd_idx"].size)
        res["dq"] = cmp(dq[:, :1][:, :, bi].cpu().numpy()[..., :d], ref["dQ"])
    if ref.get("dK") is not None and dks is not None:
        import oracle
        g = 0  # KV head of query head 0
        gk = [dks[c][:, g].cpu().numpy()[..., :d] for c in range(w.world)]
        gv = [dvs[c][:, g].cpu().numpy()[..., :d] for c in range(w.world)]
        pos = [oracle.positions(w.layout, w.seq_total, w.world, c) for c in range(w.world)]
        res["dk"] = cmp(np.concatenate(gk, axis=1),
                        np.concatenate([ref["dK"][:, g][:, p] for p in pos], axis=1))
        res["dv"] = cmp(np.concatenate(gv, axis=1),
                        np.concatenate([ref["dV"][:, g][:, p] for p in pos], axis=1))
        res["dkdv_keys"] = int(w.seq_total)
    tol = (2e-2, 2e-3, 1e-2) if w.dtype == "bf16" else (1e-5, 1e-5, 1e-5)
    ok = all(res[k]["max_abs"] <= tol[0] and res[k]["mean_abs"] <= tol[1]
             and res[k]["rel_fro"] <= tol[2] for k in ("o", "dq", "dk", "dv") if k in res)
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


def aux_summary(path):
    """Markdown table of a saved `bench.py --aux` line (the helpers' HIP-event timings)."""
    rec = json.loads([ln for ln in open(path) if ln.strip().startswith("{")][-1])
    lines = ["# HBM-bound helper kernels: standalone LSE merge and backward delta", "",
             "Commands (one MI355X):", "", "```", "python3 <repo>/bench.py --aux > <out>/aux.json",
             "python3 <repo>/bench.py --aux-summary <out>/aux.json", "```", "",
             "Each kernel is launched 50 times back to back after one warm-up launch; HIP events "
             "on the launch stream give the average duration.  Algorithmic bytes per row: the "
             "merge reads both fp32 partials and both LSEs and writes the accumulator and its "
             "LSE, (3 d + 3) x 4 B; delta reads O and dO in bf16 (2 d x 2 B) and writes 4 B.", "",
             f"| kernel | shape | bytes per launch | ms | achieved (GB/s) | fraction of {HBM_PEAK_GBS:.0f} GB/s |",
             "|---|---|---|---|---|---|"]
    for k in rec["kernels"]:
        lines.append(f"| `{k['kernel']}` | {k['shape']} | {k['bytes']} | {k['ms']} | {k['achieved']} | "
                     f"{k['frac']} |")
    c = rec.get("copy_reference")
    if c:
        lines += ["", f"Reference on the same box: a plain 1 GiB device-to-device copy through torch "
                      f"moves {c['bytes']} bytes (read + write) in {c['ms']} ms = {c['achieved']} GB/s "
                      f"({c['frac']} of {HBM_PEAK_GBS:.0f} GB/s).  The llama_share merge (203 MB) may "
                      f"partly hit the 256 MB last-level cache on repeated launches; the zigzag_fwdbwd "
                      f"shapes (0.5-1.6 GB) do not.  FETCH_SIZE / WRITE_SIZE counts for the zig-zag "
                      f"shapes are in pmc_traffic_hbm_helpers.md."]
    return "\n".join(lines)


def aux_bench(reps=50, only=None):
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

    for name, (rows, d) in AUX_SHAPES.items():
        if only is not None and name != only:
            continue
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
    if only is None:
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


def rows_parity(o, O, lse, LSE, dq=None, dQ=None):
    """bf16 parity of sampled rows: O (and dQ) element by element against the oracle at
    max abs 2e-2, mean abs 2e-3 and rel_fro 1e-2; LSE at abs 1e-3 on the rows the
    oracle finds finite, and -inf (rows that see no key, such as padding) on exactly
    the same rows."""
    import numpy as np

    def errs(a, b):
        e = np.abs(a - b)
        nb = np.linalg.norm(b)
        return {"max_abs": float(e.max()), "mean_abs": float(e.mean()),
                "rel_fro": float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))}

    fin = np.isfinite(LSE)
    par = {"o": errs(o, O),
           "lse_max_abs": float(np.abs(lse[fin] - LSE[fin]).max()) if fin.any() else 0.0,
           "lse_inf_rows_match": bool(np.array_equal(np.isneginf(lse), np.isneginf(LSE)))}
    keys = ["o"]
    if dq is not None:
        par["dq"] = errs(dq, dQ)
        keys.append("dq")
    par["pass"] = bool(all(par[k]["max_abs"] <= 2e-2 and par[k]["mean_abs"] <= 2e-3
                           and par[k]["rel_fro"] <= 1e-2 for k in keys)
                       and par["lse_max_abs"] <= 1e-3 and par["lse_inf_rows_match"])
    return par


def packed_config(name, reps, stream):
    """The packed-document share: ra_ring_fwd and ra_ring_bwd timed with HIP events over
    `reps` passes after the default warmup, with FLOP counted inside documents only;
    each live forward step timed on its own; and O, LSE and dQ on sampled rows and heads
    against the oracle (a row's dQ depends on that row alone)."""
    import numpy as np
    import torch

    from oracle.rows import attention_bwd_rows, attention_fwd_rows
    from ring_context_parallelism_amd import ra, staging
    from ring_context_parallelism_amd.workloads import WORKLOADS, generate
    w = WORKLOADS[name]
    print(f"[bench] config {name}: generating inputs", file=sys.stderr, flush=True)
    arrays = generate(w)
    bounds = arrays["bounds"]
    dev = torch.device("cuda:0")
    share = staging.stage(w, arrays, dev)
    prob = share.prob
    steps = step_flops(w, prob, ra, bounds)
    L, D, d = w.chunk_len, w.head_dim_padded, w.head_dim
    f32 = torch.float32
    out = torch.empty((w.batch, w.heads_q, L, D), dtype=staging.torch_dtype(w), device=dev)
    lse = torch.empty((w.batch, w.heads_q, L), dtype=f32, device=dev)
    ws = torch.empty(ra.ra_ring_workspace_size(prob) // 4, dtype=f32, device=dev)
    dq = torch.empty((w.batch, w.heads_q, L, D), dtype=f32, device=dev)
    dks = [torch.empty((w.batch, w.heads_kv, L, D), dtype=f32, device=dev) for _ in range(w.world)]
    dvs = [torch.empty_like(dks[0]) for _ in range(w.world)]
    wsb = torch.empty(ra.ra_ring_bwd_workspace_size(prob) // 4, dtype=f32, device=dev)

    def fwd():
        ra.ra_ring_fwd(prob, w.rank, share.q, share.k_chunks, share.v_chunks, out, lse, ws,
                       stream=stream)

    def bwd():
        ra.ra_ring_bwd(prob, w.rank, share.q, share.k_chunks, share.v_chunks, out, share.do, lse,
                       dq, dks, dvs, wsb, stream=stream)

    def run():
        fwd()
        bwd()

    _warm(run, stream)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for e in ev:
        e[0].record(stream)
        fwd()
        e[1].record(stream)
        bwd()
        e[2].record(stream)
    torch.cuda.synchronize()
    fms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    bms = np.array([e[1].elapsed_time(e[2]) for e in ev])
    fflop = sum(st["fwd_flop"] for st in steps)
    bflop = sum(st["bwd_flop"] for st in steps)
    peak = BF16_PEAK_TFLOPS
    ftf = fflop / (float(np.mean(fms)) * 1e-3) / 1e12
    btf = bflop / (float(np.mean(bms)) * 1e-3) / 1e12
    step_tf = (fflop + bflop) / (float(np.mean(fms + bms)) * 1e-3) / 1e12
    step_ms = time_fwd_steps(ra, prob, w, share, steps, ws, stream, max(3, reps))
    per_step = [dict(step=st["step"], chunk=st["chunk"],
                     visible_pairs_per_head=st["visible_pairs_per_head"],
                     fwd_ms=float(np.mean(sm)), fwd_ms_median=float(np.median(sm)),
                     fwd_pct_peak=100.0 * st["fwd_flop"] / (float(np.mean(sm)) * 1e-3) / 1e12 / peak)
                for st, sm in zip(steps, step_ms)]
    # parity on sampled rows (tile edges + random) of sampled heads
    run()
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed)
    t_idx = np.unique(np.concatenate([
        np.array([0, 1, 127, 128, L // 2, L - 129, L - 128, L - 1]),
        rng.choice(L, size=48, replace=False)]))
    heads = sorted({0, w.heads_q - 1, *rng.choice(w.heads_q, size=2, replace=False).tolist()})
    rows = share.rows[t_idx]
    O, LSE = attention_fwd_rows(arrays["q"], arrays["k"], arrays["v"], rows, w.causal,
                                heads=heads, bounds=bounds)
    dQ, _, _ = attention_bwd_rows(arrays["q"], arrays["k"], arrays["v"],
                                  arrays["do"][:, heads][:, :, rows], rows, w.causal,
                                  heads=heads, bounds=bounds)
    ti = torch.from_numpy(t_idx).to(dev)
    par = {"rows": int(t_idx.size), "heads": heads,
           **rows_parity(out[:, heads][:, :, ti].float().cpu().numpy()[..., :d], O,
                         lse[:, heads][:, :, ti].cpu().numpy(), LSE,
                         dq[:, heads][:, :, ti].cpu().numpy()[..., :d], dQ)}
    rec = {"workload": name, "dtype": w.dtype, "batch": w.batch, "heads_q": w.heads_q,
           "heads_kv": w.heads_kv, "head_dim": w.head_dim, "seq_total": w.seq_total,
           "world": w.world, "layout": w.layout, "rank": w.rank, "causal": w.causal,
           "documents": int(bounds.shape[-1] - 1), "passes": "fwd+bwd", "reps": reps,
           "fwd_ms": round(float(np.mean(fms)), 4), "bwd_ms": round(float(np.mean(bms)), 4),
           "fwd_flop": fflop, "bwd_flop": bflop, "fwd_tflops": round(ftf, 3),
           "bwd_tflops": round(btf, 3), "fwd_pct_peak": round(100.0 * ftf / peak, 2),
           "bwd_pct_peak": round(100.0 * btf / peak, 2), "step_tflops": round(step_tf, 3),
           "peak": peak, "per_step": per_step, "parity": par}
    del share, arrays, out, lse, ws, dq, dks, dvs, wsb
    torch.cuda.empty_cache()
    return rec


def _warm(fn, stream):
    """Untimed warmup: at least 2 calls and about WARM_SECONDS of work."""
    import torch
    fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    per = max(time.perf_counter() - t0, 1e-6)
    for _ in range(min(5000, int(WARM_SECONDS / per))):
        fn()
    torch.cuda.synchronize()


def other_config(name, reps, stream):
    """One forward-only workload: ra_ring_fwd timed with HIP events over `reps` passes
    after the default warmup, each live step timed on its own, and the outputs on
    sampled rows and heads against the oracle (thread pool, fp64)."""
    import numpy as np
    import torch

    from oracle.rows import attention_fwd_rows
    from ring_context_parallelism_amd import ra, staging
    from ring_context_parallelism_amd.workloads import WORKLOADS, generate
    w = WORKLOADS[name]
    print(f"[bench] config {name}: generating inputs", file=sys.stderr, flush=True)
    arrays = generate(w)
    dev = torch.device("cuda:0")
    share = staging.stage(w, arrays, dev)
    prob = share.prob
    steps = step_flops(w, prob, ra)
    L, D = w.chunk_len, w.head_dim_padded
    out = torch.empty((w.batch, w.heads_q, L, D), dtype=staging.torch_dtype(w), device=dev)
    lse = torch.empty((w.batch, w.heads_q, L), dtype=torch.float32, device=dev)
    ws = torch.empty(ra.ra_ring_workspace_size(prob) // 4, dtype=torch.float32, device=dev)

    def run():
        ra.ra_ring_fwd(prob, w.rank, share.q, share.k_chunks, share.v_chunks, out, lse, ws,
                       stream=stream)

    _warm(run, stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    flop = sum(st["fwd_flop"] for st in steps)
    peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else F32_PEAK_TFLOPS
    tf = flop / (float(np.mean(ms)) * 1e-3) / 1e12
    step_ms = time_fwd_steps(ra, prob, w, share, steps, ws, stream, max(3, reps))
    per_step = [dict(step=st["step"], chunk=st["chunk"],
                     visible_pairs_per_head=st["visible_pairs_per_head"],
                     fwd_ms=float(np.mean(sm)), fwd_ms_median=float(np.median(sm)),
                     fwd_tflops=st["fwd_flop"] / (float(np.mean(sm)) * 1e-3) / 1e12,
                     fwd_pct_peak=100.0 * st["fwd_flop"] / (float(np.mean(sm)) * 1e-3) / 1e12 / peak)
                for st, sm in zip(steps, step_ms)]
    # parity: sampled rows (tile edges + random) of sampled heads, or everything when small
    run()
    torch.cuda.synchronize()
    small = L * w.heads_q * w.batch <= 4096
    rng = np.random.default_rng(w.seed)
    t_idx = np.arange(L) if small else np.unique(np.concatenate([
        np.array([0, 1, 63, 64, 127, 128, 255, 256, L // 2, L - 129, L - 128, L - 2, L - 1]),
        rng.choice(L, size=min(48, L), replace=False)]))
    t_idx = t_idx[(t_idx >= 0) & (t_idx < L)]
    heads = list(range(w.heads_q)) if small else sorted({0, w.heads_q - 1, *rng.choice(
        w.heads_q, size=min(2, w.heads_q), replace=False).tolist()})
    rows = share.rows[t_idx]
    O, LSE = attention_fwd_rows(arrays["q"], arrays["k"], arrays["v"], rows, w.causal,
                                heads=heads)
    ti = torch.from_numpy(t_idx).to(dev)
    got = out[:, heads][:, :, ti].float().cpu().numpy()[..., :w.head_dim]
    lg = lse[:, heads][:, :, ti].cpu().numpy()
    err = np.abs(got - O)
    tol = (2e-2, 2e-3, 1e-2) if w.dtype == "bf16" else (1e-5, 1e-5, 1e-5)
    par = {"rows": int(t_idx.size), "heads": heads, "max_abs": float(err.max()),
           "mean_abs": float(err.mean()),
           "rel_fro": float(np.linalg.norm(got - O) / np.linalg.norm(O)),
           "lse_max_abs": float(np.abs(lg - LSE).max())}
    par["pass"] = bool(par["max_abs"] <= tol[0] and par["mean_abs"] <= tol[1]
                       and par["rel_fro"] <= tol[2] and par["lse_max_abs"] <= 1e-3)
    rec = {"workload": name, "dtype": w.dtype, "batch": w.batch, "heads_q": w.heads_q,
           "heads_kv": w.heads_kv, "head_dim": w.head_dim, "seq_total": w.seq_total,
           "world": w.world, "layout": w.layout, "rank": w.rank, "causal": w.causal,
           "passes": "fwd", "reps": reps, "fwd_ms": round(float(np.mean(ms)), 4),
           "fwd_ms_median": round(float(np.median(ms)), 4), "flop": flop,
           "fwd_tflops": round(tf, 3), "pct_peak": round(100.0 * tf / peak, 2),
           "peak": peak, "per_step": per_step, "parity": par}
    del share, arrays, out, lse, ws
    torch.cuda.empty_cache()
    return rec


def main():
    args = parse()
    if args.aux:
        print("[bench] source hashes " + json.dumps({k: source_hash(f) for k, (_, f) in KERNELS.items()}),
              file=sys.stderr, flush=True)
        aux_bench(only=args.aux_shape)
        return
    if args.aux_summary:
        print(aux_summary(args.aux_summary))
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
    if w.backward and len(steps) != w.world:
        raise SystemExit("bench.py: the backward step is timed on workloads whose every KV "
                         "chunk has a live step (each chunk's dK/dV is stored by its step)")

    def one_step(ev):
        ev[0].record(stream)
        ra.ra_ring_fwd(prob, w.rank, share.q, share.k_chunks, share.v_chunks, out, lse, ws,
                       stream=stream)
        ev[1].record(stream)
        if not w.backward:
            return
        # the sequence of ra_ring_bwd, split so that each kernel has its own events:
        # delta, then per live step the dK/dV kernel (storing that chunk's gradients)
        # and the dQ kernel (storing dq on the first step, adding on the others)
        ra.ra_bwd_delta(prob, out, share.do, delta, stream=stream)
        ev[2].record(stream)
        for i, st in enumerate(steps):
            c = st["chunk"]
            args_ = (prob, share.q, w.rank, share.k_chunks[c], share.v_chunks[c], c, share.do, lse,
                     delta)
            ra.ra_block_attn_bwd_dkdv(*args_, dks[c], dvs[c], mode=ra.RA_WRITE, stream=stream)
            ev[3 + 2 * i].record(stream)
            ra.ra_block_attn_bwd_dq(*args_, dq, mode=ra.RA_WRITE if i == 0 else ra.RA_MERGE,
                                    stream=stream)
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
        # the backward step: delta, then every live step
        bwd_ms_total = float(np.mean([e[1].elapsed_time(e[-1]) for e in events]))
        kernels_ms = float(np.mean([e[2].elapsed_time(e[-1]) for e in events]))
        aux_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
        bwd_tflops = bwd_flop / (bwd_ms_total * 1e-3) / 1e12
        res["bwd"] = {"ms": round(bwd_ms_total, 4), "tflops": round(bwd_tflops, 3),
                      "pct_peak": round(100.0 * bwd_tflops / peak, 2), "flop": bwd_flop,
                      "delta_ms": round(aux_ms, 4),
                      "step_kernels_pct_peak": round(
                          100.0 * bwd_flop / (kernels_ms * 1e-3) / 1e12 / peak, 2)}
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
    res["roofline"] = roofline(per_launch_flop, sum(pairs_bh) / len(steps), launch_ms, peak,
                               ALU_SLOTS_PER_PAIR[name])
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
        if w.backward:
            res["parity"] = sample_parity(w, ref, out, lse, dq, dks, dvs)
        else:
            res["parity"] = sample_parity(w, ref, out, lse)
    if not args.no_configs and args.workload == DEFAULT_WORKLOAD and args.dtype is None:
        del share, arrays, out, lse, ws
        if w.backward:
            del delta, dq, dks, dvs
        torch.cuda.empty_cache()
        res["configs"] = [other_config(name, args.steps, stream)
                          for name in OTHER_CONFIGS]
        res["configs"].append(packed_config(PACKED_CONFIG, args.steps, stream))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
