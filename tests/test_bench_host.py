"""Host-side logic of bench.py (no GPU): the one-GPU guard and the parity record."""
import json
import os
import subprocess
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from ring_context_parallelism_amd.workloads import WORKLOADS  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _fake(w, rows, noise, grad_noise=0.0):
    """Outputs equal to a random 'oracle' reference plus noise, in the layouts the
    bench's parity check reads (head 0, chunk-local dK/dV)."""
    import oracle
    rng = np.random.default_rng(0)
    L, D, d, S = w.chunk_len, w.head_dim_padded, w.head_dim, w.seq_total
    t_idx = np.sort(rng.choice(L, size=rows, replace=False))
    O = rng.standard_normal((w.batch, 1, rows, d))
    LSE = rng.standard_normal((w.batch, 1, rows))
    dQ = rng.standard_normal((w.batch, 1, L, d))
    dK = rng.standard_normal((w.batch, w.heads_kv, S, d))
    dV = rng.standard_normal((w.batch, w.heads_kv, S, d))
    out = torch.zeros((w.batch, w.heads_q, L, D), dtype=torch.float32)
    lse = torch.zeros((w.batch, w.heads_q, L), dtype=torch.float32)
    dq = torch.zeros((w.batch, w.heads_q, L, D), dtype=torch.float32)
    dks = [torch.zeros((w.batch, w.heads_kv, L, D)) for _ in range(w.world)]
    dvs = [torch.zeros((w.batch, w.heads_kv, L, D)) for _ in range(w.world)]
    ti = torch.from_numpy(t_idx)
    out[:, :1, ti, :d] = torch.from_numpy(O + noise).float()
    lse[:, :1, ti] = torch.from_numpy(LSE).float()
    dq[:, :1, :, :d] = torch.from_numpy(dQ).float()
    for c in range(w.world):
        pos = oracle.positions(w.layout, S, w.world, c)
        dks[c][:, 0, :, :d] = torch.from_numpy(dK[:, 0][:, pos] + grad_noise).float()
        dvs[c][:, 0, :, :d] = torch.from_numpy(dV[:, 0][:, pos]).float()
    ref = {"head": 0, "fwd_idx": t_idx, "O": O, "LSE": LSE, "bwd_idx": np.arange(L), "dQ": dQ,
           "dK": dK, "dV": dV}
    return ref, out, lse, dq, dks, dvs


def test_sample_parity_passes_and_fails():
    w = WORKLOADS["zigzag_fwdbwd"].resized(seq_total=1024)
    ref, out, lse, dq, dks, dvs = _fake(w, 40, 0.0)
    res = bench.sample_parity(w, ref, out, lse, dq, dks, dvs)
    assert res["pass"] and res["o"]["max_abs"] < 1e-6 and res["dq"]["max_abs"] < 1e-6
    assert res["dk"]["max_abs"] < 1e-6 and res["dv"]["max_abs"] < 1e-6
    assert res["dkdv_keys"] == 1024 and res["bwd_rows"] == w.chunk_len
    ref, out, lse, dq, dks, dvs = _fake(w, 40, 0.1)  # a 0.1 error in O breaks the bf16 gate
    res = bench.sample_parity(w, ref, out, lse, dq, dks, dvs)
    assert not res["pass"] and res["o"]["max_abs"] > 0.05
    ref, out, lse, dq, dks, dvs = _fake(w, 40, 0.0, grad_noise=0.1)  # so does one in dK
    res = bench.sample_parity(w, ref, out, lse, dq, dks, dvs)
    assert not res["pass"] and res["dk"]["max_abs"] > 0.05
    # a forward-only record carries no gradient fields
    res = bench.sample_parity(w, {k: ref[k] for k in ("head", "fwd_idx", "O", "LSE")}, out, lse)
    assert res["pass"] and "dq" not in res and "dk" not in res


def test_counter_figures_only_for_the_sources_they_were_taken_on(tmp_path, monkeypatch):
    key = "bwd_dkdv_kernel"
    now = bench.source_hash(bench.KERNELS[key][1])
    hashes = {k: bench.source_hash(f) for k, (_, f) in bench.KERNELS.items()}
    log_a, log_b = tmp_path / "cnt_1.log", tmp_path / "cnt_2.log"
    log_a.write_text("noise\n[bench] source hashes " + json.dumps(hashes) + "\n")
    log_b.write_text("[bench] source hashes " + json.dumps(hashes) + "\n")
    assert bench._logged_hashes(str(log_a), str(log_b)) == hashes
    log_b.write_text("[bench] source hashes " + json.dumps({**hashes, key: "0" * 16}) + "\n")
    assert bench._logged_hashes(str(log_a), str(log_b)) is None  # runs disagree
    assert bench._logged_hashes(str(log_a), str(tmp_path / "missing.log")) is None

    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    for stored, expect in ((now, True), ("f" * 16, False), (None, False)):
        sq = {"workload": "zigzag_fwdbwd", "kernels": {key: {
            "name": "bwd_dkdv_kernel", "source_hash": stored, "mfma_busy": 0.5,
            "effective_clock_ghz": 2.0, "lds_busy": 0.4}}}
        pmc = {"workload": "zigzag_fwdbwd", "kernels": {key: {
            "name": "bwd_dkdv_kernel", "source_hash": stored, "traffic_bytes": 123.0}}}
        (tmp_path / "sq_counters_zigzag_fwdbwd.md").write_text(
            "# t\n\n```json\n" + json.dumps(sq) + "\n```\n")
        (tmp_path / "pmc_traffic_zigzag_fwdbwd.md").write_text(
            "# t\n\n```json\n" + json.dumps(pmc) + "\n```\n")
        got_c = bench.measured_counters("zigzag_fwdbwd", key)
        got_t = bench.measured_traffic("zigzag_fwdbwd", key)
        assert (got_c is not None) == expect and (got_t is not None) == expect
        assert bench.measured_counters("gqa_striped", key) is None  # other workload


def test_roofline_picks_the_closer_roof():
    # d = 128, bf16: 4 d = 512 FLOP per pair against the matrix peak -- MFMA-bound
    pairs = 3.436e10
    slots = bench.ALU_SLOTS_PER_PAIR["fwd_kernel"]
    r = bench.roofline(512 * pairs, pairs, 14.0, bench.BF16_PEAK_TFLOPS, slots)
    assert r["bound"] == "mfma" and abs(r["frac"] - 512 * pairs / 14e-3 / 1e12 / 2516.6) < 1e-4
    assert r["alu_frac"] < r["frac"]
    # d = 24: 96 FLOP per pair; the softmax's 4.5 vector issue slots per pair bind first
    pairs = 2.8125e10
    r = bench.roofline(96 * pairs, pairs, 4.6, bench.BF16_PEAK_TFLOPS, slots)
    assert r["bound"] == "alu" and r["unit"] == "TOP/s" and r["slots_per_pair"] == 4.5
    assert abs(r["achieved"] - 4.5 * pairs / 4.6e-3 / 1e12) < 1e-2
    assert abs(bench.ALU_PEAK_TOPS - 39.3216) < 1e-3 and r["mfma_frac"] < r["frac"]
    # every kernel the bench can name has a vector cost
    assert set(bench.ALU_SLOTS_PER_PAIR) == {"fwd_kernel", "fwd_kernel_f32", "bwd_dkdv_kernel",
                                              "bwd_dq_kernel"}


def test_cpu_baseline_covers_the_whole_head_when_it_fits():
    """At a small size the backward reference spans every row of head 0 (so dK and dV of
    every key can be compared); the record names the pool and the host's cores."""
    from ring_context_parallelism_amd.workloads import generate
    w = WORKLOADS["zigzag_fwdbwd"].resized(seq_total=512, heads_q=2, heads_kv=2)
    arrays = generate(w)
    rec, ref = bench.cpu_baseline(w, arrays, target_s=0.2)
    assert ref["bwd_idx"].size == w.chunk_len and ref["dK"] is not None
    assert ref["dK"].shape == (1, 2, 512, w.head_dim) and np.abs(ref["dK"][:, 0]).max() > 0
    assert rec["kind"] == "oracle" and rec["cores"] >= 1 and rec["host_cores"] >= rec["cores"]
    assert "BLAS thread" in rec["pool"] and rec["value"] > 0
    # forward-only: no gradient reference
    wf = WORKLOADS["llama_share"].resized(seq_total=512, heads_q=2, heads_kv=2)
    rec, ref = bench.cpu_baseline(wf, generate(wf), target_s=0.2)
    assert "dK" not in ref and ref["O"].shape[2] == ref["fwd_idx"].size


def test_trace_summary_counts_the_timed_launches_only(tmp_path):
    """Warmup launches (20 ms) and the per-step forward pass after the timed steps
    (30 ms) must not enter the timed figures (10 ms)."""
    w = WORKLOADS["zigzag_fwdbwd"]
    run = tmp_path / "prof_zigzag_fwdbwd"
    run.mkdir()
    line = {"metric": "m", "value": 1.0, "warmup": 1, "steps": 2, "config": {"workload": w.name},
            "fwd": {"pct_peak": 50.0}, "bwd": {"pct_peak": 35.0},
            "roofline": {"kernel": "bwd_dkdv_kernel", "bound": "mfma", "avg_launch_ms": 10.0,
                         "achieved": 1.0, "unit": "TFLOP/s", "frac": 0.5}}
    (tmp_path / "prof_zigzag_fwdbwd.log").write_text(json.dumps(line) + "\n")
    rows, t = [], 0
    fwd = "void ra::(anonymous namespace)::fwd_bf16_kernel<128, 64, false>(ra::FwdArgs)"
    dkdv = "void ra::(anonymous namespace)::bwd_dkdv_kernel<128, false>(ra::BwdArgs)"
    for name, ms in [(fwd, 20)] * 2 + [(dkdv, 20)] * 2 + [(fwd, 10)] * 4 + [(dkdv, 10)] * 4 + \
            [(fwd, 30)] * 8:
        rows.append(f'"{name}",{t},{t + ms * 1000000}')
        t += ms * 1000000 + 1000
    (run / "run_kernel_trace.csv").write_text("Kernel_Name,Start_Timestamp,End_Timestamp\n" +
                                              "\n".join(rows) + "\n")
    text = bench.trace_summary(str(run), w.name)
    data = json.loads(text.split("```json\n")[1].split("\n```")[0])
    assert data["kernels"]["fwd_kernel"]["timed_launches"] == 4
    assert abs(data["kernels"]["fwd_kernel"]["mean_ms"] - 10.0) < 1e-9
    assert abs(data["kernels"]["bwd_dkdv_kernel"]["median_ms"] - 10.0) < 1e-9
    pairs = 2 * (2147516416 + 2147483648) / 2 * 16 / 2
    assert abs(data["kernels"]["fwd_kernel"]["tflops"] - 512 * pairs / 10e-3 / 1e12) < 1e-6


def test_rows_parity_handles_padding_rows():
    """The packed share's row check: -inf LSE rows (padding) must match exactly, finite
    rows are compared, and an error in O, dQ or one padding row fails it."""
    rng = np.random.default_rng(3)
    O = rng.standard_normal((1, 2, 10, 8))
    dQ = rng.standard_normal((1, 2, 10, 8))
    LSE = rng.standard_normal((1, 2, 10))
    O[:, :, 7:] = 0.0
    dQ[:, :, 7:] = 0.0
    LSE[:, :, 7:] = -np.inf
    res = bench.rows_parity(O.copy(), O, LSE.copy(), LSE, dQ.copy(), dQ)
    assert res["pass"] and res["lse_inf_rows_match"] and res["lse_max_abs"] == 0.0
    bad = LSE.copy()
    bad[0, 1, 8] = 0.5  # a padding row that saw something
    assert not bench.rows_parity(O, O, bad, LSE, dQ, dQ)["pass"]
    assert not bench.rows_parity(O + 0.1, O, LSE, LSE, dQ, dQ)["pass"]
    assert not bench.rows_parity(O, O, LSE, LSE, dQ + 0.1, dQ)["pass"]
    assert bench.rows_parity(O, O, LSE + 5e-4, LSE)["pass"]  # forward only, LSE within 1e-3


def test_aux_summary_renders_a_saved_line(tmp_path):
    rec = {"kernels": [{"kernel": "lse_merge_kernel", "shape": "x: 10 rows x 8", "ms": 0.5,
                        "bytes": 1000, "achieved": 2.0, "peak": 8000.0, "frac": 0.00025}],
           "copy_reference": {"bytes": 2048, "ms": 0.1, "achieved": 20.5, "frac": 0.0026}}
    f = tmp_path / "aux.json"
    f.write_text("noise\n" + json.dumps(rec) + "\n")
    md = bench.aux_summary(str(f))
    assert "| `lse_merge_kernel` | x: 10 rows x 8 | 1000 | 0.5 | 2.0 | 0.00025 |" in md
    assert "20.5 GB/s" in md


def test_source_hash_covers_the_compiler_flags(monkeypatch):
    from ring_context_parallelism_amd import build
    files = bench.KERNELS["bwd_dq_kernel"][1]
    before = bench.source_hash(files)
    monkeypatch.setitem(build.SOURCE_FLAGS, "ra_bwd.hip", ["-mllvm", "-amdgpu-sched-strategy=ilp"])
    changed = bench.source_hash(files)
    assert changed != before
    # a flag of another source leaves this kernel's hash alone
    monkeypatch.setitem(build.SOURCE_FLAGS, "ra_fwd_f32.hip", ["-O2"])
    assert bench.source_hash(files) == changed
