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


def _fake(w, rows, noise):
    rng = np.random.default_rng(0)
    L, D, d = w.chunk_len, w.head_dim_padded, w.head_dim
    t_idx = np.sort(rng.choice(L, size=rows, replace=False))
    O = rng.standard_normal((w.batch, 1, rows, d))
    LSE = rng.standard_normal((w.batch, 1, rows))
    dQ = rng.standard_normal((w.batch, 1, rows, d))
    out = torch.zeros((w.batch, w.heads_q, L, D), dtype=torch.float32)
    lse = torch.zeros((w.batch, w.heads_q, L), dtype=torch.float32)
    dq = torch.zeros((w.batch, w.heads_q, L, D), dtype=torch.float32)
    ti = torch.from_numpy(t_idx)
    out[:, :1, ti, :d] = torch.from_numpy(O + noise).float()
    lse[:, :1, ti] = torch.from_numpy(LSE).float()
    dq[:, :1, ti, :d] = torch.from_numpy(dQ).float()
    return (t_idx, O, LSE, dQ), out, lse, dq


def test_sample_parity_passes_and_fails():
    w = WORKLOADS["zigzag_fwdbwd"].resized(seq_total=1024)
    ref, out, lse, dq = _fake(w, 40, 0.0)
    res = bench.sample_parity(w, ref, out, lse, dq)
    assert res["pass"] and res["o"]["max_abs"] < 1e-6 and res["dq"]["max_abs"] < 1e-6
    ref, out, lse, dq = _fake(w, 40, 0.1)  # a 0.1 error in O breaks the bf16 gate
    res = bench.sample_parity(w, ref, out, lse, dq)
    assert not res["pass"] and res["o"]["max_abs"] > 0.05


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
    r = bench.roofline(512 * pairs, pairs, 14.0, bench.BF16_PEAK_TFLOPS)
    assert r["bound"] == "mfma" and abs(r["frac"] - 512 * pairs / 14e-3 / 1e12 / 2516.6) < 1e-4
    assert r["alu_frac"] < r["frac"]
    # d = 24: 96 FLOP per pair; the softmax's 3 vector operations per pair bind first
    pairs = 2.8125e10
    r = bench.roofline(96 * pairs, pairs, 4.6, bench.BF16_PEAK_TFLOPS)
    assert r["bound"] == "alu" and r["unit"] == "TOP/s"
    assert abs(r["achieved"] - 3 * pairs / 4.6e-3 / 1e12) < 1e-2
    assert abs(bench.ALU_PEAK_TOPS - 39.3216) < 1e-3 and r["mfma_frac"] < r["frac"]
