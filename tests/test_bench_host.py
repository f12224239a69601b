"""Host-side logic of bench.py (no GPU): the one-GPU guard and the parity record."""
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
