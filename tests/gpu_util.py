"""Shared helpers of the GPU parity tests: tolerances, comparisons, row sampling."""
from __future__ import annotations

import sys

import numpy as np
import torch

from ring_context_parallelism_amd.workloads import generate, round_bf16

# Tolerances of the parity gate: bf16 inputs with fp32 accumulation, fp32 problems,
# and the LSE.  rel_fro (normwise relative error) is an added gate: the absolute
# bounds alone would pass an all-zero output where |O| is small.
TOL = {
    "bf16": dict(max_abs=2e-2, mean_abs=2e-3, rel_fro=1e-2),
    "f32": dict(max_abs=1e-5, mean_abs=1e-5, rel_fro=1e-5),
}
LSE_TOL = 1e-3


def need_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("this test needs a GPU (it is marked gpu)")
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def stats(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    den = np.linalg.norm(ref)
    return dict(max_abs=float(err.max()) if err.size else 0.0,
                mean_abs=float(err.mean()) if err.size else 0.0,
                rel_fro=float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got)))


def assert_close(got, ref, dtype, what, tol=None):
    s = stats(got, ref)
    tol = TOL[dtype] if tol is None else tol
    bad = {k: v for k, v in s.items() if v > tol[k]}
    assert not bad, f"{what}: {s} exceeds {tol}"
    return s


def assert_lse(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    inf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf_ref), f"{what}: -inf rows differ"
    if (~inf_ref).any():
        err = np.abs(got[~inf_ref] - ref[~inf_ref]).max()
        assert err <= LSE_TOL, f"{what}: LSE max abs error {err}"


class Guarded:
    """Allocator of output buffers with a NaN guard tail (race-detection canaries):
    every buffer starts as NaN, so an element a kernel fails to write
    stays NaN and fails the comparison, and `check()` asserts that no write went
    past the end of any buffer."""

    def __init__(self, guard=4096):
        self.guard = guard
        self.tails = []

    def __call__(self, shape, dtype, device):
        n = int(np.prod(shape))
        buf = torch.full((n + self.guard,), float("nan"), dtype=dtype, device=device)
        self.tails.append(buf[n:])
        return buf[:n].view(shape)

    def check(self, what=""):
        for i, t in enumerate(self.tails):
            assert torch.isnan(t).all().item(), f"{what}: write past the end of buffer {i}"


def sample_rows(L, n_random=48, seed=0):
    """Local row indices: tile edges, both ends, the middle, plus random rows."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 129, 255, 256, L // 2 - 1, L // 2, L // 2 + 1,
             L - 129, L - 128, L - 65, L - 64, L - 2, L - 1]
    rand = rng.choice(L, size=min(n_random, L), replace=False).tolist()
    return np.array(sorted({t for t in fixed + rand if 0 <= t < L}), dtype=np.int64)


def sample_heads(H, seed=0):
    if H <= 4:
        return list(range(H))
    rng = np.random.default_rng(seed + 1)
    mid = rng.choice(np.arange(1, H - 1), size=2, replace=False).tolist()
    return sorted({0, H - 1, *mid})


def moving_max_inputs(w):
    """The workload's draw with q_i + 1 in every component and k_j + beta_j / sqrt(d):
    s_ij grows by about beta_j, with beta ramping 0 -> 40 along the sequence and one key
    at S/2 + 3 raised by 60, so the row maxima keep moving along the key axis (random
    inputs settle them on the first tile)."""
    arrays = generate(w)
    S, d = w.seq_total, w.head_dim
    beta = np.linspace(0.0, 40.0, S, dtype=np.float32)
    beta[S // 2 + 3] += 60.0
    q = arrays["q"] + 1.0
    k = arrays["k"] + (beta / np.sqrt(d))[None, None, :, None]
    if w.dtype == "bf16":
        q, k = round_bf16(q), round_bf16(k)
    arrays["q"], arrays["k"] = q.astype(np.float32), k.astype(np.float32)
    return arrays
