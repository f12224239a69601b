"""The memory-bound helpers past their capped grid, through the C ABI.

The LSE merge, the delta and the fp32 fill launch at most 2^20 workgroups of 256
threads and let every thread stride over what remains, so that any size the entry
points accept fits one launch.  These cases are large enough that the stride loops of
the merge and the fill run more than once:

* ra_lse_merge over 2^25 + 2^20 + 37 rows at d = 4 (8 lanes per row, so one pass of
  the capped grid covers 2^25 rows), compared with the oracle's merge on every row,
  -inf partials on either side included;
* ra_bwd_prepare with 65 query heads of 131,072 rows at d = 128: dQ holds more than
  2^30 floats, so the fill (4 floats per thread per pass) takes two passes.  Every
  gradient element must be exactly zero, the NaN guard tails past each buffer must be
  untouched, and delta must match the oracle on rows of every head.
"""
import numpy as np
import pytest
import torch

import oracle
from ring_context_parallelism_amd import ra
from tests.gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu

CAP_THREADS = (1 << 20) * 256  # workgroups of one capped helper launch x threads


def test_lse_merge_strides_past_the_capped_grid():
    dev = need_gpu()
    rows, d = (1 << 25) + (1 << 20) + 37, 4
    assert rows * 8 > CAP_THREADS  # the second pass of the stride loop has rows to do
    rng = np.random.default_rng(2025)
    oa = rng.standard_normal((rows, d), dtype=np.float32)
    op = rng.standard_normal((rows, d), dtype=np.float32)
    la = (rng.standard_normal(rows, dtype=np.float32) * 4).astype(np.float32)
    lp = (rng.standard_normal(rows, dtype=np.float32) * 4).astype(np.float32)
    la[::7] = -np.inf
    oa[::7] = 0.0
    lp[::5] = -np.inf
    op[::5] = 0.0
    goa, gla = torch.from_numpy(oa).to(dev), torch.from_numpy(la).to(dev)
    gop, glp = torch.from_numpy(op).to(dev), torch.from_numpy(lp).to(dev)
    say(f"lse_merge rows {rows} d {d}")
    ra.ra_lse_merge(rows, d, goa, gla, gop, glp)
    torch.cuda.synchronize()
    got_o, got_l = goa.cpu().numpy(), gla.cpu().numpy()
    step = 1 << 22
    for a in range(0, rows, step):
        e = min(a + step, rows)
        want_o, want_l = oracle.lse_merge(oa[a:e], la[a:e], op[a:e], lp[a:e])
        assert np.max(np.abs(got_o[a:e] - want_o)) < 1e-5, f"rows {a}..{e}"
        assert np.array_equal(np.isneginf(got_l[a:e]), np.isneginf(want_l)), f"rows {a}..{e}"
        fin = ~np.isneginf(want_l)
        assert np.max(np.abs(got_l[a:e][fin] - want_l[fin])) < 1e-5, f"rows {a}..{e}"


def test_bwd_prepare_fill_strides_past_the_capped_grid():
    dev = need_gpu()
    B, Hq, Hkv, L, D = 1, 65, 5, 1 << 17, 128
    n_q, n_kv = B * Hq * L * D, B * Hkv * L * D
    assert n_q > 4 * CAP_THREADS  # the fill of dQ needs a second pass
    prob = ra.make_problem(batch=B, heads_q=Hq, heads_kv=Hkv, head_dim=D, head_dim_padded=D,
                           seq_total=L, world=1, layout="contiguous", causal=True, dtype="bf16")
    rng = np.random.default_rng(2026)
    base_o = torch.from_numpy(rng.standard_normal((L, D), dtype=np.float32)).to(torch.bfloat16)
    base_do = torch.from_numpy(rng.standard_normal((L, D), dtype=np.float32)).to(torch.bfloat16)
    shift = 97  # head h holds the base rows rolled by h * shift, so heads differ
    o = torch.stack([torch.roll(base_o, h * shift, 0) for h in range(Hq)])[None].to(dev)
    do = torch.stack([torch.roll(base_do, h * shift, 0) for h in range(Hq)])[None].to(dev)
    guard = 4096
    f32 = dict(dtype=torch.float32, device=dev)
    delta = torch.full((B * Hq * L + guard,), float("nan"), **f32)
    dq = torch.full((n_q + guard,), float("nan"), **f32)
    dk = torch.full((n_kv + guard,), float("nan"), **f32)
    dv = torch.full((n_kv + guard,), float("nan"), **f32)
    say(f"bwd_prepare Hq {Hq} L {L} D {D}: dq {n_q} floats")
    ra.ra_bwd_prepare(prob, o, do, delta, dq, [dk], [dv])
    torch.cuda.synchronize()
    for t, n, what in [(dq, n_q, "dq"), (dk, n_kv, "dk"), (dv, n_kv, "dv")]:
        assert torch.count_nonzero(t[:n]).item() == 0, what
        assert torch.isnan(t[n:]).all(), f"{what} guard tail"
    assert torch.isnan(delta[B * Hq * L:]).all(), "delta guard tail"
    base = oracle.bwd_delta(base_do.float().numpy(), base_o.float().numpy())
    got = delta[:B * Hq * L].view(Hq, L).cpu().numpy()
    rows = np.r_[0:64, L // 2 - 32:L // 2 + 32, L - 64:L]
    for h in range(Hq):
        want = np.roll(base, h * shift)[rows]
        assert np.max(np.abs(got[h, rows] - want)) < 1e-3, f"head {h}"
