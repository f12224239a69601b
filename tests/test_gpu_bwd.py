"""GPU parity of the backward path against the fp64 oracle, through the C ABI.

* oracle-sized cases: every rank's share of ra_ring_bwd (delta, zero-fill, every
  live step) against the oracle's analytic gradients -- dQ of the rank's rows and
  dK, dV of every KV chunk -- element by element;
* ra_block_attn_bwd accumulates (+=) and a step with no visible pair is a no-op;
* ra_bwd_delta against the oracle's rowsum(dO * O);
* the forward+backward zigzag workload at full size: dQ on sampled rows and heads
  the oracle computes one by one, plus two identities that hold at any size,
  sum_j dV_j = sum_i dO_i and sum_j dK_j = 0 (per KV head).
"""
import numpy as np
import pytest
import torch

import oracle
from ring_context_parallelism_amd import ra, staging
from ring_context_parallelism_amd.workloads import WORKLOADS, Workload, generate
from tests.gpu_util import assert_close, need_gpu, sample_heads, sample_rows, say, stats

pytestmark = pytest.mark.gpu


def _wl(D, d, layout, p, S, causal, B, Hq, Hkv, dist="normal", scale=0.5, seed=200):
    return Workload(f"b_{D}_{layout}", seed, "bf16", B, Hq, Hkv, d, D, S, p, layout, 0, causal,
                    dist, scale, backward=True)


SMALL = [
    _wl(128, 128, "zigzag", 2, 600, True, 1, 2, 2),
    _wl(128, 128, "contiguous", 2, 600, True, 2, 4, 2),
    _wl(128, 128, "striped", 3, 600, True, 1, 4, 1),
    _wl(128, 128, "contiguous", 1, 300, True, 1, 2, 1),
    _wl(128, 96, "striped", 2, 520, False, 1, 2, 2),
    _wl(64, 64, "zigzag", 3, 780, True, 1, 4, 2),
    _wl(32, 24, "contiguous", 4, 1000, False, 2, 4, 4, dist="uniform", scale=1.0),
]


def _ids(w):
    return f"D{w.head_dim_padded}d{w.head_dim}-{w.layout}-p{w.world}-S{w.seq_total}-" \
           f"{'causal' if w.causal else 'full'}-B{w.batch}H{w.heads_q}x{w.heads_kv}"


def _np(t):
    return t.float().cpu().numpy()


@pytest.mark.parametrize("w", SMALL, ids=_ids)
def test_ring_bwd_every_rank(w):
    dev = need_gpu()
    arrays = generate(w)
    d = w.head_dim
    for r in range(w.world):
        say(f"ring_bwd {_ids(w)} rank {r}")
        share = staging.stage(w, arrays, dev, rank=r)
        out, lse = staging.ring_forward(share, w, rank=r)
        dq, dks, dvs = staging.ring_backward(share, w, out, lse, rank=r)
        torch.cuda.synchronize()
        rows = oracle.positions(w.layout, w.seq_total, w.world, r)
        dQ, dK, dV = oracle.attention_bwd(arrays["q"], arrays["k"], arrays["v"],
                                          arrays["do"][:, :, rows], rows, w.causal)
        got = _np(dq)
        s = assert_close(got[..., :d], dQ, "bf16", f"dQ rank {r}")
        assert np.all(got[..., d:] == 0.0)
        for c in range(w.world):
            pos = oracle.positions(w.layout, w.seq_total, w.world, c)
            sk = assert_close(_np(dks[c])[..., :d], dK[:, :, pos], "bf16", f"dK chunk {c} rank {r}")
            sv = assert_close(_np(dvs[c])[..., :d], dV[:, :, pos], "bf16", f"dV chunk {c} rank {r}")
        say(f"  dQ {s}  dK {sk}  dV {sv}")


def test_block_bwd_accumulates_and_skips():
    dev = need_gpu()
    w = SMALL[1]
    arrays = generate(w)
    r = 0
    share = staging.stage(w, arrays, dev, rank=r)
    out, lse = staging.ring_forward(share, w, rank=r)
    L, D = w.chunk_len, w.head_dim_padded
    delta = torch.empty((w.batch, w.heads_q, L), dtype=torch.float32, device=dev)
    ra.ra_bwd_delta(share.prob, out, share.do, delta)
    mk = lambda H: torch.zeros((w.batch, H, L, D), dtype=torch.float32, device=dev)
    dq1, dk1, dv1 = mk(w.heads_q), mk(w.heads_kv), mk(w.heads_kv)
    dq2, dk2, dv2 = mk(w.heads_q), mk(w.heads_kv), mk(w.heads_kv)
    args = (share.prob, share.q, r, share.k_chunks[0], share.v_chunks[0], 0, share.do, lse, delta)
    ra.ra_block_attn_bwd(*args, dq1, dk1, dv1)
    ra.ra_block_attn_bwd(*args, dq2, dk2, dv2)
    ra.ra_block_attn_bwd(*args, dq2, dk2, dv2)
    # rank 0 sees nothing of chunk 1 under the contiguous causal layout: a no-op
    before = dk1.clone()
    ra.ra_block_attn_bwd(share.prob, share.q, r, share.k_chunks[1], share.v_chunks[1], 1,
                         share.do, lse, delta, dq1, dk1, dv1)
    torch.cuda.synchronize()
    for a, b in ((dq1, dq2), (dk1, dk2), (dv1, dv2)):
        assert torch.allclose(2 * a, b, rtol=1e-5, atol=1e-6)
    assert torch.equal(before, dk1)


def test_bwd_delta_kernel():
    dev = need_gpu()
    for D, dtype in ((128, torch.bfloat16), (64, torch.bfloat16), (32, torch.float32)):
        rng = np.random.default_rng(D)
        o = torch.tensor(rng.standard_normal((2, 3, 77, D)), dtype=dtype)
        do = torch.tensor(rng.standard_normal((2, 3, 77, D)), dtype=dtype)
        prob = ra.make_problem(batch=2, heads_q=3, heads_kv=3, head_dim=D, head_dim_padded=D,
                               seq_total=77, world=1, layout="contiguous", causal=True,
                               dtype="bf16" if dtype == torch.bfloat16 else "f32")
        delta = torch.empty((2, 3, 77), dtype=torch.float32, device=dev)
        ra.ra_bwd_delta(prob, o.to(dev), do.to(dev), delta)
        torch.cuda.synchronize()
        want = oracle.bwd_delta(do.float().numpy(), o.float().numpy())
        assert np.max(np.abs(delta.cpu().numpy() - want)) < 1e-4


def test_bwd_prepare_delta_and_zero_fill():
    """ra_bwd_prepare: delta as the oracle's, every gradient buffer exactly zero.

    The buffers start as NaN and each has a NaN guard tail (odd L, p = 3 chunks,
    GQA), so a fill that stops short, overruns or misses a chunk shows.
    """
    dev = need_gpu()
    B, H, Hkv, p, L, D = 2, 4, 2, 3, 79, 64
    rng = np.random.default_rng(11)
    o = torch.tensor(rng.standard_normal((B, H, L, D)), dtype=torch.bfloat16)
    do = torch.tensor(rng.standard_normal((B, H, L, D)), dtype=torch.bfloat16)
    prob = ra.make_problem(batch=B, heads_q=H, heads_kv=Hkv, head_dim=D, head_dim_padded=D,
                           seq_total=p * L, world=p, layout="contiguous", causal=True,
                           dtype="bf16")
    nan = dict(dtype=torch.float32, device=dev)
    guard = 4096  # a tail past every buffer, which must stay NaN
    delta = torch.full((B * H * L,), float("nan"), **nan)
    dq = torch.full((B * H * L * D + guard,), float("nan"), **nan)
    dks = [torch.full((B * Hkv * L * D + guard,), float("nan"), **nan) for _ in range(p)]
    dvs = [torch.full((B * Hkv * L * D + guard,), float("nan"), **nan) for _ in range(p)]
    ra.ra_bwd_prepare(prob, o.to(dev), do.to(dev), delta, dq, dks, dvs)
    torch.cuda.synchronize()
    want = oracle.bwd_delta(do.float().numpy(), o.float().numpy()).reshape(-1)
    assert np.max(np.abs(delta.cpu().numpy() - want)) < 1e-4
    for t, n in [(dq, B * H * L * D)] + [(x, B * Hkv * L * D) for x in dks + dvs]:
        assert torch.count_nonzero(t[:n]).item() == 0
        assert torch.isnan(t[n:]).all()


def test_full_size_backward_sampled_and_identities():
    dev = need_gpu()
    w = WORKLOADS["zigzag_fwdbwd"]
    say("full-size backward: generating inputs")
    arrays = generate(w)
    share = staging.stage(w, arrays, dev)
    say("full-size backward: ra_ring_fwd + ra_ring_bwd")
    out, lse = staging.ring_forward(share, w)
    dq, dks, dvs = staging.ring_backward(share, w, out, lse)
    torch.cuda.synchronize()
    assert torch.isfinite(dq).all()
    L, d = w.chunk_len, w.head_dim
    t_idx = sample_rows(L, n_random=24, seed=7)
    heads = sample_heads(w.heads_q, seed=7)
    rows_all = oracle.positions(w.layout, w.seq_total, w.world, w.rank)
    rows = rows_all[t_idx]
    say(f"full-size backward: oracle dQ on {len(t_idx)} rows x {len(heads)} heads")
    dO = arrays["do"][:, heads][:, :, rows]
    dQ, _, _ = oracle.attention_bwd(arrays["q"], arrays["k"], arrays["v"], dO, rows, w.causal,
                                    heads=heads)
    got = dq[:, heads][:, :, torch.from_numpy(t_idx).to(dev)].cpu().numpy()
    s = assert_close(got[..., :d], dQ, "bf16", "dQ sampled")
    say(f"full-size backward: dQ {s}")
    # identities over the whole share: sum_j dV_j = sum_i dO_i and sum_j dK_j = 0
    g = w.heads_q // w.heads_kv
    do_sum = share.do.double().sum(dim=2)                        # [B, Hq, D]
    do_sum = do_sum.view(w.batch, w.heads_kv, g, -1).sum(dim=2)  # per KV head
    dv_sum = sum(x.double().sum(dim=2) for x in dvs)
    dk_sum = sum(x.double().sum(dim=2) for x in dks)
    dk_fro = torch.sqrt(sum((x.double() ** 2).sum(dim=(2, 3)) for x in dks))
    rel_v = ((dv_sum - do_sum).norm(dim=-1) / do_sum.norm(dim=-1)).max().item()
    rel_k = (dk_sum.norm(dim=-1) / dk_fro).max().item()
    say(f"full-size backward: |sum dV - sum dO|/|sum dO| = {rel_v:.2e}, "
        f"|sum dK|/|dK|_F = {rel_k:.2e}")
    assert rel_v < 1e-2 and rel_k < 2e-2


def test_split_entry_points_match_combined():
    """ra_block_attn_bwd_dkdv + ra_block_attn_bwd_dq equal ra_block_attn_bwd exactly
    (no atomics anywhere: every output element has a single writer)."""
    dev = need_gpu()
    w = SMALL[2]
    arrays = generate(w)
    share = staging.stage(w, arrays, dev, rank=1)
    out, lse = staging.ring_forward(share, w, rank=1)
    L, D = w.chunk_len, w.head_dim_padded
    delta = torch.empty((w.batch, w.heads_q, L), dtype=torch.float32, device=dev)
    ra.ra_bwd_delta(share.prob, out, share.do, delta)
    mk = lambda H: torch.zeros((w.batch, H, L, D), dtype=torch.float32, device=dev)
    for c in range(w.world):
        dq1, dk1, dv1 = mk(w.heads_q), mk(w.heads_kv), mk(w.heads_kv)
        dq2, dk2, dv2 = mk(w.heads_q), mk(w.heads_kv), mk(w.heads_kv)
        args = (share.prob, share.q, 1, share.k_chunks[c], share.v_chunks[c], c, share.do, lse,
                delta)
        ra.ra_block_attn_bwd(*args, dq1, dk1, dv1)
        ra.ra_block_attn_bwd_dkdv(*args, dk2, dv2)
        ra.ra_block_attn_bwd_dq(*args, dq2)
        torch.cuda.synchronize()
        assert torch.equal(dq1, dq2) and torch.equal(dk1, dk2) and torch.equal(dv1, dv2)
