"""GPU parity of packed documents and global right padding, through the C ABI.

Documents are given by global position boundaries per batch element (ringmaster
page, "Native recurrent context parallelism"); the oracle takes the same lists.

* oracle-sized cases, every rank's share, forward (bf16 and fp32) and backward:
  hand-written boundary lists with documents of length 1, empty documents,
  documents that straddle chunk and zigzag sub-block edges, right padding and a
  batch element that is all padding; and seeded random lists;
* per-step partials (RA_WRITE) and an RA_MERGE chain with documents;
* the packed forward+backward workload at full size in the launch configuration
  the benchmark times, on sampled rows and heads, plus identities that hold at any
  size: sum_j dV_j = sum of dO over rows that see a key, sum_j dK_j = 0, and
  exact zeros on padding rows and keys.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from ring_context_parallelism_amd import ra, staging
from ring_context_parallelism_amd.workloads import WORKLOADS, Workload, document_bounds, generate
from tests.gpu_util import (Guarded, assert_close, assert_lse, need_gpu, sample_heads,
                            sample_rows, say)

pytestmark = pytest.mark.gpu


def _wl(dtype, D, d, layout, p, S, causal, B, Hq, Hkv, docs, dist="normal", scale=0.5, seed=300,
        backward=False):
    return Workload(f"pk_{dtype}_{D}_{layout}", seed, dtype, B, Hq, Hkv, d, D, S, p, layout, 0,
                    causal, dist, scale, backward=backward, docs=docs)


# Hand-written lists (None = use the workload's seeded random lists).
_HAND = {
    # zigzag S 600, p 2: sub-blocks of 150; length-1 documents at 0 and 1, a document
    # across the 150 and 300 edges, padding from 580; batch 1 is one whole document
    "zz600": np.array([[0, 1, 2, 150, 151, 299, 450, 451, 580],
                       [0, 600, 600, 600, 600, 600, 600, 600, 600]], np.int32),
    # contiguous S 520: batch 1 is all padding
    "ct520": np.array([[0, 100, 100, 259, 261, 400, 510], [0, 0, 0, 0, 0, 0, 0]], np.int32),
}

FWD = [
    (_wl("bf16", 128, 128, "zigzag", 2, 600, True, 2, 2, 2, None), "zz600"),
    (_wl("bf16", 128, 128, "striped", 3, 600, True, 1, 4, 1, (1, 120, 0.2)), None),
    (_wl("bf16", 64, 64, "contiguous", 2, 520, False, 2, 2, 2, None), "ct520"),
    (_wl("bf16", 128, 128, "contiguous", 2, 520, True, 2, 4, 2, None), "ct520"),
    (_wl("bf16", 32, 24, "contiguous", 4, 1000, False, 2, 4, 4, (1, 400, 0.1), dist="uniform",
         scale=1.0), None),
    (_wl("f32", 32, 24, "contiguous", 4, 1000, False, 2, 2, 2, (1, 400, 0.1), dist="uniform",
         scale=1.0), None),
    (_wl("f32", 128, 128, "zigzag", 2, 520, True, 1, 2, 1, (3, 200, 0.15), scale=1.0), None),
    (_wl("f32", 64, 64, "striped", 2, 512, True, 1, 1, 1, (1, 64, 0.3), scale=1.0), None),
]

BWD = [
    (_wl("bf16", 128, 128, "zigzag", 2, 600, True, 2, 2, 2, None, backward=True), "zz600"),
    (_wl("bf16", 128, 128, "striped", 3, 600, False, 1, 4, 2, (1, 150, 0.2), backward=True), None),
    (_wl("bf16", 64, 64, "contiguous", 2, 520, True, 2, 4, 2, None, backward=True), "ct520"),
    (_wl("bf16", 32, 24, "contiguous", 4, 1000, False, 2, 4, 4, (1, 400, 0.1), dist="uniform",
         scale=1.0, backward=True), None),
    (_wl("bf16", 128, 128, "contiguous", 1, 300, True, 1, 2, 1, (1, 90, 0.1), backward=True), None),
]


def _ids(case):
    w, hand = case
    return f"{w.dtype}-D{w.head_dim_padded}d{w.head_dim}-{w.layout}-p{w.world}-S{w.seq_total}-" \
           f"{'causal' if w.causal else 'full'}-B{w.batch}H{w.heads_q}x{w.heads_kv}-" \
           f"{hand or 'random'}"


def _inputs(case):
    w, hand = case
    if hand is None:
        return w, generate(w)
    arrays = generate(dataclasses.replace(w, docs=None))
    arrays["bounds"] = _HAND[hand]
    return w, arrays


def _np(t):
    return t.float().cpu().numpy()


def _bounds_list(arrays):
    return [list(map(int, b)) for b in arrays["bounds"]]


@pytest.mark.parametrize("case", FWD, ids=_ids)
def test_packed_ring_fwd_every_rank(case):
    dev = need_gpu()
    w, arrays = _inputs(case)
    bounds = _bounds_list(arrays)
    d = w.head_dim
    for r in range(w.world):
        say(f"packed ring_fwd {_ids(case)} rank {r}")
        share = staging.stage(w, arrays, dev, rank=r)
        guard = Guarded()
        out, lse = staging.ring_forward(share, w, rank=r, alloc=guard)
        torch.cuda.synchronize()
        guard.check(f"packed ring_fwd rank {r}")
        rows = oracle.positions(w.layout, w.seq_total, w.world, r)
        O, LSE = oracle.attention_fwd(arrays["q"], arrays["k"], arrays["v"], rows, w.causal,
                                      bounds=bounds)
        got = _np(out)
        assert_close(got[..., :d], O, w.dtype, f"O rank {r}")
        assert np.all(got[..., d:] == 0.0)
        dead = np.isneginf(LSE)
        assert np.all(got[dead] == 0.0), "rows that see no key must be exactly 0"
        assert_lse(_np(lse), LSE, f"LSE rank {r}")


@pytest.mark.parametrize("case", [FWD[0], FWD[2], FWD[6]], ids=_ids)
def test_packed_block_fwd_partials_and_merge(case):
    """RA_WRITE partial of every (query chunk, KV chunk) pair, then an RA_MERGE chain."""
    dev = need_gpu()
    w, arrays = _inputs(case)
    bounds = _bounds_list(arrays)
    d, D, L = w.head_dim, w.head_dim_padded, w.chunk_len
    scale = 1.0 / np.sqrt(d)
    tol = "bf16" if w.dtype == "bf16" else "f32"
    for cq in range(w.world):
        share = staging.stage(w, arrays, dev, rank=cq)
        qpos = oracle.positions(w.layout, w.seq_total, w.world, cq)
        o_acc = torch.zeros((w.batch, w.heads_q, L, D), dtype=torch.float32, device=dev)
        l_acc = torch.full((w.batch, w.heads_q, L), float("-inf"), dtype=torch.float32, device=dev)
        for ck in oracle.ring_schedule(cq, w.world):
            say(f"packed block_fwd {_ids(case)} q_chunk {cq} kv_chunk {ck}")
            kpos = oracle.positions(w.layout, w.seq_total, w.world, ck)
            guard = Guarded()
            o = guard((w.batch, w.heads_q, L, D), torch.float32, dev)
            lse = guard((w.batch, w.heads_q, L), torch.float32, dev)
            ra.ra_block_attn_fwd(share.prob, share.q, cq, share.k_chunks[ck], share.v_chunks[ck],
                                 ck, o, lse, ra.RA_WRITE)
            ra.ra_block_attn_fwd(share.prob, share.q, cq, share.k_chunks[ck], share.v_chunks[ck],
                                 ck, o_acc, l_acc, ra.RA_MERGE)
            torch.cuda.synchronize()
            guard.check(f"packed partial ({cq},{ck})")
            Op, Lp = oracle.attention_partial(arrays["q"][:, :, qpos], arrays["k"][:, :, kpos],
                                              arrays["v"][:, :, kpos], qpos, kpos, w.causal,
                                              scale, w.heads_q, w.heads_kv, bounds=bounds,
                                              seq_total=w.seq_total)
            got = _np(o)
            assert_close(got[..., :d], Op, tol, f"partial ({cq},{ck})")
            assert np.all(got[np.isneginf(Lp)] == 0.0)
            assert_lse(_np(lse), Lp, f"partial LSE ({cq},{ck})")
        O, LSE = oracle.attention_fwd(arrays["q"], arrays["k"], arrays["v"], qpos, w.causal,
                                      bounds=bounds)
        assert_close(_np(o_acc)[..., :d], O, tol, f"merge chain rank {cq}")
        assert_lse(_np(l_acc), LSE, f"merge chain LSE rank {cq}")


@pytest.mark.parametrize("case", BWD, ids=_ids)
def test_packed_ring_bwd_every_rank(case):
    dev = need_gpu()
    w, arrays = _inputs(case)
    bounds = _bounds_list(arrays)
    d = w.head_dim
    for r in range(w.world):
        say(f"packed ring_bwd {_ids(case)} rank {r}")
        share = staging.stage(w, arrays, dev, rank=r)
        guard = Guarded()
        out, lse = staging.ring_forward(share, w, rank=r, alloc=guard)
        dq, dks, dvs = staging.ring_backward(share, w, out, lse, rank=r, alloc=guard)
        torch.cuda.synchronize()
        guard.check(f"packed ring fwd+bwd rank {r}")
        rows = oracle.positions(w.layout, w.seq_total, w.world, r)
        dQ, dK, dV = oracle.attention_bwd(arrays["q"], arrays["k"], arrays["v"],
                                          arrays["do"][:, :, rows], rows, w.causal, bounds=bounds)
        got = _np(dq)
        s = assert_close(got[..., :d], dQ, "bf16", f"dQ rank {r}")
        assert np.all(got[..., d:] == 0.0)
        for c in range(w.world):
            pos = oracle.positions(w.layout, w.seq_total, w.world, c)
            assert_close(_np(dks[c])[..., :d], dK[:, :, pos], "bf16", f"dK chunk {c} rank {r}")
            assert_close(_np(dvs[c])[..., :d], dV[:, :, pos], "bf16", f"dV chunk {c} rank {r}")
            for b in range(w.batch):  # padding keys get exactly zero gradient
                pad = pos >= bounds[b][-1]
                assert np.all(_np(dks[c])[b][:, pad] == 0.0) and np.all(_np(dvs[c])[b][:, pad] == 0.0)
        for b in range(w.batch):
            assert np.all(got[b][:, rows >= bounds[b][-1]] == 0.0)
        say(f"  dQ {s}")


@pytest.mark.timeout(600)
def test_packed_full_size_sampled_and_identities():
    """The packed share at full size: O and LSE on sampled rows (tile and document
    edges), dQ of every row and dK, dV of every key of both chunks for head 0 element
    by element, identities over all heads, and NaN guard tails."""
    from oracle.rows import attention_bwd_rows
    dev = need_gpu()
    w = WORKLOADS["packed_fwdbwd"]
    say("packed full size: generating inputs")
    arrays = generate(w)
    bounds = _bounds_list(arrays)
    share = staging.stage(w, arrays, dev)
    say("packed full size: ra_ring_fwd + ra_ring_bwd")
    guard = Guarded()
    out, lse = staging.ring_forward(share, w, alloc=guard)
    dq, dks, dvs = staging.ring_backward(share, w, out, lse, alloc=guard)
    torch.cuda.synchronize()
    guard.check("packed full size")
    L, d = w.chunk_len, w.head_dim
    rows_all = oracle.positions(w.layout, w.seq_total, w.world, w.rank)
    # sampled rows: tile edges and random rows, plus rows at every document edge
    edges = np.searchsorted(rows_all, np.array(bounds[0]))
    t_idx = np.unique(np.concatenate([sample_rows(L, n_random=24, seed=9),
                                      np.clip(np.concatenate([edges - 1, edges]), 0, L - 1)]))
    heads = sample_heads(w.heads_q, seed=9)
    rows = rows_all[t_idx]
    say(f"packed full size: oracle on {len(t_idx)} rows x {len(heads)} heads")
    O, LSE = oracle.attention_fwd(arrays["q"], arrays["k"], arrays["v"], rows, w.causal,
                                  heads=heads, bounds=bounds)
    ti = torch.from_numpy(t_idx).to(dev)
    got = out[:, heads][:, :, ti].float().cpu().numpy()
    assert_close(got[..., :d], O, "bf16", "O sampled")
    assert_lse(lse[:, heads][:, :, ti].cpu().numpy(), LSE, "LSE sampled")
    say("packed full size: oracle backward on every row of head 0")
    dQ, dK, dV = attention_bwd_rows(arrays["q"], arrays["k"], arrays["v"],
                                    arrays["do"][:, :1][:, :, rows_all], rows_all, w.causal,
                                    heads=[0], bounds=bounds)
    s = assert_close(dq[:, :1].cpu().numpy()[..., :d], dQ, "bf16", "dQ head 0")
    say(f"packed full size: dQ {s}")
    g0 = 0  # KV head of query head 0
    for c in range(w.world):
        pos = oracle.positions(w.layout, w.seq_total, w.world, c)
        sk = assert_close(dks[c][:, g0].cpu().numpy()[..., :d], dK[:, g0][:, pos], "bf16",
                          f"dK chunk {c}")
        sv = assert_close(dvs[c][:, g0].cpu().numpy()[..., :d], dV[:, g0][:, pos], "bf16",
                          f"dV chunk {c}")
        say(f"packed full size: chunk {c}: dK {sk}  dV {sv}")
    # identities over the whole share
    live = torch.from_numpy(rows_all < bounds[0][-1]).to(dev)
    g = w.heads_q // w.heads_kv
    do_sum = (share.do.double() * live[None, None, :, None]).sum(dim=2)
    do_sum = do_sum.view(w.batch, w.heads_kv, g, -1).sum(dim=2)
    dv_sum = sum(x.double().sum(dim=2) for x in dvs)
    dk_sum = sum(x.double().sum(dim=2) for x in dks)
    dk_fro = torch.sqrt(sum((x.double() ** 2).sum(dim=(2, 3)) for x in dks))
    rel_v = ((dv_sum - do_sum).norm(dim=-1) / do_sum.norm(dim=-1)).max().item()
    rel_k = (dk_sum.norm(dim=-1) / dk_fro).max().item()
    say(f"packed full size: |sum dV - sum dO|/|sum dO| = {rel_v:.2e}, |sum dK|/|dK|_F = {rel_k:.2e}")
    assert rel_v < 1e-2 and rel_k < 2e-2
    assert torch.all(dq[:, :, ~live] == 0) and torch.all(out[:, :, ~live] == 0)
    assert torch.all(torch.isneginf(lse[:, :, ~live]))
    for c in range(w.world):
        kpad = torch.from_numpy(oracle.positions(w.layout, w.seq_total, w.world, c)
                                >= bounds[0][-1]).to(dev)
        assert torch.all(dks[c][:, :, kpad] == 0) and torch.all(dvs[c][:, :, kpad] == 0)
