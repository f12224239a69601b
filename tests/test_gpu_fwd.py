"""GPU parity of the forward path against the fp64 oracle, through the C ABI.

* oracle-sized cases (several tiles plus a ragged tail, every layout, GQA, padded
  head dims, fp32 and bf16): every rank's share of the ring forward, compared
  element by element with the oracle's global result;
* per-step partials (RA_WRITE) for every (query chunk, KV chunk) pair, including
  rows that see nothing (0 and -inf), and RA_MERGE chains in ring order;
* the standalone LSE merge against the oracle's merge, -inf rows included;
* every workload at its full size through ra_ring_fwd (the launch configuration
  the benchmark times), on sampled rows and heads the oracle computes one by one,
  and on every row of some heads (for GQA, one workgroup's group of four heads);
* the rescaling path of the online softmax driven on most tiles (moving-max inputs),
  and run-to-run determinism.
"""
import numpy as np
import pytest
import torch

import oracle
from ring_context_parallelism_amd import ra, staging
from ring_context_parallelism_amd.workloads import WORKLOADS, Workload, generate
from tests.gpu_util import (Guarded, assert_close, assert_lse, moving_max_inputs, need_gpu,
                            sample_heads, sample_rows, say)

pytestmark = pytest.mark.gpu


def _wl(dtype, D, d, layout, p, S, causal, B, Hq, Hkv, dist="normal", scale=0.5, seed=100):
    return Workload(f"t_{dtype}_{D}_{layout}", seed, dtype, B, Hq, Hkv, d, D, S, p, layout, 0,
                    causal, dist, scale)


SMALL = [
    _wl("bf16", 128, 128, "contiguous", 2, 600, True, 2, 4, 2),
    _wl("bf16", 128, 128, "striped", 3, 600, True, 1, 4, 1),
    _wl("bf16", 128, 128, "zigzag", 2, 600, True, 1, 2, 2),
    _wl("bf16", 128, 128, "striped", 2, 520, False, 1, 2, 1),
    _wl("bf16", 128, 100, "contiguous", 1, 300, True, 1, 2, 1),
    _wl("bf16", 64, 64, "zigzag", 3, 780, True, 1, 4, 2),
    _wl("bf16", 32, 24, "contiguous", 4, 1000, False, 2, 4, 4, dist="uniform", scale=1.0),
    _wl("f32", 64, 64, "contiguous", 4, 1024, True, 1, 1, 1, scale=1.0),
    _wl("f32", 32, 24, "contiguous", 4, 1000, False, 2, 2, 2, dist="uniform", scale=1.0),
    _wl("f32", 128, 128, "striped", 2, 520, True, 1, 2, 1),
    _wl("f32", 64, 40, "zigzag", 2, 520, True, 1, 2, 2),
    _wl("bf16", 128, 128, "contiguous", 2, 520, False, 2, 8, 2),  # 4 GQA heads per workgroup
    _wl("f32", 128, 96, "striped", 2, 520, True, 1, 2, 1),       # fp32 QK^T over 3/4 of D
]


def _ids(w):
    return f"{w.dtype}-D{w.head_dim_padded}d{w.head_dim}-{w.layout}-p{w.world}-S{w.seq_total}-" \
           f"{'causal' if w.causal else 'full'}-B{w.batch}H{w.heads_q}x{w.heads_kv}"


def _np(t):
    return t.float().cpu().numpy()


@pytest.mark.parametrize("w", SMALL, ids=_ids)
def test_ring_fwd_every_rank(w):
    dev = need_gpu()
    arrays = generate(w)
    d = w.head_dim
    for r in range(w.world):
        say(f"ring_fwd {_ids(w)} rank {r}")
        share = staging.stage(w, arrays, dev, rank=r)
        guard = Guarded()
        out, lse = staging.ring_forward(share, w, rank=r, alloc=guard)
        torch.cuda.synchronize()
        guard.check(f"ring_fwd rank {r}")
        rows = oracle.positions(w.layout, w.seq_total, w.world, r)
        assert np.array_equal(rows, share.rows)
        O, LSE = oracle.attention_fwd(arrays["q"], arrays["k"], arrays["v"], rows, w.causal)
        got = _np(out)
        assert_close(got[..., :d], O, w.dtype, f"O rank {r}")
        assert np.all(got[..., d:] == 0.0), "padded head-dim columns must stay exactly 0"
        assert_lse(_np(lse), LSE, f"LSE rank {r}")


# Scores that keep growing along the key axis, plus one outlier key: the running max of
# every row moves on most tiles, so the rescaling path of the online softmax runs over
# and over (random inputs settle the max on the first tile).
MOVING_MAX = [
    _wl("bf16", 128, 128, "contiguous", 2, 1100, True, 1, 2, 1, seed=120),
    _wl("bf16", 64, 64, "zigzag", 2, 1040, False, 1, 2, 2, seed=121),
    _wl("bf16", 32, 24, "striped", 2, 1000, True, 1, 2, 1, dist="uniform", scale=1.0, seed=122),
    _wl("f32", 64, 64, "striped", 2, 1024, True, 1, 1, 1, seed=123),
    # fp32 at both contraction lengths: d = 24 in 32 columns (three quarters) and d = 128
    _wl("f32", 32, 24, "zigzag", 2, 1000, True, 1, 2, 1, dist="uniform", scale=1.0, seed=124),
    _wl("f32", 128, 128, "contiguous", 2, 900, True, 1, 2, 2, seed=125),
]


@pytest.mark.parametrize("w", MOVING_MAX, ids=_ids)
def test_ring_fwd_moving_max(w):
    dev = need_gpu()
    arrays = moving_max_inputs(w)
    d = w.head_dim
    for r in range(w.world):
        say(f"moving max {_ids(w)} rank {r}")
        share = staging.stage(w, arrays, dev, rank=r)
        guard = Guarded()
        out, lse = staging.ring_forward(share, w, rank=r, alloc=guard)
        torch.cuda.synchronize()
        guard.check(f"moving max rank {r}")
        rows = oracle.positions(w.layout, w.seq_total, w.world, r)
        O, LSE = oracle.attention_fwd(arrays["q"], arrays["k"], arrays["v"], rows, w.causal)
        assert LSE.max() - LSE.min() > 15.0, "the inputs must move the row maxima"
        got = _np(out)
        assert_close(got[..., :d], O, w.dtype, f"O rank {r}")
        assert_lse(_np(lse), LSE, f"LSE rank {r}")


@pytest.mark.parametrize("w", [SMALL[0], SMALL[1], SMALL[5], SMALL[7], SMALL[10]], ids=_ids)
def test_block_fwd_partials_and_merge(w):
    """RA_WRITE partial of every (query chunk, KV chunk) pair, then an RA_MERGE chain."""
    dev = need_gpu()
    arrays = generate(w)
    d, D, L = w.head_dim, w.head_dim_padded, w.chunk_len
    scale = 1.0 / np.sqrt(d)
    for cq in range(w.world):
        share = staging.stage(w, arrays, dev, rank=cq)
        qpos = oracle.positions(w.layout, w.seq_total, w.world, cq)
        o_acc = torch.zeros((w.batch, w.heads_q, L, D), dtype=torch.float32, device=dev)
        l_acc = torch.full((w.batch, w.heads_q, L), float("-inf"), dtype=torch.float32, device=dev)
        for s, ck in enumerate(oracle.ring_schedule(cq, w.world)):
            say(f"block_fwd {_ids(w)} q_chunk {cq} kv_chunk {ck}")
            kpos = oracle.positions(w.layout, w.seq_total, w.world, ck)
            guard = Guarded()
            o = guard((w.batch, w.heads_q, L, D), torch.float32, dev)
            lse = guard((w.batch, w.heads_q, L), torch.float32, dev)
            ra.ra_block_attn_fwd(share.prob, share.q, cq, share.k_chunks[ck], share.v_chunks[ck],
                                 ck, o, lse, ra.RA_WRITE)
            ra.ra_block_attn_fwd(share.prob, share.q, cq, share.k_chunks[ck], share.v_chunks[ck],
                                 ck, o_acc, l_acc, ra.RA_MERGE)
            torch.cuda.synchronize()
            guard.check(f"partial ({cq},{ck})")
            Op, Lp = oracle.attention_partial(arrays["q"][:, :, qpos], arrays["k"][:, :, kpos],
                                              arrays["v"][:, :, kpos], qpos, kpos, w.causal,
                                              scale, w.heads_q, w.heads_kv)
            got = _np(o)
            assert_close(got[..., :d], Op, "bf16" if w.dtype == "bf16" else "f32",
                         f"partial ({cq},{ck})")
            empty = np.isneginf(Lp)
            assert np.all(got[empty] == 0.0), "rows with no visible key must be 0"
            assert_lse(_np(lse), Lp, f"partial LSE ({cq},{ck})")
        O, LSE = oracle.attention_fwd(arrays["q"], arrays["k"], arrays["v"], qpos, w.causal)
        assert_close(_np(o_acc)[..., :d], O, "bf16" if w.dtype == "bf16" else "f32",
                     f"merge chain rank {cq}")
        assert_lse(_np(l_acc), LSE, f"merge chain LSE rank {cq}")


@pytest.mark.parametrize("rows,d", [(1, 4), (1000, 128), (777, 24), (4096, 64), (64, 1024)])
def test_lse_merge_kernel(rows, d):
    dev = need_gpu()
    rng = np.random.default_rng(rows + d)
    oa, op = rng.standard_normal((rows, d)), rng.standard_normal((rows, d))
    la, lp = rng.standard_normal(rows) * 4, rng.standard_normal(rows) * 4
    la[::7] = -np.inf
    oa[::7] = 0.0
    lp[::5] = -np.inf
    op[::5] = 0.0
    want_o, want_l = oracle.lse_merge(oa, la, op, lp)
    t = lambda x: torch.tensor(x, dtype=torch.float32, device=dev)
    goa, gla, gop, glp = t(oa), t(la), t(op), t(lp)
    say(f"lse_merge rows {rows} d {d}")
    ra.ra_lse_merge(rows, d, goa, gla, gop, glp)
    torch.cuda.synchronize()
    assert np.max(np.abs(goa.cpu().numpy() - want_o)) < 1e-5
    got_l = gla.cpu().numpy()
    assert np.array_equal(np.isneginf(got_l), np.isneginf(want_l))
    fin = ~np.isneginf(want_l)
    if fin.any():
        assert np.max(np.abs(got_l[fin] - want_l[fin])) < 1e-5


def test_ring_fwd_deterministic():
    dev = need_gpu()
    w = SMALL[1]
    arrays = generate(w)
    share = staging.stage(w, arrays, dev, rank=1)
    o1, l1 = staging.ring_forward(share, w, rank=1)
    o2, l2 = staging.ring_forward(share, w, rank=1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


FULL = [WORKLOADS["tiny_fp32"], WORKLOADS["llama_share"], WORKLOADS["gqa_striped"],
        WORKLOADS["tabular_rows"], WORKLOADS["tabular_rows"].with_dtype("bf16"),
        WORKLOADS["zigzag_fwdbwd"]]


@pytest.mark.parametrize("w", FULL, ids=lambda w: f"{w.name}-{w.dtype}")
def test_full_size_forward_sampled(w):
    dev = need_gpu()
    say(f"full-size forward {w.name} {w.dtype}: generating inputs")
    arrays = generate(w)
    share = staging.stage(w, arrays, dev)
    say(f"full-size forward {w.name} {w.dtype}: ra_ring_fwd")
    guard = Guarded()
    out, lse = staging.ring_forward(share, w, alloc=guard)
    torch.cuda.synchronize()
    guard.check(f"full-size forward {w.name}")
    L, d = w.chunk_len, w.head_dim
    full = w.name == "tiny_fp32"
    t_idx = np.arange(L) if full else sample_rows(L, seed=w.seed)
    heads = list(range(w.heads_q)) if full else sample_heads(w.heads_q, seed=w.seed)
    rows = oracle.positions(w.layout, w.seq_total, w.world, w.rank)[t_idx]
    say(f"full-size forward {w.name}: oracle on {len(t_idx)} rows x {len(heads)} heads")
    O, LSE = oracle.attention_fwd(arrays["q"], arrays["k"], arrays["v"], rows, w.causal,
                                  heads=heads)
    got = out[:, heads][:, :, torch.from_numpy(t_idx).to(dev)].float().cpu().numpy()
    s = assert_close(got[..., :d], O, w.dtype, f"{w.name} O")
    assert_lse(lse[:, heads][:, :, torch.from_numpy(t_idx).to(dev)].cpu().numpy(), LSE,
               f"{w.name} LSE")
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    if d < w.head_dim_padded:
        assert torch.all(out[..., d:] == 0)
    say(f"full-size forward {w.name}: {s}")


COMPLETE = [  # (workload, heads compared on every row)
    (WORKLOADS["gqa_striped"], [4, 5, 6, 7, 31]),  # one workgroup's group of 4 heads, and the last
    (WORKLOADS["llama_share"], [0, 15]),
    (WORKLOADS["tabular_rows"], [0, 3]),
    (WORKLOADS["tabular_rows"].with_dtype("bf16"), [1]),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("w,heads", COMPLETE, ids=[f"{w.name}-{w.dtype}" for w, _ in COMPLETE])
def test_full_size_forward_complete_heads(w, heads):
    """A workload at full size with every row of some heads (every batch element)
    compared element by element against the oracle's row-parallel driver; for the GQA
    share, heads 4..7 are the four query heads on KV head 1 that share a forward
    workgroup."""
    from oracle.rows import attention_fwd_rows, default_workers
    dev = need_gpu()
    say(f"full-size complete heads {w.name} {w.dtype}: generating inputs")
    arrays = generate(w)
    share = staging.stage(w, arrays, dev)
    guard = Guarded()
    out, lse = staging.ring_forward(share, w, alloc=guard)
    torch.cuda.synchronize()
    guard.check(f"full-size complete heads {w.name}")
    d = w.head_dim
    say(f"full-size complete heads {w.name}: oracle on all {w.chunk_len} rows of heads {heads} "
        f"x {w.batch} batch ({default_workers()} threads)")
    O, LSE = attention_fwd_rows(arrays["q"], arrays["k"], arrays["v"], share.rows, w.causal,
                                heads=heads)
    got = out[:, heads].float().cpu().numpy()
    s = assert_close(got[..., :d], O, w.dtype, f"{w.name} O")
    assert_lse(lse[:, heads].cpu().numpy(), LSE, f"{w.name} LSE")
    if d < w.head_dim_padded:
        assert np.all(got[..., d:] == 0.0)
    say(f"full-size complete heads {w.name}: {s}")
