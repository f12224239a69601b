"""GPU parity with non-default strides, through the C ABI.

The problem carries element strides (b, h, t) for q, every k/v chunk and out/dout;
callers often hold [B, L, H, D] (sequence-major) tensors, or rows padded beyond D.
These cases stage the same inputs in such layouts and compare the ring forward and
backward with the fp64 oracle.  The "rowpad" layout follows each head's L rows with
128 rows of NaN: every kernel reads its last, ragged tile through a buffer resource
bounded at row L, so those rows must read as zeros (a NaN that got in would reach the
outputs through 0 * NaN).
"""
import numpy as np
import pytest
import torch

import oracle
from ring_context_parallelism_amd import ra
from ring_context_parallelism_amd.workloads import Workload, generate
from tests.gpu_util import assert_close, assert_lse, need_gpu, say

pytestmark = pytest.mark.gpu


def _wl(dtype, D, d, layout, p, S, causal, B, Hq, Hkv, backward):
    return Workload(f"s_{dtype}", 500 + S, dtype, B, Hq, Hkv, d, D, S, p, layout, 0, causal,
                    "normal", 0.5, backward=backward)


# (workload, storage): "blhd" = [B, L, H, D] sequence-major; "pad" = [B, H, L, D + 64]
CASES = [
    (_wl("bf16", 128, 128, "zigzag", 2, 600, True, 2, 4, 2, True), "blhd"),
    (_wl("bf16", 64, 64, "striped", 3, 390, True, 1, 2, 1, True), "pad"),
    (_wl("bf16", 128, 128, "striped", 2, 520, True, 2, 8, 2, True), "blhd"),  # GQA group 4
    (_wl("f32", 64, 48, "contiguous", 2, 520, False, 1, 2, 2, False), "blhd"),
    (_wl("f32", 32, 24, "zigzag", 2, 520, True, 2, 2, 1, False), "pad"),  # d = 24 kernel, padded rows
    (_wl("f32", 32, 24, "contiguous", 2, 520, False, 1, 2, 2, False), "rowpad"),
    (_wl("bf16", 128, 128, "zigzag", 2, 600, True, 1, 2, 1, True), "rowpad"),
]
ROW_PAD = 128  # NaN rows after each head's L rows (more than any tile reaches past L)


def _ids(c):
    w, st = c
    return f"{w.dtype}-D{w.head_dim_padded}-{w.layout}-p{w.world}-S{w.seq_total}-{st}"


def _place(arr, pos, D, dtype, dev, storage):
    """arr [B, H, S, d] fp32 -> (view [B, H, L, D], element strides (b, h, t))."""
    B, H, _, d = arr.shape
    L = pos.size
    host = torch.zeros((B, H, L, D), dtype=torch.float32)
    host[..., :d] = torch.from_numpy(np.ascontiguousarray(arr[:, :, pos, :]))
    if storage == "blhd":
        buf = torch.zeros((B, L, H, D), dtype=dtype, device=dev)
        view = buf.permute(0, 2, 1, 3)
    elif storage == "rowpad":
        buf = torch.full((B, H, L + ROW_PAD, D), float("nan"), dtype=dtype, device=dev)
        view = buf[:, :, :L]
    else:
        buf = torch.zeros((B, H, L, D + 64), dtype=dtype, device=dev)
        view = buf[..., :D]
    view.copy_(host.to(dtype).to(dev))
    return view, tuple(view.stride()[:3])


def _empty_like_layout(B, H, L, D, dtype, dev, storage):
    if storage == "blhd":
        return torch.zeros((B, L, H, D), dtype=dtype, device=dev).permute(0, 2, 1, 3)
    if storage == "rowpad":
        return torch.full((B, H, L + ROW_PAD, D), float("nan"), dtype=dtype, device=dev)[:, :, :L]
    return torch.zeros((B, H, L, D + 64), dtype=dtype, device=dev)[..., :D]


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_strided_ring_fwd_bwd(case):
    dev = need_gpu()
    w, storage = case
    arrays = generate(w)
    D, d, L = w.head_dim_padded, w.head_dim, w.chunk_len
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    tol = "bf16" if w.dtype == "bf16" else "f32"
    for r in range(w.world):
        say(f"strided {_ids(case)} rank {r}")
        rows = oracle.positions(w.layout, w.seq_total, w.world, r)
        q, q_st = _place(arrays["q"], rows, D, dt, dev, storage)
        ks, vs = [], []
        for c in range(w.world):
            pos = oracle.positions(w.layout, w.seq_total, w.world, c)
            k, kv_st = _place(arrays["k"], pos, D, dt, dev, storage)
            v, _ = _place(arrays["v"], pos, D, dt, dev, storage)
            ks.append(k)
            vs.append(v)
        out = _empty_like_layout(w.batch, w.heads_q, L, D, dt, dev, storage)
        o_st = tuple(out.stride()[:3])
        prob = ra.make_problem(batch=w.batch, heads_q=w.heads_q, heads_kv=w.heads_kv,
                               head_dim=d, head_dim_padded=D, seq_total=w.seq_total,
                               world=w.world, layout=w.layout, causal=w.causal, dtype=w.dtype,
                               q_stride=q_st, kv_stride=kv_st, o_stride=o_st)
        lse = torch.empty((w.batch, w.heads_q, L), dtype=torch.float32, device=dev)
        ws = torch.empty(ra.ra_ring_workspace_size(prob) // 4, dtype=torch.float32, device=dev)
        ra.ra_ring_fwd(prob, r, q, ks, vs, out, lse, ws)
        torch.cuda.synchronize()
        O, LSE = oracle.attention_fwd(arrays["q"], arrays["k"], arrays["v"], rows, w.causal)
        got = out.float().cpu().numpy()
        assert_close(got[..., :d], O, tol, f"O rank {r}")
        assert np.all(got[..., d:] == 0.0)
        assert_lse(lse.cpu().numpy(), LSE, f"LSE rank {r}")
        if not w.backward:
            continue
        do, do_st = _place(arrays["do"], rows, D, dt, dev, storage)
        assert do_st == o_st
        dq = torch.empty((w.batch, w.heads_q, L, D), dtype=torch.float32, device=dev)
        dks = [torch.empty((w.batch, w.heads_kv, L, D), dtype=torch.float32, device=dev)
               for _ in range(w.world)]
        dvs = [torch.empty_like(dks[0]) for _ in range(w.world)]
        wsb = torch.empty(ra.ra_ring_bwd_workspace_size(prob) // 4, dtype=torch.float32,
                          device=dev)
        ra.ra_ring_bwd(prob, r, q, ks, vs, out, do, lse, dq, dks, dvs, wsb)
        torch.cuda.synchronize()
        dQ, dK, dV = oracle.attention_bwd(arrays["q"], arrays["k"], arrays["v"],
                                          arrays["do"][:, :, rows], rows, w.causal)
        assert_close(dq.cpu().numpy()[..., :d], dQ, "bf16", f"dQ rank {r}")
        for c in range(w.world):
            pos = oracle.positions(w.layout, w.seq_total, w.world, c)
            assert_close(dks[c].cpu().numpy()[..., :d], dK[:, :, pos], "bf16", f"dK {c}")
            assert_close(dvs[c].cpu().numpy()[..., :d], dV[:, :, pos], "bf16", f"dV {c}")
