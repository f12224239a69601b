"""Places one rank's share of a workload in device memory (HBM).

Takes the global-order host arrays of ``workloads.generate`` and builds the device
tensors the C ABI consumes: the rank's query chunk, every KV chunk (indexed by
chunk id), and dO for backward workloads, each [B, H, L, D] with the head dim
zero-padded to D, plus the packed-document boundaries (int32 [B, n]) of packed
workloads.  The token order inside each chunk comes from the library's own
position map (``ra_positions``), so the host never re-implements the layouts.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

from . import ra
from .workloads import Workload


def problem_for(w: Workload, scale: float = 0.0, seg_bounds=None) -> ra.Problem:
    return ra.make_problem(batch=w.batch, heads_q=w.heads_q, heads_kv=w.heads_kv,
                           head_dim=w.head_dim, head_dim_padded=w.head_dim_padded,
                           seq_total=w.seq_total, world=w.world, layout=w.layout,
                           causal=w.causal, dtype=w.dtype, scale=scale, seg_bounds=seg_bounds)


def torch_dtype(w: Workload):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def _to_device(arr: np.ndarray, pos: np.ndarray, D: int, dtype, device) -> torch.Tensor:
    """arr [B, H, S, d] (fp32, exact in dtype) -> device [B, H, len(pos), D] in dtype."""
    B, H, _, d = arr.shape
    host = torch.zeros((B, H, pos.size, D), dtype=torch.float32)
    host[..., :d] = torch.from_numpy(np.ascontiguousarray(arr[:, :, pos, :]))
    return host.to(dtype).to(device)


@dataclasses.dataclass
class Share:
    prob: ra.Problem
    q: torch.Tensor
    k_chunks: list
    v_chunks: list
    do: torch.Tensor | None
    rows: np.ndarray  # global positions of the rank's query rows (library map)
    bounds: torch.Tensor | None = None  # device int32 [B, n] (kept alive with prob)


def stage(w: Workload, arrays: dict, device="cuda", rank: int | None = None) -> Share:
    prob = problem_for(w)
    rank = w.rank if rank is None else rank
    D, dt = w.head_dim_padded, torch_dtype(w)
    rows = ra.ra_positions(prob, rank)
    ks, vs = [], []
    for c in range(w.world):
        pos = ra.ra_positions(prob, c)
        ks.append(_to_device(arrays["k"], pos, D, dt, device))
        vs.append(_to_device(arrays["v"], pos, D, dt, device))
    q = _to_device(arrays["q"], rows, D, dt, device)
    do = _to_device(arrays["do"], rows, D, dt, device) if "do" in arrays else None
    bounds = None
    if arrays.get("bounds") is not None:
        bounds = torch.from_numpy(np.ascontiguousarray(arrays["bounds"], dtype=np.int32)).to(device)
        prob = problem_for(w, seg_bounds=bounds)
    return Share(prob, q, ks, vs, do, rows, bounds)


def _empty(shape, dtype, device):
    return torch.empty(shape, dtype=dtype, device=device)


def ring_forward(share: Share, w: Workload, rank: int | None = None, stream=None, alloc=None):
    """Runs ra_ring_fwd on a staged share; returns (out [B, Hq, L, D], lse fp32).

    alloc(shape, dtype, device) -> tensor allocates the outputs and the workspace
    (default: torch.empty)."""
    rank = w.rank if rank is None else rank
    alloc = alloc or _empty
    L, D = w.chunk_len, w.head_dim_padded
    dev = share.q.device
    out = alloc((w.batch, w.heads_q, L, D), torch_dtype(w), dev)
    lse = alloc((w.batch, w.heads_q, L), torch.float32, dev)
    ws = alloc((ra.ra_ring_workspace_size(share.prob) // 4,), torch.float32, dev)
    ra.ra_ring_fwd(share.prob, rank, share.q, share.k_chunks, share.v_chunks, out, lse, ws,
                   stream=stream)
    return out, lse


def ring_backward(share: Share, w: Workload, out, lse, rank: int | None = None, stream=None,
                  alloc=None):
    """Runs ra_ring_bwd; returns (dq, dk_chunks, dv_chunks), fp32 [B, H, L, D].

    alloc as in ring_forward (gradients and workspace)."""
    rank = w.rank if rank is None else rank
    alloc = alloc or _empty
    L, D = w.chunk_len, w.head_dim_padded
    dev = share.q.device
    f32 = torch.float32
    dq = alloc((w.batch, w.heads_q, L, D), f32, dev)
    dks = [alloc((w.batch, w.heads_kv, L, D), f32, dev) for _ in range(w.world)]
    dvs = [alloc((w.batch, w.heads_kv, L, D), f32, dev) for _ in range(w.world)]
    ws = alloc((ra.ra_ring_bwd_workspace_size(share.prob) // 4,), f32, dev)
    ra.ra_ring_bwd(share.prob, rank, share.q, share.k_chunks, share.v_chunks, out, share.do,
                   lse, dq, dks, dvs, ws, stream=stream)
    return dq, dks, dvs
