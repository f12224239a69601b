"""The ring drivers under HIP graph capture, run-to-run determinism, and two ring
steps running at once on two streams.

The library allocates nothing and clears buffers with its own fill kernel (no
memset nodes), so a caller can capture a whole ring step into a graph.  The test
captures ra_ring_fwd and ra_ring_bwd, replays the graph several times with eager
work and synchronisations in between, and checks every replay bit for bit against
the eager result (the kernels use no atomics, so results are deterministic).
"""
import pytest
import torch

from ring_context_parallelism_amd import ra, staging
from ring_context_parallelism_amd.workloads import Workload, generate
from tests.gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu


def _wl():
    return Workload("graph", 600, "bf16", 1, 4, 2, 128, 128, 1024, 2, "zigzag", 0, True,
                    "normal", 0.5, backward=True)


def _buffers(w, dev):
    L, D = w.chunk_len, w.head_dim_padded
    f = dict(dtype=torch.float32, device=dev)
    return dict(
        out=torch.empty((w.batch, w.heads_q, L, D), dtype=torch.bfloat16, device=dev),
        lse=torch.empty((w.batch, w.heads_q, L), **f),
        dq=torch.empty((w.batch, w.heads_q, L, D), **f),
        dks=[torch.empty((w.batch, w.heads_kv, L, D), **f) for _ in range(w.world)],
        dvs=[torch.empty((w.batch, w.heads_kv, L, D), **f) for _ in range(w.world)])


def _step(share, w, buf, ws_f, ws_b):
    ra.ra_ring_fwd(share.prob, w.rank, share.q, share.k_chunks, share.v_chunks, buf["out"],
                   buf["lse"], ws_f)
    ra.ra_ring_bwd(share.prob, w.rank, share.q, share.k_chunks, share.v_chunks, buf["out"],
                   share.do, buf["lse"], buf["dq"], buf["dks"], buf["dvs"], ws_b)


def _snapshot(buf):
    return [buf["out"].clone(), buf["lse"].clone(), buf["dq"].clone()] + \
        [x.clone() for x in buf["dks"] + buf["dvs"]]


def test_ring_step_graph_replays_match_eager():
    dev = need_gpu()
    w = _wl()
    share = staging.stage(w, generate(w), dev)
    ws_f = torch.empty(ra.ra_ring_workspace_size(share.prob) // 4, dtype=torch.float32, device=dev)
    ws_b = torch.empty(ra.ra_ring_bwd_workspace_size(share.prob) // 4, dtype=torch.float32,
                       device=dev)
    buf = _buffers(w, dev)
    _step(share, w, buf, ws_f, ws_b)
    torch.cuda.synchronize()
    eager = _snapshot(buf)

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(share, w, buf, ws_f, ws_b)  # warm the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        _step(share, w, buf, ws_f, ws_b)
    torch.cuda.synchronize()
    for rep in range(3):
        say(f"graph replay {rep}")
        for t in [buf["out"], buf["lse"], buf["dq"]] + buf["dks"] + buf["dvs"]:
            t.fill_(float("nan") if t.dtype == torch.float32 else 7.0)  # eager work between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(_snapshot(buf), eager):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"


def test_ring_backward_is_deterministic():
    dev = need_gpu()
    w = _wl()
    share = staging.stage(w, generate(w), dev)
    out, lse = staging.ring_forward(share, w)
    first = staging.ring_backward(share, w, out, lse)
    torch.cuda.synchronize()
    first = [first[0].clone()] + [x.clone() for x in first[1] + first[2]]
    for _ in range(2):
        again = staging.ring_backward(share, w, out, lse)
        torch.cuda.synchronize()
        for a, b in zip([again[0]] + again[1] + again[2], first):
            assert torch.equal(a, b)


def test_ring_steps_on_two_streams_are_independent():
    """Two ring steps of different problems run at once on two streams (default
    priority) give bit for bit the results each gives alone: the library keeps no
    state between calls."""
    dev = need_gpu()
    wa = _wl()
    wb = Workload("graph_b", 601, "bf16", 1, 4, 1, 64, 64, 900, 3, "striped", 1, True,
                  "normal", 0.5, backward=True)
    shares = [staging.stage(w, generate(w), dev, rank=w.rank) for w in (wa, wb)]
    alone = []
    for w, sh in zip((wa, wb), shares):
        out, lse = staging.ring_forward(sh, w, rank=w.rank)
        dq, dks, dvs = staging.ring_backward(sh, w, out, lse, rank=w.rank)
        torch.cuda.synchronize()
        alone.append([out.clone(), lse.clone(), dq.clone()] + [x.clone() for x in dks + dvs])
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        say(f"two streams, repetition {rep}")
        got = [None, None]
        for i, (w, sh, s) in enumerate(zip((wa, wb), shares, streams)):
            with torch.cuda.stream(s):
                out, lse = staging.ring_forward(sh, w, rank=w.rank)
                dq, dks, dvs = staging.ring_backward(sh, w, out, lse, rank=w.rank)
                got[i] = [out, lse, dq] + dks + dvs
        torch.cuda.synchronize()
        for g, a in zip(got, alone):
            for x, y in zip(g, a):
                assert torch.equal(x, y)
