"""ra_ring_bwd_noalloc, the backward driver whose delta workspace lives in a static
device array, against ra_ring_bwd with a caller workspace, through the C ABI.

Two calls in a row, the second on a smaller problem (so a stale workspace from the
first call would show), each compared element for element with ra_ring_bwd on the
same inputs; every output starts as NaN with a NaN guard tail.  The kernels are the
same, so the results must be identical.  Also: a problem whose workspace exceeds the
static array is refused before anything is enqueued.
"""
import numpy as np
import pytest
import torch

from ring_context_parallelism_amd import ra, staging
from ring_context_parallelism_amd.workloads import Workload, generate
from tests.gpu_util import Guarded, need_gpu, say

pytestmark = pytest.mark.gpu


def _wl(S, p, layout, Hq, Hkv, D, seed):
    return Workload(f"noalloc_{S}", seed, "bf16", 1, Hq, Hkv, D, D, S, p, layout, 0, True,
                    "normal", 0.5, backward=True)


def test_noalloc_matches_ring_bwd_on_two_calls_second_smaller():
    dev = need_gpu()
    cases = [_wl(4096, 2, "zigzag", 8, 4, 128, 301), _wl(600, 3, "striped", 2, 1, 64, 302)]
    for w in cases:
        arrays = generate(w)
        for r in range(w.world):
            say(f"noalloc {w.layout} S{w.seq_total} p{w.world} rank {r}")
            share = staging.stage(w, arrays, dev, rank=r)
            out, lse = staging.ring_forward(share, w, rank=r)
            want = staging.ring_backward(share, w, out, lse, rank=r)
            guard = Guarded()
            L, D = w.chunk_len, w.head_dim_padded
            dq = guard((w.batch, w.heads_q, L, D), torch.float32, dev)
            dks = [guard((w.batch, w.heads_kv, L, D), torch.float32, dev) for _ in range(w.world)]
            dvs = [guard((w.batch, w.heads_kv, L, D), torch.float32, dev) for _ in range(w.world)]
            ra.ra_ring_bwd_noalloc(share.prob, r, share.q, share.k_chunks, share.v_chunks, out,
                                   share.do, lse, dq, dks, dvs)
            torch.cuda.synchronize()
            guard.check(f"noalloc rank {r}")
            assert torch.equal(dq, want[0])
            for c in range(w.world):
                assert torch.equal(dks[c], want[1][c]) and torch.equal(dvs[c], want[2][c])
            assert torch.count_nonzero(dq).item() > 0


def test_noalloc_refuses_a_workspace_beyond_the_static_array():
    need_gpu()
    # batch * heads_q * L = 64 * 131072 > 4,194,304 rows of fp32 delta
    p = ra.make_problem(batch=1, heads_q=64, heads_kv=8, head_dim=128, head_dim_padded=128,
                        seq_total=131072, world=1, layout="contiguous", causal=True,
                        dtype="bf16")
    fake = 1 << 20
    with pytest.raises(ra.RaError) as e:
        ra.ra_ring_bwd_noalloc(p, 0, fake, [fake], [fake], fake, fake, fake, fake, [fake],
                               [fake])
    assert e.value.status == ra.RA_ERR_WORKSPACE
    assert "static scratch" in ra.ra_last_error()
