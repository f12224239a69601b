"""GPU parity at degenerate sizes, through the C ABI.

Chunks of 1, 2, 3, 33, 65 and 66 tokens (a tile that is mostly ragged tail), zigzag
sub-blocks of a single token, the striped layout with one token per chunk, p = 1,
batch and head counts of 1 and 3, GQA groups of 4 and 8 (several query heads share a
workgroup), every rank's share, forward (bf16 and fp32) and backward, dense and packed.
"""
import numpy as np
import pytest
import torch

import oracle
from ring_context_parallelism_amd import staging
from ring_context_parallelism_amd.workloads import Workload, generate
from tests.gpu_util import Guarded, assert_close, assert_lse, need_gpu, say

pytestmark = pytest.mark.gpu


def _wl(dtype, D, d, layout, p, S, causal, B, Hq, Hkv, backward):
    return Workload(f"e_{dtype}_{D}_{layout}", 400 + S, dtype, B, Hq, Hkv, d, D, S, p, layout, 0,
                    causal, "normal", 0.5, backward=backward)


CASES = [
    _wl("bf16", 128, 128, "contiguous", 4, 4, True, 1, 2, 1, True),      # L = 1
    _wl("bf16", 64, 64, "zigzag", 2, 4, True, 1, 1, 1, True),            # sub-blocks of 1
    _wl("bf16", 128, 128, "striped", 8, 8, True, 3, 3, 3, True),         # one token per chunk
    _wl("bf16", 32, 24, "zigzag", 3, 6, False, 2, 2, 1, True),           # L = 2, non-causal
    _wl("bf16", 128, 100, "contiguous", 2, 6, True, 1, 4, 2, True),      # L = 3
    _wl("bf16", 64, 64, "striped", 3, 99, True, 1, 2, 2, True),          # L = 33
    _wl("bf16", 128, 128, "zigzag", 2, 132, True, 1, 2, 1, True),        # L = 66
    _wl("bf16", 128, 128, "contiguous", 1, 65, True, 1, 1, 1, True),     # p = 1, L = 65
    _wl("bf16", 128, 128, "contiguous", 2, 6, True, 2, 8, 2, True),      # L = 3, GQA group 4
    _wl("bf16", 128, 128, "zigzag", 2, 260, True, 1, 8, 1, True),        # L = 130, GQA group 8
    _wl("f32", 64, 64, "contiguous", 4, 4, True, 1, 1, 1, False),
    _wl("f32", 128, 128, "zigzag", 2, 4, True, 2, 2, 1, False),
    _wl("f32", 32, 24, "striped", 8, 8, False, 1, 3, 3, False),
    _wl("f32", 128, 128, "striped", 3, 99, True, 1, 1, 1, False),
]

# packed lists at degenerate sizes: a one-token document, an empty one, padding
PACKED = [
    (_wl("bf16", 64, 64, "zigzag", 3, 6, True, 2, 2, 1, True),
     np.array([[0, 1, 1, 4, 5], [0, 6, 6, 6, 6]], np.int32)),
    (_wl("bf16", 128, 128, "striped", 4, 36, True, 1, 2, 2, True),
     np.array([[0, 7, 8, 30]], np.int32)),
    (_wl("f32", 32, 24, "contiguous", 2, 66, False, 1, 1, 1, False),
     np.array([[0, 33, 34, 60]], np.int32)),
]


def _ids(w):
    return f"{w.dtype}-D{w.head_dim_padded}d{w.head_dim}-{w.layout}-p{w.world}-S{w.seq_total}-" \
           f"{'causal' if w.causal else 'full'}-B{w.batch}H{w.heads_q}x{w.heads_kv}"


def _np(t):
    return t.float().cpu().numpy()


def _check_share(w, arrays, bounds, dev):
    d = w.head_dim
    tol = "bf16" if w.dtype == "bf16" else "f32"
    for r in range(w.world):
        say(f"edge {_ids(w)} rank {r}")
        share = staging.stage(w, arrays, dev, rank=r)
        guard = Guarded()
        out, lse = staging.ring_forward(share, w, rank=r, alloc=guard)
        torch.cuda.synchronize()
        guard.check(f"edge forward rank {r}")
        rows = oracle.positions(w.layout, w.seq_total, w.world, r)
        O, LSE = oracle.attention_fwd(arrays["q"], arrays["k"], arrays["v"], rows, w.causal,
                                      bounds=bounds)
        got = _np(out)
        assert_close(got[..., :d], O, tol, f"O rank {r}")
        assert np.all(got[..., d:] == 0.0)
        assert_lse(_np(lse), LSE, f"LSE rank {r}")
        if not w.backward:
            continue
        dq, dks, dvs = staging.ring_backward(share, w, out, lse, rank=r, alloc=guard)
        torch.cuda.synchronize()
        guard.check(f"edge backward rank {r}")
        dQ, dK, dV = oracle.attention_bwd(arrays["q"], arrays["k"], arrays["v"],
                                          arrays["do"][:, :, rows], rows, w.causal, bounds=bounds)
        assert_close(_np(dq)[..., :d], dQ, "bf16", f"dQ rank {r}")
        for c in range(w.world):
            pos = oracle.positions(w.layout, w.seq_total, w.world, c)
            assert_close(_np(dks[c])[..., :d], dK[:, :, pos], "bf16", f"dK chunk {c} rank {r}")
            assert_close(_np(dvs[c])[..., :d], dV[:, :, pos], "bf16", f"dV chunk {c} rank {r}")


@pytest.mark.parametrize("w", CASES, ids=_ids)
def test_degenerate_sizes(w):
    dev = need_gpu()
    _check_share(w, generate(w), None, dev)


@pytest.mark.parametrize("case", PACKED, ids=lambda c: _ids(c[0]) if isinstance(c, tuple) else "")
def test_degenerate_sizes_packed(case):
    dev = need_gpu()
    w, bounds = case
    arrays = generate(w)
    arrays["bounds"] = bounds
    _check_share(w, arrays, [list(map(int, b)) for b in bounds], dev)
