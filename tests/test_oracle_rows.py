"""The oracle's row-parallel drivers against the oracle itself (CPU only).

attention_fwd_rows / attention_bwd_rows split a rank's rows over worker threads and
place or add the groups' results; they must reproduce attention_fwd / attention_bwd
to fp64 rounding on every layout, GQA, several batch elements, packed documents, a
subset of heads and more workers than rows, so a dropped, repeated or misplaced row
group shows.
"""
import numpy as np
import pytest

import oracle
from oracle.rows import _row_groups, attention_bwd_rows, attention_fwd_rows

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _inputs(B, Hq, Hkv, S, d, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, S, d)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, S, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, S, d)).astype(np.float32)
    do = rng.standard_normal((B, Hq, S, d)).astype(np.float32)
    return q, k, v, do


CASES = [
    # layout, p, rank, causal, B, Hq, Hkv, S, heads, bounds, workers
    ("zigzag", 2, 0, True, 1, 2, 2, 96, None, None, 4),
    ("striped", 3, 1, True, 2, 4, 2, 90, [1, 3], None, 3),
    ("contiguous", 4, 3, False, 1, 2, 1, 64, None, None, 5),
    ("zigzag", 2, 1, True, 2, 2, 1, 80, None,
     [[0, 7, 8, 8, 40, 41, 70], [0, 50, 80, 80, 80, 80, 80]], 4),
    ("contiguous", 2, 1, True, 1, 1, 1, 24, None, None, 40),  # more workers than rows
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-p{c[1]}r{c[2]}-w{c[10]}")
def test_rows_drivers_reproduce_the_oracle(case):
    layout, p, rank, causal, B, Hq, Hkv, S, heads, bounds, workers = case
    q, k, v, do_g = _inputs(B, Hq, Hkv, S, 8, seed=S + p)
    rows = oracle.positions(layout, S, p, rank)
    hs = list(range(Hq)) if heads is None else heads
    dO = do_g[:, hs][:, :, rows]
    O1, L1 = oracle.attention_fwd(q, k, v, rows, causal, heads=heads, bounds=bounds)
    O2, L2 = attention_fwd_rows(q, k, v, rows, causal, heads=heads, bounds=bounds,
                                workers=workers)
    assert np.array_equal(np.isneginf(L1), np.isneginf(L2))
    fin = np.isfinite(L1)
    assert np.max(np.abs(L1[fin] - L2[fin])) < 1e-12
    assert np.max(np.abs(O1 - O2)) < 1e-12
    g1 = oracle.attention_bwd(q, k, v, dO, rows, causal, heads=heads, bounds=bounds)
    g2 = attention_bwd_rows(q, k, v, dO, rows, causal, heads=heads, bounds=bounds,
                            workers=workers)
    for a, b in zip(g1, g2):
        assert a.shape == b.shape
        assert np.max(np.abs(a - b)) < 1e-12
    assert np.abs(g2[1]).max() > 0  # the case has gradient mass to lose


def test_row_groups_cover_every_row_once():
    rows = oracle.positions("zigzag", 1024, 2, 0)
    for causal in (True, False):
        for n in (1, 3, 16, 5000):
            gs = _row_groups(rows, causal, 1024, n)
            covered = np.concatenate([np.arange(a, b) for a, b in gs])
            assert np.array_equal(covered, np.arange(rows.size))
    # causal groups balance the visible-key cost: no group above twice the mean
    gs = _row_groups(rows, True, 1024, 8)
    cost = [float(np.sum(rows[a:b] + 1)) for a, b in gs]
    assert max(cost) < 2 * np.mean(cost)
