"""Pins for the CPU oracle: checks against things other than the oracle itself.

Every pin takes the oracle implementation as an argument (`impl`, a module with the
oracle's functions), so test_oracle_pins.py can run the same pins against copies of
the oracle with one planted mistake each and show that some pin catches it.

Kinds of pin used (none re-types the oracle's formula against itself):
  * the page's worked ring example (tests/golden/ring_walkthrough.json);
  * closed forms: Q = 0 gives LSE = ln(#visible keys) and O = mean of the visible V
    rows; V = 1 gives O = 1; a causal first token gives O = V_0, LSE = q0.k0*scale;
  * library routines on special cases: torch scaled_dot_product_attention and
    torch autograd, in fp64 on the CPU (p = 1 and shares of it, GQA included);
  * brute force in pure Python on tiny inputs (unstabilised exp sums, math.fsum);
  * exact identities: shift invariance, key-permutation invariance (non-causal),
    GQA = MHA on repeated K/V, the merge identities, blockwise = unblocked for
    random chunkings, sum_j dV_j = sum_i dO_i, sum_j dK_j = 0, dQ_0 = 0;
  * central finite differences for the backward;
  * packed documents: each document equals SDPA / autograd run on that document
    alone, Q = 0 gives LSE = ln(#visible keys of the document), values at
    right-padding positions change nothing, and the position-to-document map
    against a loop over its definition.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _shares(impl, layout, S, p):
    return [impl.positions(layout, S, p, c) for c in range(p)]


# ---------------------------------------------------------------------------- layouts

def pin_positions_partition(impl):
    """Every layout partitions [0, S) into p chunks of L ascending positions."""
    for layout in ("contiguous", "striped", "zigzag"):
        for p in (1, 2, 3, 4):
            S = 4 * p * 3
            sh = _shares(impl, layout, S, p)
            allpos = np.concatenate(sh)
            assert sorted(allpos.tolist()) == list(range(S)), (layout, p)
            for c, pos in enumerate(sh):
                assert pos.size == S // p
                assert np.all(np.diff(pos) > 0)


def pin_positions_layout_facts(impl):
    """Brute-force facts of each layout, from its plain description."""
    S, p = 48, 4
    L, h = S // p, S // (2 * p)
    for c in range(p):
        pos = impl.positions("contiguous", S, p, c)
        assert pos.tolist() == list(range(c * L, (c + 1) * L))
        pos = impl.positions("striped", S, p, c)
        assert all(x % p == c for x in pos.tolist())
        assert [x // p for x in pos.tolist()] == list(range(L))
        pos = impl.positions("zigzag", S, p, c)
        want = list(range(c * h, (c + 1) * h)) + list(range((2 * p - 1 - c) * h, (2 * p - c) * h))
        assert pos.tolist() == want


def pin_ring_golden(impl):
    """The page's 4-GPU ring walk-through, and every chunk visited once."""
    with open(os.path.join(GOLDEN, "ring_walkthrough.json")) as f:
        g = json.load(f)
    p = g["world"]
    for e in g["held"]:
        assert impl.ring_schedule(e["rank"], p)[e["step"]] == e["chunk"], e
    for p in (1, 2, 3, 5, 8):
        for r in range(p):
            sched = impl.ring_schedule(r, p)
            assert sorted(sched) == list(range(p))
            assert sched[0] == r


# ---------------------------------------------------------------------------- forward

def pin_q_zero_closed_form(impl):
    """Q = 0: every visible score is 0, so LSE_i = ln(#visible) and O_i = mean(V_vis)."""
    rng = np.random.default_rng(11)
    for layout in ("contiguous", "striped", "zigzag"):
        for causal in (True, False):
            B, Hq, Hkv, S, d, p = 1, 4, 2, 24, 3, 3 if layout != "zigzag" else 2
            Q = np.zeros((B, Hq, S, d))
            K = _rand(rng, B, Hkv, S, d)
            V = _rand(rng, B, Hkv, S, d)
            for r in range(p):
                rows = impl.positions(layout, S, p, r)
                O, LSE = impl.attention_fwd(Q, K, V, rows, causal)
                for h in range(Hq):
                    g = h // (Hq // Hkv)
                    for t, i in enumerate(rows.tolist()):
                        nvis = i + 1 if causal else S
                        assert abs(LSE[0, h, t] - math.log(nvis)) < 1e-12
                        want = V[0, g, :nvis].mean(axis=0)
                        assert np.max(np.abs(O[0, h, t] - want)) < 1e-12


def pin_v_ones(impl):
    """Softmax rows sum to one: V = 1 gives O = 1 for every visible row."""
    rng = np.random.default_rng(12)
    B, H, S, d = 2, 2, 20, 4
    Q, K = _rand(rng, B, H, S, d), _rand(rng, B, H, S, d)
    V = np.ones((B, H, S, d))
    for causal in (True, False):
        O, _ = impl.attention_fwd(Q, K, V, np.arange(S), causal)
        assert np.max(np.abs(O - 1.0)) < 1e-12


def pin_first_token(impl):
    """Causal: the token at position 0 sees only key 0, so O_0 = V_0, LSE_0 = q0.k0*scale."""
    rng = np.random.default_rng(13)
    B, H, S, d = 1, 2, 16, 5
    Q, K, V = (_rand(rng, B, H, S, d) for _ in range(3))
    for layout, p in (("contiguous", 2), ("zigzag", 2), ("striped", 4)):
        rows = impl.positions(layout, S, p, 0)
        O, LSE = impl.attention_fwd(Q, K, V, rows, True)
        t = int(np.flatnonzero(rows == 0)[0])
        for h in range(H):
            assert np.max(np.abs(O[0, h, t] - V[0, h, 0])) < 1e-14
            want = float(Q[0, h, 0] @ K[0, h, 0]) / math.sqrt(d)
            assert abs(LSE[0, h, t] - want) < 1e-12


def _torch_sdpa(Q, K, V, causal, scale):
    import torch
    import torch.nn.functional as F
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x)) for x in (Q, K, V))
    gqa = q.shape[1] != k.shape[1]
    return F.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale,
                                          enable_gqa=gqa).numpy()


def pin_sdpa_library(impl):
    """p = 1, and every rank's share of it, equal torch SDPA in fp64 (GQA included)."""
    rng = np.random.default_rng(14)
    B, Hq, Hkv, S, d = 2, 4, 2, 32, 6
    Q, K, V = _rand(rng, B, Hq, S, d), _rand(rng, B, Hkv, S, d), _rand(rng, B, Hkv, S, d)
    for causal in (True, False):
        ref = _torch_sdpa(Q, K, V, causal, 1.0 / math.sqrt(d))
        O, _ = impl.attention_fwd(Q, K, V, np.arange(S), causal)
        assert np.max(np.abs(O - ref)) < 1e-12
        for layout in ("contiguous", "striped", "zigzag"):
            for r in range(2):
                rows = impl.positions(layout, S, 2, r)
                O, _ = impl.attention_fwd(Q, K, V, rows, causal)
                assert np.max(np.abs(O - ref[:, :, rows])) < 1e-12


def pin_brute_force(impl):
    """Tiny inputs against unstabilised pure-Python sums over explicit positions."""
    rng = np.random.default_rng(15)
    B, Hq, Hkv, S, d = 1, 2, 1, 8, 3
    Q, K, V = _rand(rng, B, Hq, S, d), _rand(rng, B, Hkv, S, d), _rand(rng, B, Hkv, S, d)
    for layout, p in (("contiguous", 2), ("striped", 2), ("zigzag", 2)):
        for causal in (True, False):
            rows = impl.positions(layout, S, p, 1)
            O, LSE = impl.attention_fwd(Q, K, V, rows, causal)
            for h in range(Hq):
                for t, i in enumerate(rows.tolist()):
                    ws, keys = [], []
                    for j in range(S):
                        if causal and j > i:
                            continue
                        sc = sum(Q[0, h, i, x] * K[0, 0, j, x] for x in range(d)) / math.sqrt(d)
                        ws.append(math.exp(sc))
                        keys.append(j)
                    z = math.fsum(ws)
                    assert abs(LSE[0, h, t] - math.log(z)) < 1e-12
                    for x in range(d):
                        o = math.fsum(w * V[0, 0, j, x] for w, j in zip(ws, keys)) / z
                        assert abs(O[0, h, t, x] - o) < 1e-12


def pin_shift_invariance(impl):
    """K + 1 c^T leaves O unchanged and shifts LSE_i by q_i . c * scale."""
    rng = np.random.default_rng(16)
    B, H, S, d = 1, 2, 16, 4
    Q, K, V = (_rand(rng, B, H, S, d) for _ in range(3))
    c = rng.standard_normal(d)
    rows = impl.positions("zigzag", S, 2, 1)
    O1, L1 = impl.attention_fwd(Q, K, V, rows, True)
    O2, L2 = impl.attention_fwd(Q, K + c, V, rows, True)
    assert np.max(np.abs(O1 - O2)) < 1e-12
    shift = (Q[:, :, rows] @ c) / math.sqrt(d)
    assert np.max(np.abs(L2 - L1 - shift)) < 1e-12


def pin_gqa_repeat(impl):
    """GQA equals MHA on K/V whose heads are repeated group-consecutively."""
    rng = np.random.default_rng(17)
    B, Hq, Hkv, S, d = 1, 6, 2, 12, 3
    Q, K, V = _rand(rng, B, Hq, S, d), _rand(rng, B, Hkv, S, d), _rand(rng, B, Hkv, S, d)
    rows = impl.positions("striped", S, 3, 2)
    O1, L1 = impl.attention_fwd(Q, K, V, rows, True)
    Kr, Vr = np.repeat(K, Hq // Hkv, axis=1), np.repeat(V, Hq // Hkv, axis=1)
    O2, L2 = impl.attention_fwd(Q, Kr, Vr, rows, True)
    assert np.max(np.abs(O1 - O2)) < 1e-14 and np.max(np.abs(L1 - L2)) < 1e-14


def pin_noncausal_key_order(impl):
    """Non-causal attention does not depend on the order of the (key, value) pairs."""
    rng = np.random.default_rng(18)
    q, k, v = _rand(rng, 5, 3), _rand(rng, 9, 3), _rand(rng, 9, 2)
    perm = rng.permutation(9)
    o1, l1 = impl.attend(q, k, v, np.arange(5), np.arange(9), False, 0.7)
    o2, l2 = impl.attend(q, k[perm], v[perm], np.arange(5), np.arange(9)[perm], False, 0.7)
    assert np.max(np.abs(o1 - o2)) < 1e-13 and np.max(np.abs(l1 - l2)) < 1e-13


def pin_blockwise_equals_unblocked(impl):
    """Partials over any chunking of the keys, LSE-merged in any order, equal the
    unblocked result (empty chunks and rows that see nothing in a chunk included)."""
    rng = np.random.default_rng(19)
    S, d, n = 30, 4, 30
    q, k, v = _rand(rng, n, d), _rand(rng, S, d), _rand(rng, S, d)
    qp = np.arange(n)
    full_o, full_l = impl.attend(q, k, v, qp, np.arange(S), True, 0.5)
    for trial in range(6):
        cuts = np.sort(rng.choice(np.arange(S + 1), size=4, replace=True))
        bounds = [0] + cuts.tolist() + [S]
        pieces = [np.arange(bounds[i], bounds[i + 1]) for i in range(len(bounds) - 1)]
        order = rng.permutation(len(pieces))
        acc_o, acc_l = np.zeros((n, d)), np.full(n, -np.inf)
        for idx in order:
            kp = pieces[idx]
            po, pl = impl.attend(q, k[kp], v[kp], qp, kp, True, 0.5)
            acc_o, acc_l = impl.lse_merge(acc_o, acc_l, po, pl)
        assert np.max(np.abs(acc_o - full_o)) < 1e-12
        assert np.max(np.abs(acc_l - full_l)) < 1e-12


def pin_merge_identities(impl):
    """(0, -inf) is the identity of the merge; the merge is commutative and associative."""
    rng = np.random.default_rng(20)
    o = [_rand(rng, 7, 3) for _ in range(3)]
    lse = [_rand(rng, 7) * 3 for _ in range(3)]
    lse[1][2] = -np.inf
    o[1][2] = 0.0
    zo, zl = np.zeros((7, 3)), np.full(7, -np.inf)
    mo, ml = impl.lse_merge(o[0], lse[0], zo, zl)
    assert np.array_equal(mo, o[0]) and np.array_equal(ml, lse[0])
    mo, ml = impl.lse_merge(zo, zl, o[0], lse[0])
    assert np.array_equal(mo, o[0]) and np.array_equal(ml, lse[0])
    a = impl.lse_merge(o[0], lse[0], o[1], lse[1])
    b = impl.lse_merge(o[1], lse[1], o[0], lse[0])
    assert np.max(np.abs(a[0] - b[0])) < 1e-14 and np.max(np.abs(a[1] - b[1])) < 1e-14
    x = impl.lse_merge(*impl.lse_merge(o[0], lse[0], o[1], lse[1]), o[2], lse[2])
    y = impl.lse_merge(o[0], lse[0], *impl.lse_merge(o[1], lse[1], o[2], lse[2]))
    assert np.max(np.abs(x[0] - y[0])) < 1e-13 and np.max(np.abs(x[1] - y[1])) < 1e-13
    # the merged LSE is the log of the summed softmax mass
    assert np.max(np.abs(a[1] - np.log(np.exp(lse[0]) + np.exp(lse[1])))) < 1e-12


def pin_partial_rows_without_keys(impl):
    """A row that sees no key of a chunk gets O = 0 and LSE = -inf."""
    rng = np.random.default_rng(21)
    q, k, v = _rand(rng, 4, 3), _rand(rng, 4, 3), _rand(rng, 4, 3)
    o, l = impl.attend(q, k, v, np.array([0, 1, 2, 3]), np.array([4, 5, 6, 7]), True, 1.0)
    assert np.all(o == 0.0) and np.all(np.isneginf(l))


# ---------------------------------------------------------------------------- backward

def _loss(impl, Q, K, V, dO, rows, causal):
    O, _ = impl.attention_fwd(Q, K, V, rows, causal)
    return float(np.sum(O * dO))


def pin_bwd_finite_differences(impl):
    """Central differences (fp64, h = 1e-6) of l = sum dO . O agree with the backward."""
    rng = np.random.default_rng(22)
    B, Hq, Hkv, S, d = 1, 2, 1, 8, 3
    Q, K, V = _rand(rng, B, Hq, S, d), _rand(rng, B, Hkv, S, d), _rand(rng, B, Hkv, S, d)
    for layout, causal in (("zigzag", True), ("striped", True), ("contiguous", False)):
        rows = impl.positions(layout, S, 2, 1)
        dO = _rand(rng, B, Hq, rows.size, d)
        dQ, dK, dV = impl.attention_bwd(Q, K, V, dO, rows, causal)
        eps = 1e-6
        for name, X, G, sel in (("q", Q, dQ, rows), ("k", K, dK, None), ("v", V, dV, None)):
            for idx in np.ndindex(X.shape):
                Xp, Xm = X.copy(), X.copy()
                Xp[idx] += eps
                Xm[idx] -= eps
                args_p = {"q": Q, "k": K, "v": V}
                args_m = dict(args_p)
                args_p[name], args_m[name] = Xp, Xm
                num = (_loss(impl, args_p["q"], args_p["k"], args_p["v"], dO, rows, causal)
                       - _loss(impl, args_m["q"], args_m["k"], args_m["v"], dO, rows, causal)) / (2 * eps)
                if sel is None:
                    ana = G[idx]
                else:
                    b, h, s, x = idx
                    hit = np.flatnonzero(sel == s)
                    ana = G[b, h, hit[0], x] if hit.size else 0.0
                assert abs(num - ana) < 2e-7, (layout, name, idx, num, ana)


def pin_bwd_autograd_library(impl):
    """The backward equals torch autograd through fp64 SDPA (GQA, rank shares)."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(23)
    B, Hq, Hkv, S, d = 2, 4, 2, 24, 5
    Q, K, V = _rand(rng, B, Hq, S, d), _rand(rng, B, Hkv, S, d), _rand(rng, B, Hkv, S, d)
    for layout, causal in (("zigzag", True), ("striped", True), ("contiguous", False)):
        for r in range(2):
            rows = impl.positions(layout, S, 2, r)
            dO = _rand(rng, B, Hq, rows.size, d)
            q, k, v = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
            out = F.scaled_dot_product_attention(q, k, v, is_causal=causal, enable_gqa=True)
            g = torch.zeros_like(out)
            g[:, :, torch.from_numpy(rows)] = torch.from_numpy(dO)
            out.backward(g)
            dQ, dK, dV = impl.attention_bwd(Q, K, V, dO, rows, causal)
            assert np.max(np.abs(dQ - q.grad.numpy()[:, :, rows])) < 1e-12
            assert np.max(np.abs(dK - k.grad.numpy())) < 1e-12
            assert np.max(np.abs(dV - v.grad.numpy())) < 1e-12


def pin_bwd_identities(impl):
    """sum_j dV_j = sum_i dO_i, sum_j dK_j = 0, and dQ = 0 at global position 0."""
    rng = np.random.default_rng(24)
    B, Hq, Hkv, S, d = 1, 4, 2, 32, 4
    Q, K, V = _rand(rng, B, Hq, S, d), _rand(rng, B, Hkv, S, d), _rand(rng, B, Hkv, S, d)
    rows = impl.positions("zigzag", S, 2, 0)
    dO = _rand(rng, B, Hq, rows.size, d)
    dQ, dK, dV = impl.attention_bwd(Q, K, V, dO, rows, True)
    g = Hq // Hkv
    for kv in range(Hkv):
        want = dO[0, kv * g:(kv + 1) * g].sum(axis=(0, 1))
        assert np.max(np.abs(dV[0, kv].sum(axis=0) - want)) < 1e-12
        assert np.max(np.abs(dK[0, kv].sum(axis=0))) < 1e-12
    t0 = int(np.flatnonzero(rows == 0)[0])
    assert np.max(np.abs(dQ[0, :, t0])) < 1e-14


def pin_bwd_delta(impl):
    """D = rowsum(dO * O): with dO = O it is |O|^2; with dO = e_x it is O[:, x]."""
    rng = np.random.default_rng(25)
    O = _rand(rng, 3, 5, 4)
    assert np.max(np.abs(impl.bwd_delta(O, O) - np.linalg.norm(O, axis=-1) ** 2)) < 1e-12
    e = np.zeros_like(O)
    e[..., 2] = 1.0
    assert np.array_equal(impl.bwd_delta(e, O), O[..., 2])


# ---------------------------------------------------------------------- packed documents

# Boundary lists per batch element: documents of several lengths (one of length 1,
# one empty), one batch element with right padding, one without.
_PACK_S = 24
_PACK_BOUNDS = [[0, 5, 6, 6, 15, 20], [0, 11, 24]]


def _doc_of(bounds, i):
    """Document index of position i by a plain scan of the boundary list; -1 = padding."""
    for k in range(len(bounds) - 1):
        if bounds[k] <= i < bounds[k + 1]:
            return k
    return -1


def pin_document_ids_brute(impl):
    """document_ids against a scan of the boundary definition; bad lists are rejected."""
    for bounds, S in ((_PACK_BOUNDS[0], _PACK_S), (_PACK_BOUNDS[1], _PACK_S), ([0, 0, 3], 7),
                      ([0, 7], 7), ([0, 0], 4)):
        got = impl.document_ids(bounds, S)
        assert got.tolist() == [_doc_of(bounds, i) for i in range(S)], bounds
    for bad in ([1, 5], [0, 5, 3], [0, 30]):
        try:
            impl.document_ids(bad, _PACK_S)
        except ValueError:
            continue
        raise AssertionError(f"accepted {bad}")


def pin_packed_q_zero_closed_form(impl):
    """Q = 0 with packed documents: LSE_i = ln(#visible keys of i's document) and O_i =
    the mean of those V rows; right-padding rows get O = 0 and LSE = -inf."""
    rng = np.random.default_rng(31)
    B, Hq, Hkv, S, d = 2, 2, 1, _PACK_S, 3
    Q = np.zeros((B, Hq, S, d))
    K, V = _rand(rng, B, Hkv, S, d), _rand(rng, B, Hkv, S, d)
    for layout, p in (("contiguous", 3), ("striped", 4), ("zigzag", 2)):
        for causal in (True, False):
            for r in range(p):
                rows = impl.positions(layout, S, p, r)
                O, LSE = impl.attention_fwd(Q, K, V, rows, causal, bounds=_PACK_BOUNDS)
                for b in range(B):
                    e = _PACK_BOUNDS[b]
                    for t, i in enumerate(rows.tolist()):
                        k = _doc_of(e, i)
                        if k < 0:
                            assert np.all(O[b, :, t] == 0.0) and np.all(np.isneginf(LSE[b, :, t]))
                            continue
                        hi = i + 1 if causal else e[k + 1]
                        vis = list(range(e[k], hi))
                        assert np.max(np.abs(LSE[b, :, t] - math.log(len(vis)))) < 1e-12
                        want = V[b, 0, vis].mean(axis=0)
                        assert np.max(np.abs(O[b, :, t] - want)) < 1e-12


def _packed_sdpa_reference(Q, K, V, bounds, causal, scale, grad_out=None):
    """torch SDPA (fp64) run on every document alone; right-padding rows are 0.
    With grad_out, also the autograd gradients of sum(grad_out * O)."""
    import torch
    import torch.nn.functional as F
    q, k, v = (torch.tensor(x, requires_grad=grad_out is not None) for x in (Q, K, V))
    B, H, S, d = Q.shape
    per_batch = []
    for b in range(B):
        e = bounds[b]
        pieces = []
        for j in range(len(e) - 1):
            lo, hi = e[j], e[j + 1]
            if hi > lo:
                pieces.append(F.scaled_dot_product_attention(
                    q[b:b + 1, :, lo:hi], k[b:b + 1, :, lo:hi], v[b:b + 1, :, lo:hi],
                    is_causal=causal, scale=scale, enable_gqa=True))
        pieces.append(torch.zeros((1, H, S - e[-1], d), dtype=torch.float64))
        per_batch.append(torch.cat(pieces, dim=2))
    out = torch.cat(per_batch, dim=0)
    if grad_out is None:
        return out.detach().numpy(), None
    out.backward(torch.from_numpy(grad_out))
    return out.detach().numpy(), (q.grad.numpy(), k.grad.numpy(), v.grad.numpy())


def pin_packed_sdpa_per_document(impl):
    """Packed attention of every rank's share equals torch SDPA run on each document
    alone (fp64, GQA), with zero output on right padding."""
    rng = np.random.default_rng(32)
    B, Hq, Hkv, S, d = 2, 4, 2, _PACK_S, 5
    Q, K, V = _rand(rng, B, Hq, S, d), _rand(rng, B, Hkv, S, d), _rand(rng, B, Hkv, S, d)
    for causal in (True, False):
        ref, _ = _packed_sdpa_reference(Q, K, V, _PACK_BOUNDS, causal, 1.0 / math.sqrt(d))
        for layout, p in (("contiguous", 2), ("striped", 3), ("zigzag", 2)):
            for r in range(p):
                rows = impl.positions(layout, S, p, r)
                O, _ = impl.attention_fwd(Q, K, V, rows, causal, bounds=_PACK_BOUNDS)
                assert np.max(np.abs(O - ref[:, :, rows])) < 1e-12, (layout, r, causal)


def pin_packed_bwd_autograd_per_document(impl):
    """The packed backward equals torch autograd through per-document fp64 SDPA."""
    rng = np.random.default_rng(33)
    B, Hq, Hkv, S, d = 2, 4, 2, _PACK_S, 4
    Q, K, V = _rand(rng, B, Hq, S, d), _rand(rng, B, Hkv, S, d), _rand(rng, B, Hkv, S, d)
    for layout, causal in (("zigzag", True), ("striped", True), ("contiguous", False)):
        for r in range(2):
            rows = impl.positions(layout, S, 2, r)
            dO = _rand(rng, B, Hq, rows.size, d)
            g = np.zeros((B, Hq, S, d))
            g[:, :, rows] = dO
            _, (gq, gk, gv) = _packed_sdpa_reference(Q, K, V, _PACK_BOUNDS, causal,
                                                    1.0 / math.sqrt(d), grad_out=g)
            dQ, dK, dV = impl.attention_bwd(Q, K, V, dO, rows, causal, bounds=_PACK_BOUNDS)
            assert np.max(np.abs(dQ - gq[:, :, rows])) < 1e-12, (layout, r)
            assert np.max(np.abs(dK - gk)) < 1e-12, (layout, r)
            assert np.max(np.abs(dV - gv)) < 1e-12, (layout, r)


def pin_packed_padding_invariance(impl):
    """Values at right-padding positions change no other output or gradient, and
    padding rows/keys get zero output and zero gradient."""
    rng = np.random.default_rng(34)
    B, H, S, d = 2, 2, _PACK_S, 3
    Q, K, V = (_rand(rng, B, H, S, d) for _ in range(3))
    pad = [np.arange(S) >= _PACK_BOUNDS[b][-1] for b in range(B)]
    Q2, K2, V2 = Q.copy(), K.copy(), V.copy()
    for b in range(B):
        for X in (Q2, K2, V2):
            X[b, :, pad[b]] = 100.0 * _rand(rng, H, int(pad[b].sum()), d).transpose(1, 0, 2)
    rows = impl.positions("zigzag", S, 2, 1)
    dO = _rand(rng, B, H, rows.size, d)
    for causal in (True, False):
        O1, L1 = impl.attention_fwd(Q, K, V, rows, causal, bounds=_PACK_BOUNDS)
        O2, L2 = impl.attention_fwd(Q2, K2, V2, rows, causal, bounds=_PACK_BOUNDS)
        g1 = impl.attention_bwd(Q, K, V, dO, rows, causal, bounds=_PACK_BOUNDS)
        g2 = impl.attention_bwd(Q2, K2, V2, dO, rows, causal, bounds=_PACK_BOUNDS)
        assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
        for a, c in zip(g1, g2):
            assert np.array_equal(a, c)
        for b in range(B):
            prow = pad[b][rows]
            assert np.all(O1[b][:, prow] == 0.0) and np.all(np.isneginf(L1[b][:, prow]))
            assert np.all(g1[0][b][:, prow] == 0.0)
            assert np.all(g1[1][b][:, pad[b]] == 0.0) and np.all(g1[2][b][:, pad[b]] == 0.0)


def pin_packed_blockwise_equals_unblocked(impl):
    """Per-chunk partials with packed documents, LSE-merged in ring order, equal the
    unblocked packed result."""
    rng = np.random.default_rng(35)
    B, Hq, Hkv, S, d = 2, 2, 1, _PACK_S, 4
    Q, K, V = _rand(rng, B, Hq, S, d), _rand(rng, B, Hkv, S, d), _rand(rng, B, Hkv, S, d)
    scale = 1.0 / math.sqrt(d)
    for layout, p in (("contiguous", 3), ("zigzag", 2), ("striped", 4)):
        for causal in (True, False):
            r = p - 1
            rows = impl.positions(layout, S, p, r)
            O_ref, L_ref = impl.attention_fwd(Q, K, V, rows, causal, bounds=_PACK_BOUNDS)
            acc_o, acc_l = None, None
            for c in impl.ring_schedule(r, p):
                kp = impl.positions(layout, S, p, c)
                o, l = impl.attention_partial(Q[:, :, rows], K[:, :, kp], V[:, :, kp], rows, kp,
                                              causal, scale, Hq, Hkv, bounds=_PACK_BOUNDS,
                                              seq_total=S)
                acc_o, acc_l = (o, l) if acc_o is None else impl.lse_merge(acc_o, acc_l, o, l)
            assert np.max(np.abs(acc_o - O_ref)) < 1e-12
            fin = np.isfinite(L_ref)
            assert np.array_equal(fin, np.isfinite(acc_l))
            assert np.max(np.abs(acc_l[fin] - L_ref[fin])) < 1e-12


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
