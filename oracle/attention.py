"""Plain, slow, obviously-correct fp64 CPU oracle for the blockwise ring-attention step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute
this module: only the tests, the smoke check and the CPU-baseline leg of the
benchmark use it.  It shares no code with the HIP library and imports nothing from
it; it takes NumPy arrays and returns NumPy arrays.

What it computes is the plain definition that the blockwise method reaches exactly
(up to rounding order), not the method itself:

* attention is softmax(Q K^T / sqrt(d)) V over the whole key sequence
  (Mosaic post, "The Problem: Attention Doesn't Scale"), with the row-wise softmax
  normaliser of the "Vanilla Transformer" slides of "Ring Attention & Friends";
* the ring computes per-chunk partial results and normalises at the end, so each
  rank ends with the complete attention output for its query chunk (Mosaic post,
  "How Ring Attention Works"); the oracle therefore never rings, never rescales
  online and never merges: each query row is computed over its complete key row;
* causal masking is autoregressive, on global token positions (ringmaster page,
  "Native recurrent context parallelism": dense causal sequences; "Ring Attention &
  Friends", "Striped Attention" slide);
* the sequence layouts are the dense contiguous shard and the head/tail balancer
  of the ringmaster page ("Layout": shard.py, balancers.py) and the striped layout
  named on the "Striped Attention" slide;
* the backward is the analytic gradient of the loss sum_i dO_i . O_i over this
  rank's rows (the "flash-style reverse-ring backward" of the ringmaster page,
  "Status", recomputes exactly these quantities).

Readings taken where the pages are silent:

* scale = 1/sqrt(d_true): the sqrt(d) of the formula is the model's head dim;
  storage padding of the head dim is not the oracle's concern;
* LSE is the natural log of sum_j exp(scaled score), in the same units as the
  scaled scores;
* the causal diagonal is inclusive: key j is visible to query i iff pos_j <= pos_i;
* a row with no visible key has output 0 and LSE -inf (the identity of the merge);
* the ring passes KV from rank r to rank r+1, so at step s rank r holds chunk
  (r - s) mod p;
* striped: token i belongs to chunk i mod p; zigzag (head/tail): rank r holds the
  sub-blocks r and 2p-1-r of size S/(2p), concatenated in ascending order;
  contiguous: rank r holds [r L, (r+1) L); inside every chunk the tokens are kept
  in ascending global order;
* GQA grouping is consecutive: query head h reads KV head h // (Hq / Hkv);
* packed documents (ringmaster page, "Native recurrent context parallelism":
  packed attention by global position boundaries, globally right-padded
  batches): a batch element's sequence is cut by nondecreasing global positions
  0 = e_0 <= e_1 <= ... <= e_n <= S into documents [e_k, e_k+1); a key is visible
  only to queries of its own document (and, when causal, at or after it);
  positions at or past e_n are right padding, seen by no query and seeing
  nothing themselves (output 0, LSE -inf, no gradient).

Parity pins (tests/test_oracle_pins.py) tie every function here to something other
than itself: closed forms, special cases that reduce to a library routine
(torch scaled_dot_product_attention and autograd in fp64), brute force on tiny
inputs, finite differences, exact identities, and the page's own worked ring
example (tests/golden/).  No function here is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

LAYOUTS = ("contiguous", "zigzag", "striped")


# ----------------------------------------------------------------------------------
# Sequence layouts and the ring schedule
# ----------------------------------------------------------------------------------

def chunk_of_token(layout: str, seq_total: int, world: int) -> np.ndarray:
    """For every global token position i in [0, S), the chunk (rank) that holds it.

    contiguous -- dense sharding into p equal runs (ringmaster, "Layout": shard.py);
    striped    -- token i goes to chunk i mod p ("Ring Attention & Friends",
                  "Striped Attention"; the token assignment is the reading taken);
    zigzag     -- the head/tail balancer (ringmaster, "Layout": balancers.py): the
                  sequence is cut into 2p equal sub-blocks and rank r receives
                  sub-blocks r and 2p-1-r.
    """
    S, p = int(seq_total), int(world)
    i = np.arange(S, dtype=np.int64)
    if layout == "contiguous":
        if S % p:
            raise ValueError("S must be a multiple of p")
        return i // (S // p)
    if layout == "striped":
        if S % p:
            raise ValueError("S must be a multiple of p")
        return i % p
    if layout == "zigzag":
        if S % (2 * p):
            raise ValueError("S must be a multiple of 2p")
        sub = i // (S // (2 * p))
        return np.where(sub < p, sub, 2 * p - 1 - sub)
    raise ValueError(f"unknown layout {layout!r}")


def positions(layout: str, seq_total: int, world: int, chunk: int) -> np.ndarray:
    """Global positions of the tokens chunk `chunk` holds, in its local order.

    Local order is ascending global order within the chunk, so local index t maps to
    the t-th smallest global position owned by the chunk.
    """
    owner = chunk_of_token(layout, seq_total, world)
    return np.flatnonzero(owner == chunk).astype(np.int64)


def ring_schedule(rank: int, world: int) -> list[int]:
    """KV chunk ids rank `rank` holds at ring steps 0..p-1.

    Simulates the ring of the Mosaic post ("How Ring Attention Works"): every rank
    starts with its own chunk; after each step every rank sends what it holds to the
    next rank and receives from the previous one.
    """
    held = list(range(world))
    order = []
    for _ in range(world):
        order.append(held[rank])
        held = [held[(r - 1) % world] for r in range(world)]  # receive from r-1
    return order


# ----------------------------------------------------------------------------------
# Small helpers (named so the pin tests can plant a mistake in exactly one place)
# ----------------------------------------------------------------------------------

def _default_scale(head_dim: int) -> float:
    """1/sqrt(d) of the attention formula (Mosaic post, "The Problem")."""
    return 1.0 / math.sqrt(head_dim)


def _visible(k_pos: np.ndarray, q_pos: np.ndarray) -> np.ndarray:
    """Causal visibility matrix [n_q, n_k]: key j visible to query i iff pos_j <= pos_i."""
    return k_pos[None, :] <= q_pos[:, None]


def document_ids(bounds, seq_total: int) -> np.ndarray:
    """Document index of every global position of one batch element; -1 = padding.

    `bounds` are the global positions 0 = e_0 <= e_1 <= ... <= e_n <= S; position i
    belongs to the document k with e_k <= i < e_k+1 (an empty document, e_k = e_k+1,
    owns nothing), and positions i >= e_n are right padding.
    """
    e = np.asarray(bounds, dtype=np.int64)
    S = int(seq_total)
    if e.ndim != 1 or e.size < 2 or e[0] != 0 or np.any(np.diff(e) < 0) or e[-1] > S:
        raise ValueError("bounds must be nondecreasing global positions from 0 to at most S")
    doc = np.full(S, -1, dtype=np.int64)
    for k in range(e.size - 1):
        doc[e[k]:e[k + 1]] = k
    return doc


def _same_document(k_doc: np.ndarray, q_doc: np.ndarray) -> np.ndarray:
    """[n_q, n_k]: key in the query's document; padding (-1) matches nothing."""
    return (k_doc[None, :] == q_doc[:, None]) & (k_doc[None, :] >= 0)


def _doc_rows(bounds, batch: int, seq_total: int):
    """Per batch element document ids, or None for a dense (unpacked) problem."""
    if bounds is None:
        return None
    if len(bounds) != batch:
        raise ValueError("one boundary list per batch element")
    return [document_ids(bounds[bi], seq_total) for bi in range(batch)]


def _kv_head(h: int, heads_q: int, heads_kv: int) -> int:
    """KV head read by query head h under consecutive GQA grouping."""
    return h // (heads_q // heads_kv)


# ----------------------------------------------------------------------------------
# Forward
# ----------------------------------------------------------------------------------

def attend(q, k, v, q_pos, k_pos, causal: bool, scale: float, row_block: int = 256,
           q_doc=None, k_doc=None):
    """Exact attention of query rows q [n, d] over the keys k [m, d] / values v [m, dv].

    Implements softmax(q k^T * scale) v row by row with the row-wise normaliser, in
    fp64, over every key at once (no tiling of the key axis, no online rescaling).
    With document ids (q_doc, k_doc) a key is visible only inside its own document.
    Returns (O [n, dv], lse [n]); a row with no visible key gets O = 0, lse = -inf.
    Rows are processed in blocks of `row_block` only to bound memory.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    n = q.shape[0]
    out = np.zeros((n, v.shape[1]), dtype=np.float64)
    lse = np.full(n, -np.inf, dtype=np.float64)
    for a in range(0, n, row_block):
        b = min(n, a + row_block)
        s = (q[a:b] @ k.T) * scale
        if causal:
            s = np.where(_visible(k_pos, q_pos[a:b]), s, -np.inf)
        if q_doc is not None:
            s = np.where(_same_document(np.asarray(k_doc), np.asarray(q_doc)[a:b]), s, -np.inf)
        m = s.max(axis=1) if s.shape[1] else np.full(b - a, -np.inf)
        live = np.isfinite(m)
        m0 = np.where(live, m, 0.0)
        e = np.exp(s - m0[:, None])  # exp(-inf) = 0 for masked keys
        z = e.sum(axis=1)
        zsafe = np.where(live, z, 1.0)
        out[a:b] = np.where(live[:, None], (e @ v) / zsafe[:, None], 0.0)
        lse[a:b] = np.where(live, m0 + np.log(zsafe), -np.inf)
    return out, lse


def _visible_key_limit(q_pos_block: np.ndarray, causal: bool, seq_total: int) -> int:
    """Keys in global order that any row of the block can see (a prefix when causal).

    Masked keys contribute exact zeros, so dropping the invisible suffix is exact.
    """
    if not causal or q_pos_block.size == 0:
        return seq_total
    return int(q_pos_block.max()) + 1


def attention_fwd(Qg, Kg, Vg, rows, causal: bool, scale: float | None = None,
                  row_block: int = 256, heads=None, bounds=None):
    """Exact attention of one rank's query rows against the whole global sequence.

    Qg [B, Hq, S, d], Kg / Vg [B, Hkv, S, d] in global token order; `rows` are the
    global positions of the rank's query rows (its share), in local order.
    `heads` optionally restricts the computation to those query heads (sampling).
    `bounds` (one boundary list per batch element) packs documents; None = dense.
    Returns O [B, len(heads) or Hq, len(rows), d] and LSE [B, ..., len(rows)] in fp64.
    """
    B, Hq, S, d = Qg.shape
    Hkv = Kg.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if scale is None:
        scale = _default_scale(d)
    rows = np.asarray(rows, dtype=np.int64)
    key_pos = np.arange(S, dtype=np.int64)
    heads = list(range(Hq)) if heads is None else list(heads)
    docs = _doc_rows(bounds, B, S)
    O = np.zeros((B, len(heads), rows.size, Vg.shape[3]), dtype=np.float64)
    LSE = np.full((B, len(heads), rows.size), -np.inf, dtype=np.float64)
    for bi in range(B):
        for hi, h in enumerate(heads):
            g = _kv_head(h, Hq, Hkv)
            for a in range(0, rows.size, row_block):
                rb = rows[a:a + row_block]
                lim = _visible_key_limit(rb, causal, S)
                qd = kd = None
                if docs is not None:
                    qd, kd = docs[bi][rb], docs[bi][:lim]
                o, l = attend(Qg[bi, h, rb], Kg[bi, g, :lim], Vg[bi, g, :lim], rb,
                              key_pos[:lim], causal, scale, row_block, qd, kd)
                O[bi, hi, a:a + rb.size] = o
                LSE[bi, hi, a:a + rb.size] = l
    return O, LSE


def attention_partial(Q_rows, K_chunk, V_chunk, q_pos, k_pos, causal: bool,
                      scale: float, heads_q: int, heads_kv: int, bounds=None,
                      seq_total: int | None = None):
    """Per-step partial result: one rank's query rows against ONE KV chunk.

    Q_rows [B, Hq, n, d]; K_chunk / V_chunk [B, Hkv, m, d]; positions are global.
    `bounds` (with `seq_total`) packs documents as in attention_fwd.
    Returns (O_s, LSE_s) in fp64, with O_s = 0 and LSE_s = -inf on rows that see no
    key of this chunk.  This is the quantity each ring step emits before merging.
    """
    B = Q_rows.shape[0]
    docs = _doc_rows(bounds, B, seq_total) if bounds is not None else None
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    O = np.zeros(Q_rows.shape[:3] + (V_chunk.shape[3],), dtype=np.float64)
    LSE = np.full(Q_rows.shape[:3], -np.inf, dtype=np.float64)
    for bi in range(B):
        qd = kd = None
        if docs is not None:
            qd, kd = docs[bi][q_pos], docs[bi][k_pos]
        for h in range(heads_q):
            g = _kv_head(h, heads_q, heads_kv)
            O[bi, h], LSE[bi, h] = attend(Q_rows[bi, h], K_chunk[bi, g], V_chunk[bi, g],
                                          q_pos, k_pos, causal, scale, 256, qd, kd)
    return O, LSE


def lse_merge(o_a, lse_a, o_b, lse_b):
    """Merge two partial results computed over disjoint key sets.

    The merged LSE is log(exp(lse_a) + exp(lse_b)); the merged output is the
    average of the two partial outputs weighted by each part's share of the total
    softmax mass, exp(lse_part - lse).  A part with lse = -inf saw no key and is
    the identity.  (ringmaster page, "Layout": ring/merge.py, the online-softmax LSE
    merge; Mosaic post, "How Ring Attention Works": accumulate, normalise at the end.)
    """
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    a_empty = np.isneginf(lse_a)
    b_empty = np.isneginf(lse_b)
    both = ~a_empty & ~b_empty
    hi = np.where(both, np.maximum(lse_a, lse_b), 0.0)
    wa_raw = np.exp(np.where(both, lse_a - hi, 0.0))
    wb_raw = np.exp(np.where(both, lse_b - hi, 0.0))
    lse = np.where(both, hi + np.log(wa_raw + wb_raw), np.where(b_empty, lse_a, lse_b))
    wa = np.where(both, wa_raw / (wa_raw + wb_raw), np.where(b_empty, 1.0, 0.0))
    wb = np.where(both, wb_raw / (wa_raw + wb_raw), np.where(b_empty, 0.0, 1.0))
    o = wa[..., None] * o_a + wb[..., None] * o_b
    return o, lse


# ----------------------------------------------------------------------------------
# Backward
# ----------------------------------------------------------------------------------

def attention_bwd(Qg, Kg, Vg, dO_rows, rows, causal: bool, scale: float | None = None,
                  row_block: int = 256, heads=None, bounds=None):
    """Analytic gradient of l = sum_{i in rows} dO_i . O_i for one rank's query rows.

    With P the row softmax of the scaled, masked scores S:
      dV_j  = sum_i P_ij dO_i
      dP_ij = dO_i . v_j
      D_i   = dO_i . O_i
      dS_ij = P_ij (dP_ij - D_i)
      dQ_i  = scale * sum_j dS_ij k_j
      dK_j  = scale * sum_i dS_ij q_i
    GQA: dK, dV of a KV head are summed over the query heads that read it.
    Only this rank's rows contribute (the gradient share of one rank).

    Returns dQ [B, Hq, n, d] (rows in local order), dK and dV [B, Hkv, S, d] in
    global order, all fp64.  `heads` optionally restricts dQ to those query heads
    (dO_rows then holds only those heads; dK and dV get only their contributions).
    `bounds` packs documents as in attention_fwd; a row that sees no key (right
    padding) has P = 0 and contributes nothing.
    """
    B, Hq, S, d = Qg.shape
    Hkv = Kg.shape[1]
    if scale is None:
        scale = _default_scale(d)
    rows = np.asarray(rows, dtype=np.int64)
    key_pos = np.arange(S, dtype=np.int64)
    heads = list(range(Hq)) if heads is None else list(heads)
    docs = _doc_rows(bounds, B, S)
    dQ = np.zeros((B, len(heads), rows.size, d), dtype=np.float64)
    dK = np.zeros((B, Hkv, S, d), dtype=np.float64)
    dV = np.zeros((B, Hkv, S, Vg.shape[3]), dtype=np.float64)
    for bi in range(B):
        for hi, h in enumerate(heads):
            g = _kv_head(h, Hq, Hkv)
            Qh = Qg[bi, h]
            for a in range(0, rows.size, row_block):
                rb = rows[a:a + row_block]
                lim = _visible_key_limit(rb, causal, S)
                q = np.asarray(Qh[rb], dtype=np.float64)
                k = np.asarray(Kg[bi, g, :lim], dtype=np.float64)
                v = np.asarray(Vg[bi, g, :lim], dtype=np.float64)
                do = np.asarray(dO_rows[bi, hi, a:a + rb.size], dtype=np.float64)
                s = (q @ k.T) * scale
                if causal:
                    s = np.where(_visible(key_pos[:lim], rb), s, -np.inf)
                if docs is not None:
                    s = np.where(_same_document(docs[bi][:lim], docs[bi][rb]), s, -np.inf)
                m = s.max(axis=1)
                live = np.isfinite(m)
                e = np.exp(s - np.where(live, m, 0.0)[:, None])
                P = np.where(live[:, None], e / np.where(live, e.sum(axis=1), 1.0)[:, None], 0.0)
                O = P @ v
                D = np.sum(do * O, axis=1)
                dP = do @ v.T
                dS = P * (dP - D[:, None])
                dQ[bi, hi, a:a + rb.size] = (dS @ k) * scale
                dK[bi, g, :lim] += (dS.T @ q) * scale
                dV[bi, g, :lim] += P.T @ do
    return dQ, dK, dV


def bwd_delta(dO, O):
    """D_i = sum_d dO_i,d * O_i,d: the per-row term of dS = P (dP - D)."""
    return np.sum(np.asarray(dO, dtype=np.float64) * np.asarray(O, dtype=np.float64), axis=-1)
