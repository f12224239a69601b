"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws random numbers and rounds them to the storage dtype; it
holds none of the attention arithmetic, so both the HIP path and the CPU oracle can
take their inputs from it without sharing any of the method's code.

Recipe (the same for every workload):
  * NumPy ``default_rng(seed)`` (PCG64);
  * draw fp32 tensors in the order Q, K, V, then dO (backward workloads only), each
    in global token order [B, H, S, d] (the tabular workload draws its
    (1, rows, features, embed) tensors and folds them, see ``fold_rows_axis``);
  * multiply by the workload's value scale, then round to bf16 with
    round-to-nearest-even where the workload is bf16; the rounded values are kept
    as exactly-representable fp32 so the oracle can upcast them to fp64 exactly.

Workloads (sizes from the pages' own models):
  tiny_fp32     -- 1 head, d 64, S 1024, p 4 contiguous, rank 1, causal, fp32
  llama_share   -- 16 heads x d 128 (hidden 2048), S 16384, p 2 contiguous, rank 1,
                   causal, N(0,1)*0.5, bf16 (ringmaster page, "Benchmark": Llama
                   hidden 2048 / 16 heads)
  gqa_striped   -- 32 Q / 8 KV heads, d 128, S 131072, p 8 striped, rank 3, causal,
                   N(0,1), bf16
  tabular_rows  -- nanoTabPFN-shaped (1, 150000 rows, 5 features, embed 96), 4 heads
                   x d 24 stored padded to 32, attention over rows with the feature
                   axis folded into the batch, p 4, rank 0, non-causal, U(-1,1), fp32
                   and bf16 (Mosaic post, "The Problem" / "The Implementation");
                   tabular_rows_bf16 is the same draw in bf16
  zigzag_fwdbwd -- 16 heads x d 128, S 131072, p 2 zigzag, rank 0, causal, forward
                   then backward, N(0,1)*0.5 including dO, bf16
  packed_fwdbwd -- zigzag_fwdbwd's shape with packed documents and right padding
                   (ringmaster page, "Native recurrent context parallelism": packed
                   attention by global position boundaries, globally right-padded
                   batches); see ``document_bounds`` for the length mix

Packed documents (workloads with ``docs``): a second generator,
``default_rng([seed, 1])``, so Q/K/V/dO are the same draws as without packing.
Per batch element: the valid length is S - floor(u * pad_frac * S) with
u ~ U(0, 1) (the right padding); document lengths are drawn log-uniformly in
[min_len, max_len] (rounded down to an integer) until they reach the valid length,
the last one cut there.  The boundary lists of the batch are padded to one length
by repeating their last entry (empty documents).
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    dtype: str            # "f32" or "bf16": storage and MFMA operand type
    batch: int
    heads_q: int
    heads_kv: int
    head_dim: int         # true head dim (sets the default scale)
    head_dim_padded: int  # storage head dim (pad columns are zero)
    seq_total: int
    world: int
    layout: str           # "contiguous" | "zigzag" | "striped"
    rank: int
    causal: bool
    dist: str             # "normal" | "uniform"
    value_scale: float
    backward: bool = False
    fold: tuple | None = None  # (rows, features, embed) for the tabular fold
    docs: tuple | None = None  # (min_len, max_len, pad_frac): packed documents

    @property
    def chunk_len(self) -> int:
        return self.seq_total // self.world

    def with_dtype(self, dtype: str) -> "Workload":
        return dataclasses.replace(self, dtype=dtype)

    def resized(self, **kw) -> "Workload":
        """Same recipe at other sizes (used for the oracle-sized parity cases)."""
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 0, "f32", 1, 1, 1, 64, 64, 1024, 4, "contiguous", 1,
                          True, "normal", 1.0),
    "llama_share": Workload("llama_share", 1, "bf16", 1, 16, 16, 128, 128, 16384, 2,
                            "contiguous", 1, True, "normal", 0.5),
    "gqa_striped": Workload("gqa_striped", 2, "bf16", 1, 32, 8, 128, 128, 131072, 8,
                            "striped", 3, True, "normal", 1.0),
    "tabular_rows": Workload("tabular_rows", 3, "f32", 5, 4, 4, 24, 32, 150000, 4,
                             "contiguous", 0, False, "uniform", 1.0, fold=(150000, 5, 96)),
    "tabular_rows_bf16": Workload("tabular_rows_bf16", 3, "bf16", 5, 4, 4, 24, 32, 150000, 4,
                                  "contiguous", 0, False, "uniform", 1.0,
                                  fold=(150000, 5, 96)),
    "zigzag_fwdbwd": Workload("zigzag_fwdbwd", 4, "bf16", 1, 16, 16, 128, 128, 131072, 2,
                              "zigzag", 0, True, "normal", 0.5, backward=True),
    "packed_fwdbwd": Workload("packed_fwdbwd", 5, "bf16", 1, 16, 16, 128, 128, 131072, 2,
                              "zigzag", 0, True, "normal", 0.5, backward=True,
                              docs=(256, 32768, 0.05)),
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    bias = ((bits >> 16) & 1) + np.uint32(0x7FFF)
    out = ((bits + bias) & np.uint32(0xFFFF0000)).astype(np.uint32)
    return out.view(np.float32)


def fold_rows_axis(x: np.ndarray, heads: int) -> np.ndarray:
    """(1, rows, features, embed) -> (features, heads, rows, embed/heads).

    Moves the attended axis (rows) to the sequence slot and folds the feature axis
    into the batch, splitting the embedding into heads, as the Mosaic post's
    multi-axis attention does before dispatch ("The Implementation").  No projection
    is applied: projections are module weights, not part of the attention step.
    """
    one, rows, feats, embed = x.shape
    assert one == 1 and embed % heads == 0
    y = x.reshape(rows, feats, heads, embed // heads)
    return np.ascontiguousarray(y.transpose(1, 2, 0, 3))


def _draw(rng, shape, dist, value_scale):
    if dist == "normal":
        a = rng.standard_normal(shape, dtype=np.float32)
    elif dist == "uniform":
        a = rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)
    else:
        raise ValueError(dist)
    if value_scale != 1.0:
        a *= np.float32(value_scale)
    return a


def document_bounds(w: Workload) -> np.ndarray:
    """int32 [B, n] document boundaries (global positions) of a packed workload."""
    min_len, max_len, pad_frac = w.docs
    rng = np.random.default_rng([w.seed, 1])
    S = w.seq_total
    lists = []
    for _ in range(w.batch):
        valid = S - int(np.floor(rng.uniform() * pad_frac * S))
        e = [0]
        while e[-1] < valid:
            n = int(np.exp(rng.uniform(np.log(min_len), np.log(max_len))))
            e.append(min(valid, e[-1] + max(1, n)))
        lists.append(e)
    n = max(len(e) for e in lists)
    return np.array([e + [e[-1]] * (n - len(e)) for e in lists], dtype=np.int32)


def generate(w: Workload):
    """Global-order fp32 arrays {"q", "k", "v"[, "do"]} for workload `w`, plus
    "bounds" (int32 [B, n]) for packed workloads.

    Values are exactly bf16 where ``w.dtype == "bf16"``.  The head dim is the true
    head dim (no padding); padding is a storage detail of the GPU side.
    """
    rng = np.random.default_rng(w.seed)
    out = {}
    names = ["q", "k", "v"] + (["do"] if w.backward else [])
    for nm in names:
        if w.fold is not None:
            rows, feats, embed = w.fold
            a = fold_rows_axis(_draw(rng, (1, rows, feats, embed), w.dist, w.value_scale),
                               w.heads_q)
        else:
            heads = w.heads_kv if nm in ("k", "v") else w.heads_q
            a = _draw(rng, (w.batch, heads, w.seq_total, w.head_dim), w.dist, w.value_scale)
        if w.dtype == "bf16":
            a = round_bf16(a)
        out[nm] = a
    if w.docs is not None:
        out["bounds"] = document_bounds(w)
    return out

