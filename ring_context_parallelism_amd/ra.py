"""Python binding of the C ABI in include/ra.h (argument marshalling only).

Every function here has the name of the C entry point it calls and does nothing
but convert arguments (torch tensors -> device pointers, the current HIP stream,
Python lists -> host pointer arrays) and turn a non-zero status into an
exception.  All validation and every step of the computation happen in libra.so;
there is no fallback: if the library is missing or fails to load, the first call
raises.

A call that returns normally has only ENQUEUED its kernels (the library's RA_OK): a
device fault surfaces at the next synchronisation of the stream, which this binding
does not perform.  With RA_SYNC_CHECK=1 in the environment, every call that launches
kernels synchronises the device afterwards, so a fault is reported by the call that
caused it (a debugging aid: it serialises the host with the GPU).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libra.so")

RA_OK, RA_ERR_NULL, RA_ERR_SHAPE, RA_ERR_UNSUPPORTED, RA_ERR_WORKSPACE, RA_ERR_HIP = range(6)
RA_LAYOUT_CONTIGUOUS, RA_LAYOUT_ZIGZAG, RA_LAYOUT_STRIPED = 0, 1, 2
RA_F32, RA_BF16 = 0, 1
RA_WRITE, RA_MERGE = 0, 1

LAYOUT_IDS = {"contiguous": RA_LAYOUT_CONTIGUOUS, "zigzag": RA_LAYOUT_ZIGZAG,
              "striped": RA_LAYOUT_STRIPED}
DTYPE_IDS = {"f32": RA_F32, "bf16": RA_BF16}

EXPORTS = [
    "ra_block_attn_fwd", "ra_lse_merge", "ra_ring_workspace_size", "ra_ring_fwd",
    "ra_bwd_delta", "ra_bwd_prepare", "ra_block_attn_bwd", "ra_block_attn_bwd_dkdv", "ra_block_attn_bwd_dq",
    "ra_ring_bwd_workspace_size", "ra_ring_bwd", "ra_ring_bwd_noalloc",
    "ra_positions", "ra_visible_pairs", "ra_visible_pairs_packed", "ra_status_str",
    "ra_last_error",
]


class RaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


class Problem(ctypes.Structure):
    """Mirror of ra_problem_t."""
    _fields_ = [
        ("batch", ctypes.c_int64), ("heads_q", ctypes.c_int64), ("heads_kv", ctypes.c_int64),
        ("head_dim", ctypes.c_int64), ("head_dim_padded", ctypes.c_int64),
        ("seq_total", ctypes.c_int64), ("world", ctypes.c_int32), ("layout", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
        ("seg_count", ctypes.c_int32), ("q_stride", ctypes.c_int64 * 3),
        ("kv_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
        ("seg_bounds", ctypes.c_void_p),
    ]


SYNC_CHECK = os.environ.get("RA_SYNC_CHECK", "0") not in ("", "0")

_lib = None
_P = ctypes.c_void_p
_I32, _I64, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_PROB = ctypes.POINTER(Problem)


def lib():
    """Load libra.so once; raise loudly if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                              "python -m ring_context_parallelism_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "ra_block_attn_fwd": [_PROB, _P, _I32, _P, _P, _I32, _P, _P, _I32, _P],
            "ra_lse_merge": [_I64, _I32, _P, _P, _P, _P, _P],
            "ra_ring_workspace_size": [_PROB, ctypes.POINTER(_SZ)],
            "ra_ring_fwd": [_PROB, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P],
            "ra_bwd_delta": [_PROB, _P, _P, _P, _P],
            "ra_bwd_prepare": [_PROB, _P, _P, _P, _P, _P, _P, _P],
            "ra_block_attn_bwd": [_PROB, _P, _I32, _P, _P, _I32, _P, _P, _P, _P, _P, _P, _P],
            "ra_block_attn_bwd_dkdv": [_PROB, _P, _I32, _P, _P, _I32, _P, _P, _P, _P, _P, _I32,
                                       _P],
            "ra_block_attn_bwd_dq": [_PROB, _P, _I32, _P, _P, _I32, _P, _P, _P, _P, _I32, _P],
            "ra_ring_bwd_workspace_size": [_PROB, ctypes.POINTER(_SZ)],
            "ra_ring_bwd": [_PROB, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P],
            "ra_ring_bwd_noalloc": [_PROB, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
            "ra_positions": [_PROB, _I32, ctypes.POINTER(_I64)],
            "ra_visible_pairs": [_PROB, _I32, _I32, ctypes.POINTER(_I64)],
            "ra_visible_pairs_packed": [_PROB, _I32, _I32, ctypes.POINTER(_I32),
                                        ctypes.POINTER(_I64)],
            "ra_status_str": [_I32],
            "ra_last_error": [],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_char_p if name in ("ra_status_str", "ra_last_error") else _I32
        _lib = L
    return _lib


def _status_name(st):
    try:
        return lib().ra_status_str(st).decode()
    except Exception:
        return f"status {st}"


def _check(st):
    if st != RA_OK:
        raise RaError(st, lib().ra_last_error().decode())


def _launched(st):
    """Status check of a call that enqueues kernels (plus the RA_SYNC_CHECK sync)."""
    _check(st)
    if SYNC_CHECK:
        import torch
        torch.cuda.synchronize()


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr_array(items):
    arr = (ctypes.c_void_p * len(items))(*[_ptr(t) for t in items])
    return arr


def make_problem(*, batch, heads_q, heads_kv, head_dim, head_dim_padded, seq_total, world,
                 layout, causal, dtype, scale=0.0, q_stride=None, kv_stride=None,
                 o_stride=None, seg_bounds=None, seg_count=None) -> Problem:
    """Build an ra_problem_t.  Strides default to contiguous [B, H, L, D] tensors.

    seg_bounds: packed-document boundaries, a device int32 tensor [B, n] (or a raw
    device address with seg_count); None for a dense problem."""
    L = seq_total // world if world > 0 else 0
    D = head_dim_padded
    p = Problem()
    p.batch, p.heads_q, p.heads_kv = batch, heads_q, heads_kv
    p.head_dim, p.head_dim_padded, p.seq_total = head_dim, head_dim_padded, seq_total
    p.world = world
    p.layout = LAYOUT_IDS[layout] if isinstance(layout, str) else layout
    p.causal = int(bool(causal))
    p.dtype = DTYPE_IDS[dtype] if isinstance(dtype, str) else dtype
    p.scale = scale
    if seg_bounds is None:
        p.seg_count, p.seg_bounds = 0, None
    else:
        p.seg_bounds = _ptr(seg_bounds)
        p.seg_count = seg_count if seg_count is not None else int(seg_bounds.shape[-1])
    p.q_stride[:] = q_stride or (heads_q * L * D, L * D, D)
    p.kv_stride[:] = kv_stride or (heads_kv * L * D, L * D, D)
    p.o_stride[:] = o_stride or (heads_q * L * D, L * D, D)
    return p


# ------------------------------------------------------------------------ entry points

def ra_block_attn_fwd(prob, q, q_chunk, k, v, kv_chunk, o, lse, mode, stream=None):
    _launched(lib().ra_block_attn_fwd(ctypes.byref(prob), _ptr(q), q_chunk, _ptr(k), _ptr(v),
                                   kv_chunk, _ptr(o), _ptr(lse), mode, _stream(stream)))


def ra_lse_merge(rows, d, o_acc, lse_acc, o_part, lse_part, stream=None):
    _launched(lib().ra_lse_merge(rows, d, _ptr(o_acc), _ptr(lse_acc), _ptr(o_part),
                              _ptr(lse_part), _stream(stream)))


def ra_ring_workspace_size(prob) -> int:
    n = _SZ(0)
    _check(lib().ra_ring_workspace_size(ctypes.byref(prob), ctypes.byref(n)))
    return n.value


def ra_ring_fwd(prob, rank, q, k_chunks, v_chunks, out, lse, ws, ws_bytes=None, stream=None):
    ks, vs = _ptr_array(k_chunks), _ptr_array(v_chunks)
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _launched(lib().ra_ring_fwd(ctypes.byref(prob), rank, _ptr(q), ks, vs, _ptr(out), _ptr(lse),
                             _ptr(ws), ws_bytes, _stream(stream)))


def ra_bwd_delta(prob, out, dout, delta, stream=None):
    _launched(lib().ra_bwd_delta(ctypes.byref(prob), _ptr(out), _ptr(dout), _ptr(delta),
                              _stream(stream)))


def ra_bwd_prepare(prob, out, dout, delta, dq, dk_chunks, dv_chunks, stream=None):
    _launched(lib().ra_bwd_prepare(ctypes.byref(prob), _ptr(out), _ptr(dout), _ptr(delta), _ptr(dq),
                                _ptr_array(dk_chunks), _ptr_array(dv_chunks), _stream(stream)))


def ra_block_attn_bwd(prob, q, q_chunk, k, v, kv_chunk, dout, lse, delta, dq, dk, dv,
                      stream=None):
    _launched(lib().ra_block_attn_bwd(ctypes.byref(prob), _ptr(q), q_chunk, _ptr(k), _ptr(v),
                                   kv_chunk, _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dq),
                                   _ptr(dk), _ptr(dv), _stream(stream)))


def ra_block_attn_bwd_dkdv(prob, q, q_chunk, k, v, kv_chunk, dout, lse, delta, dk, dv,
                           mode=RA_MERGE, stream=None):
    _launched(lib().ra_block_attn_bwd_dkdv(ctypes.byref(prob), _ptr(q), q_chunk, _ptr(k), _ptr(v),
                                        kv_chunk, _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dk),
                                        _ptr(dv), mode, _stream(stream)))


def ra_block_attn_bwd_dq(prob, q, q_chunk, k, v, kv_chunk, dout, lse, delta, dq, mode=RA_MERGE,
                         stream=None):
    _launched(lib().ra_block_attn_bwd_dq(ctypes.byref(prob), _ptr(q), q_chunk, _ptr(k), _ptr(v),
                                      kv_chunk, _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dq),
                                      mode, _stream(stream)))


def ra_ring_bwd_workspace_size(prob) -> int:
    n = _SZ(0)
    _check(lib().ra_ring_bwd_workspace_size(ctypes.byref(prob), ctypes.byref(n)))
    return n.value


def ra_ring_bwd(prob, rank, q, k_chunks, v_chunks, out, dout, lse, dq, dk_chunks, dv_chunks,
                ws, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _launched(lib().ra_ring_bwd(ctypes.byref(prob), rank, _ptr(q), _ptr_array(k_chunks),
                             _ptr_array(v_chunks), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq),
                             _ptr_array(dk_chunks), _ptr_array(dv_chunks), _ptr(ws), ws_bytes,
                             _stream(stream)))


def ra_ring_bwd_noalloc(prob, rank, q, k_chunks, v_chunks, out, dout, lse, dq, dk_chunks,
                        dv_chunks, stream=None):
    _launched(lib().ra_ring_bwd_noalloc(ctypes.byref(prob), rank, _ptr(q), _ptr_array(k_chunks),
                                        _ptr_array(v_chunks), _ptr(out), _ptr(dout), _ptr(lse),
                                        _ptr(dq), _ptr_array(dk_chunks), _ptr_array(dv_chunks),
                                        _stream(stream)))


def ra_positions(prob, chunk) -> np.ndarray:
    L = prob.seq_total // prob.world if prob.world > 0 else 0
    out = np.empty(max(L, 1), dtype=np.int64)
    _check(lib().ra_positions(ctypes.byref(prob), chunk,
                              out.ctypes.data_as(ctypes.POINTER(_I64))))
    return out


def ra_visible_pairs(prob, q_chunk, kv_chunk) -> int:
    n = _I64(0)
    _check(lib().ra_visible_pairs(ctypes.byref(prob), q_chunk, kv_chunk, ctypes.byref(n)))
    return n.value


def ra_visible_pairs_packed(prob, q_chunk, kv_chunk, host_bounds) -> int:
    """host_bounds: int32 [B, seg_count] boundary lists in host memory."""
    b = np.ascontiguousarray(host_bounds, dtype=np.int32)
    n = _I64(0)
    _check(lib().ra_visible_pairs_packed(ctypes.byref(prob), q_chunk, kv_chunk,
                                         b.ctypes.data_as(ctypes.POINTER(_I32)), ctypes.byref(n)))
    return n.value


def ra_status_str(status) -> str:
    return lib().ra_status_str(status).decode()


def ra_last_error() -> str:
    return lib().ra_last_error().decode()
