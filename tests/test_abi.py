"""Host-side checks of the C ABI: no GPU needed, no kernel is launched.

* libra.so loads and exports every function include/ra.h declares;
* the host-only position map and visible-pair counts agree with the oracle's own
  (independently written) layout arithmetic;
* every validation failure returns its documented status before anything is
  enqueued (these paths never reach the HIP runtime).
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from ring_context_parallelism_amd import ra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def built_library():
    if not os.path.exists(ra.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    ra.lib()


def _declared():
    src = open(os.path.join(ROOT, "include", "ra.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 12
    L = ctypes.CDLL(ra.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(ra.EXPORTS)


def _prob(**kw):
    base = dict(batch=1, heads_q=4, heads_kv=2, head_dim=64, head_dim_padded=64,
                seq_total=48, world=4, layout="contiguous", causal=True, dtype="bf16")
    base.update(kw)
    return ra.make_problem(**base)


@pytest.mark.parametrize("layout", oracle.LAYOUTS)
@pytest.mark.parametrize("world", [1, 2, 3, 4, 8])
def test_positions_match_oracle(layout, world):
    S = 2 * world * 7
    p = _prob(seq_total=S, world=world, layout=layout)
    for c in range(world):
        assert ra.ra_positions(p, c).tolist() == oracle.positions(layout, S, world, c).tolist()


@pytest.mark.parametrize("layout", oracle.LAYOUTS)
@pytest.mark.parametrize("causal", [True, False])
def test_visible_pairs_match_brute_force(layout, causal):
    S, world = 96, 4
    p = _prob(seq_total=S, world=world, layout=layout, causal=causal)
    for cq in range(world):
        qp = oracle.positions(layout, S, world, cq)
        for ck in range(world):
            kp = oracle.positions(layout, S, world, ck)
            want = int(np.sum(kp[None, :] <= qp[:, None])) if causal else qp.size * kp.size
            assert ra.ra_visible_pairs(p, cq, ck) == want


_BOUNDS = {
    # per-batch lists (padded with repeats), documents that straddle chunks, empty
    # and length-1 documents, right padding
    96: np.array([[0, 7, 8, 8, 40, 41, 77, 90], [0, 50, 96, 96, 96, 96, 96, 96]], np.int32),
}


@pytest.mark.parametrize("layout", oracle.LAYOUTS)
@pytest.mark.parametrize("causal", [True, False])
def test_visible_pairs_packed_match_brute_force(layout, causal):
    S, world = 96, 4
    bounds = _BOUNDS[S]
    p = _prob(batch=2, seq_total=S, world=world, layout=layout, causal=causal,
              seg_bounds=FAKE, seg_count=bounds.shape[1])
    docs = [oracle.document_ids(bounds[b], S) for b in range(2)]
    for cq in range(world):
        qp = oracle.positions(layout, S, world, cq)
        for ck in range(world):
            kp = oracle.positions(layout, S, world, ck)
            want = 0
            for d in docs:
                vis = (d[kp][None, :] == d[qp][:, None]) & (d[kp][None, :] >= 0)
                if causal:
                    vis &= kp[None, :] <= qp[:, None]
                want += int(vis.sum())
            assert ra.ra_visible_pairs_packed(p, cq, ck, bounds) == want
    assert _status_of(ra.ra_visible_pairs, p, 0, 0) == ra.RA_ERR_UNSUPPORTED
    for bad in ([[1, 96]] * 2, [[0, 50, 40]] * 2, [[0, 97]] * 2):
        q = _prob(batch=2, seq_total=S, world=world, layout=layout, seg_bounds=FAKE,
                  seg_count=len(bad[0]))
        assert _status_of(ra.ra_visible_pairs_packed, q, 0, 0, np.array(bad, np.int32)) == \
            ra.RA_ERR_SHAPE


def test_workspace_sizes():
    p = _prob(batch=2, heads_q=4, seq_total=64, world=2, head_dim_padded=128, head_dim=128)
    assert ra.ra_ring_workspace_size(p) == 2 * 4 * 32 * 128 * 4
    assert ra.ra_ring_bwd_workspace_size(p) == 2 * 4 * 32 * 4


def _status_of(fn, *args):
    with pytest.raises(ra.RaError) as e:
        fn(*args)
    return e.value.status


FAKE = 1 << 20  # a 16-byte-aligned non-null address; never dereferenced on these paths


@pytest.mark.parametrize("kw,status", [
    (dict(heads_q=3, heads_kv=2), ra.RA_ERR_SHAPE),
    (dict(head_dim_padded=96, head_dim=96), ra.RA_ERR_UNSUPPORTED),
    (dict(head_dim=65), ra.RA_ERR_SHAPE),
    (dict(seq_total=50), ra.RA_ERR_SHAPE),
    (dict(seq_total=52, layout="zigzag"), ra.RA_ERR_SHAPE),
    (dict(world=0), ra.RA_ERR_SHAPE),
    (dict(batch=0), ra.RA_ERR_SHAPE),
    (dict(layout=7), ra.RA_ERR_UNSUPPORTED),
    (dict(dtype=9), ra.RA_ERR_UNSUPPORTED),
    (dict(q_stride=(0, 0, 3)), ra.RA_ERR_SHAPE),
    (dict(kv_stride=(0, 0, 1 << 24)), ra.RA_ERR_UNSUPPORTED),  # a head's rows span > 4 GiB
    (dict(o_stride=(0, 0, 1 << 24)), ra.RA_ERR_UNSUPPORTED),
    (dict(scale=-1.0), ra.RA_ERR_SHAPE),
    # batch * heads_q * (L + 256) >= 2^31: more work-items than one grid dimension holds
    (dict(batch=1 << 12, heads_q=1 << 10, heads_kv=1 << 10, seq_total=4096), ra.RA_ERR_SHAPE),
    # sizes whose products once wrapped past the checks: batch * heads_q * (L + 256) and
    # the strides are now bounded before any multiplication
    (dict(batch=1 << 31), ra.RA_ERR_SHAPE),
    (dict(batch=1 << 30, heads_q=1 << 30, heads_kv=1 << 30, seq_total=64), ra.RA_ERR_SHAPE),
    (dict(kv_stride=(0, 0, 1 << 48)), ra.RA_ERR_SHAPE),
    (dict(seg_bounds=FAKE, seg_count=1), ra.RA_ERR_SHAPE),
    (dict(seg_bounds=FAKE, seg_count=0), ra.RA_ERR_SHAPE),
    (dict(seg_bounds=FAKE + 2, seg_count=4), ra.RA_ERR_SHAPE),
])
def test_problem_validation(kw, status):
    p = _prob(**kw)
    assert _status_of(ra.ra_positions, p, 0) == status
    assert _status_of(ra.ra_block_attn_fwd, p, FAKE, 0, FAKE, FAKE, 0, FAKE, FAKE,
                      ra.RA_WRITE, 0) == status
    assert ra.ra_last_error() != ""


def test_call_validation():
    p = _prob()
    fwd = ra.ra_block_attn_fwd
    assert _status_of(fwd, p, 0, 0, FAKE, FAKE, 0, FAKE, FAKE, ra.RA_WRITE, 0) == ra.RA_ERR_NULL
    assert _status_of(fwd, p, FAKE + 2, 0, FAKE, FAKE, 0, FAKE, FAKE, ra.RA_WRITE, 0) == ra.RA_ERR_SHAPE
    assert _status_of(fwd, p, FAKE, 4, FAKE, FAKE, 0, FAKE, FAKE, ra.RA_WRITE, 0) == ra.RA_ERR_SHAPE
    assert _status_of(fwd, p, FAKE, 0, FAKE, FAKE, -1, FAKE, FAKE, ra.RA_WRITE, 0) == ra.RA_ERR_SHAPE
    assert _status_of(fwd, p, FAKE, 0, FAKE, FAKE, 0, FAKE, FAKE, 5, 0) == ra.RA_ERR_UNSUPPORTED
    ks = [FAKE] * 4
    ring = ra.ra_ring_fwd
    assert _status_of(ring, p, 1, FAKE, ks, ks, FAKE, FAKE, None, 0, 0) == ra.RA_ERR_WORKSPACE
    assert _status_of(ring, p, 1, FAKE, ks, ks, FAKE, FAKE, FAKE, 16, 0) == ra.RA_ERR_WORKSPACE
    assert _status_of(ring, p, 4, FAKE, ks, ks, FAKE, FAKE, FAKE, 1 << 30, 0) == ra.RA_ERR_SHAPE
    assert _status_of(ring, p, 1, FAKE, ks[:3] + [0], ks, FAKE, FAKE, FAKE, 1 << 30, 0) == ra.RA_ERR_NULL
    assert _status_of(ra.ra_lse_merge, 10, 6, FAKE, FAKE, FAKE, FAKE, 0) == ra.RA_ERR_SHAPE
    assert _status_of(ra.ra_lse_merge, 10, 2048, FAKE, FAKE, FAKE, FAKE, 0) == ra.RA_ERR_SHAPE
    assert _status_of(ra.ra_lse_merge, -1, 8, FAKE, FAKE, FAKE, FAKE, 0) == ra.RA_ERR_SHAPE
    assert _status_of(ra.ra_lse_merge, 1 << 34, 8, FAKE, FAKE, FAKE, FAKE, 0) == ra.RA_ERR_SHAPE
    assert _status_of(ra.ra_lse_merge, 10, 8, 0, FAKE, FAKE, FAKE, 0) == ra.RA_ERR_NULL
    f32 = _prob(dtype="f32")
    bwd = ra.ra_block_attn_bwd
    assert _status_of(bwd, f32, FAKE, 0, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, FAKE,
                      FAKE, 0) == ra.RA_ERR_UNSUPPORTED
    assert _status_of(ra.ra_ring_bwd, p, 0, FAKE, ks, ks, FAKE, FAKE, FAKE, FAKE, ks, ks,
                      FAKE, 8, 0) == ra.RA_ERR_WORKSPACE
    # the backward halves take RA_WRITE or RA_MERGE only
    for half, outs in ((ra.ra_block_attn_bwd_dkdv, (FAKE, FAKE)), (ra.ra_block_attn_bwd_dq, (FAKE,))):
        assert _status_of(half, p, FAKE, 0, FAKE, FAKE, 0, FAKE, FAKE, FAKE, *outs, 7,
                          0) == ra.RA_ERR_UNSUPPORTED
    # ra_bwd_prepare checks every pointer before its first launch
    prep = ra.ra_bwd_prepare
    assert _status_of(prep, p, FAKE, FAKE, FAKE, 0, ks, ks, 0) == ra.RA_ERR_NULL
    assert _status_of(prep, p, FAKE, FAKE, FAKE, FAKE, ks[:3] + [0], ks, 0) == ra.RA_ERR_NULL
    assert _status_of(prep, p, FAKE, FAKE, FAKE, FAKE, ks, [FAKE + 2] + ks[1:], 0) == \
        ra.RA_ERR_SHAPE
    assert _status_of(prep, p, 0, FAKE, FAKE, FAKE, ks, ks, 0) == ra.RA_ERR_NULL
    assert _status_of(prep, p, FAKE, FAKE, 0, FAKE, ks, ks, 0) == ra.RA_ERR_NULL
    assert _status_of(prep, _prob(world=0), FAKE, FAKE, FAKE, FAKE, ks, ks, 0) == ra.RA_ERR_SHAPE


def test_status_strings():
    assert ra.ra_status_str(ra.RA_OK) == "RA_OK"
    assert ra.ra_status_str(ra.RA_ERR_WORKSPACE) == "RA_ERR_WORKSPACE"


def test_noalloc_refuses_a_workspace_beyond_the_static_array_before_any_launch():
    # batch * heads_q * L = 64 * 131072 rows of fp32 delta > the 16 MiB static array
    p = _prob(heads_q=64, heads_kv=8, head_dim=128, head_dim_padded=128, seq_total=131072,
              world=1)
    ks = [FAKE]
    assert _status_of(ra.ra_ring_bwd_noalloc, p, 0, FAKE, ks, ks, FAKE, FAKE, FAKE, FAKE, ks,
                      ks, 0) == ra.RA_ERR_WORKSPACE
    assert "static scratch" in ra.ra_last_error()
    # the problem checks come first
    assert _status_of(ra.ra_ring_bwd_noalloc, _prob(world=0), 0, FAKE, ks, ks, FAKE, FAKE, FAKE,
                      FAKE, ks, ks, 0) == ra.RA_ERR_SHAPE


def test_build_flags_name_real_sources():
    """Per-source code-generation flags are keyed by file name: a key that names no
    source, or a source that is not on disk, would silently build without them."""
    from ring_context_parallelism_amd import build
    assert set(build.SOURCE_FLAGS) <= set(build.SOURCES)
    for src in build.SOURCES:
        assert os.path.exists(os.path.join(build.CSRC, src)), src
    for flags in build.SOURCE_FLAGS.values():
        assert all(isinstance(f, str) and f for f in flags)
        # every -mllvm takes exactly one backend option after it
        for k, f in enumerate(flags):
            if f == "-mllvm":
                assert k + 1 < len(flags) and flags[k + 1].startswith("-amdgpu-")


# Property-based fuzz of the host validation and size arithmetic (no launches): any
# problem description, hostile fields and strides included, must come back with a
# defined status, and a successful size or count must respect its bound.  Under the
# sanitizer copies of the library (test_abi_asan.py) an overflow or out-of-bounds
# access in that arithmetic fails the run.
from hypothesis import HealthCheck, given, settings, strategies as st  # noqa: E402

_I64 = st.one_of(st.integers(-4, 300), st.sampled_from([0, 1, 1 << 20, 1 << 31, 1 << 40,
                                                        (1 << 62), -(1 << 40)]))
_STATUSES = {ra.RA_OK, ra.RA_ERR_NULL, ra.RA_ERR_SHAPE, ra.RA_ERR_UNSUPPORTED}


def _raw_problem(f):
    p = ra.Problem()
    (p.batch, p.heads_q, p.heads_kv, p.head_dim, p.head_dim_padded, p.seq_total) = f[:6]
    p.world, p.layout, p.causal, p.dtype = f[6], f[7], f[8], f[9]
    p.scale = f[10]
    p.seg_count = 0
    p.seg_bounds = None
    for i in range(3):
        p.q_stride[i], p.kv_stride[i], p.o_stride[i] = f[11][i], f[12][i], f[13][i]
    return p


@settings(max_examples=400, deadline=None, suppress_health_check=list(HealthCheck))
@given(st.tuples(_I64, _I64, _I64, st.sampled_from([0, 24, 32, 64, 100, 128, 129, -1]),
                 st.sampled_from([0, 32, 64, 96, 128, 256]), _I64,
                 st.integers(-2, 40), st.integers(-1, 4), st.integers(0, 1), st.integers(-1, 3),
                 st.sampled_from([0.0, 0.125, -1.0, float("nan"), float("inf")]),
                 st.tuples(_I64, _I64, _I64), st.tuples(_I64, _I64, _I64),
                 st.tuples(_I64, _I64, _I64)),
       st.integers(-3, 45), st.integers(-3, 45))
def test_validation_fuzz(f, qc, kc):
    p = _raw_problem(f)
    lib = ra.lib()
    n = ctypes.c_size_t(0)
    s = lib.ra_ring_workspace_size(ctypes.byref(p), ctypes.byref(n))
    assert s in _STATUSES
    if s == ra.RA_OK:
        L = p.seq_total // p.world
        assert n.value == p.batch * p.heads_q * L * p.head_dim_padded * 4
    s2 = lib.ra_ring_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n))
    assert s2 in _STATUSES
    pairs = ctypes.c_int64(-1)
    s3 = lib.ra_visible_pairs(ctypes.byref(p), qc, kc, ctypes.byref(pairs))
    assert s3 in _STATUSES
    if s3 == ra.RA_OK:
        L = p.seq_total // p.world
        assert 0 <= pairs.value <= p.batch * L * L


_BIG = st.sampled_from([1, 2, 3, 1 << 20, 1 << 31, 1 << 40, 1 << 61])


@st.composite
def _valid_shape_problem(draw):
    """Every field passes the structural checks; sizes and strides go up to ~2^62, so
    the size and stride arithmetic of the validation sees hostile magnitudes."""
    p = ra.Problem()
    p.head_dim_padded = draw(st.sampled_from([32, 64, 128]))
    p.head_dim = draw(st.integers(1, p.head_dim_padded))
    p.heads_kv = draw(_BIG)
    g = draw(st.sampled_from([1, 2, 4, 8]))
    p.heads_q = min(p.heads_kv * g, (1 << 62) // g * g)
    p.heads_kv = p.heads_q // g
    p.batch = draw(_BIG)
    p.world = draw(st.integers(1, 8))
    p.layout = draw(st.integers(0, 2))
    p.causal = draw(st.integers(0, 1))
    p.dtype = draw(st.integers(0, 1))
    p.scale = 0.0
    div = 2 * p.world if p.layout == ra.RA_LAYOUT_ZIGZAG else p.world
    k = draw(st.sampled_from([1, 7, 64, 4096, 1 << 20, (1 << 31) // 16]))
    p.seq_total = min(k * div, ((1 << 31) - 1) // div * div)
    unit = 8 if p.dtype == ra.RA_BF16 else 4  # 16 bytes of elements
    stride = st.one_of(st.integers(0, 64).map(lambda x: x * unit),
                       st.sampled_from([1 << 40, 1 << 60, (1 << 62) - (1 << 62) % unit]))
    for i in range(3):
        p.q_stride[i], p.kv_stride[i], p.o_stride[i] = draw(stride), draw(stride), draw(stride)
    p.seg_count, p.seg_bounds = 0, None
    return p


@settings(max_examples=400, deadline=None, suppress_health_check=list(HealthCheck))
@given(_valid_shape_problem(), st.integers(0, 7), st.integers(0, 7))
def test_validation_fuzz_hostile_sizes(p, qc, kc):
    lib = ra.lib()
    n = ctypes.c_size_t(0)
    s = lib.ra_ring_workspace_size(ctypes.byref(p), ctypes.byref(n))
    assert s in _STATUSES
    if s == ra.RA_OK:
        L = p.seq_total // p.world
        assert (p.batch * p.heads_q * (L + 256)) < (1 << 31)
        assert n.value == p.batch * p.heads_q * L * p.head_dim_padded * 4
    pairs = ctypes.c_int64(-1)
    s3 = lib.ra_visible_pairs(ctypes.byref(p), min(qc, p.world - 1), min(kc, p.world - 1),
                              ctypes.byref(pairs))
    assert s3 in _STATUSES
    if s3 == ra.RA_OK:
        L = p.seq_total // p.world
        assert 0 <= pairs.value <= p.batch * L * L
