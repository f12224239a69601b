"""The C ABI from a plain C program (tests/c_client/ra_client.c): neither the Python
binding nor torch sits between the caller and libra.so.

* CPU: the host-only entry points (ra_positions, ra_visible_pairs) for every layout,
  against the oracle's position map and a brute-force count of visible pairs;
* GPU: ra_ring_fwd on every rank of a small fp32 problem and of a small bf16 GQA problem
  with a padded head dim, inputs and outputs passed through files, against the oracle.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from ring_context_parallelism_amd import build as ra_build
from ring_context_parallelism_amd.workloads import Workload, generate
from tests.gpu_util import assert_close, assert_lse, need_gpu, say

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_client", "ra_client.c")
LAYOUT_IDS = {"contiguous": 0, "zigzag": 1, "striped": 2}


@pytest.fixture(scope="module")
def client(tmp_path_factory):
    """The C client, compiled as C99 with warnings as errors and linked to libra.so."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(ra_build.LIB):
        ra_build.build()
    exe = str(tmp_path_factory.mktemp("c_client") / "ra_client")
    libdir = os.path.dirname(ra_build.LIB)
    subprocess.run([cc, "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), SRC, "-o", exe,
                    "-L", libdir, "-lra", "-L/opt/rocm/lib", "-lamdhip64",
                    f"-Wl,-rpath,{libdir}", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    return exe


@pytest.mark.parametrize("layout,S,p,causal", [
    ("contiguous", 12, 3, 1), ("zigzag", 24, 3, 1), ("striped", 20, 4, 1),
    ("zigzag", 16, 2, 0), ("striped", 7, 7, 1), ("contiguous", 5, 1, 1),
])
def test_c_client_host_entry_points(client, layout, S, p, causal):
    res = subprocess.run([client, "host", str(S), str(p), str(LAYOUT_IDS[layout]), str(causal)],
                         capture_output=True, text=True, check=True, timeout=60)
    pos, pairs = {}, {}
    for line in res.stdout.splitlines():
        f = line.split()
        if f[0] == "pos":
            pos[int(f[1])] = np.array([int(x) for x in f[2:]], dtype=np.int64)
        else:
            pairs[(int(f[1]), int(f[2]))] = int(f[3])
    for c in range(p):
        assert np.array_equal(pos[c], oracle.positions(layout, S, p, c)), f"chunk {c}"
    for cq in range(p):
        qp = oracle.positions(layout, S, p, cq)
        for ck in range(p):
            kp = oracle.positions(layout, S, p, ck)
            want = int((kp[None, :] <= qp[:, None]).sum()) if causal else qp.size * kp.size
            assert pairs[(cq, ck)] == want, f"pairs ({cq}, {ck})"


GPU_CASES = [
    Workload("c_f32", 700, "f32", 1, 2, 1, 64, 64, 520, 2, "zigzag", 0, True, "normal", 1.0),
    Workload("c_bf16", 701, "bf16", 2, 8, 2, 100, 128, 600, 3, "striped", 0, True, "normal", 0.5),
]


@pytest.mark.gpu
@pytest.mark.parametrize("w", GPU_CASES, ids=lambda w: w.name)
def test_c_client_ring_fwd(client, tmp_path, w):
    need_gpu()
    arrays = generate(w)
    L, D, d = w.chunk_len, w.head_dim_padded, w.head_dim
    es = 2 if w.dtype == "bf16" else 4

    def chunk(a, c):  # global [B, H, S, d] -> chunk c as stored: [B, H, L, D], zero pad
        x = np.zeros(a.shape[:2] + (L, D), dtype=np.float32)
        x[..., :d] = a[:, :, oracle.positions(w.layout, w.seq_total, w.world, c)]
        return x

    def raw(x):  # bf16 inputs are exact bf16 values, so the top 16 bits are the bf16
        if w.dtype == "f32":
            return x.tobytes()
        return (x.view(np.uint32) >> 16).astype(np.uint16).tobytes()

    for r in range(w.world):
        inp, outp = str(tmp_path / f"in{r}.bin"), str(tmp_path / f"out{r}.bin")
        hdr = np.array([w.batch, w.heads_q, w.heads_kv, d, D, w.seq_total, w.world,
                        LAYOUT_IDS[w.layout], int(w.causal), 1 if w.dtype == "bf16" else 0, r, 0],
                       dtype=np.int64)
        with open(inp, "wb") as f:
            f.write(hdr.tobytes())
            f.write(raw(chunk(arrays["q"], r)))
            for c in range(w.world):
                f.write(raw(chunk(arrays["k"], c)))
                f.write(raw(chunk(arrays["v"], c)))
        say(f"C client ring_fwd {w.name} rank {r}")
        subprocess.run([client, "fwd", inp, outp], check=True, timeout=120)
        data = open(outp, "rb").read()
        nq, nl = w.batch * w.heads_q * L * D, w.batch * w.heads_q * L
        assert len(data) == nq * es + nl * 4
        if w.dtype == "f32":
            out = np.frombuffer(data[:nq * 4], dtype=np.float32)
        else:
            bits = np.frombuffer(data[:nq * 2], dtype=np.uint16).astype(np.uint32) << 16
            out = bits.view(np.float32)
        out = out.reshape(w.batch, w.heads_q, L, D)
        lse = np.frombuffer(data[nq * es:], dtype=np.float32).reshape(w.batch, w.heads_q, L)
        rows = oracle.positions(w.layout, w.seq_total, w.world, r)
        O, LSE = oracle.attention_fwd(arrays["q"], arrays["k"], arrays["v"], rows, w.causal)
        assert_close(out[..., :d], O, w.dtype, f"O rank {r}")
        assert np.all(out[..., d:] == 0.0)
        assert_lse(lse, LSE, f"LSE rank {r}")
