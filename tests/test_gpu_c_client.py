"""The library called from a plain C program (tests/c_client/cs_client.c,
built in-tree by __graft_entry__.build() with gcc in C11 mode): device
memory from the HIP runtime API, the scoring calls through the C ABI of
include/candidate_scoring.h only. The program runs as a child process and
its probabilities, without and with the split workspace, are compared with
the oracle element by element (tolerance as in the other parity tests)."""
from __future__ import annotations

import subprocess
from pathlib import Path

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

CLIENT = Path(__file__).resolve().parent / "c_client" / "cs_client"
TOL = 1e-4


@pytest.mark.parametrize("name", ["clm_cos_batch8_255x512", "kev_dot_255x2560"])
def test_c_client_matches_oracle(orc, tmp_path, name):
    assert CLIENT.exists(), f"{CLIENT} is not built: run __graft_entry__.build()"
    w = workloads.make(name)
    B, K, D = w.C.shape
    sim = {"dot": 0, "cosine": 1}[w.similarity]
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(np.array([B, K, D, sim], dtype=np.int32).tobytes())
        f.write(np.float32(w.scale).tobytes())
        f.write(np.ascontiguousarray(w.Q, dtype=np.float32).tobytes())
        f.write(np.ascontiguousarray(w.C, dtype=np.float32).tobytes())
    print(f"case c client {name} B={B} K={K} D={D}", flush=True)
    r = subprocess.run([str(CLIENT), str(src), str(dst)], capture_output=True, text=True,
                       timeout=120)
    print(r.stderr.strip(), flush=True)
    assert r.returncode == 0, r.stderr
    p = np.fromfile(dst, dtype=np.float32).reshape(2, B, K).astype(np.float64)
    want = orc.score(w.Q, w.C, w.similarity, w.scale, w.temperature)
    for i, label in enumerate(("no workspace", "workspace")):
        err = float(np.max(np.abs(p[i] - want)))
        sums = float(np.max(np.abs(p[i].sum(axis=-1) - 1.0)))
        print(f"  {label}: max|c-oracle|={err:.3e} max|rowsum-1|={sums:.3e}", flush=True)
        assert err <= TOL and sums <= 1e-5, label
