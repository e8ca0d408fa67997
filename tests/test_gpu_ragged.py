"""Ragged batches: per-question candidate counts in one launch.

Each question keeps the page's limit of at most 255 candidates ("What is
fused, precisely"); the batch tests on the page mix question counts with K
"up to 255" ("Verified on hardware"). The oracle side is cso_score_ragged.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

TOL = 1e-4


def note(msg):
    print(msg, flush=True)


def run_ragged(cs, Q, C, offsets, sim, scale, status=None, out=None):
    import torch

    dev = torch.device("cuda:0")
    q = torch.from_numpy(np.ascontiguousarray(Q)).to(dev)
    c = torch.from_numpy(np.ascontiguousarray(C)).to(dev)
    o = torch.from_numpy(np.ascontiguousarray(offsets, dtype=np.int64)).to(dev)
    total = C.shape[0]
    if out is None:
        out = torch.full((total,), -5.0, device=dev)
    st = cs.cs_score_candidates_ragged(q, c, o, len(offsets) - 1, total, Q.shape[1], sim,
                                       float(scale), 1.0, out, status)
    assert st == 0, st
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(p, want, offsets, label):
    err = float(np.max(np.abs(p.astype(np.float64) - want)))
    sums = [abs(float(p[offsets[b]:offsets[b + 1]].astype(np.float64).sum()) - 1.0)
            for b in range(len(offsets) - 1)]
    note(f"  {label}: max|gpu-oracle|={err:.3e} max|rowsum-1|={max(sums):.3e}")
    assert err <= TOL and max(sums) <= 1e-5, label


@pytest.mark.parametrize("B,D,sim", [(100, 512, "cosine"), (64, 2560, "dot"), (37, 1000, "cosine"),
                                     (20, 3, "dot"), (300, 2560, "dot"),
                                     (2000, 16, "cosine")])
def test_ragged_matches_oracle(cs, orc, B, D, sim):
    offsets = workloads.ragged_offsets(41 + B, B)
    Q, C = workloads.ragged_inputs(43 + B, offsets, D)
    scale = workloads.SCALE_COSINE if sim == "cosine" else workloads.SCALE_DOT
    note(f"case ragged B={B} D={D} {sim} rows={offsets[-1]}")
    want = orc.score_ragged(Q, C, offsets, sim, scale)
    p = run_ragged(cs, Q, C, offsets, sim, scale)
    check(p, want, offsets, f"ragged B={B} D={D}")


def test_ragged_edge_counts(cs, orc):
    for counts in ([1], [255], [1] * 17, [255, 1, 254, 2, 128, 127], [255] * 9):
        offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
        Q, C = workloads.ragged_inputs(47, offsets, 512)
        for sim in ("cosine", "dot"):
            note(f"case ragged counts={counts[:6]} {sim}")
            want = orc.score_ragged(Q, C, offsets, sim, 14.285714)
            p = run_ragged(cs, Q, C, offsets, sim, 14.285714)
            check(p, want, offsets, f"counts={counts[:6]}")
            one = [b for b, k in enumerate(counts) if k == 1]
            assert all(p[offsets[b]] == 1.0 for b in one)


def test_ragged_equal_counts_equals_dense(cs):
    """With every count equal to K the ragged launch is the dense batch
    launch (one workgroup per question): bitwise the same output."""
    import torch

    B, K, D = 12, 255, 512
    Q, C = workloads.normal_inputs(53, B, K, D)
    offsets = np.arange(B + 1, dtype=np.int64) * K
    p = run_ragged(cs, Q, C.reshape(B * K, D), offsets, "cosine", 3.0)
    dev = torch.device("cuda:0")
    dense = cs.score(torch.from_numpy(Q).to(dev), torch.from_numpy(C).to(dev), "cosine", 3.0,
                     1.0, use_workspace=False)
    torch.cuda.synchronize()
    assert np.array_equal(p, dense.cpu().numpy().reshape(-1))


def test_ragged_bad_offsets_flagged_and_skipped(cs, orc):
    """Questions whose offsets are invalid write nothing and raise the
    status word; the others are scored normally."""
    import torch

    D = 64
    # q0: 5 rows; q1: 0 rows (invalid); q2: 300 rows (invalid, > 255);
    # q3: 4 rows; q4: decreasing (invalid); q5: runs past total_rows (invalid)
    offsets = np.array([0, 5, 5, 305, 309, 300, 400], dtype=np.int64)
    total = 320
    rng = np.random.default_rng(59)
    Q = rng.standard_normal((6, D), dtype=np.float32)
    C = rng.standard_normal((total, D), dtype=np.float32)
    dev = torch.device("cuda:0")
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    out = torch.full((total,), -5.0, device=dev)
    note("case ragged bad offsets")
    p = run_ragged(cs, Q, C, offsets, "dot", 1.0, status=status, out=out)
    assert int(status.item()) == cs.CS_ERR_K_RANGE
    good = {0: (0, 5), 3: (305, 309)}
    for b, (lo, hi) in good.items():
        want = orc.score(Q[b], C[lo:hi], "dot", 1.0)
        assert np.max(np.abs(p[lo:hi].astype(np.float64) - want)) <= TOL
    touched = np.zeros(total, bool)
    for lo, hi in good.values():
        touched[lo:hi] = True
    assert np.all(p[~touched] == -5.0)
    # a clean call leaves the status alone
    status.zero_()
    offsets_ok = np.array([0, 5, 9], dtype=np.int64)
    run_ragged(cs, Q[:2], C[:9], offsets_ok, "dot", 1.0, status=status)
    assert int(status.item()) == 0


def test_ragged_full_size(cs, orc):
    """The bench's ragged batch at full size (1024 questions, counts uniform
    in 1..255, D=2560, dot: the longest-first order), in the launch it times;
    every row against the oracle, every question's probabilities written and
    summing to one."""
    B, D = 1024, 2560
    offsets = workloads.ragged_offsets(61, B)
    Q, C = workloads.ragged_inputs(67, offsets, D)
    note(f"case ragged full size B={B} D={D} rows={offsets[-1]}")
    p = run_ragged(cs, Q, C, offsets, "dot", workloads.SCALE_DOT)
    assert np.all(p != -5.0), "rows left unwritten"
    check(p, orc.score_ragged(Q, C, offsets, "dot", workloads.SCALE_DOT), offsets,
          "ragged full size, every row")


def test_ragged_beyond_the_grid_cap(cs, orc):
    """More questions than the launch's grid cap (2^20 workgroups), in index
    order (the questions are far too small for the longest-first ranking to
    pay): the workgroups stride over the rest. Every row is checked."""
    B, D = (1 << 20) + 11, 4
    offsets = workloads.ragged_offsets(131, B, k_max=3)
    Q, C = workloads.ragged_inputs(137, offsets, D)
    note(f"case ragged grid cap B={B} D={D} rows={offsets[-1]}")
    p = run_ragged(cs, Q, C, offsets, "cosine", 2.0)
    check(p, orc.score_ragged(Q, C, offsets, "cosine", 2.0), offsets, "ragged grid cap")
