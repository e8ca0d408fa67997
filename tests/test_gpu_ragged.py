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


def run_ragged(cs, Q, C, offsets, sim, scale, status=None, out=None, ws=None):
    """One ragged call; ws: a zeroed uint8 device workspace (split plan) or
    None (one workgroup per question)."""
    import torch

    dev = torch.device("cuda:0")
    q = torch.from_numpy(np.ascontiguousarray(Q)).to(dev)
    c = torch.from_numpy(np.ascontiguousarray(C)).to(dev)
    o = torch.from_numpy(np.ascontiguousarray(offsets, dtype=np.int64)).to(dev)
    total = C.shape[0]
    if out is None:
        out = torch.full((total,), -5.0, device=dev)
    st = cs.cs_score_candidates_ragged(q, c, o, len(offsets) - 1, total, Q.shape[1], sim,
                                       float(scale), 1.0, out, status, ws,
                                       0 if ws is None else ws.numel())
    assert st == 0, st
    torch.cuda.synchronize()
    return out.cpu().numpy()


def split_workspace(cs, B, total, D, sim):
    import torch

    n = cs.cs_ragged_workspace_bytes(B, total, D, sim)
    assert n > 0, (B, total, D, sim)
    return torch.zeros(n, dtype=torch.uint8, device=torch.device("cuda:0"))


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


# The page's batch-path cases: batches of 1, 8, 4 and 3 questions with K up
# to 255 ("Verified on hardware", second group), here with counts that vary
# per question, as a ragged batch spread over the chip.
SPLIT_CASES = [
    ([255], 2560, "dot"),
    ([200, 3, 255, 17, 64, 128, 1, 90], 2560, "dot"),
    ([255, 255, 254, 1], 512, "cosine"),
    ([33, 255, 120], 1024, "cosine"),
    ([255, 100, 7, 255, 60, 30, 2, 250], 1000, "cosine"),   # the general kernel
    ([255, 9, 128], 4097, "dot"),                           # general kernel, q in two chunks
    ([255] * 16, 2560, "dot"),
]


@pytest.mark.parametrize("counts,D,sim", SPLIT_CASES)
def test_ragged_split_matches_oracle(cs, orc, counts, D, sim):
    """Small ragged batches cut every question into slices of the planned
    rows, over several workgroups merged by the question's last slice: the
    oracle on every row, equal to the unsplit launch within fp32 rounding,
    and the workspace zero again after each call."""
    import torch

    B = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    total = int(offsets[-1])
    Q, C = workloads.ragged_inputs(211 + B + D, offsets, D)
    scale = workloads.SCALE_COSINE if sim == "cosine" else workloads.SCALE_DOT
    st, rpg, slices = cs.cs_plan_ragged(B, total, D, sim, True)
    note(f"case ragged split counts={counts[:8]} D={D} {sim}: {rpg} rows per slice, "
         f"up to {slices} slices")
    assert st == 0 and slices > 1
    want = orc.score_ragged(Q, C, offsets, sim, scale)
    ws = split_workspace(cs, B, total, D, sim)
    for rep in range(2):
        p = run_ragged(cs, Q, C, offsets, sim, scale, ws=ws)
        check(p, want, offsets, f"split rep={rep}")
        assert np.all(p != -5.0)
        assert int(torch.count_nonzero(ws)) == 0, "workspace left nonzero"
    one = run_ragged(cs, Q, C, offsets, sim, scale)
    assert float(np.max(np.abs(one.astype(np.float64) - p))) <= 2e-6
    ones = [b for b, k in enumerate(counts) if k == 1]
    assert all(p[offsets[b]] == 1.0 for b in ones)


def test_ragged_split_bad_offsets(cs, orc):
    """A question with invalid offsets is skipped by all of its slices (no
    ticket drawn, nothing written) and flagged; the others merge normally
    and the workspace returns to zero."""
    import torch

    D = 2560
    # q0: 200 rows; q1: 0 rows (invalid); q2: 255 rows; q3: 300 rows (invalid)
    offsets = np.array([0, 200, 200, 455, 755], dtype=np.int64)
    total = 755
    rng = np.random.default_rng(223)
    Q = rng.standard_normal((4, D), dtype=np.float32)
    C = rng.standard_normal((total, D), dtype=np.float32)
    dev = torch.device("cuda:0")
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = split_workspace(cs, 4, total, D, "dot")
    note("case ragged split bad offsets")
    p = run_ragged(cs, Q, C, offsets, "dot", 0.0625, status=status, ws=ws)
    assert int(status.item()) == cs.CS_ERR_K_RANGE
    for b, (lo, hi) in {0: (0, 200), 2: (200, 455)}.items():
        want = orc.score(Q[b], C[lo:hi], "dot", 0.0625)
        assert np.max(np.abs(p[lo:hi].astype(np.float64) - want)) <= TOL
    assert np.all(p[455:] == -5.0)
    assert int(torch.count_nonzero(ws)) == 0


def test_ragged_split_equals_dense_split(cs, orc):
    """Sixteen questions of 255 rows: the ragged plan cuts them as the dense
    batch call does, and the results agree within fp32 rounding."""
    import torch

    B, K, D = 16, 255, 2560
    Q, C = workloads.normal_inputs(227, B, K, D)
    offsets = np.arange(B + 1, dtype=np.int64) * K
    ws = split_workspace(cs, B, B * K, D, "dot")
    p = run_ragged(cs, Q, C.reshape(B * K, D), offsets, "dot", 0.0625, ws=ws)
    dev = torch.device("cuda:0")
    dense = cs.score(torch.from_numpy(Q).to(dev), torch.from_numpy(C).to(dev), "dot", 0.0625)
    torch.cuda.synchronize()
    d = dense.cpu().numpy().reshape(-1)
    assert float(np.max(np.abs(p.astype(np.float64) - d))) <= 2e-6
    check(p, orc.score_ragged(Q, C.reshape(B * K, D), offsets, "dot", 0.0625), offsets,
          "16 x 255 ragged split")


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
