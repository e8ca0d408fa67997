"""Projection + scoring: the caller-side heads fused with the scoring.

Source: pull request "cuda: add a fused candidate-scoring kernel for CLM and
Kev", intro table (CLM: exp(logit_scale) * cos(state_head(s),
action_head(c)); Kev: k(h_opts) . q(h_decide) / sqrt(256)). Inputs are bf16;
the oracle (cso_score_projected) gets the same values as fp32 and works in
double. Bar: 1e-4 per probability, as for the plain scoring.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

TOL = 1e-4


def note(msg):
    print(msg, flush=True)


def to_dev16(bits, dev):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)


def run(cs, w, dev, T=1.0):
    import torch

    xq, xc = to_dev16(w.xq_bits, dev), to_dev16(w.xc_bits, dev)
    wq, wc = to_dev16(w.wq_bits, dev), to_dev16(w.wc_bits, dev)
    out = torch.full((w.B, w.K), -3.0, device=dev)
    nbytes = cs.cs_projected_workspace_bytes(w.B, w.Hc, w.P, w.similarity)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    st = cs.cs_score_projected(xq, xc, wq, wc, w.B, w.K, w.Hq, w.Hc, w.P, w.similarity,
                               float(w.scale), T, out, ws, nbytes)
    assert st == 0, st
    torch.cuda.synchronize()
    return out.cpu().numpy()


def want(orc, w, T=1.0, questions=None):
    idx = slice(None) if questions is None else questions
    return orc.score_projected(w.f32("xq")[idx], w.f32("wq"), w.f32("xc")[idx], w.f32("wc"),
                               w.similarity, w.scale, T)


def check(p, ref, label):
    err = float(np.max(np.abs(p.astype(np.float64) - ref)))
    sums = float(np.max(np.abs(p.astype(np.float64).sum(axis=-1) - 1.0)))
    note(f"  {label}: max|gpu-oracle|={err:.3e} max|rowsum-1|={sums:.3e}")
    assert np.all(np.isfinite(p)) and err <= TOL and sums <= 1e-5, label


@pytest.fixture(scope="module")
def dev(cs):
    import torch

    return torch.device("cuda:0")


@pytest.mark.parametrize("B,K,Hq,Hc,P,sim", [
    (4, 255, 2560, 2560, 256, "dot"),      # Kev-shaped heads
    (4, 255, 512, 512, 256, "cosine"),     # CLM-shaped heads: slices x 64-feature parts
    (5, 255, 512, 512, 256, "cosine"),     # one question more: slices x 128-feature parts
    (8, 255, 512, 512, 256, "cosine"),     # eight questions, 128-feature parts
    (12, 255, 512, 512, 256, "cosine"),    # 192 workgroups: the most 128-feature parts take
    (13, 255, 512, 512, 256, "cosine"),    # one question more: the tile kernel
    (6, 255, 64, 128, 192, "cosine"),      # P = 192 beyond 64-feature parts: whole-feature
                                           # slices, merged
    (3, 255, 512, 512, 64, "cosine"),
    (3, 200, 256, 520, 128, "cosine"),     # hidden not a multiple of the 64-wide chunk
    (2, 64, 128, 1000, 192, "cosine"),
    (5, 5, 64, 24, 64, "cosine"),
    (2, 1, 64, 64, 64, "cosine"),
    (2, 130, 64, 32, 128, "cosine"),       # hidden below one 64-wide chunk, a partial slice
    (3, 255, 64, 96, 192, "cosine"),       # hidden not a multiple of 64: a zeroed tail
    (2, 255, 64, 64, 256, "cosine"),       # one 64-wide chunk
    (3, 255, 64, 192, 192, "cosine"),      # three chunks: one group of four in flight
    (2, 200, 64, 320, 256, "cosine"),      # five chunks: a second group
    (3, 17, 64, 2048, 64, "cosine"),
    (3, 77, 520, 1000, 96, "dot"),
    (2, 255, 8, 8, 8, "dot"),
    (2, 100, 136, 4096, 256, "dot"),
    (3, 255, 64, 2048, 64, "dot"),         # four 16-byte pieces per lane
    (2, 50, 520, 1000, 200, "dot"),        # P not a multiple of 16 or 32
    (1, 255, 4096, 4096, 256, "cosine"),   # one question over eight slices, 64 chunks
    (1, 255, 2560, 2560, 256, "dot"),      # one question: the candidate pass is split
    (2, 200, 512, 1000, 96, "dot"),        # split, a partial last slice
    (200, 40, 256, 2048, 128, "dot"),      # 7 question blocks: the fold's four-wave tiles
    (5, 100, 520, 1000, 96, "dot"),        # eight-question matrix-vector kernels, three padded
    (8, 40, 2056, 136, 128, "dot"),        # eight questions: the last on the matrix-vector side
    (9, 100, 520, 1000, 96, "dot"),        # one question past the matrix-vector query side
    (4, 60, 1032, 72, 256, "dot"),         # matrix-vector query side: a partial head row
                                           # chunk, a partial column strip of the fold
    (3, 33, 4104, 136, 250, "dot"),        # three chunks per head row, P < 256 clamped rows
    (7, 32, 64, 136, 128, "cosine"),       # one whole 32-candidate slice
    (9, 33, 64, 200, 192, "cosine"),       # a second slice of one candidate
    (8, 250, 64, 128, 64, "cosine"),       # 8 x 8 slices: the most split questions take
    (9, 250, 64, 128, 64, "cosine"),       # one question more: the tile kernel
    (256, 32, 64, 136, 64, "cosine"),      # unsplit questions: one workgroup per compute unit
    (257, 32, 64, 136, 64, "cosine"),      # one question more: the tile kernel
    (1027, 37, 64, 1000, 96, "dot"),       # more candidate-pass workgroups than stay
                                           # resident; partial pieces per lane
    (1025, 255, 64, 512, 64, "dot"),       # 32 question blocks and one more
    (1024, 1, 8, 8, 8, "dot"),             # one row per question: most waves get none
    (600, 100, 64, 512, 64, "dot"),        # more than two questions per compute unit
    (1031, 255, 64, 1000, 96, "dot"),      # the same with partial pieces per lane
])
def test_projected_matches_oracle(cs, orc, dev, B, K, Hq, Hc, P, sim):
    w = workloads.projected_inputs(70 + B + K + P, B, K, Hq, Hc, P, sim)
    note(f"case projected B={B} K={K} Hq={Hq} Hc={Hc} P={P} {sim}")
    check(run(cs, w, dev), want(orc, w), f"B={B} K={K} Hc={Hc} P={P} {sim}")


@pytest.mark.parametrize("B,K,Hc,P", [
    (600, 33, 256, 128),   # even chunk count: the ring runs across questions
    (400, 50, 128, 192),   # two chunks: a question's softmax runs in the next one's only loop pass
    (280, 255, 128, 256),  # two chunks, full 255-row tiles
    (300, 40, 192, 64),    # three chunks: the ring restarts for every question
    (270, 10, 64, 256),    # one chunk of the ring
    (270, 12, 96, 64),     # hidden not a multiple of 64: the register-staged tile
])
def test_projected_cosine_many_questions(cs, orc, dev, B, K, Hc, P):
    """More questions than compute units, so a workgroup of the cosine kernel
    takes several questions in turn; every question is checked."""
    w = workloads.projected_inputs(97 + B, B, K, 64, Hc, P, "cosine")
    note(f"case projected many questions B={B} K={K} Hc={Hc} P={P}")
    check(run(cs, w, dev), want(orc, w), f"B={B} K={K} Hc={Hc} P={P} cosine")


def test_projected_temperature(cs, orc, dev):
    w = workloads.projected_inputs(91, 2, 50, 64, 64, 64, "cosine")
    for T in (0.5, 3.0):
        check(run(cs, w, dev, T), want(orc, w, T), f"T={T}")


def test_projected_identical_and_zero_candidates(cs, orc, dev):
    """Identical candidate rows give exactly 1/K on the matrix-core path (every
    row goes through the same MFMA and reduction order); a zero candidate
    scores a cosine of exactly 0."""
    w = workloads.projected_inputs(93, 2, 255, 512, 512, 256, "cosine")
    w.xc_bits[0] = w.xc_bits[0, :1]
    w.xc_bits[1, 17] = 0
    p = run(cs, w, dev)
    check(p, want(orc, w), "identical/zero")
    assert np.all(p[0] == np.float32(1.0 / 255))
    z = orc.score_projected(w.f32("xq")[1:], w.f32("wq"), w.f32("xc")[1:], w.f32("wc"), "cosine",
                            w.scale)
    assert abs(float(p[1, 17]) - z[0, 17]) <= TOL


def want_threaded(orc, w, T=1.0):
    """The oracle over every question, run unchanged on contiguous question
    ranges in up to 16 host threads (ctypes releases the GIL during each
    call; the oracle keeps no shared state)."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    threads = max(1, min(16, os.cpu_count() or 1))
    bounds = np.linspace(0, w.B, threads + 1).astype(int)
    ranges = [(int(a), int(b)) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
    wq, wc = w.f32("wq"), w.f32("wc")

    def work(r):
        a, b = r
        return orc.score_projected(workloads.bf16_bits_to_f32(w.xq_bits[a:b]), wq,
                                   workloads.bf16_bits_to_f32(w.xc_bits[a:b]), wc,
                                   w.similarity, w.scale, T)

    with ThreadPoolExecutor(max_workers=len(ranges)) as pool:
        return np.concatenate(list(pool.map(work, ranges)))


@pytest.mark.parametrize("name", sorted(workloads.PROJECTED_CONFIGS))
def test_projected_full_size(cs, orc, dev, name):
    """The bench's 1024-question projected workloads at full size, in the
    launch configuration it times; every element against the oracle."""
    import time

    w = workloads.make_projected(name)
    note(f"case projected full size {name}")
    p = run(cs, w, dev)
    t0 = time.perf_counter()
    ref = want_threaded(orc, w)
    note(f"  oracle over all {w.B} questions: {time.perf_counter() - t0:.1f} s")
    check(p, ref, f"{name} every question")


@pytest.mark.parametrize("sim", ["dot", "cosine"])
def test_projected_beyond_the_grid_cap(cs, orc, dev, sim):
    """More questions than the scoring launch's grid cap (2^20 workgroups):
    the candidate pass (dot) and the register-staged cosine tile (a hidden
    size below one 64-wide chunk) stride over the rest. Every element is
    checked against the oracle."""
    B, K, Hq, Hc, P = (1 << 20) + 5, 2, 8, 8, 64
    w = workloads.projected_inputs(141 if sim == "dot" else 143, B, K, Hq, Hc, P, sim)
    note(f"case projected grid cap B={B} K={K} Hq={Hq} Hc={Hc} P={P} {sim}")
    check(run(cs, w, dev), want(orc, w), f"grid cap {sim}")


@pytest.mark.parametrize("B,sim", [(3, "dot"), (10, "dot"), (2, "cosine"), (6, "cosine"),
                                   (10, "cosine")])
def test_projected_split_on_an_unprepared_workspace(cs, orc, dev, B, sim):
    """A small batch spreads each question's candidate pass over several
    workgroups (dot: behind the matrix-vector and the matrix-core query side;
    cosine: 32 candidates x 64 or 128 projected features per workgroup,
    behind either query side), merged through tickets in the workspace; the
    query projection clears them, so a workspace full of garbage (and then
    the one a previous call left) gives the same correct result."""
    import torch

    H = 2560 if sim == "dot" else 512
    w = workloads.projected_inputs(151 + B, B, 255, H, H, 256, sim)
    if sim == "dot":
        assert cs.cs_plan_groups(B, 255, 1280, "dot", True) > 1  # the same bytes per question
    xq, xc = to_dev16(w.xq_bits, dev), to_dev16(w.xc_bits, dev)
    wq, wc = to_dev16(w.wq_bits, dev), to_dev16(w.wc_bits, dev)
    nbytes = cs.cs_projected_workspace_bytes(w.B, w.Hc, w.P, sim)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=dev)
    ref = want(orc, w)
    note(f"case projected split B={B} {sim}, workspace of 0xFF bytes, two calls")
    for call in range(2):
        out = torch.full((w.B, w.K), -3.0, device=dev)
        st = cs.cs_score_projected(xq, xc, wq, wc, w.B, w.K, w.Hq, w.Hc, w.P, sim,
                                   float(w.scale), 1.0, out, ws, nbytes)
        assert st == 0, st
        torch.cuda.synchronize()
        check(out.cpu().numpy(), ref, f"unprepared workspace, call {call}")
