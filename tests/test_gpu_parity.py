"""GPU parity: the HIP path against the double-precision oracle.

Bar (pull request "cuda: add a fused candidate-scoring kernel for CLM and
Kev", "The manifest, and CI"): max |p_gpu - p_oracle| <= 1e-4 for every
element. Rows must also sum to 1 within 1e-5 (fp32 sums of <= 255 terms).
Cases follow "Verified on hardware": the fixed degenerate cases, the batch
path with 1, 8, 4 and 3 questions (single call for one question, batch
call for the rest, so both entry points must agree), and the split path
that spreads one question over many workgroups.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

TOL = 1e-4        # element-wise, against the oracle
SUM_TOL = 1e-5    # |sum_k p_k - 1|


def note(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def dev(cs):
    import torch

    return torch.device("cuda:0")


def to_dev(a, dev):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def run(cs, Q, C, sim, scale, T, dev, mode, groups=None):
    """mode: 'single' (cs_score_candidates), 'batch', or 'groups'."""
    import torch

    B, K, D = C.shape
    q, c = to_dev(Q, dev), to_dev(C, dev)
    if mode == "single":
        assert B == 1
        out = cs.score(q[0], c[0], sim, scale, T, use_workspace=groups != 1)
        torch.cuda.synchronize()
        return out.cpu().numpy()[None, :]
    if mode == "groups":
        out = cs.score(q, c, sim, scale, T, groups=groups)
    else:
        out = cs.score(q, c, sim, scale, T, use_workspace=groups != 1)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(p, want, label):
    p64 = p.astype(np.float64)
    err = float(np.max(np.abs(p64 - want)))
    sums = np.abs(p64.sum(axis=-1) - 1.0)
    note(f"  {label}: max|gpu-oracle|={err:.3e} max|rowsum-1|={float(sums.max()):.3e}")
    assert np.all(np.isfinite(p64)), label
    assert err <= TOL, label
    assert float(sums.max()) <= SUM_TOL, label
    return err


NAMED = [n for n in workloads.ALL if n != workloads.HEADLINE]


@pytest.mark.parametrize("name", NAMED)
def test_named_workloads(cs, orc, dev, name):
    w = workloads.make(name)
    note(f"case {name}: B={w.B} K={w.K} D={w.D} {w.similarity} scale={float(w.scale)}")
    want = orc.score(w.Q, w.C, w.similarity, w.scale, w.temperature)
    mode = "single" if w.call == "single" else "batch"
    outs = {}
    for ws in (False, True):
        p = run(cs, w.Q, w.C, w.similarity, float(w.scale), float(w.temperature), dev, mode,
                groups=None if ws else 1)
        check(p, want, f"{name} workspace={ws}")
        outs[ws] = p
    if name == "clm_cos_1x512_single_candidate":
        assert np.all(outs[False] == 1.0) and np.all(outs[True] == 1.0)
    if name == "clm_cos_255x512_identical":
        # every candidate's sum uses the same reduction tree: exactly fp32(1/K)
        assert np.all(outs[False] == np.float32(1.0 / 255)), "one-workgroup path"
        assert np.all(outs[True] == np.float32(1.0 / 255)), "split path"
    if name == "clm_cos_batch8_255x512_overflow":
        z = orc.logits(w.Q, w.C, w.similarity, w.scale, w.temperature)
        top2 = np.sort(z, axis=1)[:, -2:]
        note(f"  top-2 logit gaps per question: {np.round(top2[:, 1] - top2[:, 0], 1).tolist()}")
        with np.errstate(over="ignore", invalid="ignore"):
            naive = np.exp(z.astype(np.float32))
        assert not np.all(np.isfinite(naive)), "the case must overflow a naive exp"


@pytest.mark.parametrize("B", [1, 8, 4, 3])
@pytest.mark.parametrize("sim", ["dot", "cosine"])
def test_batch_paths(cs, orc, dev, B, sim):
    """K up to 255 and D up to 2560, incl. scalar (odd D) and tail shapes.
    B = 1 goes through cs_score_candidates, the rest through the batch call."""
    rng = np.random.default_rng(100 + B)
    scale = float(workloads.SCALE_COSINE if sim == "cosine" else workloads.SCALE_DOT)
    worst = 0.0
    for K in (1, 2, 5, 64, 255):
        for D in (1, 3, 4, 5, 64, 255, 256, 512, 1000, 2560):
            Q = rng.standard_normal((B, D), dtype=np.float32)
            C = rng.standard_normal((B, K, D), dtype=np.float32)
            want = orc.score(Q, C, sim, scale)
            for ws in (False, True):
                note(f"case batch B={B} K={K} D={D} {sim} workspace={ws}")
                p = run(cs, Q, C, sim, scale, 1.0, dev, "single" if B == 1 else "batch",
                        groups=None if ws else 1)
                worst = max(worst, check(p, want, f"B={B} K={K} D={D} ws={ws}"))
    note(f"worst over the sweep: {worst:.3e}")


def test_single_equals_batch_of_one(cs, dev):
    """Both entry points plan the same launch: bitwise equal results."""
    import torch

    for sim, D, K in (("cosine", 512, 255), ("dot", 2560, 255), ("cosine", 37, 9)):
        Q, C = workloads.normal_inputs(7, 1, K, D)
        q, c = to_dev(Q, dev), to_dev(C, dev)
        for ws in (False, True):
            note(f"case single-vs-batch {sim} K={K} D={D} ws={ws}")
            a = cs.score(q[0], c[0], sim, 2.0, 1.0, use_workspace=ws)
            b = cs.score(q, c, sim, 2.0, 1.0, use_workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(a, b[0])


@pytest.mark.parametrize("D", [512, 2560])
def test_split_group_sweep(cs, orc, dev, D):
    """Every slice count 1..K gives the oracle's distribution; ragged last
    slices included (K=255 does not divide evenly into most counts)."""
    import torch

    K = 255
    Q, C = workloads.normal_inputs(11, 2, K, D)
    for sim in ("cosine", "dot"):
        scale = 14.285714 if sim == "cosine" else 0.0625
        want = orc.score(Q, C, sim, scale)
        base = None
        for g in (1, 2, 3, 4, 7, 16, 51, 64, 85, 128, 255):
            rpg = -(-K // g)
            if -(-K // rpg) != g:
                continue
            note(f"case split D={D} {sim} groups={g}")
            p = run(cs, Q, C, sim, scale, 1.0, dev, "groups", groups=g)
            check(p, want, f"groups={g}")
            if base is None:
                base = p
            assert np.max(np.abs(p - base)) <= 2e-6, "slice count changes more than rounding"


@pytest.mark.parametrize("D,offset", [(4097, 0), (8193, 0), (40000, 0), (512, 1), (2560, 3)])
def test_general_kernel_shapes(cs, orc, dev, D, offset):
    """D beyond the register-query kernel, q chunked through LDS, and
    unaligned pointers (forcing the scalar kernel)."""
    import torch

    B, K = 2, 255
    Q, C = workloads.normal_inputs(13, B, K, D)
    for sim in ("cosine", "dot"):
        scale = 14.285714 if sim == "cosine" else 0.0625
        want = orc.score(Q, C, sim, scale)
        for ws in (False, True):
            note(f"case general D={D} offset={offset} {sim} ws={ws}")
            qd = torch.zeros(B * D + offset, dtype=torch.float32, device=dev)
            cd = torch.zeros(B * K * D + offset, dtype=torch.float32, device=dev)
            qd[offset:] = to_dev(Q.reshape(-1), dev)
            cd[offset:] = to_dev(C.reshape(-1), dev)
            q = qd[offset:].view(B, D)
            c = cd[offset:].view(B, K, D)
            out = cs.score(q, c, sim, scale, 1.0, use_workspace=ws)
            torch.cuda.synchronize()
            check(out.cpu().numpy(), want, f"D={D} offset={offset} {sim} ws={ws}")


def test_output_canaries_and_workspace_left_zero(cs, orc, dev):
    """Nothing is written outside out[0:B*K]; the workspace is zero after
    every call (the last slice resets its question's ticket)."""
    import torch

    B, K, D = 5, 255, 512
    Q, C = workloads.normal_inputs(17, B, K, D)
    want = orc.score(Q, C, "cosine", 3.0)
    q, c = to_dev(Q, dev), to_dev(C, dev)
    pad = 4096
    buf = torch.full((pad + B * K + pad,), -123.0, dtype=torch.float32, device=dev)
    out = buf[pad:pad + B * K].view(B, K)
    nbytes = cs.cs_workspace_bytes(B, K, D, "cosine")
    assert nbytes > 0
    ws = torch.zeros(nbytes + 2 * pad, dtype=torch.uint8, device=dev)
    wsv = ws[pad:pad + nbytes]
    for rep in range(3):
        note(f"case canaries rep={rep}")
        st = cs.cs_score_candidates_batch(q, c, B, K, D, "cosine", 3.0, 1.0, out, wsv, nbytes)
        assert st == 0
        torch.cuda.synchronize()
        check(out.cpu().numpy(), want, f"canaries rep={rep}")
        assert torch.all(buf[:pad] == -123.0) and torch.all(buf[pad + B * K:] == -123.0)
        tickets = wsv[: 4 * B].view(torch.int32)
        assert torch.all(tickets == 0), tickets
        # tickets and slice partials alike: the whole workspace is zero again
        assert torch.all(wsv == 0), int(torch.count_nonzero(wsv))
        assert torch.all(ws[:pad] == 0) and torch.all(ws[pad + nbytes:] == 0)


def test_workspace_reused_by_a_larger_batch(cs, orc, dev):
    """A split call leaves its whole workspace zero, so a later call with
    more questions on the same (cached) workspace, whose tickets then sit
    where the first call kept its slice partials, still merges correctly."""
    import torch

    K, D = 255, 2560
    first = workloads.normal_inputs(41, 1, K, D)
    second = workloads.normal_inputs(43, 100, K, D)
    g1 = cs.cs_plan_groups(1, K, D, "dot", True)
    g2 = cs.cs_plan_groups(100, K, D, "dot", True)
    note(f"case reuse: B=1 ({g1} slices) then B=100 ({g2} slices) on one workspace")
    assert g1 > 1 and g2 > 1
    # the second call's tickets overlap the first call's partials
    assert cs.cs_workspace_bytes_for_groups(100, g2) > 256 + 8 * g1
    nbytes = max(cs.cs_workspace_bytes(1, K, D, "dot"), cs.cs_workspace_bytes(100, K, D, "dot"))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    for rep in range(2):
        for Q, C in (first, second):
            B = Q.shape[0]
            q, c = to_dev(Q, dev), to_dev(C, dev)
            out = torch.empty(B, K, dtype=torch.float32, device=dev)
            st = cs.cs_score_candidates_batch(q, c, B, K, D, "dot", 0.0625, 1.0, out, ws, nbytes)
            assert st == 0
            torch.cuda.synchronize()
            want = orc.score(Q, C, "dot", 0.0625)
            check(out.cpu().numpy(), want, f"reuse rep={rep} B={B}")
            assert torch.all(ws == 0), int(torch.count_nonzero(ws))
    # the Python wrapper's cached workspace, same order
    for Q, C in (first, second):
        q, c = to_dev(Q, dev), to_dev(C, dev)
        out = cs.score(q, c, "dot", 0.0625, 1.0)
        torch.cuda.synchronize()
        check(out.cpu().numpy(), orc.score(Q, C, "dot", 0.0625), f"wrapper B={Q.shape[0]}")


def test_rejections_leave_device_output_untouched(cs, dev):
    import torch

    from pins import rejection_cases

    q = torch.randn(8, device=dev)
    c = torch.randn(4 * 8, device=dev)
    out = torch.full((64,), -7.0, device=dev)
    codes = {"NULL_POINTER": -1, "K_RANGE": -2, "D_RANGE": -3, "SCALE": -4, "TEMPERATURE": -5,
             "BATCH": -6, "SIMILARITY": -7}
    for origin, change, expect in rejection_cases():
        a = dict(query=q, candidates=c, out=out, B=1, K=4, D=8, similarity=0, scale=1.0,
                 temperature=1.0)
        a.update(change)
        st = cs.cs_score_candidates_batch(a["query"], a["candidates"], a["B"], a["K"], a["D"],
                                          a["similarity"], a["scale"], a["temperature"],
                                          a["out"])
        assert st == codes[expect], (origin, change)
    torch.cuda.synchronize()
    assert torch.all(out == -7.0)


def test_nan_propagates_to_its_row_only(cs, dev):
    import torch

    Q, C = workloads.normal_inputs(19, 3, 64, 256)
    C[1, 10, 100] = np.nan
    for ws in (False, True):
        out = cs.score(to_dev(Q, dev), to_dev(C, dev), "dot", 0.0625, 1.0, use_workspace=ws)
        torch.cuda.synchronize()
        p = out.cpu().numpy()
        assert np.all(np.isnan(p[1])) and np.all(np.isfinite(p[[0, 2]]))


def test_streams_with_own_workspaces_agree(cs, dev):
    """Two streams, each with its own workspace, run the split path
    concurrently many times; every result equals the serial one bitwise."""
    import torch

    B, K, D = 2, 255, 512
    Q, C = workloads.normal_inputs(23, B, K, D)
    q, c = to_dev(Q, dev), to_dev(C, dev)
    ref = cs.score(q, c, "cosine", 14.285714, 1.0)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    nbytes = cs.cs_workspace_bytes(B, K, D, "cosine")
    wss = [torch.zeros(nbytes, dtype=torch.uint8, device=dev) for _ in streams]
    outs = [[torch.empty(B, K, device=dev) for _ in range(50)] for _ in streams]
    torch.cuda.synchronize()
    note("case two streams x 50 split calls")
    for i in range(50):
        for s, ws, o in zip(streams, wss, outs):
            st = cs.cs_score_candidates_batch(q, c, B, K, D, "cosine", 14.285714, 1.0, o[i], ws,
                                              nbytes, stream=s)
            assert st == 0
    torch.cuda.synchronize()
    for o in outs:
        for t in o:
            assert torch.equal(t, ref)


def test_headline_batch_full_size(cs, orc, dev):
    """The 1024-question Kev batch at full size (2.67 GB of candidates), in
    the launch configuration the bench times, every element against the
    oracle."""
    import torch

    w = workloads.make(workloads.HEADLINE)
    note(f"case headline B={w.B} K={w.K} D={w.D}: oracle")
    want = orc.score(w.Q, w.C, w.similarity, w.scale, w.temperature)
    note("  copying inputs to the device")
    q, c = to_dev(w.Q, dev), to_dev(w.C, dev)
    assert cs.cs_plan_groups(w.B, w.K, w.D, w.similarity, True) == 1
    out = cs.score(q, c, w.similarity, float(w.scale), float(w.temperature))
    torch.cuda.synchronize()
    check(out.cpu().numpy(), want, "headline batch")


@pytest.mark.parametrize("B,K,D,sim,offset", [(64, 255, 2560, "dot", 0), (40, 255, 1024, "cosine", 0),
                                              (24, 200, 2049, "cosine", 0), (16, 255, 2560, "dot", 1)])
def test_streaming_paths(cs, orc, dev, B, K, D, sim, offset):
    """Candidate blocks above 32 MiB take the non-temporal streaming
    variants (register-query and general kernels), with and without a
    workspace."""
    import torch

    assert 4 * B * K * D >= 32 * 1024 * 1024
    Q, C = workloads.normal_inputs(29, B, K, D)
    scale = 14.285714 if sim == "cosine" else 0.0625
    want = orc.score(Q, C, sim, scale)
    qd = torch.zeros(B * D + offset, dtype=torch.float32, device=dev)
    cd = torch.zeros(B * K * D + offset, dtype=torch.float32, device=dev)
    qd[offset:] = to_dev(Q.reshape(-1), dev)
    cd[offset:] = to_dev(C.reshape(-1), dev)
    q, c = qd[offset:].view(B, D), cd[offset:].view(B, K, D)
    for ws in (False, True):
        note(f"case streaming B={B} K={K} D={D} {sim} offset={offset} ws={ws} "
             f"groups={cs.cs_plan_groups(B, K, D, sim, ws)}")
        out = cs.score(q, c, sim, scale, 1.0, use_workspace=ws)
        torch.cuda.synchronize()
        check(out.cpu().numpy(), want, f"streaming B={B} D={D} ws={ws}")


@pytest.mark.parametrize("name", ["clm_cos_5x512", "clm_cos_64x512", "clm_cos_255x512",
                                  "clm_cos_255x512_identical", "clm_cos_255x512_zero_row",
                                  "clm_cos_batch8_255x512", "clm_cos_batch8_255x512_overflow",
                                  "kev_dot_255x2560"])
def test_unfused_baseline(cs, orc, dev, name):
    """The unfused baseline (norm pass + scoring that loads staged norms)
    computes the same distribution."""
    import torch

    w = workloads.make(name)
    note(f"case unfused {name}")
    want = orc.score(w.Q, w.C, w.similarity, w.scale, w.temperature)
    q, c = to_dev(w.Q, dev), to_dev(w.C, dev)
    out = torch.empty(w.B, w.K, device=dev)
    norms = torch.full((w.B * w.K,), -1.0, device=dev)
    st = cs.cs_score_candidates_unfused(q, c, w.B, w.K, w.D, w.similarity, float(w.scale),
                                        float(w.temperature), out, norms)
    assert st == 0
    torch.cuda.synchronize()
    check(out.cpu().numpy(), want, f"unfused {name}")
    nref = np.linalg.norm(w.C.astype(np.float64), axis=2).reshape(-1)
    assert np.allclose(norms.cpu().numpy(), nref, rtol=1e-5, atol=1e-30)
    if name == "clm_cos_255x512_identical":
        assert np.all(out.cpu().numpy() == np.float32(1.0 / 255))


@pytest.mark.parametrize("D,offset", [(3, 0), (2560, 0), (4097, 0), (512, 1)])
def test_unfused_general_shapes(cs, orc, dev, D, offset):
    import torch

    B, K = 3, 77
    Q, C = workloads.normal_inputs(31, B, K, D)
    for sim in ("cosine", "dot"):
        want = orc.score(Q, C, sim, 3.0)
        qd = torch.zeros(B * D + offset, device=dev)
        cd = torch.zeros(B * K * D + offset, device=dev)
        qd[offset:] = to_dev(Q.reshape(-1), dev)
        cd[offset:] = to_dev(C.reshape(-1), dev)
        out = torch.empty(B, K, device=dev)
        norms = torch.empty(B * K, device=dev)
        note(f"case unfused general D={D} offset={offset} {sim}")
        st = cs.cs_score_candidates_unfused(qd[offset:], cd[offset:], B, K, D, sim, 3.0, 1.0,
                                            out, norms)
        assert st == 0
        torch.cuda.synchronize()
        check(out.cpu().numpy(), want, f"unfused D={D} {sim}")


@pytest.mark.parametrize("B,K,D,sim", [
    (300, 255, 2560, "dot"),    # 256 workgroups: 44 of them take a second question
    (600, 255, 512, "cosine"),  # several workgroups per compute unit
    (513, 255, 1000, "cosine"), # pieces past D: the partial instantiation
    (20000, 64, 64, "cosine"),  # dozens of questions per workgroup
    (3000, 64, 4, "dot"),       # the fewest rows that take the persistent grid
    (257, 130, 2560, "dot"),    # one question more than compute units
])
def test_persistent_batches(cs, orc, dev, B, K, D, sim):
    """Dense batches of more questions than compute units run the persistent
    grid, whose workgroups walk questions b, b + grid, ... and issue the next
    question's first loads before the current softmax; every element is
    checked against the oracle."""
    st, grid, block, groups = cs.cs_plan_launch(B, K, D, sim, False)
    assert st == 0 and groups == 1 and grid <= B, (st, grid, groups)
    st, name = cs.cs_plan_kernel(B, K, D, sim, False)
    assert st == 0 and name.startswith("fused_regq_stream<") and grid < B, name
    Q, C = workloads.normal_inputs(160 + B, B, K, D)
    scale = 14.285714 if sim == "cosine" else 0.0625
    note(f"case persistent B={B} K={K} D={D} {sim} grid={grid} block={block}")
    p = run(cs, Q, C, sim, scale, 1.0, dev, "batch", groups=1)
    check(p, orc.score(Q, C, sim, scale), f"persistent B={B} K={K} D={D} {sim}")


def test_persistent_identical_rows_give_exactly_one_over_k(cs, dev):
    """Identical candidates on the persistent grid: whichever wave draws a
    row group, every row goes through the same reduction, so each
    probability is exactly fp32(1/K) (the drawn row groups keep this)."""
    B, K, D = 2000, 255, 512
    rng = np.random.default_rng(171)
    Q = rng.standard_normal((B, D), dtype=np.float32)
    C = np.repeat(rng.standard_normal((B, 1, D), dtype=np.float32), K, axis=1)
    st, grid, block, groups = cs.cs_plan_launch(B, K, D, "cosine", False)
    assert st == 0 and grid < B
    note(f"case persistent identical rows B={B} K={K} D={D} grid={grid}")
    p = run(cs, Q, C, "cosine", 14.285714, 1.0, dev, "batch", groups=1)
    assert np.all(p == np.float32(1.0 / K))


def test_short_questions_keep_one_workgroup_each(cs):
    """Questions of fewer than 64 candidates stay on one workgroup per
    question, however many there are."""
    st, grid, block, groups = cs.cs_plan_launch(40000, 63, 256, "dot", False)
    assert st == 0 and grid == 40000 and groups == 1
    st, name = cs.cs_plan_kernel(40000, 63, 256, "dot", False)
    assert st == 0 and name.startswith("fused_regq<") and name.endswith("one workgroup per question>")


@pytest.mark.parametrize("sim", ["dot", "cosine"])
def test_batch_beyond_the_grid_cap(cs, orc, dev, sim):
    """More questions than the launch's grid cap (2^20 workgroups): the
    persistent grid's workgroups walk the questions. Every element is
    checked against the oracle."""
    B, K, D = (1 << 20) + 37, 3, 4
    st, grid, block, groups = cs.cs_plan_launch(B, K, D, sim, False)
    assert st == 0 and grid <= 1 << 20 and groups == 1, (st, grid, groups)
    Q, C = workloads.normal_inputs(120 if sim == "dot" else 121, B, K, D)
    note(f"case grid cap B={B} K={K} D={D} {sim} grid={grid} block={block}")
    p = run(cs, Q, C, sim, 2.0, 1.0, dev, "batch", groups=1)
    check(p, orc.score(Q, C, sim, 2.0), f"grid cap {sim}")
