"""Host-side checks of the C ABI that need no GPU: the library loads and
exports every function the header declares, arguments are rejected before
any HIP call, planning is a pure function, and the product path is separate
from the oracle.

Rejection list source: pull request "cuda: add a fused candidate-scoring
kernel for CLM and Kev", "Verified on hardware", third group.
"""
from __future__ import annotations

import ctypes
import re
import subprocess
from pathlib import Path

import numpy as np
import pytest

import candidate_scoring_amd as cs
from pins import STATUS_BY_NAME, rejection_cases

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "candidate_scoring.h"


@pytest.fixture(scope="module")
def lib():
    if not cs.LIBRARY.exists():
        from candidate_scoring_amd import build

        build.build()
    return cs.load()


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cs_[a-z_]+)\s*\(", text)))


def test_header_declares_the_page_entry_points():
    names = declared_functions()
    assert "cs_score_candidates" in names and "cs_score_candidates_batch" in names


def test_library_exports_every_declared_function(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", str(cs.LIBRARY)], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(cs_\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        assert hasattr(lib, n)


CLOCK_READERS = ("cs_phase_clocks_read", "cs_projected_phase_clocks_read",
                 "cs_ring_phase_clocks_read")


def test_measurement_build_exports_the_abi_and_its_clock_readers(lib):
    """libcs_phase.so (the same sources with CS_PHASE_CLOCKS) keeps every
    declared entry point and adds the three clock readers the bench's
    --phase-clocks sections call; the product library has none of them."""
    phase = cs.PKG / "libcs_phase.so"
    if not phase.exists():
        pytest.skip("measurement build not built (python -m candidate_scoring_amd.build "
                    "--phase-clocks)")

    def exported(path):
        out = subprocess.run(["nm", "-D", "--defined-only", str(path)], capture_output=True,
                             text=True, check=True).stdout
        return set(re.findall(r"\sT\s(cs_\w+)", out))

    in_phase, in_product = exported(phase), exported(cs.LIBRARY)
    assert not [n for n in declared_functions() if n not in in_phase]
    assert all(n in in_phase for n in CLOCK_READERS)
    assert not [n for n in CLOCK_READERS if n in in_product]


def test_bench_library_loads(lib):
    b = cs.load_bench()
    for n in ("csb_time_calls", "csb_time_graph", "csb_graph_nodes", "csb_time_empty", "csb_copy"):
        assert hasattr(b, n)


def test_version_and_status_strings(lib):
    assert cs.cs_abi_version() == cs.CS_ABI_VERSION == 1
    for code in range(-10, 1):
        s = cs.cs_status_string(code)
        assert s and s != "unknown status", code
    assert cs.cs_status_string(-99) == "unknown status"
    assert cs.cs_last_hip_error() == 0


def _host_buf(n, fill=-7.0):
    return np.full(max(n, 1), fill, dtype=np.float32)


CODE = {"OK": cs.CS_OK, "NULL_POINTER": cs.CS_ERR_NULL_POINTER, "K_RANGE": cs.CS_ERR_K_RANGE,
        "D_RANGE": cs.CS_ERR_D_RANGE, "SCALE": cs.CS_ERR_SCALE,
        "TEMPERATURE": cs.CS_ERR_TEMPERATURE, "BATCH": cs.CS_ERR_BATCH,
        "SIMILARITY": cs.CS_ERR_SIMILARITY}


def test_status_codes_match_the_oracle_numbering():
    # same published list, numbered independently on each side
    assert CODE == STATUS_BY_NAME


@pytest.mark.parametrize("case", rejection_cases(), ids=lambda c: f"{c[0]}:{list(c[1].items())[0]}")
def test_rejected_before_any_device_work(lib, case):
    """Each rejected argument returns its code; the host buffers passed as
    pointers are never touched (the call returns before any HIP call)."""
    origin, change, expect = case
    q, c, out = _host_buf(8), _host_buf(32), _host_buf(64)
    args = dict(query=q.ctypes.data, candidates=c.ctypes.data, out=out.ctypes.data, B=1, K=4,
                D=8, similarity=0, scale=1.0, temperature=1.0)
    for k, v in change.items():
        args[k] = None if v is None else v
        if k in ("query", "candidates", "out") and v is None:
            args[k] = None
    st = lib.cs_score_candidates_batch(args["query"], args["candidates"], args["B"], args["K"],
                                       args["D"], args["similarity"], args["scale"],
                                       args["temperature"], args["out"], None, 0, None)
    assert st == CODE[expect], (origin, change, st)
    assert np.all(out == -7.0) and np.all(q == -7.0) and np.all(c == -7.0)
    if "B" not in change:
        st1 = lib.cs_score_candidates(args["query"], args["candidates"], args["K"], args["D"],
                                      args["similarity"], args["scale"], args["temperature"],
                                      args["out"], None, 0, None)
        assert st1 == CODE[expect]
    # the entry point that allocates nothing validates the same way, before
    # it looks up or clears its static workspace
    st2 = lib.cs_score_candidates_batch_noalloc(args["query"], args["candidates"], args["B"],
                                                args["K"], args["D"], args["similarity"],
                                                args["scale"], args["temperature"], args["out"],
                                                None)
    assert st2 == CODE[expect], (origin, change, st2)
    assert np.all(out == -7.0) and np.all(q == -7.0) and np.all(c == -7.0)


def test_workspace_and_group_rejections(lib):
    q, c, out = _host_buf(512), _host_buf(255 * 512), _host_buf(255)
    ws = np.zeros(1 << 16, dtype=np.uint8)
    base = (q.ctypes.data, c.ctypes.data, 1, 255, 512, 1, 14.285714, 1.0, out.ctypes.data)
    # split path without a workspace
    assert lib.cs_score_candidates_batch_groups(*base, None, 0, 4, None) == cs.CS_ERR_WORKSPACE
    # too small
    need = cs.cs_workspace_bytes_for_groups(1, 4)
    assert need > 0
    assert lib.cs_score_candidates_batch_groups(*base, ws.ctypes.data, need - 1, 4,
                                                None) == cs.CS_ERR_WORKSPACE
    # misaligned
    assert lib.cs_score_candidates_batch_groups(*base, ws.ctypes.data + 4, need + 64, 4,
                                                None) == cs.CS_ERR_WORKSPACE
    # group counts outside 1..K, or leaving an empty slice (K=255, 254 groups)
    for g in (0, -1, 256, 254):
        assert lib.cs_score_candidates_batch_groups(*base, ws.ctypes.data, ws.size, g,
                                                    None) == cs.CS_ERR_WORKSPACE
    # the argument checks come first
    bad_k = (q.ctypes.data, c.ctypes.data, 1, 256, 512, 1, 1.0, 1.0, out.ctypes.data)
    assert lib.cs_score_candidates_batch_groups(*bad_k, None, 0, 4, None) == cs.CS_ERR_K_RANGE
    assert np.all(out == -7.0)
    assert lib.cs_workspace_init(None, 64, None) == cs.CS_ERR_NULL_POINTER


def test_planned_slices_fit_one_per_compute_unit(lib):
    """The planner never gives a batch more slice workgroups than MI355X has
    compute units (past that two slices share a unit), splits large
    questions in small batches, and keeps a big batch at one workgroup per
    question."""
    for D in (512, 1024, 2560, 4096):
        for B in (1, 2, 3, 8, 31, 48, 96, 128, 129, 256, 1024):
            G = cs.cs_plan_groups(B, 255, D, 0, True)
            assert G >= 1 and (G == 1 or B * G <= 256), (B, D, G)
            if B > 128:
                assert G == 1, (B, D, G)
    assert cs.cs_plan_groups(1, 255, 2560, 0, True) >= 32
    assert cs.cs_plan_groups(48, 255, 1024, 0, True) > 1   # 1 MB questions split early


def test_planning_is_pure_and_shared(lib):
    # no workspace: one workgroup per question
    for B, K, D in ((1, 5, 512), (1, 255, 512), (8, 255, 512), (1024, 255, 2560)):
        assert cs.cs_plan_groups(B, K, D, 1, False) == 1
    # with a workspace: a small batch spreads over the chip, a big one does not
    assert cs.cs_plan_groups(1, 255, 512, 1, True) > 1
    assert cs.cs_plan_groups(8, 255, 512, 1, True) > 1
    assert cs.cs_plan_groups(1024, 255, 2560, 0, True) == 1
    assert cs.cs_plan_groups(1, 1, 512, 1, True) == 1
    for B, K in ((1, 255), (3, 17), (8, 255), (100, 64)):
        G = cs.cs_plan_groups(B, K, 64, 0, True)
        rpg = -(-K // G)
        assert -(-K // rpg) == G, "planned slices must all be nonempty"
        assert cs.cs_workspace_bytes(B, K, 64, 0) == (
            cs.cs_workspace_bytes_for_groups(B, G) if G > 1 else 0)
    # invalid sizes plan nothing
    assert cs.cs_plan_groups(0, 5, 5, 0, True) == 0
    assert cs.cs_plan_groups(1, 256, 5, 0, True) == 0
    assert cs.cs_workspace_bytes(1, 0, 5, 0) == 0


def test_binding_refuses_host_tensors(lib):
    torch = pytest.importorskip("torch")
    t = torch.zeros(4)
    with pytest.raises(ValueError):
        cs._ptr(t)


def test_product_path_does_not_touch_the_oracle():
    """Neither the package nor its native code imports, links or names the
    oracle; the oracle in turn does not import the package."""
    pkg = ROOT / "candidate_scoring_amd"
    for f in list(pkg.rglob("*.py")) + list(pkg.rglob("*.hip")) + list(pkg.rglob("*.cpp")) + \
            list(pkg.rglob("*.h")):
        text = f.read_text()
        assert "import oracle" not in text and "from oracle" not in text, f
        assert "cs_oracle" not in text and "cso_" not in text, f
    for f in (ROOT / "oracle").glob("*"):
        if f.suffix in (".py", ".c", ".h"):
            text = f.read_text()
            assert "candidate_scoring_amd" not in text and "candidate_scoring.h" not in text, f
    if cs.LIBRARY.exists():
        out = subprocess.run(["nm", "-D", str(cs.LIBRARY)], capture_output=True, text=True).stdout
        assert "cso_" not in out
        deps = subprocess.run(["ldd", str(cs.LIBRARY)], capture_output=True, text=True).stdout
        assert "oracle" not in deps


def test_unfused_rejections_before_device_work(lib):
    q, c, out = _host_buf(8), _host_buf(32), _host_buf(64)
    norms = _host_buf(16)
    # missing staging buffer
    assert lib.cs_score_candidates_unfused(q.ctypes.data, c.ctypes.data, 1, 4, 8, 0, 1.0, 1.0,
                                           out.ctypes.data, None, None) == cs.CS_ERR_WORKSPACE
    for origin, change, expect in rejection_cases():
        a = dict(query=q.ctypes.data, candidates=c.ctypes.data, out=out.ctypes.data, B=1, K=4,
                 D=8, similarity=0, scale=1.0, temperature=1.0)
        a.update(change)
        st = lib.cs_score_candidates_unfused(a["query"], a["candidates"], a["B"], a["K"],
                                             a["D"], a["similarity"], a["scale"],
                                             a["temperature"], a["out"], norms.ctypes.data, None)
        assert st == CODE[expect], (origin, change)
    assert np.all(out == -7.0) and np.all(norms == -7.0)


def test_ragged_rejections_before_device_work(lib):
    q, c, out = _host_buf(16), _host_buf(64), _host_buf(64)
    offs = np.array([0, 3, 8], dtype=np.int64)
    base = dict(q=q.ctypes.data, c=c.ctypes.data, o=offs.ctypes.data, B=2, T=8, D=8, sim=0,
                scale=1.0, temp=1.0, out=out.ctypes.data)

    def call(**kw):
        a = dict(base, **kw)
        return lib.cs_score_candidates_ragged(a["q"], a["c"], a["o"], a["B"], a["T"], a["D"],
                                              a["sim"], a["scale"], a["temp"], a["out"], None,
                                              a.get("ws"), a.get("ws_bytes", 0), None)

    assert call(o=None) == cs.CS_ERR_NULL_POINTER
    assert call(q=None) == cs.CS_ERR_NULL_POINTER
    assert call(B=0) == cs.CS_ERR_BATCH
    assert call(T=1) == cs.CS_ERR_K_RANGE        # fewer rows than questions
    assert call(T=2 * 255 + 1) == cs.CS_ERR_K_RANGE
    assert call(D=0) == cs.CS_ERR_D_RANGE
    assert call(sim=5) == cs.CS_ERR_SIMILARITY
    assert call(scale=0.0) == cs.CS_ERR_SCALE
    assert call(temp=-1.0) == cs.CS_ERR_TEMPERATURE
    assert np.all(out == -7.0)
    # a split plan needs a workspace of cs_ragged_workspace_bytes(), 8-byte aligned
    qb, cb, ob = _host_buf(2560), _host_buf(255 * 2560), _host_buf(255)
    one = np.array([0, 255], dtype=np.int64)
    need = cs.cs_ragged_workspace_bytes(1, 255, 2560, "dot")
    assert need > 0
    ws = np.zeros(need + 64, dtype=np.uint8)
    wsp = (ws.ctypes.data + 15) // 16 * 16
    big = dict(q=qb.ctypes.data, c=cb.ctypes.data, o=one.ctypes.data, B=1, T=255, D=2560,
               out=ob.ctypes.data)
    assert call(**big, ws=wsp, ws_bytes=need - 1) == cs.CS_ERR_WORKSPACE
    assert call(**big, ws=wsp + 4, ws_bytes=need) == cs.CS_ERR_WORKSPACE
    assert call(**dict(big, D=0), ws=wsp, ws_bytes=need) == cs.CS_ERR_D_RANGE  # sizes first
    assert np.all(ob == -7.0)


def test_plan_queries_name_the_launch(lib):
    """cs_plan_kernel names the instantiation the batch call launches (the
    bench labels its roofline with it); both plan queries return the
    argument checks' status for invalid sizes."""
    st, name = cs.cs_plan_kernel(1024, 255, 2560, "dot", True)
    # with no device to ask for the persistent grid: one workgroup per question
    assert st == 0 and name.startswith("fused_regq<dot, 10 pieces/lane, 2 rows/wave, full")
    assert "non-temporal" in name and "one workgroup per question" in name
    st, name = cs.cs_plan_kernel(1, 255, 512, "cosine", True)
    assert st == 0 and name.startswith("fused_regq<cosine") and name.endswith("split>")
    st, name = cs.cs_plan_kernel(3, 255, 1000, "cosine", True, aligned16=False)
    assert st == 0 and name.startswith("fused_general<cosine, scalar")
    assert cs.cs_plan_kernel(0, 255, 512, "dot", True)[0] == cs.CS_ERR_BATCH
    assert cs.cs_plan_kernel(1, 256, 512, "dot", True)[0] == cs.CS_ERR_K_RANGE
    assert cs.cs_plan_launch(1, 255, 0, "dot", True)[0] == cs.CS_ERR_D_RANGE
    assert cs.cs_plan_launch(1, 255, 8, 7, True)[0] == cs.CS_ERR_SIMILARITY


def test_ragged_plan(lib):
    """Ragged slicing is planned from the mean count, like a dense question
    of that many rows, and never launches more slice workgroups than compute
    units even when every question has 255 rows."""
    # one question: the dense plan of the same question
    st, rpg, slices = cs.cs_plan_ragged(1, 255, 2560, "dot", True)
    G = cs.cs_plan_groups(1, 255, 2560, "dot", True)
    assert st == 0 and slices == G and rpg == -(-255 // G)
    # sixteen full questions: as the dense batch
    st, rpg, slices = cs.cs_plan_ragged(16, 16 * 255, 2560, "dot", True)
    G = cs.cs_plan_groups(16, 255, 2560, "dot", True)
    assert st == 0 and slices == G
    for B, rows, D in [(1, 40, 512), (3, 300, 2560), (8, 8 * 128, 2560), (16, 16 * 100, 1024),
                       (100, 100 * 255, 2560), (2, 100, 40000)]:
        st, rpg, slices = cs.cs_plan_ragged(B, rows, D, "cosine", True)
        assert st == 0 and 1 <= slices <= 64 and rpg >= 1
        assert slices == 1 or B * slices <= 256, (B, rows, D, rpg, slices)
        if slices > 1:
            assert slices == -(-255 // rpg)
            assert cs.cs_ragged_workspace_bytes(B, rows, D, "cosine") == \
                cs.cs_workspace_bytes_for_groups(B, slices)
        else:
            assert cs.cs_ragged_workspace_bytes(B, rows, D, "cosine") == 0
    # a large batch, or no workspace: one workgroup per question
    assert cs.cs_plan_ragged(1024, 1024 * 128, 2560, "dot", True)[2] == 1
    assert cs.cs_plan_ragged(1, 255, 2560, "dot", False)[1:] == (255, 1)
    assert cs.cs_plan_ragged(2, 1, 8, "dot", True)[0] == cs.CS_ERR_K_RANGE


def test_projected_rejections_before_device_work(lib):
    xq, xc = np.zeros(64, np.uint16), np.zeros(4 * 64, np.uint16)
    wq, wc = np.zeros(64 * 64, np.uint16), np.zeros(64 * 64, np.uint16)
    out = _host_buf(16)
    ws = np.zeros(1 << 16, np.uint8)
    wsp = (ws.ctypes.data + 255) // 256 * 256
    base = dict(xq=xq.ctypes.data, xc=xc.ctypes.data, wq=wq.ctypes.data, wc=wc.ctypes.data, B=1,
                K=4, Hq=64, Hc=64, P=64, sim=1, scale=1.0, T=1.0, out=out.ctypes.data, ws=wsp,
                nbytes=4096)

    def call(**kw):
        a = dict(base, **kw)
        return lib.cs_score_projected(a["xq"], a["xc"], a["wq"], a["wc"], a["B"], a["K"], a["Hq"],
                                      a["Hc"], a["P"], a["sim"], a["scale"], a["T"], a["out"],
                                      a["ws"], a["nbytes"], None)

    assert call(wq=None) == cs.CS_ERR_NULL_POINTER
    assert call(xq=None) == cs.CS_ERR_NULL_POINTER
    assert call(K=256) == cs.CS_ERR_K_RANGE
    assert call(K=0) == cs.CS_ERR_K_RANGE
    assert call(Hq=0) == cs.CS_ERR_D_RANGE
    assert call(Hc=0) == cs.CS_ERR_D_RANGE
    assert call(P=0) == cs.CS_ERR_D_RANGE
    assert call(scale=0.0) == cs.CS_ERR_SCALE
    assert call(T=-2.0) == cs.CS_ERR_TEMPERATURE
    assert call(Hq=60) == cs.CS_ERR_UNSUPPORTED          # not a multiple of 8
    assert call(P=300) == cs.CS_ERR_UNSUPPORTED          # more than 256 features
    assert call(P=96) == cs.CS_ERR_UNSUPPORTED           # cosine tiles features by 64
    assert call(sim=0, Hc=4104) == cs.CS_ERR_UNSUPPORTED  # folded query too long
    assert call(xc=xc.ctypes.data + 2) == cs.CS_ERR_UNSUPPORTED
    assert call(ws=None) == cs.CS_ERR_WORKSPACE
    assert call(nbytes=cs.cs_projected_workspace_bytes(1, 64, 64, 1) - 1) == cs.CS_ERR_WORKSPACE
    assert np.all(out == -7.0)
    assert cs.cs_projected_workspace_bytes(2, 64, 64, "dot") > cs.cs_projected_workspace_bytes(
        2, 64, 64, "cosine") > 0


def test_wrappers_check_shapes_and_dtypes_first():
    """score_ragged() and score_projected() refuse malformed arguments before
    any call into the library (host tensors suffice to show it)."""
    import torch

    q, c = torch.zeros((2, 8)), torch.zeros((4, 8))
    with pytest.raises(ValueError, match="B \\+ 1"):
        cs.score_ragged(q, c, torch.tensor([0, 4], dtype=torch.int64))
    with pytest.raises(ValueError, match="int64"):
        cs.score_ragged(q, c, torch.tensor([0, 2, 4], dtype=torch.int32))
    with pytest.raises(ValueError, match="total_rows"):
        cs.score_ragged(q, torch.zeros((4, 9)), torch.tensor([0, 2, 4], dtype=torch.int64))
    bf = torch.bfloat16
    xq, xc = torch.zeros((2, 64), dtype=bf), torch.zeros((2, 5, 64), dtype=bf)
    wq, wc = torch.zeros((64, 64), dtype=bf), torch.zeros((64, 64), dtype=bf)
    with pytest.raises(ValueError, match="shapes"):
        cs.score_projected(xq, xc[:1], wq, wc)
    with pytest.raises(ValueError, match="shapes"):
        cs.score_projected(xq, xc, wq, wc[:, :32])
    with pytest.raises(ValueError, match="bfloat16"):
        cs.score_projected(xq.float(), xc, wq, wc)
