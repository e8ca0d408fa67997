"""The convenience wrappers score_ragged() and score_projected(): the same
results as the C-ABI calls they marshal, checked against the oracle, and the
cached workspaces of the split and projected paths kept apart (the split
path needs its workspace zeroed between calls, the projection leaves
scratch in its own)."""
from __future__ import annotations

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

TOL = 1e-4


def note(msg):
    print(msg, flush=True)


def bf16(bits, dev):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)
    return t.view(torch.bfloat16)


def err(p, want):
    return float(np.max(np.abs(p.astype(np.float64) - want)))


@pytest.mark.parametrize("sim", ["cosine", "dot"])
def test_score_ragged_wrapper(cs, orc, sim):
    import torch

    dev = torch.device("cuda:0")
    offsets = workloads.ragged_offsets(301, 50)
    Q, C = workloads.ragged_inputs(302, offsets, 640)
    scale = workloads.SCALE_COSINE if sim == "cosine" else workloads.SCALE_DOT
    note(f"case score_ragged B=50 D=640 {sim}")
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    p = cs.score_ragged(torch.from_numpy(Q).to(dev), torch.from_numpy(C).to(dev),
                        torch.from_numpy(offsets.astype(np.int64)).to(dev), sim, float(scale),
                        status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    e = err(p.cpu().numpy(), orc.score_ragged(Q, C, offsets, sim, scale))
    note(f"  max|gpu-oracle|={e:.3e}")
    assert e <= TOL


def test_score_ragged_wrapper_rejects_bad_offsets(cs):
    import torch

    dev = torch.device("cuda:0")
    q = torch.zeros((2, 8), device=dev)
    c = torch.zeros((4, 8), device=dev)
    with pytest.raises(ValueError):
        cs.score_ragged(q, c, torch.tensor([0, 4], dtype=torch.int64, device=dev))
    with pytest.raises(ValueError):
        cs.score_ragged(q, c, torch.tensor([0, 2, 4], dtype=torch.int32, device=dev))


@pytest.mark.parametrize("B,K,Hq,Hc,P,sim", [
    (3, 255, 512, 512, 256, "cosine"),
    (3, 100, 520, 1000, 96, "dot"),
])
def test_score_projected_wrapper(cs, orc, B, K, Hq, Hc, P, sim):
    import torch

    dev = torch.device("cuda:0")
    w = workloads.projected_inputs(310 + K, B, K, Hq, Hc, P, sim)
    note(f"case score_projected B={B} K={K} Hq={Hq} Hc={Hc} P={P} {sim}")
    p = cs.score_projected(bf16(w.xq_bits, dev), bf16(w.xc_bits, dev), bf16(w.wq_bits, dev),
                           bf16(w.wc_bits, dev), sim, float(w.scale))
    torch.cuda.synchronize()
    want = orc.score_projected(w.f32("xq"), w.f32("wq"), w.f32("xc"), w.f32("wc"), sim, w.scale)
    e = err(p.cpu().numpy(), want)
    note(f"  max|gpu-oracle|={e:.3e}")
    assert e <= TOL


def test_split_and_projected_workspaces_interleaved(cs):
    """A split batch (several workgroups per question, which relies on its
    workspace staying zeroed between calls) before and after a projected
    call on the same stream gives the same bits both times."""
    import torch

    dev = torch.device("cuda:0")
    B, K, D = 2, 255, 2560
    st, grid, block, groups = cs.cs_plan_launch(B, K, D, "dot", True)
    assert st == 0 and groups > 1, (st, groups)
    Q, C = workloads.normal_inputs(320, B, K, D)
    q, c = torch.from_numpy(Q).to(dev), torch.from_numpy(C).to(dev)
    note(f"case split B={B} K={K} D={D} groups={groups} around a projected call")
    first = cs.score(q, c, "dot", 0.0625, 1.0).clone()
    w = workloads.projected_inputs(321, 4, 255, 2560, 2560, 256, "dot")
    cs.score_projected(bf16(w.xq_bits, dev), bf16(w.xc_bits, dev), bf16(w.wq_bits, dev),
                       bf16(w.wc_bits, dev), "dot", float(w.scale))
    second = cs.score(q, c, "dot", 0.0625, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(first, second)
