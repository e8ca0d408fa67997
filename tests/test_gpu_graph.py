"""hipGraph capture of a scoring call.

Source: pull request "cuda: add a fused candidate-scoring kernel for CLM and
Kev", "Verified on hardware", fourth group: a capture holds exactly one node
and its replay matches a direct call exactly, not merely within tolerance.
For the split path, many replays also show that the last workgroup leaves
the workspace zeroed (no reset node is needed between replays).
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)


CASES = [("clm_cos_255x512", True), ("clm_cos_255x512", False), ("kev_dot_255x2560", True),
         ("clm_cos_batch8_255x512", True), ("clm_cos_5x512", True)]


@pytest.mark.parametrize("name,use_ws", CASES)
def test_capture_one_node_and_replay_exact(cs, name, use_ws):
    import torch

    bench = cs.load_bench()
    dev = torch.device("cuda:0")
    w = workloads.make(name)
    q = torch.from_numpy(w.Q).to(dev)
    c = torch.from_numpy(w.C).to(dev)
    direct = torch.empty(w.B, w.K, device=dev)
    replayed = torch.full((w.B, w.K), -1.0, device=dev)
    nbytes = cs.cs_workspace_bytes(w.B, w.K, w.D, w.similarity) if use_ws else 0
    ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=dev) if nbytes else None
    note(f"case graph {name} workspace={use_ws}")
    st = cs.cs_score_candidates_batch(q, c, w.B, w.K, w.D, w.similarity, float(w.scale),
                                      float(w.temperature), direct, ws, nbytes)
    assert st == 0
    torch.cuda.synchronize()
    call = cs.CsbCall(q.data_ptr(), c.data_ptr(), replayed.data_ptr(), w.B, w.K, w.D,
                      cs._sim(w.similarity), float(w.scale), float(w.temperature),
                      ws.data_ptr() if ws is not None else None, nbytes, 0)
    nodes = ctypes.c_size_t()
    assert bench.csb_graph_nodes(ctypes.byref(call), ctypes.byref(nodes)) == 0
    assert nodes.value == 1
    replays = 1000 if use_ws else 50
    assert bench.csb_graph_replay(ctypes.byref(call), replays, 0) == 0
    torch.cuda.synchronize()
    assert torch.equal(replayed, direct)
    if ws is not None:
        assert torch.all(ws[: 4 * w.B].view(torch.int32) == 0)
    # eager work between replays, then replay again with a sync per replay
    replayed.fill_(-1.0)
    _ = (q * 2).sum().item()
    assert bench.csb_graph_replay(ctypes.byref(call), 5, 1) == 0
    torch.cuda.synchronize()
    assert torch.equal(replayed, direct)


def test_workspace_init_kernel_zeroes(cs):
    import torch

    dev = torch.device("cuda:0")
    for n in (1, 3, 4, 257, 4096 + 3):
        buf = torch.full((n + 16,), 0xAB, dtype=torch.uint8, device=dev)
        assert cs.cs_workspace_init(buf, n) == 0
        torch.cuda.synchronize()
        assert torch.all(buf[:n] == 0) and torch.all(buf[n:] == 0xAB), n
