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
         ("clm_cos_batch8_255x512", True), ("clm_cos_5x512", True),
         ("kev_dot_batch1024_255x2560", False)]  # the persistent grid


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


def _bits(b, dev):
    import torch

    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev)


@pytest.mark.parametrize("kind", ["ragged", "ragged_split", "projected_dot", "projected_cosine",
                                  "projected_dot_split", "projected_dot_split_tiles",
                                  "projected_cosine_slices"])
def test_capture_multi_kernel_paths_replay_exact(cs, kind):
    """The ragged and projection entry points captured into a graph (through
    torch's capture of the current stream) replay to exactly the direct
    call's result, with eager work between replays."""
    import torch

    dev = torch.device("cuda:0")
    note(f"case graph {kind}")
    if kind == "ragged":
        offsets = workloads.ragged_offsets(71, 300)
        Q, C = workloads.ragged_inputs(72, offsets, 520)
        rows = int(offsets[-1])
        q, c = torch.from_numpy(Q).to(dev), torch.from_numpy(C).to(dev)
        o = torch.from_numpy(offsets).to(dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)

        def run(out):
            assert cs.cs_score_candidates_ragged(q, c, o, 300, rows, 520, "cosine",
                                                 float(workloads.SCALE_COSINE), 1.0, out,
                                                 status) == 0

        shape = (rows,)
    elif kind == "ragged_split":
        # Eight questions of 1 to 255 rows, sliced over the chip and merged
        # through the zeroed workspace, which every call leaves zero.
        offsets = workloads.ragged_offsets(77, 8)
        Q, C = workloads.ragged_inputs(78, offsets, 2560)
        rows = int(offsets[-1])
        q, c = torch.from_numpy(Q).to(dev), torch.from_numpy(C).to(dev)
        o = torch.from_numpy(offsets).to(dev)
        nbytes = cs.cs_ragged_workspace_bytes(8, rows, 2560, "dot")
        assert nbytes > 0
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)

        def run(out):
            assert cs.cs_score_candidates_ragged(q, c, o, 8, rows, 2560, "dot",
                                                 float(workloads.SCALE_DOT), 1.0, out, None, ws,
                                                 nbytes) == 0

        shape = (rows,)
    else:
        sim = "cosine" if kind.startswith("projected_cosine") else "dot"
        if kind == "projected_dot_split":
            # Two questions of 1.3 MB: the candidate pass is split, merged
            # through tickets the query projection clears in the same graph
            # (matrix-vector query side).
            w = workloads.projected_inputs(74, 2, 255, 2560, 2560, 256, sim)
        elif kind == "projected_dot_split_tiles":
            # Ten questions: the same split behind the matrix-core query side.
            w = workloads.projected_inputs(75, 10, 255, 2560, 2560, 256, sim)
        elif kind == "projected_cosine_slices":
            # Two questions of 255 candidates, 32 per workgroup, merged
            # through the tickets.
            w = workloads.projected_inputs(76, 2, 255, 512, 512, 256, sim)
        else:
            w = workloads.projected_inputs(73, 300, 40, 136, 256, 128, sim)
        xq, xc = _bits(w.xq_bits, dev), _bits(w.xc_bits, dev)
        wq, wc = _bits(w.wq_bits, dev), _bits(w.wc_bits, dev)
        nbytes = cs.cs_projected_workspace_bytes(w.B, w.Hc, w.P, sim)
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)

        def run(out):
            assert cs.cs_score_projected(xq, xc, wq, wc, w.B, w.K, w.Hq, w.Hc, w.P, sim,
                                         float(w.scale), 1.0, out, ws, nbytes) == 0

        shape = (w.B, w.K)
    direct = torch.empty(shape, device=dev)
    run(direct)
    torch.cuda.synchronize()
    replayed = torch.full(shape, -1.0, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            run(replayed)
    torch.cuda.synchronize()
    for _ in range(3):
        replayed.fill_(-1.0)
        _ = (direct * 2).sum().item()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(replayed, direct)
