"""The entry point that allocates nothing (cs_score_candidates_batch_noalloc).

It is meant for callers that cannot allocate device memory, and it keeps
the split path's workspace in a static per-GPU array inside the library.
Here it is checked against the batch entry point with a caller-provided
workspace (same plan, same kernel: bitwise equal) and against the oracle
(1e-4 per element). The check covers two calls in a row, the second with
a smaller input, and then the first again. Every call must leave the static
array zero, or the next split call could not merge.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

TOL = 1e-4


def note(msg):
    print(msg, flush=True)


def test_noalloc_matches_the_batch_call(cs, orc):
    import torch

    dev = torch.device("cuda:0")
    cases = [  # (seed, B, K, D, similarity, scale): split plans, then a smaller one
        (301, 8, 255, 2560, "dot", 0.0625),
        (303, 1, 255, 512, "cosine", 14.285714),
        (301, 8, 255, 2560, "dot", 0.0625),
        (305, 300, 40, 256, "cosine", 14.285714),  # one workgroup per question: no scratch
    ]
    for seed, B, K, D, sim, scale in cases:
        G = cs.cs_plan_groups(B, K, D, sim, True)
        note(f"case noalloc seed={seed} B={B} K={K} D={D} {sim} slices={G}")
        assert cs.cs_workspace_bytes(B, K, D, sim) <= cs.CS_NOALLOC_SCRATCH_BYTES
        Q, C = workloads.normal_inputs(seed, B, K, D)
        q = torch.from_numpy(Q).to(dev)
        c = torch.from_numpy(C).to(dev)
        got = torch.full((B, K), -9.0, device=dev)
        ref = torch.full((B, K), -9.0, device=dev)
        nbytes = cs.cs_workspace_bytes(B, K, D, sim)
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
        st = cs.cs_score_candidates_batch_noalloc(q, c, B, K, D, sim, scale, 1.0, got)
        assert st == 0, st
        st = cs.cs_score_candidates_batch(q, c, B, K, D, sim, scale, 1.0, ref,
                                          ws if nbytes else None, nbytes)
        assert st == 0, st
        torch.cuda.synchronize()
        p, r = got.cpu().numpy(), ref.cpu().numpy()
        want = orc.score(Q, C, sim, scale)
        err = float(np.max(np.abs(p.astype(np.float64) - want)))
        note(f"  max|noalloc-oracle|={err:.3e}, bitwise equal to the batch call: "
             f"{np.array_equal(p, r)}")
        assert err <= TOL
        assert np.array_equal(p, r)
