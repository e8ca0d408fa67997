"""CS_DEBUG_POINTERS=1: pointers that are not device memory are refused with
CS_ERR_HOST_POINTER before anything is enqueued.

Pull request "cuda: add a fused candidate-scoring kernel for CLM and Kev",
"Defects the GPU found", item 1: host buffers passed to the kernel. The
switch is read once per process, so the calls run in a child process with
it set. The host buffers are pinned (allocated with pin_memory=True) and
therefore readable by the device, so even a check that let one through
could not fault the GPU.
"""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import json, sys
sys.path.insert(0, sys.argv[1])
import numpy as np
import torch
import candidate_scoring_amd as cs
dev = torch.device("cuda:0")
B, K, D = 2, 255, 2560
q = torch.randn(B, D, device=dev)
c = torch.randn(B, K, D, device=dev)
out = torch.full((B, K), -3.0, device=dev)
nb = cs.cs_workspace_bytes(B, K, D, "dot")
ws = torch.zeros(nb, dtype=torch.uint8, device=dev)
pin = lambda t: t.pin_memory()
qh, ch, oh = pin(torch.randn(B, D)), pin(torch.randn(B, K, D)), pin(torch.zeros(B, K))
wh = pin(torch.zeros(nb, dtype=torch.uint8))
r = {}
batch = lambda qq, cc, oo, ww: cs.cs_score_candidates_batch(qq, cc, B, K, D, "dot", 0.0625, 1.0,
                                                           oo, ww, nb)
r["device"] = batch(q, c, out, ws)
torch.cuda.synchronize()
r["device_out_written"] = bool(torch.all(out != -3.0).item())
out.fill_(-3.0)
torch.cuda.synchronize()
r["host_query"] = batch(qh.data_ptr(), c, out, ws)
r["host_candidates"] = batch(q, ch.data_ptr(), out, ws)
r["host_out"] = batch(q, c, oh.data_ptr(), ws)
r["host_workspace"] = batch(q, c, out, wh.data_ptr())
r["single_host_candidates"] = cs.cs_score_candidates(q[0], ch[0].data_ptr(), K, D, "dot", 0.0625,
                                                     1.0, out[0], ws, nb)
r["noalloc_host_candidates"] = cs.cs_score_candidates_batch_noalloc(q, ch.data_ptr(), B, K, D,
                                                                    "dot", 0.0625, 1.0, out)
# a valid call of the entry point that allocates nothing (its workspace is the
# library's own static array): accepted, and equal to the batch call
ref = torch.empty(B, K, device=dev)
r["noalloc_device"] = cs.cs_score_candidates_batch_noalloc(q, c, B, K, D, "dot", 0.0625, 1.0, ref)
torch.cuda.synchronize()
ref2 = torch.empty(B, K, device=dev)
cs.cs_score_candidates_batch(q, c, B, K, D, "dot", 0.0625, 1.0, ref2, ws, nb)
torch.cuda.synchronize()
r["noalloc_equals_batch"] = bool(torch.equal(ref, ref2))
norms = torch.empty(B * K, device=dev)
r["unfused_host_norms"] = cs.cs_score_candidates_unfused(q, c, B, K, D, "dot", 0.0625, 1.0, out,
                                                         pin(torch.empty(B * K)).data_ptr())
offs = torch.tensor([0, 100, 255], dtype=torch.int64)
r["ragged_host_offsets"] = cs.cs_score_candidates_ragged(q, c.reshape(-1, D), pin(offs).data_ptr(),
                                                         B, 255, D, "dot", 0.0625, 1.0,
                                                         out.reshape(-1))
xq = torch.zeros(B, 64, dtype=torch.bfloat16, device=dev)
xc = torch.zeros(B, 8, 64, dtype=torch.bfloat16, device=dev)
wq = torch.zeros(64, 64, dtype=torch.bfloat16, device=dev)
wc = pin(torch.zeros(64, 64, dtype=torch.bfloat16))
pnb = cs.cs_projected_workspace_bytes(B, 64, 64, "dot")
pws = torch.zeros(pnb, dtype=torch.uint8, device=dev)
r["projected_host_head"] = cs.cs_score_projected(xq, xc, wq, wc.data_ptr(), B, 8, 64, 64, 64, "dot",
                                                 0.0625, 1.0, out[:, :8].contiguous(), pws, pnb)
torch.cuda.synchronize()
r["out_untouched"] = bool(torch.all(out == -3.0).item())
print("RESULT " + json.dumps(r), flush=True)
"""


def test_host_pointers_refused_in_debug_mode(cs):
    env = dict(os.environ, CS_DEBUG_POINTERS="1")
    print("case CS_DEBUG_POINTERS=1 in a child process", flush=True)
    proc = subprocess.run([sys.executable, "-c", CHILD, ROOT], env=env, capture_output=True,
                          text=True, timeout=240)
    print(proc.stdout[-2000:], proc.stderr[-2000:], flush=True)
    assert proc.returncode == 0
    line = [l for l in proc.stdout.splitlines() if l.startswith("RESULT ")][-1]
    r = json.loads(line[len("RESULT "):])
    assert r["device"] == cs.CS_OK and r["device_out_written"]
    assert r["noalloc_device"] == cs.CS_OK and r["noalloc_equals_batch"]
    for key in ("host_query", "host_candidates", "host_out", "host_workspace",
                "single_host_candidates", "noalloc_host_candidates", "unfused_host_norms",
                "ragged_host_offsets", "projected_host_head"):
        assert r[key] == cs.CS_ERR_HOST_POINTER, (key, r[key])
    assert r["out_untouched"]
