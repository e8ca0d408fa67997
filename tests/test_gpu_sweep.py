"""GPU parity over seeded random shapes, every entry point against the oracle.

Same bar as the fixed cases (pull request "cuda: add a fused
candidate-scoring kernel for CLM and Kev", "The manifest, and CI"):
max |p_gpu - p_oracle| <= 1e-4 per element, row sums within 1e-5.

Each family draws its cases from its own fixed seed:
* batch sizes across the single-question, split, one-workgroup-per-question
  and persistent plans;
* K from 1 to 255, hidden sizes that are and are not multiples of the
  16-byte piece, and both similarities;
* scales around the pages' own (1/0.07 for cosine, 1/sqrt(256) for dot);
* temperatures from 0.5 to 2.

Every case is named by its index and prints its shape before the device
call.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

TOL = 1e-4
SUM_TOL = 1e-5
N_DENSE, N_RAGGED, N_PROJECTED = 36, 24, 24


def note(msg):
    print(msg, flush=True)


def _hidden(rng):
    r = rng.random()
    if r < 0.4:
        return int(rng.choice([64, 128, 256, 512, 1024, 2048, 2560, 4096]))
    if r < 0.7:
        return int(rng.integers(1, 700) * 4)
    return int(rng.integers(1, 3000))


def _scale_t(rng, sim):
    base = float(workloads.SCALE_COSINE if sim == "cosine" else workloads.SCALE_DOT)
    return base * float(rng.uniform(0.25, 2.0)), float(rng.uniform(0.5, 2.0))


def dense_cases():
    rng = np.random.default_rng(20261)
    out = []
    for _ in range(N_DENSE):
        D = _hidden(rng)
        K = int(rng.integers(64, 256)) if rng.random() < 0.5 else int(rng.integers(1, 256))
        B = int(rng.choice([1, int(rng.integers(2, 9)), int(rng.integers(9, 300)),
                            int(rng.integers(257, 2100))]))
        if B > 256:  # the persistent plan: keep the batch, shrink the rows
            D = max(4, min(D, 40_000_000 // (B * K)) // 4 * 4)
        while B * K * D > 40_000_000:
            B = max(1, B // 2)
        sim = "cosine" if rng.random() < 0.5 else "dot"
        scale, T = _scale_t(rng, sim)
        out.append((B, K, D, sim, scale, T, bool(rng.random() < 0.7), int(rng.integers(1 << 30))))
    return out


def ragged_cases():
    rng = np.random.default_rng(20262)
    out = []
    for _ in range(N_RAGGED):
        D = _hidden(rng)
        B = int(rng.choice([1, int(rng.integers(2, 17)), int(rng.integers(17, 400)),
                            int(rng.integers(257, 2000))]))
        kmax = int(rng.integers(1, 256))
        counts = rng.integers(1, kmax + 1, size=B)
        while counts.sum() * D > 40_000_000:
            B = max(1, B // 2)
            counts = counts[:B]
        sim = "cosine" if rng.random() < 0.5 else "dot"
        scale, T = _scale_t(rng, sim)
        out.append((counts.astype(np.int64), D, sim, scale, T, bool(rng.random() < 0.6),
                    int(rng.integers(1 << 30))))
    return out


def projected_cases():
    rng = np.random.default_rng(20263)
    out = []
    for _ in range(N_PROJECTED):
        sim = "cosine" if rng.random() < 0.5 else "dot"
        B = int(rng.choice([1, int(rng.integers(2, 9)), int(rng.integers(9, 300)),
                            int(rng.integers(257, 1100))]))
        K = int(rng.integers(1, 256))
        Hq = int(rng.choice([8 * int(rng.integers(1, 40)), 512, 2560]))
        Hc = int(rng.choice([8 * int(rng.integers(1, 40)), 64 * int(rng.integers(1, 17)), 512,
                             2560]))
        # the cosine path implements P in multiples of 64 (CS_ERR_UNSUPPORTED otherwise)
        P = (int(rng.choice([64, 128, 192, 256])) if sim == "cosine"
             else int(rng.choice([int(rng.integers(1, 257)), 64, 128, 256])))
        while B * K * Hc * P > 300_000_000 or B * K * Hc > 40_000_000:
            B = max(1, B // 2)
        out.append((B, K, Hq, Hc, P, sim, int(rng.integers(1 << 30))))
    return out


def check(p, want, label):
    p64 = np.asarray(p, dtype=np.float64)
    err = float(np.max(np.abs(p64 - want)))
    sums = np.abs(p64.sum(axis=-1) - 1.0)
    note(f"  {label}: max|gpu-oracle|={err:.3e} max|rowsum-1|={float(sums.max()):.3e}")
    assert np.all(np.isfinite(p64)) and err <= TOL and float(sums.max()) <= SUM_TOL, label


@pytest.mark.parametrize("i", range(N_DENSE))
def test_dense_random(cs, orc, i):
    import torch

    B, K, D, sim, scale, T, use_ws, seed = dense_cases()[i]
    label = f"dense case {i}: B={B} K={K} D={D} {sim} scale={scale:.3f} T={T:.2f} ws={use_ws}"
    note(label)
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((B, D), dtype=np.float32)
    C = rng.standard_normal((B, K, D), dtype=np.float32)
    dev = torch.device("cuda:0")
    q, c = torch.from_numpy(Q).to(dev), torch.from_numpy(C).to(dev)
    if B == 1:
        out = cs.score(q[0], c[0], sim, scale, T, use_workspace=use_ws)[None, :]
    else:
        out = cs.score(q, c, sim, scale, T, use_workspace=use_ws)
    torch.cuda.synchronize()
    check(out.cpu().numpy(), orc.score(Q, C, sim, scale, T), label)


@pytest.mark.parametrize("i", range(N_RAGGED))
def test_ragged_random(cs, orc, i):
    import torch

    counts, D, sim, scale, T, use_ws, seed = ragged_cases()[i]
    B = counts.size
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    rows = int(offsets[-1])
    label = (f"ragged case {i}: B={B} rows={rows} K<={int(counts.max())} D={D} {sim} "
             f"scale={scale:.3f} T={T:.2f} ws={use_ws}")
    note(label)
    Q, C = workloads.ragged_inputs(seed, offsets, D)
    dev = torch.device("cuda:0")
    q, c, o = (torch.from_numpy(x).to(dev) for x in (Q, C, offsets))
    out = torch.full((rows,), -3.0, dtype=torch.float32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    nb = cs.cs_ragged_workspace_bytes(B, rows, D, sim) if use_ws else 0
    ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device=dev) if use_ws else None
    st = cs.cs_score_candidates_ragged(q, c, o, B, rows, D, sim, scale, T, out, status, ws, nb)
    assert st == 0, (label, st)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, label
    p = out.cpu().numpy().astype(np.float64)
    want = orc.score_ragged(Q, C, offsets, sim, scale, T)
    err = float(np.max(np.abs(p - want)))
    sums = np.abs(np.add.reduceat(p, offsets[:-1]) - 1.0)
    note(f"  max|gpu-oracle|={err:.3e} max|rowsum-1|={float(sums.max()):.3e}")
    assert np.all(np.isfinite(p)) and err <= TOL and float(sums.max()) <= SUM_TOL, label
    if use_ws:
        assert int(torch.count_nonzero(ws[:nb])) == 0, ("workspace not left zero", label)


@pytest.mark.parametrize("i", range(N_PROJECTED))
def test_projected_random(cs, orc, i):
    import torch

    B, K, Hq, Hc, P, sim, seed = projected_cases()[i]
    label = f"projected case {i}: B={B} K={K} Hq={Hq} Hc={Hc} P={P} {sim}"
    note(label)
    w = workloads.projected_inputs(seed, B, K, Hq, Hc, P, sim)
    dev = torch.device("cuda:0")

    def dev16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)

    xq, xc, wq, wc = dev16(w.xq_bits), dev16(w.xc_bits), dev16(w.wq_bits), dev16(w.wc_bits)
    out = torch.full((B, K), -3.0, dtype=torch.float32, device=dev)
    nb = cs.cs_projected_workspace_bytes(B, Hc, P, sim)
    ws = torch.zeros(nb, dtype=torch.uint8, device=dev)
    st = cs.cs_score_projected(xq, xc, wq, wc, B, K, Hq, Hc, P, sim, float(w.scale), 1.0, out,
                               ws, nb)
    assert st == 0, (label, st)
    torch.cuda.synchronize()
    want = orc.score_projected(w.f32("xq"), w.f32("wq"), w.f32("xc"), w.f32("wc"), sim, w.scale,
                               1.0)
    check(out.cpu().numpy(), want, label)
