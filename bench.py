"""Bench for fused candidate scoring on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one call of the whole hot path (similarity + in-workgroup softmax)
over one batch: the 1024-question Kev-shaped batch (dot, K=255, D=2560, fp32,
2.67 GB of candidates), inputs resident in HBM before the timed region.
Timing uses HIP events on the stream the kernel runs on, around K
back-to-back calls issued from native code. Prints ONE JSON line.

Beside the headline it reports (same line):
  * roofline: algorithmic bytes per launch / event-timed launch duration
    against the 8 TB/s HBM peak, and the HBM traffic measured by rocprofv3
    counters when the committed profile matches the current kernel source;
  * latency: single-question and small-batch calls timed through hipGraph
    replay (2000 replays of a one-node graph in five repetitions, the page's
    protocol; median and min per call) and as back-to-back direct calls,
    each next to an empty kernel of the same grid and block timed the same
    way: the launch floors of both protocols;
  * cpu_baseline: the double-precision oracle on the host, single-threaded
    (and, under "threaded", the same oracle over up to 16 host threads),
    over the same batch.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = [ROOT / "candidate_scoring_amd" / "csrc" / n for n in ("cs_kernels.hip", "cs_device.h")]
TRAFFIC_PROFILE = ROOT / "profiles" / "fused_regq_kev_batch1024_255x2560_traffic.md"
LATENCY_CONFIGS = ["clm_cos_5x512", "clm_cos_255x512", "clm_cos_batch8_255x512",
                   "kev_dot_255x2560"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_sha256() -> str:
    """sha256 of the scoring kernels' source (kernel file and shared device
    header) with comments and whitespace removed, so that only code changes
    count as a changed kernel."""
    text = "\n".join(f.read_text() for f in KERNEL_SOURCES)
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()


OCCUPANCY_PROFILE = ROOT / "profiles" / "occupancy_kernels.md"


def committed_occupancy():
    """OccupancyPercent of the headline kernel from the committed counter
    profile, or None when missing or taken on different kernel code."""
    if not OCCUPANCY_PROFILE.exists():
        return None
    text = OCCUPANCY_PROFILE.read_text()
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_occ = re.search(r"occupancy_percent_headline:\s*([0-9.]+)", text)
    if not m_sha or not m_occ or m_sha.group(1) != source_sha256():
        return None
    return float(m_occ.group(1))


def committed_traffic():
    """HBM bytes per launch from the committed counter profile, or None when
    it is missing or was taken on a different kernel source."""
    if not TRAFFIC_PROFILE.exists():
        return None
    text = TRAFFIC_PROFILE.read_text()
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_tr = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_tr or m_sha.group(1) != source_sha256():
        return None
    return float(m_tr.group(1))


class Device:
    def __init__(self):
        import torch

        import candidate_scoring_amd as cs

        self.torch = torch
        self.cs = cs
        cs.load()
        self.bench = cs.load_bench()
        self.dev = torch.device("cuda:0")
        self.stream = torch.cuda.current_stream()

    def upload(self, w):
        t = self.torch
        q = t.from_numpy(w.Q).to(self.dev)
        c = t.from_numpy(w.C).to(self.dev)
        out = t.empty((w.B, w.K), dtype=t.float32, device=self.dev)
        return q, c, out

    def call(self, w, q, c, out, use_workspace=True, groups=0):
        cs = self.cs
        ws, nbytes = None, 0
        if groups > 0:
            nbytes = cs.cs_workspace_bytes_for_groups(w.B, groups)
        elif use_workspace:
            nbytes = cs.cs_workspace_bytes(w.B, w.K, w.D, w.similarity)
        if nbytes:
            ws = self.torch.zeros(nbytes, dtype=self.torch.uint8, device=self.dev)
        call = cs.CsbCall(q.data_ptr(), c.data_ptr(), out.data_ptr(), w.B, w.K, w.D,
                          cs._sim(w.similarity), float(w.scale), float(w.temperature),
                          ws.data_ptr() if ws is not None else None, nbytes, groups)
        return call, ws

    def time_calls(self, call, iters) -> float:
        ms = ctypes.c_float()
        st = self.bench.csb_time_calls(ctypes.byref(call), iters, self.stream.cuda_stream,
                                       ctypes.byref(ms))
        if st != 0:
            raise RuntimeError(f"csb_time_calls failed: {st}")
        return ms.value

    def time_rotating(self, call, copies, q_stride, c_stride, out_stride, iters) -> float:
        ms = ctypes.c_float()
        st = self.bench.csb_time_calls_rotating(ctypes.byref(call), copies, q_stride, c_stride,
                                                out_stride, iters, self.stream.cuda_stream,
                                                ctypes.byref(ms))
        if st != 0:
            raise RuntimeError(f"csb_time_calls_rotating failed: {st}")
        return ms.value

    def time_graph(self, call, replays, warmup=20):
        ms, nodes = ctypes.c_float(), ctypes.c_size_t()
        st = self.bench.csb_time_graph(ctypes.byref(call), 1, replays, warmup, ctypes.byref(ms),
                                       ctypes.byref(nodes))
        if st != 0:
            raise RuntimeError(f"csb_time_graph failed: {st}")
        return ms.value, nodes.value

    def time_empty(self, grid, block, iters, graph):
        ms = ctypes.c_float()
        st = self.bench.csb_time_empty(grid, block, iters, int(graph), 1,
                                       self.stream.cuda_stream, ctypes.byref(ms))
        if st != 0:
            raise RuntimeError(f"csb_time_empty failed: {st}")
        return ms.value


LATENCY_REPS = 5


def latency_section(devc, replays):
    cs = devc.cs
    res = {}
    for name in LATENCY_CONFIGS:
        w = workloads.make(name)
        q, c, out = devc.upload(w)
        row = {"B": w.B, "K": w.K, "D": w.D, "similarity": w.similarity}
        for label, use_ws in (("split", True), ("one_wg_per_question", False)):
            call, _ws = devc.call(w, q, c, out, use_workspace=use_ws)
            devc.time_calls(call, 50)
            st, grid, block, G = cs.cs_plan_launch(w.B, w.K, w.D, w.similarity, use_ws)
            assert st == 0
            # five repetitions of replays/5 calls each; median (and min) per call
            n = max(1, replays // LATENCY_REPS)
            g, d, f, fd = [], [], [], []
            nodes = 0
            for _ in range(LATENCY_REPS):
                g_ms, nodes = devc.time_graph(call, n)
                g.append(1e3 * g_ms / n)
                d.append(1e3 * devc.time_calls(call, n) / n)
                f.append(1e3 * devc.time_empty(grid, block, n, True) / n)
                fd.append(1e3 * devc.time_empty(grid, block, n, False) / n)
            direct, floor_direct = float(np.median(d)), float(np.median(fd))
            row[label] = {"groups": G, "grid": grid, "block": block,
                          "graph_us_per_call": round(float(np.median(g)), 3),
                          "graph_us_per_call_min": round(min(g), 3),
                          "direct_us_per_call": round(direct, 3),
                          "direct_us_per_call_min": round(min(d), 3),
                          "graph_nodes": nodes,
                          "empty_kernel_graph_floor_us": round(float(np.median(f)), 3),
                          "empty_kernel_direct_floor_us": round(floor_direct, 3),
                          "empty_kernel_direct_floor_us_min": round(min(fd), 3),
                          "direct_over_direct_floor": round(direct / floor_direct, 3),
                          "reps": LATENCY_REPS, "calls_per_rep": n}
        res[name] = row
        log(f"latency {name}: {row}")
        del q, c, out
    return res


PHASES = [("loads and row sums", 0, 1), ("barrier", 1, 2), ("softmax and stores", 2, 3),
          ("release fence", 3, 4), ("ticket", 4, 5)]
LAST_PHASES = [("acquire fence", 6, 7), ("read e_k and partials, merge factors", 7, 8),
               ("rescale, stores, reset", 8, 9)]
PHASE_TICK_US = 0.01  # the device clock read by the stamps runs at 100 MHz


def phase_clock_section(devc, calls=200, reps=40):
    """Where a split call's time goes: the measurement build's per-phase
    device clocks (thread 0 of each workgroup) for the last of `calls`
    back-to-back direct calls, `reps` times; medians over repetitions of
    the per-workgroup phase durations, of the merging (last) slice's phases
    and of the kernel's span, beside the direct call rate and the empty
    kernel's direct floor."""
    cs, torch = devc.cs, devc.torch
    lib = cs.load()
    slots = 16
    res = {}
    for name in LATENCY_CONFIGS:
        w = workloads.make(name)
        q, c, out = devc.upload(w)
        call, _ws = devc.call(w, q, c, out, use_workspace=True)
        st, grid, block, G = cs.cs_plan_launch(w.B, w.K, w.D, w.similarity, True)
        assert st == 0
        if G < 2:
            continue
        devc.time_calls(call, 300)
        direct = 1e3 * devc.time_calls(call, 2000) / 2000
        floor = 1e3 * devc.time_empty(grid, block, 2000, False) / 2000
        buf = np.zeros(grid * slots, dtype=np.uint64)
        runs = []
        for _ in range(reps):
            devc.time_calls(call, calls)
            torch.cuda.synchronize()
            if lib.cs_phase_clocks_read(ctypes.c_void_p(buf.ctypes.data), buf.nbytes) != 0:
                raise RuntimeError("cs_phase_clocks_read failed")
            runs.append(buf.reshape(grid, slots).astype(np.int64))
        T = np.stack(runs)                              # [rep, workgroup, slot]
        if not np.all(T[:, :, 0] > 0):
            raise RuntimeError("no phase clocks recorded: the calls did not reach libcs_phase.so")
        t0 = T[:, :, 0].min(axis=1)
        # the merging slice of the last call: slots 7..9 newer than its start
        last = (T[:, :, 9] > T[:, :, 0]) & (T[:, :, 7] >= T[:, :, 0])
        row = {"B": w.B, "K": w.K, "D": w.D, "similarity": w.similarity, "slices": G,
               "workgroups": grid, "direct_us_per_call": round(direct, 3),
               "empty_kernel_direct_floor_us": round(floor, 3)}
        for label, a, b in PHASES:
            row[label + " us"] = round(float(np.median((T[:, :, b] - T[:, :, a]) * PHASE_TICK_US)), 3)
        for label, a, b in LAST_PHASES:
            v = [float(((T[i][last[i]][:, b] - T[i][last[i]][:, a]) * PHASE_TICK_US).mean())
                 for i in range(reps) if last[i].any()]
            row["last slice: " + label + " us"] = round(float(np.median(v)), 3)
        row["start spread us"] = round(float(np.median((T[:, :, 0].max(axis=1) - t0) * PHASE_TICK_US)), 3)
        row["last ticket drawn at us"] = round(float(np.median((T[:, :, 5].max(axis=1) - t0) * PHASE_TICK_US)), 3)
        row["kernel span us"] = round(float(np.median(
            (np.maximum(T[:, :, 10].max(axis=1), T[:, :, 9].max(axis=1)) - t0) * PHASE_TICK_US)), 3)
        res[name] = row
        log(f"phase clocks {name}: {row}")
        del q, c, out
    return res


def projected_phase_section(devc, calls=6, reps=12):
    """Where the Kev projection call's time goes: the measurement build's
    clocks in its three launches (query projection, fold, bf16 candidate
    pass) for the last of `calls` back-to-back calls, `reps` times; medians
    over repetitions of each phase (per-workgroup phases as the median over
    workgroups), of the gaps between launches and of when the candidate
    pass's workgroups end, by dispatch order (blockIdx // 256) and by
    blockIdx mod 8 (the XCD under round-robin dispatch)."""
    torch, cs = devc.torch, devc.cs
    lib = cs.load()
    name = "kev_proj_dot_batch1024_255x2560_p256"
    w = workloads.make_projected(name)

    def dev16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(devc.dev)

    xq, xc, wq, wc = dev16(w.xq_bits), dev16(w.xc_bits), dev16(w.wq_bits), dev16(w.wc_bits)
    out = torch.empty(w.B, w.K, dtype=torch.float32, device=devc.dev)
    nbytes = cs.cs_projected_workspace_bytes(w.B, w.Hc, w.P, w.similarity)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=devc.dev)

    def once():
        st = cs.cs_score_projected(xq, xc, wq, wc, w.B, w.K, w.Hq, w.Hc, w.P, w.similarity,
                                   float(w.scale), 1.0, out, ws, nbytes, devc.stream)
        assert st == 0, st

    regions, wgs, slots = 4, 1024, 16
    buf = np.zeros(regions * wgs * slots, dtype=np.uint64)
    fields = {}
    nfold = None
    for _ in range(reps):
        for _ in range(calls):
            once()
        torch.cuda.synchronize()
        if lib.cs_projected_phase_clocks_read(ctypes.c_void_p(buf.ctypes.data), buf.nbytes) != 0:
            raise RuntimeError("cs_projected_phase_clocks_read failed")
        T = buf.reshape(regions, wgs, slots).astype(np.int64)
        proj, fold, cand = T[1, :256], T[2], T[3]
        if nfold is None:
            # workgroups of each launch: the ones stamped by this call
            nfold = int(np.count_nonzero(fold[:, 2] >= proj[:, 0].min()))
            ncand = int(np.count_nonzero(cand[:, 5] >= proj[:, 0].min()))
        fold, cand = fold[:nfold], cand[:ncand]
        if not (proj[:, 0].min() > 0 and nfold > 0 and cand[:, 5].min() > 0):
            raise RuntimeError("no phase clocks recorded: the calls did not reach libcs_phase.so")
        t0 = proj[:, 0].min()
        us = lambda v: float(v) * PHASE_TICK_US
        med = lambda a, b, x: us(np.median(x[:, b] - x[:, a]))
        cend = cand[:, 5] - cand[:, 0].min()
        # Bytes streamed while every workgroup of the pass is running: each
        # workgroup's progress interpolated between its stamps (u staged,
        # a quarter, half, three quarters of its rows, exit).
        marks = np.stack([cand[:, 1], cand[:, 2], cand[:, 3], cand[:, 4], cand[:, 5]], axis=1)
        ta, tb = np.median(cand[:, 1]), cand[:, 5].min()
        frac = np.array([0.0, 0.25, 0.5, 0.75, 1.0])
        done = sum(np.interp(tb, m, frac) - np.interp(ta, m, frac) for m in marks.astype(np.float64))
        qbytes = 2.0 * w.K * w.Hc * w.B / ncand  # bytes per workgroup
        row = {
            "query projection: contraction, wave 0": med(0, 1, proj),
            "query projection: wait for the other waves": med(1, 2, proj),
            "query projection: q' and parts stored": med(2, 3, proj),
            "query projection: W^T share packed": med(3, 4, proj),
            "query projection: span": us(proj[:, 4].max() - t0),
            "gap, projection to fold": us(fold[:, 0].min() - proj[:, 4].max()),
            "fold: contraction, wave 0": med(0, 1, fold),
            "fold: u stored": med(1, 2, fold),
            "fold: span": us(fold[:, 2].max() - fold[:, 0].min()),
            "gap, fold to candidate pass": us(cand[:, 0].min() - fold[:, 2].max()),
            "candidate pass: u staged": med(0, 1, cand),
            "candidate pass: first workgroup done": us(cend.min()),
            "candidate pass: TB/s while every workgroup runs":
                done * qbytes / (us(tb - ta) * 1e-6) / 1e12,
            "candidate pass: median workgroup done": us(np.median(cend)),
            "candidate pass: span": us(cend.max()),
            "call span": us(cand[:, 5].max() - t0),
        }
        for r in range(ncand // 256):
            sel = slice(256 * r, 256 * (r + 1))
            row[f"candidate pass: workgroups {256 * r}-{256 * r + 255} done, median"] = \
                us(np.median(cend[sel]))
        for x in range(8):
            row[f"candidate pass: blockIdx mod 8 = {x} done, median"] = \
                us(np.median(cend[np.arange(ncand) % 8 == x]))
        row["candidate pass: workgroups done, 10th percentile"] = us(np.percentile(cend, 10))
        row["candidate pass: workgroups done, 90th percentile"] = us(np.percentile(cend, 90))
        for k, v in row.items():
            fields.setdefault(k, []).append(v)
    res = {"workload": name, "B": w.B, "K": w.K, "Hq": w.Hq, "Hc": w.Hc, "P": w.P,
           "fold_workgroups": nfold, "candidate_pass_workgroups": ncand, "calls": calls,
           "reps": reps}
    res.update({k + ("" if "TB/s" in k else " us"): round(float(np.median(v)), 3)
                for k, v in fields.items()})
    log(f"projected phase clocks: {res}")
    del xq, xc, wq, wc, out, ws
    return res


def ring_phase_section(devc, calls=4, reps=8):
    """Where the CLM cosine ring kernel's cycles go: the measurement build's
    per-wave clocks (s_memtime) for the second question of each of the 256
    workgroups, in the last of `calls` back-to-back calls, `reps` times.
    Per chunk step: the vmcnt wait, the ring barrier, the DMA issue (waves
    0-3 only), the fragment reads and matrix instructions, and the time to
    the next step; then the epilogue's parts. Medians over workgroups, then
    over repetitions, for the DMA-issuing waves (0-3) and the others (4-7)."""
    torch, cs = devc.torch, devc.cs
    lib = cs.load()
    name = "clm_proj_cos_batch1024_255x512_p256"
    w = workloads.make_projected(name)

    def dev16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(devc.dev)

    xq, xc, wq, wc = dev16(w.xq_bits), dev16(w.xc_bits), dev16(w.wq_bits), dev16(w.wc_bits)
    out = torch.empty(w.B, w.K, dtype=torch.float32, device=devc.dev)
    nbytes = cs.cs_projected_workspace_bytes(w.B, w.Hc, w.P, w.similarity)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=devc.dev)
    groups, waves, slots = 256, 8, 49
    buf = np.zeros(groups * waves * slots, dtype=np.uint64)
    steps = ("vmcnt wait", "ring barrier", "DMA issue", "fragment reads + MFMA", "to next step")
    epi = ("row reductions", "first barrier", "second barrier", "softmax (wave 0) / exit")
    acc = {}
    for _ in range(reps):
        for _ in range(calls):
            st = cs.cs_score_projected(xq, xc, wq, wc, w.B, w.K, w.Hq, w.Hc, w.P, w.similarity,
                                       float(w.scale), 1.0, out, ws, nbytes, devc.stream)
            assert st == 0, st
        torch.cuda.synchronize()
        if lib.cs_ring_phase_clocks_read(ctypes.c_void_p(buf.ctypes.data), buf.nbytes) != 0:
            raise RuntimeError("cs_ring_phase_clocks_read failed")
        T = buf.reshape(groups, waves, slots).astype(np.int64)
        if T[:, :, 44].min() <= 0:
            raise RuntimeError("no ring clocks recorded: the calls did not reach libcs_phase.so")
        # cycles per 10 ns tick between the first and the third question's ends
        ghz = np.median((T[:, :, 47] - T[:, :, 45]) / (T[:, :, 48] - T[:, :, 46])) / 10.0
        acc.setdefault("clock GHz", []).append(ghz)
        for role, sel in (("DMA waves 0-3", slice(0, 4)), ("waves 4-7", slice(4, 8))):
            R = T[:, sel]
            for c in range(8):
                t = [R[:, :, 5 * c + k] for k in range(5)]
                nxt = R[:, :, 5 * (c + 1)] if c < 7 else R[:, :, 40]
                for name_, v in zip(steps, (t[1] - t[0], t[2] - t[1], t[3] - t[2], t[4] - t[3],
                                            nxt - t[4])):
                    acc.setdefault((role, name_), [[] for _ in range(8)])[c].append(np.median(v))
            e = [R[:, :, 40 + k] for k in range(5)]
            for k, name_ in enumerate(epi):
                acc.setdefault((role, name_), []).append(np.median(e[k + 1] - e[k]))
            acc.setdefault((role, "question"), []).append(np.median(R[:, :, 44] - R[:, :, 0]))
        acc.setdefault("wave 0 softmax", []).append(np.median(T[:, 0, 44] - T[:, 0, 43]))
    ghz = float(np.median(acc["clock GHz"]))
    res = {"workload": name, "B": w.B, "K": w.K, "Hc": w.Hc, "P": w.P, "calls": calls,
           "reps": reps, "clock_GHz": round(ghz, 3), "unit": "cycles (s_memtime)"}
    for role in ("DMA waves 0-3", "waves 4-7"):
        r = {}
        for name_ in steps:
            r[name_ + " per chunk"] = [int(round(np.median(x))) for x in acc[(role, name_)]]
        for name_ in epi:
            r["epilogue: " + name_] = int(round(np.median(acc[(role, name_)])))
        q = float(np.median(acc[(role, "question")]))
        r["question"] = int(round(q))
        r["question us"] = round(q / ghz / 1e3, 3)
        res[role] = r
    res["epilogue: softmax, wave 0"] = int(round(np.median(acc["wave 0 softmax"])))
    log(f"ring phase clocks: {res}")
    del xq, xc, wq, wc, out, ws
    return res


def ab_section(devc, iters, headline=None):
    """Fused vs the unfused baseline (separate norm pass + scoring that loads
    the staged norms) on the page's results-table shapes and the Kev batch.
    Direct back-to-back calls, warm caches for the small shapes."""
    torch = devc.torch
    res = {}
    for name in workloads.AB_SHAPES:
        if name == workloads.HEADLINE and headline is not None:
            w, q, c, out = headline
        else:
            w = workloads.make(name)
            q, c, out = devc.upload(w)
        norms = torch.empty(w.B * w.K, dtype=torch.float32, device=devc.dev)
        planned, _ws = devc.call(w, q, c, out, use_workspace=True)
        one_wg, _ = devc.call(w, q, c, out, use_workspace=False)
        unfused, _ = devc.call(w, q, c, out, use_workspace=False)
        unfused.row_norms = norms.data_ptr()
        n = iters if w.B * w.K * w.D < 50_000_000 else 10
        t = {}
        for label, call in (("fused", planned), ("fused_one_wg_per_question", one_wg),
                            ("unfused", unfused)):
            devc.time_calls(call, 3)
            t[label] = 1e3 * devc.time_calls(call, n) / n
        res[name] = {"B": w.B, "K": w.K, "D": w.D, "similarity": w.similarity,
                     "fused_us": round(t["fused"], 3),
                     "fused_one_wg_per_question_us": round(t["fused_one_wg_per_question"], 3),
                     "unfused_us": round(t["unfused"], 3),
                     "unfused_over_fused": round(t["unfused"] / t["fused"], 3),
                     "unfused_over_fused_one_wg": round(t["unfused"] / t["fused_one_wg_per_question"], 3)}
        log(f"a/b {name}: {res[name]}")
        if not (name == workloads.HEADLINE and headline is not None):
            del q, c, out
    return res


def cold_section(devc, iters, target_bytes=768 << 20):
    """Single-question and small-batch calls with cold caches: each call
    reads the next of enough input copies to exceed the 256 MB Infinity
    Cache and the L2s several times over (direct calls, planned split)."""
    torch = devc.torch
    res = {}
    for name in LATENCY_CONFIGS:
        w = workloads.make(name)
        per = w.B * w.K * w.D * 4
        copies = max(2, -(-target_bytes // per))
        q = torch.from_numpy(w.Q).to(devc.dev).reshape(-1).repeat(copies)
        c = torch.from_numpy(w.C).to(devc.dev).reshape(-1).repeat(copies)
        out = torch.empty(copies * w.B * w.K, dtype=torch.float32, device=devc.dev)
        call, _ws = devc.call(w, q, c, out, use_workspace=True)
        devc.time_rotating(call, copies, w.B * w.D, w.B * w.K * w.D, w.B * w.K, copies)
        ms = devc.time_rotating(call, copies, w.B * w.D, w.B * w.K * w.D, w.B * w.K, iters)
        res[name] = {"copies": copies, "cold_direct_us_per_call": round(1e3 * ms / iters, 3)}
        log(f"cold {name}: {res[name]}")
        del q, c, out
    return res


def ragged_section(devc, iters=20):
    """A ragged Kev-shaped batch: 1024 questions, counts uniform in 1..255,
    D=2560, dot, one launch (cs_score_candidates_ragged)."""
    torch = devc.torch
    cs = devc.cs
    B, D = 1024, 2560
    offsets = workloads.ragged_offsets(61, B)
    Q, C = workloads.ragged_inputs(67, offsets, D)
    rows = int(offsets[-1])
    q = torch.from_numpy(Q).to(devc.dev)
    c = torch.from_numpy(C).to(devc.dev)
    o = torch.from_numpy(offsets).to(devc.dev)
    out = torch.empty(rows, dtype=torch.float32, device=devc.dev)
    status = torch.zeros(1, dtype=torch.int32, device=devc.dev)

    def once():
        st = cs.cs_score_candidates_ragged(q, c, o, B, rows, D, "dot", float(workloads.SCALE_DOT),
                                           1.0, out, status, stream=devc.stream)
        assert st == 0, st

    for _ in range(3):
        once()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(devc.stream)
    for _ in range(iters):
        once()
    e1.record(devc.stream)
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / iters
    nbytes = 4 * (rows * D + B * D + rows)
    assert int(status.item()) == 0
    res = {"B": B, "rows": rows, "D": D, "similarity": "dot", "us_per_call": round(us, 2),
           "algorithmic_bytes": nbytes, "GBps": round(nbytes / us / 1e3, 1),
           "frac_of_hbm_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}
    log(f"ragged: {res}")
    del q, c, o, out
    res["small_batches"] = ragged_small_section(devc)
    return res


def ragged_small_section(devc, calls=2000):
    """Small ragged batches spread over the chip (a zeroed workspace): 16
    questions of 255 x 2560 (dot) next to the dense batch call on the same
    data, and a batch of 8 questions with counts uniform in 1..255, each
    also without a workspace (one workgroup per question). Back-to-back
    direct calls, warm caches, median of five repetitions."""
    torch, cs = devc.torch, devc.cs
    res = {}
    for label, B, counts_seed in (("16 x 255 rows", 16, None), ("8 questions, 1..255 rows", 8, 79)):
        D = 2560
        if counts_seed is None:
            offsets = np.arange(B + 1, dtype=np.int64) * 255
        else:
            offsets = workloads.ragged_offsets(counts_seed, B)
        Q, C = workloads.ragged_inputs(83, offsets, D)
        rows = int(offsets[-1])
        q, c = torch.from_numpy(Q).to(devc.dev), torch.from_numpy(C).to(devc.dev)
        o = torch.from_numpy(offsets).to(devc.dev)
        out = torch.empty(rows, dtype=torch.float32, device=devc.dev)
        nbytes = cs.cs_ragged_workspace_bytes(B, rows, D, "dot")
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=devc.dev)
        _, rpg, slices = cs.cs_plan_ragged(B, rows, D, "dot", True)

        def timed(fn):
            for _ in range(50):
                fn()
            t = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(devc.stream)
                for _ in range(calls // 5):
                    fn()
                e1.record(devc.stream)
                torch.cuda.synchronize()
                t.append(1e3 * e0.elapsed_time(e1) / (calls // 5))
            return round(float(np.median(t)), 3)

        def ragged(w, n):
            def f():
                assert cs.cs_score_candidates_ragged(q, c, o, B, rows, D, "dot",
                                                     float(workloads.SCALE_DOT), 1.0, out, None,
                                                     w, n, devc.stream) == 0
            return f

        row = {"B": B, "rows": rows, "D": D, "rows_per_slice": rpg, "max_slices": slices,
               "split_us_per_call": timed(ragged(ws, nbytes)),
               "one_wg_per_question_us_per_call": timed(ragged(None, 0))}
        if counts_seed is None:
            dq, dc = q, c.reshape(B, 255, D)
            dout = out.reshape(B, 255)
            call, _dws = devc.call(workloads.Workload("dense", "batch", "dot",
                                                      np.float32(workloads.SCALE_DOT),
                                                      np.float32(1.0), Q, C.reshape(B, 255, D),
                                                      ""), dq, dc, dout)
            devc.time_calls(call, 50)
            row["dense_batch_split_us_per_call"] = round(
                float(np.median([1e3 * devc.time_calls(call, calls // 5) / (calls // 5)
                                 for _ in range(5)])), 3)
            row["ragged_over_dense"] = round(row["split_us_per_call"] /
                                             row["dense_batch_split_us_per_call"], 3)
        res[label] = row
        log(f"ragged small {label}: {row}")
        del q, c, o, out, ws
    return res


MFMA_BF16_PEAK_TFLOPS = 2500.0


def projected_section(devc, iters=20, one_question=True):
    """Projection + scoring on the two 1024-question head workloads (bf16
    hidden states and heads): Kev (dot, heads 2560 -> 256, folded into the
    query) and CLM (cosine, heads 512 -> 256, candidate projection on the
    matrix cores). Reports us/call, HBM GB/s of the bf16 inputs and, for the
    cosine path, the dense bf16 TFLOP/s of the projections."""
    torch = devc.torch
    cs = devc.cs
    res = {}
    for name in sorted(workloads.PROJECTED_CONFIGS):
        w = workloads.make_projected(name)

        def dev16(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(devc.dev)

        xq, xc, wq, wc = dev16(w.xq_bits), dev16(w.xc_bits), dev16(w.wq_bits), dev16(w.wc_bits)
        out = torch.empty(w.B, w.K, dtype=torch.float32, device=devc.dev)
        nbytes = cs.cs_projected_workspace_bytes(w.B, w.Hc, w.P, w.similarity)
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=devc.dev)

        def once():
            st = cs.cs_score_projected(xq, xc, wq, wc, w.B, w.K, w.Hq, w.Hc, w.P, w.similarity,
                                       float(w.scale), 1.0, out, ws, nbytes, devc.stream)
            assert st == 0, st

        for _ in range(3):
            once()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(devc.stream)
        for _ in range(iters):
            once()
        e1.record(devc.stream)
        torch.cuda.synchronize()
        us = 1e3 * e0.elapsed_time(e1) / iters
        gbs = w.algorithmic_bytes / us / 1e3
        row = {"B": w.B, "K": w.K, "Hq": w.Hq, "Hc": w.Hc, "P": w.P, "similarity": w.similarity,
               "dtype": "bf16 in, fp32 accumulate", "us_per_call": round(us, 2),
               "algorithmic_bytes": w.algorithmic_bytes, "GBps": round(gbs, 1),
               "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        if w.similarity == "cosine":
            flops = 2.0 * w.B * (w.K * w.Hc * w.P + w.Hq * w.P)
            tf = flops / us / 1e6
            row.update({"flops": flops, "TFLOPs": round(tf, 1),
                        "frac_of_bf16_mfma_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)})
        del xq, xc, wq, wc, out, ws
        if not one_question:
            res[name] = row
            log(f"projected {name}: {row}")
            continue
        # One question of the same heads: latency of the call (small batches
        # spread the dot path's candidate pass over the chip).
        w1 = workloads.make_projected(name, B=1)
        xq, xc, wq, wc = (dev16(w1.xq_bits), dev16(w1.xc_bits), dev16(w1.wq_bits),
                          dev16(w1.wc_bits))
        out = torch.empty(1, w1.K, dtype=torch.float32, device=devc.dev)
        nbytes = cs.cs_projected_workspace_bytes(1, w1.Hc, w1.P, w1.similarity)
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=devc.dev)

        def one():
            st = cs.cs_score_projected(xq, xc, wq, wc, 1, w1.K, w1.Hq, w1.Hc, w1.P,
                                       w1.similarity, float(w1.scale), 1.0, out, ws, nbytes,
                                       devc.stream)
            assert st == 0, st

        for _ in range(20):
            one()
        best = float("inf")
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(devc.stream)
            for _ in range(200):
                one()
            e1.record(devc.stream)
            torch.cuda.synchronize()
            best = min(best, 1e3 * e0.elapsed_time(e1) / 200)
        row["one_question_us_per_call"] = round(best, 2)
        res[name] = row
        log(f"projected {name}: {row}")
        del xq, xc, wq, wc, out, ws
    return res


def cpu_baseline(w, max_seconds=10.0):
    """The oracle as it stands, single-threaded, on the headline batch: as
    many whole passes as fit in about max_seconds (at least one)."""
    import oracle

    orc = oracle.load()
    reps, total = 0, 0.0
    while True:
        t0 = time.perf_counter()
        orc.score(w.Q, w.C, w.similarity, w.scale, w.temperature)
        total += time.perf_counter() - t0
        reps += 1
        if total * (reps + 1) / reps > max_seconds or reps >= 30:
            break
    per_call = total / reps
    return {"value": round(w.algorithmic_bytes / per_call / 1e9, 3), "unit": "GB/s",
            "us_per_call": round(per_call * 1e6, 1), "cores": 1, "kind": "oracle",
            "sample": f"all {w.B} questions of the headline batch, {reps} pass(es), "
                      f"single-threaded C float64 oracle",
            "cpu": cpu_model(), "host_cores_available": os.cpu_count()}


def cpu_baseline_threaded(w, threads, max_seconds=10.0):
    """The same oracle over all host threads: questions are independent, so
    each thread runs the unchanged single-threaded oracle on its own
    contiguous range of questions (ctypes releases the GIL during the call)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    orc = oracle.load()
    bounds = np.linspace(0, w.B, threads + 1).astype(int)
    ranges = [(int(a), int(b)) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]

    def work(r):
        a, b = r
        orc.score(w.Q[a:b], w.C[a:b], w.similarity, w.scale, w.temperature)

    reps, total = 0, 0.0
    with ThreadPoolExecutor(max_workers=len(ranges)) as pool:
        while True:
            t0 = time.perf_counter()
            list(pool.map(work, ranges))
            total += time.perf_counter() - t0
            reps += 1
            if total * (reps + 1) / reps > max_seconds or reps >= 30:
                break
    per_call = total / reps
    return {"value": round(w.algorithmic_bytes / per_call / 1e9, 3), "unit": "GB/s",
            "us_per_call": round(per_call * 1e6, 1), "cores": len(ranges), "kind": "oracle",
            "sample": f"all {w.B} questions of the headline batch split over {len(ranges)} "
                      f"threads, {reps} pass(es)"}


def cpu_model() -> str:
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--replays", type=int, default=2000, help="graph replays per latency figure")
    ap.add_argument("--no-latency", action="store_true", help="skip the small-shape latencies")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-ab", action="store_true", help="skip the fused vs unfused table")
    ap.add_argument("--no-ragged", action="store_true", help="skip the ragged batch")
    ap.add_argument("--projected-latency", action="store_true",
                    help="time the one-question projected calls even with --no-latency")
    ap.add_argument("--no-projected", action="store_true",
                    help="skip the projection + scoring workloads")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="also run one plain copy of MIB MiB (counter calibration)")
    ap.add_argument("--phase-clocks", action="store_true",
                    help="only the per-phase clocks of the split calls, of the Kev "
                         "projection call and of the CLM cosine ring kernel, from the measurement "
                         "build candidate_scoring_amd/libcs_phase.so (python -m "
                         "candidate_scoring_amd.build --phase-clocks)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(questions would shard across GPUs with no exchange, see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    if args.phase_clocks:
        import candidate_scoring_amd as cs_pkg

        # First load in this process, and global: the native timing loop of
        # libcs_bench.so then binds its calls to this build's entry points
        # rather than to libcs.so, which it names as a dependency.
        ctypes.CDLL(str(cs_pkg.PKG / "libcs_phase.so"), mode=ctypes.RTLD_GLOBAL)
        lib = cs_pkg.load(cs_pkg.PKG / "libcs_phase.so")
        for fn in (lib.cs_phase_clocks_read, lib.cs_projected_phase_clocks_read,
                   lib.cs_ring_phase_clocks_read):
            fn.restype = ctypes.c_int
            fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
        devc = Device()
        print(json.dumps({"phase_clocks": phase_clock_section(devc),
                          "projected_phase_clocks": projected_phase_section(devc),
                          "clm_ring_phase_clocks": ring_phase_section(devc),
                          "library": "libcs_phase.so (measurement build)"}), flush=True)
        return

    devc = Device()
    torch = devc.torch
    w = workloads.make(workloads.HEADLINE)
    log(f"headline: {w.name} B={w.B} K={w.K} D={w.D} bytes={w.algorithmic_bytes}")
    q, c, out = devc.upload(w)
    call, _ws = devc.call(w, q, c, out)

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.empty(n // 4, dtype=torch.float32, device=devc.dev)
        dst = torch.empty_like(src)
        st = devc.bench.csb_copy(src.data_ptr(), dst.data_ptr(), n, devc.stream.cuda_stream)
        assert st == 0
        torch.cuda.synchronize()
        log(f"calibration copy of {n} bytes done")
        del src, dst

    if args.warmup:
        devc.time_calls(call, args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_ms = devc.time_calls(call, args.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch_s = ev_ms / 1e3 / args.steps
    gbs = w.algorithmic_bytes / per_launch_s / 1e9
    log(f"headline: {1e6 * per_launch_s:.1f} us/call, {gbs:.1f} GB/s "
        f"(wall {wall:.3f} s for {args.steps} steps)")

    # spot parity of the timed launch configuration (first and last question)
    import oracle

    orc = oracle.load()
    got = out.cpu().numpy()
    for b in (0, w.B - 1):
        want = orc.score(w.Q[b], w.C[b], w.similarity, w.scale, w.temperature)
        err = float(np.max(np.abs(got[b].astype(np.float64) - want)))
        if not err <= 1e-4:
            raise SystemExit(f"parity failure on question {b}: {err}")

    ab = None if args.no_ab else ab_section(devc, 2000, headline=(w, q, c, out))
    del q, c, out

    traffic = committed_traffic()
    result = {
        "metric": "µs/call + achieved HBM GB/s, fused score+softmax, K=255 D=512 and D=2560",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "us_per_call": round(1e6 * per_launch_s, 2),
        "questions_per_s": round(w.B / per_launch_s, 1),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * per_launch_s, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic: seeded N(0,1) fp32 queries and candidates",
        "config": {"workload": "batch of 1024 questions, dot similarity (Kev), K=255, D=2560, "
                               "scale 1/16, T=1, fp32, one launch",
                   "global_batch": w.B, "K": w.K, "D": w.D, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "occupancy_percent": committed_occupancy(),
                     "kernel": devc.cs.cs_plan_kernel(w.B, w.K, w.D, w.similarity, True)[1],
                     "algorithmic_bytes_per_launch": w.algorithmic_bytes},
    }
    if not args.no_latency:
        result["latency"] = latency_section(devc, args.replays)
        result["cold_latency"] = cold_section(devc, 2000)
    if ab is not None:
        result["fused_vs_unfused"] = ab
    if not args.no_ragged:
        result["ragged"] = ragged_section(devc)
    if not args.no_projected:
        result["projected"] = projected_section(
            devc, one_question=args.projected_latency or not args.no_latency)
    if not args.no_cpu:
        log("cpu baseline: oracle on the headline batch")
        result["cpu_baseline"] = cpu_baseline(w)
        # at most 16 host threads: a process sharing its machine may be
        # allotted fewer cores than os.cpu_count() reports
        threads = max(1, min(16, os.cpu_count() or 1))
        result["cpu_baseline"]["threaded"] = cpu_baseline_threaded(w, threads)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
