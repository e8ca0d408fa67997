"""Builds the HIP libraries in-tree for gfx950 with hipcc.

    python -m candidate_scoring_amd.build [--phase-clocks]

produces ``candidate_scoring_amd/libcs.so`` (the C ABI of
include/candidate_scoring.h) and ``candidate_scoring_amd/libcs_bench.so``
(native timing helpers for bench.py). With ``--phase-clocks`` it builds
only ``libcs_phase.so``, a measurement copy of the library whose scoring
kernels record per-phase device clocks (``bench.py --phase-clocks``).
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIBRARY = PKG / "libcs.so"
BENCH_LIBRARY = PKG / "libcs_bench.so"
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        "-Wall",
        # keep the compiler from emitting packed fp32 math (v_pk_*_f32)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
    ]


RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"


def _run(cmd: list[str], verbose: bool) -> str:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    noise = "is not a recognized feature for this target"
    lines = [l for l in res.stderr.splitlines() if noise not in l]
    err = "\n".join(l for l in lines if RESOURCE_REMARKS not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build failed ({res.returncode}):\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return "\n".join(lines)


def spilling_kernels(remarks: str) -> list[tuple[str, int]]:
    """Kernels whose resource-usage remarks report scratch (spilled) memory.

    Every kernel here is sized to keep its working set in registers: the
    hot loops hold 16-byte loads in flight and the matrix-core tiles hold
    their accumulators, and a spill would put scratch traffic into each
    iteration. The build therefore fails when any kernel uses scratch, so
    that a change which pushes one over its register budget is noticed.
    """
    out, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name is not None:
            if int(m.group(1)) > 0:
                out.append((name, int(m.group(1))))
            name = None
    return out


def build(verbose: bool = False) -> list[Path]:
    cc = hipcc()
    tmp = LIBRARY.with_suffix(".so.tmp")
    remarks = _run([cc, *common_flags(), RESOURCE_REMARKS, "-fno-caret-diagnostics", "-o", str(tmp),
                    str(CSRC / "cs_kernels.hip"), str(CSRC / "cs_project.hip"),
                    str(CSRC / "cs_api.cpp")], verbose)
    if "ScratchSize" not in remarks:
        raise RuntimeError("build: the compiler printed no kernel resource usage to check")
    spills = spilling_kernels(remarks)
    if spills:
        tmp.unlink(missing_ok=True)
        raise RuntimeError("build: kernels use scratch memory (spills), which this library "
                           "does not allow: " + ", ".join(f"{n} ({b} B/lane)"
                                                                     for n, b in spills))
    tmp.replace(LIBRARY)
    tmpb = BENCH_LIBRARY.with_suffix(".so.tmp")
    _run([cc, *common_flags(), "-o", str(tmpb), str(CSRC / "cs_bench.hip"),
          f"-L{PKG}", "-lcs", "-Wl,-rpath,$ORIGIN"], verbose)
    tmpb.replace(BENCH_LIBRARY)
    return [LIBRARY, BENCH_LIBRARY]


PHASE_LIBRARY = PKG / "libcs_phase.so"


def build_phase_clocks(verbose: bool = False) -> Path:
    """The measurement build: the same library with CS_PHASE_CLOCKS defined,
    whose scoring kernels stamp the device clock at fixed phases (read with
    cs_phase_clocks_read). Never loaded by the product path; built only on
    request, for ``bench.py --phase-clocks``."""
    cc = hipcc()
    tmp = PHASE_LIBRARY.with_suffix(".so.tmp")
    _run([cc, *common_flags(), "-DCS_PHASE_CLOCKS", "-o", str(tmp),
          str(CSRC / "cs_kernels.hip"), str(CSRC / "cs_project.hip"), str(CSRC / "cs_api.cpp")],
         verbose)
    tmp.replace(PHASE_LIBRARY)
    return PHASE_LIBRARY


if __name__ == "__main__":
    if "--phase-clocks" in sys.argv[1:]:
        print("built", build_phase_clocks(verbose=True))
    else:
        for p in build(verbose=True):
            print("built", p)
