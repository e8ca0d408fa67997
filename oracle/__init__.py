"""Double-precision CPU oracle for fused candidate scoring.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
bench's CPU-baseline leg may import this module; the product path never does.
It wraps ``cs_oracle.c`` (plain C, float64, sequential loops) through ctypes
and shares no code with the HIP library.

Source of what is computed: the pull request "cuda: add a fused
candidate-scoring kernel for CLM and Kev" -- intro (model/similarity table),
"What is fused, precisely", and "Verified on hardware" (rejected arguments).
"""
from __future__ import annotations

import ctypes
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SOURCE = HERE / "cs_oracle.c"
LIBRARY = HERE / "libcs_oracle.so"

# Status codes as the oracle defines them (cs_oracle.h).
OK = 0
ERR_NULL_POINTER = -1
ERR_K_RANGE = -2
ERR_D_RANGE = -3
ERR_SCALE = -4
ERR_TEMPERATURE = -5
ERR_BATCH = -6
ERR_SIMILARITY = -7

SIM_DOT = 0
SIM_COSINE = 1
MAX_K = 255

CFLAGS = ("-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-Wall", "-Wextra")


class OracleError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"oracle rejected the arguments with status {code}")
        self.code = code


def build(source: Path | str = SOURCE, output: Path | str = LIBRARY, extra_flags=()) -> Path:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    source, output = Path(source), Path(output)
    cmd = ["gcc", *CFLAGS, *extra_flags, "-I", str(HERE), str(source), "-lm", "-o", str(output)]
    subprocess.run(cmd, check=True)
    return output


def _sim_code(similarity) -> int:
    if isinstance(similarity, str):
        return {"dot": SIM_DOT, "cosine": SIM_COSINE}[similarity]
    return int(similarity)


def _f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """ctypes wrapper around one build of the oracle library."""

    def __init__(self, library: Path | str = LIBRARY):
        self.path = Path(library)
        lib = ctypes.CDLL(str(self.path))
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        lib.cso_validate.argtypes = [i32, i32, i32, i64, i64, i64, i32, f32, f32]
        lib.cso_logits.argtypes = [vp, vp, i32, i32, i32, i32, f32, f32, vp]
        lib.cso_score.argtypes = [vp, vp, i32, i32, i32, i32, f32, f32, vp]
        lib.cso_score_ragged.argtypes = [vp, vp, vp, i32, i32, i32, f32, f32, vp]
        lib.cso_score_projected.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, f32, vp]
        for name in ("cso_validate", "cso_logits", "cso_score", "cso_score_ragged", "cso_score_projected"):
            getattr(lib, name).restype = i32
        self.lib = lib

    def validate(self, *, query=True, candidates=True, out=True, B=1, K=1, D=1,
                 similarity=SIM_DOT, scale=1.0, temperature=1.0) -> int:
        return self.lib.cso_validate(int(bool(query)), int(bool(candidates)), int(bool(out)),
                                     B, K, D, _sim_code(similarity), scale, temperature)

    @staticmethod
    def _shapes(Q, C):
        if C.ndim == 2:  # single question: q[D], C[K, D]
            return 1, C.shape[0], C.shape[1]
        return C.shape[0], C.shape[1], C.shape[2]

    def _run(self, fn, Q, C, similarity, scale, temperature):
        Q, C = _f32(Q), _f32(C)
        B, K, D = self._shapes(Q, C)
        if Q.size != B * D:
            raise ValueError("query shape does not match candidates")
        out = np.zeros(B * K, dtype=np.float64)
        st = fn(_ptr(Q), _ptr(C), B, K, D, _sim_code(similarity),
                float(np.float32(scale)), float(np.float32(temperature)), _ptr(out))
        if st != OK:
            raise OracleError(st)
        return out.reshape((K,) if C.ndim == 2 else (B, K))

    def logits(self, Q, C, similarity, scale, temperature=1.0) -> np.ndarray:
        """Scaled similarities z = scale * s / T (double)."""
        return self._run(self.lib.cso_logits, Q, C, similarity, scale, temperature)

    def score(self, Q, C, similarity, scale, temperature=1.0) -> np.ndarray:
        """Softmax over each question's candidates (double)."""
        return self._run(self.lib.cso_score, Q, C, similarity, scale, temperature)

    def score_raw(self, Q, C, B, K, D, similarity, scale, temperature, out_present=True):
        """Call with explicit sizes (may be invalid); returns (status, out)."""
        Qa = None if Q is None else _f32(Q)
        Ca = None if C is None else _f32(C)
        n = max(int(B), 0) * max(int(K), 0)
        out = np.full(max(n, 1), -7.0, dtype=np.float64)
        st = self.lib.cso_score(_ptr(Qa), _ptr(Ca), int(B), int(K), int(D), _sim_code(similarity),
                                float(np.float32(scale)), float(np.float32(temperature)),
                                _ptr(out) if out_present else None)
        return st, out

    def score_ragged(self, Q, C, offsets, similarity, scale, temperature=1.0) -> np.ndarray:
        Q, C = _f32(Q), _f32(C)
        offsets = np.ascontiguousarray(offsets, dtype=np.int64)
        B = offsets.size - 1
        D = Q.shape[-1]
        out = np.zeros(max(int(offsets[-1]), 1), dtype=np.float64)
        st = self.lib.cso_score_ragged(_ptr(Q), _ptr(C), _ptr(offsets), B, D, _sim_code(similarity),
                                       float(np.float32(scale)), float(np.float32(temperature)),
                                       _ptr(out))
        if st != OK:
            raise OracleError(st)
        return out[: int(offsets[-1])]

    def score_projected(self, Xq, Wq, Xc, Wc, similarity, scale, temperature=1.0) -> np.ndarray:
        Xq, Wq, Xc, Wc = _f32(Xq), _f32(Wq), _f32(Xc), _f32(Wc)
        B, K, Dc = Xc.shape
        Dq = Xq.shape[-1]
        P = Wq.shape[0]
        out = np.zeros(B * K, dtype=np.float64)
        st = self.lib.cso_score_projected(_ptr(Xq), _ptr(Wq), _ptr(Xc), _ptr(Wc), B, K, Dq, Dc, P,
                                          _sim_code(similarity), float(np.float32(scale)),
                                          float(np.float32(temperature)), _ptr(out))
        if st != OK:
            raise OracleError(st)
        return out.reshape(B, K)


_DEFAULT: Oracle | None = None


def load() -> Oracle:
    """The oracle built from cs_oracle.c; built first if no library exists."""
    global _DEFAULT
    if _DEFAULT is None:
        if not LIBRARY.exists() or LIBRARY.stat().st_mtime < SOURCE.stat().st_mtime:
            build()
        _DEFAULT = Oracle(LIBRARY)
    return _DEFAULT


__all__ = ["Oracle", "OracleError", "build", "load", "MAX_K", "SIM_DOT", "SIM_COSINE"]
