"""Python binding of the fused candidate-scoring library (libcs.so).

The functions named ``cs_*`` mirror the C ABI in include/candidate_scoring.h
one to one and only marshal arguments: every step of the computation runs in
the HIP kernels. Pointer arguments accept a torch tensor on a HIP device, a
raw integer device address, or None (NULL). ``stream`` accepts None (torch's
current stream), a ``torch.cuda.Stream`` or a raw ``hipStream_t`` integer.

``score``, ``score_ragged`` and ``score_projected`` are convenience wrappers
that allocate the output (and a cached workspace) with torch and raise on a
non-OK status.

There is no fallback: if the library is not built, ``load`` raises.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

PKG = Path(__file__).resolve().parent
LIBRARY = PKG / "libcs.so"
BENCH_LIBRARY = PKG / "libcs_bench.so"

CS_ABI_VERSION = 1
CS_MAX_K = 255
CS_SIM_DOT = 0
CS_SIM_COSINE = 1

CS_OK = 0
CS_ERR_NULL_POINTER = -1
CS_ERR_K_RANGE = -2
CS_ERR_D_RANGE = -3
CS_ERR_SCALE = -4
CS_ERR_TEMPERATURE = -5
CS_ERR_BATCH = -6
CS_ERR_SIMILARITY = -7
CS_ERR_WORKSPACE = -8
CS_ERR_LAUNCH = -9
CS_ERR_HOST_POINTER = -10
CS_ERR_UNSUPPORTED = -11
CS_NOALLOC_SCRATCH_BYTES = 64 * 1024

_lib = None
_bench = None


class ScoringError(ValueError):
    def __init__(self, status: int):
        super().__init__(f"{status}: {cs_status_string(status)}")
        self.status = status


def load(path: Path | str = LIBRARY):
    """Load libcs.so (built by ``python -m candidate_scoring_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    path = Path(path)
    if not path.exists():
        raise RuntimeError(f"HIP library {path} is not built; run "
                           "`python -m candidate_scoring_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(str(path))
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    sigs = {
        "cs_abi_version": (i32, []),
        "cs_status_string": (ctypes.c_char_p, [i32]),
        "cs_last_hip_error": (i32, []),
        "cs_workspace_bytes": (sz, [i32, i32, i32, i32]),
        "cs_workspace_bytes_for_groups": (sz, [i32, i32]),
        "cs_workspace_init": (i32, [vp, sz, vp]),
        "cs_plan_groups": (i32, [i32, i32, i32, i32, i32]),
        "cs_plan_launch": (i32, [i32, i32, i32, i32, i32, i32, ctypes.POINTER(ctypes.c_uint),
                                 ctypes.POINTER(ctypes.c_uint), ctypes.POINTER(ctypes.c_int)]),
        "cs_plan_kernel": (i32, [i32, i32, i32, i32, i32, i32, ctypes.c_char_p, sz]),
        "cs_score_candidates": (i32, [vp, vp, i32, i32, i32, f32, f32, vp, vp, sz, vp]),
        "cs_score_candidates_batch": (i32, [vp, vp, i32, i32, i32, i32, f32, f32, vp, vp, sz, vp]),
        "cs_score_candidates_batch_groups": (
            i32, [vp, vp, i32, i32, i32, i32, f32, f32, vp, vp, sz, i32, vp]),
        "cs_score_candidates_batch_noalloc": (i32, [vp, vp, i32, i32, i32, i32, f32, f32, vp,
                                                    vp]),
        "cs_score_candidates_unfused": (i32, [vp, vp, i32, i32, i32, i32, f32, f32, vp, vp, vp]),
        "cs_projected_workspace_bytes": (sz, [i32, i32, i32, i32]),
        "cs_score_projected": (i32, [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, f32, vp,
                                     vp, sz, vp]),
        "cs_score_candidates_ragged": (i32, [vp, vp, vp, i32, ctypes.c_int64, i32, i32, f32, f32,
                                             vp, vp, vp, sz, vp]),
        "cs_ragged_workspace_bytes": (sz, [i32, ctypes.c_int64, i32, i32]),
        "cs_plan_ragged": (i32, [i32, ctypes.c_int64, i32, i32, i32, ctypes.POINTER(ctypes.c_int),
                                 ctypes.POINTER(ctypes.c_int)]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


class CsbCall(ctypes.Structure):
    _fields_ = [("Q", ctypes.c_void_p), ("C", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("B", ctypes.c_int), ("K", ctypes.c_int), ("D", ctypes.c_int),
                ("similarity", ctypes.c_int), ("scale", ctypes.c_float),
                ("temperature", ctypes.c_float), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("groups", ctypes.c_int),
                ("row_norms", ctypes.c_void_p)]


def load_bench(path: Path | str = BENCH_LIBRARY):
    """Load the native timing helpers (libcs_bench.so)."""
    global _bench
    if _bench is not None:
        return _bench
    load()
    path = Path(path)
    if not path.exists():
        raise RuntimeError(f"{path} is not built; run `python -m candidate_scoring_amd.build`")
    lib = ctypes.CDLL(str(path))
    vp, i32, u32, f32p = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.POINTER(ctypes.c_float)
    szp = ctypes.POINTER(ctypes.c_size_t)
    cp = ctypes.POINTER(CsbCall)
    sigs = {
        "csb_time_calls": [cp, i32, vp, f32p],
        "csb_time_calls_rotating": [cp, i32, ctypes.c_size_t, ctypes.c_size_t, ctypes.c_size_t,
                                    i32, vp, f32p],
        "csb_graph_nodes": [cp, szp],
        "csb_time_graph": [cp, i32, i32, i32, f32p, szp],
        "csb_graph_replay": [cp, i32, i32],
        "csb_time_empty": [u32, u32, i32, i32, i32, vp, f32p],
        "csb_copy": [vp, vp, ctypes.c_size_t, vp],
        "csb_read": [vp, ctypes.c_size_t, u32, u32, vp, vp],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = i32, args
    _bench = lib
    return lib


def _ptr(x):
    """Device address of a tensor / int / None, refusing host tensors."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        if not x.is_cuda:
            raise ValueError("device memory required: got a host tensor")
        return x.data_ptr()
    raise TypeError(f"cannot pass {type(x).__name__} as a device pointer")


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _sim(similarity) -> int:
    if isinstance(similarity, str):
        return {"dot": CS_SIM_DOT, "cosine": CS_SIM_COSINE}[similarity]
    return int(similarity)


# ----------------------------------------------------------------------------
# One-to-one mirrors of the C ABI.

def cs_abi_version() -> int:
    return load().cs_abi_version()


def cs_status_string(status: int) -> str:
    return load().cs_status_string(int(status)).decode()


def cs_last_hip_error() -> int:
    return load().cs_last_hip_error()


def cs_workspace_bytes(B: int, K: int, D: int, similarity) -> int:
    return load().cs_workspace_bytes(B, K, D, _sim(similarity))


def cs_workspace_bytes_for_groups(B: int, groups: int) -> int:
    return load().cs_workspace_bytes_for_groups(B, groups)


def cs_workspace_init(workspace, nbytes: int, stream=None) -> int:
    return load().cs_workspace_init(_ptr(workspace), nbytes, _stream(stream))


def cs_plan_groups(B: int, K: int, D: int, similarity, has_workspace: bool) -> int:
    return load().cs_plan_groups(B, K, D, _sim(similarity), int(bool(has_workspace)))


def cs_plan_launch(B: int, K: int, D: int, similarity, has_workspace: bool,
                   aligned16: bool = True):
    """(status, grid, block, groups) of the launch the batch call would make."""
    grid, block, groups = ctypes.c_uint(), ctypes.c_uint(), ctypes.c_int()
    st = load().cs_plan_launch(B, K, D, _sim(similarity), int(bool(has_workspace)),
                               int(bool(aligned16)), ctypes.byref(grid), ctypes.byref(block),
                               ctypes.byref(groups))
    return st, grid.value, block.value, groups.value


def cs_plan_kernel(B: int, K: int, D: int, similarity, has_workspace: bool,
                   aligned16: bool = True):
    """(status, name) of the kernel instantiation the batch call would launch."""
    buf = ctypes.create_string_buffer(256)
    st = load().cs_plan_kernel(B, K, D, _sim(similarity), int(bool(has_workspace)),
                               int(bool(aligned16)), buf, len(buf))
    return st, buf.value.decode()


def cs_score_candidates(query, candidates, K: int, D: int, similarity, scale: float,
                        temperature: float, out, workspace=None, workspace_bytes: int = 0,
                        stream=None) -> int:
    return load().cs_score_candidates(_ptr(query), _ptr(candidates), K, D, _sim(similarity),
                                      scale, temperature, _ptr(out), _ptr(workspace),
                                      workspace_bytes, _stream(stream))


def cs_score_candidates_batch(queries, candidates, B: int, K: int, D: int, similarity,
                              scale: float, temperature: float, out, workspace=None,
                              workspace_bytes: int = 0, stream=None) -> int:
    return load().cs_score_candidates_batch(_ptr(queries), _ptr(candidates), B, K, D,
                                            _sim(similarity), scale, temperature, _ptr(out),
                                            _ptr(workspace), workspace_bytes, _stream(stream))


def cs_score_candidates_batch_groups(queries, candidates, B: int, K: int, D: int, similarity,
                                     scale: float, temperature: float, out, workspace,
                                     workspace_bytes: int, groups: int, stream=None) -> int:
    return load().cs_score_candidates_batch_groups(
        _ptr(queries), _ptr(candidates), B, K, D, _sim(similarity), scale, temperature,
        _ptr(out), _ptr(workspace), workspace_bytes, groups, _stream(stream))


def cs_score_candidates_batch_noalloc(queries, candidates, B: int, K: int, D: int, similarity,
                                      scale: float, temperature: float, out,
                                      stream=None) -> int:
    return load().cs_score_candidates_batch_noalloc(_ptr(queries), _ptr(candidates), B, K, D,
                                                    _sim(similarity), scale, temperature,
                                                    _ptr(out), _stream(stream))


def cs_score_candidates_unfused(queries, candidates, B: int, K: int, D: int, similarity,
                                scale: float, temperature: float, out, row_norms,
                                stream=None) -> int:
    return load().cs_score_candidates_unfused(_ptr(queries), _ptr(candidates), B, K, D,
                                              _sim(similarity), scale, temperature, _ptr(out),
                                              _ptr(row_norms), _stream(stream))


def cs_score_candidates_ragged(queries, candidates, offsets, B: int, total_rows: int, D: int,
                               similarity, scale: float, temperature: float, out, status=None,
                               workspace=None, workspace_bytes: int = 0, stream=None) -> int:
    return load().cs_score_candidates_ragged(_ptr(queries), _ptr(candidates), _ptr(offsets), B,
                                             total_rows, D, _sim(similarity), scale, temperature,
                                             _ptr(out), _ptr(status), _ptr(workspace),
                                             workspace_bytes, _stream(stream))


def cs_ragged_workspace_bytes(B: int, total_rows: int, D: int, similarity) -> int:
    return load().cs_ragged_workspace_bytes(B, total_rows, D, _sim(similarity))


def cs_plan_ragged(B: int, total_rows: int, D: int, similarity, has_workspace: bool):
    """(status, rows_per_slice, max_slices) of the ragged call's plan."""
    rpg, slices = ctypes.c_int(), ctypes.c_int()
    st = load().cs_plan_ragged(B, total_rows, D, _sim(similarity), int(bool(has_workspace)),
                               ctypes.byref(rpg), ctypes.byref(slices))
    return st, rpg.value, slices.value


def cs_projected_workspace_bytes(B: int, Hc: int, P: int, similarity) -> int:
    return load().cs_projected_workspace_bytes(B, Hc, P, _sim(similarity))


def cs_score_projected(xq, xc, wq, wc, B: int, K: int, Hq: int, Hc: int, P: int, similarity,
                       scale: float, temperature: float, out, workspace, workspace_bytes: int,
                       stream=None) -> int:
    """bf16 tensors (torch.bfloat16 or raw uint16 device buffers)."""
    return load().cs_score_projected(_ptr(xq), _ptr(xc), _ptr(wq), _ptr(wc), B, K, Hq, Hc, P,
                                     _sim(similarity), scale, temperature, _ptr(out),
                                     _ptr(workspace), workspace_bytes, _stream(stream))


# ----------------------------------------------------------------------------
# Convenience wrappers.

_workspaces: dict = {}


def workspace(nbytes: int, device=None, stream=None, kind: str = "split"):
    """A zeroed workspace of at least ``nbytes`` cached per (device, stream,
    kind). Calls that may overlap must not share one, hence the per-stream
    key; the split path's workspace must stay zeroed between calls while the
    projection's is scratch, hence the kind."""
    import torch

    device = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    key = (str(device), _stream(stream), kind)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 4096), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def score(query, candidates, similarity="cosine", scale=1.0, temperature=1.0, out=None,
          use_workspace=True, groups=None, stream=None):
    """Probabilities for one question (query [D], candidates [K, D]) or a
    batch (queries [B, D], candidates [B, K, D]); fp32 contiguous device
    tensors. Returns out ([K] or [B, K])."""
    import torch

    single = candidates.dim() == 2
    if single:
        B, (K, D) = 1, candidates.shape
    else:
        B, K, D = candidates.shape
    if out is None:
        out = torch.empty((K,) if single else (B, K), dtype=torch.float32,
                          device=candidates.device)
    for t in (query, candidates, out):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("fp32 contiguous tensors required")
    sim = _sim(similarity)
    ws, nbytes = None, 0
    if groups is not None:
        nbytes = cs_workspace_bytes_for_groups(B, groups)
    elif use_workspace:
        nbytes = cs_workspace_bytes(B, K, D, sim)
    if nbytes > 0:
        ws = workspace(nbytes, candidates.device, stream)
        nbytes = ws.numel()
    if groups is not None:
        st = cs_score_candidates_batch_groups(query, candidates, B, K, D, sim, scale,
                                              temperature, out, ws, nbytes, groups, stream)
    elif single:
        st = cs_score_candidates(query, candidates, K, D, sim, scale, temperature, out, ws,
                                 nbytes, stream)
    else:
        st = cs_score_candidates_batch(query, candidates, B, K, D, sim, scale, temperature,
                                       out, ws, nbytes, stream)
    if st != CS_OK:
        raise ScoringError(st)
    return out


def score_ragged(queries, candidates, offsets, similarity="cosine", scale=1.0,
                 temperature=1.0, out=None, status=None, use_workspace=True, stream=None):
    """Probabilities for a ragged batch: queries [B, D], candidates
    [total_rows, D] packed by question, offsets int64 [B + 1] on the device
    (question b owns rows offsets[b] .. offsets[b+1]-1, 1 to 255 of them).
    Returns out [total_rows]. A question with bad offsets is skipped and, if
    ``status`` (an int32 device tensor) is given, flagged there. A small
    batch spreads its questions over the chip through the cached zeroed
    workspace that score() uses (use_workspace=False: one workgroup per
    question)."""
    import torch

    B, D = queries.shape
    total_rows = candidates.shape[0]
    if candidates.dim() != 2 or candidates.shape[1] != D:
        raise ValueError("candidates must be [total_rows, D]")
    if offsets.dtype != torch.int64 or offsets.numel() != B + 1 or not offsets.is_contiguous():
        raise ValueError("offsets must be a contiguous int64 tensor of B + 1 entries")
    if out is None:
        out = torch.empty(total_rows, dtype=torch.float32, device=candidates.device)
    for t in (queries, candidates, out):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("fp32 contiguous tensors required")
    ws, nbytes = None, 0
    if use_workspace:
        nbytes = cs_ragged_workspace_bytes(B, total_rows, D, similarity)
        if nbytes > 0:
            ws = workspace(nbytes, candidates.device, stream)
            nbytes = ws.numel()
    st = cs_score_candidates_ragged(queries, candidates, offsets, B, total_rows, D, similarity,
                                    scale, temperature, out, status, ws, nbytes, stream)
    if st != CS_OK:
        raise ScoringError(st)
    return out


def score_projected(xq, xc, wq, wc, similarity="cosine", scale=1.0, temperature=1.0, out=None,
                    stream=None):
    """Probabilities with the heads applied: hidden states xq [B, Hq] and
    xc [B, K, Hc], heads wq [P, Hq] and wc [P, Hc], all bfloat16 contiguous
    device tensors; q' = wq xq and c'_k = wc xc_k are scored as by score().
    Returns out [B, K] (fp32)."""
    import torch

    B, Hq = xq.shape
    B2, K, Hc = xc.shape
    P = wq.shape[0]
    if B2 != B or tuple(wq.shape) != (P, Hq) or tuple(wc.shape) != (P, Hc):
        raise ValueError("shapes must be xq [B, Hq], xc [B, K, Hc], wq [P, Hq], wc [P, Hc]")
    for t in (xq, xc, wq, wc):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError("bfloat16 contiguous tensors required")
    if out is None:
        out = torch.empty((B, K), dtype=torch.float32, device=xc.device)
    nbytes = cs_projected_workspace_bytes(B, Hc, P, similarity)
    ws = workspace(nbytes, xc.device, stream, kind="projected")
    st = cs_score_projected(xq, xc, wq, wc, B, K, Hq, Hc, P, similarity, scale, temperature, out,
                            ws, ws.numel(), stream)
    if st != CS_OK:
        raise ScoringError(st)
    return out
