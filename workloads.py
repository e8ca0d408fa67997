"""Seeded synthetic inputs for fused candidate scoring.

This module only draws and arranges input data; it holds none of the scoring
arithmetic, so both the oracle side and the HIP side can take their inputs
from it without sharing any of the method's code.

Shapes follow the pull request "cuda: add a fused candidate-scoring kernel
for CLM and Kev": the results table in "What it is worth" (cosine K=5/64/255
at D=512, a batch of 8, and Kev's dot at K=255, D=2560), the degenerate cases
in "Verified on hardware" (single candidate, identical candidates, a zero
candidate, logits that overflow a naive exp), plus one bandwidth-bound batch
of 1024 Kev-shaped questions. Values are N(0, 1) fp32 from
``numpy.random.default_rng(seed)``, query block first, then candidates.
No public dataset is involved: these synthetic arrays are the whole workload.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# CLM passes exp(logit_scale) with logit_scale = log(1/0.07); as fp32 that is
# 14.285714149475098. Kev's scale is 1/sqrt(256) = 0.0625 exactly.
SCALE_COSINE = np.float32(math.exp(math.log(1.0 / 0.07)))
SCALE_DOT = np.float32(1.0 / math.sqrt(256.0))
# The overflow case multiplies the cosine logits by 1e3.
SCALE_COSINE_OVERFLOW = np.float32(float(SCALE_COSINE) * 1e3)


@dataclass
class Workload:
    name: str
    call: str            # "single" (one q[D], C[K,D]) or "batch"
    similarity: str      # "cosine" or "dot"
    scale: np.float32
    temperature: np.float32
    Q: np.ndarray        # [B, D] fp32
    C: np.ndarray        # [B, K, D] fp32
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return self.C.shape[0]

    @property
    def K(self) -> int:
        return self.C.shape[1]

    @property
    def D(self) -> int:
        return self.C.shape[2]

    @property
    def algorithmic_bytes(self) -> int:
        """fp32 bytes that must cross HBM once: C and Q read, P written."""
        return 4 * (self.B * self.K * self.D + self.B * self.D + self.B * self.K)


def normal_inputs(seed: int, B: int, K: int, D: int):
    """Q [B,D] then C [B,K,D], fp32 N(0,1) from one seeded generator."""
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((B, D), dtype=np.float32)
    C = rng.standard_normal((B, K, D), dtype=np.float32)
    return Q, C


# name -> (call, B, K, D, similarity, scale, seed, description)
BASE_CONFIGS = {
    "clm_cos_5x512": ("single", 1, 5, 512, "cosine", SCALE_COSINE, 1,
                      "1 question, cosine, K=5, D=512"),
    "clm_cos_64x512": ("single", 1, 64, 512, "cosine", SCALE_COSINE, 6,
                       "1 question, cosine, K=64, D=512"),
    "clm_cos_255x512": ("single", 1, 255, 512, "cosine", SCALE_COSINE, 2,
                        "1 question, cosine, K=255, D=512"),
    "clm_cos_batch8_255x512": ("batch", 8, 255, 512, "cosine", SCALE_COSINE, 3,
                               "8 questions, cosine, K=255, D=512; question 7 stored x1e3"),
    "kev_dot_255x2560": ("single", 1, 255, 2560, "dot", SCALE_DOT, 4,
                         "1 question, dot, K=255, D=2560"),
    "kev_dot_batch1024_255x2560": ("batch", 1024, 255, 2560, "dot", SCALE_DOT, 5,
                                   "1024 questions, dot, K=255, D=2560 (2.67 GB of candidates)"),
}

# The bandwidth-bound shape that the bench times.
HEADLINE = "kev_dot_batch1024_255x2560"

# The shapes of the page's fused-vs-unfused table ("What it is worth"), plus
# the bandwidth-bound batch.
AB_SHAPES = ["clm_cos_5x512", "clm_cos_64x512", "clm_cos_255x512", "clm_cos_batch8_255x512",
             "kev_dot_255x2560", "kev_dot_batch1024_255x2560"]


def make(name: str, B: int | None = None) -> Workload:
    """Build one named workload. ``B`` (batch configs only) keeps the recipe
    but draws fewer questions, for quick runs; the first questions of a
    reduced draw are NOT the first questions of the full draw."""
    variants = {
        "clm_cos_1x512_single_candidate": "clm_cos_255x512",
        "clm_cos_255x512_identical": "clm_cos_255x512",
        "clm_cos_255x512_zero_row": "clm_cos_255x512",
        "clm_cos_batch8_255x512_overflow": "clm_cos_batch8_255x512",
    }
    base = variants.get(name, name)
    call, B0, K, D, sim, scale, seed, desc = BASE_CONFIGS[base]
    if B is not None:
        if call != "batch":
            raise ValueError("only batch workloads take a reduced B")
        B0 = B
    Q, C = normal_inputs(seed, B0, K, D)
    T = np.float32(1.0)
    if base == "clm_cos_batch8_255x512" and B0 >= 8:
        # "one case scaled x1e3": question 7 stored with q and C times 1e3
        Q[7] *= np.float32(1e3)
        C[7] *= np.float32(1e3)
    if name == base:
        return Workload(name, call, sim, scale, T, Q, C, desc)
    if name == "clm_cos_1x512_single_candidate":
        return Workload(name, call, sim, scale, T, Q, np.ascontiguousarray(C[:, :1]),
                        "single candidate: first row of clm_cos_255x512")
    if name == "clm_cos_255x512_identical":
        C2 = np.repeat(C[:, :1], K, axis=1)
        return Workload(name, call, sim, scale, T, Q, np.ascontiguousarray(C2),
                        "255 identical candidates: every row equals row 0")
    if name == "clm_cos_255x512_zero_row":
        C[:, 127] = 0.0
        return Workload(name, call, sim, scale, T, Q, C, "row 127 set to zero")
    if name == "clm_cos_batch8_255x512_overflow":
        return Workload(name, call, sim, SCALE_COSINE_OVERFLOW, T, Q, C,
                        "same data, logit multiplier x1e3: raw logits overflow a naive exp")
    raise KeyError(name)


ALL = [
    "clm_cos_5x512",
    "clm_cos_64x512",
    "clm_cos_255x512",
    "clm_cos_1x512_single_candidate",
    "clm_cos_255x512_identical",
    "clm_cos_255x512_zero_row",
    "clm_cos_batch8_255x512",
    "clm_cos_batch8_255x512_overflow",
    "kev_dot_255x2560",
    "kev_dot_batch1024_255x2560",
]


def ragged_offsets(seed: int, B: int, k_max: int = 255, k_min: int = 1) -> np.ndarray:
    """Per-question candidate counts drawn uniformly in [k_min, k_max],
    returned as B+1 int64 row offsets starting at 0."""
    rng = np.random.default_rng(seed)
    counts = rng.integers(k_min, k_max + 1, size=B)
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


def ragged_inputs(seed: int, offsets: np.ndarray, D: int):
    """Q [B,D] and a packed candidate block C [offsets[-1], D], fp32 N(0,1)."""
    rng = np.random.default_rng(seed)
    B = offsets.size - 1
    Q = rng.standard_normal((B, D), dtype=np.float32)
    C = rng.standard_normal((int(offsets[-1]), D), dtype=np.float32)
    return Q, C


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest bf16 (ties to even); returns the 16-bit
    patterns as uint16."""
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    # uint32 arithmetic: only NaN patterns could wrap, and inputs hold none
    rounded = (bits + np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """The fp32 values of bf16 patterns (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Projected:
    """Inputs of projection + scoring: hidden states and head weights, bf16.
    ``*_bits`` are the uint16 patterns the GPU reads; ``*_f32`` the same
    values as fp32 for the oracle."""
    name: str
    similarity: str
    scale: np.float32
    xq_bits: np.ndarray   # [B, Hq]
    xc_bits: np.ndarray   # [B, K, Hc]
    wq_bits: np.ndarray   # [P, Hq]
    wc_bits: np.ndarray   # [P, Hc]

    def f32(self, which: str) -> np.ndarray:
        return bf16_bits_to_f32(getattr(self, which + "_bits"))

    @property
    def B(self) -> int:
        return self.xc_bits.shape[0]

    @property
    def K(self) -> int:
        return self.xc_bits.shape[1]

    @property
    def Hc(self) -> int:
        return self.xc_bits.shape[2]

    @property
    def Hq(self) -> int:
        return self.xq_bits.shape[1]

    @property
    def P(self) -> int:
        return self.wc_bits.shape[0]

    @property
    def algorithmic_bytes(self) -> int:
        """bf16 inputs read once (hidden states and both heads), fp32 out."""
        return 2 * (self.B * self.K * self.Hc + self.B * self.Hq + self.P * (self.Hq + self.Hc)) \
            + 4 * self.B * self.K


def projected_inputs(seed: int, B: int, K: int, Hq: int, Hc: int, P: int, similarity: str,
                     scale=None, name: str = "projected") -> Projected:
    """Hidden states N(0,1) and head weights N(0, 1/H) (so projected features
    are O(1)), drawn in the order xq, xc, wq, wc and rounded to bf16."""
    rng = np.random.default_rng(seed)
    xq = rng.standard_normal((B, Hq), dtype=np.float32)
    xc = rng.standard_normal((B, K, Hc), dtype=np.float32)
    wq = rng.standard_normal((P, Hq), dtype=np.float32) * np.float32(1.0 / math.sqrt(Hq))
    wc = rng.standard_normal((P, Hc), dtype=np.float32) * np.float32(1.0 / math.sqrt(Hc))
    if scale is None:
        scale = SCALE_COSINE if similarity == "cosine" else SCALE_DOT
    return Projected(name, similarity, np.float32(scale), to_bf16_bits(xq), to_bf16_bits(xc),
                     to_bf16_bits(wq), to_bf16_bits(wc))


# Projection workloads: Kev's heads map a 2560-wide hidden state to 256
# features (the 1/sqrt(256) scale); CLM's map 512 to 256.
PROJECTED_CONFIGS = {
    "kev_proj_dot_batch1024_255x2560_p256": (1024, 255, 2560, 2560, 256, "dot", 7),
    "clm_proj_cos_batch1024_255x512_p256": (1024, 255, 512, 512, 256, "cosine", 8),
}


def make_projected(name: str, B: int | None = None) -> Projected:
    B0, K, Hq, Hc, P, sim, seed = PROJECTED_CONFIGS[name]
    return projected_inputs(seed, B0 if B is None else B, K, Hq, Hc, P, sim, name=name)
