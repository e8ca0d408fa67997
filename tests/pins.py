"""Checks that pin the oracle to facts other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with what the page or the mathematics fixes:
closed forms, invariants, special cases that reduce to library routines,
and 50-digit brute force on tiny inputs. They are collected in ``PINS`` so
that the same checks run against the real oracle and against copies with a
planted mistake (the mutation test), where at least one must fail.

Source: pull request "cuda: add a fused candidate-scoring kernel for CLM and
Kev" -- intro (similarities), "What is fused, precisely" (K <= 255) and
"Verified on hardware" (degenerate cases, rejected arguments).
"""
from __future__ import annotations

import math
from decimal import Decimal, getcontext
from pathlib import Path

import numpy as np
import scipy.special
from sklearn.metrics.pairwise import cosine_similarity

GOLDEN = Path(__file__).resolve().parent / "golden"

SCALE_CLM = float(np.float32(1.0 / 0.07))  # fp32 of exp(log(1/0.07))
SCALE_KEV = 0.0625


def _rng(seed):
    return np.random.default_rng(seed)


def _normal(rng, *shape):
    return rng.standard_normal(shape, dtype=np.float32)


def pin_single_candidate(orc):
    """One candidate gives probability exactly 1 for any finite input."""
    rng = _rng(11)
    for sim in ("dot", "cosine"):
        for D in (1, 3, 512):
            q, C = _normal(rng, D), _normal(rng, 1, D)
            for scale in (SCALE_CLM, SCALE_KEV, -3.5, 1e4):
                p = orc.score(q, C, sim, scale)
                assert p.shape == (1,) and p[0] == 1.0, (sim, D, scale, p)


def pin_identical_uniform(orc):
    """K identical candidates give exactly 1/K each (double)."""
    rng = _rng(12)
    for sim in ("dot", "cosine"):
        for K in (2, 3, 7, 64, 255):
            D = 33
            q = _normal(rng, D)
            C = np.repeat(_normal(rng, 1, D), K, axis=0)
            p = orc.score(q, C, sim, SCALE_CLM)
            assert np.all(p == 1.0 / K), (sim, K, p[:3])


def pin_rows_sum_to_one(orc):
    """Every row is a probability distribution: nonnegative, sums to 1."""
    rng = _rng(13)
    for sim, scale in (("dot", SCALE_KEV), ("cosine", SCALE_CLM)):
        Q, C = _normal(rng, 6, 40), _normal(rng, 6, 255, 40)
        p = orc.score(Q, C, sim, scale)
        assert p.shape == (6, 255)
        assert np.all(p >= 0.0)
        assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= 1e-12


def pin_zero_candidate_logistic(orc):
    """K=2, cosine, c0 = q, c1 = 0: cos = (1, 0), so with s = scale/T
    p0 = 1/(1+e^-s) and p1 = e^-s/(1+e^-s) (the logistic function)."""
    rng = _rng(14)
    for D in (1, 7, 512):
        q = _normal(rng, D)
        C = np.stack([q, np.zeros(D, np.float32)])
        for scale, T in ((SCALE_CLM, 1.0), (3.0, 0.5), (-2.0, 1.0)):
            p = orc.score(q, C, "cosine", scale, T)
            s = float(np.float32(scale)) / float(np.float32(T))
            p1 = math.exp(-s) / (1.0 + math.exp(-s))
            p0 = 1.0 / (1.0 + math.exp(-s))
            assert abs(p[0] - p0) <= 1e-15 and abs(p[1] - p1) <= 1e-15, (D, scale, p, p0, p1)
    # dot similarity of a zero candidate is exactly 0 as well
    q = _normal(rng, 9)
    C = np.stack([np.zeros(9, np.float32), np.zeros(9, np.float32), q])
    z = orc.logits(q, C, "dot", 1.0)
    assert z[0] == 0.0 and z[1] == 0.0


def pin_zero_query_uniform(orc):
    """A zero query (not a null one) makes every cosine 0: uniform 1/K."""
    rng = _rng(15)
    for K in (1, 5, 255):
        q = np.zeros(16, np.float32)
        C = _normal(rng, K, 16)
        p = orc.score(q, C, "cosine", SCALE_CLM)
        assert np.all(p == 1.0 / K)


def pin_overflow_stable(orc):
    """K=2, cosine, c0 = q, c1 = -q with the x1e3 logit multiplier: the
    logits are +S and -S, S ~ 1.4e4, which overflow a naive exp in fp32 and
    in double; the stable softmax is (1/(1+e^-2S), e^-2S/(1+e^-2S)) = (1, 0)."""
    rng = _rng(16)
    q = _normal(rng, 512)
    C = np.stack([q, -q])
    S = float(np.float32(SCALE_CLM * 1e3))
    with np.errstate(over="ignore", invalid="ignore"):
        naive = np.exp(np.array([S, -S])) / np.exp(np.array([S, -S])).sum()
    assert not np.all(np.isfinite(naive))  # the case really breaks a naive exp
    p = orc.score(q, C, "cosine", S)
    assert p[0] == 1.0 and p[1] == 0.0, p
    z = orc.logits(q, C, "cosine", S)
    assert abs(z[0] - S) <= 1e-9 * S and abs(z[1] + S) <= 1e-9 * S


def pin_shift_invariance(orc):
    """softmax(z + c) = softmax(z): with dot similarity, appending one
    coordinate t to every candidate and 1 to the query adds scale*t to every
    logit. Large t would overflow any unshifted exp."""
    rng = _rng(17)
    K, D = 37, 20
    q, C = _normal(rng, D), _normal(rng, K, D)
    base = orc.score(q, C, "dot", 1.0)
    for t in (1e2, 7e2, 1e6, -1e6):
        q2 = np.concatenate([q, [1.0]]).astype(np.float32)
        C2 = np.concatenate([C, np.full((K, 1), t, np.float32)], axis=1)
        p = orc.score(q2, C2, "dot", 1.0)
        if abs(t) < 1e3:
            assert np.max(np.abs(p - base)) <= 1e-12, t
        else:
            # at |t| = 1e6 the double sum itself loses the small terms' bits;
            # the distribution must still be finite and close
            assert np.all(np.isfinite(p)) and np.max(np.abs(p - base)) <= 1e-6, t


def pin_cosine_scale_invariance(orc):
    """Cosine ignores vector lengths: q -> a*q and c_k -> b_k*c_k (a, b_k > 0)
    leave the distribution unchanged."""
    rng = _rng(18)
    Q, C = _normal(rng, 3, 64), _normal(rng, 3, 30, 64)
    base = orc.score(Q, C, "cosine", SCALE_CLM)
    Q2 = Q * np.float32(8.0)                      # powers of two keep fp32 exact
    C2 = C * (np.float32(2.0) ** rng.integers(-6, 7, size=(3, 30, 1))).astype(np.float32)
    p = orc.score(Q2, C2, "cosine", SCALE_CLM)
    assert np.max(np.abs(p - base)) <= 1e-14


def pin_permutation_equivariance(orc):
    """Permuting the candidate rows permutes the probabilities."""
    rng = _rng(19)
    for sim in ("dot", "cosine"):
        Q, C = _normal(rng, 2, 48), _normal(rng, 2, 17, 48)
        base = orc.score(Q, C, sim, SCALE_CLM if sim == "cosine" else SCALE_KEV)
        perm = rng.permutation(17)
        p = orc.score(Q, C[:, perm], sim, SCALE_CLM if sim == "cosine" else SCALE_KEV)
        # z values are bitwise the same; only the order of the softmax sum moves
        assert np.max(np.abs(p - base[:, perm])) <= 1e-15


def pin_basis_rows(orc):
    """Candidates that are unit basis vectors e_{i_k} select coordinates of q:
    dot gives z_k = scale*q[i_k]/T, cosine gives scale*q[i_k]/(|q| T). The
    distribution is then scipy's softmax of that vector."""
    rng = _rng(20)
    D = 50
    q = _normal(rng, D)
    idx = rng.choice(D, size=12, replace=False)
    C = np.zeros((12, D), np.float32)
    C[np.arange(12), idx] = 1.0
    qd = q.astype(np.float64)
    for sim, scale, T in (("dot", 0.75, 1.0), ("dot", -2.0, 0.5), ("cosine", SCALE_CLM, 1.0),
                          ("cosine", 5.0, 2.0)):
        s = float(np.float32(scale)) / float(np.float32(T))
        v = qd[idx] * s
        if sim == "cosine":
            v = v / np.linalg.norm(qd)
        want = scipy.special.softmax(v)
        p = orc.score(q, C, sim, scale, T)
        assert np.max(np.abs(p - want)) <= 1e-14, (sim, scale, T)


def pin_library_routines(orc):
    """General random inputs against library routines: scikit-learn's
    cosine_similarity / numpy's matrix product, then scipy's softmax."""
    rng = _rng(21)
    for sim, scale in (("dot", SCALE_KEV), ("cosine", SCALE_CLM)):
        for B, K, D in ((1, 5, 512), (3, 255, 96), (2, 64, 2560)):
            Q, C = _normal(rng, B, D), _normal(rng, B, K, D)
            p = orc.score(Q, C, sim, scale)
            for b in range(B):
                Cb, qb = C[b].astype(np.float64), Q[b].astype(np.float64)
                s = cosine_similarity(Cb, qb[None, :])[:, 0] if sim == "cosine" else Cb @ qb
                want = scipy.special.softmax(float(np.float32(scale)) * s)
                assert np.max(np.abs(p[b] - want)) <= 1e-11, (sim, B, K, D)


def _decimal_scores(q, C, sim, scale, T):
    getcontext().prec = 50
    qd = [Decimal(float(x)) for x in q]
    z = []
    for row in C:
        cd = [Decimal(float(x)) for x in row]
        dot = sum((a * b for a, b in zip(cd, qd)), Decimal(0))
        if sim == "cosine":
            nq = max(sum((a * a for a in qd), Decimal(0)).sqrt(), Decimal("1e-12"))
            nc = max(sum((a * a for a in cd), Decimal(0)).sqrt(), Decimal("1e-12"))
            dot = dot / (nq * nc)
        z.append(Decimal(float(np.float32(scale))) * dot / Decimal(float(np.float32(T))))
    m = max(z)
    e = [(x - m).exp() for x in z]
    total = sum(e, Decimal(0))
    return [float(x / total) for x in e]


def pin_decimal_bruteforce(orc):
    """Tiny inputs (K <= 5, D <= 8) evaluated with 50-digit decimals."""
    rng = _rng(22)
    for trial in range(6):
        K, D = int(rng.integers(1, 6)), int(rng.integers(1, 9))
        sim = ("dot", "cosine")[trial % 2]
        q, C = _normal(rng, D), _normal(rng, K, D)
        scale, T = (SCALE_CLM, 1.0) if sim == "cosine" else (1.7, 0.8)
        want = np.array(_decimal_scores(q, C, sim, scale, T))
        p = orc.score(q, C, sim, scale, T)
        assert np.max(np.abs(p - want)) <= 1e-14, (K, D, sim)


def pin_temperature(orc):
    """Only scale/T enters: (scale, T) and (scale/T, 1) give the same result
    when both ratios are exact in fp32; a larger T flattens the distribution."""
    rng = _rng(23)
    q, C = _normal(rng, 24), _normal(rng, 9, 24)
    for sim in ("dot", "cosine"):
        a = orc.score(q, C, sim, 6.0, 4.0)
        b = orc.score(q, C, sim, 1.5, 1.0)
        assert np.max(np.abs(a - b)) <= 1e-15
        hot = orc.score(q, C, sim, 6.0, 0.25)
        cold = orc.score(q, C, sim, 6.0, 64.0)
        assert hot.max() > a.max() > cold.max()
        assert np.max(np.abs(cold - 1.0 / 9)) < np.max(np.abs(a - 1.0 / 9))


def pin_batch_independence(orc):
    """A batch is independent questions: each row of a batch call equals the
    single-question call on that question's own q and C."""
    rng = _rng(24)
    for sim in ("dot", "cosine"):
        Q, C = _normal(rng, 4, 32), _normal(rng, 4, 11, 32)
        p = orc.score(Q, C, sim, 2.0)
        for b in range(4):
            assert np.array_equal(p[b], orc.score(Q[b], C[b], sim, 2.0))


STATUS_BY_NAME = {"OK": 0, "NULL_POINTER": -1, "K_RANGE": -2, "D_RANGE": -3, "SCALE": -4,
                  "TEMPERATURE": -5, "BATCH": -6, "SIMILARITY": -7}


def rejection_cases():
    """Rows of golden/rejections.txt as (origin, overrides, expected name)."""
    rows = []
    for line in (GOLDEN / "rejections.txt").read_text().splitlines():
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        origin, change, expect = [x.strip() for x in line.split("|")]
        key, val = change.split("=")
        if val == "null":
            parsed = None
        elif key in ("B", "K", "D", "similarity"):
            parsed = int(val)
        else:
            parsed = float(val)
        rows.append((origin, {key: parsed}, expect))
    return rows


def pin_rejections(orc):
    """The page's six rejected arguments (and the readings added to them)
    return their error code; the valid base call returns OK."""
    rng = _rng(25)
    Q, C = _normal(rng, 1, 8), _normal(rng, 1, 4, 8)
    base = dict(query=Q, candidates=C, out=True, B=1, K=4, D=8, similarity=0, scale=1.0,
                temperature=1.0)
    st, _ = orc.score_raw(Q, C, 1, 4, 8, 0, 1.0, 1.0)
    assert st == 0
    for origin, change, expect in rejection_cases():
        args = dict(base, **change)
        st, out = orc.score_raw(args["query"], args["candidates"], args["B"], args["K"],
                                args["D"], args["similarity"], args["scale"],
                                args["temperature"], out_present=args["out"] is not None)
        assert st == STATUS_BY_NAME[expect], (origin, change, st)
        assert np.all(out == -7.0), "rejected call must leave the output untouched"


def pin_nan_propagates(orc):
    """A NaN in a candidate makes its question's whole row NaN and leaves the
    other questions alone (reading: inputs are not scanned)."""
    rng = _rng(26)
    Q, C = _normal(rng, 2, 16), _normal(rng, 2, 5, 16)
    C[1, 3, 7] = np.nan
    p = orc.score(Q, C, "dot", 1.0)
    assert np.all(np.isnan(p[1])) and np.all(np.isfinite(p[0]))


def pin_ragged(orc):
    """A ragged batch equals one single-question call per question."""
    rng = _rng(27)
    counts = [1, 255, 7, 64, 2]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    Q = _normal(rng, len(counts), 40)
    C = _normal(rng, int(offsets[-1]), 40)
    for sim in ("dot", "cosine"):
        p = orc.score_ragged(Q, C, offsets, sim, SCALE_CLM)
        for b in range(len(counts)):
            lo, hi = offsets[b], offsets[b + 1]
            assert np.array_equal(p[lo:hi], orc.score(Q[b], C[lo:hi], sim, SCALE_CLM))


def pin_projected(orc):
    """Projection then scoring: with identity weights it equals plain
    scoring; in general it equals numpy's matrix products (float64) fed to
    the plain definition via scikit-learn and scipy."""
    rng = _rng(28)
    B, K, D = 2, 9, 12
    Xq, Xc = _normal(rng, B, D), _normal(rng, B, K, D)
    eye = np.eye(D, dtype=np.float32)
    for sim in ("dot", "cosine"):
        a = orc.score_projected(Xq, eye, Xc, eye, sim, SCALE_CLM)
        b = orc.score(Xq, Xc, sim, SCALE_CLM)
        assert np.max(np.abs(a - b)) <= 1e-15
    Dq, Dc, P = 10, 14, 6
    Xq, Xc = _normal(rng, B, Dq), _normal(rng, B, K, Dc)
    Wq, Wc = _normal(rng, P, Dq), _normal(rng, P, Dc)
    for sim in ("dot", "cosine"):
        p = orc.score_projected(Xq, Wq, Xc, Wc, sim, 2.5)
        for b in range(B):
            qv = Wq.astype(np.float64) @ Xq[b].astype(np.float64)
            cv = Xc[b].astype(np.float64) @ Wc.astype(np.float64).T
            s = cosine_similarity(cv, qv[None, :])[:, 0] if sim == "cosine" else cv @ qv
            want = scipy.special.softmax(2.5 * s)
            assert np.max(np.abs(p[b] - want)) <= 1e-12, sim
    # A zero projected query: every cosine is 0, so the distribution is
    # exactly uniform (the same clamp as the plain path's zero query).
    Xq0 = np.zeros_like(Xq)
    p = orc.score_projected(Xq0, Wq, Xc, Wc, "cosine", 2.5)
    assert np.all(p == 1.0 / K)


PINS = [
    pin_single_candidate,
    pin_identical_uniform,
    pin_rows_sum_to_one,
    pin_zero_candidate_logistic,
    pin_zero_query_uniform,
    pin_overflow_stable,
    pin_shift_invariance,
    pin_cosine_scale_invariance,
    pin_permutation_equivariance,
    pin_basis_rows,
    pin_library_routines,
    pin_decimal_bruteforce,
    pin_temperature,
    pin_batch_independence,
    pin_rejections,
    pin_nan_propagates,
    pin_ragged,
    pin_projected,
]
