"""Plant plausible mistakes in copies of the oracle and check that the pins
catch every one of them (CPU only; nothing here touches a GPU).

Each mutant is the oracle's C source with one textual change, compiled with
the same flags into a temporary library. A mutant passes the suite only if
every pin passes, which would mean the pins cannot tell that mistake apart
from the correct oracle.
"""
from __future__ import annotations

import faulthandler
import multiprocessing as mp

import pytest

import oracle
from pins import PINS

MUTANTS = {
    "no_max_subtraction": ("z[k] = exp(z[k] - m);", "z[k] = exp(z[k]);"),
    "min_instead_of_max": ("if (z[k] > m) m = z[k];", "if (z[k] < m) m = z[k];"),
    "sum_of_squares_as_total": ("total += z[k];", "total += z[k] * z[k];"),
    "last_entry_not_normalised": ("for (int k = 0; k < K; ++k) z[k] = z[k] / total;",
                                  "for (int k = 0; k < K - 1; ++k) z[k] = z[k] / total;"),
    "temperature_multiplies": ("z[k] = (double)scale * s / (double)temperature;",
                               "z[k] = (double)scale * s * (double)temperature;"),
    "scale_sign_flipped": ("z[k] = (double)scale * s / (double)temperature;",
                           "z[k] = -(double)scale * s / (double)temperature;"),
    "query_norm_dropped": ("s = s / (qnorm * clamped_norm(c, D));",
                           "s = s / clamped_norm(c, D);"),
    "candidate_norm_dropped": ("s = s / (qnorm * clamped_norm(c, D));", "s = s / qnorm;"),
    "squared_norms": ("s = s / (qnorm * clamped_norm(c, D));",
                      "s = s / (qnorm * qnorm * clamped_norm(c, D) * clamped_norm(c, D));"),
    "no_norm_clamp": ("return n < CSO_NORM_EPS ? CSO_NORM_EPS : n;", "return n;"),
    "rows_reversed": ("const float *c = Cq + (size_t)k * (size_t)D;",
                      "const float *c = Cq + (size_t)(K - 1 - k) * (size_t)D;"),
    "first_query_for_all": ("question_logits(Q + (size_t)b * (size_t)D, C + (size_t)b * (size_t)K",
                            "question_logits(Q, C + (size_t)b * (size_t)K"),
    "float_accumulator": ("double s = 0.0;\n  for (int d = 0; d < D; ++d) s += (double)a[d] * (double)b[d];",
                          "float s = 0.0f;\n  for (int d = 0; d < D; ++d) s += a[d] * b[d];"),
    "dot_skips_last_element": ("for (int d = 0; d < D; ++d) s += (double)a[d] * (double)b[d];",
                               "for (int d = 0; d < D - 1; ++d) s += (double)a[d] * (double)b[d];"),
    "k_limit_256": ("if (K <= 0 || K > CSO_MAX_K) return CSO_ERR_K_RANGE;",
                    "if (K <= 0 || K > 256) return CSO_ERR_K_RANGE;"),
    "zero_scale_accepted": ("if (scale == 0.0f || isnan(scale)", "if (isnan(scale)"),
    "negative_temperature_accepted": ("if (!(temperature > 0.0f) || isinf(temperature))",
                                      "if (temperature == 0.0f || isinf(temperature))"),
    "null_query_accepted": ("if (!query_present || !candidates_present || !out_present)",
                            "if (!candidates_present || !out_present)"),
    # ragged batches
    "ragged_output_at_question_index": ("double *pb = p + offsets[b];", "double *pb = p + b;"),
    "ragged_rows_of_first_question": (
        "question_logits(Q + (size_t)b * (size_t)D, C + (size_t)offsets[b] * (size_t)D,",
        "question_logits(Q + (size_t)b * (size_t)D, C,"),
    "ragged_count_one_short": ("int K = (int)(offsets[b + 1] - offsets[b]);",
                               "int K = (int)(offsets[b + 1] - offsets[b]) - 1;"),
    # projection + scoring
    "projected_candidate_norm_dropped": ("s = s / (qnorm * cnorm);", "s = s / qnorm;"),
    "projected_query_norm_unclamped": ("if (qnorm < CSO_NORM_EPS) qnorm = CSO_NORM_EPS;", ""),
    "projected_scale_dropped": ("pb[k] = (double)scale * s / (double)temperature;",
                                "pb[k] = s / (double)temperature;"),
    "projected_candidate_times_itself": ("double s = dot_double(c, q, P);",
                                         "double s = dot_double(c, c, P);"),
    "projected_query_head_for_candidates": (
        "project(Wc, Xc + ((size_t)b * (size_t)K + (size_t)k) * (size_t)Dc, P, Dc, c);",
        "project(Wq, Xc + ((size_t)b * (size_t)K + (size_t)k) * (size_t)Dc, P, Dc, c);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    before, after = MUTANTS[name]
    src = oracle.SOURCE.read_text()
    assert src.count(before) >= 1, f"mutation anchor for {name} no longer in the oracle"
    mutated = tmp_path / "cs_oracle.c"
    mutated.write_text(src.replace(before, after))
    (tmp_path / "cs_oracle.h").write_text((oracle.HERE / "cs_oracle.h").read_text())
    lib = oracle.build(mutated, tmp_path / f"libcs_oracle_{name}.so", extra_flags=("-w",))
    # Run the pins in a child process: a mutant that dereferences a null
    # pointer it should have rejected crashes, which also counts as caught.
    ctx = mp.get_context("fork")
    queue = ctx.Queue()
    child = ctx.Process(target=_run_pins, args=(str(lib), queue))
    child.start()
    child.join(120)
    assert child.exitcode is not None, "mutant run did not finish"
    caught = queue.get() if child.exitcode == 0 else ["<crashed>"]
    assert caught, f"no pin fails on the planted mistake {name}"


def _run_pins(lib_path, queue):
    faulthandler.disable()  # a crash here is an expected outcome, not a report
    mutant = oracle.Oracle(lib_path)
    caught = []
    for pin in PINS:
        try:
            pin(mutant)
        except (AssertionError, oracle.OracleError, FloatingPointError):
            caught.append(pin.__name__)
    queue.put(caught)
