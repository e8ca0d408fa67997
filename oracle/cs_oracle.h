/*
 * cs_oracle.h -- double-precision CPU oracle for fused candidate scoring.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may include, link,
 * load or call this code: only the test suite, the package's smoke check and
 * the bench's CPU-baseline leg do. It shares no header, helper, constant or
 * table with the HIP library; the status codes below are defined here on
 * their own and carry the same numeric values because both sides implement
 * the same published rejection list.
 *
 * Source: the pull request "cuda: add a fused candidate-scoring kernel for
 * CLM and Kev".
 *   - Intro, model/similarity table: CLM scores a candidate by exp(logit_scale)
 *     times the cosine of the two projected vectors; Kev by scale times the
 *     dot product with scale = 1/sqrt(256); both take a softmax over that
 *     question's candidates.
 *   - "What is fused, precisely": at most 255 candidates per question; a
 *     batch is a set of independent questions.
 *   - "Verified on hardware", rejected-arguments bullet: K above 255, K of
 *     zero, D of zero, a zero scale, a negative temperature and a null query
 *     are errors, not scored answers.
 *
 * Readings where the page is silent (each is listed with its reason in the
 * design notes):
 *   - scale is a linear multiplier (the caller passes exp(logit_scale));
 *   - z_k = scale * s_k / T; T == 0, NaN or infinite is also rejected, as is a
 *     NaN or infinite scale, B <= 0, an unknown similarity, and a null
 *     candidate or output pointer;
 *   - cosine uses per-norm clamping: cos = q.c / (max(|q|,eps) * max(|c|,eps))
 *     with eps = 1e-12, so a zero candidate scores exactly 0 and a zero query
 *     gives the uniform distribution;
 *   - NaN or infinite inputs propagate into the output row; nothing scans for
 *     them.
 *
 * Parity pins: every function here is pinned by CPU tests against closed
 * forms, invariants, library routines and 50-digit brute force (see the
 * tests named test_oracle_pins.py and test_oracle_mutants.py).
 */
#ifndef CS_ORACLE_H
#define CS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  CSO_OK = 0,
  CSO_ERR_NULL_POINTER = -1,
  CSO_ERR_K_RANGE = -2,
  CSO_ERR_D_RANGE = -3,
  CSO_ERR_SCALE = -4,
  CSO_ERR_TEMPERATURE = -5,
  CSO_ERR_BATCH = -6,
  CSO_ERR_SIMILARITY = -7
};

enum { CSO_SIM_DOT = 0, CSO_SIM_COSINE = 1 };

#define CSO_MAX_K 255

/* Argument check in a fixed order: pointers, B, K, D, similarity, scale,
 * temperature. Returns CSO_OK or the first failing code. */
int cso_validate(int query_present, int candidates_present, int out_present,
                 int64_t B, int64_t K, int64_t D, int similarity, float scale,
                 float temperature);

/* Scaled similarities z[b*K + k] = scale * s(q_b, c_bk) / T, in double.
 * Q is [B][D], C is [B][K][D], z is [B][K]; all row-major host memory. */
int cso_logits(const float *Q, const float *C, int B, int K, int D,
               int similarity, float scale, float temperature, double *z);

/* Softmax of the scaled similarities over each question's K candidates:
 * p[b*K + k], in double. On error, p is left untouched. */
int cso_score(const float *Q, const float *C, int B, int K, int D,
              int similarity, float scale, float temperature, double *p);

/* Ragged batch: question b owns candidate rows offsets[b] .. offsets[b+1]-1
 * of C (row length D) and the same slots of p; Q is [B][D]. Each question's
 * count must lie in 1..255 and offsets[0] must be 0. */
int cso_score_ragged(const float *Q, const float *C, const int64_t *offsets,
                     int B, int D, int similarity, float scale,
                     float temperature, double *p);

/* Projection followed by scoring, all in double: the query is x_q W_q^T and
 * candidate k is x_k W_c^T, with W_q [P][Dq] and W_c [P][Dc] row-major;
 * Xq is [B][Dq], Xc is [B][K][Dc]; the scores use those P-dimensional
 * vectors exactly as cso_score does. */
int cso_score_projected(const float *Xq, const float *Wq, const float *Xc,
                        const float *Wc, int B, int K, int Dq, int Dc, int P,
                        int similarity, float scale, float temperature,
                        double *p);

#ifdef __cplusplus
}
#endif

#endif
