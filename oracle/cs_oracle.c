/*
 * cs_oracle.c -- plain, slow, double-precision reference of fused candidate
 * scoring. TEST INFRASTRUCTURE ONLY (see cs_oracle.h for who may use it).
 *
 * Every step is the textbook definition written out with sequential loops:
 * no blocking, no fusion, no reordering. Inputs are fp32 and are promoted
 * exactly to double before any arithmetic; the product of two fp32 values is
 * exact in double, so the only roundings are in the running sums, the square
 * roots, the divisions and exp().
 *
 * Source: the pull request "cuda: add a fused candidate-scoring kernel for
 * CLM and Kev" -- intro (model/similarity table), "What is fused, precisely"
 * and "Verified on hardware" (rejected arguments). The readings taken where
 * the page is silent are listed in cs_oracle.h.
 */
#include "cs_oracle.h"

#include <math.h>
#include <stddef.h>
#include <stdlib.h>

/* Norm clamp of the cosine: cos(q,c) = q.c / (max(|q|,EPS) * max(|c|,EPS)).
 * The page lists "a zero candidate" as a degenerate case without a
 * convention; this clamp makes its similarity exactly zero. */
static const double CSO_NORM_EPS = 1e-12;

int cso_validate(int query_present, int candidates_present, int out_present,
                 int64_t B, int64_t K, int64_t D, int similarity, float scale,
                 float temperature) {
  /* "Verified on hardware": a null query is rejected; null candidates and
   * output are rejected by the same reasoning. */
  if (!query_present || !candidates_present || !out_present)
    return CSO_ERR_NULL_POINTER;
  if (B <= 0) return CSO_ERR_BATCH;
  /* K of zero and K above 255 are rejected: the in-block softmax holds at
   * most 255 candidates ("What is fused, precisely"). */
  if (K <= 0 || K > CSO_MAX_K) return CSO_ERR_K_RANGE;
  if (D <= 0) return CSO_ERR_D_RANGE;
  if (similarity != CSO_SIM_DOT && similarity != CSO_SIM_COSINE)
    return CSO_ERR_SIMILARITY;
  /* A zero scale is rejected; NaN and infinities are too (reading). */
  if (scale == 0.0f || isnan(scale) || isinf(scale)) return CSO_ERR_SCALE;
  /* A negative temperature is rejected; zero, NaN and infinities are too,
   * since z = scale * s / T is undefined or degenerate there (reading). */
  if (!(temperature > 0.0f) || isinf(temperature)) return CSO_ERR_TEMPERATURE;
  /* The call forms its logits in fp32 (the page's precision) with the factor
   * scale / T; a factor beyond the fp32 range is rejected (reading). */
  if (isinf((float)((double)scale / (double)temperature))) return CSO_ERR_SCALE;
  return CSO_OK;
}

/* Dot product of two fp32 vectors of length D, summed in index order. */
static double dot_product(const float *a, const float *b, int D) {
  double s = 0.0;
  for (int d = 0; d < D; ++d) s += (double)a[d] * (double)b[d];
  return s;
}

/* Euclidean norm of an fp32 vector, clamped below at CSO_NORM_EPS. */
static double clamped_norm(const float *a, int D) {
  double n = sqrt(dot_product(a, a, D));
  return n < CSO_NORM_EPS ? CSO_NORM_EPS : n;
}

/* One question's scaled similarities: z[k] = scale * s(q, c_k) / T, where s
 * is the cosine (CLM) or the plain dot product (Kev). */
static void question_logits(const float *q, const float *Cq, int K, int D,
                            int similarity, float scale, float temperature,
                            double *z) {
  double qnorm = similarity == CSO_SIM_COSINE ? clamped_norm(q, D) : 1.0;
  for (int k = 0; k < K; ++k) {
    const float *c = Cq + (size_t)k * (size_t)D;
    double s = dot_product(c, q, D);
    if (similarity == CSO_SIM_COSINE) s = s / (qnorm * clamped_norm(c, D));
    z[k] = (double)scale * s / (double)temperature;
  }
}

/* Numerically stable softmax in place: subtract the maximum, exponentiate,
 * divide by the sum (summed in index order). A NaN anywhere makes the sum,
 * and so the whole row, NaN. */
static void softmax_in_place(double *z, int K) {
  double m = z[0];
  for (int k = 1; k < K; ++k)
    if (z[k] > m) m = z[k];
  double total = 0.0;
  for (int k = 0; k < K; ++k) {
    z[k] = exp(z[k] - m);
    total += z[k];
  }
  for (int k = 0; k < K; ++k) z[k] = z[k] / total;
}

int cso_logits(const float *Q, const float *C, int B, int K, int D,
               int similarity, float scale, float temperature, double *z) {
  int st = cso_validate(Q != NULL, C != NULL, z != NULL, B, K, D, similarity,
                        scale, temperature);
  if (st != CSO_OK) return st;
  for (int b = 0; b < B; ++b)
    question_logits(Q + (size_t)b * (size_t)D, C + (size_t)b * (size_t)K * (size_t)D,
                    K, D, similarity, scale, temperature, z + (size_t)b * (size_t)K);
  return CSO_OK;
}

int cso_score(const float *Q, const float *C, int B, int K, int D,
              int similarity, float scale, float temperature, double *p) {
  int st = cso_validate(Q != NULL, C != NULL, p != NULL, B, K, D, similarity,
                        scale, temperature);
  if (st != CSO_OK) return st;
  for (int b = 0; b < B; ++b) {
    double *pb = p + (size_t)b * (size_t)K;
    question_logits(Q + (size_t)b * (size_t)D, C + (size_t)b * (size_t)K * (size_t)D,
                    K, D, similarity, scale, temperature, pb);
    softmax_in_place(pb, K);
  }
  return CSO_OK;
}

int cso_score_ragged(const float *Q, const float *C, const int64_t *offsets,
                     int B, int D, int similarity, float scale,
                     float temperature, double *p) {
  if (offsets == NULL) return CSO_ERR_NULL_POINTER;
  /* Validate the shared arguments with a placeholder K of 1, then each
   * question's own count. */
  int st = cso_validate(Q != NULL, C != NULL, p != NULL, B, 1, D, similarity,
                        scale, temperature);
  if (st != CSO_OK) return st;
  if (offsets[0] != 0) return CSO_ERR_K_RANGE;
  for (int b = 0; b < B; ++b) {
    int64_t count = offsets[b + 1] - offsets[b];
    if (count <= 0 || count > CSO_MAX_K) return CSO_ERR_K_RANGE;
  }
  for (int b = 0; b < B; ++b) {
    int K = (int)(offsets[b + 1] - offsets[b]);
    double *pb = p + offsets[b];
    question_logits(Q + (size_t)b * (size_t)D, C + (size_t)offsets[b] * (size_t)D,
                    K, D, similarity, scale, temperature, pb);
    softmax_in_place(pb, K);
  }
  return CSO_OK;
}

/* y = W x for W [P][Din] row-major, in double. */
static void project(const float *W, const float *x, int P, int Din, double *y) {
  for (int i = 0; i < P; ++i) y[i] = dot_product(W + (size_t)i * (size_t)Din, x, Din);
}

static double dot_double(const double *a, const double *b, int n) {
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += a[i] * b[i];
  return s;
}

int cso_score_projected(const float *Xq, const float *Wq, const float *Xc,
                        const float *Wc, int B, int K, int Dq, int Dc, int P,
                        int similarity, float scale, float temperature,
                        double *p) {
  if (Wq == NULL || Wc == NULL) return CSO_ERR_NULL_POINTER;
  int st = cso_validate(Xq != NULL, Xc != NULL, p != NULL, B, K, Dq, similarity,
                        scale, temperature);
  if (st != CSO_OK) return st;
  if (Dc <= 0 || P <= 0) return CSO_ERR_D_RANGE;
  double *q = (double *)malloc(sizeof(double) * (size_t)P);
  double *c = (double *)malloc(sizeof(double) * (size_t)P);
  if (q == NULL || c == NULL) {
    free(q);
    free(c);
    return CSO_ERR_D_RANGE;
  }
  for (int b = 0; b < B; ++b) {
    double *pb = p + (size_t)b * (size_t)K;
    project(Wq, Xq + (size_t)b * (size_t)Dq, P, Dq, q);
    double qnorm = sqrt(dot_double(q, q, P));
    if (qnorm < CSO_NORM_EPS) qnorm = CSO_NORM_EPS;
    for (int k = 0; k < K; ++k) {
      project(Wc, Xc + ((size_t)b * (size_t)K + (size_t)k) * (size_t)Dc, P, Dc, c);
      double s = dot_double(c, q, P);
      if (similarity == CSO_SIM_COSINE) {
        double cnorm = sqrt(dot_double(c, c, P));
        if (cnorm < CSO_NORM_EPS) cnorm = CSO_NORM_EPS;
        s = s / (qnorm * cnorm);
      }
      pb[k] = (double)scale * s / (double)temperature;
    }
    softmax_in_place(pb, K);
  }
  free(q);
  free(c);
  return CSO_OK;
}
