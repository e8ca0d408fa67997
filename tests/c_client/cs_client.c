/* A plain C caller of the scoring library, for the GPU tests: no C++, no
 * Python, only the C ABI of include/candidate_scoring.h and the HIP runtime
 * API for device memory.
 *
 * Usage: cs_client IN OUT
 * IN holds int32 B, K, D, similarity, float32 scale, then Q [B][D] and
 * C [B][K][D] as float32. The client scores the batch on the device twice
 * through cs_score_candidates_batch (without a workspace, then with the
 * planned one), checks that a call with a null query is rejected with
 * CS_ERR_NULL_POINTER, and writes both [B][K] probability arrays to OUT.
 * Exit status 0 on success, 1 on any failure (reported on stderr). */
#include <stdio.h>
#include <stdlib.h>

#include "candidate_scoring.h"

#define CHECK_HIP(expr)                                                   \
  do {                                                                    \
    hipError_t e_ = (expr);                                               \
    if (e_ != hipSuccess) {                                               \
      fprintf(stderr, "%s failed: %s\n", #expr, hipGetErrorString(e_));   \
      return 1;                                                           \
    }                                                                     \
  } while (0)

static int read_exact(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n; }

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: cs_client IN OUT\n");
    return 1;
  }
  FILE* in = fopen(argv[1], "rb");
  if (in == NULL) {
    fprintf(stderr, "cannot open %s\n", argv[1]);
    return 1;
  }
  int32_t hdr[4];
  float scale;
  if (!read_exact(in, hdr, sizeof hdr) || !read_exact(in, &scale, sizeof scale)) {
    fprintf(stderr, "short header\n");
    return 1;
  }
  const int B = hdr[0], K = hdr[1], D = hdr[2], sim = hdr[3];
  if (B < 1 || K < 1 || D < 1) {
    fprintf(stderr, "bad sizes\n");
    return 1;
  }
  const size_t nq = (size_t)B * D, nc = (size_t)B * K * D, np = (size_t)B * K;
  float* hq = (float*)malloc(nq * sizeof(float));
  float* hc = (float*)malloc(nc * sizeof(float));
  float* hp = (float*)malloc(2 * np * sizeof(float));
  if (hq == NULL || hc == NULL || hp == NULL || !read_exact(in, hq, nq * sizeof(float)) ||
      !read_exact(in, hc, nc * sizeof(float))) {
    fprintf(stderr, "short input\n");
    return 1;
  }
  fclose(in);

  float *dq = NULL, *dc = NULL, *dp = NULL;
  void* ws = NULL;
  CHECK_HIP(hipMalloc((void**)&dq, nq * sizeof(float)));
  CHECK_HIP(hipMalloc((void**)&dc, nc * sizeof(float)));
  CHECK_HIP(hipMalloc((void**)&dp, np * sizeof(float)));
  CHECK_HIP(hipMemcpy(dq, hq, nq * sizeof(float), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dc, hc, nc * sizeof(float), hipMemcpyHostToDevice));

  if (cs_abi_version() != CS_ABI_VERSION) {
    fprintf(stderr, "ABI version %d, header %d\n", cs_abi_version(), CS_ABI_VERSION);
    return 1;
  }
  int st = cs_score_candidates_batch(dq, dc, B, K, D, sim, scale, 1.0f, dp, NULL, 0, NULL);
  if (st != CS_OK) {
    fprintf(stderr, "batch call: %s\n", cs_status_string(st));
    return 1;
  }
  CHECK_HIP(hipStreamSynchronize(NULL));
  CHECK_HIP(hipMemcpy(hp, dp, np * sizeof(float), hipMemcpyDeviceToHost));

  const size_t wb = cs_workspace_bytes(B, K, D, sim);
  if (wb > 0) {
    CHECK_HIP(hipMalloc(&ws, wb));
    st = cs_workspace_init(ws, wb, NULL);
    if (st != CS_OK) {
      fprintf(stderr, "workspace init: %s\n", cs_status_string(st));
      return 1;
    }
  }
  st = cs_score_candidates_batch(dq, dc, B, K, D, sim, scale, 1.0f, dp, ws, wb, NULL);
  if (st != CS_OK) {
    fprintf(stderr, "batch call with workspace: %s\n", cs_status_string(st));
    return 1;
  }
  CHECK_HIP(hipStreamSynchronize(NULL));
  CHECK_HIP(hipMemcpy(hp + np, dp, np * sizeof(float), hipMemcpyDeviceToHost));

  st = cs_score_candidates(NULL, dc, K, D, sim, scale, 1.0f, dp, NULL, 0, NULL);
  if (st != CS_ERR_NULL_POINTER) {
    fprintf(stderr, "null query returned %d\n", st);
    return 1;
  }

  FILE* out = fopen(argv[2], "wb");
  if (out == NULL || fwrite(hp, sizeof(float), 2 * np, out) != 2 * np) {
    fprintf(stderr, "cannot write %s\n", argv[2]);
    return 1;
  }
  fclose(out);
  fprintf(stderr, "cs_client: B=%d K=%d D=%d similarity=%d workspace=%zu bytes: ok\n", B, K, D, sim,
          wb);
  CHECK_HIP(hipFree(dq));
  CHECK_HIP(hipFree(dc));
  CHECK_HIP(hipFree(dp));
  if (ws != NULL) CHECK_HIP(hipFree(ws));
  free(hq);
  free(hc);
  free(hp);
  return 0;
}
