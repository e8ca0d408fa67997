/*
 * candidate_scoring.h -- C ABI of the fused candidate-scoring library for
 * AMD Instinct MI355X (gfx950).
 *
 * What it computes. Source: pull request "cuda: add a fused candidate-scoring
 * kernel for CLM and Kev".
 *   For each question b, a query q_b[D] and candidates C_b[K][D] (K <= 255)
 *   give a probability distribution over the K candidates:
 *       z_k = scale * s(q_b, c_bk) / temperature,
 *       p_k = exp(z_k - max_j z_j) / sum_j exp(z_j - max_j z_j),
 *   where s is the cosine similarity (CLM: intro table, "exp(logit_scale) *
 *   cos(...)", so the caller passes scale = exp(logit_scale)) or the plain
 *   dot product (Kev: intro table, scale = 1/sqrt(256)). Cosine clamps each
 *   norm below at 1e-12, so a zero candidate scores exactly 0 and a zero
 *   query gives the uniform distribution. The similarities never reach
 *   global memory ("What is fused, precisely"); a batch is one launch whose
 *   grid covers the questions.
 *
 * Memory and streams. Every pointer argument is a DEVICE pointer owned by
 * the caller ("Defects the GPU found", item 1: host buffers crash the
 * kernel rather than score wrongly). Layouts are row-major and contiguous:
 * queries [B][D], candidates [B][K][D], out [B][K], all fp32. The library
 * allocates nothing per call, keeps no pointer after returning, and enqueues
 * exactly one kernel on the caller's stream without synchronizing, so a
 * call can be captured into a hipGraph as a single node ("Verified on
 * hardware", fourth group). Stream 0 (null stream) is allowed.
 *
 * Errors. Arguments are checked on the host, in a fixed order (pointers,
 * B, K, D, similarity, scale, temperature, workspace), before any HIP call.
 * A rejected call returns a negative status, enqueues nothing and leaves
 * out untouched ("Verified on hardware", third group: K above 255, K of
 * zero, D of zero, a zero scale, a negative temperature and a null query
 * are errors). This library also rejects, as its own reading: B <= 0, null
 * candidates or out, an unknown similarity, a NaN or infinite scale, and a
 * zero, NaN or infinite temperature.
 *
 * Workspace. One-question (and small-batch) calls can spread a question's
 * candidates over several workgroups so the whole chip works on it; the
 * partial softmax results are merged by the last workgroup to finish. That
 * path needs a caller-provided workspace of cs_workspace_bytes() bytes,
 * 8-byte aligned, zeroed once with cs_workspace_init() (outside any graph
 * capture) and left zeroed by every call. Calls that may run at the same
 * time must not share a workspace. With workspace == NULL every question
 * runs in one workgroup; the result is the same distribution.
 *
 * Thread safety: no global mutable state apart from the per-thread last HIP
 * error; calls from several threads are safe given distinct workspaces.
 */
#ifndef CANDIDATE_SCORING_H
#define CANDIDATE_SCORING_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CS_ABI_VERSION 1
/* At most 255 candidates per question ("What is fused, precisely"). */
#define CS_MAX_K 255

/* Similarity selector: CS_SIM_DOT is Kev's scaled dot product,
 * CS_SIM_COSINE is CLM's scaled cosine ("normalize" cases, defect 2). */
#define CS_SIM_DOT 0
#define CS_SIM_COSINE 1

/* Status codes. */
#define CS_OK 0
#define CS_ERR_NULL_POINTER (-1) /* query (page), candidates or out (reading) is NULL */
#define CS_ERR_K_RANGE (-2)      /* K < 1 or K > 255 (page) */
#define CS_ERR_D_RANGE (-3)      /* D < 1 (page) */
#define CS_ERR_SCALE (-4)        /* scale == 0 (page), NaN or infinite, or scale /
                                    temperature beyond the fp32 range (reading) */
#define CS_ERR_TEMPERATURE (-5)  /* temperature < 0 (page), 0, NaN or infinite (reading) */
#define CS_ERR_BATCH (-6)        /* B < 1 (reading) */
#define CS_ERR_SIMILARITY (-7)   /* similarity is neither CS_SIM_DOT nor CS_SIM_COSINE */
#define CS_ERR_WORKSPACE (-8)    /* workspace too small or not 8-byte aligned; bad groups */
#define CS_ERR_LAUNCH (-9)       /* the kernel launch failed; see cs_last_hip_error() */
#define CS_ERR_HOST_POINTER (-10) /* only with CS_DEBUG_POINTERS=1: a pointer is not device memory */
#define CS_ERR_UNSUPPORTED (-11) /* valid sizes this entry point does not implement (see its comment) */

/* Returns CS_ABI_VERSION: 1, the abi_version the page's manifest records
 * ("The manifest, and CI"). */
int cs_abi_version(void);

/* Static, human-readable text for a status code (never NULL). The codes are
 * the rejections of "Verified on hardware", third group, and this library's
 * readings listed above. */
const char *cs_status_string(int status);

/* The hipError_t of this thread's last CS_ERR_LAUNCH (0 if none). The
 * library's own addition: the page names no launch-failure code. */
int cs_last_hip_error(void);

/* Workspace bytes the planned launch needs for B questions of K candidates
 * of length D with the given similarity; 0 when that plan runs one
 * workgroup per question and needs none. Invalid sizes return 0. The
 * workspace serves the whole-chip split of small batches: the page's own
 * finding ("What it is worth") is that one block per question leaves a
 * single question on one compute unit. The similarity is an argument so
 * that every size function validates the same argument set as the call. */
size_t cs_workspace_bytes(int B, int K, int D, int similarity);

/* Workspace bytes for an explicit number of workgroups per question (for
 * cs_score_candidates_batch_groups()). */
size_t cs_workspace_bytes_for_groups(int B, int groups);

/* Zero `bytes` bytes of `workspace` with a kernel on `stream` (no memset
 * node, no synchronization, so it may also be captured: "Verified on
 * hardware", fourth group, asks that calls capture cleanly). Returns CS_OK,
 * CS_ERR_NULL_POINTER or CS_ERR_LAUNCH. */
int cs_workspace_init(void *workspace, size_t bytes, hipStream_t stream);

/* Workgroups per question that cs_score_candidates_batch() would launch for
 * these sizes, with (has_workspace != 0) or without a workspace. Both entry
 * points use this same pure function, so a single-question call and a
 * batch of one pick the same kernel and give bitwise the same result (the
 * agreement "Verified on hardware", second group, asks for). The planned
 * count depends on the current device's compute-unit count. */
int cs_plan_groups(int B, int K, int D, int similarity, int has_workspace);

/* The launch cs_score_candidates_batch() would make for these sizes on the
 * current device: grid (workgroups), block (threads) and workgroups per
 * question, for pointers that are (aligned16 != 0) or are not 16-byte
 * aligned. A dense batch of more questions than compute units, one
 * workgroup per question, of 64 candidates or more each, runs a persistent
 * grid of the workgroups the device holds at once; without a device to
 * ask, grid is the
 * one-workgroup-per-question count. Returns CS_OK or a size-validation
 * status. For benches that time a matching empty kernel: the launch-bound
 * floor of "What it is worth", graph paragraph. */
int cs_plan_launch(int B, int K, int D, int similarity, int has_workspace, int aligned16,
                   unsigned *grid, unsigned *block, int *groups);

/* Writes to name (name_bytes long, NUL-terminated) a description of the
 * kernel instantiation cs_score_candidates_batch() launches for these sizes:
 * kernel, similarity, pieces per lane and rows per wave, cached or
 * non-temporal loads, split, one workgroup per question, or a persistent
 * grid (as cs_plan_launch() decides). For reports that label measurements
 * by the code that ran. Returns CS_OK, a size-validation status,
 * CS_ERR_NULL_POINTER, or CS_ERR_WORKSPACE if name_bytes is too short. */
int cs_plan_kernel(int B, int K, int D, int similarity, int has_workspace, int aligned16,
                   char *name, size_t name_bytes);

/* One question: query [D], candidates [K][D], out [K] (device, fp32).
 * Equivalent to cs_score_candidates_batch() with B = 1, bitwise.
 * Source: pull request "cuda: add a fused candidate-scoring kernel for CLM and Kev", "Verified on hardware", second group (the single-question
 * entry point, which must agree with the batch path) and fourth group (a
 * call queues on the caller's stream, never synchronizes, and captures as
 * one graph node that replays to the same result); "What is fused,
 * precisely" for what is computed. */
int cs_score_candidates(const float *query, const float *candidates, int K, int D,
                        int similarity, float scale, float temperature, float *out,
                        void *workspace, size_t workspace_bytes, hipStream_t stream);

/* B independent questions in one launch: queries [B][D], candidates
 * [B][K][D], out [B][K] (device, fp32). Source: pull request "cuda: add a fused candidate-scoring kernel for CLM and Kev", "Verified on
 * hardware", second group (the batch entry point: batches of 1, 8, 4 and 3
 * questions agree with single calls) and fourth group (one graph node,
 * replayed exactly); "What is fused, precisely" (a batch is a grid over
 * questions). */
int cs_score_candidates_batch(const float *queries, const float *candidates, int B, int K,
                              int D, int similarity, float scale, float temperature,
                              float *out, void *workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* As cs_score_candidates_batch(), with the number of workgroups per
 * question given explicitly (1 <= groups <= K; groups > 1 needs a workspace
 * of cs_workspace_bytes_for_groups(B, groups) bytes; a count that would
 * leave a slice empty is CS_ERR_WORKSPACE). For tuning and tests; the
 * distribution does not depend on groups beyond fp32 rounding. */
int cs_score_candidates_batch_groups(const float *queries, const float *candidates, int B,
                                     int K, int D, int similarity, float scale,
                                     float temperature, float *out, void *workspace,
                                     size_t workspace_bytes, int groups, hipStream_t stream);

/* For callers that cannot allocate device memory (code under hipGraph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call, plan and result as cs_score_candidates_batch() with a workspace of
 * cs_workspace_bytes() bytes, but the split path's workspace is a static
 * array of CS_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU,
 * held until the process ends. Neither this call nor its set-up calls
 * hipMalloc, hipFree or any allocating routine. The first call on each
 * device looks up that device's array and enqueues one extra kernel on
 * `stream` that clears it; every call leaves it zero again. All calls on one
 * GPU share the array, so calls that may overlap in time on one GPU (other
 * streams, other threads) race and must not be issued. A plan whose
 * workspace would exceed CS_NOALLOC_SCRATCH_BYTES returns CS_ERR_WORKSPACE
 * (the planner never makes one: split plans hold at most one slice per
 * compute unit). Errors and validation as cs_score_candidates_batch(). */
#define CS_NOALLOC_SCRATCH_BYTES (64 * 1024)
int cs_score_candidates_batch_noalloc(const float *queries, const float *candidates, int B,
                                      int K, int D, int similarity, float scale,
                                      float temperature, float *out, hipStream_t stream);

/* Ragged batch: B questions with their own candidate counts, one launch
 * (pull request "cuda: add a fused candidate-scoring kernel for CLM and
 * Kev", "Verified on hardware", second group: batches of 1, 8, 4 and 3
 * questions with K up to 255). Question b owns candidate rows
 * offsets[b] .. offsets[b+1]-1 of candidates [total_rows][D] and the same
 * slots of out [total_rows]; queries is [B][D]. offsets is a DEVICE array
 * of B+1 int64 values with offsets[0] = 0 and offsets[B] = total_rows; each
 * count must lie in 1..255 (the per-question limit of "What is fused,
 * precisely").
 * The host checks pointers (offsets included), B, total_rows in
 * [B, 255*B] (else CS_ERR_K_RANGE), D, similarity, scale and temperature,
 * then the workspace; it cannot read device offsets without synchronizing,
 * so each workgroup checks its own question: a question whose offsets fall
 * outside [0, total_rows] or whose count is outside 1..255 is skipped, its
 * output slots are left untouched, and CS_ERR_K_RANGE is stored to *status
 * (a DEVICE int the caller sets to CS_OK beforehand; may be NULL). Each
 * valid question's result equals cs_score_candidates() on its own rows.
 * Workspace: as for cs_score_candidates_batch(), optional, 8-byte aligned,
 * zeroed once with cs_workspace_init() and left zeroed by every call, not
 * shared by calls that may overlap. With one of cs_ragged_workspace_bytes()
 * bytes, a small batch cuts every question into slices of the same number
 * of rows (planned from the mean count total_rows / B), spread over the
 * compute units and merged by the last slice of each question; without one,
 * or when that size is 0, every question runs in one workgroup. */
int cs_score_candidates_ragged(const float *queries, const float *candidates,
                               const int64_t *offsets, int B, int64_t total_rows, int D,
                               int similarity, float scale, float temperature, float *out,
                               int *status, void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Workspace bytes a ragged call with these sizes uses: 0 when it runs one
 * workgroup per question. Invalid sizes return 0. */
size_t cs_ragged_workspace_bytes(int B, int64_t total_rows, int D, int similarity);

/* The slicing cs_score_candidates_ragged() plans, with (has_workspace != 0)
 * or without a workspace: rows per slice, and the most slices one question
 * (255 rows) takes; a question of K_b rows takes ceil(K_b / rows_per_slice)
 * slices. max_slices 1: one workgroup per question. Returns CS_OK or a
 * size-validation status (as the call would). */
int cs_plan_ragged(int B, int64_t total_rows, int D, int similarity, int has_workspace,
                   int *rows_per_slice, int *max_slices);

/* Projection + scoring: the caller-side heads fused with the scoring
 * (intro table of the page: CLM's state_head / action_head ahead of the
 * cosine, Kev's q() / k() ahead of the dot with scale 1/sqrt(256)). Each head
 * is a linear map without bias: q'_b = Wq x_q[b] (P features from Hq) and
 * c'_bk = Wc x_c[b][k] (P features from Hc); the result is the softmax of
 * scale * s(q'_b, c'_bk) / temperature over each question's K candidates, as
 * cs_score_candidates_batch() would give on the projected vectors.
 * All inputs are bf16 (raw 16-bit patterns) in DEVICE memory, row-major:
 * xq [B][Hq], xc [B][K][Hc], wq [P][Hq], wc [P][Hc]; out [B][K] is fp32.
 * Accumulation is fp32. For dot, the candidate head is folded into the query
 * (c' . q' = x . (Wc^T q')), so candidates are read once and never projected;
 * for cosine, each question's projected candidates are computed on the
 * matrix cores and reduced to their similarity in registers. The workspace
 * (cs_projected_workspace_bytes(), 16-byte aligned) holds the projected
 * queries, the merge state of the candidate pass (which a small batch
 * spreads over several workgroups per question; for cosine batches of up
 * to 64 questions also each row's partial sums over parts of the projected
 * features, 8 KiB per question) and, for dot, the folded
 * queries, an exact three-part bf16 split of the projected ones and Wc^T,
 * both in matrix-core fragment order; its contents are scratch between
 * calls (the call initialises what it needs). Implemented shapes: Hq and Hc multiples of 8, P <= 256,
 * 16-byte aligned inputs, P a multiple of 64 for cosine, Hc <= 4096 for dot;
 * other valid sizes return CS_ERR_UNSUPPORTED. Enqueues two (cosine) or
 * three (dot) kernels on `stream`. */
size_t cs_projected_workspace_bytes(int B, int Hc, int P, int similarity);
int cs_score_projected(const uint16_t *xq, const uint16_t *xc, const uint16_t *wq,
                       const uint16_t *wc, int B, int K, int Hq, int Hc, int P, int similarity,
                       float scale, float temperature, float *out, void *workspace,
                       size_t workspace_bytes, hipStream_t stream);

/* Unfused baseline for A/B measurement (pull request "cuda: add a fused
 * candidate-scoring kernel for CLM and Kev", "What it is worth": the same
 * block with the row norm loaded from a staged array instead of accumulated
 * beside the dot, plus a separate norm pass; Kev, which needs no norm, runs
 * both kernels too). Enqueues two kernels on `stream`: a pass writing the
 * norm of every candidate row to row_norms [B][K] (device, caller-owned,
 * 4-byte aligned; CS_ERR_WORKSPACE if NULL), then one workgroup per question
 * that loads those norms. Same arguments, checks and result as
 * cs_score_candidates_batch(); C is read twice. */
int cs_score_candidates_unfused(const float *queries, const float *candidates, int B, int K,
                                int D, int similarity, float scale, float temperature,
                                float *out, float *row_norms, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif
