// cs_api.cpp -- the C ABI declared in include/candidate_scoring.h:
// argument validation, launch planning and the one launch per call.
//
// Source: pull request "cuda: add a fused candidate-scoring kernel for CLM
// and Kev", "Verified on hardware": the single-question and batch entry
// points must agree; K above 255, K of zero, D of zero, a zero scale, a
// negative temperature and a null query are errors, not scored answers; the
// call queues on the caller's stream and never synchronizes, and a capture
// of it holds exactly one node.

#include "candidate_scoring.h"

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <cmath>

#include "cs_launch.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kWave = 64;
constexpr int kMaxWaves = 8;       // one workgroup per question: up to 512 threads
constexpr int kMaxSplitWaves = 4;  // a slice of a split question: up to 256 threads
// Slicing model. Spreading a question over G workgroups divides its
// streaming time by G but costs every slice an agent-scope release (an L2
// write-back, which the chip serialises at roughly 20 ns each) plus a merge.
// With a workgroup streaming about 120 GB/s, the time
//   bytes_q / (G * 120 GB/s) + B * G * 20 ns
// is smallest at G* = sqrt(bytes_q / (B * 2400 B)). Measured on MI355X (K =
// 255, D from 512 to 4096, B from 1 to 32, every slice count), the fastest
// counts sit somewhat above G* (fewer rows per slice cut the dependent load
// rounds of each wave), and splitting pays from G* >= 3.5 on (2.5 for
// questions of 1 MB and more). G = 1.2 G*, with its rows per slice rounded
// to whole load rounds and at most one slice workgroup per compute unit
// (plan_slices), is within 9 % of the best measured count at every point
// (B from 1 to 256) and 1.2 % on average; G* itself with a threshold of 5
// lost up to 1.8x (B = 32, D = 1536: one workgroup per question left most
// compute units idle).
constexpr double kSliceBalanceBytes = 2400.0;
constexpr double kSliceScale = 1.2;
// The merge adds about 2 us (release, ticket, acquire, rescale), so a
// question that one 8-wave workgroup streams in less than that (about
// 160 GB/s x 2 us = 320 KB) is never split.
constexpr double kMinSplitBytes = 320.0 * 1024;
// Longest-first scheduling: offsets bytes per workgroup at most 1/32 of a
// mean question's candidate bytes.
constexpr double kRankCostRatio = 32.0;
// Candidate blocks larger than all eight XCD L2 caches together are streamed
// with non-temporal loads.
constexpr double kStreamBytes = 32.0 * 1024 * 1024;
constexpr double kMinUsefulSlices = 3.5;
constexpr double kLargeQuestionBytes = 1.0e6;
constexpr double kMinUsefulSlicesLarge = 2.5;
constexpr int kMaxSlices = 64;
// Compute units assumed when the device cannot be queried (MI355X has 256).
constexpr int kDefaultComputeUnits = 256;
// Grid cap; items beyond it are strided over the resident workgroups.
constexpr long long kGridCap = 1 << 20;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t ticket_bytes(int B) { return align_up(sizeof(uint32_t) * (size_t)B, 256); }

size_t workspace_for(int B, int G) {
  if (G <= 1) return 0;
  return ticket_bytes(B) + sizeof(float) * 2 * (size_t)B * (size_t)G;
}

int validate(const void* q, const void* c, const void* out, long long B, long long K,
             long long D, int sim, float scale, float temperature) {
  if (q == nullptr || c == nullptr || out == nullptr) return CS_ERR_NULL_POINTER;
  if (B < 1) return CS_ERR_BATCH;
  if (K < 1 || K > CS_MAX_K) return CS_ERR_K_RANGE;
  if (D < 1) return CS_ERR_D_RANGE;
  if (sim != CS_SIM_DOT && sim != CS_SIM_COSINE) return CS_ERR_SIMILARITY;
  if (scale == 0.0f || isnan(scale) || isinf(scale)) return CS_ERR_SCALE;
  if (!(temperature > 0.0f) || isinf(temperature)) return CS_ERR_TEMPERATURE;
  // The kernels form every logit with the factor scale / T rounded once to
  // fp32; a quotient beyond the fp32 range would make every logit infinite.
  if (isinf((float)((double)scale / (double)temperature))) return CS_ERR_SCALE;
  return CS_OK;
}

// Optional check (CS_DEBUG_POINTERS=1) that a pointer is device memory.
bool debug_pointers() {
  static const bool on = [] {
    const char* v = getenv("CS_DEBUG_POINTERS");
    return v != nullptr && v[0] == '1';
  }();
  return on;
}

bool is_device_pointer(const void* p) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error of an unknown pointer
    return false;
  }
  return attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged;
}

// Compute units of the current device, queried once per device (0 when the
// query fails: the launchers then fall back to one workgroup per question).
int device_compute_units() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return 0;
  }
  if (dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  if (dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Compute units to plan for: the current device's, or MI355X's 256 when
// there is no device to ask (host-only planning queries).
int planning_compute_units() {
  const int n = device_compute_units();
  return n > 0 ? n : kDefaultComputeUnits;
}

// Slices per question for a candidate pass that streams bytes_q per question
// with waves of R rows each, on a device of `cus` compute units (the shared
// core of both planners; a pure function of its arguments).
int plan_slices(int B, int K, double bytes_q, int R, int cus) {
  if (K == 1) return 1;
  if (bytes_q < kMinSplitBytes) return 1;
  const double g_star = std::sqrt(bytes_q / ((double)B * kSliceBalanceBytes));
  // Large questions pay for splitting earlier: one workgroup per question
  // would leave most compute units idle for a long time.
  const bool large = bytes_q >= kLargeQuestionBytes;
  if (g_star < (large ? kMinUsefulSlicesLarge : kMinUsefulSlices)) return 1;
  int G = std::max(2, std::min({K, kMaxSlices, (int)std::lround(kSliceScale * g_star)}));
  // Whole load rounds: a slice's rows are loaded by up to kMaxSplitWaves
  // waves of R rows each, so rows just past a multiple of that cost a whole
  // further round of latency; the rows per slice are rounded to the nearest
  // multiple (ties down).
  const int per_round = kMaxSplitWaves * R;
  int rpg = (K + G - 1) / G;
  if (rpg > per_round) {
    rpg = std::max(per_round, (rpg + per_round / 2 - 1) / per_round * per_round);
    G = (K + rpg - 1) / rpg;
  }
  // At most one slice workgroup per compute unit: past that, two slices
  // share a unit and the batch took 30-50 % longer.
  G = std::min(G, std::max(1, cus / B));
  if (G < 2) return 1;
  rpg = (K + G - 1) / G;
  return (K + rpg - 1) / rpg;  // no empty slices
}

// fp32 scoring: R of the kernel variant D selects (the general kernel's 4
// when no register-query variant covers D).
int plan_groups(int B, int K, int D, int cus) {
  const int nv = D % 4 == 0 ? cs::regq_nv_for(D) : 0;
  return plan_slices(B, K, 4.0 * (double)K * (double)D, nv > 0 ? cs::regq_rows_per_wave(nv) : 4,
                     cus);
}

// Ragged batches are planned from their mean count: rows per slice as the
// dense planner would cut a question of that many rows, so a question of K_b
// rows takes ceil(K_b / rpg) slices and every slice carries about the same
// work. rpg is at least ceil(255 * B / cus), so even a batch of 255-row
// questions launches no more slice workgroups than compute units, and at
// least ceil(255 / 64), the dense planner's slice limit. max_slices 1: every
// question in one workgroup.
struct RaggedPlan {
  int rpg;
  int max_slices;
};

RaggedPlan plan_ragged(int B, long long total_rows, int D, int cus) {
  const long long mean = std::min<long long>(CS_MAX_K, std::max<long long>(1, total_rows / B));
  const int G = plan_groups(B, (int)mean, D, cus);
  if (G < 2) return {CS_MAX_K, 1};
  int rpg = (int)((mean + G - 1) / G);
  rpg = std::max({rpg, (int)((CS_MAX_K * (long long)B + cus - 1) / cus),
                  (CS_MAX_K + kMaxSlices - 1) / kMaxSlices});
  const int max_slices = (CS_MAX_K + rpg - 1) / rpg;
  if (max_slices < 2) return {CS_MAX_K, 1};
  return {rpg, max_slices};
}

// Launch shape for a validated call: kernel variant from D and alignment,
// up to four waves per workgroup (enough for the slice's rows).
cs::LaunchShape make_shape(int B, int K, int D, int G, int rpg, const void* Q, const void* C) {
  cs::LaunchShape ls;
  const bool aligned16 = (reinterpret_cast<uintptr_t>(Q) & 15u) == 0 &&
                         (reinterpret_cast<uintptr_t>(C) & 15u) == 0;
  const bool vec4 = (D % 4 == 0) && aligned16;
  ls.nv = vec4 ? cs::regq_nv_for(D) : 0;
  ls.vec = vec4 ? 4 : 1;
  ls.nt = 4.0 * (double)B * (double)K * (double)D >= kStreamBytes ? 1 : 0;
  const int rows_per_wave = ls.nv > 0 ? cs::regq_rows_per_wave(ls.nv) : 4;
  const int max_waves = G > 1 ? kMaxSplitWaves : kMaxWaves;
  const int waves = std::max(1, std::min(max_waves, (rpg + rows_per_wave - 1) / rows_per_wave));
  ls.block = (unsigned)(waves * kWave);
  ls.grid = (unsigned)std::min<long long>((long long)B * G, kGridCap);
  ls.units = device_compute_units();
  return ls;
}

// ws_in_library: the workspace is the library's own static array (the entry
// point that allocates nothing), which the debug pointer check skips.
int score(const float* Q, const float* C, int B, int K, int D, int sim, float scale,
          float temperature, float* out, void* ws, size_t ws_bytes, int groups,
          hipStream_t stream, bool ws_in_library = false) {
  int st = validate(Q, C, out, B, K, D, sim, scale, temperature);
  if (st != CS_OK) return st;
  if (groups < 1 || groups > K) return CS_ERR_WORKSPACE;
  const int rpg = (K + groups - 1) / groups;
  const int G = (K + rpg - 1) / rpg;
  if (G != groups) return CS_ERR_WORKSPACE;  // would leave a slice empty
  if (G > 1) {
    if (ws == nullptr || ws_bytes < workspace_for(B, G) ||
        (reinterpret_cast<uintptr_t>(ws) & 7u) != 0)
      return CS_ERR_WORKSPACE;
  }
  if (debug_pointers()) {
    if (!is_device_pointer(Q) || !is_device_pointer(C) || !is_device_pointer(out) ||
        (G > 1 && !ws_in_library && !is_device_pointer(ws)))
      return CS_ERR_HOST_POINTER;
  }

  cs::KernelArgs a{};  // zero: no staged norms, no offsets
  a.Q = Q;
  a.C = C;
  a.out = out;
  a.tickets = G > 1 ? static_cast<unsigned*>(ws) : nullptr;
  a.partials = G > 1 ? reinterpret_cast<float2*>(static_cast<char*>(ws) + ticket_bytes(B))
                     : nullptr;
  a.B = B;
  a.K = K;
  a.D = D;
  a.G = G;
  a.rpg = rpg;
  // scale / T rounded once to fp32 from the exact double quotient.
  a.zscale = (float)((double)scale / (double)temperature);
  a.cosine = sim == CS_SIM_COSINE;
  a.staged_norms = nullptr;

  const cs::LaunchShape ls = make_shape(B, K, D, G, rpg, Q, C);
  const hipError_t err = cs::launch_fused(a, ls, stream);
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return CS_ERR_LAUNCH;
  }
  return CS_OK;
}

// Unfused baseline: a norm pass stages |c_k| in `norms`, then the scoring
// kernel (one workgroup per question) loads it instead of accumulating it.
int score_unfused(const float* Q, const float* C, int B, int K, int D, int sim, float scale,
                  float temperature, float* out, float* norms, hipStream_t stream) {
  int st = validate(Q, C, out, B, K, D, sim, scale, temperature);
  if (st != CS_OK) return st;
  if (norms == nullptr || (reinterpret_cast<uintptr_t>(norms) & 3u) != 0) return CS_ERR_WORKSPACE;
  if (debug_pointers()) {
    if (!is_device_pointer(Q) || !is_device_pointer(C) || !is_device_pointer(out) ||
        !is_device_pointer(norms))
      return CS_ERR_HOST_POINTER;
  }
  cs::KernelArgs a{};  // zero: no staged norms, no offsets
  a.Q = Q;
  a.C = C;
  a.out = out;
  a.tickets = nullptr;
  a.partials = nullptr;
  a.B = B;
  a.K = K;
  a.D = D;
  a.G = 1;
  a.rpg = K;
  a.zscale = (float)((double)scale / (double)temperature);
  a.cosine = sim == CS_SIM_COSINE;
  a.staged_norms = norms;
  const cs::LaunchShape ls = make_shape(B, K, D, 1, K, Q, C);
  hipError_t err = cs::launch_row_norms(C, (long long)B * K, D, ls.vec, ls.nt, norms, stream);
  if (err == hipSuccess) err = cs::launch_fused(a, ls, stream);
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return CS_ERR_LAUNCH;
  }
  return CS_OK;
}

// Ragged batch: question b owns rows offsets[b] .. offsets[b+1]-1 of C and
// out; one workgroup per question, which checks its own offsets.
int score_ragged(const float* Q, const float* C, const long long* offsets, int B,
                 long long total_rows, int D, int sim, float scale, float temperature, float* out,
                 int* status, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (offsets == nullptr) return CS_ERR_NULL_POINTER;
  int st = validate(Q, C, out, B, 1, D, sim, scale, temperature);
  if (st != CS_OK) return st;
  // every question needs 1..255 rows
  if (total_rows < (long long)B || total_rows > (long long)B * CS_MAX_K) return CS_ERR_K_RANGE;
  // A workspace spreads the questions of a small batch over several
  // workgroups each; without one (or for a large batch) one per question.
  const RaggedPlan plan = ws != nullptr ? plan_ragged(B, total_rows, D, planning_compute_units())
                                        : RaggedPlan{CS_MAX_K, 1};
  const bool split = plan.max_slices > 1;
  if (split && (ws_bytes < workspace_for(B, plan.max_slices) ||
                (reinterpret_cast<uintptr_t>(ws) & 7u) != 0))
    return CS_ERR_WORKSPACE;
  if (debug_pointers()) {
    if (!is_device_pointer(Q) || !is_device_pointer(C) || !is_device_pointer(out) ||
        !is_device_pointer(offsets) || (status != nullptr && !is_device_pointer(status)) ||
        (split && !is_device_pointer(ws)))
      return CS_ERR_HOST_POINTER;
  }
  cs::KernelArgs a{};
  a.Q = Q;
  a.C = C;
  a.out = out;
  a.B = B;
  a.K = CS_MAX_K;  // upper bound; each question's own count comes from offsets
  a.D = D;
  a.G = plan.max_slices;
  a.rpg = plan.rpg;
  a.tickets = split ? static_cast<unsigned*>(ws) : nullptr;
  a.partials = split ? reinterpret_cast<float2*>(static_cast<char*>(ws) + ticket_bytes(B))
                     : nullptr;
  a.zscale = (float)((double)scale / (double)temperature);
  a.cosine = sim == CS_SIM_COSINE;
  a.offsets = offsets;
  a.total_rows = total_rows;
  a.status = status;
  // More questions than resident workgroups (one 8-wave workgroup per CU):
  // hand out the largest questions first so the batch ends evenly. Deriving
  // that order costs every workgroup one pass over the B+1 offsets, so it is
  // used only while that pass is small next to a question's own rows.
  const double mean_question_bytes = 4.0 * (double)total_rows / (double)B * (double)D;
  a.longest_first = (!split && B > planning_compute_units() &&
                     8.0 * (double)B * kRankCostRatio <= mean_question_bytes)
                        ? 1
                        : 0;
  // launch shape as for a dense batch of the same total size
  const int mean_k = (int)std::max<long long>(1, std::min<long long>(CS_MAX_K, total_rows / B));
  cs::LaunchShape ls = make_shape(B, mean_k, D, plan.max_slices, plan.rpg, Q, C);
  ls.nt = 4.0 * (double)total_rows * (double)D >= kStreamBytes ? 1 : 0;
  const hipError_t err = cs::launch_fused(a, ls, stream);
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return CS_ERR_LAUNCH;
  }
  return CS_OK;
}

// Projected-query workspace: q' [B][P] fp32 and the candidate pass's merge
// state; for dot also u [B][Hc] fp32, the three-part bf16 split of q'
// ([B rounded up to 32][3 * P16], P16 = P rounded up to 16) and Wc^T
// ([Hc rounded up to 32][P16]), both bf16 in matrix-core fragment order.
size_t projected_qp_bytes(int B, int P) {
  return align_up(sizeof(float) * (size_t)B * (size_t)P, 256);
}
size_t projected_u_bytes(int B, int Hc) {
  return align_up(sizeof(float) * (size_t)B * (size_t)Hc, 256);
}
size_t projected_parts_bytes(int B, int P) {
  const size_t p16 = (size_t)(P + 15) / 16 * 16, b32 = (size_t)(B + 31) / 32 * 32;
  return align_up(sizeof(uint16_t) * b32 * 3 * p16, 256);
}
size_t projected_wpack_bytes(int Hc, int P) {
  const size_t p16 = (size_t)(P + 15) / 16 * 16, h32 = (size_t)(Hc + 31) / 32 * 32;
  return align_up(sizeof(uint16_t) * h32 * p16, 256);
}
// The candidate pass's merge tickets and slice partials, sized for the most
// slices any call plans, so the size does not depend on K.
size_t projected_split_bytes(int B) {
  return ticket_bytes(B) + align_up(sizeof(float) * 2 * (size_t)B * (size_t)kMaxSlices, 256);
}
// Cosine batches small enough to split the projected features as well: each
// row's (dot, squared norm) per 64-feature part.
size_t projected_rowpart_bytes(int B, int P) {
  if (B > cs::kCosPartMaxB) return 0;
  return align_up(sizeof(float) * 2 * (size_t)B * 256 * (size_t)((P + 63) / 64), 256);
}
size_t projected_workspace(int B, int Hc, int P, int sim) {
  size_t bytes = projected_qp_bytes(B, P) + projected_split_bytes(B);
  if (sim == CS_SIM_DOT)
    bytes += projected_u_bytes(B, Hc) + projected_parts_bytes(B, P) + projected_wpack_bytes(Hc, P);
  else
    bytes += projected_rowpart_bytes(B, P);
  return bytes;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int score_projected(const uint16_t* xq, const uint16_t* xc, const uint16_t* wq,
                    const uint16_t* wc, int B, int K, int Hq, int Hc, int P, int sim, float scale,
                    float temperature, float* out, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  if (wq == nullptr || wc == nullptr) return CS_ERR_NULL_POINTER;
  int st = validate(xq, xc, out, B, K, Hq, sim, scale, temperature);
  if (st != CS_OK) return st;
  if (Hc < 1 || P < 1) return CS_ERR_D_RANGE;
  // Shapes this path implements: 16-byte bf16 pieces, at most 256 projected
  // features; cosine tiles the features by 64, dot holds a folded query of at
  // most 4096 floats per lane set.
  if (Hq % 8 != 0 || Hc % 8 != 0 || P > 256 || !aligned16(xq) || !aligned16(xc) ||
      !aligned16(wq) || !aligned16(wc))
    return CS_ERR_UNSUPPORTED;
  if (sim == CS_SIM_COSINE ? (P % 64 != 0) : (cs::bf16_nv_for(Hc) == 0)) return CS_ERR_UNSUPPORTED;
  if (ws == nullptr || ws_bytes < projected_workspace(B, Hc, P, sim) || !aligned16(ws))
    return CS_ERR_WORKSPACE;
  if (debug_pointers()) {
    if (!is_device_pointer(xq) || !is_device_pointer(xc) || !is_device_pointer(wq) ||
        !is_device_pointer(wc) || !is_device_pointer(out) || !is_device_pointer(ws))
      return CS_ERR_HOST_POINTER;
  }
  cs::ProjArgs p{};
  p.xq = xq;
  p.xc = xc;
  p.wq = wq;
  p.wc = wc;
  p.out = out;
  char* const base = static_cast<char*>(ws);
  p.qp = reinterpret_cast<float*>(base);
  p.tickets = reinterpret_cast<unsigned*>(base + projected_qp_bytes(B, P));
  p.partials = reinterpret_cast<float2*>(reinterpret_cast<char*>(p.tickets) + ticket_bytes(B));
  p.u = reinterpret_cast<float*>(reinterpret_cast<char*>(p.tickets) + projected_split_bytes(B));
  p.parts = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(p.u) + projected_u_bytes(B, Hc));
  p.wpack = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(p.parts) +
                                        projected_parts_bytes(B, P));
  // (Cosine uses no folded query: its row partials take that place.)
  p.rowparts = p.u;
  // Small batches spread each question's candidate pass over several
  // workgroups. Dot streams 2*K*Hc bytes per question and is planned like
  // the fp32 path. Cosine takes one workgroup per 32 candidates while the
  // batch is small, since each merge costs a few microseconds of ticket
  // round trips and the tile kernel (one workgroup per question, the next
  // question's loads in flight) wins beyond that:
  // * no question split (K <= 32): up to one workgroup per compute unit;
  // * split questions also split the projected features into parts, so a
  //   workgroup streams 64 or 128 rows of the candidate head instead of all
  //   P. 64-feature parts up to half the compute units: one question of
  //   255 x 512 -> 256 took 10.8 us against 13.2 us, four 13.2 against
  //   14.2 (eight, with 256 workgroups, 17.7 against 16.0). Else 128-feature
  //   parts up to three quarters of them: five questions 13.6 against 15.3,
  //   eight 14.9 against 16.5, nine 14.8 against 16.5 on the tile kernel,
  //   twelve 16.1-16.4 against 16.5 (sixteen, 256 workgroups, 18.7 against
  //   16.6);
  // * else whole-feature slices up to a quarter of the compute units.
  // The query projection zeroes the tickets first, so the workspace needs
  // no preparation by the caller.
  const int cus = planning_compute_units();
  const int cos_slices = (K + cs::kCosSliceRows - 1) / cs::kCosSliceRows;
  const long long slice_groups = (long long)B * cos_slices;
  p.cos_slice = 0;
  p.cos_parts = 0;
  if (sim == CS_SIM_COSINE) {
    const bool fits = B <= cs::kCosPartMaxB;  // the workspace holds its row partials
    const int parts64 = P / 64, parts128 = P % 128 == 0 && P / 128 >= 2 ? P / 128 : 0;
    if (cos_slices == 1) {
      p.cos_slice = slice_groups <= cus ? 1 : 0;
    } else if (fits && parts64 >= 2 && slice_groups * parts64 <= cus / 2) {
      p.cos_slice = 1;
      p.cos_parts = parts64;
    } else if (fits && parts128 > 0 && slice_groups * parts128 <= 3LL * cus / 4) {
      p.cos_slice = 1;
      p.cos_parts = parts128;
    } else if (slice_groups <= cus / 4) {
      // P = 64 is a single part (the same merge); P = 192 whole-feature slices.
      p.cos_slice = 1;
      p.cos_parts = fits && parts64 == 1 ? 1 : 0;
    }
  }
  p.G = sim == CS_SIM_DOT ? plan_slices(B, K, 2.0 * (double)K * (double)Hc,
                                        cs::bf16_rows_per_wave(cs::bf16_nv_for(Hc)), cus)
                          : (p.cos_slice ? cos_slices : 1);
  p.B = B;
  p.K = K;
  p.Hq = Hq;
  p.Hc = Hc;
  p.P = P;
  p.zscale = (float)((double)scale / (double)temperature);
  p.cosine = sim == CS_SIM_COSINE;
  p.nt = 2.0 * (double)B * (double)K * (double)Hc >= kStreamBytes ? 1 : 0;
  p.compute_units = planning_compute_units();
  const hipError_t err = cs::launch_projected(p, stream);
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return CS_ERR_LAUNCH;
  }
  return CS_OK;
}

// The fields of a dense call that the launch selection reads.
cs::KernelArgs plan_args(int B, int K, int D, int G, int similarity) {
  cs::KernelArgs a{};
  a.B = B;
  a.K = K;
  a.D = D;
  a.G = G;
  a.cosine = similarity == CS_SIM_COSINE;
  return a;
}

}  // namespace

extern "C" {

int cs_abi_version(void) { return CS_ABI_VERSION; }

const char* cs_status_string(int status) {
  switch (status) {
    case CS_OK: return "ok";
    case CS_ERR_NULL_POINTER: return "null query, candidates or output pointer";
    case CS_ERR_K_RANGE: return "candidate count K must be in 1..255";
    case CS_ERR_D_RANGE: return "vector length D must be at least 1";
    case CS_ERR_SCALE:
      return "scale must be finite and nonzero, and scale / temperature within the fp32 range";
    case CS_ERR_TEMPERATURE: return "temperature must be finite and positive";
    case CS_ERR_BATCH: return "batch size B must be at least 1";
    case CS_ERR_SIMILARITY: return "similarity must be CS_SIM_DOT or CS_SIM_COSINE";
    case CS_ERR_WORKSPACE: return "workspace missing, too small or misaligned, or bad group count";
    case CS_ERR_LAUNCH: return "kernel launch failed";
    case CS_ERR_HOST_POINTER: return "a pointer argument is not device memory";
    case CS_ERR_UNSUPPORTED: return "shape or alignment not implemented by this entry point";
    default: return "unknown status";
  }
}

int cs_last_hip_error(void) { return g_last_hip_error; }

int cs_plan_groups(int B, int K, int D, int similarity, int has_workspace) {
  if (validate(&B, &B, &B, B, K, D, similarity, 1.0f, 1.0f) != CS_OK) return 0;
  return has_workspace ? plan_groups(B, K, D, planning_compute_units()) : 1;
}

int cs_plan_launch(int B, int K, int D, int similarity, int has_workspace, int aligned16,
                   unsigned* grid, unsigned* block, int* groups) {
  const int st = validate(&B, &B, &B, B, K, D, similarity, 1.0f, 1.0f);
  if (st != CS_OK) return st;
  const int G = cs_plan_groups(B, K, D, similarity, has_workspace);
  const int rpg = (K + G - 1) / G;
  // 16-byte aligned or deliberately misaligned dummy addresses
  const void* p = reinterpret_cast<const void*>(uintptr_t(aligned16 ? 256 : 260));
  const cs::LaunchShape ls = make_shape(B, K, D, G, rpg, p, p);
  const unsigned persistent = cs::stream_grid(plan_args(B, K, D, G, similarity), ls);
  if (grid) *grid = persistent > 0 ? persistent : ls.grid;
  if (block) *block = ls.block;
  if (groups) *groups = G;
  return CS_OK;
}

int cs_plan_kernel(int B, int K, int D, int similarity, int has_workspace, int aligned16,
                   char* name, size_t name_bytes) {
  const int st = validate(&B, &B, &B, B, K, D, similarity, 1.0f, 1.0f);
  if (st != CS_OK) return st;
  const int G = cs_plan_groups(B, K, D, similarity, has_workspace);
  if (name == nullptr || name_bytes == 0) return CS_ERR_NULL_POINTER;
  const int rpg = (K + G - 1) / G;
  const void* p = reinterpret_cast<const void*>(uintptr_t(aligned16 ? 256 : 260));
  const cs::LaunchShape ls = make_shape(B, K, D, G, rpg, p, p);
  const unsigned persistent = cs::stream_grid(plan_args(B, K, D, G, similarity), ls);
  const char* sim = similarity == CS_SIM_COSINE ? "cosine" : "dot";
  const char* nt = ls.nt ? "non-temporal" : "cached";
  const char* mode = G > 1 ? "split" : "one workgroup per question";
  int n;
  if (persistent > 0)
    n = snprintf(name, name_bytes,
                 "fused_regq_stream<%s, %d pieces/lane, %d rows/wave, %s, %s, %u workgroups over "
                 "the questions>",
                 sim, ls.nv, cs::regq_rows_per_wave(ls.nv),
                 D / 4 == ls.nv * 64 ? "full" : "partial", nt, persistent);
  else if (ls.nv > 0)
    n = snprintf(name, name_bytes, "fused_regq<%s, %d pieces/lane, %d rows/wave, %s, %s, %s>",
                 sim, ls.nv, cs::regq_rows_per_wave(ls.nv),
                 D / 4 == ls.nv * 64 ? "full" : "partial", nt, mode);
  else
    n = snprintf(name, name_bytes, "fused_general<%s, %s, %s, %s>", sim,
                 ls.vec == 4 ? "16-byte pieces" : "scalar", nt, mode);
  return n >= 0 && (size_t)n < name_bytes ? CS_OK : CS_ERR_WORKSPACE;
}

size_t cs_workspace_bytes_for_groups(int B, int groups) {
  if (B < 1 || groups < 1) return 0;
  return workspace_for(B, groups);
}

size_t cs_workspace_bytes(int B, int K, int D, int similarity) {
  const int G = cs_plan_groups(B, K, D, similarity, 1);
  return G > 0 ? workspace_for(B, G) : 0;
}

int cs_workspace_init(void* workspace, size_t bytes, hipStream_t stream) {
  if (workspace == nullptr) return CS_ERR_NULL_POINTER;
  const hipError_t err = cs::launch_zero(workspace, bytes, stream);
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return CS_ERR_LAUNCH;
  }
  return CS_OK;
}

int cs_score_candidates_batch_groups(const float* queries, const float* candidates, int B,
                                     int K, int D, int similarity, float scale,
                                     float temperature, float* out, void* workspace,
                                     size_t workspace_bytes, int groups, hipStream_t stream) {
  return score(queries, candidates, B, K, D, similarity, scale, temperature, out, workspace,
               workspace_bytes, groups, stream);
}

int cs_score_candidates_batch(const float* queries, const float* candidates, int B, int K, int D,
                              int similarity, float scale, float temperature, float* out,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = validate(queries, candidates, out, B, K, D, similarity, scale, temperature);
  if (st != CS_OK) return st;
  const int G = workspace != nullptr ? plan_groups(B, K, D, planning_compute_units()) : 1;
  return score(queries, candidates, B, K, D, similarity, scale, temperature, out, workspace,
               workspace_bytes, G, stream);
}

int cs_score_candidates_batch_noalloc(const float* queries, const float* candidates, int B,
                                      int K, int D, int similarity, float scale,
                                      float temperature, float* out, hipStream_t stream) {
  int st = validate(queries, candidates, out, B, K, D, similarity, scale, temperature);
  if (st != CS_OK) return st;
  static_assert(cs::kStaticScratchBytes == CS_NOALLOC_SCRATCH_BYTES, "one scratch size");
  const int G = plan_groups(B, K, D, planning_compute_units());
  if (G <= 1)  // one workgroup per question: no workspace at all
    return score(queries, candidates, B, K, D, similarity, scale, temperature, out, nullptr, 0,
                 1, stream);
  const size_t need = workspace_for(B, G);
  if (need > cs::kStaticScratchBytes) return CS_ERR_WORKSPACE;
  void* ws = nullptr;
  const hipError_t err = cs::static_scratch(&ws, stream);
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return CS_ERR_LAUNCH;
  }
  return score(queries, candidates, B, K, D, similarity, scale, temperature, out, ws, need, G,
               stream, /*ws_in_library=*/true);
}

int cs_score_candidates_unfused(const float* queries, const float* candidates, int B, int K,
                                int D, int similarity, float scale, float temperature,
                                float* out, float* row_norms, hipStream_t stream) {
  return score_unfused(queries, candidates, B, K, D, similarity, scale, temperature, out,
                       row_norms, stream);
}

int cs_score_candidates_ragged(const float* queries, const float* candidates,
                               const int64_t* offsets, int B, int64_t total_rows, int D,
                               int similarity, float scale, float temperature, float* out,
                               int* status, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  static_assert(sizeof(int64_t) == sizeof(long long), "offsets are 64-bit");
  return score_ragged(queries, candidates, reinterpret_cast<const long long*>(offsets), B,
                      (long long)total_rows, D, similarity, scale, temperature, out, status,
                      workspace, workspace_bytes, stream);
}

int cs_plan_ragged(int B, int64_t total_rows, int D, int similarity, int has_workspace,
                   int* rows_per_slice, int* max_slices) {
  int st = validate(&B, &B, &B, B, 1, D, similarity, 1.0f, 1.0f);
  if (st != CS_OK) return st;
  if (total_rows < (int64_t)B || total_rows > (int64_t)B * CS_MAX_K) return CS_ERR_K_RANGE;
  const RaggedPlan plan = has_workspace
                              ? plan_ragged(B, (long long)total_rows, D, planning_compute_units())
                              : RaggedPlan{CS_MAX_K, 1};
  if (rows_per_slice) *rows_per_slice = plan.rpg;
  if (max_slices) *max_slices = plan.max_slices;
  return CS_OK;
}

size_t cs_ragged_workspace_bytes(int B, int64_t total_rows, int D, int similarity) {
  int rpg = 0, slices = 0;
  if (cs_plan_ragged(B, total_rows, D, similarity, 1, &rpg, &slices) != CS_OK) return 0;
  return workspace_for(B, slices);
}

size_t cs_projected_workspace_bytes(int B, int Hc, int P, int similarity) {
  if (B < 1 || Hc < 1 || P < 1 || (similarity != CS_SIM_DOT && similarity != CS_SIM_COSINE))
    return 0;
  return projected_workspace(B, Hc, P, similarity);
}

int cs_score_projected(const uint16_t* xq, const uint16_t* xc, const uint16_t* wq,
                       const uint16_t* wc, int B, int K, int Hq, int Hc, int P, int similarity,
                       float scale, float temperature, float* out, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  return score_projected(xq, xc, wq, wc, B, K, Hq, Hc, P, similarity, scale, temperature, out,
                         workspace, workspace_bytes, stream);
}

int cs_score_candidates(const float* query, const float* candidates, int K, int D,
                        int similarity, float scale, float temperature, float* out,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return cs_score_candidates_batch(query, candidates, 1, K, D, similarity, scale, temperature,
                                   out, workspace, workspace_bytes, stream);
}

}  // extern "C"
