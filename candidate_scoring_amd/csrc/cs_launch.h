// cs_launch.h -- internal interface between the C ABI (cs_api.cpp) and the
// kernels (cs_kernels.hip). Not installed, not part of the ABI.
#ifndef CS_LAUNCH_H
#define CS_LAUNCH_H

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

namespace cs {

// Everything a scoring kernel reads. Pointers are device pointers.
struct KernelArgs {
  const float* Q;      // [B][D]
  const float* C;      // [B][K][D]
  float* out;          // [B][K]
  float2* partials;    // [B][G] (max, sum) per slice; used when G > 1
  unsigned* tickets;   // [B] arrival counters, zero at rest; used when G > 1
  int B, K, D;
  int G;               // slices (workgroups) per question
  int rpg;             // candidates per slice: slice g owns [g*rpg, min(K,(g+1)*rpg))
  float zscale;        // scale / temperature, rounded once to fp32
  int cosine;          // 1: cosine similarity, 0: dot product
  const float* staged_norms;  // unfused baseline: [B][K] row norms from a separate pass
  const long long* offsets;   // ragged batch: [B+1] row offsets (device); else nullptr
  long long total_rows;       // ragged batch: rows of C and out
  int* status;                // ragged batch: optional device status word
  int longest_first;          // ragged batch: dispatch questions by decreasing count
};

struct LaunchShape {
  unsigned grid;   // workgroups (items are strided over them)
  unsigned block;  // threads per workgroup, a multiple of 64, <= 256
  int nv;          // > 0: register-query kernel with this many 16-byte pieces per lane
  int vec;         // general kernel: 4 (16-byte pieces) or 1 (scalar)
  int nt;          // 1: load candidates non-temporally (streamed, larger than L2)
  int units;       // compute units of the device (persistent grids); 0 if unknown
};

// Workgroups of the persistent kernel that a dense, unsplit call with this
// shape launches (a.B, a.K, a.D, a.G, a.cosine, a.offsets, a.staged_norms
// are read); 0 when it launches one workgroup per question instead (few or
// short questions, no device to ask, or another path).
unsigned stream_grid(const KernelArgs& a, const LaunchShape& ls);

// Rows per wave of the register-query kernel for a given nv.
int regq_rows_per_wave(int nv);
// Smallest instantiated nv covering D (D % 4 == 0); 0 if D is too large.
int regq_nv_for(int D);

hipError_t launch_fused(const KernelArgs& a, const LaunchShape& ls, hipStream_t stream);

// Projection + scoring (bf16 inputs as raw 16-bit patterns).
struct ProjArgs {
  const uint16_t* xq;  // [B][Hq] query hidden states
  const uint16_t* xc;  // [B][K][Hc] candidate hidden states
  const uint16_t* wq;  // [P][Hq] query head
  const uint16_t* wc;  // [P][Hc] candidate head
  float* out;          // [B][K]
  float* qp;           // workspace [B][P]: projected queries
  float* u;            // workspace [B][Hc]: folded queries (dot only)
  uint16_t* parts;     // workspace: bf16 split of q', fragment-packed (dot only)
  uint16_t* wpack;     // workspace: Wc^T, fragment-packed (dot only)
  unsigned* tickets;   // workspace [B]: merge tickets of the split candidate pass
  float2* partials;    // workspace [B][G]: (max, sum) per slice
  int G;               // slices per question of the candidate pass (1: no split)
  int cos_slice;       // cosine: one workgroup per kCosSliceRows candidates of a question
  int cos_parts;       // cosine slices: > 0 splits the P features into this many parts of 64
  float* rowparts;     // workspace [B][256][cos_parts][2]: rows' (dot, |c'|^2) per part
  int B, K, Hq, Hc, P;
  float zscale;        // scale / temperature
  int cosine;
  int nt;              // stream the candidate rows non-temporally
  int compute_units;   // compute units of the current device (persistent grids)
};
// Candidate rows per workgroup of the small-batch cosine kernel.
constexpr int kCosSliceRows = 32;
// Questions up to which a small cosine batch of split questions also splits
// the projected features (the row partials this needs: 8 KiB per question).
constexpr int kCosPartMaxB = 64;
// 16-byte pieces per lane of the bf16 dot kernel for Hc (Hc % 8 == 0); 0 if
// Hc is too large.
int bf16_nv_for(int Hc);
int bf16_rows_per_wave(int nv);
hipError_t launch_projected(const ProjArgs& p, hipStream_t stream);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream);
// Bytes of the per-GPU static split workspace of the entry point that
// allocates nothing (equal to CS_NOALLOC_SCRATCH_BYTES of the C ABI).
constexpr size_t kStaticScratchBytes = 64 * 1024;
// Device address of the current GPU's static split workspace; the first
// call on a device looks it up and enqueues its clearing on `stream`.
hipError_t static_scratch(void** ptr, hipStream_t stream);
// Unfused baseline, first pass: norms[r] = |C row r| for r < rows.
hipError_t launch_row_norms(const float* C, long long rows, int D, int vec, int nt, float* norms,
                            hipStream_t stream);

}  // namespace cs

#endif
