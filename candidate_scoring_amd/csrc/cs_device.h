// cs_device.h -- device-side building blocks shared by the scoring kernels
// (cs_kernels.hip) and the projection kernels (cs_project.hip): wave64
// cross-lane reductions, 16-byte streaming loads, the per-workgroup LDS
// state, the in-workgroup softmax and the split-question merge. Internal;
// not part of the ABI.
//
// Source of what the softmax computes: pull request "cuda: add a fused
// candidate-scoring kernel for CLM and Kev", "What is fused, precisely".
#ifndef CS_DEVICE_H
#define CS_DEVICE_H

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "cs_launch.h"

namespace cs {
namespace {

// Phase clocks: a build with CS_PHASE_CLOCKS defined (libcs_phase.so, a
// measurement build, never the product library) makes thread 0 of each
// workgroup store the 100 MHz device clock at fixed points of a kernel; in
// every other build CS_PHASE and CS_PHASE_IN expand to nothing. Each source
// file keeps its own clock array (region-major, then workgroup, 16 slots).
// Region 0, the scoring kernels and the split merge: 0 start, 1 rows
// reduced (wave 0), 2 after the barrier, 3 softmax stored, 4 release fence
// done, 5 ticket drawn, 6 after the ticket barrier, 7 acquire done (last
// slice), 8 merge factors ready, 9 rescaled and reset, 10 workgroup exit,
// 11-13 wave 0 past a quarter, half and three quarters of the slice's rows.
// Regions 1-3 belong to the dot projection's three launches and list their
// slots where they are stamped.
#ifdef CS_PHASE_CLOCKS
constexpr int kPhaseWorkgroups = 1024;
constexpr int kPhaseSlots = 16;
constexpr int kPhaseRegions = 4;
__device__ unsigned long long g_phase_clk[kPhaseRegions * kPhaseWorkgroups * kPhaseSlots];
#define CS_PHASE_IN(region, slot)                                                         \
  do {                                                                                    \
    if (threadIdx.x == 0 && blockIdx.x < (unsigned)::cs::kPhaseWorkgroups)                \
      ::cs::g_phase_clk[((region) * ::cs::kPhaseWorkgroups + blockIdx.x) *                \
                            ::cs::kPhaseSlots + (slot)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#else
#define CS_PHASE_IN(region, slot) \
  do {                            \
  } while (0)
#endif
#define CS_PHASE(slot) CS_PHASE_IN(0, slot)


constexpr int kWave = 64;
constexpr int kBlock = 512;        // threads per workgroup (upper bound)
constexpr int kMaxSlots = 256;     // LDS logit slots (K <= 255)
constexpr int kMaxK = 255;
constexpr int kStatusBadOffsets = -2;  // the K-range status of the C ABI
constexpr float kNormEps = 1e-12f;   // per-norm clamp of the cosine
constexpr float kNormEps2 = 1e-24f;  // its square, for clamping squared norms

// How a scoring launch maps work items to questions.
//  kDense: B questions of K rows each, every question in a.G slices of
//    a.rpg rows (one slice: the whole question).
//  kRagged: question b owns rows offsets[b] .. offsets[b+1]-1 (read on the
//    device); one work item per question, never split.
//  kRaggedSplit: ragged, with every question cut into slices of a.rpg rows;
//    a.G is the most slices any question can have (255 rows), and question b
//    uses ceil(K_b / a.rpg) of them, merged like a split dense question.
constexpr int kDense = 0;
constexpr int kRagged = 1;
constexpr int kRaggedSplit = 2;

// ---------------------------------------------------------------------------
// Cross-lane primitives (wave64).

// DPP controls (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppRowHalfMirror = 0x141; // lane <-> 7 - lane within 8 lanes
constexpr int kDppRowRor8 = 0x128;       // lane <-> lane ^ 8 within 16 lanes

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Candidate rows are read exactly once; when the block of candidates is far
// larger than the L2 caches, loading them non-temporally keeps them from
// evicting anything useful (the streaming read then runs at the same rate as
// a plain read-only copy kernel).
typedef float v4f_t __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ float4 load4(const float4* p) {
  if constexpr (NT) {
    const v4f_t v = __builtin_nontemporal_load(reinterpret_cast<const v4f_t*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
  } else {
    return *p;
  }
}

template <bool NT>
__device__ __forceinline__ float load1(const float* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

struct OpSum {
  __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};
struct OpMax {
  __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};

// Pairs lanes l and l^32 across two registers: afterwards lanes 0..31 hold
// op(a[l], a[l+32]) and lanes 32..63 hold op(b[l-32], b[l]).
template <class Op>
__device__ __forceinline__ float pair32(float a, float b, Op op) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, a),
                                                  __builtin_bit_cast(unsigned, b), false, false);
  // Copy the two results out before reinterpreting them: bit-casting a
  // vector element in place reads element 0 for both.
  const unsigned r0 = r[0], r1 = r[1];
  return op(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}

// Same for lanes l and l^16: rows 0 and 2 take a, rows 1 and 3 take b.
template <class Op>
__device__ __forceinline__ float pair16(float a, float b, Op op) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, a),
                                                  __builtin_bit_cast(unsigned, b), false, false);
  // Copy the two results out before reinterpreting them: bit-casting a
  // vector element in place reads element 0 for both.
  const unsigned r0 = r[0], r1 = r[1];
  return op(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}

// One halving step inside 16-lane rows through DPP: lanes whose BIT is clear
// keep value i, the others value i + N/2, each combined with its partner's.
template <int CTRL, int BIT, int N, int V, class Op>
__device__ __forceinline__ void halve_dpp(float (&v)[V], int lane, Op op) {
  if constexpr (N >= 2) {
    const bool upper = (lane & BIT) != 0;
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const float lo = v[i], hi = v[i + N / 2];
      const float keep = upper ? hi : lo;
      const float send = upper ? lo : hi;
      v[i] = op(keep, dpp_mov<CTRL>(send));
    }
  } else {
    v[0] = op(v[0], dpp_mov<CTRL>(v[0]));
  }
}

template <int N, int V, class Op>
__device__ __forceinline__ void halve32(float (&v)[V], Op op) {
  if constexpr (N >= 2) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) v[i] = pair32(v[i], v[i + N / 2], op);
  } else {
    v[0] = pair32(v[0], v[0], op);
  }
}

template <int N, int V, class Op>
__device__ __forceinline__ void halve16(float (&v)[V], Op op) {
  if constexpr (N >= 2) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) v[i] = pair16(v[i], v[i + N / 2], op);
  } else {
    v[0] = pair16(v[0], v[0], op);
  }
}

// Reduces V per-lane values (V a power of two, 1..64) over the 64 lanes of
// the wave. On return every lane l holds the reduction of value index
// l / (64 / V). Every value goes through the same lane-pairing sequence
// (32, 16, 8, mirror-4, 2, 1), so the result for a value does not depend
// on its index. Must be called by all 64 lanes.
template <int V, class Op>
__device__ __forceinline__ float wave_reduce_transposed(float (&v)[V], int lane, Op op) {
  static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "V must be a power of two <= 64");
  halve32<(V >= 2 ? V : 1), V>(v, op);
  halve16<(V >= 4 ? V / 2 : 1), V>(v, op);
  halve_dpp<kDppRowRor8, 8, (V >= 8 ? V / 4 : 1), V>(v, lane, op);
  halve_dpp<kDppRowHalfMirror, 4, (V >= 16 ? V / 8 : 1), V>(v, lane, op);
  halve_dpp<kDppQuadXor2, 2, (V >= 32 ? V / 16 : 1), V>(v, lane, op);
  halve_dpp<kDppQuadXor1, 1, (V >= 64 ? V / 32 : 1), V>(v, lane, op);
  return v[0];
}

template <class Op>
__device__ __forceinline__ float wave_allreduce(float x, int lane, Op op) {
  float v[1] = {x};
  return wave_reduce_transposed<1>(v, lane, op);
}

// Workgroup sum in a fixed order (waves 0, 1, ...). Ends with a barrier
// after which `scratch` may be reused.
__device__ __forceinline__ float block_sum(float x, float* scratch, int lane, int wave,
                                           int nwaves) {
  x = wave_allreduce(x, lane, OpSum());
  if (lane == 0) scratch[wave] = x;
  __syncthreads();
  float t = 0.0f;
  for (int w = 0; w < nwaves; ++w) t += scratch[w];
  __syncthreads();
  return t;
}

__device__ __forceinline__ float dot4(float4 a, float4 b, float acc) {
  acc = fmaf(a.x, b.x, acc);
  acc = fmaf(a.y, b.y, acc);
  acc = fmaf(a.z, b.z, acc);
  acc = fmaf(a.w, b.w, acc);
  return acc;
}

// ---------------------------------------------------------------------------
// Per-workgroup state shared by the kernel variants.

struct Lds {
  float dot[kMaxSlots];
  float ss[kMaxSlots];
  float merge[kMaxSlots];
  float red[kBlock / kWave];
  int last;
  int hist[kMaxSlots];        // ragged longest-first order: questions per count
  int wave_sum[kBlock / kWave];
  int pick[2];
  int next_group;             // the next row group of the slice not yet handed out
};

// Where one question's candidates and outputs live: rows row .. row+K-1 of
// C and of out. Dense batches: row = b*K. Ragged batches: the offsets array.
struct Question {
  size_t row;
  int K;
};

// Row groups of a slice are handed to the waves of a workgroup as they go:
// wave w starts with group w, and each wave draws its next group from an LDS
// counter (set to the wave count before the slice) while its current loads
// are in flight. With a fixed share per wave the memory pipeline, which
// serves older waves first, left wave 0 of the fp32 Kev batch done 21 us
// before the last wave of its workgroup, out of a 91 us workgroup; the
// compute unit then streamed with ever fewer waves. Which wave takes a row
// does not change how the row is reduced, so the results do not depend on
// the order.
__device__ __forceinline__ int draw_group(Lds& s, int lane) {
  int g = 0;
  if (lane == 0) g = atomicAdd(&s.next_group, 1);
  return __builtin_amdgcn_readfirstlane(g);
}

// Resolves question b. For a ragged batch the workgroup checks the offsets
// it was given (0 <= lo, hi <= total rows, 1 <= hi - lo <= 255); a bad
// question is skipped, writes nothing, and raises the caller's status word.
template <bool RAGGED>
__device__ __forceinline__ bool resolve_question(const KernelArgs& a, int b, int tid,
                                                 Question& qn) {
  if constexpr (!RAGGED) {
    qn.row = (size_t)b * (size_t)a.K;
    qn.K = a.K;
    return true;
  }
  const long long lo = a.offsets[b], hi = a.offsets[b + 1];
  if (!(lo >= 0 && hi <= a.total_rows && hi - lo >= 1 && hi - lo <= kMaxK)) {
    if (tid == 0 && a.status != nullptr) *a.status = kStatusBadOffsets;
    return false;
  }
  // Uniform across the workgroup; saying so keeps the row addresses in
  // scalar registers.
  const unsigned long long row = (unsigned long long)lo;
  qn.row = (size_t)(((unsigned long long)(unsigned)__builtin_amdgcn_readfirstlane(
                         (int)(row >> 32)) << 32) |
                    (unsigned)__builtin_amdgcn_readfirstlane((int)(row & 0xffffffffu)));
  qn.K = __builtin_amdgcn_readfirstlane((int)(hi - lo));
  return true;
}

// Sort key of a ragged question: 0 for 255 candidates ... 254 for one; an
// invalid count sorts last (its workgroup then flags it).
__device__ __forceinline__ int count_key(const KernelArgs& a, int b) {
  const long long c = a.offsets[b + 1] - a.offsets[b];
  return (c >= 1 && c <= kMaxK) ? kMaxK - (int)c : kMaxK;
}

// Longest-first schedule for a ragged batch larger than the resident
// workgroups: the question of dispatch rank `rank` when questions are
// ordered by decreasing candidate count, ties by index. Every workgroup
// derives the same order from the offsets (a histogram of counts, then the
// rank's position inside its count class), so each question is taken by
// exactly one workgroup. Called by all threads; uses s.hist, s.wave_sum and
// s.pick.
__device__ __forceinline__ int question_of_rank(const KernelArgs& a, int rank, Lds& s, int tid, int lane,
                                int wave) {
  const int nt = blockDim.x, nwaves = nt / kWave;
#pragma unroll 1
  for (int i = tid; i < kMaxSlots; i += nt) s.hist[i] = 0;
  __syncthreads();
#pragma unroll 1
  for (int b = tid; b < a.B; b += nt) atomicAdd(&s.hist[count_key(a, b)], 1);
  __syncthreads();
  // Wave 0 finds the key class holding `rank`: lane l owns keys 4l .. 4l+3,
  // an inclusive scan of the per-lane counts brackets the rank, and the one
  // lane whose bracket holds it walks its four keys.
  if (wave == 0) {
    int c[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = s.hist[4 * lane + i];
      sum += c[i];
    }
    int incl = sum;
    for (int d = 1; d < kWave; d <<= 1) {
      const int v = __shfl_up(incl, d, kWave);
      if (lane >= d) incl += v;
    }
    int before = incl - sum;
    if (rank >= before && rank < incl) {
      int key = 4 * lane;
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        if (rank < before + c[i]) break;
        before += c[i];
        ++key;
      }
      s.pick[0] = key;
      s.pick[1] = rank - before;  // position among the questions with this key
    }
  }
  __syncthreads();
  const int key = s.pick[0], j = s.pick[1];
  // Each thread owns a contiguous run of questions; an exclusive scan of the
  // per-thread match counts finds the run holding the j-th match.
  const int chunk = (a.B + nt - 1) / nt;
  const int lo = min(a.B, tid * chunk), hi = min(a.B, lo + chunk);
  int mine = 0;
#pragma unroll 1
  for (int b = lo; b < hi; ++b) mine += count_key(a, b) == key;
  int incl = mine;
  for (int d = 1; d < kWave; d <<= 1) {
    const int v = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += v;
  }
  if (lane == kWave - 1) s.wave_sum[wave] = incl;
  __syncthreads();
  int before = incl - mine;
#pragma unroll 1
  for (int w = 0; w < wave; ++w) before += s.wave_sum[w];
  if (j >= before && j < before + mine) {
    int seen = before;
#pragma unroll 1
    for (int b = lo; b < hi; ++b) {
      if (count_key(a, b) == key) {
        if (seen == j) s.pick[0] = b;
        ++seen;
      }
    }
  }
  __syncthreads();
  // The pick is the same for every lane; saying so keeps the addresses
  // derived from it in scalar registers.
  const int b = __builtin_amdgcn_readfirstlane(s.pick[0]);
  __syncthreads();
  (void)nwaves;
  return b;
}

// Writes the reduced value of slot `slot` (dot for slots < R, squared norm
// for slots >= R) of the row group starting at candidate k0.
template <bool COS, int R>
__device__ __forceinline__ void store_group(Lds& s, float total, int lane, int k0, int r0,
                                            int r1) {
  constexpr int V = COS ? 2 * R : R;
  constexpr int kLanesPerSlot = kWave / V;
  if ((lane & (kLanesPerSlot - 1)) == 0) {
    const int slot = lane / kLanesPerSlot;
    const int r = slot % R;
    const int k = k0 + r;
    if (k < r1) {
      if (slot < R)
        s.dot[k - r0] = total;
      else
        s.ss[k - r0] = total;
    }
  }
}

// Softmax of this slice's n logits (wave 0 only) and the store of either the
// final probabilities (the question has one slice) or the unnormalised e_k
// plus the slice's (max, sum) partial (partial g of question b at
// b * a.G + g; the question has nslices <= a.G slices). VPL logits per lane (n <= 64 * VPL); the
// slots past n hold -inf and exp 0, which leave the max and the sums
// bitwise unchanged, so every VPL gives the same result.
// MAYSPLIT = false: the caller never splits a question (nslices is 1).
template <bool COS, bool MAYSPLIT, int VPL>
__device__ __forceinline__ void slice_softmax_vpl(const Lds& s, const KernelArgs& a,
                                                  const Question& qn, int b, int g, int r0, int n,
                                                  float zfac, int lane, int nslices) {
  float z[VPL];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int k = lane + kWave * i;
    if (k < n) {
      float v = s.dot[k];
      if (COS) {
        v = v * rsqrtf(fmaxf(s.ss[k], kNormEps2));
      } else if (a.staged_norms != nullptr) {
        // Unfused baseline: the row norm comes from the staged array that a
        // separate pass wrote. The dot-product similarity has no use for it
        // beyond passing on a NaN row, but still pays for loading it.
        const float nrm = a.staged_norms[qn.row + r0 + k];
        v = a.cosine ? v / fmaxf(nrm, kNormEps) : v * (nrm >= 0.0f ? 1.0f : NAN);
      }
      z[i] = v * zfac;
      m = fmaxf(m, z[i]);
    } else {
      z[i] = -INFINITY;
    }
  }
  m = wave_allreduce(m, lane, OpMax());
  float e[VPL];
  float l = 0.0f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int k = lane + kWave * i;
    e[i] = (k < n) ? expf(z[i] - m) : 0.0f;
    l += e[i];
  }
  l = wave_allreduce(l, lane, OpSum());
  float* out = a.out + qn.row + r0;
  if (!MAYSPLIT || nslices == 1) {
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int k = lane + kWave * i;
      if (k < n) out[k] = e[i] / l;
    }
  } else {
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int k = lane + kWave * i;
      if (k < n) out[k] = e[i];
    }
    if (lane == 0) a.partials[(size_t)b * a.G + g] = make_float2(m, l);
  }
}

// A slice of at most 64 candidates (every slice of a split question, and
// small questions) takes one logit per lane: a quarter of the LDS reads and
// exponentials, on the critical path of every split call.
template <bool COS, bool MAYSPLIT = true>
__device__ __forceinline__ void slice_softmax(const Lds& s, const KernelArgs& a, const Question& qn,
                                              int b, int g, int r0, int n, float zfac, int lane,
                                              int nslices) {
  if (n <= kWave)
    slice_softmax_vpl<COS, MAYSPLIT, 1>(s, a, qn, b, g, r0, n, zfac, lane, nslices);
  else
    slice_softmax_vpl<COS, MAYSPLIT, kMaxSlots / kWave>(s, a, qn, b, g, r0, n, zfac, lane,
                                                         nslices);
}

// Called by every thread of a slice's workgroup after slice_softmax, when
// question b has nslices > 1 slices of a.rpg rows (its partials start at
// b * a.G): the last slice to arrive merges.
__device__ __forceinline__ void split_merge(Lds& s, const KernelArgs& a, const Question& qn,
                                            int b, int tid, int lane, int wave, int nslices) {
  // Only wave 0 wrote global memory (e_k and the partial). It publishes them
  // at agent scope (all XCDs: L2 write-back) and draws the ticket; the
  // release fence orders the stores before the relaxed ticket increment.
  if (wave == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    CS_PHASE(4);
    if (lane == 0) {
      const unsigned t = __hip_atomic_fetch_add(a.tickets + b, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
      s.last = (t == (unsigned)(nslices - 1));
    }
    CS_PHASE(5);
  }
  __syncthreads();
  CS_PHASE(6);
  if (!s.last) return;  // uniform across the workgroup
  // Last slice: acquire the other slices' stores (L2 invalidate), fetch the
  // e_k to rescale while wave 0 reads the partials.
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  CS_PHASE(7);
  float* out = a.out + qn.row;
  float ek[kMaxSlots / kWave];
#pragma unroll
  for (int i = 0; i < kMaxSlots / kWave; ++i) {
    const int k = tid + (int)blockDim.x * i;
    ek[i] = (k < qn.K) ? out[k] : 0.0f;
  }
  if (wave == 0) {
    const float2* part = a.partials + (size_t)b * a.G;
    float mg[4], lg[4];
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = lane + kWave * i;
      const float2 v = (g < nslices) ? part[g] : make_float2(-INFINITY, 0.0f);
      mg[i] = v.x;
      lg[i] = v.y;
      M = fmaxf(M, mg[i]);
    }
    M = wave_allreduce(M, lane, OpMax());
    float w[4];
    float L = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = lane + kWave * i;
      w[i] = (g < nslices) ? expf(mg[i] - M) : 0.0f;
      L += lg[i] * w[i];
    }
    L = wave_allreduce(L, lane, OpSum());
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = lane + kWave * i;
      if (g < nslices) s.merge[g] = w[i] / L;
    }
  }
  __syncthreads();
  CS_PHASE(8);
#pragma unroll
  for (int i = 0; i < kMaxSlots / kWave; ++i) {
    const int k = tid + (int)blockDim.x * i;
    if (k < qn.K) out[k] = ek[i] * s.merge[k / a.rpg];
  }
  // Return this question's part of the workspace to zero: its G partials
  // (read above, before the barrier) and its ticket. The ticket array's
  // length depends on B, so a later call with more questions finds its
  // tickets where this call kept partials; those must read as zero.
  for (int g = tid; g < nslices; g += (int)blockDim.x)
    a.partials[(size_t)b * a.G + g] = make_float2(0.0f, 0.0f);
  if (tid == 0) __hip_atomic_store(a.tickets + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  CS_PHASE(9);
}

}  // namespace
}  // namespace cs

#endif
