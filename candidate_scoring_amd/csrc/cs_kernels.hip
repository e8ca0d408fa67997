// cs_kernels.hip -- gfx950 kernels for fused candidate scoring.
//
// Source: pull request "cuda: add a fused candidate-scoring kernel for CLM
// and Kev". "What is fused, precisely": for cosine, a candidate's norm and
// its dot with the query come from the same elements, so both accumulate in
// one read of C; the softmax runs inside the workgroup with no second
// kernel, no atomics and no global buffer for the similarities; K <= 255
// keeps it in one workgroup's LDS; a batch is a grid over questions.
// "Defects the GPU found", item 2: the query norm is reduced once per
// workgroup, never once per wave and then summed again.
//
// Design for CDNA4 (wave64, 256 CUs in 8 XCDs):
//  * Work item = (question b, candidate slice g). A slice is `rpg`
//    consecutive candidates. With one slice per question this is the batch
//    path; with several, the slices of one question run on many CUs and the
//    last slice to finish merges their partial softmax results (below).
//  * A wave owns R consecutive candidate rows at a time. Lane l reads
//    16-byte pieces l, l+64, ... of every row (1 KiB per wave instruction,
//    fully coalesced) and accumulates dot and, for cosine, the squared norm
//    side by side from the same registers: C crosses HBM exactly once.
//    Large candidate blocks are loaded non-temporally (streamed).
//  * For D <= 4096 each wave holds its pieces of q in registers, loaded in
//    the same burst as its first rows; wave 0 reduces |q|^2 once per
//    workgroup. Larger or unaligned D use the general kernel, which stages q
//    through LDS in chunks and reduces |q|^2 once per workgroup there.
//  * The R (or 2R) per-lane partial sums are reduced together with a
//    transposed butterfly: v_permlane32_swap and v_permlane16_swap halve the
//    set across the two 32-lane halves and the 16-lane rows, then DPP steps
//    finish inside rows. Every candidate's sum uses the same pairing tree
//    whatever its slot, so identical candidates give bitwise identical
//    logits (and exactly 1/K).
//  * Logits land in LDS only; wave 0 runs the max-subtracted softmax there
//    and writes each probability once.
//
// Split merge (several slices per question): slice g writes its unnormalised
// e_k = exp(z_k - m_g) into its own part of out and (m_g, l_g) into the
// workspace, publishes them with an agent-scope release, and takes a ticket.
// The slice that draws the last ticket acquires, computes M = max m_g and
// L = sum_g l_g exp(m_g - M) over g in a fixed order (not arrival order), and
// rescales out[k] by exp(m_g - M) / L. It then resets the ticket, so the
// workspace is zero again and graph replays need no reset node. Nothing ever
// waits on another workgroup.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "cs_device.h"
#include "cs_launch.h"

// Split-path workspace of the entry point that allocates nothing: one copy
// per GPU, held until the process ends. In host code this name is only a
// stand-in for the symbol; the device address comes from
// hipGetSymbolAddress (static_scratch below) and is the only form passed to
// kernels or copies. Every call leaves it zero again (the last slice of a
// question clears its ticket and partials), so it is cleared only once per
// device, before its first use.
static __device__ __align__(256) unsigned char scratch[cs::kStaticScratchBytes];

namespace cs {
namespace {

// ---------------------------------------------------------------------------
// Register-query kernel: D % 4 == 0, 16-byte aligned rows, D <= 256 * NV.
// Lane l owns 16-byte pieces l + 64 j (j < NV) of q and of every row. Each
// wave loads its pieces of q straight into registers, in the same burst as
// its first candidate rows, so no separate staging round trip precedes the
// hot loop; the query's squared norm is reduced once per workgroup (by wave
// 0, which holds all of q) right before the softmax.

template <bool COS, int NV, int R, bool FULL, bool NT, int MODE, bool DRAWN>
__global__ __launch_bounds__(kBlock) void fused_regq(KernelArgs a) {
  __shared__ Lds s;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int nwaves = blockDim.x / kWave;
  const int D4 = a.D >> 2;
  // Work items per question: one for an unsplit ragged batch.
  const int G = MODE == kRagged ? 1 : a.G;
  const long long items = (long long)a.B * G;
  CS_PHASE(0);
  // DRAWN (unsplit questions): row groups come from the LDS counter. The
  // slices of a split question hold one or two groups per wave and keep a
  // fixed share; compiled apart, so their code is unchanged (with the
  // counter's barrier and draws a 16-question split call measured 3-5 %
  // slower).
  constexpr bool drawn = DRAWN;
  if constexpr (drawn) {
    if (tid == 0) s.next_group = nwaves;
    __syncthreads();
  }
  for (long long item = blockIdx.x; item < items; item += gridDim.x) {
    int b = (int)(item / G);
    if constexpr (MODE == kRagged) {
      if (a.longest_first) b = question_of_rank(a, (int)item, s, tid, lane, wave);
    }
    const int g = (int)(item % G);
    Question qn;
    if (!resolve_question<MODE != kDense>(a, b, tid, qn)) continue;  // uniform per workgroup
    const int r0 = MODE == kRagged ? 0 : g * a.rpg;
    // A ragged question has only ceil(K_b / rpg) of the a.G slices.
    if (MODE == kRaggedSplit && r0 >= qn.K) continue;  // uniform per workgroup
    const int r1 = MODE == kRagged ? qn.K : min(qn.K, r0 + a.rpg);
    const int nslices =
        MODE == kDense ? a.G : MODE == kRagged ? 1 : (qn.K + a.rpg - 1) / a.rpg;
    const float4* q4 = reinterpret_cast<const float4*>(a.Q + (size_t)b * (size_t)a.D);
    float4 qr[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int idx = lane + kWave * j;
      qr[j] = (FULL || idx < D4) ? q4[idx] : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    const float* Cb = a.C + qn.row * (size_t)a.D;
#ifdef CS_PHASE_CLOCKS
    int quarter = 1;
#endif
    for (int k0 = r0 + wave * R; k0 < r1;) {
#ifdef CS_PHASE_CLOCKS
      if (quarter <= 3 && 4 * (k0 - r0) >= quarter * (r1 - r0)) {
        CS_PHASE(10 + quarter);
        ++quarter;
      }
#endif
      constexpr int V = COS ? 2 * R : R;
      float acc[V];
#pragma unroll
      for (int v = 0; v < V; ++v) acc[v] = 0.0f;
      const float4* rows[R];
#pragma unroll
      for (int r = 0; r < R; ++r)
        rows[r] = reinterpret_cast<const float4*>(Cb + (size_t)min(k0 + r, r1 - 1) * (size_t)a.D);
      float4 c[R][NV];
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int idx = lane + kWave * j;
#pragma unroll
        for (int r = 0; r < R; ++r)
          c[r][j] = (FULL || idx < D4) ? load4<NT>(rows[r] + idx) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      // Every load of the row group is issued before the first product.
      // Left alone, the scheduler interleaves loads and products to save
      // registers (103 instead of 161 VGPRs for the Kev shape, about 3
      // loads in flight instead of 20). The large batch then hides that
      // with more resident waves, but a split question's slice has only one
      // 4-wave workgroup per compute unit: 16 questions of 255 x 2560 took
      // 20.0 us instead of 14.2 us, with no change for the 1024-question
      // batch (384.5 / 385.1 us).
      __builtin_amdgcn_sched_barrier(0);
      const int next = drawn ? draw_group(s, lane) : 0;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          acc[r] = dot4(c[r][j], qr[j], acc[r]);
          if (COS) acc[R + r] = dot4(c[r][j], c[r][j], acc[R + r]);
        }
      }
      const float total = wave_reduce_transposed<V>(acc, lane, OpSum());
      store_group<COS, R>(s, total, lane, k0, r0, r1);
      k0 = drawn ? r0 + next * R : k0 + nwaves * R;
    }
    CS_PHASE(1);
    __syncthreads();
    CS_PHASE(2);
    if (drawn && tid == 0) s.next_group = nwaves;  // every draw of this slice has returned
    if (wave == 0) {
      float zfac = a.zscale;
      if (COS || (a.cosine && a.staged_norms != nullptr)) {
        float qq = 0.0f;
#pragma unroll
        for (int j = 0; j < NV; ++j) qq = dot4(qr[j], qr[j], qq);
        qq = wave_allreduce(qq, lane, OpSum());
        zfac = a.zscale * rsqrtf(fmaxf(qq, kNormEps2));
      }
      slice_softmax<COS, MODE != kRagged>(s, a, qn, b, g, r0, r1 - r0, zfac, lane, nslices);
      CS_PHASE(3);
    }
    if (MODE != kRagged && nslices > 1) split_merge(s, a, qn, b, tid, lane, wave, nslices);
    __syncthreads();
  }
  CS_PHASE(10);
}

// ---------------------------------------------------------------------------
// The same register-query scoring for batches larger than the chip holds at
// once (dense, one slice per question, no staged norms): a persistent grid
// of the workgroups the compute units hold, each walking questions
// blockIdx.x, blockIdx.x + gridDim.x, ... Each wave issues its first row
// group of the next question, and that question's q, as soon as it has no
// row group left in the current one, so the loads are in flight during the
// barrier and the softmax that end the current question instead of after
// them (with one workgroup per question, every compute unit also paid a
// workgroup launch and a first round trip of loads per question).
template <bool COS, int NV, int R, bool FULL, bool NT>
__global__ __launch_bounds__(kBlock) void fused_regq_stream(KernelArgs a) {
  __shared__ Lds s;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int nwaves = blockDim.x / kWave;
  const int D4 = a.D >> 2;
  const int K = a.K;
  int b = blockIdx.x;
  if (b >= a.B) return;  // uniform; the launch keeps the grid within B
  CS_PHASE(0);
  if (tid == 0) s.next_group = nwaves;
  constexpr int V = COS ? 2 * R : R;
  float4 qr[NV];
  float4 c[R][NV];
  auto load_q = [&](int bq) {
    const float4* q4 = reinterpret_cast<const float4*>(a.Q + (size_t)bq * (size_t)a.D);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int idx = lane + kWave * j;
      qr[j] = (FULL || idx < D4) ? q4[idx] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto load_rows = [&](int bq, int k0) {
    const float* Cb = a.C + (size_t)bq * (size_t)K * (size_t)a.D;
    const float4* rows[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
      rows[r] = reinterpret_cast<const float4*>(Cb + (size_t)min(k0 + r, K - 1) * (size_t)a.D);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int idx = lane + kWave * j;
#pragma unroll
      for (int r = 0; r < R; ++r)
        c[r][j] = (FULL || idx < D4) ? load4<NT>(rows[r] + idx) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  load_q(b);
  int k0 = wave * R;
  if (k0 < K) load_rows(b, k0);
  __syncthreads();  // the counter is set
  for (;;) {
    while (k0 < K) {
      // Every load of the group was issued before its first product.
      __builtin_amdgcn_sched_barrier(0);
      const int next = draw_group(s, lane);
      float acc[V];
#pragma unroll
      for (int v = 0; v < V; ++v) acc[v] = 0.0f;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          acc[r] = dot4(c[r][j], qr[j], acc[r]);
          if (COS) acc[R + r] = dot4(c[r][j], c[r][j], acc[R + r]);
        }
      }
      const float total = wave_reduce_transposed<V>(acc, lane, OpSum());
      store_group<COS, R>(s, total, lane, k0, 0, K);
      k0 = next * R;
      if (k0 < K) load_rows(b, k0);
    }
    // This wave holds no row group of question b any more.
    float qq = 0.0f;
    if (COS && wave == 0) {
#pragma unroll
      for (int j = 0; j < NV; ++j) qq = dot4(qr[j], qr[j], qq);
      qq = wave_allreduce(qq, lane, OpSum());
    }
    const int bn = b + (int)gridDim.x;
    const bool more = bn < a.B;  // uniform
    if (more) {
      load_q(bn);
      k0 = wave * R;
      if (k0 < K) load_rows(bn, k0);
    }
    CS_PHASE(1);
    __syncthreads();  // every logit of question b is in LDS and every draw has returned
    CS_PHASE(2);
    if (wave == 0) {
      const float zfac = COS ? a.zscale * rsqrtf(fmaxf(qq, kNormEps2)) : a.zscale;
      const Question qn{(size_t)b * (size_t)K, K};
      slice_softmax<COS, false>(s, a, qn, b, 0, 0, K, zfac, lane, 1);
      CS_PHASE(3);
    }
    if (tid == 0) s.next_group = nwaves;
    if (!more) break;
    __syncthreads();  // the softmax has read the logits before the next question writes them
    b = bn;
  }
  CS_PHASE(10);
}

// ---------------------------------------------------------------------------
// General kernel: any D, scalar (VEC = 1) or 16-byte (VEC = 4) pieces. The
// query passes through LDS in chunks of at most kQChunk floats; each row's
// partial sums of a chunk are added into its LDS slot (one wave owns a row,
// so the additions are race-free and in chunk order).

constexpr int kQChunk = 8192;

template <bool COS, int VEC, bool NT, int MODE>
__global__ __launch_bounds__(kBlock) void fused_general(KernelArgs a) {
  extern __shared__ float q_dyn[];
  __shared__ Lds s;
  using VecT = typename std::conditional<VEC == 4, float4, float>::type;
  constexpr int R = 4;
  constexpr int V = COS ? 2 * R : R;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int nwaves = blockDim.x / kWave;
  // Work items per question: one for an unsplit ragged batch.
  const int G = MODE == kRagged ? 1 : a.G;
  const long long items = (long long)a.B * G;
  for (long long item = blockIdx.x; item < items; item += gridDim.x) {
    int b = (int)(item / G);
    if constexpr (MODE == kRagged) {
      if (a.longest_first) b = question_of_rank(a, (int)item, s, tid, lane, wave);
    }
    const int g = (int)(item % G);
    Question qn;
    if (!resolve_question<MODE != kDense>(a, b, tid, qn)) continue;  // uniform per workgroup
    const int r0 = MODE == kRagged ? 0 : g * a.rpg;
    // A ragged question has only ceil(K_b / rpg) of the a.G slices.
    if (MODE == kRaggedSplit && r0 >= qn.K) continue;  // uniform per workgroup
    const int r1 = MODE == kRagged ? qn.K : min(qn.K, r0 + a.rpg);
    const int nslices =
        MODE == kDense ? a.G : MODE == kRagged ? 1 : (qn.K + a.rpg - 1) / a.rpg;
    const float* qb = a.Q + (size_t)b * (size_t)a.D;
    const float* Cb = a.C + qn.row * (size_t)a.D;
    const bool need_qq = COS || (a.cosine && a.staged_norms != nullptr);
    float qq = 0.0f;
    for (int c0 = 0; c0 < a.D; c0 += kQChunk) {
      const int clen = min(kQChunk, a.D - c0);
      const int nv = clen / VEC;  // VEC == 4 implies D % 4 == 0
      VecT* ql = reinterpret_cast<VecT*>(q_dyn);
      const VecT* qs = reinterpret_cast<const VecT*>(qb + c0);
      __syncthreads();  // the previous chunk is no longer read
      for (int i = tid; i < nv; i += blockDim.x) {
        const VecT v = qs[i];
        ql[i] = v;
        if (need_qq) {
          if constexpr (VEC == 4)
            qq = dot4(v, v, qq);
          else
            qq = fmaf(v, v, qq);
        }
      }
      __syncthreads();
      for (int k0 = r0 + wave * R; k0 < r1; k0 += nwaves * R) {
        float acc[V];
#pragma unroll
        for (int v = 0; v < V; ++v) acc[v] = 0.0f;
        const VecT* rows[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
          rows[r] = reinterpret_cast<const VecT*>(Cb + (size_t)min(k0 + r, r1 - 1) * (size_t)a.D +
                                                  c0);
        for (int i = lane; i < nv; i += kWave) {
          const VecT qv = ql[i];
#pragma unroll
          for (int r = 0; r < R; ++r) {
            VecT cv;
            if constexpr (VEC == 4)
              cv = load4<NT>(rows[r] + i);
            else
              cv = load1<NT>(rows[r] + i);
            if constexpr (VEC == 4) {
              acc[r] = dot4(cv, qv, acc[r]);
              if (COS) acc[R + r] = dot4(cv, cv, acc[R + r]);
            } else {
              acc[r] = fmaf(cv, qv, acc[r]);
              if (COS) acc[R + r] = fmaf(cv, cv, acc[R + r]);
            }
          }
        }
        const float total = wave_reduce_transposed<V>(acc, lane, OpSum());
        if ((lane & (kWave / V - 1)) == 0) {
          const int slot = lane / (kWave / V);
          const int r = slot % R;
          const int k = k0 + r;
          if (k < r1) {
            float* dst = (slot < R) ? &s.dot[k - r0] : &s.ss[k - r0];
            *dst = (c0 == 0) ? total : *dst + total;
          }
        }
      }
    }
    float zfac = a.zscale;
    if (need_qq) {
      const float qn2 = block_sum(qq, s.red, lane, wave, nwaves);
      zfac = a.zscale * rsqrtf(fmaxf(qn2, kNormEps2));
    } else {
      __syncthreads();
    }
    if (wave == 0)
      slice_softmax<COS, MODE != kRagged>(s, a, qn, b, g, r0, r1 - r0, zfac, lane, nslices);
    if (MODE != kRagged && nslices > 1) split_merge(s, a, qn, b, tid, lane, wave, nslices);
    __syncthreads();
  }
}

// Unfused baseline, first pass: the Euclidean norm of every candidate row,
// written to a staged array (R = 4 rows per wave, rows strided over waves).
template <int VEC, bool NT>
__global__ __launch_bounds__(256) void row_norms(const float* __restrict__ C, long long rows,
                                                 int D, float* __restrict__ norms) {
  using VecT = typename std::conditional<VEC == 4, float4, float>::type;
  constexpr int R = 4;
  const int lane = threadIdx.x & (kWave - 1);
  const long long wave = ((long long)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const long long nwaves = ((long long)gridDim.x * blockDim.x) / kWave;
  const int nv = D / VEC;
  for (long long r0 = wave * R; r0 < rows; r0 += nwaves * R) {
    float acc[R];
    const VecT* rp[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      acc[r] = 0.0f;
      rp[r] = reinterpret_cast<const VecT*>(C + (size_t)min(r0 + r, rows - 1) * (size_t)D);
    }
    for (int i = lane; i < nv; i += kWave) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if constexpr (VEC == 4) {
          const float4 c = load4<NT>(rp[r] + i);
          acc[r] = dot4(c, c, acc[r]);
        } else {
          const float c = load1<NT>(rp[r] + i);
          acc[r] = fmaf(c, c, acc[r]);
        }
      }
    }
    const float total = wave_reduce_transposed<R>(acc, lane, OpSum());
    if ((lane & (kWave / R - 1)) == 0) {
      const long long row = r0 + lane / (kWave / R);
      if (row < rows) norms[row] = sqrtf(total);
    }
  }
}

__global__ void zero_words(uint32_t* p, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

__global__ void zero_bytes(uint8_t* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Launch selection.

template <bool COS, int NV, int R, bool NT, int MODE, bool DRAWN>
void launch_regq_drawn(const KernelArgs& a, const LaunchShape& ls, hipStream_t stream) {
  const bool full = (a.D >> 2) == NV * kWave;
  if (full)
    hipLaunchKernelGGL((fused_regq<COS, NV, R, true, NT, MODE, DRAWN>), dim3(ls.grid),
                       dim3(ls.block), 0, stream, a);
  else
    hipLaunchKernelGGL((fused_regq<COS, NV, R, false, NT, MODE, DRAWN>), dim3(ls.grid),
                       dim3(ls.block), 0, stream, a);
}

// Workgroups of fused_regq_stream<COS, NV, R, FULL, NT> with `block` threads
// that one compute unit of the current device holds at once (cached per
// instantiation, device and block size); 0 when the runtime cannot tell
// (no device).
template <bool COS, int NV, int R, bool FULL, bool NT>
int stream_resident(unsigned block) {
  constexpr int kDevices = 64, kSlots = kBlock / kWave + 1;
  static std::atomic<int> cached[kDevices][kSlots];
  const unsigned slot = block / kWave;
  int dev = 0;
  if (slot >= (unsigned)kSlots || hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return 0;
  }
  if (dev < kDevices) {
    const int n = cached[dev][slot].load(std::memory_order_relaxed);
    if (n > 0) return n;
  }
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, fused_regq_stream<COS, NV, R, FULL, NT>, (int)block, 0) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return 0;
  }
  if (dev < kDevices) cached[dev][slot].store(n, std::memory_order_relaxed);
  return n;
}

// Dense, unsplit batches of more questions than compute units, of at least
// kStreamMinRows candidates each, run the persistent kernel over the
// workgroups the chip holds at once. Measured against one workgroup per
// question: 1024 x 255 x 512 (cosine) 83.0 -> 78.7 us, 8192 x 64 x 512
// 158.0 -> 156.5 us, 4096 x 255 x 1024 (dot) 620 -> 615 us; but
// 65536 x 16 x 256 (dot) 163 -> 170 us, where the hardware's dispatch of
// consecutive questions streams through memory in order.
constexpr int kStreamMinRows = 64;

bool stream_eligible(const KernelArgs& a, const LaunchShape& ls) {
  return a.offsets == nullptr && a.G == 1 && a.staged_norms == nullptr && ls.nv > 0 &&
         ls.units > 0 && (long long)a.B > ls.units && a.K >= kStreamMinRows;
}

template <bool COS, int NV, int R, bool NT>
unsigned stream_grid_nv(const KernelArgs& a, const LaunchShape& ls) {
  const bool full = (a.D >> 2) == NV * kWave;
  const int per_unit = full ? stream_resident<COS, NV, R, true, NT>(ls.block)
                            : stream_resident<COS, NV, R, false, NT>(ls.block);
  if (per_unit <= 0) return 0;
  return (unsigned)std::min<long long>(a.B, (long long)ls.units * per_unit);
}

template <bool COS, int NV, int R, bool NT, int MODE>
hipError_t launch_regq_nv(const KernelArgs& a, const LaunchShape& ls, hipStream_t stream) {
  if constexpr (MODE == kDense) {
    if (stream_eligible(a, ls)) {
      const unsigned grid = stream_grid_nv<COS, NV, R, NT>(a, ls);
      if (grid > 0) {
        if ((a.D >> 2) == NV * kWave)
          hipLaunchKernelGGL((fused_regq_stream<COS, NV, R, true, NT>), dim3(grid),
                             dim3(ls.block), 0, stream, a);
        else
          hipLaunchKernelGGL((fused_regq_stream<COS, NV, R, false, NT>), dim3(grid),
                             dim3(ls.block), 0, stream, a);
        return hipGetLastError();
      }
    }
  }
  if constexpr (MODE == kRagged)
    launch_regq_drawn<COS, NV, R, NT, MODE, true>(a, ls, stream);
  else if constexpr (MODE == kRaggedSplit)
    launch_regq_drawn<COS, NV, R, NT, MODE, false>(a, ls, stream);
  else if (a.G == 1)
    launch_regq_drawn<COS, NV, R, NT, MODE, true>(a, ls, stream);
  else
    launch_regq_drawn<COS, NV, R, NT, MODE, false>(a, ls, stream);
  return hipGetLastError();
}

template <bool COS, bool NT, int MODE>
hipError_t launch_regq(const KernelArgs& a, const LaunchShape& ls, hipStream_t stream) {
  switch (ls.nv) {
    case 1: return launch_regq_nv<COS, 1, 8, NT, MODE>(a, ls, stream);
    case 2: return launch_regq_nv<COS, 2, 8, NT, MODE>(a, ls, stream);
    case 4: return launch_regq_nv<COS, 4, 4, NT, MODE>(a, ls, stream);
    case 6: return launch_regq_nv<COS, 6, 2, NT, MODE>(a, ls, stream);
    case 8: return launch_regq_nv<COS, 8, 2, NT, MODE>(a, ls, stream);
    case 10: return launch_regq_nv<COS, 10, 2, NT, MODE>(a, ls, stream);
    case 12: return launch_regq_nv<COS, 12, 1, NT, MODE>(a, ls, stream);
    case 16: return launch_regq_nv<COS, 16, 1, NT, MODE>(a, ls, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool COS, bool NT, int MODE>
hipError_t launch_general(const KernelArgs& a, const LaunchShape& ls, hipStream_t stream) {
  const size_t lds = sizeof(float) * (size_t)min(a.D, kQChunk);
  if (ls.vec == 4)
    hipLaunchKernelGGL((fused_general<COS, 4, NT, MODE>), dim3(ls.grid), dim3(ls.block), lds,
                       stream, a);
  else
    hipLaunchKernelGGL((fused_general<COS, 1, NT, MODE>), dim3(ls.grid), dim3(ls.block), lds,
                       stream, a);
  return hipGetLastError();
}

template <bool COS, int MODE>
hipError_t launch_kind(const KernelArgs& a, const LaunchShape& ls, hipStream_t stream) {
  if (ls.nv > 0)
    return ls.nt ? launch_regq<COS, true, MODE>(a, ls, stream)
                 : launch_regq<COS, false, MODE>(a, ls, stream);
  return ls.nt ? launch_general<COS, true, MODE>(a, ls, stream)
               : launch_general<COS, false, MODE>(a, ls, stream);
}

}  // namespace

int regq_rows_per_wave(int nv) {
  switch (nv) {
    case 1: case 2: return 8;
    case 4: return 4;
    case 6: case 8: case 10: return 2;
    default: return 1;
  }
}

int regq_nv_for(int D) {
  const int d4 = D / 4;
  const int need = (d4 + kWave - 1) / kWave;
  static const int kNv[] = {1, 2, 4, 6, 8, 10, 12, 16};
  for (int nv : kNv)
    if (nv >= need) return nv;
  return 0;
}

hipError_t launch_fused(const KernelArgs& a, const LaunchShape& ls, hipStream_t stream) {
  // With staged norms (unfused baseline) the hot loop accumulates dots only.
  const bool accumulate_norms = a.cosine && a.staged_norms == nullptr;
  if (a.offsets != nullptr && a.G > 1)
    return accumulate_norms ? launch_kind<true, kRaggedSplit>(a, ls, stream)
                            : launch_kind<false, kRaggedSplit>(a, ls, stream);
  if (a.offsets != nullptr)
    return accumulate_norms ? launch_kind<true, kRagged>(a, ls, stream)
                            : launch_kind<false, kRagged>(a, ls, stream);
  return accumulate_norms ? launch_kind<true, kDense>(a, ls, stream)
                          : launch_kind<false, kDense>(a, ls, stream);
}

template <bool COS, bool NT>
unsigned stream_grid_kind(const KernelArgs& a, const LaunchShape& ls) {
  switch (ls.nv) {
    case 1: return stream_grid_nv<COS, 1, 8, NT>(a, ls);
    case 2: return stream_grid_nv<COS, 2, 8, NT>(a, ls);
    case 4: return stream_grid_nv<COS, 4, 4, NT>(a, ls);
    case 6: return stream_grid_nv<COS, 6, 2, NT>(a, ls);
    case 8: return stream_grid_nv<COS, 8, 2, NT>(a, ls);
    case 10: return stream_grid_nv<COS, 10, 2, NT>(a, ls);
    case 12: return stream_grid_nv<COS, 12, 1, NT>(a, ls);
    case 16: return stream_grid_nv<COS, 16, 1, NT>(a, ls);
    default: return 0;
  }
}

unsigned stream_grid(const KernelArgs& a, const LaunchShape& ls) {
  if (!stream_eligible(a, ls)) return 0;
  if (a.cosine)
    return ls.nt ? stream_grid_kind<true, true>(a, ls) : stream_grid_kind<true, false>(a, ls);
  return ls.nt ? stream_grid_kind<false, true>(a, ls) : stream_grid_kind<false, false>(a, ls);
}

hipError_t launch_row_norms(const float* C, long long rows, int D, int vec, int nt, float* norms,
                            hipStream_t stream) {
  const long long groups = (rows + 3) / 4;  // four rows per wave
  const unsigned grid = (unsigned)std::min<long long>((groups + 3) / 4, 1 << 20);
  if (vec == 4) {
    if (nt)
      hipLaunchKernelGGL((row_norms<4, true>), dim3(grid), dim3(256), 0, stream, C, rows, D, norms);
    else
      hipLaunchKernelGGL((row_norms<4, false>), dim3(grid), dim3(256), 0, stream, C, rows, D, norms);
  } else {
    if (nt)
      hipLaunchKernelGGL((row_norms<1, true>), dim3(grid), dim3(256), 0, stream, C, rows, D, norms);
    else
      hipLaunchKernelGGL((row_norms<1, false>), dim3(grid), dim3(256), 0, stream, C, rows, D, norms);
  }
  return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream) {
  uint8_t* base = static_cast<uint8_t*>(p);
  const size_t head = std::min<size_t>((4 - (reinterpret_cast<uintptr_t>(base) & 3)) & 3, bytes);
  if (head > 0) hipLaunchKernelGGL(zero_bytes, dim3(1), dim3(64), 0, stream, base, head);
  const size_t words = (bytes - head) / 4;
  if (words > 0) {
    const size_t blocks = std::min<size_t>((words + 255) / 256, 4096);
    hipLaunchKernelGGL(zero_words, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<uint32_t*>(base + head), words);
  }
  const size_t tail = bytes - head - words * 4;
  if (tail > 0)
    hipLaunchKernelGGL(zero_bytes, dim3(1), dim3(64), 0, stream, base + head + words * 4, tail);
  return hipGetLastError();
}

// Device address of this GPU's `scratch` array, looked up once per device
// with that device current, and cleared by a fill kernel enqueued on
// `stream` ahead of its first use (no memset node, no synchronization).
hipError_t static_scratch(void** ptr, hipStream_t stream) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];
  static std::mutex setup;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(setup);
    p = addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (err != hipSuccess) return err;
      if (p == nullptr) return hipErrorInvalidSymbol;
      err = launch_zero(p, kStaticScratchBytes, stream);
      if (err != hipSuccess) return err;
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace cs

#ifdef CS_PHASE_CLOCKS
// Measurement build only: copies the phase clocks of the last launches
// (workgroup-major, 16 slots each) to host memory, or clears them.
extern "C" int cs_phase_clocks_read(void* dst, size_t bytes) {
  return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(cs::g_phase_clk), bytes, 0,
                                  hipMemcpyDeviceToHost);
}
extern "C" int cs_phase_clocks_clear(void) {
  static unsigned long long zeros[cs::kPhaseRegions * cs::kPhaseWorkgroups * cs::kPhaseSlots];
  return (int)hipMemcpyToSymbol(HIP_SYMBOL(cs::g_phase_clk), zeros, sizeof(zeros), 0,
                                hipMemcpyHostToDevice);
}
#endif
