// cs_project.hip -- projection + scoring on gfx950: the caller-side heads
// ahead of candidate scoring, fused with it.
//
// Source: pull request "cuda: add a fused candidate-scoring kernel for CLM
// and Kev", intro table: CLM scores exp(logit_scale) * cos(state_head(s),
// action_head(c)); Kev scores (k(h_opts) . q(h_decide)) / sqrt(256); both take
// a softmax over the question's candidates. The page leaves the heads to the
// caller; here they are linear maps without bias, q' = Wq x_q and
// c'_k = Wc x_k, with bf16 inputs and weights and fp32 accumulation.
//
// Two shapes of the same computation:
//  * dot (Kev): c'_k . q' = x_k . (Wc^T q'), so the candidate head folds into
//    the query. proj_query_mfma makes q' [B][P], fold_query_mfma makes
//    u = Wc^T q' [B][Hc], and fused_bf16_dot streams the bf16 candidate rows once against
//    u, with the same in-workgroup softmax as the plain scoring kernels. The
//    candidate side stays a bandwidth-bound pass; no candidate is projected.
//    For eight questions or fewer, proj_query_gemv and fold_query_gemv make
//    q' and u as matrix-vector products from the heads' own layout instead.
//  * cosine (CLM): the norm |Wc x_k| needs the projected rows, a dense
//    contraction: proj_cos_mfma_async (hidden sizes in whole 64-wide chunks;
//    proj_cos_mfma otherwise) computes, per question, the tile
//    C' = X Wc^T (255 x P, X [K][Hc]) with v_mfma_f32_32x32x16_bf16, keeps it
//    in registers, and reduces each row to (c'.q', |c'|^2) in its epilogue;
//    the projected candidates never reach global memory. Small batches use
//    proj_cos_slice instead: one workgroup per 32 candidates, the slices of
//    a question merged like the split scoring kernels.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "cs_device.h"
#include "cs_launch.h"

namespace cs {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// bf16 halves of a 32-bit word, widened exactly to fp32.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// One 16-byte piece (8 bf16), read through the fp32 streaming load (bits are
// moved, not converted).
template <bool NT>
__device__ __forceinline__ uint4 load_piece(const uint16_t* p) {
  const float4 f = load4<NT>(reinterpret_cast<const float4*>(p));
  return make_uint4(__float_as_uint(f.x), __float_as_uint(f.y), __float_as_uint(f.z),
                    __float_as_uint(f.w));
}

// 8 bf16 times 8 fp32, accumulated in order.
__device__ __forceinline__ float dot8_bf(uint4 x, const float (&u)[8], float acc) {
  acc = fmaf(bf_lo(x.x), u[0], acc);
  acc = fmaf(bf_hi(x.x), u[1], acc);
  acc = fmaf(bf_lo(x.y), u[2], acc);
  acc = fmaf(bf_hi(x.y), u[3], acc);
  acc = fmaf(bf_lo(x.z), u[4], acc);
  acc = fmaf(bf_hi(x.z), u[5], acc);
  acc = fmaf(bf_lo(x.w), u[6], acc);
  acc = fmaf(bf_hi(x.w), u[7], acc);
  return acc;
}

// Reduces V values per lane over each 32-lane half of the wave (lanes that
// differ in bits 0..4); lane l ends with value index l % 32 of its half.
template <int V, class Op>
__device__ __forceinline__ float halfwave_reduce_transposed(float (&v)[V], int lane, Op op) {
  static_assert(V >= 1 && V <= 32 && (V & (V - 1)) == 0, "V must be a power of two <= 32");
  halve16<(V >= 2 ? V : 1), V>(v, op);
  halve_dpp<kDppRowRor8, 8, (V >= 4 ? V / 2 : 1), V>(v, lane, op);
  halve_dpp<kDppRowHalfMirror, 4, (V >= 8 ? V / 4 : 1), V>(v, lane, op);
  halve_dpp<kDppQuadXor2, 2, (V >= 16 ? V / 8 : 1), V>(v, lane, op);
  halve_dpp<kDppQuadXor1, 1, (V >= 32 ? V / 16 : 1), V>(v, lane, op);
  return v[0];
}

// ---------------------------------------------------------------------------
// LDS staging helpers shared by the matrix-core kernels.

typedef __attribute__((address_space(1))) const void* global_ptr_t;
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Physical 16-byte position of logical piece `piece` of a 128-byte LDS row
// `row`. The mapping depends on row % 16 only (so 32-row blocks share it),
// and any 16 consecutive rows reading the same logical piece hit distinct
// banks.
__device__ __forceinline__ int swizzled_piece(int row, int piece) {
  return piece ^ ((row & 7) ^ ((row >> 3) & 1));
}

// s_waitcnt with only the vector-memory count limited to n (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}


// Fragment-packed operand of v_mfma_f32_32x32x16_bf16: element (row, k) of
// an R x Kd matrix, with nks = Kd / 16 steps, sits in fragment (row / 32,
// k / 16) at lane (row % 32) + 32 * ((k % 16) / 8), position k % 8; a
// fragment is 64 lanes x 8 bf16 = 1 KiB, so one wave reads a whole fragment
// with one contiguous 16-byte-per-lane load.
__device__ __forceinline__ size_t frag_offset(long long row, int k, int nks) {
  const long long rb = row / 32;
  const int lane = (int)(row % 32) + 32 * ((k % 16) / 8);
  return ((size_t)(rb * nks + k / 16) * kWave + lane) * 8 + (k % 8);
}

// x = hi + mid + lo exactly (bar underflow): each part is the bf16 rounding
// of what the parts before it leave over; both residues are exact in fp32
// and the last one has at most 8 significant bits. The parts are returned as
// fp32 values that bf16 represents exactly.
__device__ __forceinline__ float bf16_round(float x) { return (float)(__bf16)x; }
__device__ __forceinline__ float3 split3(float x) {
  const float hi = bf16_round(x);
  const float r1 = x - hi;
  const float mid = bf16_round(r1);
  return make_float3(hi, mid, bf16_round(r1 - mid));
}
// Bits of a float that bf16 represents exactly.
__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return (uint16_t)(__float_as_uint(x) >> 16);
}

// W^T in fragment order for the fold: fragment (h / 32, p / 16) of the
// H x P16 matrix w^T (zero past P and past H), in 8 x 8 blocks (rows
// p .. p+8, columns h .. h+8; the 8-column groups are padded to whole
// fragments). Block t: eight 16-byte row loads (consecutive blocks read
// consecutive 16 bytes of a row), a transpose in registers, and eight 16-byte
// stores, one per column h, which land in consecutive lanes of one fragment.
__host__ __device__ inline long long pack_wt_blocks(int H, int P) {
  return (long long)((H + 31) / 32 * 4) * ((P + 15) / 16 * 2);
}

__device__ __forceinline__ void pack_wt_block(const uint16_t* __restrict__ w,
                                              uint16_t* __restrict__ wp, int H, int P,
                                              long long t) {
  const int nks = (P + 15) / 16;
  const int hg8 = (H + 31) / 32 * 4;
  const int hgrp = (int)(t % hg8), pgrp = (int)(t / hg8);
  const int h0 = 8 * hgrp, p0 = 8 * pgrp;
  uint4 v[8];
#pragma unroll
  for (int r = 0; r < 8; ++r)
    v[r] = (p0 + r < P && h0 < H)
               ? *reinterpret_cast<const uint4*>(w + (size_t)(p0 + r) * (size_t)H + h0)
               : make_uint4(0u, 0u, 0u, 0u);
  const uint32_t* vw = reinterpret_cast<const uint32_t*>(v);  // vw[4r + c/2] = w[p0+r][h0+c]
  const int ks = p0 / 16, half = (p0 % 16) / 8;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t e0 = vw[4 * (2 * j) + c / 2], e1 = vw[4 * (2 * j + 1) + c / 2];
      o[j] = (c & 1) ? ((e0 >> 16) | (e1 & 0xffff0000u)) : ((e0 & 0xffffu) | (e1 << 16));
    }
    const int h = h0 + c;
    const size_t piece = ((size_t)(h / 32) * nks + ks) * kWave + (h % 32) + 32 * half;
    *reinterpret_cast<uint4*>(wp + piece * 8) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// ---------------------------------------------------------------------------
// q'[b][p] = sum_h x[b][h] * w[p][h]  (x [B][H], w [P][H], bf16; H % 8 == 0)
// on the matrix cores (v_mfma_f32_16x16x32_bf16; bf16 products are exact in
// fp32). One workgroup of 8 waves per 32 x 32 tile of q'; the hidden sum is
// split over the waves in 32-wide blocks (wave w takes blocks w, w+8, ...),
// and a wave issues the loads of up to R blocks before its first multiply,
// so its share of the tile's operands is in flight at once. The 8 partial
// tiles are added in wave order through LDS.
//
// The operands are loaded contiguously, four lanes to a row's 64-byte run
// of a block (lane l: row l/4 of a 16-row half, 16-byte piece l%4), and
// each wave passes them through a private LDS slot to reach the fragment
// layout (lane l: row l%16, piece l/16). Loading fragments straight from
// global memory puts 16 rows in one instruction with no two neighbouring
// lanes in the same row, which costs the L1 one lookup per lane instead of
// one per four and bounded the kernel.
constexpr int kPqWaves = 8;

__device__ __forceinline__ void mfma_block(f32x4_t (&acc)[2][2], const bf16x8_t (&a)[2],
                                           const bf16x8_t (&b)[2]) {
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
      acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rb], b[cb], acc[rb][cb], 0, 0, 0);
}

template <int R>
__global__ __launch_bounds__(kPqWaves * kWave) void proj_query_mfma(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, float* __restrict__ q,
    uint16_t* __restrict__ parts, int B, int H, int P, const uint16_t* __restrict__ wc,
    uint16_t* __restrict__ wpack, int Hc, unsigned* __restrict__ tickets, long long ntiles) {
  __shared__ float part[kPqWaves][16][kWave];
  __shared__ uint4 stage[kPqWaves][2][4][kWave];  // [wave][slot][x0, x1, w0, w1][lane]
  // Phase clocks (region 1): 0 start, 1 wave 0's partial tile in LDS, 2 after
  // the barrier, 3 q' and its parts stored, 4 exit (W^T share packed).
  CS_PHASE_IN(1, 0);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int ptiles = (P + 31) / 32;
  // Consecutive workgroups go to different XCDs (each with its own L2), so
  // when the grid divides evenly, XCD j is given tiles j*(grid/8) ..: the
  // tiles of a few question blocks, which then read their rows of x from
  // one L2 instead of every XCD reading all of x.
  long long tile = blockIdx.x;
  if (gridDim.x % 8 == 0) tile = (long long)(blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
  // With few questions the grid is widened so that the W^T packing spreads
  // over every compute unit; workgroups past the last tile only pack.
  if (tile < ntiles) {
    const long long b0 = (tile / ptiles) * 32;
    const int p0 = (int)(tile % ptiles) * 32;
    f32x4_t acc4[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc4[rb][cb][i] = 0.0f;

    // Whole 32-wide blocks: wave w takes blocks w + 8 j, j < mine.
    const int nfull = H / 32;
    const int mine = (nfull - wave + kPqWaves - 1) / kPqWaves;
    const int r4 = lane >> 2, pc = lane & 3;
    const uint16_t* cr[4];  // this lane's rows of x (two 16-row halves), then of w
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      cr[h] = x + (size_t)min(b0 + 16 * h + r4, (long long)B - 1) * (size_t)H;
      cr[2 + h] = w + (size_t)min(p0 + 16 * h + r4, P - 1) * (size_t)H;
    }
    // LDS positions: the piece index is XORed with bits 1..2 of the row, so
    // the eight lanes of an LDS pass (two rows of four pieces when writing,
    // eight rows of one piece when reading) hit eight distinct 16-byte bank
    // groups.
    const int wslot = r4 * 4 + (pc ^ ((r4 >> 1) & 3));
    const int rrow = lane & 15, rpc = lane >> 4;
    const int rslot = rrow * 4 + (rpc ^ ((rrow >> 1) & 3));
    for (int r0 = 0; r0 < mine; r0 += R) {
      uint4 cv[R][4];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        // Past this wave's blocks the load repeats its last block (always in
        // bounds); the products of those repeats are zeroed below.
        const int k = 32 * (wave + kPqWaves * min(r0 + i, mine - 1)) + 8 * pc;
#pragma unroll
        for (int t = 0; t < 4; ++t) cv[i][t] = *reinterpret_cast<const uint4*>(cr[t] + k);
      }
#pragma unroll
      for (int i = 0; i < R; ++i) {
        // A select rather than a branch: a branch here would split the round
        // and let the compiler sink each block's loads down to their use.
        const bool use = r0 + i < mine;
#pragma unroll
        for (int t = 0; t < 4; ++t) stage[wave][i & 1][t][wslot] = cv[i][t];
        bf16x8_t fa[2], fb[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint4 z = make_uint4(0u, 0u, 0u, 0u);
          const uint4 ra = stage[wave][i & 1][h][rslot], rb = stage[wave][i & 1][2 + h][rslot];
          fa[h] = __builtin_bit_cast(bf16x8_t, use ? ra : z);
          fb[h] = __builtin_bit_cast(bf16x8_t, use ? rb : z);
        }
        mfma_block(acc4, fa, fb);
      }
    }
    if (H % 32 != 0 && wave == nfull % kPqWaves) {
      // The last, partial block, loaded straight into the fragment layout;
      // lanes past H contribute zeros.
      const int k = 32 * nfull + 8 * rpc;
      bf16x8_t fa[2], fb[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const size_t xrow = (size_t)min(b0 + 16 * h + rrow, (long long)B - 1);
        const size_t wrow = (size_t)min(p0 + 16 * h + rrow, P - 1);
        if (k < H) {
          fa[h] = *reinterpret_cast<const bf16x8_t*>(x + xrow * (size_t)H + k);
          fb[h] = *reinterpret_cast<const bf16x8_t*>(w + wrow * (size_t)H + k);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            fa[h][e] = (__bf16)0.0f;
            fb[h][e] = (__bf16)0.0f;
          }
        }
      }
      mfma_block(acc4, fa, fb);
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) part[wave][4 * (2 * rb + cb) + i][lane] = acc4[rb][cb][i];
    CS_PHASE_IN(1, 1);
    __syncthreads();
    CS_PHASE_IN(1, 2);
    // Element i of tile (rb, cb) in lane l is q'[b0 + 16*rb + 4*(l/16) + i][p0 + 16*cb + l%16].
    for (int e = wave; e < 16; e += kPqWaves) {
      float v = 0.0f;
#pragma unroll
      for (int ww = 0; ww < kPqWaves; ++ww) v += part[ww][e][lane];
      const int t = e / 4, i = e % 4, rb = t / 2, cb = t % 2;
      const long long bq = b0 + 16 * rb + 4 * (lane / 16) + i;
      const int pp = p0 + 16 * cb + (lane & 15);
      if (bq < B && pp < P) q[(size_t)bq * (size_t)P + pp] = v;
      const int p16 = (P + 15) / 16 * 16;
      if (parts != nullptr && bq < B && pp < p16) {
        float3 sp = make_float3(0.0f, 0.0f, 0.0f);
        if (pp < P) sp = split3(v);
        const int nks = 3 * p16 / 16;
        parts[frag_offset(bq, pp, nks)] = bf16_bits(sp.x);
        parts[frag_offset(bq, p16 + pp, nks)] = bf16_bits(sp.y);
        parts[frag_offset(bq, 2 * p16 + pp, nks)] = bf16_bits(sp.z);
      }
    }
    // The split candidate pass's merge tickets start at zero: the first tile
    // of each 32-question block clears its questions' tickets (the candidate
    // pass runs two launches later on the same stream).
    if (tickets != nullptr && p0 == 0 && tid < 32 && b0 + tid < B) tickets[b0 + tid] = 0u;
    CS_PHASE_IN(1, 3);
  }
  if (wpack != nullptr) {
    // This workgroup's share of the fold's W^T packing (independent of q'),
    // after its own loads so that it does not delay them.
    const long long total = pack_wt_blocks(Hc, P);
    const long long per = (total + gridDim.x - 1) / gridDim.x;
    const long long end = min(total, per * ((long long)blockIdx.x + 1));
    for (long long t = per * blockIdx.x + (long long)lane * kPqWaves + wave; t < end;
         t += blockDim.x)
      pack_wt_block(wc, wpack, Hc, P, t);
  }
  CS_PHASE_IN(1, 4);
}

// u[b][h] = sum_p q'[b][p] * w[p][h]  (q' [B][P] fp32, w [P][H] bf16,
// P <= 256, H % 8 == 0) on the bf16 matrix cores, from the three-part split
// of q' that proj_query_mfma wrote (hi | mid | lo along the contraction):
// the three products with a bf16 weight are exact and only the fp32
// accumulation rounds, as in an fp32 dot product. Both operands come
// fragment-packed (parts and w^T by proj_query_mfma), so every
// operand load is one contiguous 1 KiB per wave and no LDS is involved. A
// wave computes 32 questions x 128 h (four accumulators); per 16-wide step
// over p it loads three part fragments and four weight fragments and issues
// twelve matrix instructions, with the next step's loads in flight.
constexpr int kFoldNb = 4;  // 32-column blocks per wave

__global__ __launch_bounds__(256) void fold_query_mfma(const uint16_t* __restrict__ parts,
                                                       const uint16_t* __restrict__ wp,
                                                       float* __restrict__ u, int B, int H,
                                                       int P) {
  // Phase clocks (region 2, both folds): 0 start, 1 wave 0's contraction
  // done, 2 exit.
  CS_PHASE_IN(2, 0);
  const int lane = threadIdx.x & (kWave - 1);
  // Workgroups numbered per XCD, as in proj_query_mfma: XCD j takes a run of
  // question blocks and reads only their parts from its own L2.
  long long wg = blockIdx.x;
  if (gridDim.x % 8 == 0) wg = (long long)(blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
  const long long wid = wg * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int hgroups = (H + 32 * kFoldNb - 1) / (32 * kFoldNb);
  const long long qb = wid / hgroups;
  const int hg = (int)(wid % hgroups);
  if (qb * 32 >= B) return;  // uniform across the wave
  const int sp = (P + 15) / 16;           // 16-wide steps over p
  const int hblocks = (H + 31) / 32;
  const uint4* ap = reinterpret_cast<const uint4*>(parts) + (size_t)qb * (3 * sp) * kWave + lane;
  const uint4* bp = reinterpret_cast<const uint4*>(wp) + lane;
  f32x16_t acc[kFoldNb];
#pragma unroll
  for (int nb = 0; nb < kFoldNb; ++nb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[nb][e] = 0.0f;
  auto load = [&](int ks, uint4 (&a)[3], uint4 (&w)[kFoldNb]) {
#pragma unroll
    for (int c = 0; c < 3; ++c) a[c] = ap[(size_t)(c * sp + ks) * kWave];
#pragma unroll
    for (int nb = 0; nb < kFoldNb; ++nb) {
      const int hb = min(hg * kFoldNb + nb, hblocks - 1);
      w[nb] = bp[((size_t)hb * sp + ks) * kWave];
    }
  };
  uint4 a[2][3], w[2][kFoldNb];
  load(0, a[0], w[0]);
  for (int ks = 0; ks < sp; ks += 2) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (ks + i < sp) {  // uniform
        if (ks + i + 1 < sp) load(ks + i + 1, a[i ^ 1], w[i ^ 1]);
#pragma unroll
        for (int c = 0; c < 3; ++c)
#pragma unroll
          for (int nb = 0; nb < kFoldNb; ++nb)
            acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8_t, a[i][c]), __builtin_bit_cast(bf16x8_t, w[i][nb]),
                acc[nb], 0, 0, 0);
      }
    }
  }
  CS_PHASE_IN(2, 1);
  // Accumulator e of lane l: question 32*qb + 8*(e/4) + 4*(l/32) + e%4,
  // column 32*(hg*4 + nb) + l%32.
#pragma unroll
  for (int nb = 0; nb < kFoldNb; ++nb) {
    const int hcol = 32 * (hg * kFoldNb + nb) + (lane & 31);
    if (hcol >= H) continue;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const long long b = qb * 32 + 8 * (e / 4) + 4 * (lane / 32) + (e % 4);
      if (b < B) u[(size_t)b * (size_t)H + hcol] = acc[nb][e];
    }
  }
  CS_PHASE_IN(2, 2);
}

// The same fold for batches too small to fill the chip: with few question
// blocks, one wave per tile walks its 16 dependent steps on a handful of
// compute units. Here four waves share a tile, each taking a quarter of the
// contraction with all its loads issued at once (clamped to valid steps, so
// the count of loads in flight is the same on every path), and the partial
// tiles are added in wave order through LDS.
constexpr int kFoldSplitWaves = 4;
constexpr int kFoldSplitSteps = (256 / 16 + kFoldSplitWaves - 1) / kFoldSplitWaves;  // P <= 256

__global__ __launch_bounds__(kFoldSplitWaves * kWave) void fold_query_mfma_split(
    const uint16_t* __restrict__ parts, const uint16_t* __restrict__ wp, float* __restrict__ u,
    int B, int H, int P) {
  // Partial tiles as four float4 rows per block, lane-contiguous, so each
  // 16-byte LDS access of a wave covers consecutive banks.
  __shared__ float4 red[kFoldSplitWaves][kFoldNb][4][kWave];
  CS_PHASE_IN(2, 0);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int hgroups = (H + 32 * kFoldNb - 1) / (32 * kFoldNb);
  const long long qb = blockIdx.x / hgroups;
  const int hg = (int)(blockIdx.x % hgroups);
  const int sp = (P + 15) / 16;
  const int s0 = wave * sp / kFoldSplitWaves, s1 = (wave + 1) * sp / kFoldSplitWaves;
  const int hblocks = (H + 31) / 32;
  const uint4* ap = reinterpret_cast<const uint4*>(parts) + (size_t)qb * (3 * sp) * kWave + lane;
  const uint4* bp = reinterpret_cast<const uint4*>(wp) + lane;
  uint4 a[kFoldSplitSteps][3], w[kFoldSplitSteps][kFoldNb];
#pragma unroll
  for (int i = 0; i < kFoldSplitSteps; ++i) {
    const int ks = min(s0 + i, sp - 1);
#pragma unroll
    for (int c = 0; c < 3; ++c) a[i][c] = ap[(size_t)(c * sp + ks) * kWave];
#pragma unroll
    for (int nb = 0; nb < kFoldNb; ++nb) {
      const int hb = min(hg * kFoldNb + nb, hblocks - 1);
      w[i][nb] = bp[((size_t)hb * sp + ks) * kWave];
    }
  }
  f32x16_t acc[kFoldNb];
#pragma unroll
  for (int nb = 0; nb < kFoldNb; ++nb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[nb][e] = 0.0f;
#pragma unroll
  for (int i = 0; i < kFoldSplitSteps; ++i)
    if (s0 + i < s1)
#pragma unroll
      for (int c = 0; c < 3; ++c)
#pragma unroll
        for (int nb = 0; nb < kFoldNb; ++nb)
          acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, a[i][c]), __builtin_bit_cast(bf16x8_t, w[i][nb]),
              acc[nb], 0, 0, 0);
#pragma unroll
  for (int nb = 0; nb < kFoldNb; ++nb)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      red[wave][nb][j][lane] =
          make_float4(acc[nb][4 * j], acc[nb][4 * j + 1], acc[nb][4 * j + 2], acc[nb][4 * j + 3]);
  CS_PHASE_IN(2, 1);
  __syncthreads();
  // Wave w sums and stores column block w (kFoldNb == kFoldSplitWaves).
  const int nb = wave;
  f32x16_t sum;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float4 t = red[0][nb][j][lane];
#pragma unroll
    for (int kk = 1; kk < kFoldSplitWaves; ++kk) {
      const float4 v = red[kk][nb][j][lane];
      t.x += v.x;
      t.y += v.y;
      t.z += v.z;
      t.w += v.w;
    }
    sum[4 * j] = t.x;
    sum[4 * j + 1] = t.y;
    sum[4 * j + 2] = t.z;
    sum[4 * j + 3] = t.w;
  }
  const int hcol = 32 * (hg * kFoldNb + nb) + (lane & 31);
  if (hcol < H) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const long long b = qb * 32 + 8 * (e / 4) + 4 * (lane / 32) + (e % 4);
      if (b < B) u[(size_t)b * (size_t)H + hcol] = sum[e];
    }
  }
  CS_PHASE_IN(2, 2);
}
static_assert(kFoldNb == kFoldSplitWaves, "one column block per wave in the split fold's sum");

// ---------------------------------------------------------------------------
// The dot path's query side for a batch of at most kGemvMaxB questions. There
// the 32-question matrix-core tiles would be mostly padding, and packing Wc^T
// for them costs more than the products, so both heads are applied as plain
// matrix-vector products straight from their row-major layout, each reading
// its head once with fp32 accumulation (the bf16 x bf16 products are exact).

constexpr int kGemvMaxB = 8;
constexpr int kGemvUnroll = 4;  // 512-wide chunks of a head row in flight per wave

// 8 bf16 times 8 bf16, widened exactly and accumulated in order.
__device__ __forceinline__ float dot8_bf_bf(uint4 w, uint4 x) {
  float acc = bf_lo(w.x) * bf_lo(x.x);
  acc = fmaf(bf_hi(w.x), bf_hi(x.x), acc);
  acc = fmaf(bf_lo(w.y), bf_lo(x.y), acc);
  acc = fmaf(bf_hi(w.y), bf_hi(x.y), acc);
  acc = fmaf(bf_lo(w.z), bf_lo(x.z), acc);
  acc = fmaf(bf_hi(w.z), bf_hi(x.z), acc);
  acc = fmaf(bf_lo(w.w), bf_lo(x.w), acc);
  acc = fmaf(bf_hi(w.w), bf_hi(x.w), acc);
  return acc;
}

// q'[b][p] = sum_h Wq[p][h] x_q[b][h]: one wave per head row p, its 16-byte
// pieces spread over the lanes (kGemvUnroll per lane in flight), the
// questions' matching pieces loaded beside them; per-lane sums are added
// over the wave. Loads past the row are clamped to its last piece, which is
// then zeroed, so every lane issues the same loads.
// Workgroup 0 also clears the merge tickets of the candidate pass (B <= 64,
// at most one per lane).
template <int NB>
__global__ __launch_bounds__(256) void proj_query_gemv(const uint16_t* __restrict__ xq,
                                                       const uint16_t* __restrict__ wq,
                                                       float* __restrict__ qp, int B, int Hq,
                                                       int P, unsigned* __restrict__ tickets) {
  const int lane = threadIdx.x & (kWave - 1);
  const int p = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (tickets != nullptr && blockIdx.x == 0 && (int)threadIdx.x < B) tickets[threadIdx.x] = 0u;
  if (p >= P) return;  // uniform across the wave
  const int n = Hq / 8;  // 16-byte pieces per row
  const uint4* wr = reinterpret_cast<const uint4*>(wq + (size_t)p * (size_t)Hq);
  const uint4* xr[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
    xr[b] = reinterpret_cast<const uint4*>(xq + (size_t)min(b, B - 1) * (size_t)Hq);
  float acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = 0.0f;
  for (int c0 = 0; c0 < n; c0 += kWave * kGemvUnroll) {  // uniform trip count
    uint4 w[kGemvUnroll], x[kGemvUnroll][NB];
#pragma unroll
    for (int i = 0; i < kGemvUnroll; ++i) {
      const int c = min(c0 + kWave * i + lane, n - 1);
      w[i] = wr[c];
#pragma unroll
      for (int b = 0; b < NB; ++b) x[i][b] = xr[b][c];
    }
#pragma unroll
    for (int i = 0; i < kGemvUnroll; ++i) {
      // A clamped piece is zeroed (a bit select, not a branch) so it adds 0.
      const uint32_t keep = c0 + kWave * i + lane < n ? ~0u : 0u;
      const uint4 wi = make_uint4(w[i].x & keep, w[i].y & keep, w[i].z & keep, w[i].w & keep);
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[b] += dot8_bf_bf(wi, x[i][b]);
    }
  }
  // Lane l ends with the sum of question l / (64 / NB).
  const float total = wave_reduce_transposed<NB>(acc, lane, OpSum());
  const int b = lane / (kWave / NB);
  if (lane % (kWave / NB) == 0 && b < B) qp[(size_t)b * (size_t)P + p] = total;
}

// u[b][h] = sum_p q'[b][p] Wc[p][h]: a workgroup takes kFoldGemvCols columns
// (four 16-byte pieces of every row) and all P <= 256 rows as 64 row phases;
// the lane of phase r loads rows r, r + 64, ... in one round, multiplies them
// by q' staged in LDS, and the phases are then added in order through LDS
// (padded so that neither the stores nor the column sums collide on a bank).
// With 64 columns per workgroup (40 workgroups for 2560 columns) eight
// questions took 21.3 us per call against 20.2 us with 32, four 16.0 against
// 15.6; 16 columns gave nothing more and one question 0.4 us less.
constexpr int kFoldGemvCols = 32;
constexpr int kFoldGemvPieces = kFoldGemvCols / 8;
constexpr int kFoldGemvPhases = 256 / kFoldGemvPieces;
constexpr int kFoldGemvRows = 256 / kFoldGemvPhases;  // rows per lane at P = 256
constexpr int kFoldGemvPad = kFoldGemvPhases + 1;

template <int NB>
__global__ __launch_bounds__(256) void fold_query_gemv(const float* __restrict__ qp,
                                                       const uint16_t* __restrict__ wc,
                                                       float* __restrict__ u, int B, int Hc,
                                                       int P) {
  __shared__ float qs[NB][256];
  __shared__ float red[NB][8][kFoldGemvPad][kFoldGemvPieces];
  const int tid = threadIdx.x;
  const int pc = tid % kFoldGemvPieces, ph = tid / kFoldGemvPieces;
  const int n = Hc / 8;
  const int piece = min((int)blockIdx.x * kFoldGemvPieces + pc, n - 1);
  uint4 w[kFoldGemvRows];
#pragma unroll
  for (int r = 0; r < kFoldGemvRows; ++r) {
    const int row = min(ph + kFoldGemvPhases * r, P - 1);
    w[r] = reinterpret_cast<const uint4*>(wc + (size_t)row * (size_t)Hc)[piece];
  }
  // q' of every question and row, zero past P (rows clamped above then add 0).
#pragma unroll
  for (int i = tid; i < NB * 256; i += 256) {
    const int b = i / 256, row = i % 256;
    const float v = qp[(size_t)min(b, B - 1) * (size_t)P + min(row, P - 1)];
    qs[b][row] = (b < B && row < P) ? v : 0.0f;
  }
  __syncthreads();
  float acc[NB][8];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[b][j] = 0.0f;
#pragma unroll
  for (int r = 0; r < kFoldGemvRows; ++r) {
    const int row = ph + kFoldGemvPhases * r;
    const uint32_t keep = row < P ? ~0u : 0u;  // clamped rows add 0
    const uint4 x = make_uint4(w[r].x & keep, w[r].y & keep, w[r].z & keep, w[r].w & keep);
    const float f[8] = {bf_lo(x.x), bf_hi(x.x), bf_lo(x.y), bf_hi(x.y),
                        bf_lo(x.z), bf_hi(x.z), bf_lo(x.w), bf_hi(x.w)};
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float q = qs[b][row];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[b][j] = fmaf(q, f[j], acc[b][j]);
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int j = 0; j < 8; ++j) red[b][j][ph][pc] = acc[b][j];
  __syncthreads();
  // Output o (threads take o = t, t + 256, ...) is column
  // 8 * (o % kFoldGemvPieces) + (o / kFoldGemvPieces) % 8 of question
  // o / kFoldGemvCols.
#pragma unroll
  for (int o = tid; o < NB * kFoldGemvCols; o += 256) {
    const int b = o / kFoldGemvCols, j = (o / kFoldGemvPieces) % 8, c = o % kFoldGemvPieces;
    float sum = 0.0f;
#pragma unroll
    for (int r = 0; r < kFoldGemvPhases; ++r) sum += red[b][j][r][c];
    const int h = ((int)blockIdx.x * kFoldGemvPieces + c) * 8 + j;
    if (b < B && h < Hc) u[(size_t)b * (size_t)Hc + h] = sum;
  }
}
static_assert(kFoldGemvPieces * kFoldGemvPhases == 256 && kFoldGemvPhases * kFoldGemvRows == 256,
              "the small-batch fold covers 256 rows with 256 threads");

// ---------------------------------------------------------------------------
// Dot scoring of bf16 candidate rows against the folded fp32 query u: the
// register-query kernel's structure with 16-byte pieces of 8 bf16. Lane l
// owns pieces l + 64 j (j < NV) of every row; a wave takes R rows at a time;
// one workgroup per question. u sits in LDS (its low and high halves of each
// piece in two arrays, so a wave's reads are contiguous) rather than in 8*NV
// registers per lane, which leaves room for more loads in flight.
template <int NV, int R, bool FULL, bool NT>
__global__ __launch_bounds__(kBlock) void fused_bf16_dot(KernelArgs a,
                                                         const uint16_t* __restrict__ xc,
                                                         const float* __restrict__ u) {
  __shared__ Lds s;
  __shared__ float4 us_lo[8 * kWave], us_hi[8 * kWave];
  // Phase clocks (region 3): 0 start, 1 u staged in LDS, 2-4 wave 0 past a
  // quarter, half and three quarters of the slice's rows, 5 exit.
  CS_PHASE_IN(3, 0);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int nwaves = blockDim.x / kWave;
  const int pieces = a.D >> 3;
  // Items are (question, slice): with G > 1 slices per question, slice g
  // takes candidates g*rpg .. and the last slice to finish merges, as in the
  // fp32 kernels.
  const int G = a.G;
  const long long items = (long long)a.B * G;
  // Unsplit questions take their row groups from the LDS counter, slices of
  // a split question a fixed share (as in the fp32 kernels).
  const bool drawn = G == 1;
  if (tid == 0) s.next_group = nwaves;
  for (long long item = blockIdx.x; item < items; item += gridDim.x) {
    const int b = (int)(item / G), g = (int)(item % G);
    const Question qn{(size_t)b * (size_t)a.K, a.K};
    const int r0 = g * a.rpg, r1 = min(a.K, r0 + a.rpg);
    for (int idx = tid; idx < NV * kWave; idx += blockDim.x) {
      float4 u0 = make_float4(0.f, 0.f, 0.f, 0.f), u1 = u0;
      if (FULL || idx < pieces) {
        const float4* up = reinterpret_cast<const float4*>(u + (size_t)b * (size_t)a.D) + 2 * idx;
        u0 = up[0];
        u1 = up[1];
      }
      us_lo[idx] = u0;
      us_hi[idx] = u1;
    }
    __syncthreads();
    CS_PHASE_IN(3, 1);
    const uint16_t* Xb = xc + qn.row * (size_t)a.D;
#ifdef CS_PHASE_CLOCKS
    int quarter = 1;
#endif
    for (int k0 = r0 + wave * R; k0 < r1;) {
#ifdef CS_PHASE_CLOCKS
      if (quarter <= 3 && 4 * (k0 - r0) >= quarter * (r1 - r0)) {
        CS_PHASE_IN(3, 1 + quarter);
        ++quarter;
      }
#endif
      float acc[R];
      const uint16_t* rows[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        acc[r] = 0.0f;
        rows[r] = Xb + (size_t)min(k0 + r, r1 - 1) * (size_t)a.D;
      }
      uint4 c[R][NV];
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int idx = lane + kWave * j;
#pragma unroll
        for (int r = 0; r < R; ++r)
          c[r][j] = (FULL || idx < pieces) ? load_piece<NT>(rows[r] + 8 * idx)
                                           : make_uint4(0u, 0u, 0u, 0u);
      }
      const int next = drawn ? draw_group(s, lane) : 0;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const float4 u0 = us_lo[lane + kWave * j], u1 = us_hi[lane + kWave * j];
        const float ur[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = dot8_bf(c[r][j], ur, acc[r]);
      }
      const float total = wave_reduce_transposed<R>(acc, lane, OpSum());
      store_group<false, R>(s, total, lane, k0, r0, r1);
      k0 = drawn ? r0 + next * R : k0 + nwaves * R;
    }
    __syncthreads();
    if (drawn && tid == 0) s.next_group = nwaves;  // every draw of this slice has returned
    if (wave == 0) slice_softmax<false>(s, a, qn, b, g, r0, r1 - r0, a.zscale, lane, G);
    if (G > 1) split_merge(s, a, qn, b, tid, lane, wave, G);
    __syncthreads();
  }
  CS_PHASE_IN(3, 5);
}

// Epilogue of the cosine tile: each row of C' reduced to c'.q' and |c'|^2,
// the two feature halves added in a fixed order into the softmax's LDS
// slots, then the softmax itself. Called by every thread of the workgroup.
template <int TN>
__device__ __forceinline__ void cos_epilogue(Lds& s, const KernelArgs& a,
                                             const float* __restrict__ qp,
                                             const f32x16_t (&acc)[2][TN], int b, int K,
                                             int lane, int wave, int wr, int wcb) {
  constexpr int P = 64 * TN;
  // Epilogue. Accumulator e of tile (rb, tn) in lane l holds C'[row][col]
  // with row = 64*wr + 32*rb + 8*(e/4) + 4*(l/32) + e%4 and
  // col = 32*TN*wcb + 32*tn + l%32.
  float qv[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn)
    qv[tn] = qp[(size_t)b * P + 32 * TN * wcb + 32 * tn + (lane & 31)];
  float dv[32], ev[32];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float d = 0.0f, q2 = 0.0f;
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const float c = acc[rb][tn][e];
        d = fmaf(c, qv[tn], d);
        q2 = fmaf(c, c, q2);
      }
      dv[16 * rb + e] = d;
      ev[16 * rb + e] = q2;
    }
  const float dsum = halfwave_reduce_transposed<32>(dv, lane, OpSum());
  const float esum = halfwave_reduce_transposed<32>(ev, lane, OpSum());
  const int v = lane & 31, rb = v >> 4, e = v & 15;
  const int row = 64 * wr + 32 * rb + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
  // The two column halves of a row are added in a fixed order.
  if (wcb == 0) {
    s.dot[row] = dsum;
    s.ss[row] = esum;
  }
  __syncthreads();
  if (wcb == 1) {
    s.dot[row] += dsum;
    s.ss[row] += esum;
  }
  __syncthreads();
  if (wave == 0) {
    float qq = 0.0f;
    for (int p = lane; p < P; p += kWave) {
      const float x = qp[(size_t)b * P + p];
      qq = fmaf(x, x, qq);
    }
    qq = wave_allreduce(qq, lane, OpSum());
    const float zfac = a.zscale * rsqrtf(fmaxf(qq, kNormEps2));
    const Question qn{(size_t)b * (size_t)K, K};
    slice_softmax<true>(s, a, qn, b, 0, 0, K, zfac, lane, a.G);
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Cosine: per question, C' = X Wc^T on the matrix cores, fused with the
// similarity and the softmax. One workgroup of 8 waves per question; wave w
// owns rows 64*(w % 4) .. +64 (two 32-row MFMA tiles) and columns
// 32*TN*(w / 4) .. +32*TN (TN 32-column tiles), so P = 64 * TN <= 256.
// The hidden dimension is staged through LDS 64 bf16 at a time (rows padded
// by 16 bytes against bank conflicts), double-buffered (2 x 72 KiB).
constexpr int kChunk = 64;
constexpr int kRowStride = kChunk + 8;  // bf16 per LDS row

template <int TN, bool NT>
__global__ __launch_bounds__(512) void proj_cos_mfma(KernelArgs a,
                                                     const uint16_t* __restrict__ xc,
                                                     const uint16_t* __restrict__ wc,
                                                     const float* __restrict__ qp) {
  __shared__ __attribute__((aligned(16))) uint16_t sX[2][256 * kRowStride];
  __shared__ __attribute__((aligned(16))) uint16_t sW[2][256 * kRowStride];
  __shared__ Lds s;
  constexpr int P = 64 * TN;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int wr = wave & 3, wcb = wave >> 2;
  const int H = a.D, K = a.K;
  for (int b = blockIdx.x; b < a.B; b += gridDim.x) {
    f32x16_t acc[2][TN];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[rb][tn][e] = 0.0f;
    const uint16_t* Xb = xc + (size_t)b * (size_t)K * (size_t)H;
    // Double-buffered staging: while the matrix cores work on chunk c from
    // one LDS buffer, the loads of chunk c+1 are in flight to registers; they
    // land in the other buffer before the one barrier per chunk.
    const int nchunks = (H + kChunk - 1) / kChunk;
    uint4 px[4], pw[4];
    auto fetch = [&](int c) {
      const int h0 = c * kChunk;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int id = tid + 512 * i;
        const int row = id >> 3, c8 = id & 7;
        const int hh = h0 + 8 * c8;
        const bool in_h = hh < H;
        px[i] = (row < K && in_h) ? load_piece<NT>(Xb + (size_t)row * (size_t)H + hh)
                                  : make_uint4(0u, 0u, 0u, 0u);
        pw[i] = (row < P && in_h) ? load_piece<false>(wc + (size_t)row * (size_t)H + hh)
                                  : make_uint4(0u, 0u, 0u, 0u);
      }
    };
    auto deposit = [&](int buf) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int id = tid + 512 * i;
        const int row = id >> 3, c8 = id & 7;
        *reinterpret_cast<uint4*>(&sX[buf][row * kRowStride + 8 * c8]) = px[i];
        *reinterpret_cast<uint4*>(&sW[buf][row * kRowStride + 8 * c8]) = pw[i];
      }
    };
    fetch(0);
    deposit(0);
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
      const int buf = c & 1;
      if (c + 1 < nchunks) fetch(c + 1);
#pragma unroll
      for (int ks = 0; ks < kChunk / 16; ++ks) {
        // Lane l feeds row/column l % 32 and hidden elements 8*(l/32) .. +8
        // of this 16-wide step, the same slots for both operands.
        const int kofs = 16 * ks + 8 * (lane >> 5);
        bf16x8_t af[2], bfr[TN];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          af[rb] = *reinterpret_cast<const bf16x8_t*>(
              &sX[buf][(64 * wr + 32 * rb + (lane & 31)) * kRowStride + kofs]);
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          bfr[tn] = *reinterpret_cast<const bf16x8_t*>(
              &sW[buf][(32 * TN * wcb + 32 * tn + (lane & 31)) * kRowStride + kofs]);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int tn = 0; tn < TN; ++tn)
            acc[rb][tn] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[rb], bfr[tn], acc[rb][tn], 0, 0, 0);
      }
      if (c + 1 < nchunks) deposit(buf ^ 1);
      __syncthreads();
    }
    cos_epilogue<TN>(s, a, qp, acc, b, K, lane, wave, wr, wcb);
  }
}

// ---------------------------------------------------------------------------
// Cosine for small batches (B * ceil(K / 32) workgroups fit the compute
// units): one workgroup per 32-candidate slice of a question, so a single
// question is spread over up to eight compute units instead of one. Eight
// waves share the slice's 32 x P tile C' = X Wc^T: wave w owns the 32-feature
// block w when it exists (P = 64 * TN has 2 * TN of them). The hidden
// dimension moves through two LDS buffers 64 bf16 at a time, with the loads
// of the next kCosSliceAhead chunks in flight in registers (all of a
// 512-wide hidden size in one round); loads past the last chunk repeat it
// and hidden positions past Hc are zeroed in the deposit, so every lane
// issues the same loads. Each row is reduced to (c'.q', |c'|^2) in registers, the waves'
// parts are added in wave order, and the slice's softmax partial is merged
// with the question's other slices by the last to finish.
constexpr int kCosSliceWaves = 8;
constexpr int kCosSliceAhead = 8;

template <int TN>
__global__ __launch_bounds__(kCosSliceWaves * kWave) void proj_cos_slice(
    KernelArgs a, const uint16_t* __restrict__ xc, const uint16_t* __restrict__ wc,
    const float* __restrict__ qp) {
  constexpr int kThreads = kCosSliceWaves * kWave;
  constexpr int P = 64 * TN;
  constexpr int kRows = kCosSliceRows;
  constexpr int kWPer = P * 8 / kThreads;  // W pieces per thread per chunk
  static_assert(kRows * 8 == 256 && kWPer == TN, "X pieces of a chunk: one per thread of 256");
  __shared__ __attribute__((aligned(16))) uint16_t sX[2][kRows * kRowStride];
  __shared__ __attribute__((aligned(16))) uint16_t sW[2][P * kRowStride];
  __shared__ float qs[256];
  __shared__ float red[kCosSliceWaves][kRows][2];
  __shared__ Lds s;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int H = a.D, K = a.K;
  const int b = (int)blockIdx.x / a.G, g = (int)blockIdx.x % a.G;
  const int r0 = g * kRows, n = min(kRows, K - r0);
  const uint16_t* Xs = xc + ((size_t)b * (size_t)K + (size_t)r0) * (size_t)H;
  const int nchunks = (H + kChunk - 1) / kChunk;
  // q' is needed only after the contraction: held in a register until then,
  // so the chunk loads do not wait behind it.
  const float qv = qp[(size_t)b * P + min(tid & 255, P - 1)];
  // This thread's pieces of a chunk: row (tid % 256) / 8 of X (clamped to
  // the slice's last row; the upper 256 threads load the same pieces and
  // do not deposit them) and rows tid / 8 + 64 i of W, hidden piece tid % 8.
  const int pc = tid & 7, xrow = min((tid & 255) >> 3, n - 1);
  auto fetch = [&](int c, uint4& px, uint4 (&pw)[kWPer]) {
    const int h = min(c * kChunk + 8 * pc, H - 8);
    px = load_piece<false>(Xs + (size_t)xrow * (size_t)H + h);
#pragma unroll
    for (int i = 0; i < kWPer; ++i)
      pw[i] = load_piece<false>(wc + (size_t)((tid >> 3) + 64 * i) * (size_t)H + h);
  };
  auto deposit = [&](int buf, int c, const uint4& px, const uint4 (&pw)[kWPer]) {
    const uint32_t keep = c * kChunk + 8 * pc < H ? ~0u : 0u;
    if (tid < 256)  // uniform across the wave
      *reinterpret_cast<uint4*>(&sX[buf][(tid >> 3) * kRowStride + 8 * pc]) =
          make_uint4(px.x & keep, px.y & keep, px.z & keep, px.w & keep);
#pragma unroll
    for (int i = 0; i < kWPer; ++i)
      *reinterpret_cast<uint4*>(&sW[buf][((tid >> 3) + 64 * i) * kRowStride + 8 * pc]) =
          make_uint4(pw[i].x & keep, pw[i].y & keep, pw[i].z & keep, pw[i].w & keep);
  };
  uint4 px[kCosSliceAhead], pw[kCosSliceAhead][kWPer];
#pragma unroll
  for (int i = 0; i < kCosSliceAhead; ++i) fetch(min(i, nchunks - 1), px[i], pw[i]);
  // A block past the tile (TN < 4) is still multiplied, on a clamped W row,
  // so the matrix instructions need no branch; the epilogue drops it.
  const int wrow = min(32 * wave + (lane & 31), P - 1);
  f32x16_t acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
  // A group of kCosSliceAhead chunks. With another group to come, each
  // chunk's registers are refilled with the chunk kCosSliceAhead later as
  // soon as it sits in LDS; the last group issues no loads (so none is left
  // in flight for the epilogue to wait on) and stops at the last chunk.
  auto group = [&](auto refill, int c0) {
    constexpr bool kRefill = decltype(refill)::value;
#pragma unroll
    for (int i = 0; i < kCosSliceAhead; ++i) {
      const int c = c0 + i, buf = i & 1;
      if (!kRefill && c >= nchunks) break;  // uniform (scalar)
      // Buffer buf was last read for chunk c - 2, which every wave finished
      // before the previous barrier.
      deposit(buf, c, px[i], pw[i]);
      __syncthreads();
      if (kRefill) fetch(min(c + kCosSliceAhead, nchunks - 1), px[i], pw[i]);
#pragma unroll
      for (int ks = 0; ks < kChunk / 16; ++ks) {
        // Lane l feeds row/column l % 32 and hidden elements 8*(l/32) .. +8
        // of this 16-wide step, the same slots for both operands.
        const int kofs = 16 * ks + 8 * (lane >> 5);
        const bf16x8_t af =
            *reinterpret_cast<const bf16x8_t*>(&sX[buf][(lane & 31) * kRowStride + kofs]);
        const bf16x8_t bw =
            *reinterpret_cast<const bf16x8_t*>(&sW[buf][wrow * kRowStride + kofs]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bw, acc, 0, 0, 0);
      }
    }
  };
  int c0 = 0;
  for (; c0 + kCosSliceAhead < nchunks; c0 += kCosSliceAhead)
    group(std::integral_constant<bool, true>(), c0);
  group(std::integral_constant<bool, false>(), c0);
  if (tid < 256) qs[tid] = tid < P ? qv : 0.0f;
  __syncthreads();
  // Accumulator e of lane l: row 8*(e/4) + 4*(l/32) + e%4 of the slice,
  // feature 32*wave + l%32.
  const bool own = wave < 2 * TN;
  const float qf = qs[(32 * wave + (lane & 31)) & 255];
  float v[32];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float x = own ? acc[e] : 0.0f;
    v[e] = x * qf;
    v[16 + e] = x * x;
  }
  // Lane l ends with value l % 32 of its half: a dot (< 16) or a squared
  // norm (>= 16) of accumulator element l % 16.
  const float tot = halfwave_reduce_transposed<32>(v, lane, OpSum());
  {
    const int idx = lane & 31, e = idx & 15;
    red[wave][8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)][idx >> 4] = tot;
  }
  __syncthreads();
  if (tid < 2 * kRows) {
    const int row = tid >> 1, kind = tid & 1;
    float sum = red[0][row][kind];
#pragma unroll
    for (int w = 1; w < kCosSliceWaves; ++w) sum += red[w][row][kind];
    if (kind == 0)
      s.dot[row] = sum;
    else
      s.ss[row] = sum;
  }
  __syncthreads();
  const Question qn{(size_t)b * (size_t)K, K};
  if (wave == 0) {
    float qq = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) qq = fmaf(qs[lane + kWave * i], qs[lane + kWave * i], qq);
    qq = wave_allreduce(qq, lane, OpSum());
    const float zfac = a.zscale * rsqrtf(fmaxf(qq, kNormEps2));
    slice_softmax<true>(s, a, qn, b, g, r0, n, zfac, lane, a.G);
  }
  if (a.G > 1) split_merge(s, a, qn, b, tid, lane, wave, a.G);
}

// ---------------------------------------------------------------------------
// Cosine for small batches whose questions are split into 32-candidate
// slices anyway: the projected features are split too, one workgroup per
// (question, slice, 64-feature part). A workgroup then streams 64 rows of
// the candidate head instead of all P (a quarter for P = 256), and one
// question of 255 candidates runs on 32 compute units instead of 8. A dot
// and a squared norm are sums over the features, so each workgroup stores
// its rows' (c'.q', |c'|^2) over its part; the question's last workgroup to
// finish adds the parts in part order, forms the cosines and runs the
// softmax of the whole question.
constexpr int kCosPartWaves = 4;

template <int kF>  // projected features per part: 64 or 128
__global__ __launch_bounds__(kCosPartWaves * kWave) void proj_cos_part(
    KernelArgs a, const uint16_t* __restrict__ xc, const uint16_t* __restrict__ wc,
    const float* __restrict__ qp, float* __restrict__ rowparts, int Q) {
  constexpr int kRows = kCosSliceRows;
  constexpr int kThreads = kCosPartWaves * kWave;
  constexpr int kWPer = kF * 8 / kThreads;  // W pieces per thread per chunk
  static_assert(kF == 64 || kF == 128, "64 or 128 features per part");
  static_assert(kRows * 8 == kThreads, "one X piece per thread per chunk");
  // LDS buffers: a batch of kStages chunks is deposited, then one barrier,
  // then multiplied (all eight chunks of a 512-wide hidden size at once for
  // 64-feature parts, in two batches for 128-feature ones).
  constexpr int kStages = kF == 64 ? 8 : 4;
  static_assert(kCosSliceAhead % kStages == 0, "whole batches per group");
  __shared__ __attribute__((aligned(16))) uint16_t sX[kStages][kRows * kRowStride];
  __shared__ __attribute__((aligned(16))) uint16_t sW[kStages][kF * kRowStride];
  __shared__ float red[kF / 32][kRows][2];
  __shared__ Lds s;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int H = a.D, K = a.K, P = kF * Q;
  const int per_q = a.G * Q;  // workgroups of one question
  const int b = (int)blockIdx.x / per_q, rem = (int)blockIdx.x % per_q;
  const int g = rem / Q, j = rem % Q;
  const int r0 = g * kRows, n = min(kRows, K - r0);
  const uint16_t* Xs = xc + ((size_t)b * (size_t)K + (size_t)r0) * (size_t)H;
  const uint16_t* Ws = wc + (size_t)(kF * j) * (size_t)H;
  const int nchunks = (H + kChunk - 1) / kChunk;
  // Waves 0 .. kF/32 - 1 own the part's 32-feature blocks; all four load.
  const bool mma = wave < kF / 32;  // uniform per wave
  const float qv = qp[(size_t)b * P + kF * j + ((32 * wave + (lane & 31)) & (kF - 1))];
  // This thread's pieces of a chunk: row tid / 8 of X (clamped to the
  // slice's last row) and rows tid / 8 + 32 i (i < kWPer) of the part's W
  // rows, hidden piece tid % 8.
  const int pc = tid & 7, xrow = min(tid >> 3, n - 1);
  auto fetch = [&](int c, uint4& px, uint4 (&pw)[kWPer]) {
    const int h = min(c * kChunk + 8 * pc, H - 8);
    px = load_piece<false>(Xs + (size_t)xrow * (size_t)H + h);
#pragma unroll
    for (int i = 0; i < kWPer; ++i)
      pw[i] = load_piece<false>(Ws + (size_t)((tid >> 3) + 32 * i) * (size_t)H + h);
  };
  auto deposit = [&](int buf, int c, const uint4& px, const uint4 (&pw)[kWPer]) {
    const uint32_t keep = c * kChunk + 8 * pc < H ? ~0u : 0u;
    *reinterpret_cast<uint4*>(&sX[buf][(tid >> 3) * kRowStride + 8 * pc]) =
        make_uint4(px.x & keep, px.y & keep, px.z & keep, px.w & keep);
#pragma unroll
    for (int i = 0; i < kWPer; ++i)
      *reinterpret_cast<uint4*>(&sW[buf][((tid >> 3) + 32 * i) * kRowStride + 8 * pc]) =
          make_uint4(pw[i].x & keep, pw[i].y & keep, pw[i].z & keep, pw[i].w & keep);
  };
  uint4 px[kCosSliceAhead], pw[kCosSliceAhead][kWPer];
#pragma unroll
  for (int i = 0; i < kCosSliceAhead; ++i) fetch(min(i, nchunks - 1), px[i], pw[i]);
  const int wrow = (32 * wave + (lane & 31)) & (kF - 1);
  f32x16_t acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
  // Groups of kCosSliceAhead chunks in registers (as in proj_cos_slice),
  // each passed through LDS in batches of kStages chunks.
  auto group = [&](auto refill, int c0) {
    constexpr bool kRefill = decltype(refill)::value;
#pragma unroll
    for (int s0 = 0; s0 < kCosSliceAhead; s0 += kStages) {
      if (!kRefill && c0 + s0 >= nchunks) break;  // uniform (scalar)
      // Every wave has read the previous batch before it is overwritten.
      if (c0 + s0 > 0) __syncthreads();
#pragma unroll
      for (int i = s0; i < s0 + kStages; ++i)
        if (kRefill || c0 + i < nchunks) deposit(i - s0, c0 + i, px[i], pw[i]);
      __syncthreads();
      if (kRefill) {
#pragma unroll
        for (int i = s0; i < s0 + kStages; ++i)
          fetch(min(c0 + i + kCosSliceAhead, nchunks - 1), px[i], pw[i]);
      }
      if (mma) {
#pragma unroll
        for (int i = s0; i < s0 + kStages; ++i) {
          if (!kRefill && c0 + i >= nchunks) break;  // uniform (scalar)
#pragma unroll
          for (int ks = 0; ks < kChunk / 16; ++ks) {
            const int kofs = 16 * ks + 8 * (lane >> 5);
            const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(
                &sX[i - s0][(lane & 31) * kRowStride + kofs]);
            const bf16x8_t bw =
                *reinterpret_cast<const bf16x8_t*>(&sW[i - s0][wrow * kRowStride + kofs]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bw, acc, 0, 0, 0);
          }
        }
      }
    }
  };
  int c0 = 0;
  for (; c0 + kCosSliceAhead < nchunks; c0 += kCosSliceAhead)
    group(std::integral_constant<bool, true>(), c0);
  group(std::integral_constant<bool, false>(), c0);
  // Accumulator e of lane l (the matrix waves): row 8*(e/4) + 4*(l/32) + e%4
  // of the slice, feature kF*j + 32*wave + l%32.
  if (mma) {
    float v[32];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      v[e] = acc[e] * qv;
      v[16 + e] = acc[e] * acc[e];
    }
    const float tot = halfwave_reduce_transposed<32>(v, lane, OpSum());
    const int idx = lane & 31, e = idx & 15;
    red[wave][8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)][idx >> 4] = tot;
  }
  __syncthreads();
  // Wave 0 stores the rows' partials over this part: row k of question b,
  // part j at ((b * 256 + k) * Q + j) * 2 (+1 for the squared norm).
  float* const rq = rowparts + (size_t)b * kMaxSlots * (size_t)Q * 2;
  if (tid < 2 * kRows) {
    const int row = tid >> 1, kind = tid & 1;
    float sum = red[0][row][kind];
#pragma unroll
    for (int w = 1; w < kF / 32; ++w) sum += red[w][row][kind];
    if (row < n) rq[((size_t)(r0 + row) * Q + j) * 2 + kind] = sum;
  }
  // Wave 0 publishes its stores at agent scope (every XCD) and draws the
  // question's ticket; the last of the question's workgroups merges.
  if (wave == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (lane == 0) {
      const unsigned t =
          __hip_atomic_fetch_add(a.tickets + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s.last = t == (unsigned)(per_q - 1);
    }
  }
  __syncthreads();
  if (!s.last) return;  // uniform across the workgroup
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  for (int k = tid; k < K; k += kThreads) {
    float d = 0.0f, q2 = 0.0f;
    for (int jj = 0; jj < Q; ++jj) {
      d += rq[((size_t)k * Q + jj) * 2];
      q2 += rq[((size_t)k * Q + jj) * 2 + 1];
    }
    s.dot[k] = d;
    s.ss[k] = q2;
  }
  __syncthreads();
  if (wave == 0) {
    float qq = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxSlots / kWave; ++i) {
      const int f = lane + kWave * i;
      const float x = f < P ? qp[(size_t)b * P + f] : 0.0f;
      qq = fmaf(x, x, qq);
    }
    qq = wave_allreduce(qq, lane, OpSum());
    const float zfac = a.zscale * rsqrtf(fmaxf(qq, kNormEps2));
    const Question qn{(size_t)b * (size_t)K, K};
    slice_softmax<true, false>(s, a, qn, b, 0, 0, K, zfac, lane, 1);
  }
  if (tid == 0) __hip_atomic_store(a.tickets + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// The same cosine tile with asynchronous staging (Hc % 64 == 0): the hidden
// dimension moves through two LDS stages of 64 bf16 per row, filled by
// global_load_lds_dwordx4 (no staging registers): one chunk is in flight
// while the matrix cores work on the other. Rows of 128 bytes make every
// request to L2 a whole cache line (half-line requests held the per-CU
// request queue to half the bytes in flight). The DMA writes each wave's 64
// lanes to 1 KiB of consecutive LDS, i.e. 8 rows; to keep the fragment reads
// free of bank conflicts, the lane that fills 16-byte position p of row r
// fetches piece p ^ f(r) of that row (an XOR swizzle instead of padding),
// and readers undo it.
//
// Every stage of each operand is an LDS object of its own, and the fragment
// reads are ordinary loads. The compiler tracks which LDS object a DMA in
// flight writes, so a read from one stage does not wait for the refill of the
// other; where a read does depend on this wave's own DMA, the compiler's wait
// covers it. The ring's explicit vmcnt waits and barriers add what the
// compiler cannot see: that the other waves' DMAs into a stage have landed.
constexpr int kAChunk = 64;                        // bf16 per row per stage
constexpr int kAStages = 2;                        // 128 KiB of LDS
constexpr int kARowBytes = 2 * kAChunk;            // 128
constexpr int kAPieces = kARowBytes / 16;          // 8 pieces of 16 bytes per row
constexpr int kARowsPerLoad = 1024 / kARowBytes;   // 8 rows per DMA instruction
constexpr int kATileBytes = 256 * kARowBytes;      // X or W tile of one stage: 32 KiB
constexpr int kAKSteps = kAChunk / 16;             // 4 MFMA k-steps per chunk

__shared__ __attribute__((aligned(1024))) uint8_t g_xs0[kATileBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_xs1[kATileBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_ws0[kATileBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_ws1[kATileBytes];
__shared__ __attribute__((aligned(1024))) float g_qp[256];  // q' of the current question

#ifdef CS_PHASE_CLOCKS
// Measurement build only: per-wave cycle clocks of the cosine ring kernel.
// Record (workgroup < 256, wave) holds, for the workgroup's second question,
// s_memtime at five points of each of its first eight chunk steps (entry,
// after the vmcnt wait, after the barrier, after the DMA issue, after the
// matrix work: slots 5c .. 5c+4) and at five points of its epilogue (entry,
// after the row reductions, after the first and the second barrier, exit:
// slots 40-44). Slots 45-48 hold s_memtime and s_memrealtime at the epilogue
// exit of the first and the third question, which convert cycles to time.
constexpr int kRingClkGroups = 256, kRingClkSlots = 49;
}  // namespace
// (Outside the anonymous namespace, so the host can copy it by symbol.)
__device__ unsigned long long g_ring_clk[kRingClkGroups * 8 * kRingClkSlots];
namespace {
#define CS_RING_CLK(cond, slot, value)                                                   \
  do {                                                                                   \
    if ((cond) && lane == 0 && blockIdx.x < (unsigned)kRingClkGroups)                    \
      g_ring_clk[(blockIdx.x * 8 + wave) * kRingClkSlots + (slot)] = (value);            \
  } while (0)
#else
#define CS_RING_CLK(cond, slot, value) \
  do {                                 \
  } while (0)
#endif

// X tile (W == false) or W tile (W == true) of stage S.
template <int S, bool W>
__device__ __forceinline__ uint8_t* stage_tile() {
  static_assert(S >= 0 && S < kAStages, "stage index");
  if constexpr (S == 0)
    return W ? g_ws0 : g_xs0;
  else
    return W ? g_ws1 : g_xs1;
}

// Workgroup barrier for the stage ring: this wave's LDS reads are complete
// (lgkmcnt 0) before it arrives, and no memory access is moved across it by
// the compiler. Unlike __syncthreads it does not wait for the DMA loads still
// in flight; the callers wait for exactly the ones they need.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// DMA of hidden chunk c into stage S: this wave fills rows RPW*wave .. +RPW
// of the X tile and of the W tile (RPW = 256 / waves). X rows past K repeat
// row K-1 and W rows past P repeat row P-1; those rows are never read. (The
// helpers take plain pointers: restrict-qualified parameters of an inlined
// function would give every call site alias scopes of its own.)
// DMA of hidden chunk c into stage S: this wave fills rows RPW*wave .. +RPW
// of the X tile and of the W tile. X rows past K repeat row K-1 and W rows
// past P repeat row P-1; those rows are never read. The per-lane offsets
// (32-bit: the host keeps K*H*2 below 2^31) are recomputed for every fill
// from an opaque copy of the lane index, so the compiler cannot hoist them
// out of the chunk loop and hold them in registers beside the accumulators.
template <int S, int RPW, bool NT>
__device__ __forceinline__ void stage_fill(const uint16_t* Xb, const uint16_t* wc, int c, int K,
                                           int P, int H, int wave, int lane) {
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(Xb) + (size_t)c * kARowBytes;
  const uint8_t* wb = reinterpret_cast<const uint8_t*>(wc) + (size_t)c * kARowBytes;
#pragma unroll
  for (int j = 0; j < RPW / kARowsPerLoad; ++j) {
    const int r0 = RPW * wave + kARowsPerLoad * j;
    const int row = r0 + ln / kAPieces;
    const int piece = swizzled_piece(row, ln % kAPieces);
    const uint32_t xo = (uint32_t)(2 * (min(row, K - 1) * H + 8 * piece));
    const uint32_t wo = (uint32_t)(2 * (min(row, P - 1) * H + 8 * piece));
    __builtin_amdgcn_global_load_lds((global_ptr_t)(xb + xo),
                                     (lds_ptr_t)(stage_tile<S, false>() + r0 * kARowBytes), 16, 0,
                                     NT ? 2 : 0);
    __builtin_amdgcn_global_load_lds((global_ptr_t)(wb + wo),
                                     (lds_ptr_t)(stage_tile<S, true>() + r0 * kARowBytes), 16, 0,
                                     0);
  }
}

// Fragment reads of one 16-wide step: N 32-row blocks, 4 KiB apart, from
// base (an address inside one stage tile).
template <int N>
__device__ __forceinline__ void lds_blocks(bf16x8_t (&f)[N], const uint8_t* base) {
  static_assert(N >= 1 && N <= 8, "blocks per step");
#pragma unroll
  for (int i = 0; i < N; ++i)
    f[i] = *reinterpret_cast<const bf16x8_t*>(base + i * 32 * kARowBytes);
}

// Per-lane byte offsets of the 16-wide steps of a chunk inside an X tile
// (rows 32*RB*wr + lane%32, +32, ...) and a W tile (rows 32*TN*wcb + lane%32,
// +32, ...). The swizzle depends on row % 16 only, so the 32-row blocks of
// one lane share it and sit 4 KiB apart.
struct StageOffsets {
  uint32_t x[kAKSteps], w[kAKSteps];
};

template <int TN, int RB>
__device__ __forceinline__ StageOffsets stage_offsets(int lane, int wr, int col0) {
  StageOffsets o;
  const int rx = 32 * RB * wr + (lane & 31), rw = col0 + (lane & 31);
#pragma unroll
  for (int ks = 0; ks < kAKSteps; ++ks) {
    const int piece = 2 * ks + (lane >> 5);
    o.x[ks] = (uint32_t)(rx * kARowBytes + 16 * swizzled_piece(rx, piece));
    o.w[ks] = (uint32_t)(rw * kARowBytes + 16 * swizzled_piece(rw, piece));
  }
  return o;
}

// The matrix-core work of one chunk: RB x TN accumulators, four 16-wide
// steps. The fragments of step ks+1 are read while the matrix cores work on
// step ks (scheduling barriers keep the compiler from merging the phases).
template <int S, int TN, int RB>
__device__ __forceinline__ void stage_mfma(f32x16_t (&acc)[RB][TN], const StageOffsets& o) {
  const uint8_t* xs = stage_tile<S, false>();
  const uint8_t* ws = stage_tile<S, true>();
  bf16x8_t af[2][RB], bfr[2][TN];
  lds_blocks<RB>(af[0], xs + o.x[0]);
  lds_blocks<TN>(bfr[0], ws + o.w[0]);
#pragma unroll
  for (int ks = 0; ks < kAKSteps; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < kAKSteps) {
      lds_blocks<RB>(af[cur ^ 1], xs + o.x[ks + 1]);
      lds_blocks<TN>(bfr[cur ^ 1], ws + o.w[ks + 1]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        acc[rb][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][rb], bfr[cur][tn],
                                                              acc[rb][tn], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One chunk of the ring: wait until chunk c (stage S) of the current question
// has landed for every wave, refill the stage freed by chunk c-1 with chunk
// c+1, multiply chunk c. Chunk c+1 may be the first of the next question of
// this workgroup (Xn; null when there is none or when questions do not carry
// the ring). The step with c < 0 only fills (the start of the ring).
constexpr int kDmaWaves = 4;

template <int S, int TN, int RB, bool NT, bool DMA>
__device__ __forceinline__ void stage_step(f32x16_t (&acc)[RB][TN], const StageOffsets& o,
                                           const uint16_t* Xb, const uint16_t* Xn,
                                           const uint16_t* wc, int c, int nchunks, int K, int H,
                                           int wave, int lane, int P, int qi) {
  if (c >= nchunks) return;
  [[maybe_unused]] const bool clk = qi == 1 && c >= 0 && c < 8;
  CS_RING_CLK(clk, 5 * c, __builtin_amdgcn_s_memtime());
  if (c >= 0) {
    // With two stages the only chunk in flight is c itself (issued at the
    // start of the previous step); stores issued since only add to the wait.
    // The other waves issue no DMA and do not wait for their stores.
    if constexpr (DMA) wait_vmcnt<0>();
    CS_RING_CLK(clk, 5 * c + 1, __builtin_amdgcn_s_memtime());
    stage_barrier();
    CS_RING_CLK(clk, 5 * c + 2, __builtin_amdgcn_s_memtime());
  }
  int next = c + kAStages - 1;
  const uint16_t* src = Xb;
  if (next >= nchunks) {
    next -= nchunks;
    src = Xn;
  }
  // Waves 0 .. 3 (one per SIMD, DMA) issue the chunk's DMAs, 64 rows each;
  // the other wave of each SIMD goes straight to its matrix work, so the
  // SIMD's matrix core is not idle while the DMA instructions queue for the
  // memory pipeline (all eight waves issuing measured 3-5 % slower).
  if (DMA && next >= 0 && src != nullptr)
    stage_fill<(S + kAStages - 1) % kAStages, 256 / kDmaWaves, NT>(src, wc, next, K, P, H,
                                                                   wave, lane);
  CS_RING_CLK(clk, 5 * c + 3, __builtin_amdgcn_s_memtime());
  if (c >= 0) stage_mfma<S, TN, RB>(acc, o);
  CS_RING_CLK(clk, 5 * c + 4, __builtin_amdgcn_s_memtime());
}

// DMA of the current question's q' (P floats) into g_qp by one wave: lane l
// brings floats 4l .. 4l+3 (lanes past P repeat the last four; unused).
__device__ __forceinline__ void qp_fill(const float* qrow, int P, int lane) {
  const float* src = qrow + min(4 * lane, P - 4);
  __builtin_amdgcn_global_load_lds((global_ptr_t)src, (lds_ptr_t)g_qp, 16, 0, 0);
}

// Epilogue of the ring kernel: as cos_epilogue, with q' taken from g_qp
// (brought in by DMA when the question started, so nothing here waits on the
// vector-memory counter) and barriers that do not wait for the next
// question's DMAs already in flight. The ring's last wait covered the q' DMA,
// which wave 0 issued before the question's later chunks.
template <int TN, int RB, int PT>
__device__ __forceinline__ void cos_epilogue_ring(Lds& s, const KernelArgs& a,
                                                  const f32x16_t (&acc)[RB][TN], int b, int K,
                                                  int lane, int wave, int wr, int wcb, int col0,
                                                  int qi, bool now) {
  CS_RING_CLK(qi == 1, 40, __builtin_amdgcn_s_memtime());
  float qv[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) qv[tn] = g_qp[col0 + 32 * tn + (lane & 31)];
  // Accumulator e of tile (rb, tn) in lane l holds C'[row][col] with
  // row = 32*RB*wr + 32*rb + 8*(e/4) + 4*(l/32) + e%4 and
  // col = 32*TN*wcb + 32*tn + l%32; pairs of row blocks are reduced at once.
  float dsum[RB / 2], esum[RB / 2];
#pragma unroll
  for (int pr = 0; pr < RB / 2; ++pr) {
    float dv[32], ev[32];
#pragma unroll
    for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float d = 0.0f, q2 = 0.0f;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const float c = acc[2 * pr + r2][tn][e];
          d = fmaf(c, qv[tn], d);
          q2 = fmaf(c, c, q2);
        }
        dv[16 * r2 + e] = d;
        ev[16 * r2 + e] = q2;
      }
    dsum[pr] = halfwave_reduce_transposed<32>(dv, lane, OpSum());
    esum[pr] = halfwave_reduce_transposed<32>(ev, lane, OpSum());
  }
  const int v = lane & 31, e = v & 15;
  const int row0 = 32 * RB * wr + 32 * (v >> 4) + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
  CS_RING_CLK(qi == 1, 41, __builtin_amdgcn_s_memtime());
  // The two column halves of a row are added in a fixed order.
  if (wcb == 0) {
#pragma unroll
    for (int pr = 0; pr < RB / 2; ++pr) {
      s.dot[row0 + 64 * pr] = dsum[pr];
      s.ss[row0 + 64 * pr] = esum[pr];
    }
  }
  stage_barrier();
  CS_RING_CLK(qi == 1, 42, __builtin_amdgcn_s_memtime());
  if (wcb == 1) {
#pragma unroll
    for (int pr = 0; pr < RB / 2; ++pr) {
      s.dot[row0 + 64 * pr] += dsum[pr];
      s.ss[row0 + 64 * pr] += esum[pr];
    }
  }
  stage_barrier();
  CS_RING_CLK(qi == 1, 43, __builtin_amdgcn_s_memtime());
  if (wave == 0) {
    float qpv[PT];
#pragma unroll
    for (int i = 0; i < PT; ++i) qpv[i] = g_qp[lane + kWave * i];
    float qq = 0.0f;
#pragma unroll
    for (int i = 0; i < PT; ++i) qq = fmaf(qpv[i], qpv[i], qq);
    qq = wave_allreduce(qq, lane, OpSum());
    const float zfac = a.zscale * rsqrtf(fmaxf(qq, kNormEps2));
    if (now) {
      const Question qn{(size_t)b * (size_t)K, K};
      slice_softmax<true>(s, a, qn, b, 0, 0, K, zfac, lane, a.G);
    } else if (lane == 0) {
      s.red[0] = zfac;  // for the softmax that the next question's first chunk step runs
    }
  }
  // No barrier here: the next question's first ring barrier orders these
  // LDS writes before the deferred softmax reads them, and s.dot / s.ss /
  // s.red are written again only by the next epilogue.
}

// The softmax of a workgroup's question other than its last runs on wave
// kSoftmaxWave after that wave's share of the next question's first chunk:
// those waves (4-7) wait ~1.4k cycles per chunk step at the next barrier,
// while on wave 0 at the end of the epilogue the ~1.9k-cycle softmax held
// up every wave at the next question's first barrier. The second chunk's
// barrier then separates it from the next epilogue's writes of the row
// sums, so questions of one chunk keep the softmax in the epilogue.
constexpr int kSoftmaxWave = 4;

// A workgroup takes questions blockIdx.x, blockIdx.x + gridDim.x, ... and,
// when the chunk count is even, keeps the ring running across them: the first
// chunk of the next question is in flight during the last step and the
// epilogue of the current one. 8 waves; wave w owns rows 64 (w % 4) .. +64
// (RB = 2 row blocks of 32) and a run of TNW 32-feature column blocks
// starting at feature col0. The two waves of a SIMD share its matrix core,
// and the one that issues the chunk's DMAs (waves 0-3, stalled while the
// requests queue) takes TN - 1 of the question's 2 TN column blocks, the
// other TN + 1: with TN each, the 1024-question CLM batch took 84.7 us
// (kernel trace) against 81.3 us, and a 2 / 6 split spills.
template <int TNW, int PT, bool NT, int RB, bool DMA>
__device__ __forceinline__ void cos_ring_role(Lds& s, const KernelArgs& a,
                                              const uint16_t* __restrict__ xc,
                                              const uint16_t* __restrict__ wc,
                                              const float* __restrict__ qp, int wave, int lane,
                                              int wr, int wcb, int col0) {
  constexpr int P = 64 * PT;
  const int H = a.D, K = a.K;
  const int nchunks = H / kAChunk;
  // The host launches this kernel for H >= 64 only. Knowing that the chunk
  // loop runs, the compiler sees every path to the epilogue pass a step's
  // vmcnt(0) wait after the q' DMA, and lets the epilogue's reads of g_qp go
  // ahead while the next question's first chunk is in flight.
  __builtin_assume(nchunks >= 1);
  const bool carry = nchunks % kAStages == 0;
  const int stride = (int)gridDim.x;
  const StageOffsets o = stage_offsets<TNW, RB>(lane, wr, col0);
  int pending = -1;  // question whose softmax is still to run (wave kSoftmaxWave)
  for (int b = blockIdx.x; b < a.B; b += stride) {
    [[maybe_unused]] const int qi = (b - (int)blockIdx.x) / stride;  // clocks only
    const uint16_t* Xb = xc + (size_t)b * (size_t)K * (size_t)H;
    const uint16_t* Xn =
        (carry && b + stride < a.B) ? xc + (size_t)(b + stride) * (size_t)K * (size_t)H : nullptr;
    if (DMA && wave == 0) qp_fill(qp + (size_t)b * P, P, lane);
    f32x16_t acc[RB][TNW];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int tn = 0; tn < TNW; ++tn)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[rb][tn][e] = 0.0f;
    if (!carry || b == (int)blockIdx.x)
      stage_step<1, TNW, RB, NT, DMA>(acc, o, Xb, Xn, wc, -1, nchunks, K, H, wave, lane, P, qi);
    for (int c = 0; c < nchunks; c += kAStages) {
      stage_step<0, TNW, RB, NT, DMA>(acc, o, Xb, Xn, wc, c, nchunks, K, H, wave, lane, P, qi);
      if (!DMA && c == 0 && wave == kSoftmaxWave && pending >= 0) {
        const Question qn{(size_t)pending * (size_t)K, K};
        slice_softmax<true>(s, a, qn, pending, 0, 0, K, s.red[0], lane, a.G);
      }
      stage_step<1, TNW, RB, NT, DMA>(acc, o, Xb, Xn, wc, c + 1, nchunks, K, H, wave, lane, P, qi);
    }
    const bool now = b + stride >= a.B || nchunks < 2;  // uniform
    cos_epilogue_ring<TNW, RB, PT>(s, a, acc, b, K, lane, wave, wr, wcb, col0, qi, now);
    pending = now ? -1 : b;
    CS_RING_CLK(qi == 1, 44, __builtin_amdgcn_s_memtime());
    CS_RING_CLK(qi == 0 || qi == 2, qi == 0 ? 45 : 47, __builtin_amdgcn_s_memtime());
    CS_RING_CLK(qi == 0 || qi == 2, qi == 0 ? 46 : 48, __builtin_amdgcn_s_memrealtime());
  }
}

template <int TN, bool NT, int RB>
__global__ __launch_bounds__(64 * (16 / RB)) void proj_cos_mfma_async(
    KernelArgs a, const uint16_t* __restrict__ xc, const uint16_t* __restrict__ wc,
    const float* __restrict__ qp) {
  static_assert(kAStages == 2, "the chunk loop is unrolled by the stage count");
  static_assert(RB == 2, "row blocks per wave");
  __shared__ Lds s;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int wr = wave % 4, wcb = wave / 4;
  static_assert(kDmaWaves == 4 && kSoftmaxWave >= 4, "waves 0-3 issue the DMAs");
  if constexpr (TN >= 2) {
    if (wcb == 0)
      cos_ring_role<TN - 1, TN, NT, RB, true>(s, a, xc, wc, qp, wave, lane, wr, 0, 0);
    else
      cos_ring_role<TN + 1, TN, NT, RB, false>(s, a, xc, wc, qp, wave, lane, wr, 1, 32 * (TN - 1));
  } else {
    if (wcb == 0)
      cos_ring_role<TN, TN, NT, RB, true>(s, a, xc, wc, qp, wave, lane, wr, 0, 0);
    else
      cos_ring_role<TN, TN, NT, RB, false>(s, a, xc, wc, qp, wave, lane, wr, 1, 32 * TN);
  }
}

// ---------------------------------------------------------------------------
// Launch helpers.

template <int NV, int R, bool NT>
hipError_t launch_bf16_dot_nv(const KernelArgs& a, const ProjArgs& p, unsigned grid,
                              unsigned block, hipStream_t stream) {
  const bool full = (p.Hc >> 3) == NV * kWave;
  if (full)
    hipLaunchKernelGGL((fused_bf16_dot<NV, R, true, NT>), dim3(grid), dim3(block), 0, stream, a,
                       p.xc, p.u);
  else
    hipLaunchKernelGGL((fused_bf16_dot<NV, R, false, NT>), dim3(grid), dim3(block), 0, stream, a,
                       p.xc, p.u);
  return hipGetLastError();
}

template <bool NT>
hipError_t launch_bf16_dot(const KernelArgs& a, const ProjArgs& p, int nv, hipStream_t stream) {
  const int R = bf16_rows_per_wave(nv);
  // Four waves per question: at 127 registers a CU holds four such
  // workgroups, so a 1024-question batch is resident at once (eight-wave
  // workgroups ran in two rounds and measured about 1 % slower). A split
  // batch has at most one slice per compute unit, so its slices take eight
  // waves: twice the loads in flight on each unit.
  const int rpg = (p.K + p.G - 1) / p.G;
  const int waves = std::max(1, std::min(p.G > 1 ? 8 : 4, (rpg + R - 1) / R));
  const unsigned grid = (unsigned)std::min<long long>((long long)p.B * p.G, 1 << 20);
  const unsigned block = (unsigned)(waves * kWave);
  switch (nv) {
    case 1: return launch_bf16_dot_nv<1, 8, NT>(a, p, grid, block, stream);
    case 2: return launch_bf16_dot_nv<2, 4, NT>(a, p, grid, block, stream);
    case 3: return launch_bf16_dot_nv<3, 4, NT>(a, p, grid, block, stream);
    case 4: return launch_bf16_dot_nv<4, 2, NT>(a, p, grid, block, stream);
    case 5: return launch_bf16_dot_nv<5, 2, NT>(a, p, grid, block, stream);
    case 6: return launch_bf16_dot_nv<6, 2, NT>(a, p, grid, block, stream);
    case 8: return launch_bf16_dot_nv<8, 2, NT>(a, p, grid, block, stream);
    default: return hipErrorInvalidValue;
  }
}

// Eight waves of 64-row tiles. (Four waves of 128-row tiles would need fewer
// fragment reads per matrix instruction, but their 256 accumulators leave
// too few vector registers and the compiler spills.)
constexpr int kCosRowBlocks = 2;

template <int TN, bool NT>
void launch_cos_tile(const KernelArgs& a, const ProjArgs& p, unsigned grid, hipStream_t stream) {
  // The ring's DMA offsets are 32-bit byte offsets into a question's rows.
  if (p.Hc % kAChunk == 0 && 2LL * p.K * p.Hc < (1LL << 31))
    // One resident workgroup per compute unit (its LDS allows no more), each
    // working through its share of the questions.
    hipLaunchKernelGGL((proj_cos_mfma_async<TN, NT, kCosRowBlocks>),
                       dim3(p.compute_units > 0 ? std::min(grid, (unsigned)p.compute_units) : grid),
                       dim3(64 * (16 / kCosRowBlocks)), 0, stream, a, p.xc, p.wc, p.qp);
  else
    hipLaunchKernelGGL((proj_cos_mfma<TN, NT>), dim3(grid), dim3(512), 0, stream, a, p.xc, p.wc,
                       p.qp);
}

template <bool NT>
hipError_t launch_cos_mfma(const KernelArgs& a, const ProjArgs& p, hipStream_t stream) {
  if (p.cos_parts > 0) {
    // Small batch of split questions: B * G * (P / 64) workgroups.
    const dim3 grid((unsigned)(p.B * p.G * p.cos_parts)), block(kCosPartWaves * kWave);
    if (p.P / p.cos_parts == 128)
      hipLaunchKernelGGL(proj_cos_part<128>, grid, block, 0, stream, a, p.xc, p.wc, p.qp,
                         p.rowparts, p.cos_parts);
    else
      hipLaunchKernelGGL(proj_cos_part<64>, grid, block, 0, stream, a, p.xc, p.wc, p.qp,
                         p.rowparts, p.cos_parts);
    return hipGetLastError();
  }
  if (p.cos_slice) {
    // Small batch: B * G workgroups (at most one per compute unit).
    const dim3 grid((unsigned)(p.B * p.G)), block(kCosSliceWaves * kWave);
    switch (p.P / 64) {
      case 1: hipLaunchKernelGGL(proj_cos_slice<1>, grid, block, 0, stream, a, p.xc, p.wc, p.qp); break;
      case 2: hipLaunchKernelGGL(proj_cos_slice<2>, grid, block, 0, stream, a, p.xc, p.wc, p.qp); break;
      case 3: hipLaunchKernelGGL(proj_cos_slice<3>, grid, block, 0, stream, a, p.xc, p.wc, p.qp); break;
      case 4: hipLaunchKernelGGL(proj_cos_slice<4>, grid, block, 0, stream, a, p.xc, p.wc, p.qp); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const unsigned grid = (unsigned)std::min(p.B, 1 << 20);
  switch (p.P / 64) {
    case 1: launch_cos_tile<1, NT>(a, p, grid, stream); break;
    case 2: launch_cos_tile<2, NT>(a, p, grid, stream); break;
    case 3: launch_cos_tile<3, NT>(a, p, grid, stream); break;
    case 4: launch_cos_tile<4, NT>(a, p, grid, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int bf16_rows_per_wave(int nv) { return nv <= 1 ? 8 : nv <= 3 ? 4 : 2; }

int bf16_nv_for(int Hc) {
  const int pieces = Hc / 8;
  const int need = (pieces + kWave - 1) / kWave;
  static const int kNv[] = {1, 2, 3, 4, 5, 6, 8};
  for (int nv : kNv)
    if (nv >= need) return nv;
  return 0;
}

hipError_t launch_projected(const ProjArgs& p, hipStream_t stream) {
  KernelArgs a{};
  a.out = p.out;
  a.B = p.B;
  a.K = p.K;
  a.D = p.Hc;
  a.G = p.G;
  a.rpg = p.cosine ? kCosSliceRows : (p.K + p.G - 1) / p.G;
  a.tickets = a.G > 1 ? p.tickets : nullptr;
  a.partials = a.G > 1 ? p.partials : nullptr;
  a.zscale = p.zscale;
  a.cosine = p.cosine;
  const bool few = p.B <= kGemvMaxB;
  if (few) {
    // At most eight questions: q' as matrix-vector products from Wq's own
    // layout (and, for dot, u from Wc's, with no packing).
    // One wave (one head row) per workgroup, so the rows spread over every
    // compute unit: each wave also loads all the questions' rows, and with
    // four waves per workgroup a compute unit carried four such copies
    // (eight questions of the Kev heads 20.2 -> 18.9 us per call, one
    // 11.45 -> 11.2 us; with two waves 19.2 and 11.3 us).
    const unsigned qgroups = (unsigned)p.P;
    auto launch = [&](auto query) {
      hipLaunchKernelGGL(query, dim3(qgroups), dim3(kWave), 0, stream, p.xq, p.wq, p.qp, p.B, p.Hq,
                         p.P, a.tickets);
    };
    if (p.B == 1) launch(proj_query_gemv<1>);
    else if (p.B == 2) launch(proj_query_gemv<2>);
    else if (p.B <= 4) launch(proj_query_gemv<4>);
    else launch(proj_query_gemv<8>);
  } else {
    // q' = Wq x_q for every question: one workgroup per 32 x 32 tile.
    const long long tiles = (long long)((p.B + 31) / 32) * ((p.P + 31) / 32);
    // Dot also packs Wc^T in this launch: at least one workgroup per compute
    // unit, so that a small batch does not pack it on a few of them.
    const long long cus = p.compute_units > 0 ? p.compute_units : 256;
    const long long groups = p.cosine ? tiles : std::max(tiles, cus);
    // Blocks in flight per wave: every whole block of a wave's share up to
    // ten (more take further rounds), so short hidden sizes issue no
    // repeated loads.
    const int per_wave = (p.Hq / 32 + kPqWaves - 1) / kPqWaves;
    auto launch = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, dim3((unsigned)groups), dim3(kPqWaves * kWave), 0, stream, p.xq,
                         p.wq, p.qp, p.cosine ? nullptr : p.parts, p.B, p.Hq, p.P, p.wc,
                         p.cosine ? nullptr : p.wpack, p.Hc, a.tickets, tiles);
    };
    if (per_wave <= 1) launch(proj_query_mfma<1>);
    else if (per_wave <= 2) launch(proj_query_mfma<2>);
    else if (per_wave <= 4) launch(proj_query_mfma<4>);
    else if (per_wave <= 6) launch(proj_query_mfma<6>);
    else launch(proj_query_mfma<10>);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (p.cosine) return p.nt ? launch_cos_mfma<true>(a, p, stream) : launch_cos_mfma<false>(a, p, stream);
  // u = Wc^T q', then one bandwidth-bound pass over the candidates.
  if (few) {
    const unsigned fgroups = (unsigned)((p.Hc / 8 + kFoldGemvPieces - 1) / kFoldGemvPieces);
    auto launch = [&](auto fold) {
      hipLaunchKernelGGL(fold, dim3(fgroups), dim3(256), 0, stream, p.qp, p.wc, p.u, p.B, p.Hc,
                         p.P);
    };
    if (p.B == 1) launch(fold_query_gemv<1>);
    else if (p.B == 2) launch(fold_query_gemv<2>);
    else if (p.B <= 4) launch(fold_query_gemv<4>);
    else launch(fold_query_gemv<8>);
  } else {
    // One wave per 32 questions x 128 h.
    const long long tiles =
        (long long)((p.B + 31) / 32) * ((p.Hc + 32 * kFoldNb - 1) / (32 * kFoldNb));
    const long long cus = p.compute_units > 0 ? p.compute_units : 256;
    if (tiles < cus)  // too few tiles to fill the chip: four waves per tile
      hipLaunchKernelGGL(fold_query_mfma_split, dim3((unsigned)tiles),
                         dim3(kFoldSplitWaves * kWave), 0, stream, p.parts, p.wpack, p.u, p.B,
                         p.Hc, p.P);
    else
      hipLaunchKernelGGL(fold_query_mfma, dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0, stream,
                         p.parts, p.wpack, p.u, p.B, p.Hc, p.P);
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int nv = bf16_nv_for(p.Hc);
  return p.nt ? launch_bf16_dot<true>(a, p, nv, stream) : launch_bf16_dot<false>(a, p, nv, stream);
}

}  // namespace cs

#ifdef CS_PHASE_CLOCKS
// Measurement build only: the phase clocks of this file's kernels (regions
// 1-3, same layout as cs_phase_clocks_read), copied to host memory.
extern "C" int cs_projected_phase_clocks_read(void* dst, size_t bytes) {
  return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(cs::g_phase_clk), bytes, 0,
                                  hipMemcpyDeviceToHost);
}

// The cosine ring kernel's per-wave clocks (256 x 8 records of 49 values).
extern "C" int cs_ring_phase_clocks_read(void* dst, size_t bytes) {
  return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(cs::g_ring_clk), bytes, 0,
                                  hipMemcpyDeviceToHost);
}
#endif
