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
//    the query. proj_query makes q' [B][P], fold_query makes u = Wc^T q'
//    [B][Hc], and fused_bf16_dot streams the bf16 candidate rows once against
//    u, with the same in-workgroup softmax as the plain scoring kernels. The
//    candidate side stays a bandwidth-bound pass; no candidate is projected.
//  * cosine (CLM): the norm |Wc x_k| needs the projected rows, a dense
//    contraction: proj_cos_mfma computes, per question, the tile
//    C' = X Wc^T (255 x P, X [K][Hc]) with v_mfma_f32_32x32x16_bf16, keeps it
//    in registers, and reduces each row to (c'.q', |c'|^2) in its epilogue;
//    the projected candidates never reach global memory.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>

#include "cs_device.h"
#include "cs_launch.h"

namespace cs {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

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
// q'[b][p] = sum_h x[b][h] * w[p][h]  (x [B][H], w [P][H], bf16; H % 8 == 0).
// A wave computes an 8-question x 8-output tile: lane l reads 16-byte pieces
// 8l, 8l + 512, ... of the 8 query rows and the 8 weight rows (every load a
// contiguous 1 KiB across the wave), accumulates the 64 partial dots, and one
// transposed 64-value reduction leaves output (l / 8, l % 8) in lane l.
__global__ __launch_bounds__(256) void proj_query(const uint16_t* __restrict__ x,
                                                  const uint16_t* __restrict__ w,
                                                  float* __restrict__ q, int B, int H, int P) {
  const int lane = threadIdx.x & (kWave - 1);
  const long long wid = (long long)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int ptiles = (P + 7) / 8;
  const long long b0 = (wid / ptiles) * 8;
  const int p0 = (int)(wid % ptiles) * 8;
  if (b0 >= B) return;  // uniform across the wave
  float acc[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) acc[i] = 0.0f;
  for (int h = 8 * lane; h < H; h += 8 * kWave) {
    float wf[8][8];
#pragma unroll
    for (int pp = 0; pp < 8; ++pp) {
      const uint4 v = (p0 + pp < P) ? load_piece<false>(w + (size_t)(p0 + pp) * (size_t)H + h)
                                    : make_uint4(0u, 0u, 0u, 0u);
      wf[pp][0] = bf_lo(v.x); wf[pp][1] = bf_hi(v.x); wf[pp][2] = bf_lo(v.y); wf[pp][3] = bf_hi(v.y);
      wf[pp][4] = bf_lo(v.z); wf[pp][5] = bf_hi(v.z); wf[pp][6] = bf_lo(v.w); wf[pp][7] = bf_hi(v.w);
    }
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) {
      const uint4 v = (b0 + bb < B) ? load_piece<false>(x + (size_t)(b0 + bb) * (size_t)H + h)
                                    : make_uint4(0u, 0u, 0u, 0u);
      const float xf[8] = {bf_lo(v.x), bf_hi(v.x), bf_lo(v.y), bf_hi(v.y),
                           bf_lo(v.z), bf_hi(v.z), bf_lo(v.w), bf_hi(v.w)};
#pragma unroll
      for (int pp = 0; pp < 8; ++pp)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[8 * bb + pp] = fmaf(xf[e], wf[pp][e], acc[8 * bb + pp]);
    }
  }
  const float total = wave_reduce_transposed<64>(acc, lane, OpSum());
  const long long b = b0 + lane / 8;
  const int p = p0 + lane % 8;
  if (b < B && p < P) q[(size_t)b * (size_t)P + p] = total;
}

// u[b][h] = sum_p q'[b][p] * w[p][h]  (q' [B][P] fp32, w [P][H] bf16,
// P <= 256, H % 8 == 0). A workgroup computes 4 questions x 512 consecutive
// h; lane l owns h = 8l .. 8l+7. The feature sum is split over the 4 waves
// (wave w takes features p = w, w+4, ...), each reading one 16-byte piece of
// weight row p per step (1 KiB contiguous across the wave) and the 4
// questions' q'[.][p] as one broadcast LDS read; the four partial sums are
// then added in wave order through LDS.
__global__ __launch_bounds__(256) void fold_query(const float* __restrict__ q,
                                                  const uint16_t* __restrict__ w,
                                                  float* __restrict__ u, int B, int H, int P) {
  __shared__ float4 qs[256];              // q'[b0 .. b0+3][p] as one float4 per p
  __shared__ float part[4][4][8][kWave];  // [wave][question][element][lane]
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int htiles = (H + 8 * kWave - 1) / (8 * kWave);
  const long long b0 = ((long long)blockIdx.x / htiles) * 4;
  const int h = (int)(blockIdx.x % htiles) * 8 * kWave + 8 * lane;
  for (int p = threadIdx.x; p < P; p += blockDim.x) {
    float v[4];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
      v[bb] = (b0 + bb < B) ? q[(size_t)(b0 + bb) * (size_t)P + p] : 0.0f;
    qs[p] = make_float4(v[0], v[1], v[2], v[3]);
  }
  __syncthreads();
  float acc[4][8];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[bb][e] = 0.0f;
  if (h < H) {
#pragma unroll 4
    for (int p = wave; p < P; p += 4) {
      const uint4 v = load_piece<false>(w + (size_t)p * (size_t)H + h);
      const float wf[8] = {bf_lo(v.x), bf_hi(v.x), bf_lo(v.y), bf_hi(v.y),
                           bf_lo(v.z), bf_hi(v.z), bf_lo(v.w), bf_hi(v.w)};
      const float4 qv = qs[p];
      const float qb[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
      for (int bb = 0; bb < 4; ++bb)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[bb][e] = fmaf(qb[bb], wf[e], acc[bb][e]);
    }
  }
#pragma unroll
  for (int bb = 0; bb < 4; ++bb)
#pragma unroll
    for (int e = 0; e < 8; ++e) part[wave][bb][e][lane] = acc[bb][e];
  __syncthreads();
  // wave w now finishes question b0 + w
  const long long b = b0 + wave;
  if (b >= B || h >= H) return;
  float r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    r[e] = ((part[0][wave][e][lane] + part[1][wave][e][lane]) + part[2][wave][e][lane]) +
           part[3][wave][e][lane];
  float4* dst = reinterpret_cast<float4*>(u + (size_t)b * (size_t)H + h);
  dst[0] = make_float4(r[0], r[1], r[2], r[3]);
  dst[1] = make_float4(r[4], r[5], r[6], r[7]);
}

// ---------------------------------------------------------------------------
// Dot scoring of bf16 candidate rows against the folded fp32 query u: the
// register-query kernel's structure with 16-byte pieces of 8 bf16. Lane l
// owns pieces l + 64 j (j < NV) of u and of every row; a wave takes R rows at
// a time; one workgroup per question.
template <int NV, int R, bool FULL, bool NT>
__global__ __launch_bounds__(kBlock) void fused_bf16_dot(KernelArgs a,
                                                         const uint16_t* __restrict__ xc,
                                                         const float* __restrict__ u) {
  __shared__ Lds s;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int nwaves = blockDim.x / kWave;
  const int pieces = a.D >> 3;
  for (int b = blockIdx.x; b < a.B; b += gridDim.x) {
    const Question qn{(size_t)b * (size_t)a.K, a.K};
    float ur[NV][8];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int idx = lane + kWave * j;
      if (FULL || idx < pieces) {
        const float4* up = reinterpret_cast<const float4*>(u + (size_t)b * (size_t)a.D) + 2 * idx;
        const float4 u0 = up[0], u1 = up[1];
        ur[j][0] = u0.x; ur[j][1] = u0.y; ur[j][2] = u0.z; ur[j][3] = u0.w;
        ur[j][4] = u1.x; ur[j][5] = u1.y; ur[j][6] = u1.z; ur[j][7] = u1.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) ur[j][e] = 0.0f;
      }
    }
    const uint16_t* Xb = xc + qn.row * (size_t)a.D;
    for (int k0 = wave * R; k0 < a.K; k0 += nwaves * R) {
      float acc[R];
      const uint16_t* rows[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        acc[r] = 0.0f;
        rows[r] = Xb + (size_t)min(k0 + r, a.K - 1) * (size_t)a.D;
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
#pragma unroll
      for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = dot8_bf(c[r][j], ur[j], acc[r]);
      const float total = wave_reduce_transposed<R>(acc, lane, OpSum());
      store_group<false, R>(s, total, lane, k0, 0, a.K);
    }
    __syncthreads();
    if (wave == 0) slice_softmax<false>(s, a, qn, b, 0, 0, a.K, a.zscale, lane);
    __syncthreads();
  }
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
      slice_softmax<true>(s, a, qn, b, 0, 0, K, zfac, lane);
    }
    __syncthreads();
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
  const int waves = std::max(1, std::min(8, (p.K + R - 1) / R));
  const unsigned grid = (unsigned)std::min(p.B, 1 << 20), block = (unsigned)(waves * kWave);
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

template <bool NT>
hipError_t launch_cos_mfma(const KernelArgs& a, const ProjArgs& p, hipStream_t stream) {
  const unsigned grid = (unsigned)std::min(p.B, 1 << 20);
  switch (p.P / 64) {
    case 1:
      hipLaunchKernelGGL((proj_cos_mfma<1, NT>), dim3(grid), dim3(512), 0, stream, a, p.xc, p.wc,
                         p.qp);
      break;
    case 2:
      hipLaunchKernelGGL((proj_cos_mfma<2, NT>), dim3(grid), dim3(512), 0, stream, a, p.xc, p.wc,
                         p.qp);
      break;
    case 3:
      hipLaunchKernelGGL((proj_cos_mfma<3, NT>), dim3(grid), dim3(512), 0, stream, a, p.xc, p.wc,
                         p.qp);
      break;
    case 4:
      hipLaunchKernelGGL((proj_cos_mfma<4, NT>), dim3(grid), dim3(512), 0, stream, a, p.xc, p.wc,
                         p.qp);
      break;
    default:
      return hipErrorInvalidValue;
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
  // q' = Wq x_q for every question: one wave per 8 x 8 tile.
  {
    const long long waves = (long long)((p.B + 7) / 8) * ((p.P + 7) / 8);
    hipLaunchKernelGGL(proj_query, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, p.xq,
                       p.wq, p.qp, p.B, p.Hq, p.P);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  KernelArgs a{};
  a.out = p.out;
  a.B = p.B;
  a.K = p.K;
  a.D = p.Hc;
  a.G = 1;
  a.rpg = p.K;
  a.zscale = p.zscale;
  a.cosine = p.cosine;
  if (p.cosine) return p.nt ? launch_cos_mfma<true>(a, p, stream) : launch_cos_mfma<false>(a, p, stream);
  // u = Wc^T q' (one workgroup per 4 questions x 512 h), then one
  // bandwidth-bound pass over the candidates.
  {
    const long long groups = (long long)((p.B + 3) / 4) * ((p.Hc + 511) / 512);
    hipLaunchKernelGGL(fold_query, dim3((unsigned)groups), dim3(256), 0, stream, p.qp, p.wc, p.u,
                       p.B, p.Hc, p.P);
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int nv = bf16_nv_for(p.Hc);
  return p.nt ? launch_bf16_dot<true>(a, p, nv, stream) : launch_bf16_dot<false>(a, p, nv, stream);
}

}  // namespace cs
