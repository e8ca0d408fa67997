// cs_bench.hip -- native timing helpers for the bench and the graph tests.
//
// Timing follows the page's protocol (pull request "cuda: add a fused
// candidate-scoring kernel for CLM and Kev", "What it is worth": the same
// launch timed directly and replayed from a graph), with HIP events recorded
// on the stream that runs the kernels. Loops run here in C so that host
// overhead of the caller's language does not enter the per-call figures.
//
// Entry points (all return 0 or a negative code; HIP errors are -1000 - err):
//   csb_time_calls   events around `iters` back-to-back direct calls
//   csb_time_calls_rotating  the same, each call on the next of several
//                    copies of the inputs (cold caches)
//   csb_time_graph   capture `calls_per_graph` calls into one graph, check the
//                    node count, then events around `replays` graph launches
//   csb_graph_nodes  capture one call and report its node count
//   csb_time_empty   the same protocol for an empty kernel of a given
//                    grid/block: the launch floor
//   csb_copy         plain device copy of `bytes` (counter calibration)
//   csb_read         plain streaming read of `bytes` (the practical HBM read
//                    ceiling that the scoring kernel is compared with)

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "candidate_scoring.h"

extern "C" {

typedef struct {
  const float* Q;
  const float* C;
  float* out;
  int B, K, D, similarity;
  float scale, temperature;
  void* workspace;
  size_t workspace_bytes;
  int groups;         // <= 0: the library's own plan
  float* row_norms;   // non-NULL: the unfused baseline (norm pass + scoring)
} csb_call;

}  // extern "C"

namespace {

__global__ void empty_kernel() {}

__global__ void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = src[i];
}

// Streams n 16-byte pieces, four in flight per thread; the sum only keeps
// the loads alive and is stored only if it hits an impossible value.
__global__ void read_kernel(const float4* __restrict__ src, size_t n, float* sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  float acc = 0.0f;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const float4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc += (a.x + b.x) + (c.x + d.x) + (a.w + b.w) + (c.w + d.w);
  }
  for (; i < n; i += stride) acc += src[i].x;
  if (acc == -1.2345e-30f) sink[0] = acc;
}

int hip_code(hipError_t e) { return e == hipSuccess ? 0 : -1000 - (int)e; }

#define CSB_TRY(expr)                       \
  do {                                      \
    hipError_t _e = (expr);                 \
    if (_e != hipSuccess) return hip_code(_e); \
  } while (0)

int issue(const csb_call* c, hipStream_t s) {
  if (c->row_norms != nullptr)
    return cs_score_candidates_unfused(c->Q, c->C, c->B, c->K, c->D, c->similarity, c->scale,
                                       c->temperature, c->out, c->row_norms, s);
  if (c->groups > 0)
    return cs_score_candidates_batch_groups(c->Q, c->C, c->B, c->K, c->D, c->similarity,
                                            c->scale, c->temperature, c->out, c->workspace,
                                            c->workspace_bytes, c->groups, s);
  return cs_score_candidates_batch(c->Q, c->C, c->B, c->K, c->D, c->similarity, c->scale,
                                   c->temperature, c->out, c->workspace, c->workspace_bytes, s);
}

struct Events {
  hipEvent_t a = nullptr, b = nullptr;
  ~Events() {
    if (a) (void)hipEventDestroy(a);
    if (b) (void)hipEventDestroy(b);
  }
};

struct Graph {
  hipGraph_t g = nullptr;
  hipGraphExec_t x = nullptr;
  hipStream_t s = nullptr;
  ~Graph() {
    if (x) (void)hipGraphExecDestroy(x);
    if (g) (void)hipGraphDestroy(g);
    if (s) (void)hipStreamDestroy(s);
  }
};

// Captures `n` calls made by `body` on a fresh non-blocking stream.
template <class F>
int capture(Graph& gr, int n, F body, size_t* nodes) {
  CSB_TRY(hipStreamCreateWithFlags(&gr.s, hipStreamNonBlocking));
  CSB_TRY(hipStreamBeginCapture(gr.s, hipStreamCaptureModeThreadLocal));
  int st = 0;
  for (int i = 0; i < n && st == 0; ++i) st = body(gr.s);
  hipGraph_t g = nullptr;
  const hipError_t e = hipStreamEndCapture(gr.s, &g);
  gr.g = g;
  if (st != 0) return st;
  CSB_TRY(e);
  if (nodes != nullptr) {
    size_t count = 0;
    CSB_TRY(hipGraphGetNodes(gr.g, nullptr, &count));
    *nodes = count;
  }
  CSB_TRY(hipGraphInstantiate(&gr.x, gr.g, nullptr, nullptr, 0));
  return 0;
}

template <class F>
int time_loop(hipStream_t s, int iters, F body, float* ms) {
  Events ev;
  CSB_TRY(hipEventCreate(&ev.a));
  CSB_TRY(hipEventCreate(&ev.b));
  CSB_TRY(hipEventRecord(ev.a, s));
  for (int i = 0; i < iters; ++i) {
    const int st = body(s);
    if (st != 0) return st;
  }
  CSB_TRY(hipEventRecord(ev.b, s));
  CSB_TRY(hipEventSynchronize(ev.b));
  CSB_TRY(hipEventElapsedTime(ms, ev.a, ev.b));
  return 0;
}

}  // namespace

extern "C" {

int csb_time_calls(const csb_call* c, int iters, hipStream_t stream, float* ms) {
  return time_loop(stream, iters, [&](hipStream_t s) { return issue(c, s); }, ms);
}

// Cold-cache variant: call i reads copy (i % copies) of the inputs, the
// copies lying q_stride / c_stride floats apart (and the output likewise
// out_stride apart), so that repeated calls do not hit in any cache when
// the copies together exceed the caches.
int csb_time_calls_rotating(const csb_call* c, int copies, size_t q_stride, size_t c_stride,
                            size_t out_stride, int iters, hipStream_t stream, float* ms) {
  if (copies < 1) return -1;
  int i = 0;
  return time_loop(stream, iters, [&](hipStream_t s) {
    csb_call k = *c;
    const size_t j = (size_t)(i++ % copies);
    k.Q = c->Q + j * q_stride;
    k.C = c->C + j * c_stride;
    k.out = c->out + j * out_stride;
    return issue(&k, s);
  }, ms);
}

int csb_graph_nodes(const csb_call* c, size_t* nodes) {
  Graph gr;
  return capture(gr, 1, [&](hipStream_t s) { return issue(c, s); }, nodes);
}

int csb_time_graph(const csb_call* c, int calls_per_graph, int replays, int warmup, float* ms,
                   size_t* nodes) {
  Graph gr;
  int st = capture(gr, calls_per_graph, [&](hipStream_t s) { return issue(c, s); }, nodes);
  if (st != 0) return st;
  for (int i = 0; i < warmup; ++i) CSB_TRY(hipGraphLaunch(gr.x, gr.s));
  st = time_loop(gr.s, replays, [&](hipStream_t s) { return hip_code(hipGraphLaunch(gr.x, s)); },
                 ms);
  return st;
}

int csb_graph_replay(const csb_call* c, int replays, int sync_each) {
  Graph gr;
  int st = capture(gr, 1, [&](hipStream_t s) { return issue(c, s); }, nullptr);
  if (st != 0) return st;
  for (int i = 0; i < replays; ++i) {
    CSB_TRY(hipGraphLaunch(gr.x, gr.s));
    if (sync_each) CSB_TRY(hipStreamSynchronize(gr.s));
  }
  CSB_TRY(hipStreamSynchronize(gr.s));
  return 0;
}

int csb_time_empty(unsigned grid, unsigned block, int iters, int use_graph, int calls_per_graph,
                   hipStream_t stream, float* ms) {
  auto launch = [&](hipStream_t s) {
    hipLaunchKernelGGL(empty_kernel, dim3(grid), dim3(block), 0, s);
    return hip_code(hipGetLastError());
  };
  if (!use_graph) return time_loop(stream, iters, launch, ms);
  Graph gr;
  int st = capture(gr, calls_per_graph, launch, nullptr);
  if (st != 0) return st;
  CSB_TRY(hipGraphLaunch(gr.x, gr.s));
  return time_loop(gr.s, iters, [&](hipStream_t s) { return hip_code(hipGraphLaunch(gr.x, s)); },
                   ms);
}

int csb_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  if (src == nullptr || dst == nullptr || (bytes % 16) != 0) return -1;
  const size_t n = bytes / 16;
  hipLaunchKernelGGL(copy_kernel, dim3(4096), dim3(256), 0, stream,
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), n);
  return hip_code(hipGetLastError());
}

int csb_read(const void* src, size_t bytes, unsigned grid, unsigned block, float* sink,
             hipStream_t stream) {
  if (src == nullptr || sink == nullptr || (bytes % 16) != 0 || block == 0 || block > 1024)
    return -1;
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(block), 0, stream,
                     static_cast<const float4*>(src), bytes / 16, sink);
  return hip_code(hipGetLastError());
}

}  // extern "C"
