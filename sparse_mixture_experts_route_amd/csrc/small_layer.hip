// The whole layer of a small float32 problem in one launch.
//
// "Distributed training part 4" (jesamkim's AI tech blog), section 3: router
// Linear + Softmax, the k best experts per token, each an independent FFN
// GELU_tanh(x W1_e) W2_e, and y = sum over the selected experts of the gate
// times the expert output. The MOSAIC summary ("Compute-Optimal Is Not
// Cluster-Optimal", gist.science, method item 2) singles out dispatch
// latency for small micro-batches: a layer of a few dozen tokens spends most
// of its time between launches.
//
// One workgroup per token, no dispatch: wave 0 computes the token's logits
// (route_row_fma) and selects (select_topk), the code the router's own launch
// runs; then, for groups of the selected experts (as many as LDS holds), the
// threads share out the (expert, hidden unit) pairs, each a GELU_tanh of a dot
// product over d_model taken in order with fmaf (the order the float32
// grouped GEMM takes), into LDS; then the (expert, output column) pairs, each
// a dot product over the hidden row in order; then each output column adds
// gate * expert output over the group in selection order (the combine's
// order). The output is the same bits as route -> permute -> grouped FFN ->
// combine.
// Each workgroup reads the k experts' weights it needs (from L2 once they are
// there), so the form only pays while T k d d_expert is small.
#include "common.h"
#include "internal.h"
#include "route_fma.h"
#include "topk.h"

namespace moe {

namespace {

constexpr int kSmallLayerThreads = 512;
constexpr int kSmallLayerMaxOut = 8;   // output columns per thread: d_model <= 8 * 512
constexpr int kDotBatch = 32;          // weight loads in flight per thread (d_model, d_expert: multiples of 64)
constexpr int kSmallLayerLds = 60 * 1024;  // dynamic LDS bytes

// acc + sum over c < len of a[c] * w[c * stride], one fmaf at a time in c
// order (the order of a sequential dot product); the weights are loaded
// kDotBatch at a time, the next batch issued before the current one is used
__device__ __forceinline__ float dot_in_order(const float* a, const float* __restrict__ w, int64_t stride, int len,
                                              float acc) {
  float cur[kDotBatch], nxt[kDotBatch];
#pragma unroll
  for (int u = 0; u < kDotBatch; ++u) cur[u] = w[u * stride];
  for (int c0 = 0; c0 < len; c0 += kDotBatch) {
    const bool more = c0 + kDotBatch < len;
#pragma unroll
    for (int u = 0; u < kDotBatch; ++u) nxt[u] = more ? w[(c0 + kDotBatch + u) * stride] : 0.0f;
#pragma unroll
    for (int u = 0; u < kDotBatch; ++u) acc = fmaf(a[c0 + u], cur[u], acc);
#pragma unroll
    for (int u = 0; u < kDotBatch; ++u) cur[u] = nxt[u];
  }
  return acc;
}

// LDS of the kernel: the token's row, then for a group of G experts their
// hidden rows [G][de] and output rows [G][d]
inline int small_layer_group(int d, int de, int k) {
  const int g = (kSmallLayerLds / 4 - d) / (de + d);
  return g < 1 ? 1 : (g < k ? g : k);
}

__global__ __launch_bounds__(kSmallLayerThreads) void small_layer_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias,
    const float* __restrict__ W1, const float* __restrict__ W2, float* __restrict__ y, int d, int E, int k,
    int de, int G) {
  extern __shared__ float dyn[];  // x row [d], hidden rows [G][de], expert output rows [G][d]
  __shared__ float lg[256];
  __shared__ int32_t s_idx[256];
  __shared__ float s_gate[256];
  float* const xs = dyn;
  float* const hs = dyn + d;
  float* const vs = hs + G * de;
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  const float* xr = x + t * d;
  if (tid < kWave) {
    route_row_fma(xr, wr, bias, d, E, true, lg);
    select_topk(lg, E, k, 0, nullptr, s_idx, s_gate);  // the token's k experts and gates, in LDS
  }
  for (int c = tid; c < d; c += kSmallLayerThreads) xs[c] = xr[c];
  __syncthreads();

  float acc[kSmallLayerMaxOut];
#pragma unroll
  for (int u = 0; u < kSmallLayerMaxOut; ++u) acc[u] = 0.0f;
  for (int j0 = 0; j0 < k; j0 += G) {
    const int g_n = min(G, k - j0);
    // hidden rows of the group's experts: one (expert, unit) pair per thread at a time
    for (int q = tid; q < g_n * de; q += kSmallLayerThreads) {
      const int j = q / de, n = q - j * de;
      const float* w1 = W1 + (int64_t)s_idx[j0 + j] * d * de;
      hs[q] = gelu_tanh(dot_in_order(xs, w1 + n, de, d, 0.0f));
    }
    __syncthreads();
    // their output rows
    for (int q = tid; q < g_n * d; q += kSmallLayerThreads) {
      const int j = q / d, n = q - j * d;
      const float* w2 = W2 + (int64_t)s_idx[j0 + j] * de * d;
      vs[q] = dot_in_order(hs + j * de, w2 + n, d, de, 0.0f);
    }
    __syncthreads();
    // gate-weighted sum in selection order
#pragma unroll
    for (int u = 0; u < kSmallLayerMaxOut; ++u) {
      const int n = tid + u * kSmallLayerThreads;
      if (n < d)
        for (int j = 0; j < g_n; ++j) acc[u] = fmaf(s_gate[j0 + j], vs[j * d + n], acc[u]);
    }
    __syncthreads();  // the next group rewrites the hidden and output rows
  }
#pragma unroll
  for (int u = 0; u < kSmallLayerMaxOut; ++u) {
    const int n = tid + u * kSmallLayerThreads;
    if (n < d) y[t * d + n] = acc[u];
  }
}

}  // namespace

// Rounds of kDotBatch weight loads one thread waits for, one after another:
// the time of a workgroup (~1.1 us each on MI355X, plus ~6 us)
int64_t small_layer_rounds(const moe_problem_t& p) {
  const int64_t d = p.d_model, de = p.d_expert, k = p.k;
  return ceil_div(k * de, kSmallLayerThreads) * (d / kDotBatch) + ceil_div(k * d, kSmallLayerThreads) * (de / kDotBatch);
}

// Used for float32 problems whose workgroups finish sooner than the staged
// launches would: at most 48 load rounds per thread, and T k d d_expert <=
// 2^24 multiply-adds per GEMM (each workgroup reads its experts' weights
// again, from L2), with rows that fit in LDS. Measured on MI355X, µs per
// moe_forward (one launch against the staged launches): 64 x 128, 8 experts,
// top-2, 256 wide (12 rounds) 19.4 against 44.7; 60 x 256, 64 experts, top-8,
// 128 wide (32 rounds) 75 against 90; 32 x 512, 16 experts, top-4, 256 wide
// (64 rounds) 85.7 against 85.5; 4 x 1024, 8 experts, top-2, 1024 wide (256
// rounds, four workgroups) 271 against 167. MOE_SMALL_LAYER=0 turns it off.
bool small_layer_fused(const moe_problem_t& p) {
  const char* f = getenv("MOE_SMALL_LAYER");
  if (f && f[0] && atoi(f) == 0) return false;
  return p.dtype == MOE_DTYPE_F32 && p.d_model <= kSmallLayerMaxOut * kSmallLayerThreads &&
         (int64_t)(2 * p.d_model + p.d_expert) * 4 <= kSmallLayerLds &&
         p.T * p.k * (int64_t)p.d_model * p.d_expert <= (int64_t)1 << 24 && small_layer_rounds(p) <= 48;
}

hipError_t launch_small_layer(const moe_problem_t& p, const void* x, const void* w_router, const float* bias,
                              const void* W1, const void* W2, void* y, hipStream_t s) {
  if (!small_layer_fused(p) || p.T > INT32_MAX) return hipErrorInvalidValue;
  const int G = small_layer_group(p.d_model, p.d_expert, p.k);
  const size_t lds = (size_t)(p.d_model + G * (p.d_expert + p.d_model)) * sizeof(float);
  if (lds > (size_t)kSmallLayerLds) return hipErrorInvalidValue;
  hipLaunchKernelGGL(small_layer_f32_kernel, dim3((unsigned)p.T), dim3(kSmallLayerThreads), lds, s,
                     (const float*)x, (const float*)w_router, bias, (const float*)W1, (const float*)W2, (float*)y,
                     p.d_model, p.E, p.k, p.d_expert, G);
  return hipGetLastError();
}

}  // namespace moe
