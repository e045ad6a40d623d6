// Router: logits = x W_r (+ b), softmax over the E experts, top-k selection.
//
// "Distributed training part 4" (jesamkim's AI tech blog), section 3, structure:
// the gating network is a Linear layer followed by a Softmax giving each expert
// a probability, and only the k best experts are used for a token. Selection is
// made on the float32 logits: descending value, ties to the lower expert index.
// The gate of a selected expert is its softmax probability over all E experts.
//
// One wavefront per token. The contraction over d_model runs with lanes
// striding the hidden dimension and float32 accumulators for 8 experts at a
// time; the per-expert partial sums are reduced across the wave. Softmax and
// top-k then run on the wave: every lane owns up to 4 experts, and each of the
// k rounds is a wave-wide max over 64-bit keys (order-preserving logit key in
// the upper half, inverted expert index in the lower half, so equal logits
// favour the lower index).
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kRouteWaves = 4;  // tokens per block

template <typename Tin>
__device__ __forceinline__ float load_val(const Tin* p);
template <>
__device__ __forceinline__ float load_val<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_val<bf16_bits>(const bf16_bits* p) { return bf16_to_f32(*p); }

template <typename Tin>
__global__ __launch_bounds__(kRouteWaves * kWave) void route_kernel(
    const Tin* __restrict__ x, const Tin* __restrict__ wr, const float* __restrict__ bias,
    float* __restrict__ logits, int32_t* __restrict__ idx, float* __restrict__ gate,
    int64_t T, int d, int E, int k) {
  __shared__ float lg[kRouteWaves][256];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int64_t t = (int64_t)blockIdx.x * kRouteWaves + wave;
  const bool valid = t < T;
  const Tin* xr = x + (valid ? t : 0) * (int64_t)d;

  for (int e0 = 0; e0 < E; e0 += 8) {
    const int ne = min(8, E - e0);
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
    if (valid) {
      for (int c = lane; c < d; c += kWave) {
        const float xv = load_val(xr + c);
        const Tin* w = wr + (int64_t)c * E + e0;
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (q < ne) acc[q] = fmaf(xv, load_val(w + q), acc[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = wave_sum(acc[q]);
    if (lane == 0) {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q < ne) lg[wave][e0 + q] = acc[q] + (bias ? bias[e0 + q] : 0.0f);
    }
  }
  __syncthreads();
  if (!valid) return;

  // softmax statistics over all E logits
  float m = -INFINITY;
  for (int e = lane; e < E; e += kWave) m = fmaxf(m, lg[wave][e]);
  m = wave_max(m);
  float ssum = 0.0f;
  for (int e = lane; e < E; e += kWave) ssum += expf(lg[wave][e] - m);
  ssum = wave_sum(ssum);
  if (logits) {
    for (int e = lane; e < E; e += kWave) logits[t * E + e] = lg[wave][e];
  }

  // k rounds of a wave-wide max over (logit key, inverted index)
  uint32_t taken = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + kWave * i;
      if (e < E && !((taken >> i) & 1u)) {
        const uint64_t key = ((uint64_t)float_order_key(lg[wave][e]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
        best = key > best ? key : best;
      }
    }
    best = wave_max_u64(best);
    const int es = (int)(0xFFFFFFFFu - (uint32_t)best);
    if ((es & (kWave - 1)) == lane) taken |= 1u << (es / kWave);
    if (lane == 0) {
      idx[t * k + j] = es;
      gate[t * k + j] = expf(lg[wave][es] - m) / ssum;
    }
  }
}

}  // namespace

hipError_t launch_route(const moe_problem_t& p, const void* x, const void* w_router, const float* bias,
                        float* logits, int32_t* idx, float* gate, hipStream_t s) {
  const int64_t blocks = ceil_div(p.T, kRouteWaves);
  if (p.dtype == MOE_DTYPE_BF16) {
    hipLaunchKernelGGL(route_kernel<bf16_bits>, dim3((unsigned)blocks), dim3(kRouteWaves * kWave), 0, s,
                       (const bf16_bits*)x, (const bf16_bits*)w_router, bias, logits, idx, gate, p.T,
                       p.d_model, p.E, p.k);
  } else {
    hipLaunchKernelGGL(route_kernel<float>, dim3((unsigned)blocks), dim3(kRouteWaves * kWave), 0, s,
                       (const float*)x, (const float*)w_router, bias, logits, idx, gate, p.T, p.d_model,
                       p.E, p.k);
  }
  return hipGetLastError();
}

}  // namespace moe
