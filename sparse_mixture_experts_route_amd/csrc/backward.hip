// Elementwise and per-token kernels of the layer backward (the grouped GEMMs
// are in grouped_gemm_bwd.hip).
//
// The layer ("Distributed training part 4", jesamkim's AI tech blog, section
// 3): y[t] = sum over j < k of g[t, j] E_{e(t, j)}(x[t]), g = the softmax
// probability over all E router logits of the selected expert. Given dy:
//   combine backward   dYp[row of (t, j)] = g[t, j] dy[t], dG[t, j] = dy[t] . Y[row]
//   router backward    p = softmax(logits[t]); dp[e] = sum of dG[t, j] over the j
//                      with idx[t, j] = e; dlogit[t, e] = p[e] (dp[e] - sum_e' p dp)
//                      (no gradient through the choice of experts)
//   dispatch backward  dx[t] = sum over j of dX[row of (t, j)] + (dlogit W_r^T)[t]
// and the router statistics: load_frac[e] = counts[e] / (T k), mean_prob[e] =
// mean over tokens of p[t, e], dbias[e] = sum over tokens of dlogit[t, e].
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kBwdWaves = 4;  // tokens per block (one wave each)

__device__ __forceinline__ void bf16x8_to_f32(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_to_f32(v[i] & 0xFFFFu);
    f[2 * i + 1] = bf16_to_f32(v[i] >> 16);
  }
}

// One wave per token (k <= 8): dG[j] from the token's dy row and its k
// expert-output rows, the rows of dYp, then the router's softmax backward
// over the E logits (lane l owns experts l, l + 64, ...).
__global__ __launch_bounds__(kBwdWaves * kWave) void bwd_combine_kernel(
    const u32x4* __restrict__ dy, const float* __restrict__ gate, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ inv, const u32x4* __restrict__ Y, const float* __restrict__ logits,
    u32x4* __restrict__ dYp, float* __restrict__ dlogit, bf16_bits* __restrict__ dlogit_b,
    float* __restrict__ prob, int64_t T, int k, int E, int Ep, int64_t row_vecs) {
  const int lane = threadIdx.x % kWave;
  const int64_t t = (int64_t)blockIdx.x * kBwdWaves + threadIdx.x / kWave;
  if (t >= T) return;
  int64_t rows[8];
  float g[8], dg[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    rows[j] = j < k ? inv[t * k + j] : 0;
    g[j] = j < k ? gate[t * k + j] : 0.0f;
    dg[j] = 0.0f;
  }
  const u32x4* dyr = dy + t * row_vecs;
  for (int64_t c = lane; c < row_vecs; c += kWave) {
    float a[8];
    bf16x8_to_f32(dyr[c], a);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k) {
        float b[8];
        bf16x8_to_f32(Y[rows[j] * row_vecs + c], b);
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) s = fmaf(a[i], b[i], s);
        dg[j] += s;
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(g[j] * a[2 * i], g[j] * a[2 * i + 1]);
        dYp[rows[j] * row_vecs + c] = o;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) dg[j] = wave_sum(dg[j]);
  // softmax over the E logits, then dlogit = p (dp - sum p dp)
  const float* lg = logits + t * E;
  float m = -INFINITY;
  for (int e = lane; e < E; e += kWave) m = fmaxf(m, lg[e]);
  m = wave_max(m);
  float ssum = 0.0f;
  for (int e = lane; e < E; e += kWave) ssum += expf(lg[e] - m);
  ssum = wave_sum(ssum);
  float pdp = 0.0f;
  for (int e = lane; e < E; e += kWave) {
    const float p = expf(lg[e] - m) / ssum;
    float dp = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < k && idx[t * k + j] == e) dp += dg[j];
    pdp += p * dp;
  }
  pdp = wave_sum(pdp);
  for (int e = lane; e < Ep; e += kWave) {
    float dl = 0.0f;
    if (e < E) {
      const float p = expf(lg[e] - m) / ssum;
      float dp = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < k && idx[t * k + j] == e) dp += dg[j];
      dl = p * (dp - pdp);
      dlogit[t * E + e] = dl;
      prob[t * E + e] = p;
    }
    dlogit_b[t * Ep + e] = (bf16_bits)f32_to_bf16(dl);
  }
}

// dx[t] = sum over j of dXp[row of (t, j)] (selection order) + dxr[t], one wave per token
__global__ __launch_bounds__(kBwdWaves * kWave) void bwd_dx_kernel(const u32x4* __restrict__ dXp,
                                                                   const int32_t* __restrict__ inv,
                                                                   const u32x4* __restrict__ dxr,
                                                                   u32x4* __restrict__ dx, int64_t T, int k,
                                                                   int64_t row_vecs) {
  const int lane = threadIdx.x % kWave;
  const int64_t t = (int64_t)blockIdx.x * kBwdWaves + threadIdx.x / kWave;
  if (t >= T) return;
  for (int64_t c = lane; c < row_vecs; c += kWave) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = 0; j < k; ++j) {
      float a[8];
      bf16x8_to_f32(dXp[(int64_t)inv[t * k + j] * row_vecs + c], a);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += a[i];
    }
    float r[8];
    bf16x8_to_f32(dxr[t * row_vecs + c], r);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i] + r[2 * i], acc[2 * i + 1] + r[2 * i + 1]);
    dx[t * row_vecs + c] = o;
  }
}

// H = GELU_tanh(U) elementwise (bf16 in and out, 8 values per thread)
__global__ __launch_bounds__(256) void gelu_rows_kernel(const u32x4* __restrict__ U, u32x4* __restrict__ H,
                                                        int64_t n_vecs) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n_vecs; i += (int64_t)gridDim.x * 256) {
    float a[8];
    bf16x8_to_f32(U[i], a);
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(gelu_tanh(a[2 * q]), gelu_tanh(a[2 * q + 1]));
    H[i] = o;
  }
}

constexpr int kStatTokens = 256;  // tokens per partial sum

// Per chunk of kStatTokens tokens: sums of p[t, e] and dlogit[t, e]. With EP =
// the next power of two >= E, thread (e = tid % EP, j = tid / EP) adds tokens
// j, j + 256 / EP, ... of the chunk; the 256 / EP sums of an expert are then
// added in j order (a fixed order: deterministic).
__global__ __launch_bounds__(256) void bwd_stats_partial_kernel(const float* __restrict__ prob,
                                                                const float* __restrict__ dlogit,
                                                                float* __restrict__ part, int64_t T, int E, int EP) {
  __shared__ float s_p[256], s_d[256];
  const int tid = threadIdx.x, e = tid % EP, j = tid / EP, tpe = 256 / EP;
  const int64_t t0 = (int64_t)blockIdx.x * kStatTokens, t1 = min(T, t0 + kStatTokens);
  float sp = 0.0f, sd = 0.0f;
  if (e < E)
    for (int64_t t = t0 + j; t < t1; t += tpe) {
      sp += prob[t * E + e];
      sd += dlogit[t * E + e];
    }
  s_p[tid] = sp;
  s_d[tid] = sd;
  __syncthreads();
  if (j == 0 && e < E) {
    float ap = 0.0f, ad = 0.0f;
    for (int jj = 0; jj < tpe; ++jj) {
      ap += s_p[jj * EP + e];
      ad += s_d[jj * EP + e];
    }
    part[((int64_t)blockIdx.x * 2) * E + e] = ap;
    part[((int64_t)blockIdx.x * 2 + 1) * E + e] = ad;
  }
}

// Chunk sums added in chunk order (deterministic); outputs may be null
__global__ __launch_bounds__(256) void bwd_stats_final_kernel(const float* __restrict__ part, int64_t chunks,
                                                              const int32_t* __restrict__ counts,
                                                              float* __restrict__ load_frac,
                                                              float* __restrict__ mean_prob,
                                                              float* __restrict__ dbias, int64_t T, int k, int E) {
  const int e = threadIdx.x;
  if (e >= E) return;
  float sp = 0.0f, sd = 0.0f;
  for (int64_t c = 0; c < chunks; ++c) {
    sp += part[(c * 2) * E + e];
    sd += part[(c * 2 + 1) * E + e];
  }
  if (mean_prob) mean_prob[e] = sp / (float)T;
  if (dbias) dbias[e] = sd;
  if (load_frac) load_frac[e] = (float)counts[e] / (float)(T * k);
}

}  // namespace

int64_t bwd_stat_chunks(int64_t T) { return ceil_div(T, kStatTokens); }

hipError_t launch_bwd_combine(const moe_problem_t& p, const void* dy, const float* gate, const int32_t* idx,
                              const int32_t* inv, const void* Y_perm, const float* logits, void* dYp,
                              float* dlogit, bf16_bits* dlogit_b, float* prob, int Ep, hipStream_t s) {
  if (p.k > 8) return hipErrorInvalidValue;
  const int64_t row_vecs = (int64_t)p.d_model * 2 / 16;
  hipLaunchKernelGGL(bwd_combine_kernel, dim3((unsigned)ceil_div(p.T, kBwdWaves)), dim3(kBwdWaves * kWave), 0, s,
                     (const u32x4*)dy, gate, idx, inv, (const u32x4*)Y_perm, logits, (u32x4*)dYp, dlogit, dlogit_b,
                     prob, p.T, p.k, p.E, Ep, row_vecs);
  return hipGetLastError();
}

hipError_t launch_bwd_dx(const moe_problem_t& p, const void* dXp, const int32_t* inv, const void* dxr, void* dx,
                         hipStream_t s) {
  const int64_t row_vecs = (int64_t)p.d_model * 2 / 16;
  hipLaunchKernelGGL(bwd_dx_kernel, dim3((unsigned)ceil_div(p.T, kBwdWaves)), dim3(kBwdWaves * kWave), 0, s,
                     (const u32x4*)dXp, inv, (const u32x4*)dxr, (u32x4*)dx, p.T, p.k, row_vecs);
  return hipGetLastError();
}

hipError_t launch_gelu_rows(const void* U, void* H, int64_t elems, hipStream_t s) {
  const int64_t n_vecs = elems / 8;
  const int64_t blocks = min(ceil_div(n_vecs, 256), (int64_t)device_cus() * 8);
  if (n_vecs <= 0) return hipSuccess;
  hipLaunchKernelGGL(gelu_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const u32x4*)U, (u32x4*)H, n_vecs);
  return hipGetLastError();
}

hipError_t launch_bwd_stats(const moe_problem_t& p, const float* prob, const float* dlogit, const int32_t* counts,
                            float* part, float* load_frac, float* mean_prob, float* dbias, hipStream_t s) {
  const int64_t chunks = bwd_stat_chunks(p.T);
  int ep = 1;
  while (ep < p.E) ep <<= 1;
  hipLaunchKernelGGL(bwd_stats_partial_kernel, dim3((unsigned)chunks), dim3(256), 0, s, prob, dlogit, part, p.T,
                     p.E, ep);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_stats_final_kernel, dim3(1), dim3(256), 0, s, (const float*)part, chunks, counts, load_frac,
                     mean_prob, dbias, p.T, p.k, p.E);
  return hipGetLastError();
}

}  // namespace moe
