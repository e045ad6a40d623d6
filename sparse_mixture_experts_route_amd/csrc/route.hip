// Router: logits = x W_r (+ b), softmax over the E experts, top-k selection.
//
// "Distributed training part 4" (jesamkim's AI tech blog), section 3, structure:
// the gating network is a Linear layer followed by a Softmax giving each expert
// a probability, and only the k best experts are used for a token. Selection is
// made on the float32 logits: descending value, ties to the lower expert index.
// The gate of a selected expert is its softmax probability over all E experts.
//
// Two contraction paths, one selection epilogue:
//   * bf16 with E a multiple of 8: matrix cores. A block takes 64 tokens and
//     all experts, padded with zero columns to EP = the next multiple of 64;
//     four waves in a 2x2 grid each own 32 tokens x EP/2 experts as 32x32
//     MFMA tiles (v_mfma_f32_32x32x16_bf16, float32 accumulators).
//     x tiles sit K-contiguous in LDS; w_router tiles stay E-contiguous and are
//     read with ds_read_b64_tr_b16 (4 consecutive k of one column per lane).
//     The float32 logits of the block land in LDS for the epilogue.
//   * otherwise (float32, or E not a multiple of 8): one wave per token; each
//     lane takes 16-byte pieces of the token's row and multiplies them with
//     the matching w_router rows for up to 8 experts at a time; per-expert
//     partial sums are reduced across the wave.
//   * epilogue, one wave per token: max and sum of exponentials over the E
//     logits, then k rounds of a wave-wide max over 64-bit keys
//     (order-preserving logit key in the upper half, inverted expert index in
//     the lower half, so equal logits favour the lower index).
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Softmax statistics and top-k of one token whose E logits are in LDS (`lg`).
__device__ __forceinline__ void select_topk(const float* lg, int E, int k, int64_t t, float* __restrict__ logits,
                                            int32_t* __restrict__ idx, float* __restrict__ gate) {
  const int lane = threadIdx.x % kWave;
  float m = -INFINITY;
  for (int e = lane; e < E; e += kWave) m = fmaxf(m, lg[e]);
  m = wave_max(m);
  float ssum = 0.0f;
  for (int e = lane; e < E; e += kWave) ssum += expf(lg[e] - m);
  ssum = wave_sum(ssum);
  if (logits) {
    for (int e = lane; e < E; e += kWave) logits[t * E + e] = lg[e];
  }
  uint32_t taken = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + kWave * i;
      if (e < E && !((taken >> i) & 1u)) {
        const uint64_t key = ((uint64_t)float_order_key(lg[e]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
        best = key > best ? key : best;
      }
    }
    best = wave_max_u64(best);
    const int es = (int)(0xFFFFFFFFu - (uint32_t)best);
    if ((es & (kWave - 1)) == lane) taken |= 1u << (es / kWave);
    if (lane == 0) {
      idx[t * k + j] = es;
      gate[t * k + j] = expf(lg[es] - m) / ssum;
    }
  }
}

// ---------------------------------------------------------------- matrix-core path

constexpr int RT = 64;   // tokens per block
constexpr int RK = 64;   // K step

// E_T: padded experts per wave column = EP / 2 (32 .. 128); E (<= EP, multiple of 8) at run time
template <int E_T>
__global__ __launch_bounds__(256) void route_mfma_kernel(const bf16_bits* __restrict__ x,
                                                         const bf16_bits* __restrict__ wr,
                                                         const float* __restrict__ bias, float* __restrict__ logits,
                                                         int32_t* __restrict__ idx, float* __restrict__ gate,
                                                         int64_t T, int d, int E_real, int k) {
  constexpr int E = 2 * E_T;  // padded width
  constexpr int TN = E_T / 32;       // 32x32 tiles per wave along experts
  constexpr int X_ROW = RK * 2;      // bytes per token row of an x tile
  constexpr int W_ROW = E * 2;       // bytes per k row of a w tile
  __shared__ __attribute__((aligned(16))) char xs[RT * X_ROW];
  __shared__ __attribute__((aligned(16))) char ws[RK * W_ROW];
  __shared__ float lg[RT][E + 1];

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int64_t t0 = (int64_t)blockIdx.x * RT;
  const int wm0 = (wave >> 1) * 32, wn0 = (wave & 1) * E_T;

  f32x16 acc[TN];
#pragma unroll
  for (int ni = 0; ni < TN; ++ni)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[ni][v] = 0.0f;

  // fragment read offsets
  const int a_row = wm0 + (lane & 31);
  const int q = lane & 15, g = lane >> 4, kr = q >> 2;
  int b_rd[TN];
#pragma unroll
  for (int ni = 0; ni < TN; ++ni) {
    const int col = wn0 + ni * 32 + (g & 1) * 16 + (q & 3) * 4;
    b_rd[ni] = ((g >> 1) * 8 + kr) * W_ROW + (((col >> 3) ^ (2 * kr)) << 4) + (col & 7) * 2;
  }

  for (int c0 = 0; c0 < d; c0 += RK) {
    // x tile: 64 tokens x 64 k, 16-byte pieces, chunk XOR-ed by ((row >> 1) & 7)
    for (int p = tid; p < RT * 8; p += 256) {
      const int row = p >> 3, c = p & 7;
      const int64_t t = min(t0 + row, T - 1);
      const u32x4 v = *(const u32x4*)(x + t * d + c0 + c * 8);
      *(u32x4*)(xs + row * X_ROW + ((c ^ ((row >> 1) & 7)) << 4)) = v;
    }
    // w tile: 64 k rows x EP (zero past E_real), chunk XOR-ed by 2*(k & 3)
    for (int p = tid; p < RK * (E / 8); p += 256) {
      const int kk = p / (E / 8), c = p % (E / 8);
      u32x4 v = {0u, 0u, 0u, 0u};
      if (c * 8 < E_real) v = *(const u32x4*)(wr + (int64_t)(c0 + kk) * E_real + c * 8);
      *(u32x4*)(ws + kk * W_ROW + ((c ^ (2 * (kk & 3))) << 4)) = v;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < RK / 16; ++ks) {
      const int kc = ks * 2 + (lane >> 5);
      const bf16x8 fa = *(const bf16x8*)(xs + a_row * X_ROW + ((kc ^ ((a_row >> 1) & 7)) << 4));
#pragma unroll
      for (int ni = 0; ni < TN; ++ni) {
        const char* p0 = ws + ks * 16 * W_ROW + b_rd[ni];
        const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(__attribute__((address_space(3))) char*)p0);
        const s16x4 hi4 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(__attribute__((address_space(3))) char*)(p0 + 4 * W_ROW));
        const s16x8 v = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v), fa, acc[ni], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // logits to LDS: lane holds token (lane & 31) of the wave's rows, experts 8g + 4*(lane>>5) + 0..3
#pragma unroll
  for (int ni = 0; ni < TN; ++ni)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int e = wn0 + ni * 32 + 8 * gq + 4 * (lane >> 5) + qq;
        if (e < E_real) lg[wm0 + (lane & 31)][e] = acc[ni][4 * gq + qq] + (bias ? bias[e] : 0.0f);
      }
  __syncthreads();
  for (int r = wave; r < RT; r += 4) {
    const int64_t t = t0 + r;
    if (t < T) select_topk(lg[r], E_real, k, t, logits, idx, gate);
  }
}

// ---------------------------------------------------------------- FMA path

constexpr int kRouteWaves = 4;  // tokens per block

template <typename Tin>
struct Vec;
template <>
struct Vec<bf16_bits> {
  static constexpr int N = 8;  // elements per 16-byte piece
  __device__ static void load(const bf16_bits* p, float* f) {
    const u32x4 v = *(const u32x4*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_to_f32(v[i] & 0xFFFFu);
      f[2 * i + 1] = bf16_to_f32(v[i] >> 16);
    }
  }
};
template <>
struct Vec<float> {
  static constexpr int N = 4;
  __device__ static void load(const float* p, float* f) {
    const f32x4 v = *(const f32x4*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = v[i];
  }
};

template <typename Tin>
__device__ __forceinline__ float load_one(const Tin* p);
template <>
__device__ __forceinline__ float load_one<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_one<bf16_bits>(const bf16_bits* p) { return bf16_to_f32(*p); }

template <typename Tin>
__global__ __launch_bounds__(kRouteWaves * kWave) void route_fma_kernel(
    const Tin* __restrict__ x, const Tin* __restrict__ wr, const float* __restrict__ bias,
    float* __restrict__ logits, int32_t* __restrict__ idx, float* __restrict__ gate, int64_t T, int d, int E,
    int k) {
  constexpr int VN = Vec<Tin>::N;
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
      // lane takes 16-byte pieces c0 = lane*VN, lane*VN + 64*VN, ...
      for (int c0 = lane * VN; c0 < d; c0 += kWave * VN) {
        float xv[VN];
        Vec<Tin>::load(xr + c0, xv);
#pragma unroll
        for (int i = 0; i < VN; ++i) {
          const Tin* w = wr + (int64_t)(c0 + i) * E + e0;
#pragma unroll
          for (int q = 0; q < 8; ++q)
            if (q < ne) acc[q] = fmaf(xv[i], load_one(w + q), acc[q]);
        }
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
  if (valid) select_topk(lg[wave], E, k, t, logits, idx, gate);
}

}  // namespace

hipError_t launch_route(const moe_problem_t& p, const void* x, const void* w_router, const float* bias,
                        float* logits, int32_t* idx, float* gate, hipStream_t s) {
  if (p.dtype == MOE_DTYPE_BF16 && p.E % 8 == 0) {
    const int64_t blocks = ceil_div(p.T, RT);
    const bf16_bits* xb = (const bf16_bits*)x;
    const bf16_bits* wb = (const bf16_bits*)w_router;
    const int ep = (p.E + 63) / 64 * 64;  // padded expert count
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, s, xb, wb, bias, logits, idx, gate, p.T,
                         p.d_model, p.E, p.k);
      return hipGetLastError();
    };
    switch (ep) {
      case 64:
        return go(route_mfma_kernel<32>);
      case 128:
        return go(route_mfma_kernel<64>);
      case 192:
        return go(route_mfma_kernel<96>);
      default:
        return go(route_mfma_kernel<128>);
    }
  }
  const int64_t blocks = ceil_div(p.T, kRouteWaves);
  if (p.dtype == MOE_DTYPE_BF16) {
    hipLaunchKernelGGL(route_fma_kernel<bf16_bits>, dim3((unsigned)blocks), dim3(kRouteWaves * kWave), 0, s,
                       (const bf16_bits*)x, (const bf16_bits*)w_router, bias, logits, idx, gate, p.T, p.d_model,
                       p.E, p.k);
  } else {
    hipLaunchKernelGGL(route_fma_kernel<float>, dim3((unsigned)blocks), dim3(kRouteWaves * kWave), 0, s,
                       (const float*)x, (const float*)w_router, bias, logits, idx, gate, p.T, p.d_model, p.E,
                       p.k);
  }
  return hipGetLastError();
}

}  // namespace moe
