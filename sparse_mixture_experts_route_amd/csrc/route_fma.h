// One token's router logits on the vector ALUs (float32, or bf16 with E not a
// multiple of 8), shared by the router's FMA path and the fused small-layer
// kernel so that both give the same bits: one wave per token; lane l takes
// the 16-byte pieces of the token's row at l*VN, l*VN + 64*VN, ... and
// multiplies them with the matching w_router rows, eight experts at a time;
// the lanes' partial sums are added with wave_sum; the bias follows.
#pragma once

#include "common.h"

namespace moe {

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

// logits of the token whose row is xr into lg[0..E) (LDS), by the whole calling
// wave; with valid == false the wave still joins the reductions (and writes
// the bias alone)
template <typename Tin>
__device__ __forceinline__ void route_row_fma(const Tin* __restrict__ xr, const Tin* __restrict__ wr,
                                              const float* __restrict__ bias, int d, int E, bool valid, float* lg) {
  constexpr int VN = Vec<Tin>::N;
  const int lane = threadIdx.x % kWave;
  for (int e0 = 0; e0 < E; e0 += 8) {
    const int ne = min(8, E - e0);
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
    if (valid) {
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
        if (q < ne) lg[e0 + q] = acc[q] + (bias ? bias[e0 + q] : 0.0f);
    }
  }
}

}  // namespace moe
