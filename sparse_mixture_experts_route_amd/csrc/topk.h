// Per-token routing epilogue shared by the router kernels and the small-batch
// permute: softmax statistics and top-k selection of one token's logits.
//
// "Distributed training part 4" (jesamkim's AI tech blog), section 3,
// structure: a Softmax gives each expert a probability and only the k best
// experts are used. Selection is on the float32 logits, descending, ties to
// the lower expert index; the gate is the softmax probability over all E.
#pragma once

#include "common.h"

namespace moe {

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

// Top-k (k <= kTopkFast) of the RT tokens of a block whose logits are in LDS
// (row r at lg + r * ld): four threads per token; thread q of the group takes
// experts q, q + 4, ... eight at a time. Keys are those of select_topk
// (order-preserving logit bits above the inverted expert index, all
// distinct). Each group of eight is sorted by a bitonic network and merged
// into the thread's running top eight (the larger of top[i] and chunk[7 - i]
// for every i is a bitonic sequence that holds the eight largest of both;
// a bitonic merge sorts it), then the four threads' lists are merged the same
// way over two rounds of lane exchanges. The keys being distinct, the result
// is the unique top eight in descending order, as select_topk selects.
// Softmax maximum and sum are combined over the four threads in fixed order.
constexpr int kTopkFast = 8;

__device__ __forceinline__ void cswap_desc(uint64_t& a, uint64_t& b) {  // a >= b afterwards
  const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
  a = hi;
  b = lo;
}

// eight keys into descending order (bitonic sorting network, 24 compare-swaps)
__device__ __forceinline__ void sort8_desc(uint64_t (&v)[kTopkFast]) {
#pragma unroll
  for (int kk = 2; kk <= kTopkFast; kk <<= 1)
#pragma unroll
    for (int j = kk >> 1; j > 0; j >>= 1)
#pragma unroll
      for (int i = 0; i < kTopkFast; ++i) {
        const int l = i ^ j;
        if (l > i) {
          if ((i & kk) == 0)
            cswap_desc(v[i], v[l]);
          else
            cswap_desc(v[l], v[i]);
        }
      }
}

// top (descending) becomes the eight largest of top and b (both descending)
__device__ __forceinline__ void merge_top8(uint64_t (&top)[kTopkFast], const uint64_t (&b)[kTopkFast]) {
#pragma unroll
  for (int i = 0; i < kTopkFast; ++i) top[i] = top[i] > b[kTopkFast - 1 - i] ? top[i] : b[kTopkFast - 1 - i];
#pragma unroll
  for (int j = kTopkFast >> 1; j > 0; j >>= 1)
#pragma unroll
    for (int i = 0; i < kTopkFast; ++i) {
      const int l = i ^ j;
      if (l > i) cswap_desc(top[i], top[l]);
    }
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  const uint32_t lo = __shfl_xor((uint32_t)v, o, kWave), hi = __shfl_xor((uint32_t)(v >> 32), o, kWave);
  return ((uint64_t)hi << 32) | lo;
}

template <int RT_, int NT_ = 256>
__device__ __forceinline__ void select_topk_block(const float* lg, int ld, int64_t t0, int64_t T, int E, int k,
                                                  int32_t* __restrict__ idx, float* __restrict__ gate) {
  static_assert(RT_ * 4 == NT_, "four threads per token");
  const int r = threadIdx.x >> 2, q = threadIdx.x & 3;
  const float* row = lg + r * ld;
  uint64_t top[kTopkFast];
#pragma unroll
  for (int j = 0; j < kTopkFast; ++j) top[j] = 0;  // below every finite logit's key
  float m = -INFINITY;
  for (int e0 = q; e0 < E; e0 += 4 * kTopkFast) {
    uint64_t c[kTopkFast];
#pragma unroll
    for (int j = 0; j < kTopkFast; ++j) {
      const int e = e0 + 4 * j;
      c[j] = 0;
      if (e < E) {
        const float l = row[e];
        m = fmaxf(m, l);
        c[j] = ((uint64_t)float_order_key(l) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
      }
    }
    sort8_desc(c);
    merge_top8(top, c);
  }
  m = fmaxf(m, __shfl_xor(m, 1, kWave));
  m = fmaxf(m, __shfl_xor(m, 2, kWave));
  float ssum = 0.0f;
  for (int e = q; e < E; e += 4) ssum += expf(row[e] - m);
  ssum += __shfl_xor(ssum, 1, kWave);
  ssum += __shfl_xor(ssum, 2, kWave);
#pragma unroll
  for (int o = 1; o <= 2; o <<= 1) {
    uint64_t other[kTopkFast];
#pragma unroll
    for (int j = 0; j < kTopkFast; ++j) other[j] = shfl_xor_u64(top[j], o);
    merge_top8(top, other);
  }
  const int64_t t = t0 + r;
  if (q == 0 && t < T) {
#pragma unroll
    for (int j = 0; j < kTopkFast; ++j)
      if (j < k) {
        const int es = (int)(0xFFFFFFFFu - (uint32_t)top[j]);
        idx[t * k + j] = es;
        gate[t * k + j] = expf(row[es] - m) / ssum;
      }
  }
}

// One wave: the logits of token t of a router split over d_model, i.e. the
// nsplit float32 partial logits part[s][t][e] added in split order, plus the
// bias, into `row` (lane l owns experts 4l .. 4l+3, 16-byte loads, eight
// splits in flight). Every kernel that completes a split uses this, so the
// logits do not depend on which one did. E is a multiple of 4, at most 256.
__device__ __forceinline__ void sum_partial_logits(const float* __restrict__ part, int nsplit,
                                                   const float* __restrict__ bias, int64_t T, int E, int64_t t,
                                                   float* row) {
  const int e0 = (threadIdx.x % kWave) * 4;
  if (e0 >= E) return;
  const float* src = part + t * E + e0;
  const int64_t stride = T * E;
  f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
  int s2 = 0;
  for (; s2 + 8 <= nsplit; s2 += 8) {
    f32x4 w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) w[u] = *(const f32x4*)(src + (s2 + u) * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) v += w[u];
  }
  for (; s2 < nsplit; ++s2) v += *(const f32x4*)(src + s2 * stride);
#pragma unroll
  for (int q = 0; q < 4; ++q) row[e0 + q] = v[q] + (bias ? bias[e0 + q] : 0.0f);
}

}  // namespace moe
