// Weighted combine: y[t] = sum over j < k of gate[t, j] * y_perm[inv[t*k + j]].
//
// "Distributed training part 4" (jesamkim's AI tech blog), section 3: the layer
// output is the sum over the selected experts of the router weight times the
// expert output; section 4, combine: the expert results return to the token
// they came from. Gather form: one wave per (token, chunk of its row) reads
// that chunk of the token's k expert rows and writes the same chunk of its
// output row, so no atomics are needed and the result is deterministic.
// Accumulation is float32, in selection order. With chunks, a few-token batch
// still spreads over many waves instead of a few long chains of loads.
#include <stdlib.h>

#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kCombineWaves = 4;

__device__ __forceinline__ void unpack8(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_to_f32(v[i] & 0xFFFFu);
    f[2 * i + 1] = bf16_to_f32(v[i] >> 16);
  }
}

constexpr int kCombineFastK = 8;  // selections per token whose rows are loaded together
constexpr int kCombineU = 2;      // 16-byte pieces per lane per row in flight
constexpr int kChunkVecs = kWave * kCombineU;  // 16-byte pieces of a row per wave
constexpr int64_t kCombineStreamBytes = 128ll << 20;  // y_perm size from which loads and stores stream

// NT: non-temporal loads of y_perm and stores of y (streamed once; see launch_combine)
template <bool NT>
__global__ __launch_bounds__(kCombineWaves * kWave) void combine_bf16_kernel(
    const u32x4* __restrict__ y_perm, const int32_t* __restrict__ inv, const float* __restrict__ gate,
    u32x4* __restrict__ y, int64_t T, int k, int64_t row_vecs, int64_t rows, int chunks) {
  const int lane = threadIdx.x % kWave;
  const int64_t w = (int64_t)blockIdx.x * kCombineWaves + threadIdx.x / kWave;
  const int64_t t = w / chunks;
  if (t >= T) return;
  const int64_t cv = (row_vecs + chunks - 1) / chunks;  // 16-byte pieces per chunk
  const int64_t c_lo = (w - t * chunks) * cv, c_hi = min(row_vecs, c_lo + cv);
  if (k <= kCombineFastK) {
    // the token's k source rows and gates, once; invalid selections contribute nothing
    int64_t src[kCombineFastK];
    float g[kCombineFastK];
#pragma unroll
    for (int j = 0; j < kCombineFastK; ++j) {
      const int32_t r = j < k ? inv[t * k + j] : -1;
      const bool ok = r >= 0 && r < rows;
      src[j] = ok ? (int64_t)r * row_vecs : -1;
      g[j] = ok ? gate[t * k + j] : 0.0f;
    }
    for (int64_t c0 = c_lo + lane; c0 < c_hi; c0 += kChunkVecs) {
      // all loads of this step first, then the accumulation in selection order
      u32x4 v[kCombineFastK][kCombineU];
#pragma unroll
      for (int j = 0; j < kCombineFastK; ++j)
#pragma unroll
        for (int u = 0; u < kCombineU; ++u)
          if (src[j] >= 0 && c0 + u * kWave < c_hi)
            v[j][u] = NT ? __builtin_nontemporal_load(y_perm + src[j] + c0 + u * kWave)
                         : y_perm[src[j] + c0 + u * kWave];
#pragma unroll
      for (int u = 0; u < kCombineU; ++u) {
        if (c0 + u * kWave >= c_hi) continue;
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
        for (int j = 0; j < kCombineFastK; ++j) {
          if (src[j] < 0) continue;
          float f[8];
          unpack8(v[j][u], f);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(g[j], f[i], acc[i]);
        }
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
        if (NT)
          __builtin_nontemporal_store(o, y + t * row_vecs + c0 + u * kWave);
        else
          y[t * row_vecs + c0 + u * kWave] = o;
      }
    }
    return;
  }
  for (int64_t c = c_lo + lane; c < c_hi; c += kWave) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int32_t r = inv[t * k + j];
      if (r < 0 || r >= rows) continue;
      const float g = gate[t * k + j];
      float v[8];
      unpack8(y_perm[(int64_t)r * row_vecs + c], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(g, v[i], acc[i]);
    }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
    y[t * row_vecs + c] = o;
  }
}

__global__ __launch_bounds__(kCombineWaves * kWave) void combine_f32_kernel(
    const f32x4* __restrict__ y_perm, const int32_t* __restrict__ inv, const float* __restrict__ gate,
    f32x4* __restrict__ y, int64_t T, int k, int64_t row_vecs, int64_t rows, int chunks) {
  const int lane = threadIdx.x % kWave;
  const int64_t w = (int64_t)blockIdx.x * kCombineWaves + threadIdx.x / kWave;
  const int64_t t = w / chunks;
  if (t >= T) return;
  const int64_t cv = (row_vecs + chunks - 1) / chunks;
  const int64_t c_lo = (w - t * chunks) * cv, c_hi = min(row_vecs, c_lo + cv);
  for (int64_t c = c_lo + lane; c < c_hi; c += kWave) {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j = 0; j < k; ++j) {
      const int32_t r = inv[t * k + j];
      if (r < 0 || r >= rows) continue;
      const float g = gate[t * k + j];
      const f32x4 v = y_perm[(int64_t)r * row_vecs + c];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(g, v[i], acc[i]);
    }
    y[t * row_vecs + c] = acc;
  }
}

}  // namespace

bool combine_streams(const moe_problem_t& p) {
  if (p.dtype != MOE_DTYPE_BF16) return false;
  bool nt = (double)p.T * p.k * p.d_model * 2 >= (double)kCombineStreamBytes;
  const char* force = getenv("MOE_COMBINE_NT");
  if (force && force[0]) nt = atoi(force) != 0;
  return nt;
}

hipError_t launch_combine(const moe_problem_t& p, const void* y_perm, const int32_t* inv, const float* gate,
                          void* y, hipStream_t s) {
  const int64_t rows = p.T * p.k;
  const int64_t row_vecs = p.d_model / (p.dtype == MOE_DTYPE_BF16 ? 8 : 4);
  // one pass of kChunkVecs pieces per wave (measured against 2, 3 and whole-row
  // passes: equal at 2048-wide rows, 4-7 % faster at 8k-16k tokens, 2.5x faster
  // at 8 tokens of 7168)
  const int chunks = (int)ceil_div(row_vecs, kChunkVecs);
  const int64_t blocks = ceil_div(p.T * chunks, kCombineWaves);
  if (p.dtype == MOE_DTYPE_BF16) {
    // Non-temporal accesses when y_perm is large: measured on MI355X with the
    // layer's stages in sequence, 256 MB of y_perm (8192 tokens, top-8, 2048
    // wide) combine in 49 instead of 58 us, 1.75 GB in 352 instead of 402 us;
    // at 32 MB (still in the last-level cache after the expert GEMM) plain
    // accesses are ~1 us faster. MOE_COMBINE_NT=0|1 forces the choice.
    if (combine_streams(p))
      hipLaunchKernelGGL(combine_bf16_kernel<true>, dim3((unsigned)blocks), dim3(kCombineWaves * kWave), 0, s,
                         (const u32x4*)y_perm, inv, gate, (u32x4*)y, p.T, p.k, row_vecs, rows, chunks);
    else
      hipLaunchKernelGGL(combine_bf16_kernel<false>, dim3((unsigned)blocks), dim3(kCombineWaves * kWave), 0, s,
                         (const u32x4*)y_perm, inv, gate, (u32x4*)y, p.T, p.k, row_vecs, rows, chunks);
  } else {
    hipLaunchKernelGGL(combine_f32_kernel, dim3((unsigned)blocks), dim3(kCombineWaves * kWave), 0, s,
                       (const f32x4*)y_perm, inv, gate, (f32x4*)y, p.T, p.k, row_vecs, rows, chunks);
  }
  return hipGetLastError();
}

}  // namespace moe
