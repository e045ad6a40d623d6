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
//     Operands stream HBM -> LDS through a ring of stages with direct-to-LDS
//     loads and one barrier per K step; x tiles sit K-contiguous in LDS,
//     w_router tiles stay E-contiguous and are read with ds_read_b64_tr_b16
//     (4 consecutive k of one column per lane). The float32 logits of the
//     block land in the (then idle) ring for the epilogue.
//   * otherwise (float32, or E not a multiple of 8): one wave per token; each
//     lane takes 16-byte pieces of the token's row and multiplies them with
//     the matching w_router rows for up to 8 experts at a time; per-expert
//     partial sums are reduced across the wave.
//   * epilogue, one wave per token: max and sum of exponentials over the E
//     logits, then k rounds of a wave-wide max over 64-bit keys
//     (order-preserving logit key in the upper half, inverted expert index in
//     the lower half, so equal logits favour the lower index).
#include "common.h"
#include "gemm_lanes.h"
#include "internal.h"
#include "lds_dma.h"
#include "route_fma.h"
#include "topk.h"

namespace moe {

namespace {

// ---------------------------------------------------------------- matrix-core path

constexpr int RT64 = 64;  // tokens per block (RT32: a block of 32 tokens and two waves)
constexpr int RT32 = 32;
constexpr int RBK = 64; // K step

// true when c ^ m < n for every chunk c < n and mask m' <= m (all XOR masks
// the swizzle uses), i.e. the XOR permutes the row's n chunks
constexpr bool xor_stays_in_row(int n, int m) {
  for (int mm = 0; mm <= m; ++mm)
    for (int c = 0; c < n; ++c)
      if ((c ^ mm) >= n) return false;
  return true;
}

// Block: RT tokens x EP experts (E padded), RT / 16 waves in a (RT / 32) x 2
// grid, each 32 tokens x EP/2 experts. Operands stream HBM -> LDS through a ring of S
// stages with direct-to-LDS loads (x rows K-contiguous, chunk XOR-swizzled;
// w_router rows E-contiguous, read with the transposing LDS read), one
// barrier per K step, the fragments of the next K sub-step read while the
// MFMAs of the current one run. After the last step the ring holds the
// block's float32 logits (+ bias) for the selection epilogue.
//
// Split over d_model (gridDim.y = nsplit > 1): block (b, s) takes K steps
// [s nk / nsplit, (s+1) nk / nsplit) and writes its float32 partial logits
// (no bias) to part[s][t][e]; route_finalize_kernel adds them up and selects.
template <int EP, int S, int RT = 64>
__global__ __launch_bounds__(RT * 4) void route_mfma_kernel(const bf16_bits* __restrict__ x,
                                                         const bf16_bits* __restrict__ wr,
                                                         const float* __restrict__ bias, float* __restrict__ logits,
                                                         int32_t* __restrict__ idx, float* __restrict__ gate,
                                                         float* __restrict__ part, int64_t T, int d, int E_real,
                                                         int k) {
  constexpr int NW = RT / 16;                 // 2 x 2 waves for 64 tokens, 1 x 2 for 32
  static_assert(RT == 64 || RT == 32, "router block of 64 or 32 tokens");
  constexpr int WTN = EP / 2, TN = WTN / 32;  // experts per wave, 32-wide MFMA tiles
  constexpr int KS = RBK / 16;                // MFMA K sub-steps per stage
  constexpr int A_ROW = RBK * 2, A_STAGE = RT * A_ROW;
  constexpr int B_ROW = EP * 2, B_SLOTS = EP / 8, B_STAGE = RBK * B_ROW;
  constexpr int STAGE = A_STAGE + B_STAGE;
  constexpr int A_LD = A_STAGE / 1024 / NW, B_LD = B_STAGE / 1024 / NW, NL = A_LD + B_LD;
  // B chunk swizzle: XOR by BSW * (k & 3), a permutation of the row's chunks
  // (24 chunks, E padded to 192, only take XORs below 8)
  constexpr int BSW = B_SLOTS % 16 == 0 ? 4 : 2;
  static_assert(xor_stays_in_row(B_SLOTS, BSW * 3), "router B swizzle leaves the row");
  constexpr int LG_ROW = EP + 1;              // float32 logits row in the epilogue
  constexpr int RING = S * STAGE;
  constexpr int SMEM = RING > RT * LG_ROW * 4 ? RING : RT * LG_ROW * 4;
  static_assert(A_LD * 1024 * NW == A_STAGE && B_LD * 1024 * NW == B_STAGE && TN >= 1, "router tile");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int64_t t0 = (int64_t)blockIdx.x * RT;
  const int wm0 = (wave >> 1) * 32, wn0 = (wave & 1) * WTN;
  lds_char* const lds = (lds_char*)smem;
  const uint32_t lds_base = lds_addr(smem);
  const int nk_all = d / RBK;
  const int nsplit = gridDim.y, split = blockIdx.y;
  const int kt0 = (int)((int64_t)nk_all * split / nsplit);
  const int nk = (int)((int64_t)nk_all * (split + 1) / nsplit) - kt0;  // >= 1: nsplit <= nk_all

  // tokens past T and k past d read as zero (descriptor ranges)
  const int rows = (int)min((int64_t)RT, T - t0);
  const i32x4 rsA = buffer_rsrc(x + t0 * d, (uint32_t)(rows * d * 2));
  const i32x4 rsB = buffer_rsrc(wr, (uint32_t)(d * E_real * 2));

  // per-lane DMA offsets: x piece (row, chunk), w piece (k, chunk); chunks of
  // padded experts (>= E_real) point past the range and load zeros, also with
  // the scalar K offset added (no 32-bit wrap: see lanes::kOutOfRange)
  uint32_t a_off[A_LD], b_off[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int p = (wave * A_LD + i) * kWave + lane;
    const int row = p / 8, c = (p % 8) ^ ((row >> 1) & 7);
    a_off[i] = (uint32_t)(row * d + c * 8) * 2u;
  }
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int p = (wave * B_LD + i) * kWave + lane;
    const int kk = p / B_SLOTS, c = (p % B_SLOTS) ^ (BSW * (kk & 3));
    b_off[i] = c * 8 < E_real ? (uint32_t)(kk * E_real + c * 8) * 2u : lanes::kOutOfRange;
  }
  auto issue_one = [&](int kt, int buf, int i) {
    const uint32_t st = lds_base + buf * STAGE;
    if (i < A_LD)
      buffer_load_lds16(rsA, a_off[i], (uint32_t)(kt0 + kt) * RBK * 2, st + (wave * A_LD + i) * 1024);
    else
      buffer_load_lds16(rsB, b_off[i - A_LD], (uint32_t)(kt0 + kt) * RBK * E_real * 2,
                        st + A_STAGE + (wave * B_LD + i - A_LD) * 1024);
  };

  // fragment read offsets
  const int a_rd = (wm0 + (lane & 31)) * A_ROW;
  int a_x[KS];
  {
    const int sw = ((lane & 31) >> 1) & 7;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a_x[ks] = ((ks * 2 + (lane >> 5)) ^ sw) << 4;
  }
  const int q = lane & 15, g = lane >> 4, kr = q >> 2;
  int b_rd[TN];
#pragma unroll
  for (int ni = 0; ni < TN; ++ni) {
    const int col = wn0 + ni * 32 + (g & 1) * 16 + (q & 3) * 4;
    b_rd[ni] = A_STAGE + ((g >> 1) * 8 + kr) * B_ROW + (((col >> 3) ^ (BSW * kr)) << 4) + (col & 7) * 2;
  }
  bf16x8 fa[2], fb[2][TN];
  auto read_set = [&](int buf, int ks, int set) {
    lds_char* const st = lds + buf * STAGE;
    fa[set] = *(lds_bf16x8*)(st + a_rd + a_x[ks]);
#pragma unroll
    for (int ni = 0; ni < TN; ++ni) {
      lds_char* const p0 = st + ks * 16 * B_ROW + b_rd[ni];
      const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
      const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 4 * B_ROW));
      fb[set][ni] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  f32x16 acc[TN];
#pragma unroll
  for (int ni = 0; ni < TN; ++ni)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[ni][v] = 0.0f;

#pragma unroll
  for (int s2 = 0; s2 < S; ++s2)
    if (s2 < nk)
#pragma unroll
      for (int i = 0; i < NL; ++i) issue_one(s2, s2, i);
  if (nk > S - 1)
    wait_vmem<NL * (S - 1)>();
  else
    wait_vmem<0>();
  __syncthreads();
  read_set(0, 0, 0);

  int buf = 0;
  for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int set = ks & 1;
      if (ks + 1 < KS) read_set(buf, ks + 1, set ^ 1);
#pragma unroll
      for (int ni = 0; ni < TN; ++ni)
        acc[ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[set][ni], fa[set], acc[ni], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      // stage kt+1 has landed once at most the loads of stages kt+2 .. kt+S-1 are outstanding
      if (kt + S - 1 < nk)
        wait_vmem<NL * (S - 2)>();
      else
        wait_vmem<0>();
      __syncthreads();  // every wave is done with `buf`; stage kt+1 is visible
      if (kt + S < nk)
#pragma unroll
        for (int i = 0; i < NL; ++i) issue_one(kt + S, buf, i);
      buf = buf + 1 == S ? 0 : buf + 1;
      read_set(buf, 0, 0);
    }
  }
  __syncthreads();  // the ring becomes the logits buffer

  // lane holds token (lane & 31) of the wave's rows, experts 8 gq + 4 (lane >> 5) + 0..3 of each tile
  float* const lg = (float*)smem;
#pragma unroll
  for (int ni = 0; ni < TN; ++ni)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int e = wn0 + ni * 32 + 8 * gq + 4 * (lane >> 5) + qq;
        if (e < E_real)
          lg[(wm0 + (lane & 31)) * LG_ROW + e] = acc[ni][4 * gq + qq] + (bias && nsplit == 1 ? bias[e] : 0.0f);
      }
  __syncthreads();
  if (nsplit > 1) {  // partial logits of this K range, rows of the block, coalesced
    float* const dst = part + ((int64_t)split * T + t0) * E_real;
    for (int i = tid; i < rows * E_real; i += NW * kWave) {
      const int r = i / E_real, e = i - r * E_real;
      dst[i] = lg[r * LG_ROW + e];
    }
    return;
  }
  if (k <= kTopkFast) {
    select_topk_block<RT, RT * 4>(lg, LG_ROW, t0, T, E_real, k, idx, gate);
    if (logits)  // rows of the block, coalesced
      for (int i = tid; i < RT * E_real; i += NW * kWave) {
        const int r = i / E_real, e = i - r * E_real;
        if (t0 + r < T) logits[(t0 + r) * E_real + e] = lg[r * LG_ROW + e];
      }
  } else {
    for (int r = wave; r < RT; r += NW) {
      const int64_t t = t0 + r;
      if (t < T) select_topk(lg + r * LG_ROW, E_real, k, t, logits, idx, gate);
    }
  }
}

// Completion of a router split over d_model, one wave per token: the token's
// partial logits are added in split order (sum_partial_logits) and the row
// goes to select_topk through the wave's LDS row. No block-wide barrier:
// waves past T leave at once.
constexpr int kFinalizeWaves = 4;

__global__ __launch_bounds__(kFinalizeWaves * kWave) void route_finalize_kernel(
    const float* __restrict__ part, int nsplit, const float* __restrict__ bias, float* __restrict__ logits,
    int32_t* __restrict__ idx, float* __restrict__ gate, int64_t T, int E, int k) {
  __shared__ float lg[kFinalizeWaves][256];
  const int wave = threadIdx.x / kWave;
  const int64_t t = (int64_t)blockIdx.x * kFinalizeWaves + wave;
  if (t >= T) return;
  sum_partial_logits(part, nsplit, bias, T, E, t, lg[wave]);
  // LDS accesses of one wave execute in order: the row is complete for the reads below
  select_topk(lg[wave], E, k, t, logits, idx, gate);
}

// ---------------------------------------------------------------- FMA path

constexpr int kRouteWaves = 4;  // tokens per block

template <typename Tin>
__global__ __launch_bounds__(kRouteWaves * kWave) void route_fma_kernel(
    const Tin* __restrict__ x, const Tin* __restrict__ wr, const float* __restrict__ bias,
    float* __restrict__ logits, int32_t* __restrict__ idx, float* __restrict__ gate, int64_t T, int d, int E,
    int k) {
  __shared__ float lg[kRouteWaves][256];
  const int wave = threadIdx.x / kWave;
  const int64_t t = (int64_t)blockIdx.x * kRouteWaves + wave;
  const bool valid = t < T;
  route_row_fma(x + (valid ? t : 0) * (int64_t)d, wr, bias, d, E, valid, lg[wave]);
  __syncthreads();
  if (valid) select_topk(lg[wave], E, k, t, logits, idx, gate);
}

}  // namespace

// Tokens per matrix-core router block. MOE_ROUTE_RT=32|64 forces a size.
int route_rt(const moe_problem_t& p) {
  const char* force = getenv("MOE_ROUTE_RT");
  if (force && force[0]) return atoi(force) == 32 ? RT32 : RT64;
  // 32-token blocks where 64-token blocks would leave CUs idle but are too
  // many to split over d_model (a quarter to all of the CUs), and the router
  // tile is narrow enough that twice the w_router reads per token stay cheap.
  // Measured on MI355X: 8192 tokens x 64 experts x 2048, 19.1 against 21.2 us;
  // 4096 tokens x 8 experts (split) and 16384 tokens keep 64.
  const int64_t b64 = ceil_div(p.T, RT64);
  const int cus = device_cus();
  if (p.E <= 128 && b64 * 4 > cus && b64 < cus) return RT32;
  return RT64;
}

// the router kernel for the padded expert count and block size
template <typename Go>
hipError_t route_dispatch(const moe_problem_t& p, Go go) {
  const bool small = route_rt(p) == RT32;
  switch ((p.E + 63) / 64 * 64) {
    case 64:
      return small ? go(route_mfma_kernel<64, 4, RT32>, RT32) : go(route_mfma_kernel<64, 4>, RT64);
    case 128:
      return small ? go(route_mfma_kernel<128, 4, RT32>, RT32) : go(route_mfma_kernel<128, 4>, RT64);
    case 192:
      return small ? go(route_mfma_kernel<192, 3, RT32>, RT32) : go(route_mfma_kernel<192, 3>, RT64);
    default:
      return small ? go(route_mfma_kernel<256, 3, RT32>, RT32) : go(route_mfma_kernel<256, 3>, RT64);
  }
}

int route_splits(const moe_problem_t& p) {
  if (p.dtype != MOE_DTYPE_BF16 || p.E % 8 != 0) return 1;
  const int64_t blocks = ceil_div(p.T, route_rt(p));
  const int nk = p.d_model / RBK;
  // MOE_ROUTE_SPLITS=<n> forces n splits (clamped to the K steps and the finalize's 64 KB per token)
  const char* force = getenv("MOE_ROUTE_SPLITS");
  if (force && force[0]) {
    int64_t ns = max(1, atoi(force));
    ns = min(ns, (int64_t)nk);
    ns = min(ns, (int64_t)(64 * 1024) / (p.E * 4));
    return (int)max(ns, (int64_t)1);
  }
  const int cus = device_cus();
  // measured on MI355X: with a quarter of the CUs or more busy the single pass
  // (contraction and selection in one launch) is faster than a split plus the
  // wave-per-token finalize (e.g. 8192 tokens, 64 experts, top-8: 27 against 32 us)
  if (blocks * 4 > cus) return 1;
  int64_t ns = ceil_div(2 * cus, blocks);  // about two router blocks per CU
  ns = min(ns, (int64_t)nk / 4);           // at least four K steps per split
  // partial logits that one finalize wave adds up for its token: at most 64 KB
  ns = min(ns, (int64_t)(64 * 1024) / (p.E * 4));
  return (int)max(ns, (int64_t)1);
}

size_t route_partials_bytes(const moe_problem_t& p) {
  const int ns = route_splits(p);
  return ns > 1 ? (size_t)ns * p.T * p.E * sizeof(float) : 0;
}

hipError_t launch_route_partials(const moe_problem_t& p, const void* x, const void* w_router, float* part,
                                 hipStream_t s) {
  const int ns = route_splits(p);
  if (ns <= 1 || !part) return hipErrorInvalidValue;
  const bf16_bits* xb = (const bf16_bits*)x;
  const bf16_bits* wb = (const bf16_bits*)w_router;
  return route_dispatch(p, [&](auto kern, int rt) {
    hipLaunchKernelGGL(kern, dim3((unsigned)ceil_div(p.T, rt), (unsigned)ns), dim3(rt * 4), 0, s, xb, wb, nullptr,
                       nullptr, nullptr, nullptr, part, p.T, p.d_model, p.E, p.k);
    return hipGetLastError();
  });
}

hipError_t launch_route(const moe_problem_t& p, const void* x, const void* w_router, const float* bias,
                        float* logits, int32_t* idx, float* gate, float* part, hipStream_t s) {
  if (p.dtype == MOE_DTYPE_BF16 && p.E % 8 == 0) {
    const bf16_bits* xb = (const bf16_bits*)x;
    const bf16_bits* wb = (const bf16_bits*)w_router;
    const int ns = part ? route_splits(p) : 1;
    // ring stages: 4 while a stage is small, 3 for the widest tiles (LDS: S * (RT * 128 + 128 * EP B))
    return route_dispatch(p, [&](auto kern, int rt) {
      hipLaunchKernelGGL(kern, dim3((unsigned)ceil_div(p.T, rt), (unsigned)ns), dim3(rt * 4), 0, s, xb, wb, bias,
                         logits, idx, gate, part, p.T, p.d_model, p.E, p.k);
      if (ns > 1)
        hipLaunchKernelGGL(route_finalize_kernel, dim3((unsigned)ceil_div(p.T, kFinalizeWaves)),
                           dim3(kFinalizeWaves * kWave), 0, s,
                           (const float*)part, ns, bias, logits, idx, gate, p.T, p.E, p.k);
      return hipGetLastError();
    });
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
