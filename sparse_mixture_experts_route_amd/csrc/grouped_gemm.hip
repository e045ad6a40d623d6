// Expert FFN GEMMs over ragged per-expert row groups.
//
// "Distributed training part 4" (jesamkim's AI tech blog), section 3: the
// experts are independent FFNs. The MOSAIC summary ("Compute-Optimal Is Not
// Cluster-Optimal", gist.science, method item 2) counts their cost as grouped
// GEMMs. For every expert e with rows [offsets[e], offsets[e+1]):
//   C[rows] = act(A[rows] B[e]),  A [R, K] (K contiguous), B [E, K, N] (N contiguous)
// with act = GELU_tanh for the first expert GEMM and identity for the second.
//
// bf16 path (gfx950 matrix cores):
//   * v_mfma_f32_32x32x16_bf16, float32 accumulators, 64-wide wavefronts;
//   * block tile BM x BN, K step 64, LDS double buffer; each wave owns a
//     (BM/WM) x (BN/WN) sub-tile of 32x32 MFMA tiles;
//   * both operands sit in LDS K-contiguous ([row][64] bf16, 128 B per row)
//     with the 16-byte chunk index XOR-ed by (row & 7), so the 8 lanes of a
//     16-byte LDS access phase hit 8 different chunk positions;
//   * B arrives N-contiguous from HBM; each thread loads an 8(k) x 8(n)
//     sub-block (eight 16-byte row pieces) and transposes it in registers
//     before the LDS store;
//   * operands are passed to the MFMA as (B, A), so each lane's accumulators
//     hold 4 consecutive output columns of one row: the epilogue applies
//     GELU in float32, rounds to bf16 and stores 8 bytes per group;
//   * the tile of a block is found on the device from offsets[] (tiles of
//     expert e = ceil(rows_e / BM), enumerated expert by expert), so no host
//     synchronisation on the routing is needed; empty groups own no tiles;
//   * blocks are renumbered so that each XCD (the hardware deals blocks to
//     the 8 XCDs round robin) works on a contiguous run of tiles, which share
//     A rows and expert weights in that XCD's L2.
// float32 path: a plain LDS-tiled FMA kernel (the fp32 workload is small).
#include <stdlib.h>
#include <string.h>

#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int BK = 64;  // K step (bf16 path)

// Locate the m-tile `m_tile` in the expert-by-expert tile enumeration.
// Writes {expert, first row, end row} to info (expert -1 when past the end).
template <int BM>
__device__ __forceinline__ void find_tile(const int32_t* __restrict__ offsets, int E, int64_t R, int m_tile,
                                          int* info) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int cnt[4];
    int local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane * 4 + i;
      int c = 0;
      if (e < E) {
        const int64_t lo = offsets[e], hi = min((int64_t)offsets[e + 1], R);
        c = hi > lo ? (int)ceil_div(hi - lo, BM) : 0;
      }
      cnt[i] = c;
      local += c;
    }
    int incl = local;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    const int excl = incl - local;
    const bool mine = m_tile >= excl && m_tile < incl;
    const uint64_t who = __ballot(mine);
    if (mine) {
      int run = excl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (m_tile >= run && m_tile < run + cnt[i]) {
          const int e = lane * 4 + i;
          const int64_t lo = offsets[e];
          info[0] = e;
          info[1] = (int)(lo + (int64_t)(m_tile - run) * BM);
          info[2] = (int)min((int64_t)offsets[e + 1], R);
        }
        run += cnt[i];
      }
    }
    if (who == 0 && lane == 0) info[0] = -1;
  }
  __syncthreads();
}

__device__ __forceinline__ int xcd_remap(int nblk) {
  // blocks are dealt to the 8 XCDs round robin; give XCD x the run [x*n/8, (x+1)*n/8)
  return (blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8;
}

template <int BM, int BN, int WM, int WN, bool GELU>
__global__ __launch_bounds__(WM* WN* kWave) void gemm_bf16_kernel(
    const bf16_bits* __restrict__ A, const int32_t* __restrict__ offsets, const bf16_bits* __restrict__ B,
    bf16_bits* __restrict__ C, int64_t R, int K, int N, int E, int n_tiles, int grid_tiles) {
  constexpr int NT = WM * WN * kWave;
  constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;  // 32x32 MFMA tiles per wave
  constexpr int A_ITERS = BM * (BK / 8) / NT;  // 16-byte A pieces per thread per K step
  constexpr int B_SUBS = (BK / 8) * (BN / 8);  // 8x8 sub-blocks of a B tile
  constexpr int B_ITERS = (B_SUBS + NT - 1) / NT;
  static_assert(BM * (BK / 8) % NT == 0, "A tile must split evenly over the block");
  static_assert(TM >= 1 && TN >= 1, "wave tile must hold a 32x32 MFMA tile");

  __shared__ __attribute__((aligned(16))) bf16_bits As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) bf16_bits Bs[2][BN * BK];
  __shared__ int s_info[3];

  const int bid = xcd_remap(gridDim.x);
  if (bid >= grid_tiles) return;
  const int m_tile = bid / n_tiles, n_tile = bid % n_tiles;
  find_tile<BM>(offsets, E, R, m_tile, s_info);
  const int e = s_info[0];
  if (e < 0) return;
  const int64_t row0 = s_info[1], row_end = s_info[2];
  if (row0 >= row_end) return;
  const int n0 = n_tile * BN;
  const bf16_bits* __restrict__ Be = B + (int64_t)e * K * N;

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int wm0 = (wave / WN) * WTM, wn0 = (wave % WN) * WTN;

  // global -> LDS addressing
  const bf16_bits* a_src[A_ITERS];
  int a_dst[A_ITERS];
#pragma unroll
  for (int i = 0; i < A_ITERS; ++i) {
    const int q = tid + NT * i, row = q >> 3, kc = q & 7;
    const int64_t grow = min(row0 + row, row_end - 1);
    a_src[i] = A + grow * K + kc * 8;
    a_dst[i] = row * BK + ((kc ^ (row & 7)) << 3);
  }
  const bf16_bits* b_src[B_ITERS];
  int b_ng[B_ITERS], b_kg[B_ITERS];
  bool b_on[B_ITERS];
#pragma unroll
  for (int i = 0; i < B_ITERS; ++i) {
    const int s = tid + NT * i;
    b_on[i] = s < B_SUBS;
    const int kg = s & 7, ng = (s >> 3) % (BN / 8);
    const int n = min(n0 + ng * 8, N - 8);
    b_src[i] = Be + (int64_t)(kg * 8) * N + n;
    b_ng[i] = ng;
    b_kg[i] = kg;
  }

  u32x4 ra[A_ITERS];
  u32x4 rb[B_ITERS][8];

  auto gload = [&](int kt) {
    const int64_t koff = (int64_t)kt * BK;
#pragma unroll
    for (int i = 0; i < A_ITERS; ++i) ra[i] = *(const u32x4*)(a_src[i] + koff);
#pragma unroll
    for (int i = 0; i < B_ITERS; ++i)
      if (b_on[i]) {
#pragma unroll
        for (int r = 0; r < 8; ++r) rb[i][r] = *(const u32x4*)(b_src[i] + (koff + r) * N);
      }
  };

  auto sts = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_ITERS; ++i) *(u32x4*)(&As[buf][a_dst[i]]) = ra[i];
#pragma unroll
    for (int i = 0; i < B_ITERS; ++i)
      if (b_on[i]) {
        // 8x8 transpose: rb[r] holds k = r for n = 0..7; w holds n = c for k = 0..7
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          u32x4 w;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t lo = rb[i][2 * j][c >> 1], hi = rb[i][2 * j + 1][c >> 1];
            w[j] = (c & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
          }
          const int n = b_ng[i] * 8 + c;
          *(u32x4*)(&Bs[buf][n * BK + ((b_kg[i] ^ c) << 3)]) = w;
        }
      }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int mi = 0; mi < TM; ++mi)
#pragma unroll
    for (int ni = 0; ni < TN; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;

  const int nk = K / BK;
  gload(0);
  sts(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int kc = ks * 2 + (lane >> 5);
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int mi = 0; mi < TM; ++mi) {
        const int row = wm0 + mi * 32 + (lane & 31);
        af[mi] = *(const bf16x8*)(&As[cur][row * BK + ((kc ^ (row & 7)) << 3)]);
      }
#pragma unroll
      for (int ni = 0; ni < TN; ++ni) {
        const int n = wn0 + ni * 32 + (lane & 31);
        bfr[ni] = *(const bf16x8*)(&Bs[cur][n * BK + ((kc ^ (n & 7)) << 3)]);
      }
#pragma unroll
      for (int mi = 0; mi < TM; ++mi)
#pragma unroll
        for (int ni = 0; ni < TN; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ni], af[mi], acc[mi][ni], 0, 0, 0);
    }
    if (kt + 1 < nk) sts(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds row (lane & 31) of each MFMA tile, columns 8g + 4*(lane>>5) + 0..3
#pragma unroll
  for (int mi = 0; mi < TM; ++mi) {
    const int64_t row = row0 + wm0 + mi * 32 + (lane & 31);
    if (row >= row_end) continue;
    bf16_bits* crow = C + row * N;
#pragma unroll
    for (int ni = 0; ni < TN; ++ni)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn0 + ni * 32 + 8 * g + 4 * (lane >> 5);
        if (n >= N) continue;
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[q] = acc[mi][ni][4 * g + q];
          if (GELU) v[q] = gelu_tanh(v[q]);
        }
        u32x2 o;
        o[0] = pack_bf16x2(v[0], v[1]);
        o[1] = pack_bf16x2(v[2], v[3]);
        *(u32x2*)(crow + n) = o;
      }
  }
}

// ---------------------------------------------------------------- float32 path

constexpr int F_BM = 64, F_BN = 64, F_BK = 16;

template <bool GELU>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A,
                                                       const int32_t* __restrict__ offsets,
                                                       const float* __restrict__ B, float* __restrict__ C,
                                                       int64_t R, int K, int N, int E, int n_tiles,
                                                       int grid_tiles) {
  __shared__ __attribute__((aligned(16))) float As[F_BK][F_BM + 4];
  __shared__ __attribute__((aligned(16))) float Bs[F_BK][F_BN];
  __shared__ int s_info[3];
  const int bid = blockIdx.x;
  if (bid >= grid_tiles) return;
  const int m_tile = bid / n_tiles, n_tile = bid % n_tiles;
  find_tile<F_BM>(offsets, E, R, m_tile, s_info);
  const int e = s_info[0];
  if (e < 0) return;
  const int64_t row0 = s_info[1], row_end = s_info[2];
  if (row0 >= row_end) return;
  const int n0 = n_tile * F_BN;
  const float* __restrict__ Be = B + (int64_t)e * K * N;
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;

  float acc[4][4] = {};
  const int a_row = tid / 4, a_k = (tid % 4) * 4;
  const int64_t a_grow = min(row0 + a_row, row_end - 1);
  const int b_k = tid / 16, b_n = min(n0 + (tid % 16) * 4, N - 4);
  for (int k0 = 0; k0 < K; k0 += F_BK) {
    const f32x4 av = *(const f32x4*)(A + a_grow * K + k0 + a_k);
#pragma unroll
    for (int i = 0; i < 4; ++i) As[a_k + i][a_row] = av[i];
    *(f32x4*)(&Bs[b_k][(tid % 16) * 4]) = *(const f32x4*)(Be + (int64_t)(k0 + b_k) * N + b_n);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < F_BK; ++kk) {
      const f32x4 a = *(const f32x4*)(&As[kk][ty * 4]);
      const f32x4 b = *(const f32x4*)(&Bs[kk][tx * 4]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = row0 + ty * 4 + i;
    const int n = n0 + tx * 4;
    if (row >= row_end || n >= N) continue;
    f32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = GELU ? gelu_tanh(acc[i][j]) : acc[i][j];
    *(f32x4*)(C + row * N + n) = o;
  }
}

// ---------------------------------------------------------------- host side

struct TileCfg {
  int bm, bn;
};

template <int BM, int BN, int WM, int WN>
hipError_t launch_bf16(const void* A, const int32_t* offsets, const void* B, void* C, int64_t R, int K, int N,
                       int E, bool gelu, hipStream_t s) {
  const int n_tiles = (int)ceil_div(N, BN);
  const int64_t m_tiles = (R + (int64_t)E * (BM - 1)) / BM;  // >= sum over experts of ceil(rows_e / BM)
  const int64_t grid_tiles = m_tiles * n_tiles;
  const int64_t blocks = ceil_div(grid_tiles, 8) * 8;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if (gelu)
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, true>), dim3((unsigned)blocks), dim3(WM * WN * kWave),
                       0, s, (const bf16_bits*)A, offsets, (const bf16_bits*)B, (bf16_bits*)C, R, K, N, E,
                       n_tiles, (int)grid_tiles);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, false>), dim3((unsigned)blocks),
                       dim3(WM * WN * kWave), 0, s, (const bf16_bits*)A, offsets, (const bf16_bits*)B,
                       (bf16_bits*)C, R, K, N, E, n_tiles, (int)grid_tiles);
  return hipGetLastError();
}

// Pick the block tile from the expected tile count: fewer, larger tiles
// use the matrix cores better, but a last partial wave of tiles over the 256
// CUs and padding rows of half-empty M tiles cost time.
int pick_tile(int64_t R, int N, int E) {
  const char* force = getenv("MOE_GEMM_TILE");
  if (force && force[0]) {
    if (!strcmp(force, "256x256")) return 0;
    if (!strcmp(force, "256x128")) return 1;
    if (!strcmp(force, "128x128")) return 2;
  }
  const TileCfg cfgs[3] = {{256, 256}, {256, 128}, {128, 128}};
  const double tile_eff[3] = {1.0, 0.92, 0.80};  // relative MFMA efficiency of one busy CU
  int best = 0;
  double best_score = -1.0;
  for (int c = 0; c < 3; ++c) {
    const double m_tiles = (double)R / cfgs[c].bm + 0.5 * E;
    const double tiles = m_tiles * ceil_div(N, cfgs[c].bn);
    const double waves = tiles / 256.0;
    const double wave_eff = tiles / (256.0 * (double)(int64_t)(waves + 0.999));
    const double pad_eff = (double)R / (m_tiles * cfgs[c].bm);
    const double score = tile_eff[c] * wave_eff * pad_eff;
    if (score > best_score) {
      best_score = score;
      best = c;
    }
  }
  return best;
}

}  // namespace

hipError_t launch_grouped_gemm(int dtype, const void* A, const int32_t* offsets, const void* B, void* C,
                               int64_t R, int K, int N, int E, bool gelu, hipStream_t s) {
  if (dtype == MOE_DTYPE_F32) {
    const int n_tiles = (int)ceil_div(N, F_BN);
    const int64_t m_tiles = (R + (int64_t)E * (F_BM - 1)) / F_BM;
    const int64_t grid_tiles = m_tiles * n_tiles;
    if (grid_tiles > INT32_MAX) return hipErrorInvalidValue;
    if (gelu)
      hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3((unsigned)grid_tiles), dim3(256), 0, s, (const float*)A,
                         offsets, (const float*)B, (float*)C, R, K, N, E, n_tiles, (int)grid_tiles);
    else
      hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3((unsigned)grid_tiles), dim3(256), 0, s, (const float*)A,
                         offsets, (const float*)B, (float*)C, R, K, N, E, n_tiles, (int)grid_tiles);
    return hipGetLastError();
  }
  switch (pick_tile(R, N, E)) {
    case 0:
      return launch_bf16<256, 256, 2, 2>(A, offsets, B, C, R, K, N, E, gelu, s);
    case 1:
      return launch_bf16<256, 128, 2, 2>(A, offsets, B, C, R, K, N, E, gelu, s);
    default:
      return launch_bf16<128, 128, 2, 2>(A, offsets, B, C, R, K, N, E, gelu, s);
  }
}

}  // namespace moe
