// Tile list of the grouped GEMMs over ragged expert row groups, shared by the
// forward and backward kernels.
#pragma once

#include "common.h"

namespace moe {

// Tile list of a grouped GEMM whose rows are grouped by expert: tstart[e] = first tile of expert e (exclusive
// prefix over experts of m_tiles(e) * n_tiles), tstart[E] = total;
// mtiles[e] = ceil(rows_e / BM). Computed by wave 0, shared through LDS.
template <int BM>
__device__ __forceinline__ void build_tile_list(const int32_t* __restrict__ offsets, int E, int64_t R,
                                                int n_tiles, int* tstart, int* mtiles) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int cnt[4];
    int local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane * 4 + i;
      int c = 0;
      if (e < E) {
        const int64_t lo = max((int64_t)offsets[e], (int64_t)0), hi = min((int64_t)offsets[e + 1], R);
        c = hi > lo ? (int)ceil_div(hi - lo, BM) : 0;
        mtiles[e] = c;
      }
      cnt[i] = c * n_tiles;
      local += cnt[i];
    }
    int incl = local;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    int run = incl - local;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane * 4 + i;
      if (e < E) tstart[e] = run;
      run += cnt[i];
    }
    if (lane == kWave - 1) tstart[E] = incl;
  }
  __syncthreads();
}

}  // namespace moe
