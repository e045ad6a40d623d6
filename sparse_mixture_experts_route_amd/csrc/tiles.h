// Tile list of the grouped GEMMs over ragged expert row groups and the split
// of a persistent launch's last round, shared by the forward and backward kernels.
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

// Position of tile `local` (0 .. mt * n_tiles - 1) among one expert's mt m-tiles
// x n_tiles n-tiles. The m-tiles go in groups of gm (the last group holds the
// rest); inside a group the n-tile is the major index and the m-tile the minor
// one. A round of consecutive tiles then covers gm row slabs and a few weight
// slabs, which the blocks of an XCD read together through its L2, also for an
// expert with many m-tiles (one n-tile major order over all of them would put
// up to a whole round of row slabs next to a single weight slab).
// gm <= 0 or mt <= gm: one group.
__host__ __device__ __forceinline__ void tile_coords(int local, int mt, int n_tiles, int gm, int& nt, int& m) {
  if (gm <= 0 || mt <= gm) {
    nt = local / mt;
    m = local - nt * mt;
    return;
  }
  const int per = gm * n_tiles, full = mt / gm;
  const int grp = local / per, in = local - grp * per;
  const int g = grp < full ? gm : mt - full * gm;
  nt = in / g;
  m = grp * gm + (in - nt * g);
}

// m-tiles per raster group of the grouped GEMMs (tile_coords); MOE_GEMM_GROUP_M
// overrides it (0: one group per expert).
constexpr int kGroupM = 8;
int group_m();

// Work of one block of a persistent launch over `tiles` tiles of `nk` K steps
// shared by `nb` blocks (index j): `full` whole tiles (tiles j, j + nb, ...),
// then units [s0, s1) of the remaining rem * nk (tile, K step) units, counted
// tile-major over the last `rem` tiles; they touch leftover tiles
// r_first .. r_first + n_items - full - 1 (at most two, as rem < nb).
// The leftover tiles are split only when they fill at most a third of a round
// (a fuller last round runs on partly idle CUs anyway) and when the K steps it
// saves, (nb - rem) / nb of a tile, outweigh the partial-sum traffic and the
// fixup launch, which cost about as much as `min_steps` K steps (24 measured
// on gfx950 with 256 x 256 tiles).
template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

struct SplitK {
  int full, rem, r_first, n_items;
  int64_t s0, s1;
};

constexpr int kSplitMinSteps = 24;

// `max_rem` caps the leftover tiles that may be split: nb / 3 for the tiles
// that fill the matrix cores, nb - 1 for the small-M tile of decode-sized
// batches, whose one partly filled round would otherwise leave most blocks
// idle while a few stream whole weight slabs.
__host__ __device__ __forceinline__ bool split_leftover(int rem, int nb, int nk, int min_steps, int max_rem) {
  return rem > 0 && rem <= max_rem && (int64_t)nk * (nb - rem) >= (int64_t)min_steps * nb;
}

__device__ __forceinline__ SplitK split_k(int tiles, int nb, int j, int nk, int min_steps, int max_rem) {
  SplitK r;
  r.full = tiles / nb;
  r.rem = tiles - r.full * nb;
  if (!split_leftover(r.rem, nb, nk, min_steps, max_rem)) {
    r.full += j < r.rem ? 1 : 0;  // one more round of whole tiles for the first rem blocks
    r.rem = 0;
    r.s0 = r.s1 = 0;
    r.r_first = 0;
    r.n_items = r.full;
    return r;
  }
  const int64_t W = (int64_t)r.rem * nk;
  r.s0 = W * j / nb;
  r.s1 = W * (j + 1) / nb;
  r.r_first = r.s1 > r.s0 ? (int)(r.s0 / nk) : 0;
  const int n_rem = r.s1 > r.s0 ? (int)((r.s1 - 1) / nk) - r.r_first + 1 : 0;
  r.n_items = r.full + n_rem;
  return r;
}

}  // namespace moe
