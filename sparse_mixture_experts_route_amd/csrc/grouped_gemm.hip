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
//   * v_mfma_f32_32x32x16_bf16 with float32 accumulators; block tile BM x BN,
//     K step BK, WM x WN waves each owning (BM/WM) x (BN/WN). The default
//     tile is 256 x 256 with 8 waves (two per SIMD): issuing a direct-to-LDS
//     load stalls the issuing wave for tens of cycles, and the second wave on
//     the SIMD keeps the matrix core busy meanwhile;
//   * operands go HBM -> LDS with buffer_load_dwordx4 ... lds (no register
//     staging): every lane of a wave writes 16 bytes to consecutive LDS
//     slots, and the lane's global address is chosen so that the slot holds
//     the swizzled piece;
//   * A sits K-contiguous in LDS ([row][BK] bf16) with the 16-byte chunk index
//     XOR-ed by the row's position in its 256-byte bank period: the LDS has 64
//     banks (a 256-byte period), and the 16 lanes served together read 16
//     consecutive rows, which this spreads over all 64 banks; fragments are
//     ds_read_b128;
//   * B stays N-contiguous in LDS ([k][BN]) with the 16-byte chunk index
//     XOR-ed by 4*(k & 3) (conflict-free for the reads below); fragments are
//     read with ds_read_b64_tr_b16, which hands each lane 4 consecutive k of
//     one column (two reads give the 8 k an MFMA lane needs), so no transpose
//     pass is needed anywhere;
//   * a ring of S LDS stages with one barrier per K step; fragments of the
//     next K sub-step are read while the MFMAs of the current one run (two
//     fragment register sets), the refill loads go out after the barrier;
//   * operands are passed to the MFMA as (B, A), so each lane's accumulators
//     hold 4 consecutive output columns of one row;
//   * epilogue through LDS: GELU in float32, bf16 rounding, each wave stages
//     its piece row-major in the idle ring and writes whole row segments with
//     16 bytes per lane;
//   * persistent blocks (OCC per CU): every block derives the tile list from
//     offsets[] on the device (expert by expert; inside an expert, n-tile
//     major and m-tile minor, so the tiles sharing an expert's weight slab
//     run side by side). The list is cut into 8 contiguous ranges, one per
//     XCD (the hardware deals blocks to the XCDs round robin), so each XCD's
//     L2 serves the experts it works on. Empty groups own no tiles, and no
//     host synchronisation on the routing is needed;
//   * a small last round of long tiles is split over all of the XCD's blocks
//     by K steps (stream-K style): float32 partial sums go to a workspace and
//     gemm_fixup_kernel adds them in K order (deterministic) and stores. The
//     32-row weight-streaming tile of decode-sized batches may instead finish
//     them inside its own launch (INK): the last block to store a tile's
//     partial sums, found with a per-tile counter, adds them in the same
//     order, so the bits are the same either way.
// float32 path: a plain LDS-tiled FMA kernel (the fp32 workload is small).
#include <stdlib.h>
#include <string.h>

#include "common.h"
#include "gemm_lanes.h"
#include "internal.h"
#include "lds_dma.h"
#include "tiles.h"

namespace moe {

namespace {

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

// The partial-sum slots of leftover tile r of XCD x's tile range, in block
// (= K) order, as split_k cuts the rem * nk (tile, K step) units over the XCD's
// nb blocks; a block's slot for its leftover tile i is 2 * (block index) + i.
// Wave 0 only (lane jj checks block jj, nb <= 64). Returns the number of slots
// (written to s_slots), or -1 when one block ran the whole tile and stored it.
__device__ __forceinline__ int split_tile_slots(int r, int rem, int nb, int nk, int x, int* s_slots) {
  const int64_t W = (int64_t)rem * nk, u0 = (int64_t)r * nk, u1 = u0 + nk;
  const int jj = threadIdx.x;
  bool touch = false, whole = false;
  int slot = 0;
  if (jj < nb) {
    const int64_t s0 = W * jj / nb, s1 = W * (jj + 1) / nb;
    touch = s1 > s0 && s0 < u1 && s1 > u0;
    whole = touch && s0 <= u0 && s1 >= u1;
    slot = (jj * 8 + x) * 2 + (r - (int)(s0 / nk));
  }
  const uint64_t tm = __ballot(touch), wm = __ballot(whole);  // every lane of the wave votes
  if (touch) s_slots[__popcll(tm & ((1ull << jj) - 1ull))] = slot;
  return wm ? -1 : __popcll(tm);
}

// Completion of a split tile from its partial-sum slots: the float32x4
// entries ebase + u * STRIDE (u < PER) of the slot layout the GEMM kernel
// writes (thread-major per MFMA register group of its WM x WN waves) are
// summed over slots[0 .. ns) in that order (deterministic: the same bits
// whichever block completes the tile), then activation, bf16 rounding and
// stores of the rows before row_end and the columns inside [0, N). G slots'
// loads are in flight together.
template <int BM, int BN, int WM, int WN, int PER, int STRIDE, int G, bool GELU>
__device__ __forceinline__ void complete_split_entries(const float* __restrict__ partials, const int* slots, int ns,
                                                       int ebase, bf16_bits* __restrict__ C, int64_t row0,
                                                       int64_t row_end, int n0, int N) {
  constexpr int NW = WM * WN, WTM = BM / WM, WTN = BN / WN, TN = WTN / 32;
  f32x4 acc[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int si = 0; si < ns; si += G) {
    f32x4 v[G][PER];
#pragma unroll
    for (int q4 = 0; q4 < G; ++q4) {
      const int sl = si + q4 < ns ? slots[si + q4] : -1;
#pragma unroll
      for (int u = 0; u < PER; ++u)
        v[q4][u] = sl >= 0 ? ((const f32x4*)(partials + (int64_t)sl * (BM * BN)))[ebase + u * STRIDE]
                           : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int q4 = 0; q4 < G; ++q4)
#pragma unroll
      for (int u = 0; u < PER; ++u) acc[u] += v[q4][u];
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    // entry -> (MFMA register group, thread) -> (row, 4 columns) of the tile
    const int en = ebase + u * STRIDE, grp = en / (NW * kWave), tt = en % (NW * kWave);
    const int mi = grp / (TN * 4), ni = (grp / 4) % TN, gq = grp % 4;
    const int wave = tt / kWave, lane = tt % kWave;
    const int row = (wave / WN) * WTM + mi * 32 + (lane & 31);
    const int col = (wave % WN) * WTN + ni * 32 + 8 * gq + 4 * (lane >> 5);
    const int64_t grow = row0 + row;
    const int n = n0 + col;
    if (grow >= row_end || n < 0 || n >= N) continue;
    float v[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) v[qq] = GELU ? gelu_tanh(acc[u][qq]) : acc[u][qq];
    u32x2 o;
    o[0] = pack_bf16x2(v[0], v[1]);
    o[1] = pack_bf16x2(v[2], v[3]);
    *(u32x2*)(C + grow * N + n) = o;
  }
}

// Block tile BM x BN over K steps of BK, a ring of S LDS stages, OCC blocks per
// CU, WM x WN waves (each owns a (BM/WM) x (BN/WN) piece of the tile).
// GATHER: row r of A is row perm[r] of a [a_rows, K] matrix (the first expert
// GEMM reading the tokens straight from x, with no permuted copy).
// INK: split tiles are completed inside the launch: the last of a tile's
// blocks to store its partial sums (a counter per leftover tile in
// `counters`, zero at the start, reset by that block) adds the slots in K
// order and stores the tile, as gemm_fixup_kernel would; no block waits.
template <int BM, int BN, int BK, int S, int OCC, int WM, int WN, bool GELU, bool GATHER = false, bool INK = false>
__global__ __launch_bounds__(WM * WN * 64, OCC) void gemm_bf16_kernel(const bf16_bits* __restrict__ A,
                                                                      const int32_t* __restrict__ offsets,
                                                                      const bf16_bits* __restrict__ B,
                                                                      bf16_bits* __restrict__ C,
                                                                      float* __restrict__ partials, int64_t R, int K,
                                                                      int N, int E, int n_tiles, int min_steps,
                                                                      int max_rem,
                                                                      const int32_t* __restrict__ perm,
                                                                      int64_t a_rows, int gm,
                                                                      int32_t* __restrict__ counters) {
  constexpr int NW = WM * WN;                  // waves
  constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;  // 32x32 MFMA tiles per wave
  constexpr int KS = BK / 16;                  // MFMA K sub-steps per stage
  constexpr int A_ROW = BK * 2;                // bytes per A row of a stage
  constexpr int A_CH = BK / 8;                 // 16-byte chunks per A row
  constexpr int A_STAGE = BM * A_ROW;
  constexpr int B_ROW = BN * 2;                // bytes per k row of a B stage
  constexpr int B_SLOTS = BN / 8;              // 16-byte slots per k row
  constexpr int B_STAGE = BK * B_ROW;
  constexpr int STAGE = A_STAGE + B_STAGE;
  constexpr int A_LD = A_STAGE / 1024 / NW;    // 1 KB direct-to-LDS loads per wave per stage
  constexpr int B_LD = B_STAGE / 1024 / NW;
  constexpr int NL = A_LD + B_LD;
  // A: 16 consecutive rows are read together and span 16 * A_ROW bytes; the
  // chunk swizzle makes them cover the 64 banks (256 bytes) exactly once
  constexpr int A_RPP = 256 / A_ROW;           // rows per 256-byte bank period
  static_assert(A_LD >= 1 && B_LD >= 1 && KS >= 2 && S >= 2 && B_SLOTS >= 16, "unsupported tile");
  static_assert(A_LD * 1024 * NW == A_STAGE && B_LD * 1024 * NW == B_STAGE && TM >= 1 && TN >= 1, "unsupported tile");
  static_assert(A_RPP * A_CH == 16, "A swizzle assumes 16 chunks per bank period");
  // epilogue staging: per wave WTM rows of WTN bf16
  constexpr int EP_ROW = WTN * 2, EP_CH = WTN / 8, EP_WAVE = WTM * EP_ROW;
  constexpr int EP_ITERS = WTM * EP_ROW / (16 * kWave);
  static_assert(NW * EP_WAVE <= S * STAGE && EP_ITERS * 16 * kWave == WTM * EP_ROW, "epilogue staging");

  __shared__ __attribute__((aligned(1024))) char smem[S * STAGE];
  __shared__ int s_tstart[257];
  __shared__ int s_mtiles[256];
  __shared__ int s_slots[INK ? 64 : 1];  // INK: slots of the split tile being completed
  __shared__ int s_done;

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  build_tile_list<BM>(offsets, E, R, n_tiles, s_tstart, s_mtiles);
  const int total = s_tstart[E];

  // contiguous share of the tile list for this block's XCD
  const int xcd = blockIdx.x % 8, nb = gridDim.x / 8, j = blockIdx.x / 8;
  const int lo = (int)((int64_t)total * xcd / 8), hi = (int)((int64_t)total * (xcd + 1) / 8);
  const int nk = K / BK;
  // whole tiles for `full` rounds, then the K steps of the `rem` leftover tiles
  // split evenly over the XCD's blocks (stream-K)
  const SplitK sk = split_k(hi - lo, nb, j, nk, min_steps, max_rem);

  lds_char* const lds = (lds_char*)smem;
  const uint32_t lds_base = lds_addr(smem);
  const int wm0 = (wave / WN) * WTM, wn0 = (wave % WN) * WTN;

  // per-lane LDS read offsets (bytes, within a stage)
  int a_rd[TM];
#pragma unroll
  for (int mi = 0; mi < TM; ++mi) a_rd[mi] = (wm0 + mi * 32 + (lane & 31)) * A_ROW;
  int a_x[KS];
  {
    const int r = lane & 31;  // row within an MFMA tile; tiles start at multiples of 32
    const int sw = (r / A_RPP) & (A_CH - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a_x[ks] = ((ks * 2 + (lane >> 5)) ^ sw) << 4;
  }
  // B: lane q of its 16-lane group reads row (q >> 2) of a 4-row block, columns 4*(q & 3)..+3;
  // lanes 32..63 take the upper 8 k of each 16-k sub-step
  const int q = lane & 15, g = lane >> 4;
  int b_rd[TN];
#pragma unroll
  for (int ni = 0; ni < TN; ++ni) {
    const int col = wn0 + ni * 32 + (g & 1) * 16 + (q & 3) * 4;
    const int kr = q >> 2;  // == k & 3 for every k this lane reads
    b_rd[ni] = A_STAGE + ((g >> 1) * 8 + kr) * B_ROW + (((col >> 3) ^ (4 * kr)) << 4) + (col & 7) * 2;
  }

  // ---- per-item state: tile coordinates, buffer descriptors, K range, partial slot
  struct Tile {
    int e, n0;
    int64_t row0, row_end;
    i32x4 rsA, rsB;
    int kb, kn, slot;  // first K step, K steps, partial-sum slot (-1: the item completes the tile)
    int r;             // leftover tile index in the XCD's range (split items)
    uint32_t ga[GATHER ? A_LD : 1];  // GATHER: per-lane byte offsets of the A loads in A
  };
  auto locate = [&](int t) {
    // expert e with tstart[e] <= t < tstart[e+1] (upper bound - 1)
    int a0 = 0, a1 = E;
    while (a1 - a0 > 1) {
      const int mid = (a0 + a1) >> 1;
      if (s_tstart[mid] <= t) a0 = mid; else a1 = mid;
    }
    Tile tl;
    tl.e = __builtin_amdgcn_readfirstlane(a0);
    const int local = t - __builtin_amdgcn_readfirstlane(s_tstart[tl.e]);
    const int mt = __builtin_amdgcn_readfirstlane(s_mtiles[tl.e]);
    int n_tile, m_idx;
    tile_coords(local, mt, n_tiles, gm, n_tile, m_idx);
    tl.row0 = (int64_t)__builtin_amdgcn_readfirstlane(offsets[tl.e]) + (int64_t)m_idx * BM;
    tl.row_end = min((int64_t)__builtin_amdgcn_readfirstlane(offsets[tl.e + 1]), R);
    tl.n0 = lanes::tile_n0(n_tile, n_tiles, N, BN);
    // A: rows row0.. of the group; rows past the group's end fall outside the
    // descriptor's range and read as zero. B: the expert's [K, N] slab.
    if constexpr (GATHER)
      tl.rsA = buffer_rsrc(A, (uint32_t)(a_rows * K * 2));
    else
      tl.rsA = buffer_rsrc(A + tl.row0 * K, (uint32_t)(min(tl.row_end - tl.row0, (int64_t)BM) * K * 2));
    tl.rsB = buffer_rsrc(B + (int64_t)tl.e * K * N, (uint32_t)((int64_t)K * N * 2));
    tl.kb = 0;
    tl.kn = nk;
    tl.slot = -1;
    tl.r = -1;
    return tl;
  };
  auto make_item = [&](int i) {
    if (i < sk.full) return locate(lo + j + i * nb);
    const int r = sk.r_first + (i - sk.full);
    Tile tl = locate(lo + sk.full * nb + r);
    const int64_t a0 = max(sk.s0, (int64_t)r * nk), b0 = min(sk.s1, (int64_t)(r + 1) * nk);
    tl.kb = (int)(a0 - (int64_t)r * nk);
    tl.kn = (int)(b0 - a0);
    tl.slot = tl.kn == nk ? -1 : (int)blockIdx.x * 2 + (i - sk.full);
    tl.r = r;
    return tl;
  };
  // per-lane byte offsets of the direct-to-LDS loads (A part does not depend on the tile)
  uint32_t a_off[A_LD];
  int a_row[A_LD], a_c8[A_LD];  // row of the tile and first element of the lane's A piece
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const lanes::Piece pc = lanes::a_piece<BK>((wave * A_LD + i) * 64 + lane);  // LDS slot -> piece
    a_off[i] = lanes::a_lane_off(pc, K);
    a_row[i] = pc.row;
    a_c8[i] = pc.c * 8;
  }
  // GATHER: the token rows of a tile's A pieces (-1 past the group's end), and
  // the byte offsets made from them; padding rows point past the range (read
  // as zero, or as other rows of A: they are never stored)
  auto load_perm = [&](const Tile& t_, int (&pv)[A_LD]) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int64_t r = t_.row0 + a_row[i];
      pv[i] = r < t_.row_end ? perm[r] : -1;
    }
  };
  auto set_ga = [&](Tile& t_, const int (&pv)[A_LD]) {
    if constexpr (GATHER) {
#pragma unroll
      for (int i = 0; i < A_LD; ++i)
        t_.ga[i] = pv[i] >= 0 ? (uint32_t)(((int64_t)pv[i] * K + a_c8[i]) * 2) : lanes::kOutOfRange;
    }
  };
  uint32_t b_off0[B_LD];  // for n0 = 0
#pragma unroll
  for (int i = 0; i < B_LD; ++i) b_off0[i] = lanes::b_lane_off(lanes::b_piece<BN>((wave * B_LD + i) * 64 + lane), N);

  // load `i` (0 .. NL-1) of stage kt into ring buffer buf
  auto issue_one = [&](const Tile& tl, int kt, int buf, int i) {
    const uint32_t st = lds_base + buf * STAGE;
    if (i < A_LD)
      buffer_load_lds16(tl.rsA, GATHER ? tl.ga[i] : a_off[i], (uint32_t)kt * BK * 2, st + (wave * A_LD + i) * 1024);
    else
      buffer_load_lds16(tl.rsB, b_off0[i - A_LD] + (uint32_t)tl.n0 * 2u, (uint32_t)kt * BK * N * 2,
                        st + A_STAGE + (wave * B_LD + i - A_LD) * 1024);
  };

  bf16x8 fa[2][TM], fb[2][TN];
  constexpr int NR = TM + 2 * TN;  // LDS reads per fragment set
  // read `r` (0 .. NR-1) of the fragments of sub-step ks of ring buffer buf into set
  auto read_one = [&](int buf, int ks, int set, int r) {
    lds_char* const st = lds + buf * STAGE;
    if (r < TM) {
      fa[set][r] = *(lds_bf16x8*)(st + a_rd[r] + a_x[ks]);
    } else {
      const int ni = (r - TM) >> 1, hi = (r - TM) & 1;
      lds_char* const p0 = st + ks * 16 * B_ROW + b_rd[ni] + hi * 4 * B_ROW;
      const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
      s16x8 w = __builtin_bit_cast(s16x8, fb[set][ni]);
      if (hi) {
        w[4] = v[0]; w[5] = v[1]; w[6] = v[2]; w[7] = v[3];
      } else {
        w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
      }
      fb[set][ni] = __builtin_bit_cast(bf16x8, w);
    }
  };

  f32x16 acc[TM][TN];
  auto mfma_one = [&](int set, int idx) {
    const int mi = idx / TN, ni = idx % TN;
    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[set][ni], fa[set][mi], acc[mi][ni], 0, 0, 0);
  };

  constexpr int NM = TM * TN;  // MFMAs per sub-step
  constexpr int H = NM / 2;    // MFMAs of the last sub-step before the step's barrier
  // fragment reads issued after each MFMA: a set's reads all go out in the first
  // half of the sub-step, so they have landed when the next sub-step starts
  constexpr int RPM = (NR + NM / 2 - 1) / (NM / 2);

  Tile tl;
  if (sk.n_items > 0) {
    tl = make_item(0);
    if constexpr (GATHER) {
      int pv[A_LD];
      load_perm(tl, pv);
      set_ga(tl, pv);
    }
#pragma unroll
    for (int s2 = 0; s2 < (S >= 3 ? S - 1 : S); ++s2)
      if (s2 < tl.kn)
#pragma unroll
        for (int i = 0; i < NL; ++i) issue_one(tl, tl.kb + s2, s2, i);
  }

  // With three or more stages the refill of a buffer is spread over all the
  // MFMAs of a K step (a direct-to-LDS load stalls the issuing wave, and the
  // waves leave each barrier together: a burst of loads right after it idles
  // the matrix cores). Step kt then loads stage kt+S-1 into the buffer that
  // step kt-1 freed, and an item's prologue issues stages 0 .. S-2.
  constexpr bool SPREAD = S >= 3;
  constexpr int PRO = SPREAD ? S - 1 : S;  // stages issued by an item's prologue

  // With two stages, the next item's stage 0 is issued right after the K loop
  // into buffer 0 while the epilogue stages its output through buffer 1 in two
  // passes, then stage 1 follows. Every store of an epilogue is issued (range
  // checks drop the ones outside C), so `pend`, the vector-memory operations
  // issued after an item's stage 0, is known when the item starts.
  constexpr bool EARLY = S == 2 && NW * EP_WAVE / 2 <= STAGE && TM % 2 == 0;
  static_assert(!(INK && EARLY), "in-launch completion waits for all of the block's memory operations");
  constexpr int PART_ST = TM * TN * 4;  // float32 partial-sum stores per wave
  int pend = tl.kn > 1 ? NL : 0;
  auto wait_pend = [&](int n) {
    // at most `n` operations may remain in flight (vmcnt holds at most 63: waiting for
    // fewer is only stricter)
    if (n <= 0) wait_vmem<0>();
    else if (n == NL) wait_vmem<(NL < 63 ? NL : 63)>();
    else if (n == EP_ITERS) wait_vmem<(EP_ITERS < 63 ? EP_ITERS : 63)>();
    else if (n == EP_ITERS + NL) wait_vmem<(EP_ITERS + NL < 63 ? EP_ITERS + NL : 63)>();
    else if (n == PART_ST) wait_vmem<(PART_ST < 63 ? PART_ST : 63)>();
    else if (n == PART_ST + NL) wait_vmem<(PART_ST + NL < 63 ? PART_ST + NL : 63)>();
    else wait_vmem<0>();
  };

  for (int item = 0; item < sk.n_items; ++item) {
    const int kn = tl.kn;
    // ---- wait for stage 0 of this item (and everything issued before it)
    if constexpr (EARLY) {
      wait_pend(pend);
    } else {
      if (kn >= PRO)
        wait_vmem<NL * (PRO - 1)>();
      else
        wait_vmem<0>();
    }
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < TM; ++mi)
#pragma unroll
      for (int ni = 0; ni < TN; ++ni)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;

    // GATHER: the next item's token rows are loaded now; their values are first
    // used after this item's K loop, which ends with no load in flight
    Tile nxt = tl;
    int npv[A_LD];
    if constexpr (GATHER) {
      if (item + 1 < sk.n_items) {
        nxt = make_item(item + 1);
        load_perm(nxt, npv);
      }
    }
    // a wave whose whole slab of rows lies past the expert group's end (the
    // last, partly filled M tile of a group) skips its fragment reads and
    // MFMAs but still issues its share of the loads and joins the barriers;
    // the other wave on its SIMD then has the matrix core to itself
    auto kloop = [&](auto live_c) {
      constexpr bool LIVE = decltype(live_c)::value;
      auto mfma_x = [&](int set, int idx) {
        if constexpr (LIVE) mfma_one(set, idx);
      };
      auto read_x = [&](int b_, int ks_, int set_, int r_) {
        if constexpr (LIVE) read_one(b_, ks_, set_, r_);
      };
#pragma unroll
      for (int r = 0; r < NR; ++r) read_x(0, 0, 0, r);
      int buf = 0;
      if constexpr (SPREAD) {
        constexpr int STEP_M = KS * NM;            // MFMAs per K step
        constexpr int BAR_M = (KS - 1) * NM + H;   // MFMAs before the step's barrier
        // refill load d goes out after MFMA (d * STEP_M) / NL of the step; NB of them precede the barrier
        constexpr int NB = (BAR_M * NL + STEP_M - 1) / STEP_M;
        constexpr int LAST = (KS - 1) & 1;
        for (int kt = 0; kt < kn; ++kt) {
          const bool refill = kt + S - 1 < kn;
          const int rbuf = buf == 0 ? S - 1 : buf - 1;  // freed by step kt-1
          auto dma_after = [&](int m) {
#pragma unroll
            for (int d = 0; d < NL; ++d)
              if ((d * STEP_M) / NL == m && refill) issue_one(tl, tl.kb + kt + S - 1, rbuf, d);
          };
#pragma unroll
          for (int ks = 0; ks < KS - 1; ++ks) {
#pragma unroll
            for (int i = 0; i < NM; ++i) {
              mfma_x(ks & 1, i);
#pragma unroll
              for (int u = 0; u < RPM; ++u)
                if (i * RPM + u < NR) read_x(buf, ks + 1, (ks + 1) & 1, i * RPM + u);
              dma_after(ks * NM + i);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
#pragma unroll
          for (int i = 0; i < H; ++i) {
            mfma_x(LAST, i);
            dma_after((KS - 1) * NM + i);
            __builtin_amdgcn_sched_barrier(0);
          }
          const bool more = kt + 1 < kn;
          const int nbuf = buf + 1 == S ? 0 : buf + 1;
          if (more) {
            // stage kt+1 must have landed: still in flight may be stages kt+2 .. kt+S-2
            // and the NB loads of stage kt+S-1 issued so far
            if (refill)
              wait_vmem<NL * (S - 3) + NB>();
            else
              wait_vmem<0>();
            __syncthreads();  // stage kt+1 is visible; every wave is done reading `buf`
          }
          constexpr int PER = (NR + (NM - H) - 1) / (NM - H);  // next-stage fragment reads per MFMA
#pragma unroll
          for (int i = 0; i < NM - H; ++i) {
            mfma_x(LAST, H + i);
#pragma unroll
            for (int u = 0; u < PER; ++u)
              if (i * PER + u < NR && more) read_x(nbuf, 0, 0, i * PER + u);
            dma_after((KS - 1) * NM + H + i);
            __builtin_amdgcn_sched_barrier(0);
          }
          buf = nbuf;
        }
      } else {
      for (int kt = 0; kt < kn; ++kt) {
        // sub-steps 0 .. KS-2: MFMAs of the current fragments, one LDS read of the next set after each
#pragma unroll
        for (int ks = 0; ks < KS - 1; ++ks) {
#pragma unroll
          for (int i = 0; i < NM; ++i) {
            mfma_x(ks & 1, i);
#pragma unroll
            for (int u = 0; u < RPM; ++u)
              if (i * RPM + u < NR) read_x(buf, ks + 1, (ks + 1) & 1, i * RPM + u);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // last sub-step: H MFMAs, the step's barrier, then the rest of the MFMAs
        // with the refill of this buffer (stage kt+S) and the next stage's first
        // fragment reads spread between them
        constexpr int LAST = (KS - 1) & 1;
#pragma unroll
        for (int i = 0; i < H; ++i) {
          mfma_x(LAST, i);
          __builtin_amdgcn_sched_barrier(0);
        }
        const bool more = kt + 1 < kn;
        const int nbuf = buf + 1 == S ? 0 : buf + 1;
        if (more) {
          // stage kt+1 must have landed; stages kt+2 .. kt+S-1 may still be in flight
          if (kt + S - 1 < kn)
            wait_vmem<NL * (S - 2)>();
          else
            wait_vmem<0>();
          __syncthreads();  // every wave's stage kt+1 is in; every wave is done reading `buf`
        }
        const bool refill = kt + S < kn;
#pragma unroll
        for (int i = 0; i < NM - H; ++i) {
          mfma_x(LAST, H + i);
          constexpr int PER = (NL + NR + (NM - H) - 1) / (NM - H);  // memory ops per MFMA
#pragma unroll
          for (int u = 0; u < PER; ++u) {
            // the next stage's first fragments first (needed soonest), then the refill loads
            const int op = i * PER + u;
            if (op < NR) {
              if (more) read_x(nbuf, 0, 0, op);
            } else if (op < NR + NL) {
              if (refill) issue_one(tl, tl.kb + kt + S, buf, op - NR);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        buf = nbuf;
      }
      }
    };
    if (tl.row_end - tl.row0 > wm0)
      kloop(BoolC<true>{});
    else
      kloop(BoolC<false>{});
    __syncthreads();  // every wave is done with every buffer

    const bool has_next = item + 1 < sk.n_items;
    Tile nx = tl;
    if constexpr (EARLY) {
      if (has_next) {
        if constexpr (GATHER) {
          nx = nxt;
          set_ga(nx, npv);
        } else {
          nx = make_item(item + 1);
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) issue_one(nx, nx.kb, 0, i);
      }
    }

    if (tl.slot >= 0) {
      // ---- part of a split tile: float32 partial sums in the accumulator
      // layout (thread-major per MFMA register group, 16 bytes per lane)
      float* const dst = partials + (int64_t)tl.slot * (BM * BN);
#pragma unroll
      for (int mi = 0; mi < TM; ++mi)
#pragma unroll
        for (int ni = 0; ni < TN; ++ni)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            f32x4 v;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) v[qq] = acc[mi][ni][4 * gq + qq];
            *(f32x4*)(dst + ((int64_t)((mi * TN + ni) * 4 + gq) * (NW * kWave) + tid) * 4) = v;
          }
      if constexpr (INK) {
        // the block's partial sums are made visible to the device before it
        // counts itself in (every wave's stores acknowledged, then one release
        // by wave 0); the block that brings the count to the number of
        // contributing blocks completes the tile and resets the count
        wait_vmem<0>();
        __syncthreads();
        if (wave == 0) {
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
          const int ns = split_tile_slots(tl.r, sk.rem, nb, nk, xcd, s_slots);
          if (lane == 0) {
            int32_t* const ctr = counters + xcd * kSplitCountersPerXcd + tl.r;
            const int old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const bool last = old == ns - 1;
            if (last) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_done = last ? ns : 0;
          }
        }
        __syncthreads();
        const int ns = s_done;
        if (ns > 0) {
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // the other blocks' partial sums
          constexpr int NT = NW * kWave, PER = BM * BN / 4 / NT;
          static_assert(PER * NT * 4 == BM * BN, "completion split");
          complete_split_entries<BM, BN, WM, WN, PER, NT, 8, GELU>(partials, s_slots, ns, tid, C, tl.row0,
                                                                  tl.row_end, tl.n0, N);
        }
      }
    } else {
      // ---- epilogue through LDS: each wave stages its WTM x WTN piece as bf16
      // in its own LDS region (row-major, 16-byte chunks XOR-swizzled by the
      // row), then writes whole row segments to C with 16 bytes per lane. With
      // EARLY the region lies in buffer 1 and the piece goes in two passes of
      // WTM / 2 rows. Stores go through a buffer descriptor whose range ends at
      // the group's last row; columns past N are sent out of range.
      constexpr int PASSES = EARLY ? 2 : 1;
      constexpr int PM = TM / PASSES;                        // MFMA row groups per pass
      constexpr int P_ITERS = EP_ITERS / PASSES;             // 16-byte stores per lane per pass
      lds_char* const ep = lds + (EARLY ? STAGE + wave * (EP_WAVE / 2) : wave * EP_WAVE);
      const __amdgpu_buffer_rsrc_t rsC = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(C + tl.row0 * N), (short)0, (int)(min(tl.row_end - tl.row0, (int64_t)BM) * N * 2), kBufferFlags);
#pragma unroll
      for (int pass = 0; pass < PASSES; ++pass) {
#pragma unroll
        for (int m2 = 0; m2 < PM; ++m2)
#pragma unroll
          for (int ni = 0; ni < TN; ++ni)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const int mi = pass * PM + m2;
              // lane holds row (lane & 31) of MFMA tile (mi, ni), columns 8 gq + 4 (lane >> 5) + 0..3
              float v[4];
#pragma unroll
              for (int qq = 0; qq < 4; ++qq) {
                v[qq] = acc[mi][ni][4 * gq + qq];
                if (GELU) v[qq] = gelu_tanh(v[qq]);
              }
              u32x2 o;
              o[0] = pack_bf16x2(v[0], v[1]);
              o[1] = pack_bf16x2(v[2], v[3]);
              const int row = m2 * 32 + (lane & 31), ch = ni * 4 + gq;
              *(__attribute__((address_space(3))) u32x2*)(ep + row * EP_ROW + ((ch ^ (row & (EP_CH - 1))) << 4) +
                                                            (lane >> 5) * 8) = o;
              __builtin_amdgcn_sched_barrier(0);  // bounds the live values of the GELU pass
            }
        // LDS operations of one wave complete in order: no barrier between the
        // wave's own writes and reads (nor before the next pass overwrites them)
        constexpr int EP_G = P_ITERS < 4 ? P_ITERS : 4;  // reads in flight per group
#pragma unroll
        for (int it0 = 0; it0 < P_ITERS; it0 += EP_G) {
          u32x4 v[EP_G];
#pragma unroll
          for (int u = 0; u < EP_G; ++u) {
            const int idx = (it0 + u) * kWave + lane, row = idx / EP_CH, ch = idx % EP_CH;
            v[u] = *(__attribute__((address_space(3))) u32x4*)(ep + row * EP_ROW + ((ch ^ (row & (EP_CH - 1))) << 4));
          }
#pragma unroll
          for (int u = 0; u < EP_G; ++u) {
            const int idx = (it0 + u) * kWave + lane, row = idx / EP_CH, ch = idx % EP_CH;
            const int n = tl.n0 + wn0 + ch * 8;
            const int off = lanes::c_store_off(wm0 + pass * (WTM / PASSES) + row, n, N);
            __builtin_amdgcn_raw_buffer_store_b128(v[u], rsC, off, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }

    // ---- the next item's first stages (the ring is free once every wave has read its piece)
    if (has_next) {
      __syncthreads();
      if constexpr (EARLY) {
        if (nx.kn > 1)
#pragma unroll
          for (int i = 0; i < NL; ++i) issue_one(nx, nx.kb + 1, 1, i);
        pend = (tl.slot >= 0 ? PART_ST : EP_ITERS) + (nx.kn > 1 ? NL : 0);
        tl = nx;
      } else {
        if constexpr (GATHER) {
          tl = nxt;
          set_ga(tl, npv);
        } else {
          tl = make_item(item + 1);
        }
#pragma unroll
        for (int s2 = 0; s2 < PRO; ++s2)
          if (s2 < tl.kn)
#pragma unroll
            for (int i = 0; i < NL; ++i) issue_one(tl, tl.kb + s2, s2, i);
      }
    }
  }
}

// Completion of the tiles that the stream-K phase split: block (b, x, r) takes
// part b of SUB of leftover tile r of XCD x's tile range, sums the partial
// slots of the blocks that worked on it in K order (deterministic), applies
// the activation, rounds to bf16 and stores. Slots and the split follow the
// GEMM kernel's own arithmetic (split_k, block index j * 8 + x).
template <int BM, int BN, int WM, int WN, int SUB, bool GELU>
__global__ __launch_bounds__(256) void gemm_fixup_kernel(const int32_t* __restrict__ offsets,
                                                         const float* __restrict__ partials,
                                                         bf16_bits* __restrict__ C, int64_t R, int nk, int N,
                                                         int E, int n_tiles, int nb, int min_steps,
                                                         int max_rem, int gm) {
  constexpr int ENT = BM * BN / 4;           // float32x4 entries per slot
  constexpr int PER = ENT / SUB / 256;       // entries per thread
  static_assert(PER * SUB * 256 == ENT, "fixup split");
  constexpr int kMaxSlots = 64;  // >= blocks per XCD of any launch (kMaxCUs / 8 * 2), one lane each
  __shared__ int s_tstart[257];
  __shared__ int s_mtiles[256];
  __shared__ int s_slots[kMaxSlots];
  __shared__ int s_nslots;

  // block (b, x, r0) takes part b of leftover tiles r0, r0 + rstep, ... of XCD x
  const int b = blockIdx.x % SUB, x = (blockIdx.x / SUB) % 8, r0 = blockIdx.x / SUB / 8;
  const int rstep = gridDim.x / (SUB * 8);
  build_tile_list<BM>(offsets, E, R, n_tiles, s_tstart, s_mtiles);
  const int total = s_tstart[E];
  const int lo = (int)((int64_t)total * x / 8), hi = (int)((int64_t)total * (x + 1) / 8);
  const int full = (hi - lo) / nb, rem = (hi - lo) - full * nb;
  if (!split_leftover(rem, nb, nk, min_steps, max_rem)) return;
  for (int r = r0; r < rem; r += rstep) {
    // the slots of the blocks that touch tile r, in block (= K) order (nb <= kMaxSlots = 64 lanes)
    if (threadIdx.x < kWave) {
      const int ns = split_tile_slots(r, rem, nb, nk, x, s_slots);
      if (threadIdx.x == 0) s_nslots = ns;
    }
    __syncthreads();
    const int ns = s_nslots;
    if (ns <= 0) {
      __syncthreads();  // s_slots is rewritten for the next tile
      continue;
    }

    // the tile: same enumeration as the GEMM kernel
    const int t = lo + full * nb + r;
    int a0 = 0, a1 = E;
    while (a1 - a0 > 1) {
      const int mid = (a0 + a1) >> 1;
      if (s_tstart[mid] <= t) a0 = mid; else a1 = mid;
    }
    const int e = a0, local = t - s_tstart[e], mt = s_mtiles[e];
    int n_tile, m_idx;
    tile_coords(local, mt, n_tiles, gm, n_tile, m_idx);
    const int64_t row0 = (int64_t)offsets[e] + (int64_t)m_idx * BM;
    const int64_t row_end = min((int64_t)offsets[e + 1], R);
    const int n0 = lanes::tile_n0(n_tile, n_tiles, N, BN);

    complete_split_entries<BM, BN, WM, WN, PER, 256, 8, GELU>(partials, s_slots, ns, b * (ENT / SUB) + threadIdx.x, C,
                                                             row0, row_end, n0, N);
    __syncthreads();  // s_slots is rewritten for the next tile
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

// persistent grids are sized for at most this many CUs (MI355X has 256); with two
// blocks per CU an XCD holds at most 64 blocks, which bounds the blocks that
// can share one split tile (gemm_fixup_kernel's slot list)
constexpr int kMaxCUs = 256;

}  // namespace

int device_cus() {
  // initialised once, thread-safely (a function-local static); callers on
  // several threads never see a partial or unclamped value
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    return min(max(n, 8), kMaxCUs);
  }();
  return cus;
}

namespace {

// Tile configurations of the bf16 path: block tile, K step, LDS ring stages,
// blocks per CU. LDS per block = stages * (BM + BN) * BK * 2 bytes.
struct TileShape {
  const char* name;
  int bm, bn, bk, stages, occ;
  bool fill;  // decode-sized batches: a block per CU slot, any partial round split
};
constexpr TileShape kShapes[] = {
    {"256x256", 256, 256, 64, 2, 1},     // 128 KB
    {"256x256k32", 256, 256, 32, 4, 1},  // 128 KB
    {"256x128", 256, 128, 32, 3, 2},     // 72 KB
    {"128x128", 128, 128, 64, 2, 2},     // 64 KB
    {"128x128k32", 128, 128, 32, 4, 2},  // 64 KB
    {"256x256w8", 256, 256, 64, 2, 1},   // 128 KB, 8 waves
    {"256x256w8k32", 256, 256, 32, 4, 1},  // 128 KB, 8 waves
    {"32x256", 32, 256, 64, 4, 1, true},  // 144 KB, 4 waves of 32 x 64: weight streaming
};
constexpr int kNumShapes = sizeof(kShapes) / sizeof(kShapes[0]);
constexpr int kDecodeTile = 7;

// persistent grid: OCC blocks per CU, a multiple of 8 so every XCD holds the
// same number of blocks; with `fill` every slot, so that split tiles spread
// over the whole GPU. MOE_GEMM_MAX_BLOCKS=<n> lowers the cap (several rounds
// of tiles on small problems: exercises the leftover-tile split).
int64_t persistent_grid(int64_t tiles_ub, int occ, bool fill = false) {
  int64_t slots = (int64_t)device_cus() / 8 * 8 * occ;
  const char* cap = getenv("MOE_GEMM_MAX_BLOCKS");
  if (cap && cap[0]) slots = min(slots, max((int64_t)8, (int64_t)atoi(cap) / 8 * 8));
  return max((int64_t)8, fill ? slots : min(ceil_div(tiles_ub, 8) * 8, slots));
}

int64_t tiles_upper_bound(int64_t R, int N, int E, int bm, int bn) {
  const int64_t m_tiles = (R + (int64_t)E * (bm - 1)) / bm;  // >= sum over experts of ceil(rows_e / bm)
  return m_tiles * ceil_div(N, bn);
}

// fixup blocks per split tile: 16, or fewer when a tile has fewer than 16 x 256 float32x4 entries
template <int BM, int BN>
constexpr int fixup_sub() {
  return BM * BN / 4 / 256 >= 16 ? 16 : BM * BN / 4 / 256;
}
// split tiles one fixup block may take in turn: a grid for a quarter of the
// most leftover tiles per XCD (MOE_FIXUP_ROUNDS=<n> overrides). Measured on
// MI355X against one tile per block: the FFN phase equal within noise on
// four workloads, ~1 % shorter at 8192 tokens x 64 experts
constexpr int kFixupRounds = 4;
int fixup_rounds() {
  const char* fr = getenv("MOE_FIXUP_ROUNDS");
  return fr && fr[0] ? max(1, atoi(fr)) : kFixupRounds;
}

bool env_flag(const char* name) {
  const char* f = getenv(name);
  return f && f[0] && atoi(f) != 0;
}

// Whether a launch of the 32-row weight-streaming tile (a block per CU slot)
// completes its split tiles itself (counters, no fixup launch) rather than in
// a fixup launch. Each block that stores partial sums then writes back its
// XCD's L2 before counting itself in, and one block sums the tile. Measured on
// MI355X at 1..128 tokens of the four bf16 workloads: for the first GEMM this
// is 1.5-3 us faster per layer once the batch holds at least E/2 rows (the
// tile list then mostly fills whole rounds, and the fixup launch it saves has
// little or nothing to do), ~5 us slower below that (tiles split over four or
// more blocks); for the second GEMM (tiles split over 4-16 blocks) it is slower
// at every size. MOE_GEMM_SPLIT_FIXUP=1 forces the fixup launch,
// MOE_GEMM_SPLIT_INLAUNCH=1 the in-launch completion for both GEMMs.
bool split_in_launch(int64_t R, int E, bool gelu) {
  if (env_flag("MOE_GEMM_SPLIT_FIXUP")) return false;
  if (env_flag("MOE_GEMM_SPLIT_INLAUNCH")) return true;
  return gelu && 2 * R >= E;
}

template <int BM, int BN, int BK, int S, int OCC, int WM, int WN, bool GELU, bool GATHER, bool INK>
void launch_kernel(unsigned grid, hipStream_t s, const void* A, const int32_t* offsets, const void* B, void* C,
                   float* partials, int64_t R, int K, int N, int E, int n_tiles, int min_steps, int max_rem,
                   const int32_t* perm, int64_t a_rows, int gm, int32_t* counters) {
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BK, S, OCC, WM, WN, GELU, GATHER, INK>), dim3(grid),
                     dim3(WM * WN * 64), 0, s, (const bf16_bits*)A, offsets, (const bf16_bits*)B, (bf16_bits*)C,
                     partials, R, K, N, E, n_tiles, min_steps, max_rem, perm, a_rows, gm, counters);
}

template <int BM, int BN, int BK, int S, int OCC, int WM = 2, int WN = 2, bool FILL = false>
hipError_t launch_bf16(const GemmGeom& geo, const void* A, const int32_t* offsets, const void* B, void* C,
                       float* partials, int32_t* counters, int64_t R, int K, int N, int E, bool gelu,
                       const int32_t* perm, int64_t a_rows, hipStream_t s) {
  if (geo.bm != BM || geo.bn != BN || geo.bk != BK || tiles_upper_bound(R, N, E, BM, BN) > INT32_MAX || K % BK != 0)
    return hipErrorInvalidValue;
  const int n_tiles = geo.n_tiles, nb = geo.nb, nk = geo.nk, min_steps = geo.min_steps, max_rem = geo.max_rem;
  const int64_t grid = geo.grid;
  const int gm = group_m();
  const bool ink = FILL && geo.in_launch;
  if (ink && (!counters || max_rem > kSplitCountersPerXcd)) return hipErrorInvalidValue;
  // fixup blocks: FS per split tile, each looping over up to kFixupRounds tiles
  constexpr int FS = fixup_sub<BM, BN>();
  const int fix_r = (max_rem + fixup_rounds() - 1) / fixup_rounds();
  const unsigned fix_grid = !ink && nk >= min_steps && max_rem > 0 ? (unsigned)(8 * fix_r * FS) : 0u;
  const unsigned g = (unsigned)grid;
#define MOE_LAUNCH(GELU_, GATHER_)                                                                              \
  do {                                                                                                           \
    if (ink)                                                                                                     \
      launch_kernel<BM, BN, BK, S, OCC, WM, WN, GELU_, GATHER_, FILL>(g, s, A, offsets, B, C, partials, R, K, N, \
                                                                      E, n_tiles, min_steps, max_rem, perm,      \
                                                                      a_rows, gm, counters);                     \
    else                                                                                                         \
      launch_kernel<BM, BN, BK, S, OCC, WM, WN, GELU_, GATHER_, false>(g, s, A, offsets, B, C, partials, R, K,   \
                                                                       N, E, n_tiles, min_steps, max_rem, perm,  \
                                                                       a_rows, gm, nullptr);                     \
    if (fix_grid)                                                                                                \
      hipLaunchKernelGGL((gemm_fixup_kernel<BM, BN, WM, WN, FS, GELU_>), dim3(fix_grid), dim3(256), 0, s,        \
                         offsets, (const float*)partials, (bf16_bits*)C, R, nk, N, E, n_tiles, nb, min_steps,    \
                         max_rem, gm);                                                                           \
  } while (0)
  if (perm) {
    if (gelu) MOE_LAUNCH(true, true);
    else MOE_LAUNCH(false, true);  // the first GEMM without its activation (training keeps U = x W1)
  } else {
    if (gelu) MOE_LAUNCH(true, false);
    else MOE_LAUNCH(false, false);
  }
#undef MOE_LAUNCH
  return hipGetLastError();
}

}  // namespace

// The fixup of split tiles for launches that share the 8-wave 256 x 256 tile's
// partial-sum layout and tile enumeration (the backward kernel's row-grouped
// launches); no activation.
hipError_t launch_split_fixup_256(const int32_t* offsets, const float* partials, uint16_t* C, int64_t R, int nk, int N,
                                  int E, int nb, int min_steps, int max_rem, hipStream_t s) {
  const int fix_r = (max_rem + fixup_rounds() - 1) / fixup_rounds();
  if (nk < min_steps || max_rem <= 0) return hipSuccess;
  constexpr int FS = fixup_sub<256, 256>();
  hipLaunchKernelGGL((gemm_fixup_kernel<256, 256, 2, 4, FS, false>), dim3((unsigned)(8 * fix_r * FS)),
                     dim3(256), 0, s, offsets, partials, (bf16_bits*)C, R, nk, N, E, (int)ceil_div(N, 256), nb,
                     min_steps, max_rem, group_m());
  return hipGetLastError();
}

int group_m() {
  const char* g = getenv("MOE_GEMM_GROUP_M");
  return g && g[0] ? max(0, atoi(g)) : kGroupM;
}

int split_min_steps() {
  int min_steps = kSplitMinSteps;
  const char* ms = getenv("MOE_GEMM_SPLIT_MIN_STEPS");
  if (ms && ms[0]) min_steps = max(0, atoi(ms));
  return min_steps;
}

namespace {

// Block tile for a GEMM: fewer, larger tiles use the matrix cores better, but
// padding rows of half-empty M tiles and a last partial round of tiles over
// the block slots cost time (unless that round is split over the blocks, see
// split_leftover). tile_eff: measured matrix-core efficiency of a busy CU,
// relative to the 8-wave 256 x 256 tile; 0 = only on request.
// MOE_GEMM_TILE=<name of a kShapes entry> forces a shape.
int pick_tile(int64_t R, int K, int N, int E) {
  const char* force = getenv("MOE_GEMM_TILE");
  if (force && force[0])
    for (int c = 0; c < kNumShapes; ++c)
      if (!strcmp(force, kShapes[c].name)) return c;
  // decode-sized batches (at most ~40 rows per expert on average): the weight
  // slabs dominate; 32-row tiles stream them from every CU
  if (R <= 40 * (int64_t)E && K % 64 == 0) return kDecodeTile;
  const double tile_eff[kNumShapes] = {0.0, 0.0, 0.8, 0.75, 0.0, 1.0, 0.0, 0.0};
  const double cus = device_cus();
  int best = 5;
  double best_score = -1.0;
  for (int c = 0; c < kNumShapes; ++c) {
    const TileShape& ts = kShapes[c];
    if (tile_eff[c] <= 0.0 || K % ts.bk != 0) continue;
    const double m_tiles = (double)R / ts.bm + 0.5 * E;
    const double tiles = m_tiles * ceil_div(N, ts.bn);
    const double rounds = tiles / (cus * ts.occ);
    const double whole = (double)(int64_t)rounds, frac = rounds - whole;
    const int nk = K / ts.bk;
    double round_eff;
    if (rounds < 1.0)
      round_eff = rounds;
    else if (frac * 3.0 <= 1.0 && nk * (1.0 - frac) >= kSplitMinSteps)
      round_eff = rounds / (rounds + 0.1);  // leftover split over the blocks
    else
      round_eff = rounds / (frac > 0.0 ? whole + 1.0 : whole);
    const double pad_eff = (double)R / (m_tiles * ts.bm);
    const double score = tile_eff[c] * round_eff * pad_eff;
    if (score > best_score) {
      best_score = score;
      best = c;
    }
  }
  return best;
}

}  // namespace

GemmGeom gemm_geom(int64_t R, int K, int N, int E, bool gelu) {
  GemmGeom g;
  g.shape = pick_tile(R, K, N, E);
  const TileShape& ts = kShapes[g.shape];
  g.bm = ts.bm;
  g.bn = ts.bn;
  g.bk = ts.bk;
  g.n_tiles = (int)ceil_div(N, ts.bn);
  g.grid = (int)persistent_grid(tiles_upper_bound(R, N, E, ts.bm, ts.bn), ts.occ, ts.fill);
  g.nb = g.grid / 8;
  g.nk = K / ts.bk;
  // MOE_GEMM_SPLIT_MIN_STEPS=<n> overrides the split threshold (0: split every small leftover)
  g.min_steps = split_min_steps();
  // split leftover tiles number at most max_rem per XCD, and none when K is short (split_leftover)
  g.max_rem = ts.fill ? g.nb - 1 : g.nb / 3;
  g.in_launch = ts.fill && split_in_launch(R, E, gelu);
  return g;
}

void gemm_xcd_plan(const GemmGeom& g, const int32_t* counts, int E, GemmXcdPlan* out) {
  int64_t total = 0;
  for (int e = 0; e < E; ++e) total += counts[e] > 0 ? ceil_div((int64_t)counts[e], g.bm) * g.n_tiles : 0;
  out->tiles = total;
  out->full = out->rem = out->split = out->split_xcds = 0;
  int64_t most = -1;
  for (int x = 0; x < 8; ++x) {
    // the same ranges and split rule as the kernels (contiguous eighths of the tile list)
    const int64_t t = total * (x + 1) / 8 - total * x / 8;
    const int full = (int)(t / g.nb), rem = (int)(t - (int64_t)full * g.nb);
    const bool split = split_leftover(rem, g.nb, g.nk, g.min_steps, g.max_rem);
    out->split_xcds += split ? 1 : 0;
    if (t > most) {
      most = t;
      out->full = full;
      out->rem = rem;
      out->split = split ? 1 : 0;
    }
  }
}

size_t grouped_gemm_partials_bytes(int dtype, int64_t R, int K, int N, int E) {
  if (dtype != MOE_DTYPE_BF16) return 0;
  const TileShape& ts = kShapes[pick_tile(R, K, N, E)];
  const int64_t grid = persistent_grid(tiles_upper_bound(R, N, E, ts.bm, ts.bn), ts.occ, ts.fill);
  return (size_t)grid * 2 * ts.bm * ts.bn * sizeof(float);  // two split segments per block at most
}

bool grouped_gemm_uses_counters(int dtype, int64_t R, int K, int N, int E, bool gelu) {
  return dtype == MOE_DTYPE_BF16 && kShapes[pick_tile(R, K, N, E)].fill && split_in_launch(R, E, gelu);
}

hipError_t launch_grouped_gemm(int dtype, const void* A, const int32_t* offsets, const void* B, void* C,
                               float* partials, int32_t* counters, int64_t R, int K, int N, int E, bool gelu,
                               hipStream_t s, const int32_t* perm, int64_t a_rows) {
  if (perm && (dtype != MOE_DTYPE_BF16 || a_rows * K * 2 >= (int64_t)INT32_MAX))
    return hipErrorInvalidValue;  // row gathering: bf16, A addressable with 31-bit offsets
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
  const GemmGeom geo = gemm_geom(R, K, N, E, gelu);
  switch (geo.shape) {
    case 0:
      return launch_bf16<256, 256, 64, 2, 1>(geo, A, offsets, B, C, partials, counters, R, K, N, E, gelu, perm,
                                             a_rows, s);
    case 1:
      return launch_bf16<256, 256, 32, 4, 1>(geo, A, offsets, B, C, partials, counters, R, K, N, E, gelu, perm,
                                             a_rows, s);
    case 2:
      return launch_bf16<256, 128, 32, 3, 2>(geo, A, offsets, B, C, partials, counters, R, K, N, E, gelu, perm,
                                             a_rows, s);
    case 3:
      return launch_bf16<128, 128, 64, 2, 2>(geo, A, offsets, B, C, partials, counters, R, K, N, E, gelu, perm,
                                             a_rows, s);
    case 4:
      return launch_bf16<128, 128, 32, 4, 2>(geo, A, offsets, B, C, partials, counters, R, K, N, E, gelu, perm,
                                             a_rows, s);
    case 5:
      return launch_bf16<256, 256, 64, 2, 1, 2, 4>(geo, A, offsets, B, C, partials, counters, R, K, N, E, gelu, perm,
                                                   a_rows, s);
    case kDecodeTile:
      return launch_bf16<32, 256, 64, 4, 1, 1, 4, true>(geo, A, offsets, B, C, partials, counters, R, K, N, E, gelu,
                                                        perm, a_rows, s);
    default:
      return launch_bf16<256, 256, 32, 4, 1, 2, 4>(geo, A, offsets, B, C, partials, counters, R, K, N, E, gelu, perm,
                                                   a_rows, s);
  }
}

}  // namespace moe
