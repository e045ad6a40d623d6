// Host replay of the grouped GEMM's operand loads and output stores.
//
// For one block-tile shape (BM x BN, K step BK, NW waves) and one problem
// shape (K, N, rows of an expert group), this walks every direct-to-LDS load
// of every tile and K step and every 16-byte output store, computing each
// lane's offsets with the kernel's own lane arithmetic (gemm_lanes.h), and
// checks them against a buffer descriptor's range under both ways a
// hardware range check may treat the scalar offset:
//   V: only the vector offset is compared with the range; the access goes to
//      vector + scalar offset;
//   S: the 32-bit sum of both offsets is compared and used.
// Every access that is not sent out of range must lie inside the operand's
// bytes, and every element the tile needs must be read from (or stored to)
// exactly its own address.
//
// Usage: gemm_lanes_check BM BN BK NW K N ROWS A_ROWS
//   ROWS: rows of the expert group (several m-tiles when > BM)
//   A_ROWS: rows of the gathered operand for the row-gathering form (0: skip)
// Prints "ok <loads checked>" and exits 0, or prints the first violation and exits 1.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <initializer_list>

#include "gemm_lanes.h"

using namespace moe::lanes;

static long checked = 0;

static int fail(const char* what, long a, long b, long c) {
  printf("FAIL %s (%ld, %ld, %ld)\n", what, a, b, c);
  exit(1);
}

// One load of 16 bytes with vector offset v and scalar offset s against a
// range of `num` bytes. `want` >= 0: the byte offset the lane must read.
static void check_load(const char* what, uint32_t v, uint32_t s, uint64_t num, int64_t want) {
  ++checked;
  // semantics V
  if ((uint64_t)v < num) {
    const uint64_t at = (uint64_t)v + s;
    if (at + 16 > num) fail(what, (long)v, (long)s, (long)num);
    if (want >= 0 && (int64_t)at != want) fail(what, (long)at, want, 1);
  } else if (want >= 0) {
    fail(what, (long)v, want, 2);  // a needed element read as zero
  }
  // semantics S
  const uint32_t sum = v + s;
  if ((uint64_t)sum < num) {
    if ((uint64_t)sum + 16 > num) fail(what, (long)sum, (long)num, 3);
    if (want >= 0 && (int64_t)sum != want) fail(what, (long)sum, want, 4);
  } else if (want >= 0) {
    fail(what, (long)sum, want, 5);
  }
}

template <int BM, int BN, int BK, int NW>
static void run(int K, int N, int rows, int a_rows) {
  constexpr int A_LD = BM * BK * 2 / 1024 / NW, B_LD = BK * BN * 2 / 1024 / NW;
  static_assert(A_LD * 1024 * NW == BM * BK * 2 && B_LD * 1024 * NW == BK * BN * 2, "tile");
  const int nk = K / BK, n_tiles = (N + BN - 1) / BN, m_tiles = (rows + BM - 1) / BM;
  // B: every n-tile, K step and lane of the expert's [K, N] slab
  const uint64_t b_num = (uint64_t)K * N * 2;
  for (int nt = 0; nt < n_tiles; ++nt) {
    const int n0 = tile_n0(nt, n_tiles, N, BN);
    if (n0 + BN != N - (n_tiles - 1 - nt) * BN) fail("tile_n0", nt, n0, N);
    for (int kt = 0; kt < nk; ++kt)
      for (int w = 0; w < NW; ++w)
        for (int i = 0; i < B_LD; ++i)
          for (int lane = 0; lane < 64; ++lane) {
            const Piece pc = b_piece<BN>((w * B_LD + i) * 64 + lane);
            const uint32_t v = b_lane_off(pc, N) + (uint32_t)n0 * 2u;
            const uint32_t s = (uint32_t)kt * BK * N * 2;
            const int col = n0 + pc.c * 8, k = kt * BK + pc.row;
            const int64_t want = col >= 0 && col < N ? ((int64_t)k * N + col) * 2 : -1;
            check_load("B", v, s, b_num, want);
          }
  }
  // the B pieces of a stage cover its BK x BN slots exactly once
  {
    static char seen[BK][BN / 8];
    for (int k = 0; k < BK; ++k)
      for (int c = 0; c < BN / 8; ++c) seen[k][c] = 0;
    for (int p = 0; p < BK * BN / 8; ++p) {
      const Piece pc = b_piece<BN>(p);
      if (pc.row < 0 || pc.row >= BK || pc.c < 0 || pc.c >= BN / 8 || seen[pc.row][pc.c]++) fail("B cover", p, 0, 0);
    }
    static char seen_a[BM][BK / 8];
    for (int r = 0; r < BM; ++r)
      for (int c = 0; c < BK / 8; ++c) seen_a[r][c] = 0;
    for (int p = 0; p < BM * BK / 8; ++p) {
      const Piece pc = a_piece<BK>(p);
      if (pc.row < 0 || pc.row >= BM || pc.c < 0 || pc.c >= BK / 8 || seen_a[pc.row][pc.c]++) fail("A cover", p, 0, 0);
    }
  }
  // A: each m-tile's descriptor starts at its first row and spans at most BM rows of the group
  for (int m = 0; m < m_tiles; ++m) {
    const int live = rows - m * BM < BM ? rows - m * BM : BM;
    const uint64_t a_num = (uint64_t)live * K * 2;
    for (int kt = 0; kt < nk; ++kt)
      for (int w = 0; w < NW; ++w)
        for (int i = 0; i < A_LD; ++i)
          for (int lane = 0; lane < 64; ++lane) {
            const Piece pc = a_piece<BK>((w * A_LD + i) * 64 + lane);
            const int64_t want = pc.row < live ? ((int64_t)pc.row * K + kt * BK + pc.c * 8) * 2 : -1;
            check_load("A", a_lane_off(pc, K), (uint32_t)kt * BK * 2, a_num, want);
          }
    // output stores of the tile: rows past the group and columns outside [0, N) are dropped
    const uint64_t c_num = (uint64_t)live * N * 2;
    for (int nt = 0; nt < n_tiles; ++nt) {
      const int n0 = tile_n0(nt, n_tiles, N, BN);
      for (int r = 0; r < BM; ++r)
        for (int c = 0; c < BN / 8; ++c) {
          const int n = n0 + c * 8;
          const int off = c_store_off(r, n, N);
          const bool need = r < live && n >= 0 && n < N;
          ++checked;
          if (need && (off < 0 || (uint64_t)off + 16 > c_num || off != (r * N + n) * 2)) fail("C", r, n, off);
          if (!need && off >= 0 && (uint64_t)off < c_num) fail("C dropped", r, n, off);
        }
    }
  }
  // gathered A: rows of a [a_rows, K] operand through a permutation, padding rows out of range
  if (a_rows > 0) {
    const uint64_t g_num = (uint64_t)a_rows * K * 2;
    for (int kt = 0; kt < nk; ++kt)
      for (int w = 0; w < NW; ++w)
        for (int i = 0; i < A_LD; ++i)
          for (int lane = 0; lane < 64; ++lane) {
            const Piece pc = a_piece<BK>((w * A_LD + i) * 64 + lane);
            for (int pv : {-1, 0, a_rows - 1}) {
              const uint32_t v = pv >= 0 ? (uint32_t)(((int64_t)pv * K + pc.c * 8) * 2) : kOutOfRange;
              const int64_t want = pv >= 0 ? ((int64_t)pv * K + kt * BK + pc.c * 8) * 2 : -1;
              check_load("gathered A", v, (uint32_t)kt * BK * 2, g_num, want);
            }
          }
  }
}

int main(int argc, char** argv) {
  if (argc != 9) {
    printf("usage: %s BM BN BK NW K N ROWS A_ROWS\n", argv[0]);
    return 2;
  }
  const int BM = atoi(argv[1]), BN = atoi(argv[2]), BK = atoi(argv[3]), NW = atoi(argv[4]);
  const int K = atoi(argv[5]), N = atoi(argv[6]), rows = atoi(argv[7]), a_rows = atoi(argv[8]);
  if (K % BK || N % 8 || rows < 1) return 2;
#define SHAPE(bm, bn, bk, nw) \
  if (BM == bm && BN == bn && BK == bk && NW == nw) run<bm, bn, bk, nw>(K, N, rows, a_rows); else
  // the kernel's block tiles (grouped_gemm.hip, kShapes)
  SHAPE(256, 256, 64, 4)
  SHAPE(256, 256, 32, 4)
  SHAPE(256, 128, 32, 4)
  SHAPE(128, 128, 64, 4)
  SHAPE(128, 128, 32, 4)
  SHAPE(256, 256, 64, 8)
  SHAPE(256, 256, 32, 8)
  SHAPE(32, 256, 64, 4) {
    printf("unknown tile\n");
    return 2;
  }
  printf("ok %ld\n", checked);
  return 0;
}
