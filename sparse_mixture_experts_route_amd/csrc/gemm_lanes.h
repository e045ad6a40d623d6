// Lane address arithmetic of the grouped GEMM's direct-to-LDS operand loads:
// which 16-byte piece of a stage each lane fetches, and its byte offset in
// the operand. Shared by the kernel and by a host-side check that replays
// every load of a launch and asserts that each one reads inside its operand
// or is sent past the buffer descriptor's range (and so reads zero).
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define MOE_LANES_FN __host__ __device__ __forceinline__
#else
#define MOE_LANES_FN inline
#endif

namespace moe {
namespace lanes {

// A byte offset past every buffer range this library builds (ranges stay
// below 2^31), which stays past it when a K-step offset below 2^31 is added,
// so no 32-bit sum wraps back into range.
constexpr uint32_t kOutOfRange = 0x80000000u;

// One 16-byte piece of a stage: row of A (or k row of B) and chunk index.
struct Piece {
  int row, c;
};

// A stage holds BM rows of BK bf16 (K contiguous). LDS slot p (16 bytes each,
// in order) holds row p / (BK / 8) and the chunk whose index is the slot's
// XOR-ed with the row's position in its 256-byte bank period.
template <int BK>
MOE_LANES_FN Piece a_piece(int p) {
  constexpr int A_CH = BK / 8, A_RPP = 256 / (BK * 2);
  const int row = p / A_CH;
  return {row, (p % A_CH) ^ ((row / A_RPP) & (A_CH - 1))};
}

// A B stage holds BK k rows of BN bf16 (N contiguous). Slot p holds k row
// p / (BN / 8), chunk (p % (BN / 8)) XOR 4 (k & 3).
template <int BN>
MOE_LANES_FN Piece b_piece(int p) {
  constexpr int B_SLOTS = BN / 8;
  const int k = p / B_SLOTS;
  return {k, (p % B_SLOTS) ^ (4 * (k & 3))};
}

// Offset of an A piece inside the tile's first row, K step 0 (the K step
// adds kt * BK * 2 bytes).
MOE_LANES_FN uint32_t a_lane_off(Piece pc, int K) { return (uint32_t)(pc.row * K + pc.c * 8) * 2u; }

// Offset of a B piece of a tile at column 0, K step 0, in the expert's
// [K, N] slab. The kernel adds the tile's first column as 2 * n0 (modulo
// 2^32: n0 may be negative, see tile_n0) and passes kt * BK * N * 2 as the
// scalar offset of K step kt.
MOE_LANES_FN uint32_t b_lane_off(Piece pc, int N) { return (uint32_t)(pc.row * N + pc.c * 8) * 2u; }

// First column of n-tile nt of n_tiles tiles of BN columns over N columns.
// The tiles end at column N: when N is not a multiple of BN, the first tile
// starts left of column 0. Its lanes that fetch negative columns of a weight
// row read the end of the row before (or, on the slab's first row, fall past
// the buffer range and read zero), and their outputs are never stored, so no
// load of any tile reaches past the end of an expert's weight slab.
MOE_LANES_FN int tile_n0(int nt, int n_tiles, int N, int BN) {
  return N - (n_tiles - nt) * BN;
}


// Byte offset of the 16-byte store of output columns n .. n + 7 of row
// `row` of a tile (C rows are N contiguous), or an offset past any store
// range for columns outside [0, N) (the first tile of a row of tiles may
// start left of column 0).
MOE_LANES_FN int c_store_off(int row, int n, int N) { return n >= 0 && n < N ? (row * N + n) * 2 : 0x7FFFFFF0; }

}  // namespace lanes
}  // namespace moe
