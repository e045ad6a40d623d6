// Internal launchers of the MoE layer kernels (host side). Each enqueues on
// `s` and returns the launch status; arguments were validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kPermuteTokensPerBlock = 256;
// batches of at most this many tokens (and k <= 8) are permuted by one workgroup
constexpr int kSmallPermuteT = 1024;
// ... and with at most kFusedTokens (kFusedRouteT at most), that workgroup
// also completes a split router
constexpr int kFusedRouteT = 32;
constexpr int kFusedTokens = 16;

inline int64_t permute_blocks(int64_t T) { return (T + kPermuteTokensPerBlock - 1) / kPermuteTokensPerBlock; }

// Multiprocessor count of the current device (at most 256; 256 when unknown).
int device_cus();

// Router. With `part` (route_partials_bytes(p) bytes, float32) the bf16 path
// splits the contraction over d_model when the token blocks alone do not fill
// the GPU (route_splits(p) > 1) and finishes with a second launch.
hipError_t launch_route(const moe_problem_t& p, const void* x, const void* w_router, const float* bias,
                        float* logits, int32_t* idx, float* gate, float* part, hipStream_t s);
int route_splits(const moe_problem_t& p);
size_t route_partials_bytes(const moe_problem_t& p);
// The first launch of a split router alone (route_splits(p) > 1 required):
// float32 partial logits to part.
hipError_t launch_route_partials(const moe_problem_t& p, const void* x, const void* w_router, float* part,
                                 hipStream_t s);
// Decode-sized batches (route_permute_fused(p)): one workgroup completes a
// split router from its partial logits (idx, gate as launch_route would give
// them) and permutes (counts, offsets, perm, inv as launch_permute_index).
bool route_permute_fused(const moe_problem_t& p);
// With `zero`, both permute launchers also set its first nzero (<= 1024)
// int32 to 0 on the way (the grouped GEMMs' split-tile counters).
hipError_t launch_finalize_permute_small(const moe_problem_t& p, const float* part, int nsplit, const float* bias,
                                        int32_t* idx, float* gate, int32_t* counts, int32_t* offsets,
                                        int32_t* perm, int32_t* inv, hipStream_t s, int32_t* zero = nullptr,
                                        int nzero = 0);

// counts/offsets/perm/inv from the routing table; blockcounts/blockbase are
// workspace arrays of permute_blocks(T) * E int32 each.
hipError_t launch_permute_index(const moe_problem_t& p, const int32_t* idx, int32_t* counts,
                                int32_t* offsets, int32_t* perm, int32_t* inv,
                                int32_t* blockcounts, int32_t* blockbase, hipStream_t s, int32_t* zero = nullptr,
                                int nzero = 0);

// Form of launch_permute_index for p: 0 one workgroup (T <= kSmallPermuteT,
// k <= 8), 1 per-block histograms then a scatter that scans for itself,
// 2 histograms, a scan launch and the scatter.
int permute_form(const moe_problem_t& p);
// Whether launch_combine streams y_perm and y with non-temporal accesses.
bool combine_streams(const moe_problem_t& p);
// Tokens per router block (32 or 64).
int route_rt(const moe_problem_t& p);

// p[0 .. n) = 0 (one small block)
hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s);

// x_perm[inv[t*k+j]] = x[t] for every valid selection.
hipError_t launch_gather(const moe_problem_t& p, const void* x, const int32_t* inv, void* x_perm,
                         hipStream_t s);

// C[r] = act(A[r] B[e]) for rows r of every expert group e (offsets[E+1]).
// A [R, K], B [E, K, N], C [R, N]; act = GELU_tanh or identity. `partials` is
// workspace of grouped_gemm_partials_bytes() for split tiles (bf16 path).
// With `perm` (bf16) row r of A is row perm[r] of A [a_rows, K]; returns
// hipErrorInvalidValue when a_rows * K * 2 does not fit in 31 bits.
// `counters` (kGemmSplitCounters int32) must be zero when the launch starts
// if grouped_gemm_uses_counters() says the launch completes split tiles
// itself (gelu: the launch's activation); it leaves them zero again.
// Launches on one stream may share them.
hipError_t launch_grouped_gemm(int dtype, const void* A, const int32_t* offsets, const void* B, void* C,
                               float* partials, int32_t* counters, int64_t R, int K, int N, int E, bool gelu,
                               hipStream_t s, const int32_t* perm = nullptr, int64_t a_rows = 0);
// split-tile counters: one per leftover tile of each XCD's range
constexpr int kSplitCountersPerXcd = 64;
constexpr int kGemmSplitCounters = 8 * kSplitCountersPerXcd;
bool grouped_gemm_uses_counters(int dtype, int64_t R, int K, int N, int E, bool gelu);

// Launch geometry of a bf16 grouped GEMM as launch_grouped_gemm picks it
// (host only): block tile (index into the tile table), persistent grid, K
// steps per tile, split rule, and whether split tiles are completed inside the
// launch (gelu: the launch's activation).
struct GemmGeom {
  int shape, bm, bn, bk;
  int grid, nb, nk, n_tiles;
  int max_rem, min_steps;
  bool in_launch;
};
GemmGeom gemm_geom(int64_t R, int K, int N, int E, bool gelu);
// The tile list the kernels derive on the device for per-expert row counts
// (host copy): total tiles, the whole rounds and leftover tiles of the XCD
// with the most tiles and whether its leftover is split by K steps, and the
// number of XCDs whose leftover is split.
struct GemmXcdPlan {
  int64_t tiles;
  int full, rem, split, split_xcds;
};
void gemm_xcd_plan(const GemmGeom& g, const int32_t* counts, int E, GemmXcdPlan* out);

// Host-only bound of the partial-sum workspace one launch_grouped_gemm call may use.
size_t grouped_gemm_partials_bytes(int dtype, int64_t R, int K, int N, int E);

// The whole layer of a small float32 problem in one launch (small_layer.hip):
// the same y, bit for bit, as route -> permute -> grouped FFN -> combine.
bool small_layer_fused(const moe_problem_t& p);
hipError_t launch_small_layer(const moe_problem_t& p, const void* x, const void* w_router, const float* bias,
                              const void* W1, const void* W2, void* y, hipStream_t s);

hipError_t launch_combine(const moe_problem_t& p, const void* y_perm, const int32_t* inv,
                          const float* gate, void* y, hipStream_t s);

// ---- backward (bf16)
// C[rows] = A[rows] B_e^T (* GELU_tanh'(U) when U is given) for the expert
// row groups of offsets (nullptr: one group of R rows): A [R, lda] (K
// contiguous), B_e = B + e * b_estride as [N, ldb] rows (K contiguous), C and
// U [R, N]; K a multiple of 64.
hipError_t launch_bwd_gemm_nt(const uint16_t* A, int lda, const int32_t* offsets, int64_t R, int E,
                              const uint16_t* B, int ldb, int64_t b_estride, uint16_t* C, int N, int K,
                              const uint16_t* U, float* partials, hipStream_t s);
// With `partials` (bwd_partials_bytes) and no U, a small last round of long
// tiles is split over the blocks by K steps and completed by the fixup.
// C_e = A_e^T B_e for every expert e (offsets; nullptr: E equal groups of R rows),
// reducing over the group's rows: A [rows, lda] (M contiguous; with perm,
// row r is row perm[r] of A [a_rows, lda]), B [rows, ldb] (N contiguous),
// C_e = C + e * M * N as [M, N]. Experts without rows get zeros.
hipError_t launch_bwd_gemm_tn(const uint16_t* A, int lda, const int32_t* perm, int64_t a_rows,
                              const int32_t* offsets, int64_t R, int E, const uint16_t* B, int ldb, uint16_t* C,
                              int M, int N, float* partials, hipStream_t s);
// Partial-sum slots (256 x 256 float32 each) that the K-grouped launches with
// expert row groups may use to cut hot experts' reductions into chunks; the
// workspace holds kKGroupSlots of them.
constexpr int kKGroupSlots = 256;
int kgroup_slots();
// Split-tile fixup of an 8-wave 256 x 256 row-grouped launch (no activation),
// and the split threshold in K steps (MOE_GEMM_SPLIT_MIN_STEPS overrides it).
hipError_t launch_split_fixup_256(const int32_t* offsets, const float* partials, uint16_t* C, int64_t R, int nk, int N,
                                  int E, int nb, int min_steps, int max_rem, hipStream_t s);
int split_min_steps();
// Float32 partial-sum bytes launch_bwd_gemm_nt may use for R rows, E groups, N columns.
size_t bwd_partials_bytes(int64_t R, int E, int N);
// Rows of x^T dlogit per split of the router weight gradient, and the number of splits.
int bwd_router_splits(int64_t T, int d, int E);
hipError_t launch_sum_splits(const uint16_t* part, int splits, int64_t n, uint16_t* out, hipStream_t s);
hipError_t launch_bwd_combine(const moe_problem_t& p, const void* dy, const float* gate, const int32_t* idx,
                              const int32_t* inv, const void* Y_perm, const float* logits, void* dYp,
                              float* dlogit, uint16_t* dlogit_b, float* prob, int Ep, hipStream_t s);
hipError_t launch_bwd_dx(const moe_problem_t& p, const void* dXp, const int32_t* inv, const void* dxr, void* dx,
                         hipStream_t s);
hipError_t launch_gelu_rows(const void* U, void* H, int64_t elems, hipStream_t s);
int64_t bwd_stat_chunks(int64_t T);
hipError_t launch_bwd_stats(const moe_problem_t& p, const float* prob, const float* dlogit, const int32_t* counts,
                            float* part, float* load_frac, float* mean_prob, float* dbias, hipStream_t s);

}  // namespace moe
