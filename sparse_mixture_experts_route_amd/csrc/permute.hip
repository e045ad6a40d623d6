// Dispatch as a local permutation.
//
// "Distributed training part 4" (jesamkim's AI tech blog), section 4,
// dispatch: every token is sent to the expert it selected. With all experts
// on one GPU the exchange becomes a reordering of the T*k selections into
// contiguous per-expert row groups, which the grouped GEMMs then read.
//
// The reordering is a stable counting sort, deterministic by construction:
//   hist    per block of 256 tokens, a bit mask mask[e] marks the tokens that
//           selected expert e (LDS atomicOr: the result does not depend on
//           the order of the atomics); counts per (block, expert) = popcounts.
//   scan    one workgroup: counts[e] over blocks, offsets[] as the exclusive
//           prefix sum over experts, and the first row of every (block, expert),
//           from the per-block counts staged in LDS. Up to kFusedScanBlocks
//           blocks of tokens, each scatter block derives its own first rows
//           from all the per-block counts instead (one launch fewer).
//   scatter the row of selection (t, j) is the base of (block, e) plus the
//           number of tokens before t in the block that selected e (popcount
//           of the mask below t), so rows follow token order inside a group.
//   gather  token-major: each x row is read once and written to its k rows.
//
// Batches of at most kSmallPermuteT tokens (decode-sized) run the same
// counting sort in one workgroup (permute_small_kernel): one launch instead
// of three, each a few microseconds of mostly launch and memory latency. Its
// FIN form first completes a router split over d_model (partial logits summed
// in split order, then the per-token selection), so that a decode-sized layer
// goes from the router's partial logits to perm and inv in one launch.
#include <stdlib.h>

#include "common.h"
#include "internal.h"
#include "topk.h"

namespace moe {

namespace {

constexpr int kTB = kPermuteTokensPerBlock;  // tokens per block, one thread each
constexpr int kWords = kTB / 32;             // mask words per expert

__device__ __forceinline__ void build_mask(const int32_t* __restrict__ idx, int64_t T, int k, int E,
                                           uint32_t (*mask)[kWords], int64_t t0) {
  uint32_t* flat = &mask[0][0];
  for (int i = threadIdx.x; i < E * kWords; i += kTB) flat[i] = 0u;
  __syncthreads();
  const int64_t t = t0 + threadIdx.x;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      if ((unsigned)e < (unsigned)E) atomicOr(&mask[e][threadIdx.x >> 5], 1u << (threadIdx.x & 31));
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kTB) void hist_kernel(const int32_t* __restrict__ idx, int64_t T, int k, int E,
                                                   int32_t* __restrict__ blockcounts, int32_t* __restrict__ zero,
                                                   int nzero) {
  __shared__ uint32_t mask[256][kWords];
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < nzero; i += kTB) zero[i] = 0;
  build_mask(idx, T, k, E, mask, (int64_t)blockIdx.x * kTB);
  const int e = threadIdx.x;
  if (e < E) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kWords; ++w) c += __popc(mask[e][w]);
    blockcounts[(int64_t)blockIdx.x * E + e] = c;
  }
}

// One workgroup. The per-block counts come into LDS with coalesced loads, in
// chunks of whole blocks when they do not fit at once. Thread (q, e) owns
// expert e and a contiguous quarter of the chunk's blocks. The first pass
// gives the totals per expert, then their exclusive prefix sum over experts
// is the offsets. The second pass writes the first row of every
// (block, expert): offsets[e] plus the counts of e in the earlier blocks.
constexpr int kScanThreads = 1024;
constexpr int kScanQ = kScanThreads / 256;  // threads per expert
constexpr int kScanLds = 16384;             // int32 counts staged per chunk

__global__ __launch_bounds__(kScanThreads) void scan_kernel(const int32_t* __restrict__ blockcounts, int64_t nb,
                                                            int E, int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ blockbase) {
  __shared__ int32_t s_c[kScanLds];
  __shared__ int32_t s_part[kScanQ][256];
  __shared__ int32_t s_run[256];
  const int tid = threadIdx.x, e = tid % 256, q = tid / 256;
  const int64_t cb = kScanLds / E;  // blocks per chunk (E <= 256, so at least 64)
  const int64_t nchunks = (nb + cb - 1) / cb;
  auto load_chunk = [&](int64_t b0, int64_t nbc) {
    const int32_t* src = blockcounts + b0 * E;
    for (int64_t i = tid; i < nbc * E; i += kScanThreads) s_c[i] = src[i];
  };
  // pass 1: totals per expert
  int32_t part = 0;
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t b0 = c * cb, nbc = min(cb, nb - b0);
    __syncthreads();  // the previous chunk has been read
    load_chunk(b0, nbc);
    __syncthreads();
    if (e < E)
      for (int64_t b = nbc * q / kScanQ; b < nbc * (q + 1) / kScanQ; ++b) part += s_c[b * E + e];
  }
  s_part[q][e] = part;
  __syncthreads();
  int32_t total = 0;
  if (q == 0) {
#pragma unroll
    for (int i = 0; i < kScanQ; ++i) total += s_part[i][e];
    s_run[e] = total;
  }
  __syncthreads();
  // inclusive Hillis-Steele scan over the 256 expert slots (slots >= E hold 0)
  for (int o = 1; o < 256; o <<= 1) {
    const int32_t v = (q == 0 && e >= o) ? s_run[e - o] : 0;
    __syncthreads();
    if (q == 0) s_run[e] += v;
    __syncthreads();
  }
  if (q == 0) {
    const int32_t incl = s_run[e];
    if (e < E) {
      counts[e] = total;
      offsets[e] = incl - total;
      if (e == E - 1) offsets[E] = incl;
    }
    s_run[e] = incl - total;  // running first row of expert e, from offsets[e]
  }
  // pass 2: first row of every (block, expert)
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t b0 = c * cb, nbc = min(cb, nb - b0);
    if (nchunks > 1) {
      __syncthreads();
      load_chunk(b0, nbc);
    }
    __syncthreads();
    const int64_t lo = nbc * q / kScanQ, hi = nbc * (q + 1) / kScanQ;
    int32_t sum = 0;
    if (e < E)
      for (int64_t b = lo; b < hi; ++b) sum += s_c[b * E + e];
    s_part[q][e] = sum;
    __syncthreads();
    if (e < E) {
      int32_t run = s_run[e];
      for (int i = 0; i < q; ++i) run += s_part[i][e];
      for (int64_t b = lo; b < hi; ++b) {
        blockbase[(b0 + b) * E + e] = run;
        run += s_c[b * E + e];
      }
    }
    __syncthreads();
    if (q == 0) {
#pragma unroll
      for (int i = 0; i < kScanQ; ++i) s_run[e] += s_part[i][e];
    }
  }
}

// Up to this many blocks of tokens the scatter blocks derive their first rows
// from the per-block counts themselves (each reads all nb x E counts), and the
// separate scan launch is skipped.
constexpr int kFusedScanBlocks = 64;

// SCAN: `blockcounts` holds the per-block counts of hist_kernel (nb blocks);
// every block sums them per expert (in total and over the blocks before it),
// scans the totals over the experts, and block 0 writes counts and offsets.
// Otherwise `blockcounts` is scan_kernel's first row of every (block, expert).
template <bool SCAN>
__global__ __launch_bounds__(kTB) void scatter_kernel(const int32_t* __restrict__ idx, int64_t T, int k, int E,
                                                      const int32_t* __restrict__ blockcounts, int64_t nb,
                                                      int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  __shared__ uint32_t mask[256][kWords];
  __shared__ int32_t s_base[256];
  const int64_t t0 = (int64_t)blockIdx.x * kTB;
  const int e0 = threadIdx.x;  // kTB = 256 threads: one expert slot each
  if constexpr (SCAN) {
    int32_t tot = 0, before = 0;
    if (e0 < E)
      for (int64_t b0 = 0; b0 < nb; b0 += 16) {  // sixteen loads in flight
        int32_t c[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) c[u] = b0 + u < nb ? blockcounts[(b0 + u) * E + e0] : 0;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          tot += c[u];
          before += b0 + u < (int64_t)blockIdx.x ? c[u] : 0;
        }
      }
    // inclusive Hillis-Steele scan of the totals over the 256 expert slots
    s_base[e0] = tot;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const int32_t v = e0 >= o ? s_base[e0 - o] : 0;
      __syncthreads();
      s_base[e0] += v;
      __syncthreads();
    }
    const int32_t incl = s_base[e0];
    if (blockIdx.x == 0 && e0 < E) {
      counts[e0] = tot;
      offsets[e0] = incl - tot;
      if (e0 == E - 1) offsets[E] = incl;
    }
    __syncthreads();  // every slot has been read
    s_base[e0] = incl - tot + before;
  } else {
    if (e0 < E) s_base[e0] = blockcounts[(int64_t)blockIdx.x * E + e0];
  }
  // this block's first row per expert is visible after build_mask's barriers
  build_mask(idx, T, k, E, mask, t0);
  const int64_t t = t0 + threadIdx.x;
  if (t >= T) return;
  const int w = threadIdx.x >> 5;
  const uint32_t below = (1u << (threadIdx.x & 31)) - 1u;
  // the selections in groups of 8, whose indices are loaded together
  for (int j0 = 0; j0 < k; j0 += 8) {
    int ev[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) ev[u] = j0 + u < k ? idx[t * k + j0 + u] : -1;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (j0 + u < k) {
        const int e = ev[u];
        int32_t r = -1;
        if ((unsigned)e < (unsigned)E) {
          int rank = __popc(mask[e][w] & below);
          for (int w2 = 0; w2 < w; ++w2) rank += __popc(mask[e][w2]);
          r = s_base[e] + rank;
          perm[r] = (int32_t)t;
        }
        inv[t * k + j0 + u] = r;
      }
    }
  }
}

constexpr int kSmallWords = kSmallPermuteT / 32;  // mask words per expert
constexpr int kSmallThreads = 1024;
static_assert(kSmallPermuteT <= kSmallThreads, "one token per thread");
static_assert(kFusedRouteT <= 2 * kSmallThreads / kWave, "at most two tokens per wave");

// One workgroup, T <= kSmallPermuteT tokens (thread t owns token t), k <= 8.
// FIN (T <= kFusedRouteT, one or two tokens per wave): the routing of the batch is
// completed first, as the router's own finalize launch does it
// (sum_partial_logits, then select_topk), so idx and gates are bitwise the
// same; idx stays in LDS until the end, gates go out directly. Otherwise idx is read
// from idx_in. Then the counting sort of the header: token bit masks per
// expert, counts and offsets from popcounts and a scan, rows in token order
// inside each group.
template <bool FIN>
__global__ __launch_bounds__(kSmallThreads) void permute_small_kernel(
    const int32_t* __restrict__ idx_in, const float* __restrict__ part, int nsplit, const float* __restrict__ bias,
    float* __restrict__ gate, int32_t* __restrict__ idx_out, int T, int k, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    int32_t* __restrict__ zero, int nzero) {
  __shared__ uint32_t mask[256][kSmallWords];
  if ((int)threadIdx.x < nzero) zero[threadIdx.x] = 0;
  __shared__ int32_t s_idx[kSmallPermuteT * 8];
  __shared__ float lg[FIN ? kFusedRouteT : 1][256];
  __shared__ int32_t s_scan[256];
  __shared__ int32_t s_off[256];
  const int tid = threadIdx.x, wave = tid / kWave;
  const int P = T * k;
  const int words = (T + 31) / 32;
  uint32_t* flat = &mask[0][0];
  for (int i = tid; i < E * kSmallWords; i += kSmallThreads) flat[i] = 0u;
  if constexpr (FIN) {
    // T <= kFusedRouteT: token t goes to wave t mod (the workgroup's waves), with an LDS row of its own
    for (int t = wave; t < T; t += kSmallThreads / kWave) {
      sum_partial_logits(part, nsplit, bias, T, E, t, lg[t]);
      select_topk(lg[t], E, k, t, nullptr, s_idx, gate);
    }
  } else {
    for (int i = tid; i < P; i += kSmallThreads) s_idx[i] = idx_in[i];
  }
  __syncthreads();
  if (tid < T)
    for (int j = 0; j < k; ++j) {
      const int e = s_idx[tid * k + j];
      if ((unsigned)e < (unsigned)E) atomicOr(&mask[e][tid >> 5], 1u << (tid & 31));
    }
  __syncthreads();
  // counts per expert, then an inclusive scan over the 256 expert slots
  int32_t c = 0;
  if (tid < 256) {
    if (tid < E)
      for (int w = 0; w < words; ++w) c += __popc(mask[tid][w]);
    s_scan[tid] = c;
  }
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int32_t v = tid < 256 && tid >= o ? s_scan[tid - o] : 0;
    __syncthreads();
    if (tid < 256) s_scan[tid] += v;
    __syncthreads();
  }
  if (tid < E) {
    s_off[tid] = s_scan[tid] - c;
    counts[tid] = c;
    offsets[tid] = s_scan[tid] - c;
    if (tid == E - 1) offsets[E] = s_scan[tid];
  }
  __syncthreads();
  if (tid < T) {
    const int w = tid >> 5;
    const uint32_t below = (1u << (tid & 31)) - 1u;
    for (int j = 0; j < k; ++j) {
      const int e = s_idx[tid * k + j];
      int32_t r = -1;
      if ((unsigned)e < (unsigned)E) {
        int rank = __popc(mask[e][w] & below);
        for (int w2 = 0; w2 < w; ++w2) rank += __popc(mask[e][w2]);
        r = s_off[e] + rank;
        perm[r] = tid;
      }
      inv[tid * k + j] = r;
    }
  }
  if constexpr (FIN)
    for (int i = tid; i < P; i += kSmallThreads) idx_out[i] = s_idx[i];
}

// One wave per token: the row is read once in 16-byte pieces and written to
// each of the token's k rows.
constexpr int kGatherWaves = 4;
constexpr int kGatherFastK = 8;  // selections per token handled with the rows held in registers
constexpr int kGatherU = 4;      // 16-byte pieces per lane in flight per row

// One wave per token: the token's row is read once, U pieces per lane at a
// time, and written to each of its k rows of x_perm. The k destination rows
// are read once per token.
__global__ __launch_bounds__(kGatherWaves * kWave) void gather_kernel(const u32x4* __restrict__ x,
                                                                      const int32_t* __restrict__ inv,
                                                                      u32x4* __restrict__ x_perm, int64_t T,
                                                                      int k, int64_t row_vecs, int64_t rows) {
  const int lane = threadIdx.x % kWave;
  const int64_t t = (int64_t)blockIdx.x * kGatherWaves + threadIdx.x / kWave;
  if (t >= T) return;
  const u32x4* src = x + t * row_vecs;
  if (k <= kGatherFastK) {
    int64_t dst[kGatherFastK];
#pragma unroll
    for (int j = 0; j < kGatherFastK; ++j) {
      const int32_t r = j < k ? inv[t * k + j] : -1;
      dst[j] = (r >= 0 && r < rows) ? (int64_t)r * row_vecs : -1;
    }
    for (int64_t c0 = lane; c0 < row_vecs; c0 += kWave * kGatherU) {
      u32x4 v[kGatherU];
#pragma unroll
      for (int u = 0; u < kGatherU; ++u)
        if (c0 + u * kWave < row_vecs) v[u] = src[c0 + u * kWave];
#pragma unroll
      for (int j = 0; j < kGatherFastK; ++j)
        if (dst[j] >= 0)
#pragma unroll
          for (int u = 0; u < kGatherU; ++u)
            if (c0 + u * kWave < row_vecs) x_perm[dst[j] + c0 + u * kWave] = v[u];
    }
    return;
  }
  for (int64_t c = lane; c < row_vecs; c += kWave) {
    const u32x4 v = src[c];
    for (int j = 0; j < k; ++j) {
      const int32_t r = inv[t * k + j];
      if (r >= 0 && r < rows) x_perm[(int64_t)r * row_vecs + c] = v;
    }
  }
}

}  // namespace

// Batches of at most kFusedTokens tokens complete a split router inside the
// one-workgroup permute (MOE_FUSED_ROUTE_T=<n> overrides, at most kFusedRouteT).
int fused_route_tokens() {
  const char* f = getenv("MOE_FUSED_ROUTE_T");
  return f && f[0] ? std::min(std::max(atoi(f), 0), kFusedRouteT) : kFusedTokens;
}

bool route_permute_fused(const moe_problem_t& p) {
  const int ns = route_splits(p);
  return ns > 1 && p.T <= fused_route_tokens() && p.k <= 8 && (int64_t)ns * p.T * p.E * 4 <= 256 * 1024;
}

int permute_form(const moe_problem_t& p) {
  if (p.T <= kSmallPermuteT && p.k <= 8) return 0;
  // MOE_PERMUTE_FUSED_SCAN=0|1 forces the choice (1 only within kFusedScanBlocks)
  bool fused = permute_blocks(p.T) <= kFusedScanBlocks;
  const char* force = getenv("MOE_PERMUTE_FUSED_SCAN");
  if (force && force[0]) fused = fused && atoi(force) != 0;
  return fused ? 1 : 2;
}

hipError_t launch_permute_index(const moe_problem_t& p, const int32_t* idx, int32_t* counts, int32_t* offsets,
                                int32_t* perm, int32_t* inv, int32_t* blockcounts, int32_t* blockbase,
                                hipStream_t s, int32_t* zero, int nzero) {
  if (!zero) nzero = 0;
  if (nzero < 0 || nzero > kSmallThreads) return hipErrorInvalidValue;
  const int form = permute_form(p);
  if (form == 0) {
    hipLaunchKernelGGL(permute_small_kernel<false>, dim3(1), dim3(kSmallThreads), 0, s, idx, nullptr, 0, nullptr,
                       nullptr, nullptr, (int)p.T, p.k, p.E, counts, offsets, perm, inv, zero, nzero);
    return hipGetLastError();
  }
  const int64_t nb = permute_blocks(p.T);
  hipLaunchKernelGGL(hist_kernel, dim3((unsigned)nb), dim3(kTB), 0, s, idx, p.T, p.k, p.E, blockcounts, zero,
                     nzero);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (form == 1) {
    hipLaunchKernelGGL(scatter_kernel<true>, dim3((unsigned)nb), dim3(kTB), 0, s, idx, p.T, p.k, p.E, blockcounts,
                       nb, counts, offsets, perm, inv);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, s, blockcounts, nb, p.E, counts, offsets,
                     blockbase);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(scatter_kernel<false>, dim3((unsigned)nb), dim3(kTB), 0, s, idx, p.T, p.k, p.E, blockbase, nb,
                     counts, offsets, perm, inv);
  return hipGetLastError();
}

hipError_t launch_finalize_permute_small(const moe_problem_t& p, const float* part, int nsplit, const float* bias,
                                        int32_t* idx, float* gate, int32_t* counts, int32_t* offsets,
                                        int32_t* perm, int32_t* inv, hipStream_t s, int32_t* zero, int nzero) {
  if (!zero) nzero = 0;
  if (p.T > kFusedRouteT || p.k > 8 || p.E % 4 != 0 || nzero < 0 || nzero > kSmallThreads)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(permute_small_kernel<true>, dim3(1), dim3(kSmallThreads), 0, s, nullptr, part, nsplit, bias,
                     gate, idx, (int)p.T, p.k, p.E, counts, offsets, perm, inv, zero, nzero);
  return hipGetLastError();
}

namespace {
__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t* __restrict__ p, int n) {
  for (int i = threadIdx.x; i < n; i += 256) p[i] = 0;
}
}  // namespace

hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s) {
  hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_gather(const moe_problem_t& p, const void* x, const int32_t* inv, void* x_perm,
                         hipStream_t s) {
  const int es = p.dtype == MOE_DTYPE_BF16 ? 2 : 4;
  const int64_t row_vecs = (int64_t)p.d_model * es / 16;
  const int64_t blocks = ceil_div(p.T, kGatherWaves);
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(kGatherWaves * kWave), 0, s, (const u32x4*)x,
                     inv, (u32x4*)x_perm, p.T, p.k, row_vecs, p.T * p.k);
  return hipGetLastError();
}

}  // namespace moe
