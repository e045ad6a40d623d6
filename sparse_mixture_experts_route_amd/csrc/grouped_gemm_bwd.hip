// Expert FFN GEMMs of the layer backward.
//
// The experts are independent FFNs ("Distributed training part 4", jesamkim's
// AI tech blog, section 3); the MOSAIC summary ("Compute-Optimal Is Not
// Cluster-Optimal", gist.science, method item 2) counts them as grouped GEMMs,
// forward and backward. With U = X W1_e, H = GELU_tanh(U), Y = H W2_e per
// expert row group, the backward needs
//   dU  = (dYp W2_e^T) * GELU_tanh'(U)       rows grouped by expert (M-grouped)
//   dX  = dU W1_e^T                           M-grouped
//   dW2_e = H^T dYp,  dW1_e = X^T dU          K grouped: the expert's rows are
//                                             the reduction dimension
// so, next to the forward kernel's layout (A rows K-contiguous, B [K, N]
// N-contiguous), operands appear transposed: the weights as [N, K]
// (K-contiguous rows, e.g. W2_e [d_expert, d_model] for dYp W2_e^T) and the
// activations as [K, M] (M-contiguous rows, e.g. H [rows, d_expert] for
// H^T dYp).
//
// One kernel covers these cases with two operand stagings, both straight
// from HBM to LDS (buffer_load_dwordx4 ... lds):
//   * K-contiguous operand (a tile of 256 rows x 64 k): LDS [row][64] bf16,
//     16-byte chunks XOR-swizzled by (row >> 1) & 7; fragments are
//     ds_read_b128 (8 consecutive k of one row per lane);
//   * MN-contiguous operand (64 k x 256 columns): LDS [k][256] bf16, chunks
//     XOR-swizzled by 4 (k & 3); fragments are two ds_read_b64_tr_b16 (4
//     consecutive k of one column per lane each).
// Both give the v_mfma_f32_32x32x16_bf16 operand layout (lane l: row or
// column l & 31, k 8 (l >> 5) .. + 7). Tiles are 256 x 256 with 8 waves (2 x 4
// wave grid of 128 x 64), K steps of 64, two LDS stages (128 KB) and one
// barrier per step; the next step's loads are issued right after the barrier
// and the next sub-step's fragments are read while the current MFMAs run.
//
// M-grouped launches take their tiles from the expert row groups (offsets[],
// as the forward kernel); K-grouped launches run E x (M / 256) x (N / 256)
// tiles, each reducing over its expert's rows (zero rows: the tile stores
// zeros), experts taken in order of decreasing row count so that the long
// tiles of hot experts start first. When a hot expert's reduction is much
// longer than a block's fair share of the launch, its tiles are cut into
// chunks of K steps (kgroup_schedule): each chunk writes float32 partial sums
// and kgroup_fixup_kernel adds them in chunk order (deterministic, no
// atomics). The A operand of a K-grouped launch may
// be gathered: row r read as row perm[r] of a [a_rows, M] matrix (dW1 reads
// the tokens straight from x). The epilogue stages bf16 results through LDS
// and writes whole row segments; EPI_DGELU multiplies by GELU_tanh'(U) at the
// same positions before rounding.
#include <stdlib.h>

#include "common.h"
#include "gemm_lanes.h"
#include "internal.h"
#include "lds_dma.h"
#include "tiles.h"

namespace moe {

namespace {

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kWM = 2, kWN = 4, kNW = kWM * kWN;
constexpr int kWTM = kBM / kWM, kWTN = kBN / kWN;  // 128 x 64 per wave
constexpr int kTM = kWTM / 32, kTN = kWTN / 32;     // MFMA tiles per wave
constexpr int kKS = kBK / 16;                       // MFMA sub-steps per K step
constexpr int kOp = 256 * kBK * 2;                  // bytes of one operand tile per stage (32 KB)
constexpr int kStage = 2 * kOp;
constexpr int kLd = kOp / 1024 / kNW;               // 1 KB loads per wave per operand per stage (4)
constexpr int kThreads = kNW * kWave;

enum { EPI_PLAIN = 0, EPI_DGELU = 1 };

// GELU_tanh'(u) = (1 + tanh z)/2 + u/2 (1 - tanh^2 z) sqrt(2/pi) (1 + 3 * 0.044715 u^2),
// z = sqrt(2/pi) (u + 0.044715 u^3); tanh z = 1 - 2 / (1 + e^(2z)) with the hardware exp2
// and reciprocal (saturates to +-1 for large |z|).
__device__ __forceinline__ float gelu_tanh_grad(float u) {
  const float c = 0.7978845608028654f, a = 0.044715f;
  const float z = c * fmaf(a * u, u * u, u);
  const float th = 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(2.8853900817779268f * z));
  return 0.5f * (1.0f + th) + 0.5f * u * (1.0f - th * th) * c * fmaf(3.0f * a, u * u, 1.0f);
}

// K-grouped schedule (both the GEMM kernel and its fixup derive it, the same
// way, from the row groups): experts by decreasing row count (ties: lower
// index first) in order[]; with partial-sum slots available (max_slots > 0),
// an expert of nk K steps is cut into c = ceil(nk / L) chunks when nk > L, with
// L = max(kMinChunk, ceil(W / (4 nb))) doubled until the chunked experts' items
// fit in max_slots (W: the K steps of all tiles, nb: blocks of the launch).
// Items: rank by rank, chunk-major, then tile; ibase[r] = first item of rank
// r, ibase[E] = items. The chunked experts rank first, so their items are the
// partial-sum slots 0 ... Returns L (huge when nothing is cut).
constexpr int kMinChunk = 16;
template <typename Grp>
__device__ int kgroup_schedule(Grp grp, int E, int per, int nb, int max_slots, int* order, int* chunks,
                               int* ibase) {
  __shared__ int s_L;
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += blockDim.x) {
    const int64_t c = grp(e + 1) - grp(e);
    int rank = 0;
    for (int f = 0; f < E; ++f) {
      const int64_t cf = grp(f + 1) - grp(f);
      rank += (cf > c || (cf == c && f < e)) ? 1 : 0;
    }
    order[rank] = e;
  }
  __syncthreads();
  if (tid < kWave) {
    const int lane = tid;
    int64_t nk[4];
    int64_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = lane * 4 + i;
      nk[i] = r < E ? ceil_div(max(grp(order[r] + 1) - grp(order[r]), (int64_t)0), kBK) : 0;
      w += nk[i] * per;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) w += __shfl_xor(w, o, kWave);
    int64_t L = max((int64_t)kMinChunk, ceil_div(w, (int64_t)4 * nb));
    if (max_slots <= 0) L = INT32_MAX / 2;
    for (;;) {  // coarser chunks until the partial sums fit
      int64_t slots = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t c = ceil_div(nk[i], L);
        slots += c > 1 ? c * per : 0;
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) slots += __shfl_xor(slots, o, kWave);
      if (slots <= max_slots || L >= INT32_MAX / 4) break;
      L *= 2;
    }
    int c[4], local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = lane * 4 + i < E ? (int)max((int64_t)1, ceil_div(nk[i], L)) : 0;
      local += c[i] * per;
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
      const int r = lane * 4 + i;
      if (r < E) {
        chunks[r] = c[i];
        ibase[r] = run;
      }
      run += c[i] * per;
    }
    if (lane == kWave - 1) ibase[E] = incl;
    if (lane == 0) s_L = (int)L;
  }
  __syncthreads();
  return s_L;
}

struct BwdArgs {
  const bf16_bits* A;   // M-grouped: [R, lda] rows; K-grouped: [rows, lda] (or [a_rows, lda] gathered)
  const bf16_bits* B;   // M-grouped: expert e at B + e * b_estride, [N, ldb] rows (K-contiguous);
                        // K-grouped: [rows, ldb] (N-contiguous)
  bf16_bits* C;         // M-grouped: [R, N]; K-grouped: expert e at C + e * M * N, [M, N]
  const bf16_bits* U;   // EPI_DGELU: [R, N], same positions as C
  const int32_t* offsets;  // expert row groups (nullptr: one group of R rows, or, K-grouped,
                           // E equal groups)
  const int32_t* perm;     // K-grouped gathered A: row r is row perm[r] of A
  float* partials;         // M-grouped: float32 partial sums of split tiles (max_rem > 0)
  int64_t R, a_rows, b_estride;
  int M, N, K, lda, ldb, E;
  int min_steps, max_rem;  // M-grouped split of the last round (split_leftover)
  int gm;                  // M-grouped: m-tiles per raster group (tile_coords)
  int kslots;              // K-grouped: partial-sum slots for chunked tiles (0: no chunks)
};

template <bool KGROUP, bool A_MN, bool B_MN, bool GATHER_A, int EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_bwd_kernel(BwdArgs args) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kStage];
  __shared__ int s_tstart[257];
  __shared__ int s_mtiles[256];
  __shared__ int s_order[256];
  __shared__ int s_chunks[256];
  __shared__ int s_ibase[257];

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm0 = (wave / kWN) * kWTM, wn0 = (wave % kWN) * kWTN;
  lds_char* const lds = (lds_char*)smem;
  const uint32_t lds_base = lds_addr(smem);
  const int E = (KGROUP || args.offsets) ? args.E : 1;
  // K-grouped row group e: offsets[e] .. offsets[e + 1], or the e-th of E equal parts of R
  auto grp = [&](int e) -> int64_t { return args.offsets ? (int64_t)args.offsets[e] : args.R * e / E; };
  const int n_tiles = (int)ceil_div(args.N, kBN);
  const int m_fixed = (int)ceil_div(args.M, kBM);  // K-grouped: m tiles per expert

  int total, kL = 0;
  if constexpr (KGROUP) {
    kL = kgroup_schedule(grp, E, m_fixed * n_tiles, (int)gridDim.x, args.partials ? args.kslots : 0, s_order,
                         s_chunks, s_ibase);
    total = s_ibase[E];
  } else {
    if (args.offsets) {
      build_tile_list<kBM>(args.offsets, E, args.R, n_tiles, s_tstart, s_mtiles);
    } else {
      if (tid == 0) {
        s_tstart[0] = 0;
        s_mtiles[0] = (int)ceil_div(args.R, kBM);
        s_tstart[1] = s_mtiles[0] * n_tiles;
      }
      __syncthreads();
    }
    total = s_tstart[E];
  }

  // ---- fragment read offsets (bytes within an operand tile of a stage)
  // K-contiguous tile: row r at r * 128, chunk c at ((c ^ ((r >> 1) & 7)) << 4)
  int kc_x[kKS];
  {
    const int sw = ((lane & 31) >> 1) & 7;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) kc_x[ks] = ((ks * 2 + (lane >> 5)) ^ sw) << 4;
  }
  // MN-contiguous tile: lane q of its 16-lane group reads k row (q >> 2) of a
  // 4-row block, columns 4 (q & 3) .. + 3; lanes 32..63 take the upper 8 k
  const int q = lane & 15, g = lane >> 4, kr = q >> 2;
  auto mn_rd = [&](int col0) {
    const int col = col0 + (g & 1) * 16 + (q & 3) * 4;
    return ((g >> 1) * 8 + kr) * 512 + (((col >> 3) ^ (4 * kr)) << 4) + (col & 7) * 2;
  };
  int a_rd[kTM], b_rd[kTN];
#pragma unroll
  for (int mi = 0; mi < kTM; ++mi)
    a_rd[mi] = A_MN ? mn_rd(wm0 + mi * 32) : (wm0 + mi * 32 + (lane & 31)) * 128;
#pragma unroll
  for (int ni = 0; ni < kTN; ++ni)
    b_rd[ni] = B_MN ? mn_rd(wn0 + ni * 32) : (wn0 + ni * 32 + (lane & 31)) * 128;

  bf16x8 fa[2][kTM], fb[2][kTN];
  auto read_frag = [&](const lds_char* op, bool mn, int rd, int ks) {
    if (mn) {
      const lds_char* p0 = op + ks * 16 * 512 + rd;
      const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
      const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 4 * 512));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    return *(const lds_bf16x8*)(op + rd + kc_x[ks]);
  };
  auto read_set = [&](int buf, int ks, int set) {
    const lds_char* st = lds + buf * kStage;
#pragma unroll
    for (int mi = 0; mi < kTM; ++mi) fa[set][mi] = read_frag(st, A_MN, a_rd[mi], ks);
#pragma unroll
    for (int ni = 0; ni < kTN; ++ni) fb[set][ni] = read_frag(st + kOp, B_MN, b_rd[ni], ks);
  };

  // ---- DMA offsets of this lane (bytes), per operand kind
  // K-contiguous tile: slot p holds row p / 8, chunk (p % 8) ^ ((row >> 1) & 7)
  // MN-contiguous tile: slot p holds k row p / 32, chunk (p % 32) ^ (4 (k & 3))
  int kc_row[kLd], kc_c8[kLd], mn_k[kLd], mn_c8[kLd];
#pragma unroll
  for (int i = 0; i < kLd; ++i) {
    const int p = (wave * kLd + i) * kWave + lane;
    kc_row[i] = p / 8;
    kc_c8[i] = ((p % 8) ^ ((kc_row[i] >> 1) & 7)) * 8;
    mn_k[i] = p / 32;
    mn_c8[i] = ((p % 32) ^ (4 * (mn_k[i] & 3))) * 8;
  }

  f32x16 acc[kTM][kTN];

  // ---- work items. K-grouped: tiles blockIdx.x, + gridDim.x, ... M-grouped:
  // the tile list is cut into 8 contiguous ranges, one per XCD (blocks are dealt
  // to the XCDs round robin), whole tiles round by round, then a small last
  // round of long tiles split over the XCD's blocks by K steps (split_k); split
  // shares write float32 partial sums that the fixup kernel adds in K order.
  const int nkt = KGROUP ? 0 : args.K / kBK;
  const int xcd = blockIdx.x % 8, nbk = gridDim.x / 8, jb = blockIdx.x / 8;
  const int lo = KGROUP ? 0 : (int)((int64_t)total * xcd / 8);
  SplitK sk{};
  int n_items;
  if constexpr (KGROUP) {
    n_items = (int)blockIdx.x < total ? (total - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
  } else {
    const int hi = (int)((int64_t)total * (xcd + 1) / 8);
    sk = split_k(hi - lo, nbk, jb, nkt, args.min_steps, args.max_rem);
    n_items = sk.n_items;
  }

  for (int item = 0; item < n_items; ++item) {
    int t, kb = 0, kn = nkt, slot = -1;
    if constexpr (KGROUP) {
      t = (int)blockIdx.x + item * (int)gridDim.x;
    } else if (item < sk.full) {
      t = lo + jb + item * nbk;
    } else {
      const int r = sk.r_first + (item - sk.full);
      t = lo + sk.full * nbk + r;
      const int64_t a0 = max(sk.s0, (int64_t)r * nkt), b0 = min(sk.s1, (int64_t)(r + 1) * nkt);
      kb = (int)(a0 - (int64_t)r * nkt);
      kn = (int)(b0 - a0);
      slot = kn == nkt ? -1 : (int)blockIdx.x * 2 + (item - sk.full);
    }
    // ---- the tile: rows (M side), columns (N side), K range, operand bases
    int e, mt, nt;
    int64_t row0, row_end;  // M-grouped: rows of A and C; K-grouped: rows of the expert (K range)
    if constexpr (KGROUP) {
      // rank r with ibase[r] <= t < ibase[r + 1]; chunk ch of its reduction, tile lt
      const int per = m_fixed * n_tiles;
      int a0 = 0, a1 = E;
      while (a1 - a0 > 1) {
        const int mid = (a0 + a1) >> 1;
        if (s_ibase[mid] <= t) a0 = mid; else a1 = mid;
      }
      e = s_order[a0];
      const int local = t - s_ibase[a0], ch = local / per, lt = local - ch * per;
      nt = lt / m_fixed;
      mt = lt - nt * m_fixed;
      row0 = grp(e);
      row_end = grp(e + 1);
      if (s_chunks[a0] > 1) {  // a chunk: float32 partial sums to slot t
        row0 += (int64_t)ch * kL * kBK;
        row_end = min(row_end, row0 + (int64_t)kL * kBK);
        slot = t;
      }
    } else {
      int a0 = 0, a1 = E;
      while (a1 - a0 > 1) {
        const int mid = (a0 + a1) >> 1;
        if (s_tstart[mid] <= t) a0 = mid; else a1 = mid;
      }
      e = a0;
      const int local = t - s_tstart[e], mtl = s_mtiles[e];
      tile_coords(local, mtl, n_tiles, args.gm, nt, mt);
      const int64_t g0 = args.offsets ? args.offsets[e] : 0;
      row0 = g0 + (int64_t)mt * kBM;
      row_end = args.offsets ? min((int64_t)args.offsets[e + 1], args.R) : args.R;
    }
    e = __builtin_amdgcn_readfirstlane(e);
    const int m0 = KGROUP ? mt * kBM : 0, n0 = nt * kBN;
    const int nk = KGROUP ? (int)ceil_div(row_end - row0, kBK) : kn;

    // operand descriptors (byte ranges end the valid data: loads past them read zero)
    i32x4 rsA, rsB;
    if constexpr (KGROUP) {
      if constexpr (GATHER_A)
        rsA = buffer_rsrc(args.A, (uint32_t)(args.a_rows * args.lda * 2));
      else
        rsA = buffer_rsrc(args.A + row0 * args.lda, (uint32_t)((row_end - row0) * args.lda * 2));
      rsB = buffer_rsrc(args.B + row0 * args.ldb, (uint32_t)((row_end - row0) * args.ldb * 2));
    } else {
      rsA = buffer_rsrc(args.A + row0 * args.lda, (uint32_t)(min(row_end - row0, (int64_t)kBM) * args.lda * 2));
      rsB = buffer_rsrc(args.B + (int64_t)e * args.b_estride, (uint32_t)((int64_t)args.N * args.ldb * 2));
    }
    // per-lane offsets that do not depend on the K step
    uint32_t a_off[kLd], b_off[kLd];
#pragma unroll
    for (int i = 0; i < kLd; ++i) {
      if constexpr (A_MN)  // K-grouped: k row mn_k (+ 64 kt) of the group, columns m0 + c8
        a_off[i] = (uint32_t)(mn_k[i] * args.lda + m0 + mn_c8[i]) * 2u;
      else  // rows row0 + kc_row, k chunk c8 (+ 64 kt)
        a_off[i] = (uint32_t)(kc_row[i] * args.lda + kc_c8[i]) * 2u;
      if constexpr (B_MN)
        b_off[i] = (uint32_t)(mn_k[i] * args.ldb + n0 + mn_c8[i]) * 2u;
      else  // weight rows n0 + kc_row ([N, K] storage), columns past N point past the range
        b_off[i] = n0 + kc_row[i] < args.N ? (uint32_t)((n0 + kc_row[i]) * args.ldb + kc_c8[i]) * 2u : lanes::kOutOfRange;
    }
    // gathered A rows: the token of each k row of the next stage, looked up one stage ahead
    int gat[kLd];
    auto gather_rows = [&](int kt) {
      if constexpr (GATHER_A) {
#pragma unroll
        for (int i = 0; i < kLd; ++i) {
          const int64_t r = row0 + (int64_t)kt * kBK + mn_k[i];
          gat[i] = r < row_end ? args.perm[r] : -1;
        }
      }
    };
    auto issue = [&](int kt, int buf) {
      kt += kb;  // absolute K step (M-grouped split shares start at kb)
      const uint32_t st = lds_base + buf * kStage;
#pragma unroll
      for (int i = 0; i < kLd; ++i) {
        const uint32_t la = st + (wave * kLd + i) * 1024;
        if constexpr (GATHER_A) {
          const uint32_t off = gat[i] >= 0 ? (uint32_t)(((int64_t)gat[i] * args.lda + m0 + mn_c8[i]) * 2) : lanes::kOutOfRange;
          buffer_load_lds16(rsA, off, 0u, la);
        } else if constexpr (A_MN) {
          buffer_load_lds16(rsA, a_off[i], (uint32_t)kt * kBK * args.lda * 2u, la);
        } else {
          buffer_load_lds16(rsA, a_off[i], (uint32_t)kt * kBK * 2u, la);
        }
      }
#pragma unroll
      for (int i = 0; i < kLd; ++i) {
        const uint32_t lb = st + kOp + (wave * kLd + i) * 1024;
        if constexpr (B_MN)
          buffer_load_lds16(rsB, b_off[i], (uint32_t)kt * kBK * args.ldb * 2u, lb);
        else
          buffer_load_lds16(rsB, b_off[i], (uint32_t)kt * kBK * 2u, lb);
      }
    };

#pragma unroll
    for (int mi = 0; mi < kTM; ++mi)
#pragma unroll
      for (int ni = 0; ni < kTN; ++ni)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;

    if (nk > 0) {
      gather_rows(0);
      issue(0, 0);
      if (nk > 1) gather_rows(1);
    }
    // a wave whose rows all lie past its group's end (the last, partly filled
    // M tile of a row-grouped launch) skips its fragment reads and MFMAs but
    // still issues its share of the loads and joins the barriers
    auto kloop = [&](auto live_c) {
      constexpr bool LIVE = decltype(live_c)::value;
      for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        wait_vmem<0>();
        __syncthreads();  // stage kt is visible; every wave is done with buffer buf ^ 1
        if (kt + 1 < nk) {
          issue(kt + 1, buf ^ 1);
          if (kt + 2 < nk) gather_rows(kt + 2);
        }
        if constexpr (LIVE) {
          read_set(buf, 0, 0);
#pragma unroll
          for (int ks = 0; ks < kKS; ++ks) {
            const int set = ks & 1;
            if (ks + 1 < kKS) read_set(buf, ks + 1, set ^ 1);
#pragma unroll
            for (int mi = 0; mi < kTM; ++mi)
#pragma unroll
              for (int ni = 0; ni < kTN; ++ni)
                acc[mi][ni] =
                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[set][ni], fa[set][mi], acc[mi][ni], 0, 0, 0);
          }
        }
      }
    };
    if (KGROUP || row_end - row0 > wm0)
      kloop(BoolC<true>{});
    else
      kloop(BoolC<false>{});
    __syncthreads();  // every wave is done with both buffers: the ring becomes the staging area
    if (slot >= 0) {
      // ---- a split share: float32 partial sums in the accumulator layout
      // (thread-major per MFMA register group, 16 bytes per lane), the layout
      // of the forward kernel's 8-wave 256 x 256 tile that the fixup reads
      float* const dst = args.partials + (int64_t)slot * (kBM * kBN);
#pragma unroll
      for (int mi = 0; mi < kTM; ++mi)
#pragma unroll
        for (int ni = 0; ni < kTN; ++ni)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            f32x4 v;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) v[qq] = acc[mi][ni][4 * gq + qq];
            *(f32x4*)(dst + ((int64_t)((mi * kTN + ni) * 4 + gq) * (kNW * kWave) + tid) * 4) = v;
          }
      continue;  // block-uniform: every thread takes this branch together
    }

    // ---- epilogue: lane holds row (lane & 31) of MFMA tile (mi, ni), columns
    // 8 gq + 4 (lane >> 5) .. + 3; each wave stages its 128 x 64 piece as bf16
    // (row-major, 16-byte chunks XOR-swizzled by the row) and writes row segments
    constexpr int EP_ROW = kWTN * 2, EP_CH = kWTN / 8;
    lds_char* const ep = lds + wave * (kWTM * EP_ROW);
    const int64_t c_row0 = KGROUP ? m0 : row0;                       // first row of C of this tile
    const int64_t c_rows = KGROUP ? (int64_t)args.M : row_end;       // rows of C (exclusive end)
    bf16_bits* const Cb = args.C + (KGROUP ? (int64_t)e * args.M * args.N : 0);
#pragma unroll
    for (int mi = 0; mi < kTM; ++mi)
#pragma unroll
      for (int ni = 0; ni < kTN; ++ni)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          float v[4];
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) v[qq] = acc[mi][ni][4 * gq + qq];
          const int row = mi * 32 + (lane & 31);
          if constexpr (EPI == EPI_DGELU) {
            const int64_t grow = c_row0 + wm0 + row;
            const int gcol = n0 + wn0 + ni * 32 + 8 * gq + 4 * (lane >> 5);
            if (grow < c_rows && gcol < args.N) {
              const u32x2 uu = *(const u32x2*)(args.U + grow * args.N + gcol);
              v[0] *= gelu_tanh_grad(bf16_to_f32(uu[0] & 0xFFFFu));
              v[1] *= gelu_tanh_grad(bf16_to_f32(uu[0] >> 16));
              v[2] *= gelu_tanh_grad(bf16_to_f32(uu[1] & 0xFFFFu));
              v[3] *= gelu_tanh_grad(bf16_to_f32(uu[1] >> 16));
            }
          }
          u32x2 o;
          o[0] = pack_bf16x2(v[0], v[1]);
          o[1] = pack_bf16x2(v[2], v[3]);
          const int ch = ni * 4 + gq;
          *(__attribute__((address_space(3))) u32x2*)(ep + row * EP_ROW + ((ch ^ (row & (EP_CH - 1))) << 4) +
                                                        (lane >> 5) * 8) = o;
        }
    // LDS operations of one wave complete in order: its own staged rows are readable now
    const __amdgpu_buffer_rsrc_t rsC = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Cb + c_row0 * args.N), (short)0, (int)max((int64_t)0, (c_rows - c_row0) * args.N * 2), kBufferFlags);
    constexpr int ITERS = kWTM * EP_ROW / (16 * kWave);
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int idx = it * kWave + lane, row = idx / EP_CH, ch = idx % EP_CH;
      const u32x4 v = *(__attribute__((address_space(3))) u32x4*)(ep + row * EP_ROW + ((ch ^ (row & (EP_CH - 1))) << 4));
      const int n = n0 + wn0 + ch * 8;
      const int off = n < args.N ? (int)(((int64_t)(wm0 + row) * args.N + n) * 2) : 0x7FFFFFF0;
      __builtin_amdgcn_raw_buffer_store_b128(v, rsC, off, 0, 0);
    }
    __syncthreads();  // the staging area is the next tile's ring
  }
}

// Completion of the chunked tiles of a K-grouped launch: the schedule of the
// GEMM kernel (kgroup_schedule with the launch's block count nb), then, per
// (chunked tile, part of kFixParts), the tile's partial-sum slots added in
// chunk order, rounded to bf16 and stored to C_e (row and column bounds M, N).
constexpr int kFixParts = 16;
__global__ __launch_bounds__(256) void kgroup_fixup_kernel(BwdArgs args, int nb) {
  __shared__ int s_order[256];
  __shared__ int s_chunks[256];
  __shared__ int s_ibase[257];
  const int E = args.E;
  auto grp = [&](int e) -> int64_t { return args.offsets ? (int64_t)args.offsets[e] : args.R * e / E; };
  const int n_tiles = (int)ceil_div(args.N, kBN), m_fixed = (int)ceil_div(args.M, kBM), per = m_fixed * n_tiles;
  kgroup_schedule(grp, E, per, nb, args.kslots, s_order, s_chunks, s_ibase);
  int n_chunked = 0;  // the chunked experts rank first
  while (n_chunked < E && s_chunks[n_chunked] > 1) ++n_chunked;
  constexpr int ENT = kBM * kBN / 4;         // float32x4 entries per slot
  constexpr int PER = ENT / kFixParts / 256;  // entries per thread and unit
  const int units = n_chunked * per * kFixParts;
  for (int w = blockIdx.x; w < units; w += gridDim.x) {
    const int u = w / kFixParts, part = w - u * kFixParts;
    const int r = u / per, lt = u - r * per;
    const int e = s_order[r], c = s_chunks[r];
    const int nt = lt / m_fixed, mt = lt - nt * m_fixed;
    const int ebase = part * (ENT / kFixParts) + threadIdx.x;
    f32x4 acc[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int ch = 0; ch < c; ++ch) {
      const f32x4* src = (const f32x4*)(args.partials + (int64_t)(s_ibase[r] + ch * per + lt) * (kBM * kBN));
#pragma unroll
      for (int q = 0; q < PER; ++q) acc[q] += src[ebase + q * 256];
    }
    bf16_bits* const Cb = args.C + (int64_t)e * args.M * args.N;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      // entry -> (MFMA register group, thread) -> (row, 4 columns) of the tile
      const int en = ebase + q * 256, grp_ = en / kThreads, tt = en % kThreads;
      const int mi = grp_ / (kTN * 4), ni = (grp_ / 4) % kTN, gq = grp_ % 4;
      const int wave = tt / kWave, lane = tt % kWave;
      const int row = mt * kBM + (wave / kWN) * kWTM + mi * 32 + (lane & 31);
      const int col = nt * kBN + (wave % kWN) * kWTN + ni * 32 + 8 * gq + 4 * (lane >> 5);
      if (row >= args.M || col >= args.N) continue;
      u32x2 o;
      o[0] = pack_bf16x2(acc[q][0], acc[q][1]);
      o[1] = pack_bf16x2(acc[q][2], acc[q][3]);
      *(u32x2*)(Cb + (int64_t)row * args.N + col) = o;
    }
  }
}

// persistent grid: one block per CU at most, a multiple of 8 (the XCD ranges);
// MOE_GEMM_MAX_BLOCKS=<n> lowers the cap as for the forward GEMMs (several
// rounds on small problems: exercises the split of the last round)
int64_t bwd_grid(int64_t tiles) {
  int64_t slots = (int64_t)device_cus() / 8 * 8;
  const char* cap = getenv("MOE_GEMM_MAX_BLOCKS");
  if (cap && cap[0]) slots = min(slots, max((int64_t)8, (int64_t)atoi(cap) / 8 * 8));
  return max((int64_t)8, min(ceil_div(tiles, 8) * 8, slots));
}

int64_t nt_tiles_ub(int64_t R, int E, int N, bool grouped) {
  return (grouped ? (R + (int64_t)E * (kBM - 1)) / kBM : ceil_div(R, kBM)) * ceil_div(N, kBN);
}

template <bool KGROUP, bool A_MN, bool B_MN, bool GATHER_A, int EPI>
hipError_t launch(const BwdArgs& a, int64_t grid, hipStream_t s) {
  hipLaunchKernelGGL((gemm_bwd_kernel<KGROUP, A_MN, B_MN, GATHER_A, EPI>), dim3((unsigned)grid), dim3(kThreads), 0,
                     s, a);
  return hipGetLastError();
}

constexpr int kStatRowsPerSplit = 256;  // at least four K steps per split of x^T dlogit

__global__ __launch_bounds__(256) void sum_splits_kernel(const u32x4* __restrict__ part, int splits, int64_t n_vecs,
                                                         u32x4* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n_vecs; i += (int64_t)gridDim.x * 256) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int sp = 0; sp < splits; ++sp) {
      const u32x4 v = part[(int64_t)sp * n_vecs + i];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += bf16_to_f32(v[q] & 0xFFFFu);
        acc[2 * q + 1] += bf16_to_f32(v[q] >> 16);
      }
    }
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    out[i] = o;
  }
}

}  // namespace

size_t bwd_partials_bytes(int64_t R, int E, int N) {
  return (size_t)bwd_grid(nt_tiles_ub(R, E, N, true)) * 2 * kBM * kBN * sizeof(float);
}

int bwd_router_splits(int64_t T, int d, int E) {
  const int64_t per = ceil_div(d, kBM) * ceil_div(E, kBN);  // tiles of one split
  int64_t s = min((int64_t)device_cus() / per, T / kStatRowsPerSplit);
  return (int)max((int64_t)1, min(s, (int64_t)32));
}

hipError_t launch_sum_splits(const bf16_bits* part, int splits, int64_t n, bf16_bits* out, hipStream_t s) {
  if (n % 8) return hipErrorInvalidValue;
  const int64_t n_vecs = n / 8;
  hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)max((int64_t)1, min(ceil_div(n_vecs, 256), (int64_t)1024))),
                     dim3(256), 0, s, (const u32x4*)part, splits, n_vecs, (u32x4*)out);
  return hipGetLastError();
}

hipError_t launch_bwd_gemm_nt(const bf16_bits* A, int lda, const int32_t* offsets, int64_t R, int E,
                              const bf16_bits* B, int ldb, int64_t b_estride, bf16_bits* C, int N, int K,
                              const bf16_bits* U, float* partials, hipStream_t s) {
  if (K % kBK != 0 || K <= 0 || N <= 0 || lda % 8 || ldb % 8 || N % 8) return hipErrorInvalidValue;
  if (R * (int64_t)lda * 2 >= INT32_MAX || (int64_t)N * ldb * 2 >= INT32_MAX) return hipErrorInvalidValue;
  BwdArgs a{};
  a.A = A; a.B = B; a.C = C; a.U = U; a.offsets = offsets; a.perm = nullptr; a.partials = partials;
  a.R = R; a.a_rows = R; a.b_estride = b_estride;
  a.M = 0; a.N = N; a.K = K; a.lda = lda; a.ldb = ldb; a.E = E;
  const int64_t grid = bwd_grid(nt_tiles_ub(R, E, N, offsets != nullptr));
  const int nb = (int)(grid / 8);
  a.min_steps = split_min_steps();
  a.gm = group_m();
  // the split needs the fixup's tile enumeration (expert groups) and a plain epilogue
  a.max_rem = (partials && offsets && !U) ? nb / 3 : 0;
  hipError_t e = U ? launch<false, false, false, false, EPI_DGELU>(a, grid, s)
                   : launch<false, false, false, false, EPI_PLAIN>(a, grid, s);
  if (e != hipSuccess || a.max_rem == 0) return e;
  return launch_split_fixup_256(offsets, partials, C, R, K / kBK, N, E, nb, a.min_steps, a.max_rem, s);
}

hipError_t launch_bwd_gemm_tn(const bf16_bits* A, int lda, const int32_t* perm, int64_t a_rows,
                              const int32_t* offsets, int64_t R, int E, const bf16_bits* B, int ldb, bf16_bits* C,
                              int M, int N, float* partials, hipStream_t s) {
  if (M <= 0 || N <= 0 || lda % 8 || ldb % 8 || M % 8 || N % 8) return hipErrorInvalidValue;
  if ((perm ? a_rows : R) * (int64_t)lda * 2 >= INT32_MAX || R * (int64_t)ldb * 2 >= INT32_MAX)
    return hipErrorInvalidValue;
  BwdArgs a{};
  a.A = A; a.B = B; a.C = C; a.U = nullptr; a.offsets = offsets; a.perm = perm; a.partials = nullptr;
  a.R = R; a.a_rows = a_rows; a.b_estride = 0;
  a.M = M; a.N = N; a.K = 0; a.lda = lda; a.ldb = ldb; a.E = E;
  a.min_steps = 0; a.max_rem = 0;
  // chunked tiles of hot experts need the partial-sum slots (kgroup_slots)
  a.partials = offsets ? partials : nullptr;
  a.kslots = a.partials ? kgroup_slots() : 0;
  const int64_t tiles = (int64_t)E * ceil_div(M, kBM) * ceil_div(N, kBN);
  const int64_t grid = min(tiles, (int64_t)device_cus());
  if (tiles <= 0) return hipSuccess;
  hipError_t e = perm ? launch<true, true, true, true, EPI_PLAIN>(a, grid, s)
                      : launch<true, true, true, false, EPI_PLAIN>(a, grid, s);
  if (e != hipSuccess || !a.partials) return e;
  hipLaunchKernelGGL(kgroup_fixup_kernel, dim3((unsigned)device_cus()), dim3(256), 0, s, a, (int)grid);
  return hipGetLastError();
}

int kgroup_slots() {
  // MOE_BWD_KGROUP_SLOTS=<n> lowers the slot count (0: never cut a tile's reduction)
  const char* v = getenv("MOE_BWD_KGROUP_SLOTS");
  return v && v[0] ? min(max(0, atoi(v)), kKGroupSlots) : kKGroupSlots;  // the workspace holds kKGroupSlots
}

}  // namespace moe
