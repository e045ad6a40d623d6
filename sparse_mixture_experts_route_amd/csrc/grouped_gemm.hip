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
//     K step 64, four waves in a 2x2 grid, each owning (BM/2) x (BN/2);
//   * operands go HBM -> LDS with global_load_lds_dwordx4 (no register
//     staging): every lane of a wave writes 16 bytes to consecutive LDS
//     slots, and the lane's global address is chosen so that the slot holds
//     the swizzled piece;
//   * A sits K-contiguous in LDS ([row][64] bf16, 128 B per row) with the
//     16-byte chunk index XOR-ed by ((row >> 1) & 7): the LDS has 64 banks (a
//     256-byte period, two rows), and the 16 lanes served together read 16
//     consecutive rows, which this spreads over all 64 banks; fragments are
//     ds_read_b128;
//   * B stays N-contiguous in LDS ([k][BN]) with the 16-byte chunk index
//     XOR-ed by 2*(k & 3); fragments are read with ds_read_b64_tr_b16, which
//     hands each lane 4 consecutive k of one column (two reads give the 8 k
//     an MFMA lane needs), so no transpose pass is needed anywhere;
//   * two LDS stages: the loads of stage s+2 are issued right after the one
//     barrier of step s, fragments of the next K sub-step are read while the
//     MFMAs of the current one run (two fragment register sets);
//   * operands are passed to the MFMA as (B, A), so each lane's accumulators
//     hold 4 consecutive output columns of one row: the epilogue applies
//     GELU in float32, rounds to bf16 and stores 8 bytes per group;
//   * persistent blocks (one per CU): every block derives the tile list from
//     offsets[] on the device (expert by expert; inside an expert, n-tile
//     major and m-tile minor, so the tiles sharing an expert's weight slab
//     run side by side). The list is cut into 8 contiguous ranges, one per
//     XCD (the hardware deals blocks to the XCDs round robin), so each XCD's
//     L2 serves the experts it works on. Empty groups own no tiles, and no
//     host synchronisation on the routing is needed.
// float32 path: a plain LDS-tiled FMA kernel (the fp32 workload is small).
#include <stdlib.h>
#include <string.h>

#include "common.h"
#include "internal.h"

namespace moe {

namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

// dword 3 of a raw buffer descriptor on gfx9-family GPUs (32-bit data format, no swizzle)
constexpr int kBufferFlags = 0x00020000;
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor: base address, stride 0, byte range `bytes` (loads at
// or past it return zero), made wave-uniform.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xFFFFu));
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = kBufferFlags;
  return r;
}

// 16 bytes per lane from buffer offset voff + soff straight into LDS: lane i
// writes bytes [16 i, 16 i + 16) after the wave-uniform LDS address lds.
// Issued as inline assembly so that the compiler does not wait on it before
// unrelated LDS reads; the caller waits (vmcnt) before the barrier that
// publishes the data.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void buffer_load_lds16(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}
#pragma clang diagnostic pop


// LDS byte address of a shared-memory pointer, made wave-uniform
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(lds_void*)p);
}

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

// Tile list of the bf16 path: tstart[e] = first tile of expert e (exclusive
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

// Wait until at most N of this wave's vector-memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Block tile BM x BN over K steps of BK, a ring of S LDS stages, OCC blocks per CU.
template <int BM, int BN, int BK, int S, int OCC, bool GELU>
__global__ __launch_bounds__(256, OCC) void gemm_bf16_kernel(const bf16_bits* __restrict__ A,
                                                             const int32_t* __restrict__ offsets,
                                                             const bf16_bits* __restrict__ B,
                                                             bf16_bits* __restrict__ C, int64_t R, int K, int N,
                                                             int E, int n_tiles) {
  constexpr int NW = 4;                        // waves, 2 x 2
  constexpr int WTM = BM / 2, WTN = BN / 2;    // wave tile
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
  static_assert(A_LD >= 1 && B_LD >= 1 && KS >= 2 && S >= 2, "unsupported tile");
  static_assert(A_RPP * A_CH == 16, "A swizzle assumes 16 chunks per bank period");

  __shared__ __attribute__((aligned(1024))) char smem[S * STAGE];
  __shared__ int s_tstart[257];
  __shared__ int s_mtiles[256];

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  build_tile_list<BM>(offsets, E, R, n_tiles, s_tstart, s_mtiles);
  const int total = s_tstart[E];

  // contiguous share of the tile list for this block's XCD
  const int xcd = blockIdx.x % 8, nb = gridDim.x / 8, j = blockIdx.x / 8;
  const int lo = (int)((int64_t)total * xcd / 8), hi = (int)((int64_t)total * (xcd + 1) / 8);

  lds_char* const lds = (lds_char*)smem;
  const uint32_t lds_base = lds_addr(smem);
  const int wm0 = (wave >> 1) * WTM, wn0 = (wave & 1) * WTN;

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
    b_rd[ni] = A_STAGE + ((g >> 1) * 8 + kr) * B_ROW + (((col >> 3) ^ (2 * kr)) << 4) + (col & 7) * 2;
  }

  // ---- per-tile state: tile coordinates, buffer descriptors, per-lane load offsets
  struct Tile {
    int e, n0;
    int64_t row0, row_end;
    i32x4 rsA, rsB;
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
    const int n_tile = local / mt, m_idx = local - n_tile * mt;
    tl.row0 = (int64_t)__builtin_amdgcn_readfirstlane(offsets[tl.e]) + (int64_t)m_idx * BM;
    tl.row_end = min((int64_t)__builtin_amdgcn_readfirstlane(offsets[tl.e + 1]), R);
    tl.n0 = n_tile * BN;
    // A: rows row0.. of the group; rows past the group's end fall outside the
    // descriptor's range and read as zero. B: the expert's [K, N] slab.
    tl.rsA = buffer_rsrc(A + tl.row0 * K, (uint32_t)((tl.row_end - tl.row0) * K * 2));
    tl.rsB = buffer_rsrc(B + (int64_t)tl.e * K * N, (uint32_t)((int64_t)K * N * 2));
    return tl;
  };
  // per-lane byte offsets of the direct-to-LDS loads (A part does not depend on the tile)
  uint32_t a_off[A_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int p = (wave * A_LD + i) * 64 + lane;  // LDS slot
    const int row = p / A_CH, c = (p % A_CH) ^ ((row / A_RPP) & (A_CH - 1));
    a_off[i] = (uint32_t)(row * K + c * 8) * 2u;
  }
  uint32_t b_off0[B_LD];  // for n0 = 0
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int p = (wave * B_LD + i) * 64 + lane;
    const int k = p / B_SLOTS, c = (p % B_SLOTS) ^ (2 * (k & 3));
    b_off0[i] = (uint32_t)(k * N + c * 8) * 2u;
  }

  // load `i` (0 .. NL-1) of stage kt into ring buffer buf
  auto issue_one = [&](const Tile& tl, int kt, int buf, int i) {
    const uint32_t st = lds_base + buf * STAGE;
    if (i < A_LD)
      buffer_load_lds16(tl.rsA, a_off[i], (uint32_t)kt * BK * 2, st + (wave * A_LD + i) * 1024);
    else
      buffer_load_lds16(tl.rsB, b_off0[i - A_LD] + (uint32_t)tl.n0 * 2, (uint32_t)kt * BK * N * 2,
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

  const int nk = K / BK;
  constexpr int NM = TM * TN;  // MFMAs per sub-step
  constexpr int H = NM / 2;    // MFMAs of the last sub-step before the step's barrier
  // fragment reads issued after each MFMA: a set's reads all go out in the first
  // half of the sub-step, so they have landed when the next sub-step starts
  constexpr int RPM = (NR + NM / 2 - 1) / (NM / 2);

  int t = lo + j;
  Tile tl;
  if (t < hi) {
    tl = locate(t);
#pragma unroll
    for (int s2 = 0; s2 < S; ++s2)
      if (s2 < nk)
#pragma unroll
        for (int i = 0; i < NL; ++i) issue_one(tl, s2, s2, i);
  }

  for (; t < hi; t += nb) {
    // ---- stages 0 .. S-1 of this tile were issued; wait for all of them (and older stores)
    wait_vmem<0>();
    __syncthreads();
#pragma unroll
    for (int r = 0; r < NR; ++r) read_one(0, 0, 0, r);
#pragma unroll
    for (int mi = 0; mi < TM; ++mi)
#pragma unroll
      for (int ni = 0; ni < TN; ++ni)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;

    int buf = 0;
    for (int kt = 0; kt < nk; ++kt) {
      // sub-steps 0 .. KS-2: MFMAs of the current fragments, one LDS read of the next set after each
#pragma unroll
      for (int ks = 0; ks < KS - 1; ++ks) {
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          mfma_one(ks & 1, i);
#pragma unroll
          for (int u = 0; u < RPM; ++u)
            if (i * RPM + u < NR) read_one(buf, ks + 1, (ks + 1) & 1, i * RPM + u);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // last sub-step: H MFMAs, the step's barrier, then the rest of the MFMAs
      // with the refill of this buffer (stage kt+S) and the next stage's first
      // fragment reads spread between them
      constexpr int LAST = (KS - 1) & 1;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        mfma_one(LAST, i);
        __builtin_amdgcn_sched_barrier(0);
      }
      const bool more = kt + 1 < nk;
      const int nbuf = buf + 1 == S ? 0 : buf + 1;
      if (more) {
        // stage kt+1 must have landed; stages kt+2 .. kt+S-1 may still be in flight
        if (kt + S - 1 < nk)
          wait_vmem<NL * (S - 2)>();
        else
          wait_vmem<0>();
        __syncthreads();  // every wave's stage kt+1 is in; every wave is done reading `buf`
      }
      const bool refill = kt + S < nk;
#pragma unroll
      for (int i = 0; i < NM - H; ++i) {
        mfma_one(LAST, H + i);
        constexpr int PER = (NL + NR + (NM - H) - 1) / (NM - H);  // memory ops per MFMA
#pragma unroll
        for (int u = 0; u < PER; ++u) {
          // the next stage's first fragments first (needed soonest), then the refill loads
          const int op = i * PER + u;
          if (op < NR) {
            if (more) read_one(nbuf, 0, 0, op);
          } else if (op < NR + NL) {
            if (refill) issue_one(tl, kt + S, buf, op - NR);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      buf = nbuf;
    }
    __syncthreads();  // every wave is done with every buffer

    // ---- the next tile's first stages go out before this tile's epilogue
    const Tile cur = tl;
    if (t + nb < hi) {
      tl = locate(t + nb);
#pragma unroll
      for (int s2 = 0; s2 < S; ++s2)
        if (s2 < nk)
#pragma unroll
          for (int i = 0; i < NL; ++i) issue_one(tl, s2, s2, i);
    }

    // ---- epilogue: lane holds row (lane & 31) of each MFMA tile, columns 8g + 4*(lane>>5) + 0..3
#pragma unroll
    for (int mi = 0; mi < TM; ++mi) {
      const int64_t row = cur.row0 + wm0 + mi * 32 + (lane & 31);
      if (row >= cur.row_end) continue;
      bf16_bits* crow = C + row * N;
#pragma unroll
      for (int ni = 0; ni < TN; ++ni)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int n = cur.n0 + wn0 + ni * 32 + 8 * gq + 4 * (lane >> 5);
          if (n >= N) continue;
          float v[4];
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            v[qq] = acc[mi][ni][4 * gq + qq];
            if (GELU) v[qq] = gelu_tanh(v[qq]);
          }
          u32x2 o;
          o[0] = pack_bf16x2(v[0], v[1]);
          o[1] = pack_bf16x2(v[2], v[3]);
          *(u32x2*)(crow + n) = o;
        }
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

int device_cus() {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
  }
  return cus;
}

// Tile configurations of the bf16 path.
//   0: 256 x 256, K step 64, 2 stages (128 KB LDS), one block per CU
//   1: 256 x 128, K step 32, 3 stages (72 KB LDS), two blocks per CU
//   2: 128 x 128, K step 64, 2 stages (64 KB LDS), two blocks per CU
struct TileShape {
  int bm, bn, occ;
};
constexpr TileShape kShapes[3] = {{256, 256, 1}, {256, 128, 2}, {128, 128, 2}};

template <int BM, int BN, int BK, int S, int OCC>
hipError_t launch_bf16(const void* A, const int32_t* offsets, const void* B, void* C, int64_t R, int K, int N,
                       int E, bool gelu, hipStream_t s) {
  const int n_tiles = (int)ceil_div(N, BN);
  const int64_t m_tiles = (R + (int64_t)E * (BM - 1)) / BM;  // >= sum over experts of ceil(rows_e / BM)
  const int64_t tiles_ub = m_tiles * n_tiles;
  if (tiles_ub > INT32_MAX) return hipErrorInvalidValue;
  // persistent grid: OCC blocks per CU, a multiple of 8 so every XCD holds the same number of blocks
  const int64_t slots = (int64_t)device_cus() / 8 * 8 * OCC;
  const int64_t grid = max((int64_t)8, min(ceil_div(tiles_ub, 8) * 8, slots));
  if (gelu)
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BK, S, OCC, true>), dim3((unsigned)grid), dim3(256), 0, s,
                       (const bf16_bits*)A, offsets, (const bf16_bits*)B, (bf16_bits*)C, R, K, N, E, n_tiles);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BK, S, OCC, false>), dim3((unsigned)grid), dim3(256), 0, s,
                       (const bf16_bits*)A, offsets, (const bf16_bits*)B, (bf16_bits*)C, R, K, N, E, n_tiles);
  return hipGetLastError();
}

// Block tile for a GEMM: fewer, larger tiles use the matrix cores better, but
// a last partial round of tiles over the block slots and padding rows of
// half-empty M tiles cost time. MOE_GEMM_TILE=256x256|256x128|128x128 forces a shape.
int pick_tile(int64_t R, int N, int E) {
  const char* force = getenv("MOE_GEMM_TILE");
  if (force && force[0]) {
    if (!strcmp(force, "256x256")) return 0;
    if (!strcmp(force, "256x128")) return 1;
    if (!strcmp(force, "128x128")) return 2;
  }
  const double tile_eff[3] = {0.9, 1.0, 0.8};  // relative matrix-core efficiency of a busy CU
  const double cus = device_cus();
  int best = 0;
  double best_score = -1.0;
  for (int c = 0; c < 3; ++c) {
    const TileShape& ts = kShapes[c];
    const double m_tiles = (double)R / ts.bm + 0.5 * E;
    const double tiles = m_tiles * ceil_div(N, ts.bn);
    const double rounds = tiles / (cus * ts.occ);
    const double round_eff = rounds / (double)(int64_t)(rounds + 0.999);
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
      return launch_bf16<256, 256, 64, 2, 1>(A, offsets, B, C, R, K, N, E, gelu, s);
    case 1:
      return launch_bf16<256, 128, 32, 3, 2>(A, offsets, B, C, R, K, N, E, gelu, s);
    default:
      return launch_bf16<128, 128, 64, 2, 2>(A, offsets, B, C, R, K, N, E, gelu, s);
  }
}

}  // namespace moe
