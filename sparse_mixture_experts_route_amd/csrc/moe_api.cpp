// C ABI of the MoE layer forward: argument checks, workspace layout and
// launch order. Every check runs on the host before anything is enqueued.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cstring>
#include <mutex>

#include "internal.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kAlign = 256;

inline bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

inline size_t elem_size(int32_t dtype) { return dtype == MOE_DTYPE_BF16 ? 2 : 4; }

moe_status_t check_problem(const moe_problem_t* p) {
  if (!p) return MOE_ERR_INVALID_ARGUMENT;
  if (p->dtype != MOE_DTYPE_F32 && p->dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARGUMENT;
  if (p->T < 1 || p->E < 1 || p->k < 1 || p->k > p->E || p->d_model < 1 || p->d_expert < 1)
    return MOE_ERR_INVALID_ARGUMENT;
  if (p->E > 256) return MOE_ERR_UNSUPPORTED;
  if (p->T > (int64_t)INT32_MAX / p->k) return MOE_ERR_UNSUPPORTED;
  if (p->d_model % 64 != 0 || p->d_expert % 64 != 0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Sequential sub-allocation of a caller-provided workspace (or size counting when base is null).
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <typename T>
  T* take(size_t n) {
    off = (off + kAlign - 1) / kAlign * kAlign;
    T* ptr = base ? (T*)(base + off) : nullptr;
    off += n * sizeof(T);
    return ptr;
  }
};

struct PermuteWs {
  int32_t* blockcounts;
  int32_t* blockbase;
};

PermuteWs carve_permute(Carver& c, const moe_problem_t& p) {
  const size_t n = (size_t)moe::permute_blocks(p.T) * (size_t)p.E;
  PermuteWs w;
  w.blockcounts = c.take<int32_t>(n);
  w.blockbase = c.take<int32_t>(n);
  return w;
}

struct FfnWs {
  void* h;            // hidden activations [T*k, d_expert]
  float* partials;    // split-tile partial sums of either GEMM
  int32_t* counters;  // split-tile counters of either GEMM (zero between launches)
};

// whether the grouped GEMMs of the layer complete split tiles with counters
// that must be zero when they start
bool ffn_uses_counters(const moe_problem_t& p) {
  const int64_t R = p.T * p.k;
  return moe::grouped_gemm_uses_counters(p.dtype, R, p.d_model, p.d_expert, p.E, true) ||
         moe::grouped_gemm_uses_counters(p.dtype, R, p.d_expert, p.d_model, p.E, false);
}

FfnWs carve_ffn(Carver& c, const moe_problem_t& p) {
  const int64_t R = p.T * p.k;
  FfnWs w;
  w.counters = c.take<int32_t>(moe::kGemmSplitCounters);
  w.h = c.take<char>((size_t)R * p.d_expert * elem_size(p.dtype));
  const size_t pb = std::max(moe::grouped_gemm_partials_bytes(p.dtype, R, p.d_model, p.d_expert, p.E),
                             moe::grouped_gemm_partials_bytes(p.dtype, R, p.d_expert, p.d_model, p.E));
  w.partials = c.take<float>(pb / sizeof(float));
  return w;
}

// float32 partial logits of a router split over d_model (none when unsplit)
float* carve_route(Carver& c, const moe_problem_t& p) {
  const size_t n = moe::route_partials_bytes(p) / sizeof(float);
  return n ? c.take<float>(n) : nullptr;
}

struct ForwardWs {
  int32_t *idx, *counts, *offsets, *perm, *inv;
  float *gate, *route_part;
  PermuteWs pw;
  FfnWs fw;
  void *x_perm, *y_perm;
};

ForwardWs carve_forward(Carver& c, const moe_problem_t& p) {
  const size_t R = (size_t)p.T * p.k;
  const size_t es = elem_size(p.dtype);
  ForwardWs w;
  w.idx = c.take<int32_t>(R);
  w.gate = c.take<float>(R);
  w.counts = c.take<int32_t>(p.E);
  w.offsets = c.take<int32_t>(p.E + 1);
  w.perm = c.take<int32_t>(R);
  w.inv = c.take<int32_t>(R);
  w.pw = carve_permute(c, p);
  w.route_part = carve_route(c, p);
  w.x_perm = c.take<char>(R * p.d_model * es);
  w.fw = carve_ffn(c, p);
  w.y_perm = c.take<char>(R * p.d_model * es);
  return w;
}

// Training: what moe_forward_train keeps for moe_backward, then the backward's own buffers.
struct TrainWs {
  float *logits, *gate;                              // [T, E], [T, k]
  int32_t *idx, *counts, *offsets, *perm, *inv;
  void *U, *H, *y_perm;                              // [R, d_expert] x2, [R, d_model] (bf16)
  PermuteWs pw;
  float *route_part, *partials;
  int32_t* counters;                                 // split-tile counters of the forward GEMMs
  uint16_t* dwr_part;                                // [splits, d, E] bf16: x^T dlogit per token split
  void *dYp, *dU, *dXp, *dxr;                        // [R, d], [R, de], [R, d], [T, d] (bf16)
  float *dlogit, *prob, *stat_part;                  // [T, E], [T, E], [chunks, 2, E]
  uint16_t* dlogit_b;                                // [T, E64] bf16, zero columns past E
};

inline int padded_experts(const moe_problem_t& p) { return (p.E + 63) / 64 * 64; }

TrainWs carve_train(Carver& c, const moe_problem_t& p) {
  const size_t R = (size_t)p.T * p.k, T = (size_t)p.T;
  TrainWs w;
  w.logits = c.take<float>(T * p.E);
  w.gate = c.take<float>(R);
  w.idx = c.take<int32_t>(R);
  w.counts = c.take<int32_t>(p.E);
  w.offsets = c.take<int32_t>(p.E + 1);
  w.perm = c.take<int32_t>(R);
  w.inv = c.take<int32_t>(R);
  w.U = c.take<uint16_t>(R * p.d_expert);
  w.H = c.take<uint16_t>(R * p.d_expert);
  w.y_perm = c.take<uint16_t>(R * p.d_model);
  w.pw = carve_permute(c, p);
  w.route_part = carve_route(c, p);
  // one region for the split partial sums of every GEMM of the step, used in turn
  const size_t pb = std::max({moe::grouped_gemm_partials_bytes(p.dtype, (int64_t)R, p.d_model, p.d_expert, p.E),
                              moe::grouped_gemm_partials_bytes(p.dtype, (int64_t)R, p.d_expert, p.d_model, p.E),
                              moe::bwd_partials_bytes((int64_t)R, p.E, p.d_model),
                              (size_t)moe::kKGroupSlots * 256 * 256 * sizeof(float)});
  w.partials = c.take<float>(pb / sizeof(float));
  w.counters = c.take<int32_t>(moe::kGemmSplitCounters);
  w.dwr_part = c.take<uint16_t>((size_t)moe::bwd_router_splits(p.T, p.d_model, p.E) * p.d_model * p.E);
  w.dYp = c.take<uint16_t>(R * p.d_model);
  w.dU = c.take<uint16_t>(R * p.d_expert);
  w.dXp = c.take<uint16_t>(R * p.d_model);
  w.dxr = c.take<uint16_t>(T * p.d_model);
  w.dlogit = c.take<float>(T * p.E);
  w.prob = c.take<float>(T * p.E);
  w.stat_part = c.take<float>((size_t)moe::bwd_stat_chunks(p.T) * 2 * p.E);
  w.dlogit_b = c.take<uint16_t>(T * padded_experts(p));
  return w;
}

size_t stage_bytes(const moe_problem_t& p, int32_t stage) {
  Carver c(nullptr);
  switch (stage) {
    case MOE_STAGE_PERMUTE:
      carve_permute(c, p);
      break;
    case MOE_STAGE_GROUPED_FFN:
      carve_ffn(c, p);
      break;
    case MOE_STAGE_ROUTE:
      carve_route(c, p);
      break;
    case MOE_STAGE_TRAIN:
      carve_train(c, p);
      break;
    default:
      carve_forward(c, p);
      break;
  }
  return c.off + kAlign;  // slack so a 16-byte aligned base can be rounded up to kAlign
}

inline char* align_ws(void* ws) { return (char*)(((uintptr_t)ws + kAlign - 1) / kAlign * kAlign); }

inline moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// The first GEMM reads x rows through perm with 32-bit byte offsets into x
// (bf16 path only).
inline bool gather_supported(const moe_problem_t& p) {
  return p.dtype == MOE_DTYPE_BF16 && p.T * (int64_t)p.d_model * 2 < (int64_t)INT32_MAX;
}

}  // namespace

MOE_API moe_status_t moe_workspace_size(const moe_problem_t* p, int32_t stage, size_t* bytes) {
  const moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
  if (stage != MOE_STAGE_PERMUTE && stage != MOE_STAGE_GROUPED_FFN && stage != MOE_STAGE_FORWARD &&
      stage != MOE_STAGE_ROUTE && stage != MOE_STAGE_TRAIN)
    return MOE_ERR_INVALID_ARGUMENT;
  *bytes = stage_bytes(*p, stage);
  return MOE_OK;
}

MOE_API moe_status_t moe_route(const moe_problem_t* p, const void* x, const void* w_router,
                               const float* router_bias, float* logits, int32_t* topk_idx, float* topk_gate,
                               void* stream) {
  const moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!x || !w_router || !topk_idx || !topk_gate) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(topk_idx) || !aligned16(topk_gate) ||
      (router_bias && !aligned16(router_bias)) || (logits && !aligned16(logits)))
    return MOE_ERR_INVALID_ARGUMENT;
  return hip_status(moe::launch_route(*p, x, w_router, router_bias, logits, topk_idx, topk_gate, nullptr,
                                      (hipStream_t)stream));
}

MOE_API moe_status_t moe_route_ws(const moe_problem_t* p, const void* x, const void* w_router,
                                  const float* router_bias, float* logits, int32_t* topk_idx, float* topk_gate,
                                  void* ws, size_t ws_bytes, void* stream) {
  const moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!x || !w_router || !topk_idx || !topk_gate || !ws) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(topk_idx) || !aligned16(topk_gate) || !aligned16(ws) ||
      (router_bias && !aligned16(router_bias)) || (logits && !aligned16(logits)))
    return MOE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < stage_bytes(*p, MOE_STAGE_ROUTE)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  Carver c(align_ws(ws));
  float* part = carve_route(c, *p);
  return hip_status(moe::launch_route(*p, x, w_router, router_bias, logits, topk_idx, topk_gate, part,
                                      (hipStream_t)stream));
}

MOE_API moe_status_t moe_permute(const moe_problem_t* p, const int32_t* topk_idx, const void* x, int32_t* counts,
                                 int32_t* offsets, int32_t* perm, int32_t* inv, void* x_perm, void* ws,
                                 size_t ws_bytes, void* stream) {
  const moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!topk_idx || !x || !counts || !offsets || !perm || !inv || !x_perm || !ws) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(topk_idx) || !aligned16(x) || !aligned16(counts) || !aligned16(offsets) || !aligned16(perm) ||
      !aligned16(inv) || !aligned16(x_perm) || !aligned16(ws))
    return MOE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < stage_bytes(*p, MOE_STAGE_PERMUTE)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  Carver c(align_ws(ws));
  const PermuteWs w = carve_permute(c, *p);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = moe::launch_permute_index(*p, topk_idx, counts, offsets, perm, inv, w.blockcounts, w.blockbase, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(moe::launch_gather(*p, x, inv, x_perm, s));
}

MOE_API moe_status_t moe_permute_index(const moe_problem_t* p, const int32_t* topk_idx, int32_t* counts,
                                       int32_t* offsets, int32_t* perm, int32_t* inv, void* ws, size_t ws_bytes,
                                       void* stream) {
  const moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!topk_idx || !counts || !offsets || !perm || !inv || !ws) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(topk_idx) || !aligned16(counts) || !aligned16(offsets) || !aligned16(perm) || !aligned16(inv) ||
      !aligned16(ws))
    return MOE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < stage_bytes(*p, MOE_STAGE_PERMUTE)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  Carver c(align_ws(ws));
  const PermuteWs w = carve_permute(c, *p);
  return hip_status(moe::launch_permute_index(*p, topk_idx, counts, offsets, perm, inv, w.blockcounts,
                                              w.blockbase, (hipStream_t)stream));
}

MOE_API moe_status_t moe_grouped_ffn_gather(const moe_problem_t* p, const void* x, const int32_t* perm,
                                            const int32_t* offsets, const void* W1, const void* W2, void* y_perm,
                                            void* ws, size_t ws_bytes, void* stream) {
  const moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!x || !perm || !offsets || !W1 || !W2 || !y_perm || !ws) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(perm) || !aligned16(offsets) || !aligned16(W1) || !aligned16(W2) ||
      !aligned16(y_perm) || !aligned16(ws))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!gather_supported(*p)) return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < stage_bytes(*p, MOE_STAGE_GROUPED_FFN)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  Carver c(align_ws(ws));
  const FfnWs fw = carve_ffn(c, *p);
  hipStream_t s = (hipStream_t)stream;
  const int64_t R = p->T * p->k;
  hipError_t e = ffn_uses_counters(*p) ? moe::launch_zero_i32(fw.counters, moe::kGemmSplitCounters, s) : hipSuccess;
  if (e == hipSuccess)
    e = moe::launch_grouped_gemm(p->dtype, x, offsets, W1, fw.h, fw.partials, fw.counters, R, p->d_model,
                                 p->d_expert, p->E, true, s, perm, p->T);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(moe::launch_grouped_gemm(p->dtype, fw.h, offsets, W2, y_perm, fw.partials, fw.counters, R,
                                             p->d_expert, p->d_model, p->E, false, s));
}

MOE_API moe_status_t moe_grouped_ffn(const moe_problem_t* p, const void* x_perm, const int32_t* offsets,
                                     const void* W1, const void* W2, void* y_perm, void* ws, size_t ws_bytes,
                                     void* stream) {
  const moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!x_perm || !offsets || !W1 || !W2 || !y_perm || !ws) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x_perm) || !aligned16(offsets) || !aligned16(W1) || !aligned16(W2) || !aligned16(y_perm) ||
      !aligned16(ws))
    return MOE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < stage_bytes(*p, MOE_STAGE_GROUPED_FFN)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  Carver c(align_ws(ws));
  const FfnWs fw = carve_ffn(c, *p);
  hipStream_t s = (hipStream_t)stream;
  const int64_t R = p->T * p->k;
  hipError_t e = ffn_uses_counters(*p) ? moe::launch_zero_i32(fw.counters, moe::kGemmSplitCounters, s) : hipSuccess;
  if (e == hipSuccess)
    e = moe::launch_grouped_gemm(p->dtype, x_perm, offsets, W1, fw.h, fw.partials, fw.counters, R, p->d_model,
                                 p->d_expert, p->E, true, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(moe::launch_grouped_gemm(p->dtype, fw.h, offsets, W2, y_perm, fw.partials, fw.counters, R,
                                             p->d_expert, p->d_model, p->E, false, s));
}

MOE_API moe_status_t moe_combine(const moe_problem_t* p, const void* y_perm, const int32_t* inv,
                                 const float* topk_gate, void* y, void* stream) {
  const moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!y_perm || !inv || !topk_gate || !y) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(y_perm) || !aligned16(inv) || !aligned16(topk_gate) || !aligned16(y))
    return MOE_ERR_INVALID_ARGUMENT;
  return hip_status(moe::launch_combine(*p, y_perm, inv, topk_gate, y, (hipStream_t)stream));
}

MOE_API moe_status_t moe_forward(const moe_problem_t* p, const void* x, const void* w_router,
                                 const float* router_bias, const void* W1, const void* W2, void* y, void* ws,
                                 size_t ws_bytes, void* stream) {
  const moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!x || !w_router || !W1 || !W2 || !y || !ws) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(W1) || !aligned16(W2) || !aligned16(y) ||
      !aligned16(ws) || (router_bias && !aligned16(router_bias)))
    return MOE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < stage_bytes(*p, MOE_STAGE_FORWARD)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = (hipStream_t)stream;
  // a small float32 layer: one launch, one workgroup per token
  if (moe::small_layer_fused(*p))
    return hip_status(moe::launch_small_layer(*p, x, w_router, router_bias, W1, W2, y, s));
  Carver c(align_ws(ws));
  const ForwardWs w = carve_forward(c, *p);
  const int64_t R = p->T * p->k;
  hipError_t e;
  if (moe::route_permute_fused(*p)) {
    // decode-sized batch: router partial logits, then one workgroup completes
    // the routing and permutes (the same results as the two stages)
    e = moe::launch_route_partials(*p, x, w_router, w.route_part, s);
    if (e == hipSuccess)
      e = moe::launch_finalize_permute_small(*p, w.route_part, moe::route_splits(*p), router_bias, w.idx, w.gate,
                                             w.counts, w.offsets, w.perm, w.inv, s, w.fw.counters,
                                             moe::kGemmSplitCounters);
  } else {
    e = moe::launch_route(*p, x, w_router, router_bias, nullptr, w.idx, w.gate, w.route_part, s);
    if (e == hipSuccess)
      e = moe::launch_permute_index(*p, w.idx, w.counts, w.offsets, w.perm, w.inv, w.pw.blockcounts,
                                    w.pw.blockbase, s, w.fw.counters, moe::kGemmSplitCounters);
  }
  // (the permute launch also cleared the GEMMs' split-tile counters)
  if (gather_supported(*p)) {
    // dispatch folded into the first GEMM: its A rows are read as x[perm[r]]
    if (e == hipSuccess)
      e = moe::launch_grouped_gemm(p->dtype, x, w.offsets, W1, w.fw.h, w.fw.partials, w.fw.counters, R, p->d_model,
                                   p->d_expert, p->E, true, s, w.perm, p->T);
  } else {
    if (e == hipSuccess) e = moe::launch_gather(*p, x, w.inv, w.x_perm, s);
    if (e == hipSuccess)
      e = moe::launch_grouped_gemm(p->dtype, w.x_perm, w.offsets, W1, w.fw.h, w.fw.partials, w.fw.counters, R,
                                   p->d_model, p->d_expert, p->E, true, s);
  }
  if (e == hipSuccess)
    e = moe::launch_grouped_gemm(p->dtype, w.fw.h, w.offsets, W2, w.y_perm, w.fw.partials, w.fw.counters, R,
                                 p->d_expert, p->d_model, p->E, false, s);
  if (e == hipSuccess) e = moe::launch_combine(*p, w.y_perm, w.inv, w.gate, y, s);
  return hip_status(e);
}

// Training path: bf16, x addressable by the gathering GEMMs, k <= 8, E a multiple of 8.
inline bool train_supported(const moe_problem_t& p) {
  return gather_supported(p) && p.k <= 8 && p.E % 8 == 0;
}

MOE_API moe_status_t moe_forward_train(const moe_problem_t* p, const void* x, const void* w_router,
                                       const float* router_bias, const void* W1, const void* W2, void* y, void* ws,
                                       size_t ws_bytes, void* stream) {
  const moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!x || !w_router || !W1 || !W2 || !y || !ws) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(W1) || !aligned16(W2) || !aligned16(y) ||
      !aligned16(ws) || (router_bias && !aligned16(router_bias)))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!train_supported(*p)) return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < stage_bytes(*p, MOE_STAGE_TRAIN)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  Carver c(align_ws(ws));
  const TrainWs w = carve_train(c, *p);
  hipStream_t s = (hipStream_t)stream;
  const int64_t R = p->T * p->k;
  hipError_t e = moe::launch_route(*p, x, w_router, router_bias, w.logits, w.idx, w.gate, w.route_part, s);
  if (e == hipSuccess)
    e = moe::launch_permute_index(*p, w.idx, w.counts, w.offsets, w.perm, w.inv, w.pw.blockcounts,
                                  w.pw.blockbase, s, w.counters, moe::kGemmSplitCounters);
  // U = x W1 per expert (rows read through perm), kept; H = GELU_tanh(U)
  if (e == hipSuccess)
    e = moe::launch_grouped_gemm(p->dtype, x, w.offsets, W1, w.U, w.partials, w.counters, R, p->d_model,
                                 p->d_expert, p->E, false, s, w.perm, p->T);
  if (e == hipSuccess) e = moe::launch_gelu_rows(w.U, w.H, R * p->d_expert, s);
  if (e == hipSuccess)
    e = moe::launch_grouped_gemm(p->dtype, w.H, w.offsets, W2, w.y_perm, w.partials, w.counters, R, p->d_expert,
                                 p->d_model, p->E, false, s);
  if (e == hipSuccess) e = moe::launch_combine(*p, w.y_perm, w.inv, w.gate, y, s);
  return hip_status(e);
}

MOE_API moe_status_t moe_backward(const moe_problem_t* p, const void* x, const void* w_router, const void* W1,
                                  const void* W2, const void* dy, void* dx, void* dw_router, float* dbias,
                                  void* dW1, void* dW2, float* load_frac, float* mean_prob, void* ws,
                                  size_t ws_bytes, void* stream) {
  const moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!x || !w_router || !W1 || !W2 || !dy || !dx || !dw_router || !dW1 || !dW2 || !ws)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(W1) || !aligned16(W2) || !aligned16(dy) ||
      !aligned16(dx) || !aligned16(dw_router) || !aligned16(dW1) || !aligned16(dW2) || !aligned16(ws) ||
      (dbias && !aligned16(dbias)) || (load_frac && !aligned16(load_frac)) || (mean_prob && !aligned16(mean_prob)))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!train_supported(*p)) return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < stage_bytes(*p, MOE_STAGE_TRAIN)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  Carver c(align_ws(ws));
  const TrainWs w = carve_train(c, *p);
  hipStream_t s = (hipStream_t)stream;
  const int64_t R = p->T * p->k;
  const int d = p->d_model, de = p->d_expert, Ep = padded_experts(*p);
  typedef const uint16_t* cb;
  hipError_t e = moe::launch_bwd_combine(*p, dy, w.gate, w.idx, w.inv, w.y_perm, w.logits, w.dYp, w.dlogit,
                                         w.dlogit_b, w.prob, Ep, s);
  // dU = (dYp W2_e^T) * GELU_tanh'(U), dX = dU W1_e^T
  if (e == hipSuccess)
    e = moe::launch_bwd_gemm_nt((cb)w.dYp, d, w.offsets, R, p->E, (cb)W2, d, (int64_t)de * d, (uint16_t*)w.dU, de,
                                d, (cb)w.U, nullptr, s);
  if (e == hipSuccess)
    e = moe::launch_bwd_gemm_nt((cb)w.dU, de, w.offsets, R, p->E, (cb)W1, de, (int64_t)d * de, (uint16_t*)w.dXp, d,
                                de, nullptr, w.partials, s);
  // dW2_e = H^T dYp, dW1_e = x[perm]^T dU over each expert's rows
  if (e == hipSuccess)
    e = moe::launch_bwd_gemm_tn((cb)w.H, de, nullptr, R, w.offsets, R, p->E, (cb)w.dYp, d, (uint16_t*)dW2, de, d,
                                w.partials, s);
  if (e == hipSuccess)
    e = moe::launch_bwd_gemm_tn((cb)x, d, w.perm, p->T, w.offsets, R, p->E, (cb)w.dU, de, (uint16_t*)dW1, d, de,
                                w.partials, s);
  // router: dx_r = dlogit W_r^T, dW_r = x^T dlogit (one group of T rows)
  if (e == hipSuccess)
    e = moe::launch_bwd_gemm_nt(w.dlogit_b, Ep, nullptr, p->T, 1, (cb)w_router, p->E, 0, (uint16_t*)w.dxr, d, Ep,
                                nullptr, nullptr, s);
  // x^T dlogit over `splits` equal token ranges (one tile row each would leave
  // most CUs idle), then the bf16 partial products added in split order
  const int splits = moe::bwd_router_splits(p->T, d, p->E);
  if (e == hipSuccess)
    e = moe::launch_bwd_gemm_tn((cb)x, d, nullptr, p->T, nullptr, p->T, splits, w.dlogit_b, Ep,
                                splits > 1 ? w.dwr_part : (uint16_t*)dw_router, d, p->E, nullptr, s);
  if (e == hipSuccess && splits > 1)
    e = moe::launch_sum_splits(w.dwr_part, splits, (int64_t)d * p->E, (uint16_t*)dw_router, s);
  if (e == hipSuccess) e = moe::launch_bwd_dx(*p, w.dXp, w.inv, w.dxr, dx, s);
  if (e == hipSuccess && (dbias || load_frac || mean_prob))
    e = moe::launch_bwd_stats(*p, w.prob, w.dlogit, w.counts, w.stat_part, load_frac, mean_prob, dbias, s);
  return hip_status(e);
}

MOE_API moe_status_t moe_plan(const moe_problem_t* p, const int32_t* host_counts, moe_plan_t* plan) {
  const moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!plan) return MOE_ERR_INVALID_ARGUMENT;
  if (host_counts)
    for (int e = 0; e < p->E; ++e)
      if (host_counts[e] < 0) return MOE_ERR_INVALID_ARGUMENT;
  moe_plan_t out;
  memset(&out, 0, sizeof(out));
  out.route_splits = moe::route_splits(*p);
  out.route_tokens_per_block = moe::route_rt(*p);
  out.route_fused_permute = moe::route_permute_fused(*p) ? 1 : 0;
  out.permute_form = moe::permute_form(*p);
  out.gather_in_gemm = gather_supported(*p) ? 1 : 0;
  out.combine_streaming = moe::combine_streams(*p) ? 1 : 0;
  out.forward_one_launch = moe::small_layer_fused(*p) ? 1 : 0;
  const int64_t R = p->T * p->k;
  for (int i = 0; i < 2; ++i) {
    moe_gemm_plan_t& g = out.gemm[i];
    if (p->dtype != MOE_DTYPE_BF16) {
      memset(&g, 0xff, sizeof(g));  // every field -1: the float32 path has no persistent plan
      continue;
    }
    const int K = i == 0 ? p->d_model : p->d_expert, N = i == 0 ? p->d_expert : p->d_model;
    const moe::GemmGeom geo = moe::gemm_geom(R, K, N, p->E, i == 0);
    g.tile = geo.shape;
    g.bm = geo.bm;
    g.bn = geo.bn;
    g.bk = geo.bk;
    g.grid = geo.grid;
    g.k_steps = geo.nk;
    g.max_split = geo.max_rem;
    g.min_steps = geo.min_steps;
    g.split_in_launch = geo.in_launch ? 1 : 0;
    g.tiles = -1;
    g.xcd_rounds = g.xcd_leftover = g.xcd_split = g.split_xcds = -1;
    if (host_counts) {
      moe::GemmXcdPlan xp;
      moe::gemm_xcd_plan(geo, host_counts, p->E, &xp);
      g.tiles = xp.tiles;
      g.xcd_rounds = xp.full;
      g.xcd_leftover = xp.rem;
      g.xcd_split = xp.split;
      g.split_xcds = xp.split_xcds;
    }
  }
  *plan = out;
  return MOE_OK;
}

// ---- the index permute without a workspace argument

namespace {

// Per-block counts and per-block first rows of the counting sort (kNoAllocSlots
// int32 each) in device memory of the library itself: each GPU the library
// runs on holds its own copy until the process ends. In host code `scratch`
// names a host-side stand-in; kernels get the device address that
// hipGetSymbolAddress returns for the current device.
constexpr int64_t kNoAllocSlots = MOE_NOALLOC_PERMUTE_SLOTS;
static __device__ __align__(256) int32_t scratch[2 * kNoAllocSlots];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch[kMaxDevices];  // device address of `scratch` per device, looked up once

// Device address of `scratch` on the current device (looked up on the first
// call made with that device current).
hipError_t device_scratch(int32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
    g_scratch[dev] = (int32_t*)ptr;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

MOE_API moe_status_t moe_permute_index_noalloc(const moe_problem_t* p, const int32_t* topk_idx, int32_t* counts,
                                               int32_t* offsets, int32_t* perm, int32_t* inv, void* stream) {
  const moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!topk_idx || !counts || !offsets || !perm || !inv) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(topk_idx) || !aligned16(counts) || !aligned16(offsets) || !aligned16(perm) || !aligned16(inv))
    return MOE_ERR_INVALID_ARGUMENT;
  if (moe::permute_blocks(p->T) * (int64_t)p->E > kNoAllocSlots) return MOE_ERR_WORKSPACE_TOO_SMALL;
  int32_t* base = nullptr;
  if (device_scratch(&base) != hipSuccess) return MOE_ERR_HIP;
  // the kernels overwrite both arrays before reading them: nothing to clear
  return hip_status(moe::launch_permute_index(*p, topk_idx, counts, offsets, perm, inv, base, base + kNoAllocSlots,
                                              (hipStream_t)stream));
}

MOE_API const char* moe_status_str(int32_t status) {
  switch (status) {
    case MOE_OK:
      return "ok";
    case MOE_ERR_INVALID_ARGUMENT:
      return "invalid argument";
    case MOE_ERR_UNSUPPORTED:
      return "unsupported problem (outside the library's contract)";
    case MOE_ERR_WORKSPACE_TOO_SMALL:
      return "workspace too small";
    case MOE_ERR_HIP:
      return "HIP runtime error";
    default:
      return "unknown status";
  }
}
