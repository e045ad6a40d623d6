/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse Mixture-of-Experts layer forward.
 *
 * The layer (from "Distributed training part 4", jesamkim's AI tech blog,
 * section 3 "Mixture of Experts" and section 4 "Expert Parallelism"):
 *   router: a Linear layer followed by a Softmax over the E experts;
 *   selection: the k experts with the largest router output per token;
 *   dispatch: each token goes to the experts it selected;
 *   experts: E independent FFNs, E_i(x) = GELU_tanh(x W1_i) W2_i (no biases);
 *   combine: y = sum over the selected i of G(x)_i * E_i(x), where G(x)_i is
 *            the router probability of expert i.
 * All experts live on one GPU, so dispatch and combine are a local permutation
 * (rows grouped by expert) and its inverse gather.
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers to row-major, contiguous buffers,
 *     16-byte aligned. `p` is a HOST pointer, read during the call only.
 *   - Ownership: the caller owns every buffer and the workspace. The library
 *     allocates no device memory, keeps no pointer after returning, never
 *     writes its inputs and fully overwrites its outputs (no accumulation).
 *   - Asynchrony: each call only enqueues kernels on `stream` (a hipStream_t;
 *     NULL is the null stream) and returns; it never synchronizes and never
 *     copies device data to the host. Results are ready once the stream
 *     reaches that point. Calls on different streams that share no output or
 *     workspace buffer may run concurrently: the library has no global
 *     mutable state.
 *   - Errors: all argument checks run on the host before anything is
 *     enqueued; on any error nothing is written. A failed kernel launch
 *     returns MOE_ERR_HIP. Faults during execution show at the caller's next
 *     synchronization. No C++ exception crosses this interface.
 *   - Contract: T >= 1; 1 <= k <= E <= 256; T*k <= INT32_MAX; d_model and
 *     d_expert are multiples of 64. The dtype of x, w_router, W1, W2, x_perm,
 *     y_perm and y is p->dtype. Logits, gates and the router bias are float32;
 *     indices, counts and offsets are int32. Inputs must be finite.
 *   - Routing rule: selection is made on the float32 logits, in descending
 *     order, ties going to the lower expert index; gates are the softmax over
 *     all E logits (not renormalised over the k selected).
 */
#ifndef MOE_MI355X_MOE_H_
#define MOE_MI355X_MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,  /* NULL pointer, bad size, misaligned pointer */
  MOE_ERR_UNSUPPORTED = 2,       /* legal in principle but outside this build's contract */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4                /* a HIP runtime call or kernel launch failed */
} moe_status_t;

typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype_t;

/* Which entry point a workspace size is asked for. */
typedef enum {
  MOE_STAGE_PERMUTE = 0,
  MOE_STAGE_GROUPED_FFN = 1,
  MOE_STAGE_FORWARD = 2,
  MOE_STAGE_ROUTE = 3,
  MOE_STAGE_TRAIN = 4
} moe_stage_t;

typedef struct {
  int64_t T;        /* tokens */
  int32_t d_model;  /* hidden size */
  int32_t E;        /* experts */
  int32_t k;        /* experts selected per token */
  int32_t d_expert; /* expert FFN width (G = d_ff / d_expert in the MOSAIC summary) */
  int32_t dtype;    /* a moe_dtype_t */
} moe_problem_t;

/* Workspace bytes that `stage` needs for problem `p` (host only, no HIP call).
 * moe_route and moe_combine need none; moe_route_ws takes MOE_STAGE_ROUTE;
 * moe_forward_train and moe_backward share one MOE_STAGE_TRAIN workspace. */
moe_status_t moe_workspace_size(const moe_problem_t* p, int32_t stage, size_t* bytes);

/* The launch plan the library picks for problem p, for callers that model or
 * check the layer's performance (the MOSAIC summary's operator-level
 * performance model, method item 2, costs each operator from exactly these
 * choices). Host only: enqueues nothing and reads no device memory; it may
 * query the current device's compute-unit count, as the launchers do.
 * Environment overrides that the launchers honour are honoured here too.
 *   host_counts  NULL, or E int32 selections per expert in HOST memory (e.g. a
 *                copy of moe_permute's counts): then each grouped GEMM's tile
 *                list is given as the kernels derive it from the offsets
 *   plan         HOST pointer, written on success
 * MOE_ERR_INVALID_ARGUMENT for a bad problem or negative counts. */
typedef struct {
  int32_t tile;            /* block tile: 0 256x256, 1 256x256k32, 2 256x128, 3 128x128,
                              4 128x128k32, 5 256x256w8, 6 256x256w8k32, 7 32x256 */
  int32_t bm, bn, bk;      /* block tile rows, columns and K step */
  int32_t grid;            /* persistent blocks (a multiple of 8, dealt to 8 XCDs) */
  int32_t k_steps;         /* K steps of a whole tile */
  int32_t max_split;       /* leftover tiles per XCD that may be split by K steps */
  int32_t min_steps;       /* ... only when the split saves at least this many K steps */
  int32_t split_in_launch; /* 1: split tiles completed inside the launch, 0: by a fixup launch */
  /* with host_counts (else -1): */
  int64_t tiles;           /* tiles of the launch */
  int32_t xcd_rounds;      /* whole rounds of the XCD with the most tiles */
  int32_t xcd_leftover;    /* its leftover tiles */
  int32_t xcd_split;       /* 1 if that leftover is split over its blocks */
  int32_t split_xcds;      /* XCDs whose leftover is split */
} moe_gemm_plan_t;

typedef struct {
  int32_t route_splits;           /* router contraction split over d_model (1: one pass) */
  int32_t route_tokens_per_block; /* 32 or 64 */
  int32_t route_fused_permute;    /* 1: moe_forward's permute workgroup completes the split router */
  int32_t permute_form;           /* 0 one workgroup, 1 histograms + self-scanning scatter,
                                     2 histograms + scan launch + scatter */
  int32_t gather_in_gemm;         /* 1: moe_forward folds the dispatch into the first GEMM */
  int32_t combine_streaming;      /* 1: y_perm and y streamed with non-temporal accesses */
  moe_gemm_plan_t gemm[2];        /* first (x W1, GELU) and second (H W2) grouped GEMM;
                                     every field -1 for float32 problems */
  int32_t forward_one_launch;     /* 1: moe_forward runs the whole (small float32) layer as one
                                     launch, one workgroup per token */
} moe_plan_t;

moe_status_t moe_plan(const moe_problem_t* p, const int32_t* host_counts, moe_plan_t* plan);

/* Router Linear + Softmax + top-k (blog section 3, structure: the gating
 * network is a Linear layer and a Softmax; only the top-k experts are used).
 *   x            [T, d_model]      input tokens
 *   w_router     [d_model, E]      router weight (logit = x w_router + bias)
 *   router_bias  [E] float32 or NULL
 *   logits       [T, E] float32 or NULL: the float32 logits the selection used
 *   topk_idx     [T, k] int32: selected experts, descending logit, ties to the lower index
 *   topk_gate    [T, k] float32: softmax probability of each selected expert */
moe_status_t moe_route(const moe_problem_t* p, const void* x, const void* w_router,
                       const float* router_bias, float* logits, int32_t* topk_idx,
                       float* topk_gate, void* stream);

/* moe_route with a workspace (same arguments and results). When the tokens
 * alone give too few blocks to fill the GPU (small T: decode-sized batches,
 * where the MOSAIC summary's performance model, method item 2, singles out
 * dispatch latency), the bf16 contraction is split over d_model: blocks write
 * float32 partial logits to ws and a second launch adds them in a fixed order
 * (deterministic), adds the bias and selects. The selection then sees logits
 * summed in another order than moe_route's, so near-ties may resolve
 * differently between the two.
 *   ws at least moe_workspace_size(p, MOE_STAGE_ROUTE) bytes (may be 1 byte
 *   when no split is used; ws must still be non-NULL and 16-byte aligned) */
moe_status_t moe_route_ws(const moe_problem_t* p, const void* x, const void* w_router,
                          const float* router_bias, float* logits, int32_t* topk_idx,
                          float* topk_gate, void* ws, size_t ws_bytes, void* stream);

/* Dispatch as a local permutation (blog section 4, dispatch: each token is
 * sent to the expert it chose). Rows are grouped by expert; inside a group
 * tokens keep their order.
 *   topk_idx [T, k] int32 in [0, E), distinct within a token (entries outside
 *            [0, E) are ignored; duplicates give unspecified but in-bounds output)
 *   x        [T, d_model]
 *   counts   [E]     int32: selections per expert
 *   offsets  [E + 1] int32: exclusive prefix sum of counts, offsets[E] = T*k
 *   perm     [T*k]   int32: token of each permuted row
 *   inv      [T*k]   int32: inv[t*k + j] = row of selection (t, j) (-1 if ignored)
 *   x_perm   [T*k, d_model]: x_perm[r] = x[perm[r]]
 *   ws       workspace of at least moe_workspace_size(p, MOE_STAGE_PERMUTE) bytes */
moe_status_t moe_permute(const moe_problem_t* p, const int32_t* topk_idx, const void* x,
                         int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                         void* x_perm, void* ws, size_t ws_bytes, void* stream);

/* The expert FFNs over their row groups as two grouped GEMMs (blog section 3:
 * independent FFN experts; the MOSAIC summary's performance model counts them
 * as grouped GEMMs). For every expert e and row r in [offsets[e], offsets[e+1]):
 *   y_perm[r] = GELU_tanh(x_perm[r] W1[e]) W2[e]
 * with float32 accumulation; the hidden activation is stored in p->dtype.
 *   x_perm  [T*k, d_model]
 *   offsets [E + 1] int32, non-decreasing, offsets[0] = 0, offsets[E] <= T*k
 *   W1      [E, d_model, d_expert]
 *   W2      [E, d_expert, d_model]
 *   y_perm  [T*k, d_model]: rows outside [0, offsets[E]) are left untouched
 *   ws      at least moe_workspace_size(p, MOE_STAGE_GROUPED_FFN) bytes */
moe_status_t moe_grouped_ffn(const moe_problem_t* p, const void* x_perm, const int32_t* offsets,
                             const void* W1, const void* W2, void* y_perm,
                             void* ws, size_t ws_bytes, void* stream);

/* moe_permute without the row copy: counts, offsets, perm and inv as above,
 * for callers that feed x itself to moe_grouped_ffn_gather.
 *   ws at least moe_workspace_size(p, MOE_STAGE_PERMUTE) bytes */
moe_status_t moe_permute_index(const moe_problem_t* p, const int32_t* topk_idx, int32_t* counts,
                               int32_t* offsets, int32_t* perm, int32_t* inv, void* ws,
                               size_t ws_bytes, void* stream);

/* moe_permute_index for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops or harnesses that forbid
 * allocation): the same counts, offsets, perm and inv, bit for bit, with no
 * workspace argument. The counting sort's per-block counts and first rows
 * live in a static device array of the library (2 * MOE_NOALLOC_PERMUTE_SLOTS
 * int32, 2 MiB, held on each GPU the library runs on until the process ends),
 * so ceil(T / 256) * E must not exceed MOE_NOALLOC_PERMUTE_SLOTS (e.g. T up
 * to 262144 tokens with 256 experts): larger problems return
 * MOE_ERR_WORKSPACE_TOO_SMALL before anything is enqueued. Every call on a
 * GPU uses that GPU's one array: calls that overlap on one GPU (different
 * streams, or threads) race and must be ordered by the caller. The array is
 * fully rewritten by each call before it is read. */
#define MOE_NOALLOC_PERMUTE_SLOTS 262144
moe_status_t moe_permute_index_noalloc(const moe_problem_t* p, const int32_t* topk_idx, int32_t* counts,
                                       int32_t* offsets, int32_t* perm, int32_t* inv, void* stream);

/* moe_grouped_ffn with the dispatch folded into the first GEMM: row r of the
 * permuted input is read as x[perm[r]] (the same values moe_permute's x_perm
 * holds), so no permuted copy of x is written or read; y_perm is the same,
 * bit for bit, as moe_grouped_ffn gives on that x_perm.
 *   x    [T, d_model], perm [T*k] int32 in [0, T) for rows in [0, offsets[E])
 *   other arguments as for moe_grouped_ffn (same workspace size)
 * MOE_ERR_UNSUPPORTED for float32 problems and when x spans 2 GiB or more. */
moe_status_t moe_grouped_ffn_gather(const moe_problem_t* p, const void* x, const int32_t* perm,
                                    const int32_t* offsets, const void* W1, const void* W2,
                                    void* y_perm, void* ws, size_t ws_bytes, void* stream);

/* Weighted combine (blog section 3 output formula; section 4, combine:
 * expert results return to their token):
 *   y[t] = sum over j < k of topk_gate[t, j] * y_perm[inv[t*k + j]]
 * accumulated in float32 in selection order; entries of inv outside
 * [0, T*k) contribute nothing.
 *   y_perm [T*k, d_model], inv [T*k] int32, topk_gate [T, k] float32, y [T, d_model] */
moe_status_t moe_combine(const moe_problem_t* p, const void* y_perm, const int32_t* inv,
                         const float* topk_gate, void* y, void* stream);

/* The whole layer: route, permute, grouped FFN, combine on one stream, with
 * every intermediate in the workspace. bf16 problems whose x spans less than
 * 2 GiB take the moe_permute_index + moe_grouped_ffn_gather path (no x_perm
 * copy); the result is the same either way.
 *   ws at least moe_workspace_size(p, MOE_STAGE_FORWARD) bytes */
moe_status_t moe_forward(const moe_problem_t* p, const void* x, const void* w_router,
                         const float* router_bias, const void* W1, const void* W2, void* y,
                         void* ws, size_t ws_bytes, void* stream);

/* Training forward: moe_forward's result, and in ws what moe_backward needs
 * (router logits, routing, permutation, U = x W1 per expert row, H =
 * GELU_tanh(U), the expert outputs). H is GELU_tanh of the bf16-rounded U,
 * so y can differ from moe_forward's (which rounds once, after GELU) in the
 * last bits. bf16 only, k <= 8, E a multiple of 8, x under 2 GiB;
 * otherwise MOE_ERR_UNSUPPORTED.
 *   ws at least moe_workspace_size(p, MOE_STAGE_TRAIN) bytes; the caller keeps
 *   it untouched until the matching moe_backward call has been enqueued */
moe_status_t moe_forward_train(const moe_problem_t* p, const void* x, const void* w_router,
                               const float* router_bias, const void* W1, const void* W2, void* y,
                               void* ws, size_t ws_bytes, void* stream);

/* Layer backward for the last moe_forward_train call on the same ws (same p,
 * x, w_router, W1, W2), given dy = dL/dy: the chain rule of the layer of blog
 * section 3 (y = sum over the selected experts of gate * expert output), with
 * no gradient through the choice of experts:
 *   dx [T, d_model] bf16           input gradient (expert paths + router path)
 *   dw_router [d_model, E] bf16    router weight gradient
 *   dbias [E] float32 or NULL      router bias gradient (sum over tokens of dlogit)
 *   dW1 [E, d_model, d_expert], dW2 [E, d_expert, d_model] bf16
 *                                  expert weight gradients (zero for experts without tokens)
 *   load_frac [E] float32 or NULL  share of the T*k selections per expert
 *   mean_prob [E] float32 or NULL  mean router probability per expert
 * The last two are the ingredients of a load-balancing loss, whose formula
 * the pages do not give. Products accumulate in float32; the intermediates
 * (dYp, dU, dX, router logit gradients) are rounded to bf16 between GEMMs. */
moe_status_t moe_backward(const moe_problem_t* p, const void* x, const void* w_router,
                          const void* W1, const void* W2, const void* dy, void* dx,
                          void* dw_router, float* dbias, void* dW1, void* dW2,
                          float* load_frac, float* mean_prob, void* ws, size_t ws_bytes,
                          void* stream);

/* Static text for a status code. */
const char* moe_status_str(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_MOE_H_ */
