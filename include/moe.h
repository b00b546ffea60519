/*
 * moe.h -- C ABI of libmoe.so, a sparse mixture-of-experts layer (forward,
 * and the backward of its training pass) for AMD Instinct MI355X (gfx950).
 *
 * The layer (defined on "Mixture of experts and speculative decoding", section
 * "Opening the hood: the MoE layer precisely", and on "MoE inference: the call
 * centre with 256 specialists ...", section "The bare mechanism"):
 *
 *   r      = x W_r^T (+ logit_bias)                 router scores, fp32
 *   key    = r + select_bias                        selection key (one fp32 add)
 *   TopK   = the k largest keys, ties to the lower expert index,
 *            slot 0 = largest key
 *   g      = softmax over the k kept r (unbiased)   gates, sum to 1
 *   E_e(x) = W_down[e] ( SiLU(W_gate[e] x) * (W_up[e] x) )   SwiGLU expert
 *   y      = sum_{slot} g_slot E_{TopK_slot}(x) + sum_s E_shared_s(x)
 *
 * plus the load-balance statistics of "Keeping the experts busy" (same page)
 * and of the routing-collapse passage of "Mixture of Experts and Guided
 * Decoding": f_e = count_e / (T k), P_e = mean_t softmax(r_t)_e,
 * loss = alpha * N * sum_e f_e P_e.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer to a dense row-major array owned
 *    by the caller.  The library never allocates, frees, or synchronises the
 *    device; all work is enqueued on `stream` (a hipStream_t; NULL = the null
 *    stream) and completes asynchronously.
 *  - Arguments are validated on the host before anything is enqueued; on any
 *    error nothing is launched and the status says why.  A HIP launch failure
 *    returns MOE_ERR_HIP.
 *  - Weights use the linear layer's [out, in] layout: W_r [N, d],
 *    W_gate/W_up [N, F, d], W_down [N, d, F]; shared experts [S, F, d] and
 *    [S, d, F].  x and y are [T, d].  The element type of x, y and every weight
 *    is cfg->dtype (expert weights: see moe_weight_format); biases, logits,
 *    gates, scales and statistics are fp32.
 *  - Arithmetic: bf16 inputs are multiplied on the matrix cores with fp32
 *    accumulation; the expert hidden activations and per-expert outputs are
 *    held in the input dtype (bf16 rounding to nearest even); y is rounded once.
 *  - Results are deterministic: the same inputs give bitwise the same outputs.
 *  - Calls are thread-safe; concurrent calls must use distinct workspaces.
 *  - Supported sizes: 1 <= k <= min(N, 16), N <= 512, 0 <= S <= 4, capacity >= 0,
 *    d and F positive multiples of 64, T >= 0 (T = 0 launches nothing and
 *    returns MOE_OK, except that moe_layer_backward writes zero weight
 *    gradients); FP8 expert weights with dtype MOE_BF16 only.  Other sizes
 *    return MOE_ERR_UNSUPPORTED.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* null required pointer, k > N, negative size ... */
  MOE_ERR_UNSUPPORTED = 2,  /* valid but outside the supported sizes above */
  MOE_ERR_WORKSPACE = 3,    /* workspace NULL or smaller than moe_workspace_size */
  MOE_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Storage of the expert weights (routed and shared; W_r always uses dtype).
 * The pages size expert weights at one byte per parameter for FP8 ("MoE
 * inference: the call centre with 256 specialists ...", the weight-memory
 * estimate under "Total memory") but define no format; this library takes
 * OCP FP8 E4M3 codes (bias 7, no infinities, S.1111.111 = NaN, largest
 * finite 448) with one fp32 scale per output channel:
 *   W[e][n][j] = decode(code[e][n][j]) * scale[e][n]
 * (n = row of the [out, in] matrix: F rows of W_gate/W_up, d rows of W_down).
 * Decoded values are exact in bf16; the scale multiplies each fp32 sum in
 * the GEMM epilogue (before SiLU for gate and up).  A NaN code gives NaN. */
typedef enum {
  MOE_WEIGHTS_DTYPE = 0,    /* expert weights in cfg->dtype, like x and y     */
  MOE_WEIGHTS_FP8_E4M3 = 1  /* 1-byte E4M3 codes + fp32 scales (dtype BF16)   */
} moe_weight_format;

/* Layer sizes.  T tokens, d_model, N routed experts, top_k kept per token,
 * d_ff hidden size of every expert (routed and shared), n_shared always-on
 * experts, dtype a moe_dtype.
 *
 * capacity: 0 = dropless.  C > 0 caps every routed expert at C (token, slot)
 * assignments per call ("Mixture of experts and speculative decoding",
 * "Keeping the experts busy": the extras are dropped).  Kept are an expert's
 * first C assignments in token order; a dropped assignment adds nothing to y
 * (the token's other gates are not renormalised).  topk_idx, topk_gate,
 * counts and prob_sum still describe the router's choice before dropping.
 *
 * weight_format: a moe_weight_format (0 = weights in dtype). */
typedef struct {
  int32_t T;
  int32_t d_model;
  int32_t n_experts;
  int32_t top_k;
  int32_t d_ff;
  int32_t n_shared;
  int32_t dtype;
  int32_t capacity;
  int32_t weight_format;
} moe_config;

/* Layer parameters (device pointers, caller-owned, read-only). */
typedef struct {
  const void* w_router;     /* [N, d]                                         */
  const void* w_gate;       /* [N, F, d]   (unused by moe_route)              */
  const void* w_up;         /* [N, F, d]   (unused by moe_route)              */
  const void* w_down;       /* [N, d, F]   (unused by moe_route)              */
  const void* ws_gate;      /* [S, F, d] or NULL when S = 0                   */
  const void* ws_up;        /* [S, F, d] or NULL when S = 0                   */
  const void* ws_down;      /* [S, d, F] or NULL when S = 0                   */
  const float* logit_bias;  /* [N] added to the logits (moves selection,
                               gates and P), or NULL                          */
  const float* select_bias; /* [N] added to the selection key only (the
                               auxiliary-loss-free routing bias of "The bare
                               mechanism"), or NULL                           */
  /* Per-output-channel scales of FP8 expert weights (MOE_WEIGHTS_FP8_E4M3;
     ignored otherwise).  The routed ones are required by moe_layer_forward,
     the shared ones when S > 0.                                              */
  const float* w_gate_scale;  /* [N, F] */
  const float* w_up_scale;    /* [N, F] */
  const float* w_down_scale;  /* [N, d] */
  const float* ws_gate_scale; /* [S, F] */
  const float* ws_up_scale;   /* [S, F] */
  const float* ws_down_scale; /* [S, d] */
} moe_weights;

/* Routing outputs (device pointers, caller-owned, written by the call).  For
 * moe_layer_forward every field is optional (NULL = not wanted); moe_route
 * requires topk_idx and topk_gate.  f, P and aux are the balance statistics
 * moe_balance_stats computes (bitwise the same values), produced inside the
 * call's grouping step instead of a launch of their own. */
typedef struct {
  float* logits;      /* [T, N]  r including logit_bias                       */
  int32_t* topk_idx;  /* [T, k]  chosen experts, slot 0 = largest key          */
  float* topk_gate;   /* [T, k]  softmax over the kept unbiased logits        */
  int32_t* counts;    /* [N]     (token, slot) assignments per routed expert  */
  float* prob_sum;    /* [N]     sum over tokens of softmax(r_t) over all N   */
  float* f;           /* [N]     counts / (T k)                               */
  float* P;           /* [N]     prob_sum / T                                 */
  float* aux;         /* [2]     N sum_e f_e P_e, then balance_alpha times it */
  float balance_alpha;/*         coefficient of aux[1] (not a pointer)        */
} moe_routing;

/* Stage markers for moe_layer_forward_timed. */
enum {
  MOE_STAGE_ROUTE = 0,      /* router GEMM + top-k + gates + block statistics */
  MOE_STAGE_PERMUTE = 1,    /* per-expert offsets, tile lists, token grouping  */
  MOE_STAGE_EXPERT_UP = 2,  /* grouped gate/up GEMM with SiLU(gate)*up         */
  MOE_STAGE_EXPERT_DOWN = 3,/* grouped down GEMM                               */
  MOE_STAGE_COMBINE = 4,    /* gate-weighted combine into y                    */
  MOE_STAGE_COUNT = 5
};

/* Bytes of device workspace moe_layer_forward / moe_route need for `cfg`
 * (a multiple of 256).  Returns 0 for an invalid or unsupported cfg. */
size_t moe_workspace_size(const moe_config* cfg);

/* How moe_layer_forward runs `cfg` on the current device (kernel choices and
 * reduction splits, all decided on the host from cfg and the device's
 * compute-unit count), for tests and profiling.  The kernels and splits do
 * not change the results' definition; they only change where the work runs.
 *   up_kernel / down_kernel: 0 = register-staged tiles (fp32 layers and
 *     batches of few rows per expert), 1 = large-tile kernel (bf16 prefill);
 *   up_tile_rows / down_tile_rows: rows per tile of each grouped GEMM;
 *   route_split: workgroups the router GEMM's reduction is split over
 *     (1 = the router GEMM and the selection run in one kernel);
 *   route_kernel: 0 = the router kernel (64-token tiles), 1 = the router
 *     GEMM on the large-tile expert GEMM kernel (256-token tiles, bf16, 128
 *     to 256 experts, 2048 or more tokens); either way a selection kernel
 *     adds the route_split partial logits in a fixed order when it is > 1;
 *   down_split: pieces every row of the down pass is split into over its
 *     reduction (decode shapes), else 1;
 *   tail_split_cols: column tiles of the down pass when its last row tiles
 *     may be split over the reduction (0 = never);
 *   up_narrow_tails / down_narrow_tails: 1 when an expert's last row tile
 *     of at most 64 rows runs as one tile over two column tiles (the
 *     ping-pong large-tile kernel, an even number of column tiles; the down
 *     pass only with at most 384 rows per expert on average);
 *   compute_units: the device's compute units, as the plan used them;
 *   all_token_pass: 1 when every expert (routed and shared) runs on all T
 *     tokens: batches of at most 32 tokens, at most 64 experts, bf16 or
 *     fp32 expert weights, where one 32-row tile per expert holds the whole
 *     batch and (nearly) every expert is chosen anyway (expected idle
 *     experts N (1 - k/N)^T at most 1/2).
 *     The routing then runs inside the gate/up launch and only the combine
 *     uses it; the result is the same y (each row's arithmetic is unchanged,
 *     rows no slot chose are computed and never read);
 *   split_plan_offset: byte offset in the workspace of the split plan each
 *     forward writes there on the device, int32 [4] = {pieces, first split
 *     row, rows per piece, split row tiles} (pieces = 0: nothing split);
 *   workspace_bytes: moe_workspace_size(cfg).
 * MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED for a bad cfg or NULL out. */
typedef struct {
  int32_t up_kernel;
  int32_t up_tile_rows;
  int32_t down_kernel;
  int32_t down_tile_rows;
  int32_t route_split;
  int32_t route_kernel;
  int32_t down_split;
  int32_t tail_split_cols;
  int32_t up_narrow_tails;
  int32_t down_narrow_tails;
  int32_t compute_units;
  int32_t all_token_pass;
  uint64_t split_plan_offset;
  uint64_t workspace_bytes;
} moe_plan_info;

moe_status moe_forward_plan(const moe_config* cfg, moe_plan_info* out);

/* Static, human-readable text for a status code (never NULL). */
const char* moe_status_string(int status);

/* Detail of the last MOE_ERR_* returned on the calling thread (static text
 * or a thread-local buffer; never NULL, "" when none). */
const char* moe_last_error(void);

/* Routing only (steps r, key, TopK, g and the statistics' raw sums):
 * x [T, d]; w->w_router, optional w->logit_bias / w->select_bias; writes
 * out->topk_idx and out->topk_gate (required) and out->logits, out->counts,
 * out->prob_sum when non-NULL.  `workspace` must hold moe_workspace_size(cfg)
 * bytes, 256-byte aligned; its contents are scratch.  The logits, selection
 * and statistics are bitwise those moe_layer_forward computes for the same
 * cfg and inputs (a batch that takes the all-token pass is routed here with
 * the same one-workgroup reduction as inside that forward). */
moe_status moe_route(const moe_config* cfg, const void* x, const moe_weights* w,
                     moe_routing* out, void* workspace, size_t ws_bytes,
                     void* stream);

/* Whole layer forward: routing as moe_route, then the SwiGLU experts on the
 * tokens routed to them (experts no token chose are never read, except in
 * the all-token pass of moe_plan_info, which runs every expert on every
 * token of a small batch and combines only the routed rows), the shared
 * experts on every token, and the combine y [T, d] (required).  Optional
 * routing outputs as described at moe_routing. */
moe_status moe_layer_forward(const moe_config* cfg, const void* x,
                             const moe_weights* w, void* y, moe_routing* out,
                             void* workspace, size_t ws_bytes, void* stream);

/* moe_layer_forward that also records stage_events[i] (hipEvent_t, created by
 * the caller) on `stream` before stage i and stage_events[MOE_STAGE_COUNT]
 * after the last one, so the caller can time each stage.  stage_events may be
 * NULL (then identical to moe_layer_forward), and so may any entry (that
 * marker is skipped: a caller timing one stage records only its two). */
moe_status moe_layer_forward_timed(const moe_config* cfg, const void* x,
                                   const moe_weights* w, void* y,
                                   moe_routing* out, void* workspace,
                                   size_t ws_bytes, void* stream,
                                   void* const* stage_events);

/* Bytes of the device array that moe_layer_forward_noalloc uses as its
 * workspace: one array per GPU the library runs on, held until the process
 * ends. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* moe_layer_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, kernels and results as moe_layer_forward, but
 * no workspace argument: the workspace is a library-owned device array of
 * MOE_NOALLOC_SCRATCH_BYTES on the current GPU, so the call never allocates.
 * A cfg whose workspace (moe_workspace_size) exceeds that returns
 * MOE_ERR_WORKSPACE and launches nothing: decode batches and small prefill
 * batches fit (the Mixtral-shaped layer at 32 tokens needs 4 MB), large
 * prefill batches do not.  Every call on one GPU shares that GPU's array,
 * which keeps the last call's contents (the forward reads nothing from its
 * workspace that it has not written in the same call): calls that overlap
 * on one GPU (concurrent streams, or threads) race and must be serialised
 * by the caller. */
moe_status moe_layer_forward_noalloc(const moe_config* cfg, const void* x,
                                     const moe_weights* w, void* y,
                                     moe_routing* out, void* stream);

/* Balance statistics from the routing sums of T tokens, N experts, top-k:
 * f_out[e] = counts[e] / (T k), P_out[e] = prob_sum[e] / T,
 * aux_out[0] = N * sum_e f_e P_e, aux_out[1] = alpha * aux_out[0]
 * (all fp32 device arrays; T = 0 writes zeros).  Enqueued on `stream`. */
moe_status moe_balance_stats(int32_t T, int32_t N, int32_t k,
                             const int32_t* counts, const float* prob_sum,
                             float alpha, float* f_out, float* P_out,
                             float* aux_out, void* stream);

/* ------------------------------------------------------------- backward
 *
 * Gradients of  L = sum(y * dy) + aux_grad * alpha * N * sum_e f_e P_e  with
 * respect to x and every parameter, through the forward above.  The balance
 * loss reaches the router through P only: f comes from a hard choice and is
 * a constant ("Mixture of Experts and Guided Decoding", routing-collapse
 * passage after the auxiliary-loss equation).  The selection (top-k on the
 * keys) and the capacity mask are held fixed; select_bias gets no gradient.
 *
 *   kept slot j of token t:  d(expert input) = g_tj dy_t,
 *                            dg_tj = <dy_t, E_e(x_t)>
 *   gates (kept softmax):    dr_t[idx_tj] += g_tj (dg_tj - sum_l g_tl dg_tl)
 *   balance loss:            dr_t[e] += p_te (c_e - sum_j c_j p_tj),
 *                            c_e = aux_grad alpha N f_e / T, p_t = softmax(r_t)
 *   router:                  dW_r = dr^T x, dx += dr W_r,
 *                            d logit_bias = sum_t dr_t
 * plus the chain rule through every SwiGLU expert for dx, dW_gate, dW_up and
 * dW_down (shared experts with gate 1).
 *
 * The call recomputes the routing and the gate/up projections from x (it
 * takes no state from a forward call).  Arithmetic: bf16 operands on the
 * matrix cores with fp32 accumulation; the intermediate per-row tensors (gate
 * and up projections, dy W_down, the SwiGLU gradients, each row's dx
 * contribution) are held in dtype; the router gradient and every reduction
 * are fp32; each output is rounded once to its type.  Deterministic.
 * Expert weights must be in dtype (MOE_WEIGHTS_DTYPE): FP8 codes have no
 * gradient, so MOE_ERR_UNSUPPORTED.  T = 0 writes zero weight gradients. */
typedef struct {
  void* dx;           /* [T, d]     dtype, required when T > 0                  */
  void* dw_router;    /* [N, d]     dtype, required                             */
  float* dlogit_bias; /* [N]        fp32, or NULL                               */
  void* dw_gate;      /* [N, F, d]  dtype, required (experts no token chose: 0) */
  void* dw_up;        /* [N, F, d]  dtype, required                             */
  void* dw_down;      /* [N, d, F]  dtype, required                             */
  void* dws_gate;     /* [S, F, d]  dtype, required when S > 0                  */
  void* dws_up;       /* [S, F, d]                                              */
  void* dws_down;     /* [S, d, F]                                              */
} moe_grads;

/* Bytes of device workspace moe_layer_backward needs for `cfg` (a multiple
 * of 256): per-row activations and their K-major segments, plus transposed
 * copies of the expert weights for fp32 layers (bf16 layers whose d_model is
 * a multiple of 128 read the weights as K-rows and hold no copies).  0 for an
 * invalid cfg. */
size_t moe_backward_workspace_size(const moe_config* cfg);

/* Layer backward: x [T, d] and weights as for moe_layer_forward, dy [T, d]
 * the gradient of L with respect to y (dtype), alpha the balance-loss
 * coefficient and aux_grad the weight of that loss in L.  Writes every
 * gradient of `grads` (caller-owned device arrays, 16-byte aligned).
 * `workspace` holds moe_backward_workspace_size(cfg) bytes, 256-byte
 * aligned; its contents are scratch. */
moe_status moe_layer_backward(const moe_config* cfg, const void* x,
                              const moe_weights* w, const void* dy, float alpha,
                              float aux_grad, moe_grads* grads, void* workspace,
                              size_t ws_bytes, void* stream);

/* Stage markers for moe_layer_backward_timed. */
enum {
  MOE_BSTAGE_ROUTE = 0,       /* routing and grouping, recomputed               */
  MOE_BSTAGE_TRANSPOSE_W = 1, /* W_r transposed; W_down, [W_gate | W_up] only where not
                                 read as K-rows (fp32 layers)                       */
  MOE_BSTAGE_RECOMPUTE = 2,   /* gate and up projections of the rows (2 GEMMs)   */
  MOE_BSTAGE_GRAD_H = 3,      /* dy W_down (GEMM), then the SwiGLU backward      */
  MOE_BSTAGE_GRAD_X = 4,      /* [dA dB] [W_gate; W_up] (GEMM), router, dx       */
  MOE_BSTAGE_SEGMENTS = 5,    /* per-expert operands of the weight gradients     */
  MOE_BSTAGE_GRAD_W = 6,      /* dW_down, dW_gate, dW_up (3 grouped GEMMs)       */
  MOE_BSTAGE_GRAD_WR = 7,     /* dW_r                                            */
  MOE_BSTAGE_COUNT = 8
};

/* moe_layer_backward that also records stage_events[i] (hipEvent_t, created
 * by the caller) on `stream` before stage i and stage_events[MOE_BSTAGE_COUNT]
 * after the last; NULL array or NULL entries are skipped, as for
 * moe_layer_forward_timed.  With T = 0 no marker is recorded. */
moe_status moe_layer_backward_timed(const moe_config* cfg, const void* x,
                                    const moe_weights* w, const void* dy,
                                    float alpha, float aux_grad, moe_grads* grads,
                                    void* workspace, size_t ws_bytes, void* stream,
                                    void* const* stage_events);

/* Auxiliary-loss-free balancing ("MoE inference: the call centre with 256
 * specialists ...", "The bare mechanism": a routing bias adjusted during
 * training keeps the experts balanced without a loss term).  The pages give
 * no rule; this library's reading is one step toward the mean load:
 *   select_bias[e] += rate * sign(mean_j counts[j] - counts[e])
 * (fp32 addition; the sign is taken exactly on the integer counts), counts
 * being the (token, slot) assignments per routed expert of a batch
 * (moe_routing.counts).  N <= 512; device arrays; enqueued on `stream`. */
moe_status moe_update_select_bias(int32_t N, const int32_t* counts, float rate,
                                  float* select_bias, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
