/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse Mixture-of-Experts SwiGLU
 * feed-forward layer: forward pass (moe_forward and its steps) and backward
 * pass (moe_backward, or moe_forward_train followed by moe_backward_saved).
 *
 * The layer (pages cited by title and section):
 *  - Router: "Mixture of experts: por qué un modelo enorme apenas usa sus
 *    parámetros", section "El router: la pieza que de verdad decide", and the
 *    glossary "MoE (Mixture of Experts - Mezcla de Expertos)", section 2
 *    diagram row 2: p = Softmax(TopK(W_g x)).  Each token keeps its k highest
 *    router scores; the softmax runs over those k only.
 *  - Experts: glossary section 3, step 3: every chosen expert is a SwiGLU FFN,
 *    h = SiLU(W_a x) * (W_b x), out = W_down h.
 *  - Combine: glossary section 3 step 4 and diagram row 4:
 *    y = sum_i p_i * Expert_i(x).  The residual of that row is the caller's.
 *  - Shared expert: glossary section 2, item 3: always active, weight 1.
 *  - Dispatch/regroup: "Mixture of Experts optimiza Transformers y LLMs",
 *    section "Ejecución eficiente: backends de expertos": tokens are sent to
 *    the chosen experts' weights, grouped by expert id, and the weighted
 *    results are returned in the original token order.
 *  - Packed weights: "Transformers v5 El Secreto Detrás de los Modelos MoE
 *    Más Rápidos", section "La Solución: WeightConverter": experts stacked on
 *    dim 0 and the two input projections concatenated on dim 1.
 *
 * Conventions shared by every entry point
 *  - Tensors are row-major and contiguous; "bf16" is IEEE bfloat16 stored as
 *    16-bit words.  Device pointers are HIP device (or managed) memory on the
 *    current device and must be 16-byte aligned.
 *  - x         bf16 [T, D]
 *  - w_g       bf16 [E, D]        router weight, one row per expert
 *  - router_bias fp32 [E] or NULL.  has_router_bias == MOE_ROUTER_BIAS_LOGITS:
 *              added to the fp32 router logits before the selection and the
 *              softmax.  MOE_ROUTER_BIAS_SELECT: the load balancer without an
 *              auxiliary loss of the glossary "MoE (Mixture of Experts -
 *              Mezcla de Expertos)", section 2 item 4 (per-expert router
 *              biases): the top-k is taken on the fp32 sum logit + bias, the
 *              weights are the softmax of the plain logits of the chosen
 *              experts, so the bias moves the load and not the weights
 *  - w_gate_up bf16 [E, 2F, D]    rows 0..F-1 of expert e are the activated
 *              (SiLU) projection, rows F..2F-1 the one it multiplies
 *  - w_down    bf16 [E, D, F]
 *  - ws_gate_up bf16 [2Fs, D], ws_down bf16 [D, Fs]: the shared expert, or
 *              NULL when F_shared == 0
 *  - the four expert tensors may instead hold E4M3 codes with per-row fp32
 *    scales (MOE_WEIGHTS_FP8_E4M3 below)
 *  - y         fp32 [T, D] (written, never read)
 *  - topk_ids  int32 [T, k], topk_w fp32 [T, k]: slot j is the j-th highest
 *              logit (ties to the lower expert index); weights sum to 1.
 *  - Sizes: 0 <= T, 1 <= k <= min(E, 8), 1 <= E <= 256, D and F (and Fs when
 *    nonzero) positive multiples of 8, T*k + E*BM + T < 2^31.
 *  - Ownership: the caller owns every buffer.  The library allocates no device
 *    memory and keeps no state between calls except a cached device-property
 *    lookup (and, for moe_forward_noalloc only, its static per-GPU workspace
 *    array and that array's cached address).  The workspace is
 *    caller-provided, sized by moe_workspace_size
 *    (moe_backward_workspace_size for the backward pass,
 *    moe_train_workspace_size for the training forward), and its contents
 *    need not be initialised.
 *  - Execution: all work is enqueued on `stream` (a hipStream_t; NULL is the
 *    default stream) with no host synchronisation.  Calls on different streams
 *    are independent when each has its own workspace and outputs.
 *  - Errors: arguments are checked on the host before anything is enqueued;
 *    a non-zero return means nothing was launched, except MOE_ERR_HIP, which
 *    reports a failed launch (earlier kernels of the same call may have been
 *    enqueued).  Faults inside kernels surface at the caller's next
 *    synchronisation.  Non-finite inputs are outside the contract.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, size out of range, k > E, D or F not a multiple of 8 */
  MOE_ERR_UNSUPPORTED = -2, /* E > 256, k > 8, or sizes overflowing 32-bit row indices */
  MOE_ERR_WORKSPACE = -3,   /* workspace smaller than the call's *_workspace_size() */
  MOE_ERR_ALIGNMENT = -4,   /* a pointer not 16-byte aligned */
  MOE_ERR_HIP = -5,         /* a HIP launch failed; moe_strerror gives HIP's text */
  MOE_ERR_SCRATCH = -6      /* moe_forward_noalloc: the shape needs more than the static array */
};

/* moe_shape.weight_format (any other value: MOE_ERR_INVALID_ARG).
 * Per-expert quantised expert weights ("Mixture of Experts optimiza
 * Transformers y LLMs", section on the resources the method needs;
 * "Transformers v5 El Secreto Detrás de los Modelos MoE Más Rápidos", section
 * on its limits): with MOE_WEIGHTS_FP8_E4M3, w_gate_up, w_down, ws_gate_up and
 * ws_down hold one byte per weight, an OCP FP8 E4M3 code (bias 7, no
 * infinities, NaN codes outside the contract), and the *_scale arrays of
 * moe_weights give one fp32 scale per row: weight = value(code) * scale[row].
 * x, w_g and everything downstream stay as for bf16 weights.  (With D, F or
 * F_shared not a multiple of 16, moe_block_m returns at most 32 for them.) */
#define MOE_WEIGHTS_BF16 0
#define MOE_WEIGHTS_FP8_E4M3 1

/* moe_shape.has_router_bias (any other value: MOE_ERR_INVALID_ARG) */
#define MOE_ROUTER_BIAS_NONE 0   /* no bias; router_bias is not read */
#define MOE_ROUTER_BIAS_LOGITS 1 /* bias inside the logits: selection and weights */
#define MOE_ROUTER_BIAS_SELECT 2 /* bias for the top-k selection only */

typedef struct moe_shape {
  int32_t T;               /* tokens */
  int32_t D;               /* model width */
  int32_t E;               /* routed experts */
  int32_t F;               /* routed expert hidden width (d_ff) */
  int32_t k;               /* experts per token */
  int32_t F_shared;        /* shared expert hidden width, 0 = none */
  int32_t has_router_bias; /* MOE_ROUTER_BIAS_*: how weights->router_bias is used */
  /* Expert-parallel shard ("Mixture of Experts optimiza Transformers y LLMs",
   * section "Expert Parallelism"; "Transformers v5 El Secreto Detrás de los
   * Modelos MoE Más Rápidos", section "Paralelismo de Expertos").  With
   * num_local_experts > 0 the call holds only experts expert_begin ..
   * expert_begin + num_local_experts - 1: w_gate_up / w_down have
   * num_local_experts leading entries, the router still scores all E, and
   * only assignments to the held experts contribute, so y is this shard's
   * part of the layer (the shards' y add up to the whole layer; pass the
   * shared expert to one shard only).  Both 0: every expert (no sharding). */
  int32_t expert_begin;
  int32_t num_local_experts;
  int32_t weight_format;   /* MOE_WEIGHTS_*: storage of the four expert tensors */
} moe_shape;

typedef struct moe_weights {
  const void* x;            /* bf16 [T, D] */
  const void* w_g;          /* bf16 [E, D] */
  const float* router_bias; /* fp32 [E], or NULL with MOE_ROUTER_BIAS_NONE */
  /* the four expert tensors: bf16, or E4M3 bytes (weight_format) */
  const void* w_gate_up;    /* [E, 2F, D] ([num_local_experts, 2F, D] for a shard) */
  const void* w_down;       /* [E, D, F] ([num_local_experts, D, F] for a shard) */
  const void* ws_gate_up;   /* bf16 [2*F_shared, D] or NULL */
  const void* ws_down;      /* bf16 [D, F_shared] or NULL */
  /* MOE_WEIGHTS_FP8_E4M3 only (not read otherwise); 4-byte aligned:
   * fp32 scale of each row of the four tensors above */
  const float* w_gate_up_scale;  /* [E, 2F] ([num_local_experts, 2F] for a shard) */
  const float* w_down_scale;     /* [E, D]  ([num_local_experts, D] for a shard) */
  const float* ws_gate_up_scale; /* [2*F_shared] or NULL */
  const float* ws_down_scale;    /* [D] or NULL */
} moe_weights;

/*
 * Bytes of device workspace moe_forward / moe_forward_routed need for `shape`.
 * Host only; touches no GPU.  Returns MOE_OK or MOE_ERR_INVALID_ARG /
 * MOE_ERR_UNSUPPORTED for a shape the other calls would reject.
 */
int moe_workspace_size(const moe_shape* shape, size_t* bytes);

/*
 * Row-tile height BM the grouped GEMMs use for `shape`: every expert's group
 * of rows is padded to a multiple of it (see moe_align).  Host only.
 * Returns BM > 0, or a negative error code.
 */
int moe_block_m(const moe_shape* shape);

/*
 * Whole layer: router -> expert grouping -> gate/up GEMM with SwiGLU ->
 * down GEMM -> weighted combine (+ shared expert, weight 1).
 *   y         fp32 [T, D] out
 *   topk_ids  int32 [T, k] out, or NULL (then kept in the workspace)
 *   topk_w    fp32 [T, k] out, or NULL
 *   workspace device buffer of ws_bytes >= moe_workspace_size(shape)
 * Deterministic: the same inputs give bitwise the same outputs.
 */
int moe_forward(const moe_shape* shape, const moe_weights* w, float* y, int32_t* topk_ids,
                float* topk_w, void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  There
 * is no workspace argument: the workspace is a static device array of
 * MOE_STATIC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends (the first call on a device looks up its address,
 * with hipGetSymbolAddress, while that device is current).  No call
 * allocates or frees memory or calls a routine that does.
 *   shape, w, y, topk_ids, topk_w, stream: as for moe_forward (the caller
 *             still owns and passes the inputs and outputs)
 * Limit: shapes whose moe_workspace_size exceeds MOE_STATIC_SCRATCH_BYTES
 * (decode-sized calls fit: e.g. T <= 64 at D = F = 2880, E = 32, k = 4 needs
 * about 13 MB) return MOE_ERR_SCRATCH and launch nothing; use moe_forward.
 * All calls on one GPU share its array, which keeps the last call's contents
 * (nothing in it needs clearing: every byte a kernel reads is written first
 * in the same call).  Calls that overlap on one GPU -- on different streams,
 * or from host threads without an order between them -- race on the array
 * and give wrong results: keep them on one stream.
 * Same results as moe_forward, bitwise; otherwise the same errors.
 */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_forward_noalloc(const moe_shape* shape, const moe_weights* w, float* y, int32_t* topk_ids,
                        float* topk_w, void* stream);

/*
 * Router only: fp32 logits x . W_g^T (+ bias), top-k, softmax over the k
 * chosen (same definition as moe_forward's first step).
 * Uses w->x, w->w_g, w->router_bias; writes topk_ids [T,k] and topk_w [T,k].
 */
int moe_route(const moe_shape* shape, const moe_weights* w, int32_t* topk_ids, float* topk_w,
              void* stream);

/*
 * Expert grouping of a routing (dispatch step).  Assignment a = t*k + j.
 * Groups g = 0..E-1 hold the assignments routed to expert g in ascending a;
 * when shared_rows > 0 a last group g = E holds rows t = 0..shared_rows-1 in
 * order (the shared expert).  Each group is padded to a multiple of block_m.
 *   topk_ids       int32 [T*k] in, every id in [0, E)  (ids outside are skipped:
 *                  they get row_of = -1 and no row)
 *   counts         int32 [G]      rows of each group, G = E + (shared_rows > 0)
 *   offsets        int32 [G+1]    exclusive prefix sum of counts
 *   padded_offsets int32 [G+1]    exclusive prefix sum of ceil(count/block_m)*block_m
 *   sorted_assign  int32 [T*k]    the assignments in (expert, a) order
 *   row_of         int32 [T*k]    padded row of each assignment
 *   row_token      int32 [T*k + G*(block_m-1) + shared_rows]  token of each
 *                  padded row, -1 on padding rows (entries past the last
 *                  padded row are left untouched)
 *   tile_group     int32 [(T*k + G*(block_m-1) + shared_rows)/block_m + 1]
 *                  group of each block_m-row tile
 *   n_tiles        int32 [1]      number of tiles (padded_offsets[G] / block_m)
 * All outputs are device buffers.  1 <= block_m <= 1024.
 */
int moe_align(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t block_m,
              int32_t shared_rows, int32_t* counts, int32_t* offsets, int32_t* padded_offsets,
              int32_t* sorted_assign, int32_t* row_of, int32_t* row_token, int32_t* tile_group,
              int32_t* n_tiles, void* stream);

/*
 * moe_forward with the routing given instead of computed (w->w_g and
 * w->router_bias are not read): topk_ids int32 [T,k] with distinct ids per
 * token in [0, E), topk_w fp32 [T,k].
 */
int moe_forward_routed(const moe_shape* shape, const moe_weights* w, const int32_t* topk_ids,
                       const float* topk_w, float* y, void* workspace, size_t ws_bytes,
                       void* stream);

/*
 * moe_forward that also records a HIP event before its first kernel and after
 * each of its five kernels, on `stream`, so a caller can time every step
 * (router, align, gate/up GEMM, down GEMM, combine) with hipEventElapsedTime.
 *   events  array of 6 hipEvent_t created by the caller (hipEventCreate);
 *           events[0] precedes the router, events[i] follows kernel i.
 * Same results and errors as moe_forward; events are not recorded when T == 0.
 */
int moe_forward_timed(const moe_shape* shape, const moe_weights* w, float* y, int32_t* topk_ids,
                      float* topk_w, void* workspace, size_t ws_bytes, void* stream,
                      void* const* events);

/*
 * Per-expert load of the last moe_forward / moe_forward_timed /
 * moe_forward_routed call that ran with this shape and this workspace, for a
 * load-balancing signal: "Mixture of experts: por qué un modelo enorme apenas
 * usa sus parámetros", section on the cost of the approach (the auxiliary
 * balancing loss is computed from how many tokens each expert receives), and
 * the balancer of the glossary "MoE (Mixture of Experts - Mezcla de
 * Expertos)", section 2 item 4, which adjusts the router biases from the same
 * loads.
 *   counts  device int32 [G] out, G = E (num_local_experts for a shard), plus
 *           one last entry = T when F_shared > 0 (the shared expert's rows):
 *           counts[g] = number of assignments (t, j) routed to held expert g.
 * Enqueued on `stream` after that call (a device-to-device copy out of the
 * workspace; all zeros when T == 0).  The workspace must not have been used
 * by another call in between.  Errors: as moe_workspace_size for the shape;
 * MOE_ERR_INVALID_ARG for a NULL counts (or NULL workspace with T > 0);
 * MOE_ERR_WORKSPACE when ws_bytes is below moe_workspace_size; MOE_ERR_ALIGNMENT
 * for a counts pointer not 4-byte aligned.
 */
int moe_expert_load(const moe_shape* shape, const void* workspace, size_t ws_bytes,
                    int32_t* counts, void* stream);

/*
 * Backward pass: the gradients of sum_t <dy[t], y[t]> for the routing a
 * moe_forward call returned, by the chain rule of the forward pass.  The
 * pages' training sections ("Mixture of Experts optimiza Transformers y
 * LLMs", section on training; "Transformers v5 El Secreto Detrás de los
 * Modelos MoE Más Rápidos", section "Entrenamiento MoE") run training on
 * grouped-GEMM kernels; the gradients themselves are those of the function:
 *  - the top-k choice is piecewise constant and passes no gradient; the
 *    softmax over the chosen gives dl_j = p_j (dp_j - sum_i p_i dp_i),
 *    dp_j = <dy, O_j> (O_j: slot j's expert output); other logits get 0;
 *  - SwiGLU: dg = dh u SiLU'(g), du = dh SiLU(g), dh = W_down^T (p_j dy);
 *  - dx = sum_j W_gate_up^T [dg du] (+ shared) + sum_j dl_j W_g[e_j];
 *  - dW_down[e] = sum over e's rows of (p dy) h^T, dW_gate_up[e] = [dg du] x^T,
 *    dW_g[e] = sum dl x, d_bias[e] = sum dl (a bias inside the logits only; a
 *    selection-only bias or none: d_bias is zero), the shared expert with weight 1.
 * bf16 expert weights and no shard (MOE_ERR_UNSUPPORTED otherwise).
 *   shape, w       as for the moe_forward call (w->x, w->w_g, the expert
 *                  weights; the bias is not read)
 *   topk_ids, topk_w  that call's routing [T, k]
 *   dy             fp32 [T, D]
 *   grads          outputs, fp32, overwritten
 *   workspace      device buffer of ws_bytes >= moe_backward_workspace_size(shape)
 * The dx rows and every sum run in a fixed order: the gradients are bitwise
 * reproducible.  Gradient products take bf16 operands (dy, h, dg, du, x are
 * rounded to bf16 for the MFMAs) with fp32 accumulation.
 */
typedef struct moe_grads {
  float* dx;          /* [T, D] */
  float* dw_g;        /* [E, D] */
  float* d_bias;      /* [E], or NULL */
  float* dw_gate_up;  /* [E, 2F, D] */
  float* dw_down;     /* [E, D, F] */
  float* dws_gate_up; /* [2*F_shared, D], or NULL when F_shared == 0 */
  float* dws_down;    /* [D, F_shared], or NULL when F_shared == 0 */
} moe_grads;

int moe_backward_workspace_size(const moe_shape* shape, size_t* bytes);
int moe_backward(const moe_shape* shape, const moe_weights* w, const int32_t* topk_ids,
                 const float* topk_w, const float* dy, const moe_grads* grads, void* workspace,
                 size_t ws_bytes, void* stream);

/*
 * Training forward: moe_forward (same results, bitwise) that also keeps, in
 * its larger workspace, the grouping of the rows and g | u of every row
 * (bf16), so that moe_backward_saved can skip recomputing them.
 *   workspace  device buffer of ws_bytes >= moe_train_workspace_size(shape);
 *              topk_ids and topk_w are required.
 * Restrictions and errors as moe_backward's (bf16 weights, whole layer).
 */
int moe_train_workspace_size(const moe_shape* shape, size_t* bytes);
int moe_forward_train(const moe_shape* shape, const moe_weights* w, float* y, int32_t* topk_ids,
                      float* topk_w, void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_backward using the workspace of a moe_forward_train call with the same
 * shape, weights, x and the routing it returned (train_workspace, untouched
 * since, and only read here): its grouping, g | u and h replace the
 * backward's own.  The gradients equal moe_backward's up to g and u being
 * bf16 here (fp32 there).
 */
int moe_backward_saved(const moe_shape* shape, const moe_weights* w, const int32_t* topk_ids,
                       const float* topk_w, const float* dy, const moe_grads* grads,
                       const void* train_workspace, size_t train_ws_bytes, void* workspace,
                       size_t ws_bytes, void* stream);

/* Static text for an error code (for MOE_ERR_HIP: the last HIP error seen by
 * this thread).  Never NULL. */
const char* moe_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
