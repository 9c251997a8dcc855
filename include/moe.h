/*
 * moe.h - C ABI of the MI355X sparse Mixture-of-Experts layer forward.
 *
 * The layer computes y = sum_i G(x)_i * E_i(x): a router scores every token
 * against every expert, a selection rule keeps some (token, expert) pairs with a
 * weight, each kept pair runs its expert's SwiGLU feed-forward network, and the
 * weighted expert outputs are summed back into token order (dongbusteel page
 * "mixture-of-experts", section on how MoE differs from the Transformer: the
 * gate-weighted sum over experts; section on experts and the router).
 *
 * Problem statement (the arguments of every call): T tokens of width d_model,
 * E experts, top-k, expert hidden width d_ff (hrletsgo page
 * "moe-vs-mot-routing-inference-cost", basic MoE structure: N copies of the FFN,
 * each token passes through k of them), capacity factor gamma with
 * N-bar = T*k/E (Capacity-Aware Inference summary on gist.science, Methodology,
 * Capacity-Aware Token Drop), an optional shared expert that every token passes
 * through with weight 1 (gillilab page on active parameters and routing, section
 * on how routing allocates the compute budget).
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers, allocated and owned by the caller.
 *    The library allocates no device memory and keeps no state between calls;
 *    calls on different streams are independent. Each call only enqueues work
 *    on `stream` (no host synchronisation); routing counts stay on the device.
 *  - Row-major layouts. Expert weights use the [out, in] (K-contiguous) layout:
 *    w_gate, w_up [E, d_ff, d_model]; w_down [E, d_model, d_ff]; shared
 *    expert ws_gate, ws_up [d_ff_shared, d_model], ws_down [d_model, d_ff_shared].
 *    w_router is [d_model, E] float32, bias [E] float32 (or NULL).
 *  - Element type of x, expert weights and x_perm: float32 if problem.dtype ==
 *    MOE_F32, bfloat16 (uint16 storage) if MOE_BF16. y has problem.y_dtype.
 *    Expert outputs o_perm and o_shared, router weights, logits and all
 *    gates/weights are float32 (the expert outputs stay unrounded until the
 *    combine, which rounds once into y).
 *  - Inputs must be finite; the hot path does not look for NaN or infinity. Debug mode
 *    (environment variable MOE_DEBUG set to anything but "" or "0", read at every call):
 *    each entry point first scans its floating-point inputs on the device (activations,
 *    router weights and bias or given logits, expert weights, expert outputs and combine
 *    weights for moe_combine), synchronises `stream`, and returns MOE_ERR_INVALID_ARG with
 *    nothing further enqueued if any value is NaN or infinite. The scan uses one flag in
 *    device memory per GPU, so debug-mode calls on one GPU must not overlap.
 *  - Row capacity R = T*k rows suffices for every selection form; buffers sized
 *    "[R, ...]" are indexed by dispatched row.
 *  - Errors: arguments are checked on the host BEFORE anything is enqueued. On
 *    MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED and MOE_ERR_WORKSPACE nothing of the call
 *    is enqueued and the outputs are untouched (in debug mode the input scans above are
 *    enqueued and synchronised first; a NaN or infinity they find is reported as
 *    MOE_ERR_INVALID_ARG before any kernel of the layer is enqueued).
 *      MOE_ERR_INVALID_ARG  bad shape (T, d_model, E, k, d_ff < 1; k > E;
 *                           expert choice with k*T < E or gamma > 0; y_dtype
 *                           bf16 with dtype f32), a NULL
 *                           required pointer, a pointer not 16-byte aligned,
 *                           unknown enum value
 *      MOE_ERR_UNSUPPORTED  valid but without a kernel: bf16 with d_model or d_ff
 *                           (or d_ff_shared) not a multiple of 64; E > 1024; operand
 *                           or output panels past the GEMMs' 32-bit byte offsets
 *      MOE_ERR_WORKSPACE    ws_bytes below moe_workspace_bytes(problem)
 *      MOE_ERR_HIP          a HIP launch failed (the HIP error is not cleared). This one
 *                           can come after earlier kernels of the same call were
 *                           enqueued: the call's outputs are then unspecified.
 *    Device faults surface at the caller's next synchronisation. Inputs must be
 *    finite; NaN/Inf in x or weights is not detected outside debug mode.
 *  - Environment: MOE_GRID_CUS (read at every call) caps the persistent grids at that
 *    many workgroups; no result depends on it (every K split and every sum order is
 *    fixed independently of the grid).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_HIP = 4
} moe_status;

/* Selection rule.
 * MOE_TOKEN_CHOICE: each token keeps its k experts with the largest logit (ties:
 *   lower expert index); gate = softmax over all E, renormalised over the k picks
 *   when renorm_topk (dongbusteel page, TopK(G(x), k); hrletsgo page, top-2 of 8).
 *   With gamma > 0, capacity-aware token drop follows: an expert with more than
 *   C = floor(gamma * T*k/E) candidates keeps the C with the highest routing score
 *   (ties: lower token index); dropped pairs weigh 0, kept gates are not
 *   renormalised again (Capacity-Aware Inference summary, Token Drop).
 *   Two variants of the capacity rule (same summary, Methodology), both with gamma > 0:
 *   - expand_m = m > 0, Expanded Drop: each token also ranks its next m experts by
 *     logit (slots k .. k+m-1). After the token drop of the top-k pairs, a token that
 *     lost d picks offers its m extra candidates; expert e admits offered pairs into
 *     its C - (kept top-k pairs) remaining places by the same routing score (ties:
 *     lower token), and the token keeps its first d admitted extra pairs in slot
 *     order. An extra pair weighs its softmax probability over the softmax mass of
 *     the token's top-k (the scale of the top-k gates). Needs k + m <= E.
 *   - cap_groups = D > 0, device-level capacity: the E experts form D groups of E/D
 *     consecutive experts (one group per device of an expert-parallel layout); a group
 *     with more than C_D = floor(gamma * T*k/D) candidate pairs keeps the C_D best by
 *     routing score (ties: lower token, then lower slot), whatever their expert.
 *     Needs D dividing E and k <= 16; not combined with expand_m.
 * MOE_EXPERT_CHOICE: each expert keeps the c = floor(k*T/E) tokens with the
 *   largest logit in its column (ties: lower token index); weight = softmax over
 *   all T tokens of that column; a token may get 0..E experts (hrletsgo page,
 *   Mixture-of-Tokens section: c = k*T/N). */
typedef enum { MOE_TOKEN_CHOICE = 0, MOE_EXPERT_CHOICE = 1 } moe_routing_kind;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* moe_route flag: skip the router, read `logits` as given (selection-only path). */
enum { MOE_ROUTE_LOGITS_IN = 1 };

typedef struct {
  int32_t T, d_model, E, k, d_ff; /* tokens, model width, experts, top-k, expert hidden width */
  int32_t d_ff_shared;            /* shared-expert hidden width; 0 = no shared expert          */
  int32_t routing;                /* moe_routing_kind                                          */
  float gamma;                    /* capacity factor; <= 0 = no capacity limit                 */
  int32_t renorm_topk;            /* 1 = renormalise the k gates over the picks                */
  int32_t dtype;                  /* moe_dtype of x, expert weights, x_perm and the hidden h   */
  int32_t y_dtype;                /* moe_dtype of y; MOE_F32 allowed for either dtype, MOE_BF16
                                     only when dtype is MOE_BF16                               */
  int32_t expand_m;               /* Expanded Drop: extra candidate experts per token; 0 = off  */
  int32_t cap_groups;             /* capacity per group of E/cap_groups experts; 0 = per expert */
} moe_problem;

/* Routing result, all device pointers owned by the caller.
 *  logits     [T, E]   float32; input when MOE_ROUTE_LOGITS_IN, else output
 *  topk_ids   [T, S]   int32, token choice: picks in descending logit order (NULL allowed
 *                      for expert choice, required for token choice); S = k + expand_m
 *                      (slots k.. hold the Expanded Drop's extra candidates)
 *  topk_w     [T, S]   float32, token choice: gate of each pick before any drop
 *  kept       [T, S]   uint8, token choice: 1 kept / 0 dropped by capacity (may be NULL,
 *                      except with expand_m > 0 or cap_groups > 0)
 *  counts     [E]      int32, rows per expert after selection
 *  offsets    [E+1]    int32, exclusive prefix sum of counts; offsets[E] = rows in use
 *  perm_token [R]      int32, dispatched row p holds token perm_token[p]; rows are grouped
 *                      by expert (expert e owns [offsets[e], offsets[e+1])), ascending
 *                      token inside a group
 *  perm_w     [R]      float32, combine weight of row p
 *  tok_ptr    [T+1]    int32, CSR over tokens: token t's rows are
 *  tok_pos    [R]      int32  tok_pos[tok_ptr[t] .. tok_ptr[t+1]), in slot order (token
 *                      choice) or ascending expert (expert choice)
 * Rows p >= offsets[E] of perm_token/perm_w/tok_pos are unspecified. */
typedef struct {
  float *logits;
  int32_t *topk_ids;
  float *topk_w;
  uint8_t *kept;
  int32_t *counts, *offsets;
  int32_t *perm_token;
  float *perm_w;
  int32_t *tok_ptr, *tok_pos;
} moe_routing;

/* Bytes of device workspace every entry point below needs for `problem` (one size for all
 * of them; 256-byte aligned regions inside). This is the library's own convention, not an
 * operation of the pages. Validates `problem` exactly as the compute calls do; writes
 * *bytes only on MOE_OK. Host only, enqueues nothing. */
moe_status moe_workspace_bytes(const moe_problem *problem, size_t *bytes);

/* Router + selection + dispatch indices. Steps and the passages that define them:
 *   logits = x W_r + b: the router scores every token for every expert (dongbusteel page,
 *     section on the roles of the expert and the router);
 *   softmax scores: the router probability P_i (hrletsgo page "MoE vs MoT routing inference
 *     cost", section on the basic MoE structure);
 *   one selection rule (see moe_routing_kind): TopK(G(x), k) (dongbusteel page, same
 *     section), expert choice with c = k T / N (hrletsgo page, Mixture-of-Tokens part of the
 *     basic-structure section), capacity C = gamma N-bar with the lowest gating scores
 *     dropped, Expanded Drop and device-level capacity (gist.science summary of
 *     "Capacity-Aware Inference", section 2 Methodology, items 1-3);
 *   per-expert histogram, prefix scan and stable permutation: the dispatch that sends each
 *     token to its experts (hrletsgo page, basic-structure section, the dispatch step).
 * x [T, d_model] (dtype), w_router [d_model, E] float32, bias [E] float32 or NULL (x,
 * w_router and bias are not read with MOE_ROUTE_LOGITS_IN and may be NULL then).
 * flags: 0 or MOE_ROUTE_LOGITS_IN. Fills every non-NULL field of `routing` (logits too
 * unless MOE_ROUTE_LOGITS_IN). Routing decisions depend only on the float32 logits and are
 * reproducible bit for bit; the capacity drop ranks pairs by a fixed float32 encoding of
 * the softmax probability (Cody-Waite exponential, left-to-right sum over experts, IEEE
 * division). Uses the routing scratch of `ws`. */
moe_status moe_route(const moe_problem *problem, const void *x, const float *w_router,
                     const float *bias, int flags, moe_routing *routing, void *ws,
                     size_t ws_bytes, hipStream_t stream);

/* moe_route without a workspace, for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops or harnesses that forbid allocation). Same arguments,
 * results and errors as moe_route minus ws/ws_bytes: the routing scratch lives in a
 * library-held device array of 32 MiB, one per GPU the library runs on, held until the
 * process ends; the call allocates nothing. A problem whose routing scratch exceeds 32 MiB is
 * rejected with MOE_ERR_WORKSPACE before anything is enqueued. The routing scratch is about
 * 24*T*S bytes with S = k + expand_m slots per token (S = E and another 4*E*T bytes for
 * expert choice), plus 6*d_model*E bytes of split router weights for bf16: 16384 tokens with
 * 128 experts and top-8 need about 5 MiB, the other named workloads less.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (different
 * streams, or different host threads) race and must be serialised by the caller. */
moe_status moe_route_noalloc(const moe_problem *problem, const void *x, const float *w_router,
                             const float *bias, int flags, moe_routing *routing,
                             hipStream_t stream);

/* Row gather of the dispatch: x_perm[p] = x[perm_token[p]] for p < offsets[E] (hrletsgo
 * page, basic-structure section: the dispatch that moves each token to its experts;
 * devcy0922 page "Ugh, bandwidth", section on MoE not being a light dense model: token and
 * activation movement to the selected experts). x [T, d_model], x_perm [R, d_model], both
 * of the problem dtype; reads routing->perm_token and routing->offsets (as moe_route left
 * them). Needs no workspace, so it takes none. Rows p >= offsets[E] of x_perm are left
 * untouched. The layer path (moe_layer_forward) folds this gather into the gate/up GEMM's
 * operand loads instead. */
moe_status moe_dispatch(const moe_problem *problem, const void *x, const moe_routing *routing,
                        void *x_perm, hipStream_t stream);

/* Expert SwiGLU FFN as a grouped GEMM over the dispatched rows (hrletsgo page, basic-structure
 * section: the layer holds N copies of the FFN and each token passes through the ones it
 * was routed to; gillilab page on active parameters, section on how routing allocates the
 * compute budget: a shared expert that every token passes through):
 *   o_perm[p] = W_down_e ( silu(W_gate_e x_perm[p]) * (W_up_e x_perm[p]) ),  e = expert of row p
 * plus, when d_ff_shared > 0, the shared expert over all T tokens of x:
 *   o_shared[t] = Ws_down ( silu(Ws_gate x[t]) * (Ws_up x[t]) ).
 * The hidden activation is rounded to the problem dtype between the two GEMMs;
 * accumulation is float32. x_perm [R, d_model] (dtype), o_perm [R, d_model] float32;
 * x [T, d_model] (dtype), o_shared [T, d_model] float32
 * (x, ws_* and o_shared may be NULL without a shared expert). Reads routing->counts and
 * routing->offsets; uses the h and partial-sum regions of `ws`. */
moe_status moe_expert_ffn(const moe_problem *problem, const void *x_perm,
                          const moe_routing *routing, const void *w_gate, const void *w_up,
                          const void *w_down, const void *x, const void *ws_gate,
                          const void *ws_up, const void *ws_down, void *o_perm, void *o_shared,
                          void *ws, size_t ws_bytes, hipStream_t stream);

/* Gate-weighted combine back to token order (dongbusteel page, section on how MoE differs
 * from the Transformer: y = sum_i G(x)_i E_i(x), the gate-weighted sum of expert outputs):
 *   y[t] = sum over rows p of token t of perm_w[p] * o_perm[p]  (+ o_shared[t])
 * summed in float32 in CSR order; a token without rows gets 0 (+ o_shared[t]).
 * o_perm, o_shared float32; y [T, d_model] in problem.y_dtype (one rounding, to nearest
 * even, for bf16). Reads routing->tok_ptr, tok_pos and perm_w; needs no workspace. */
moe_status moe_combine(const moe_problem *problem, const void *o_perm, const void *o_shared,
                       const moe_routing *routing, void *y, hipStream_t stream);

/* The whole layer, y = sum_i G(x)_i E_i(x) (dongbusteel page, section on how MoE differs
 * from the Transformer), as the pages' per-token path token -> router -> selected experts
 * -> combine (devcy0922 page, section on MoE not being a light dense model): the results
 * of moe_route, moe_dispatch, moe_expert_ffn and moe_combine, on `stream`. The dispatch row gather is folded into the gate/up GEMM's operand loads
 * (routed row p is read as x[perm_token[p]]), so no x_perm is materialised; the output is
 * bit-identical to the four separate calls. routing may be NULL (then the routing arrays
 * live inside the workspace). */
moe_status moe_layer_forward(const moe_problem *problem, const void *x, const float *w_router,
                             const float *bias, const void *w_gate, const void *w_up,
                             const void *w_down, const void *ws_gate, const void *ws_up,
                             const void *ws_down, void *y, moe_routing *routing, void *ws,
                             size_t ws_bytes, hipStream_t stream);

/* Stage boundaries recorded by moe_layer_forward_traced: events[i] is recorded on
 * `stream` before stage i starts and events[MOE_STAGE_COUNT] after the last. */
enum {
  MOE_STAGE_ROUTE = 0,    /* router, selection, dispatch indices */
  MOE_STAGE_DISPATCH = 1, /* row gather (empty: folded into the gate/up GEMM) */
  MOE_STAGE_GATE_UP = 2,  /* grouped GEMM x W_gate, x W_up + SwiGLU (routed + shared) */
  MOE_STAGE_DOWN = 3,     /* grouped GEMM h W_down (routed + shared) */
  MOE_STAGE_COMBINE = 4,  /* weighted combine                    */
  MOE_STAGE_COUNT = 5
};

/* moe_layer_forward with stage timing for measurement (the same passages): the same kernels
 * in the same order, plus hipEventRecord(events[i], stream) at each stage boundary.
 * n_events must be MOE_STAGE_COUNT + 1; events are created and owned by the caller
 * (MOE_ERR_INVALID_ARG for a NULL array or event). */
moe_status moe_layer_forward_traced(const moe_problem *problem, const void *x,
                                    const float *w_router, const float *bias,
                                    const void *w_gate, const void *w_up, const void *w_down,
                                    const void *ws_gate, const void *ws_up, const void *ws_down,
                                    void *y, moe_routing *routing, void *ws, size_t ws_bytes,
                                    hipStream_t stream, hipEvent_t *events, int n_events);

/* Expert-utilisation statistics of a routing result (hrletsgo page "MoE vs MoT routing
 * inference cost", section on the basic MoE structure, load-imbalance paragraph: the
 * balance term is the sum over experts of f_i, the share of tokens expert i received,
 * times P_i, its router probability; gillilab page on active parameters, routing section:
 * the utilisation distribution is the leading indicator of routing collapse).
 * Reads routing->logits, counts, offsets (as moe_route left them). out [2*E + 4] float32
 * on the device, written in one pass of two small kernels on `stream`:
 *   out[0..E)     f_i = counts[i] / offsets[E]        (0 if no rows)
 *   out[E..2E)    P_i = mean over tokens of softmax_E(logits)[t, i]
 *   out[2E]       sum_i f_i P_i  (no scale factor: uniform routing gives 1/E)
 *   out[2E+1]     max_i counts[i] / (offsets[E] / E)  (0 if no rows)
 *   out[2E+2]     assignments dropped by capacity (T*k - offsets[E] for token choice, else 0)
 *   out[2E+3]     number of experts with no rows
 * Uses the workspace's statistics region; errors as for every entry point. */
moe_status moe_routing_stats(const moe_problem *problem, const moe_routing *routing, float *out,
                             void *ws, size_t ws_bytes, hipStream_t stream);

const char *moe_status_str(moe_status status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
