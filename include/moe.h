/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse Mixture-of-Experts layer: the
 * forward pass, and its backward for training.
 *
 * One sparse MoE layer in five steps, each a HIP kernel on the caller's stream:
 *   router logits -> top-k + gates -> counts/capacity/dispatch -> grouped expert
 *   FFN -> gate-weighted combine (+ load-balance statistics).
 *
 * Sources (page title and section):
 *   [MoE&SMS]  "Mixture-of-Experts & Sparse Model Scaling": Mathematical
 *              Formulation (softmax, top-k weighted sum, L_aux); Advanced Theory &
 *              Extensions (capacity and dropping, shared experts); labs 1-3.
 *   [MoEM]     "Mixture-of-experts Models", Level 2 (top-k dispatch, tie rule,
 *              capacity, overflow contract) and Level 3 (balance diagnostics).
 *   [SMoE-arch] "Scaling Capacity via Sparse Mixture of Experts (MoE)
 *              Architectures": router module and grouping tokens by expert.
 *   [LLM-09]   "Large Language Models part 09: Sparse Mixture-of-Experts":
 *              s.2 noisy top-k gating, s.3 capacity, s.4 auxiliary loss.
 *   [3D-lab]   "3D mixture-of-experts routing lab": Router and Capacity panels.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns every
 *     buffer, including the workspace; the library never allocates, never frees,
 *     never synchronises the stream and never throws.
 *   - All work is enqueued on `stream` (a hipStream_t; 0 = the null stream), in
 *     order.  A return of MOE_OK means the launches were enqueued; faults inside
 *     a kernel surface at the caller's next synchronisation.
 *   - Validation (null pointers, shapes, workspace size, alignment) happens on
 *     the host before any HIP call; on any error nothing is enqueued.
 *   - Layouts are row-major; weights are stored out x in (nn.Linear form), so
 *     every product is A * B^T with both operands contiguous along the
 *     reduction axis:
 *       x [T,d]; w_g, w_noise [E,d]; b_g [E]; eps [T,E];
 *       w1, w3 [E,h,d]; w2 [E,d,h]; b1 [E,h]; b2 [E,d];
 *       shared experts ws1, ws3 [S,h,d]; ws2 [S,d,h].
 *   - Activations and weights have the config dtype (float32 or bfloat16 bit
 *     patterns); biases, eps, logits, gates, expert outputs and statistics are
 *     float32; every index and count is int32.
 *   - All device pointers must be 16-byte aligned; d and h must be multiples
 *     of 8; E <= 256 (<= 128 with router noise); k <= 8; n_shared <= 64
 *     (MOE_ERR_UNSUPPORTED otherwise).
 *   - Entry points are stateless and may be called from several host threads;
 *     calls that share a workspace or outputs must be ordered by the caller.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad shape, k > E, ...        */
  MOE_ERR_UNSUPPORTED = 2,        /* valid, but outside what the kernels cover  */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4                 /* a HIP launch or runtime call failed        */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

/* Expert non-linearity: exact-erf GELU, ReLU, or SwiGLU silu(x w1^T) * (x w3^T). */
typedef enum { MOE_ACT_GELU = 0, MOE_ACT_RELU = 1, MOE_ACT_SWIGLU = 2 } moe_act_t;

/* Who chooses: every token its k best experts (top-k, capacity drops in
 * arrival order), or every expert its C' best tokens (expert choice,
 * [MoE&SMS] Advanced Theory & Extensions). */
typedef enum { MOE_ROUTE_TOKEN_CHOICE = 0, MOE_ROUTE_EXPERT_CHOICE = 1 } moe_routing_t;

/* What a full expert does to a token-choice assignment ([MoEM] "Overflow
 * handling defines an output contract"): drop it, or re-route it to the
 * token's lower-ranked experts (moe_dispatch_reroute). */
typedef enum { MOE_OVERFLOW_DROP = 0, MOE_OVERFLOW_REROUTE = 1 } moe_overflow_t;

typedef struct moe_config {
  int64_t T;                /* tokens in the batch                               */
  int64_t d;                /* model width                                       */
  int64_t E;                /* routed experts                                    */
  int64_t k;                /* experts per token, 1 <= k <= min(E, 8)            */
  int64_t h;                /* expert hidden width                               */
  int64_t n_shared;         /* always-on shared experts (same act and h), >= 0   */
  double capacity_factor;   /* > 0: C = floor(factor*T*k/E); <= 0: dropless, C=T */
  int32_t act;              /* moe_act_t                                         */
  int32_t dtype;            /* moe_dtype_t of x, y and every weight matrix       */
  int32_t ffn_bias;         /* nonzero: b1 [E,h], b2 [E,d] are given             */
  int32_t router_bias;      /* nonzero: b_g [E] is given                         */
  int32_t router_noise;     /* nonzero: w_noise [E,d] and eps [T,E] are given    */
  int32_t routing;          /* moe_routing_t (0 = token choice)                  */
  int32_t overflow;         /* moe_overflow_t (0 = drop); token choice only      */
} moe_config_t;

/* Device pointers to the layer's parameters (unused ones may be NULL). */
typedef struct moe_weights {
  const void* w_g;      const float* b_g;     const void* w_noise;
  const void* w1;       const void* w3;       const void* w2;
  const float* b1;      const float* b2;
  const void* ws1;      const void* ws3;      const void* ws2;
} moe_weights_t;

/* Optional outputs of moe_layer_forward: each non-NULL member receives the
 * same values the stage entry points would write; NULL members live in the
 * workspace instead. */
typedef struct moe_aux {
  float*   logits;      /* [T,E]                                              */
  int32_t* topk_idx;    /* [T,k]                                              */
  float*   topk_gate;   /* [T,k]                                              */
  float*   prob_sum;    /* [E]                                                */
  int32_t* counts;      /* [E]                                                */
  int32_t* offsets;     /* [E+1]                                              */
  int32_t* dest;        /* [T,k]                                              */
  int32_t* row_token;   /* [T*k]                                              */
  float*   stats;       /* [2E+2]                                             */
  float*   scores;      /* [T,E]   expert choice only                         */
  int32_t* slot;        /* [T,E]   expert choice only                         */
  float*   diag;        /* [8+2E]  token choice only: moe_router_diagnostics  */
  int32_t* final_expert;/* [T,k]   re-routing only: expert of each slot, -1  */
  /* Saved for moe_layer_backward.  Rows: the R = moe_routed_rows_bound(cfg)
   * routed rows, then n_shared blocks of T rows (shared expert s, token t at
   * row R + s*T + t). */
  void*    hidden;      /* [R + n_shared*T, h]  config dtype: act(...)       */
  void*    pre;         /* [R + n_shared*T, h, or 2h for SwiGLU] config dtype:
                           u = x w1^T (+ b1) in [0,h), then v = x w3^T       */
  float*   y_rows;      /* [R + n_shared*T, d]  expert outputs before gates  */
} moe_aux_t;

/* (host) Human-readable name of a status code; never NULL. */
const char* moe_status_string(int status);

/* (host) Expert capacity C = floor(capacity_factor * T * k / E) evaluated in
 * IEEE double left to right ([3D-lab] Capacity panel; at k = 1 this is [LLM-09]
 * s.3's factor * T / E), or T when capacity_factor <= 0 (dropless: a token's k
 * experts are distinct, so no expert can receive more than T assignments).
 * No clamp: C may be 0, and then every routed assignment is dropped.
 * Returns -1 for an invalid config. */
int64_t moe_capacity(const moe_config_t* cfg);

/* (host) Upper bound on the rows any routed expert buffer can hold in total:
 * min(T*k, E*C) for token choice, E*min(C, T) (exactly) for expert choice.
 * Returns -1 for an invalid config. */
int64_t moe_routed_rows_bound(const moe_config_t* cfg);

/* (host) Workspace bytes that suffice for every entry point below and for
 * moe_layer_forward with all moe_aux_t members NULL.  0 for an invalid config. */
size_t moe_workspace_bytes(const moe_config_t* cfg);

/* (host) Launch shape of the router kernel of moe_route for this config, no
 * GPU call: `waves` (host) receives the wavefronts per 16-token block and
 * `lds_bytes` (host) the block's LDS (dynamic plus static).  `device_logits`
 * nonzero describes the bf16 path that computes the logits on the device,
 * zero the replay or float32 path.  A bf16 batch of 1024 tokens or more
 * whose router has 32 logit columns or more (E, or 2E with noise) computes its
 * logits in a kernel of its own (64-token blocks) and the router kernel
 * replays them, so it has the replay shape either way.  A block's waves take its 16 tokens in
 * turn (token m to wave m mod waves) for the top-k step, so every token is
 * routed whatever the count.  For tests and capacity planning; returns
 * MOE_OK, or the status moe_route would return for an invalid config. */
moe_status_t moe_route_launch_shape(const moe_config_t* cfg, int device_logits, int* waves,
                                    size_t* lds_bytes);

/*
 * Router and gating ([MoE&SMS] Mathematical Formulation; [LLM-09] s.2;
 * [3D-lab] Router).
 *   logits[t,e] = x[t] . w_g[e] (+ b_g[e]) (+ eps[t,e] * softplus(x[t] . w_noise[e]))
 *   topk_idx[t,s]: the k experts with the largest float32 logits, slot 0 best;
 *     equal logits go to the lower expert index ([MoEM] asks for a fixed tie
 *     rule); -0.0 and +0.0 compare equal.
 *   topk_gate[t,s] = exp(l_s - l_0) / sum_j exp(l_j - l_0) over the k selected
 *     logits, which equals the renormalised full-softmax probabilities.
 *   prob_sum[e] = sum_t softmax(logits[t])_e (the P_i numerator of L_aux).
 * x == NULL selects replay mode: `logits` is then an INPUT [T,E] (for example
 * logits computed elsewhere) and w_g, b_g, w_noise, eps are ignored.
 * Products accumulate in float32 (bf16 inputs on MFMA).  Deterministic.
 * Workspace: at least moe_workspace_bytes(cfg).
 */
moe_status_t moe_route(const moe_config_t* cfg, const void* x, const void* w_g,
                       const float* b_g, const void* w_noise, const float* eps,
                       float* logits, int32_t* topk_idx, float* topk_gate,
                       float* prob_sum, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Counts, capacity and dispatch tables ([MoE&SMS] lab 3 and Advanced Theory;
 * [MoEM] "Capacity limits make dispatch observable"; [SMoE-arch] grouping).
 * Assignments are taken in arrival order i = t*k + s.  With C = moe_capacity:
 *   counts[e]     number of assignments routed to e (before capacity)
 *   rank(t,s)     number of earlier assignments (smaller i) to the same expert
 *   kept          rank < C; dropped assignments contribute nothing later
 *   offsets[e]    exclusive prefix sum over experts of min(counts, C); [E+1]
 *   dest[t,s]     offsets[e] + rank if kept, else -1
 *   row_token[r]  token of buffer row r, for r < offsets[E]; rows of one
 *                 expert are in arrival (token) order
 *   x_perm[r,:]   = x[row_token[r],:]  (optional: x and x_perm may both be NULL)
 * Integer results are exact and deterministic.  row_token rows at or beyond
 * offsets[E] and x_perm rows beyond it are left untouched.
 */
moe_status_t moe_dispatch(const moe_config_t* cfg, const int32_t* topk_idx,
                          const void* x, int32_t* counts, int32_t* offsets,
                          int32_t* dest, int32_t* row_token, void* x_perm,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Counts, capacity and dispatch with overflow re-routing ([MoEM] Level 2:
 * "Overflow handling defines an output contract" -- an assignment that finds
 * its expert full goes to a lower-ranked expert; [3D-lab] Capacity panel).
 * cfg->overflow must be MOE_OVERFLOW_REROUTE.  First the arrival-order pass of
 * moe_dispatch; then rounds: every unplaced assignment proposes its token's
 * next untried fallback (the experts ranked below the token's top k by the
 * float32 logits, ties to the lower index, each tried at most once; a token's
 * unplaced slots, in slot order, take consecutive ones), and every expert
 * accepts proposals in arrival order up to its spare capacity C - load; the
 * rest retry in the next round; an assignment whose token has no untried
 * fallback left is dropped.  A re-routed slot keeps its gate.
 *   counts[e]        primary assignments routed to e (before capacity)
 *   offsets[e]       exclusive prefix sum of the final loads; [E+1]
 *   dest[t,s]        final row of slot s, or -1
 *   row_token[r]     token of row r, r < offsets[E]: an expert's primary kept
 *                    rows, then each round's accepted rows, in arrival order
 *   final_expert[t,s] the expert that processes slot s, or -1
 * logits are the float32 logits the top-k was taken on.  Exact and
 * deterministic.  Workspace: at least moe_workspace_bytes(cfg).
 */
moe_status_t moe_dispatch_reroute(const moe_config_t* cfg, const int32_t* topk_idx,
                                  const float* logits, int32_t* counts, int32_t* offsets,
                                  int32_t* dest, int32_t* row_token, int32_t* final_expert,
                                  void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Grouped expert FFN over expert-contiguous rows ([MoE&SMS] Core Concepts:
 * each expert is an FFN with its own weights; [SMoE-arch] each expert runs
 * once on its grouped tokens).  For every group g < n_groups and every row r in
 * [offsets[g], offsets[g+1]):
 *   y_rows[r,:] (+)= act(a_r w1[g]^T (+ b1[g]) [, a_r w3[g]^T]) w2[g]^T (+ b2[g])
 * where a_r = x_rows[r] if row_token == NULL, else x_rows[row_token[r]] (a
 * gather straight from the token matrix, so no permuted copy is needed).
 * The hidden layer is stored in the config dtype (bf16 for bf16 configs).
 *   offsets      [n_groups+1] device int32, nondecreasing, offsets[0] = 0
 *   rows_bound   (host) upper bound on offsets[n_groups]; sizes the launch.
 *                A HARD bound: rows at or past it are not computed.
 *   group_bound  (host) upper bound on any single group's row count; small
 *                bounds (<= 32) select the weight-streaming kernels.  A HARD
 *                bound: the offsets live on the device, so the host cannot
 *                check them; when group_bound <= 32 and a group holds more
 *                than 32 rows, that group's output rows (below rows_bound) are
 *                all set to NaN instead of being computed, so a broken promise
 *                shows in the result rather than passing as plausible values.
 *   accumulate   nonzero: add into y_rows instead of overwriting
 * n_groups <= E, and w1/w3/w2/b1/b2 hold at least n_groups experts.
 * Workspace: at least moe_workspace_bytes(cfg).
 */
moe_status_t moe_expert_ffn(const moe_config_t* cfg, int64_t n_groups,
                            const void* x_rows, const int32_t* row_token,
                            const int32_t* offsets, int64_t rows_bound,
                            int64_t group_bound, const void* w1, const void* w3,
                            const void* w2, const float* b1, const float* b2,
                            float* y_rows, int accumulate, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/*
 * The two halves of moe_expert_ffn, for callers that time or reuse them:
 *   moe_expert_up:   hidden[r,:] = act(a_r w1[g]^T (+ b1[g]) [, a_r w3[g]^T])
 *                    hidden has rows_bound rows of h elements, config dtype.
 *   moe_expert_down: y_rows[r,:] (+)= hidden[r] w2[g]^T (+ b2[g])
 * Arguments mean what they mean for moe_expert_ffn.  Both halves rebuild the
 * same tile schedule from `offsets`, so they must be given the same offsets,
 * rows_bound and group_bound.
 */
moe_status_t moe_expert_up(const moe_config_t* cfg, int64_t n_groups,
                           const void* x_rows, const int32_t* row_token,
                           const int32_t* offsets, int64_t rows_bound, int64_t group_bound,
                           const void* w1, const void* w3, const float* b1,
                           void* hidden, void* ws, size_t ws_bytes, hipStream_t stream);

moe_status_t moe_expert_down(const moe_config_t* cfg, int64_t n_groups,
                             const void* hidden, const int32_t* offsets,
                             int64_t rows_bound, int64_t group_bound, const void* w2,
                             const float* b2, float* y_rows, int accumulate,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Gate-weighted combine and statistics ([MoE&SMS] Mathematical Formulation:
 * weighted sum over the selected experts and L_aux = N sum f_i P_i; [LLM-09]
 * s.1 and s.4; [MoEM] "Overflow handling defines an output contract").
 *   y[t,:] = sum_{s < n_shared} y_shared[s,t,:] + sum_{slot} [dest >= 0]
 *            topk_gate[t,slot] * y_rows[dest[t,slot],:]
 * accumulated in float32 in that order (shared experts first, then slot 0,
 * 1, ...) and stored in the config dtype (bf16 with round-to-nearest-even).
 * Dropped slots add nothing and the surviving gates are not rescaled.
 *   y_shared  [n_shared, T, d] float32, or NULL when n_shared == 0
 *   stats     optional [2E+2]: f[E] = counts/(T*k), P[E] = prob_sum/T,
 *             L_aux = E * sum f P (alpha = 1), drop_rate = 1 - sum min(counts,C)/(T*k)
 *             (with re-routing: the fraction of slots whose dest is -1)
 */
moe_status_t moe_combine(const moe_config_t* cfg, const float* y_rows,
                         const int32_t* dest, const float* topk_gate,
                         const float* y_shared, const int32_t* counts,
                         const float* prob_sum, void* y, float* stats,
                         hipStream_t stream);

/*
 * Router z-loss and routing diagnostics of a token-choice batch ([MoE&SMS]
 * Advanced Theory & Extensions: a z-loss keeps router logits small; Benchmark
 * Datasets & Evaluation: utilisation, routing entropy, fraction of tokens
 * dropped; [MoEM] Level 3: overflow and an imbalance measure).  The pages give
 * no z-loss formula; the one used is the mean squared log-partition.
 *   logits [T,E] float32; counts [E] and dest [T,k] as moe_dispatch wrote them
 *   diag   [8 + 2E] float32:
 *     [0] z-loss  mean_t (log sum_e exp logits[t,e])^2   (alpha = 1)
 *     [1] routing entropy  mean_t -sum_e p log p, p = softmax(logits[t]), nats
 *     [2] load coefficient of variation  std(counts)/mean(counts), population
 *     [3] absolute deviation from the equal share  sum_e |counts[e] - T*k/E|
 *     [4] peak-to-mean load  max(counts)/mean(counts)
 *     [5] assignments over capacity  sum_e max(counts[e] - C, 0)
 *     [6] fraction of tokens all of whose k assignments were dropped
 *     [7] fraction of tokens that lost some but not all of them
 *     [8 .. 8+E)     assignments over capacity per expert
 *     [8+E .. 8+2E)  utilisation min(counts[e], C) / C (0 when C = 0)
 * Token choice only (expert choice reports its uncovered tokens in the
 * statistics of moe_combine_expert_choice).  Deterministic.  Workspace: at
 * least moe_workspace_bytes(cfg).
 */
moe_status_t moe_router_diagnostics(const moe_config_t* cfg, const float* logits,
                                    const int32_t* counts, const int32_t* dest, float* diag,
                                    void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Expert-choice routing ([MoE&SMS] Advanced Theory & Extensions: every expert
 * takes the tokens it scores highest, up to its capacity; a token may be
 * taken by no expert or by several).  cfg->routing must be
 * MOE_ROUTE_EXPERT_CHOICE.  With C = moe_capacity(cfg) and C' = min(C, T):
 *   scores[t,e]   softmax over experts of logits[t,:], float32 (written when
 *                 logits != NULL; with logits == NULL `scores` is an INPUT,
 *                 e.g. scores computed elsewhere, which this call only ranks)
 *   expert e takes the C' tokens with the largest float32 score; equal
 *   scores go to the lower token index
 *   counts[e] = C'; offsets[e] = e*C' ([E+1])
 *   row_token[e*C' + i]  the i-th taken token of e, in ascending token order
 *   slot[t,e]            row of (t, e), or -1 when e did not take t
 * Exact and deterministic; no workspace.
 */
moe_status_t moe_expert_choice(const moe_config_t* cfg, const float* logits, float* scores,
                               int32_t* counts, int32_t* offsets, int32_t* row_token,
                               int32_t* slot, hipStream_t stream);

/*
 * Combine and statistics for expert-choice routing:
 *   y[t,:] = sum_{s < n_shared} y_shared[s,t,:] + sum_{e ascending, slot[t,e] >= 0}
 *            scores[t,e] * y_rows[slot[t,e],:]
 * in float32 in that order, stored in the config dtype; the gate is the raw
 * score (not renormalised over the experts that took t); a token no expert
 * took gets the shared part only.
 *   stats  optional [2E+2]: f[e] = counts[e] / sum(counts), P[e] = prob_sum/T,
 *          L_aux = E * sum f P, drop_rate = fraction of tokens no expert took
 */
moe_status_t moe_combine_expert_choice(const moe_config_t* cfg, const float* y_rows,
                                       const int32_t* slot, const float* scores,
                                       const float* y_shared, const int32_t* counts,
                                       const float* prob_sum, void* y, float* stats,
                                       hipStream_t stream);

/*
 * The whole layer: moe_route -> moe_dispatch -> grouped FFN over the routed
 * experts and the shared experts -> moe_combine, on one stream, with no host
 * synchronisation.  `logits_in` != NULL replays supplied float32 logits [T,E]
 * instead of computing them (w_g, b_g, w_noise and eps are then unused).
 * `eps` is the [T,E] noise for noisy gating (required when router_noise).
 * With cfg->routing == MOE_ROUTE_EXPERT_CHOICE the dispatch and combine steps
 * are moe_expert_choice and moe_combine_expert_choice (aux->topk_idx,
 * topk_gate, dest and diag are then not written).  With token choice,
 * aux->diag != NULL also runs moe_router_diagnostics on the layer's routing,
 * and cfg->overflow == MOE_OVERFLOW_REROUTE uses moe_dispatch_reroute.
 * A top-1 layer without shared experts (token choice, dropping) whose groups
 * hold at most 32 rows, called without aux->y_rows, skips the float32 expert
 * rows and the combine: the down projection stores gate * row straight into
 * each kept token's row of y (the same bf16 values the combine would form)
 * and the router zeroes y's rows first, so dropped tokens read zero.
 * Any other bf16 token-choice layer called without aux->y_rows keeps its
 * expert rows in its workspace as bf16 (each rounded once from its float32
 * sum, bias included) instead of float32, which halves the bytes the down
 * projection writes and the combine reads; the combine still accumulates in
 * float32 in the same fixed order.  With aux->y_rows the rows are float32, as
 * the stage entry points give them.  Without it, two shared experts of such a
 * layer on the tiled path (h a multiple of 64) are summed in the down
 * projection's float32 accumulators (one shared row per token) rather than
 * by the combine.
 * Intermediates live in `ws` unless `aux` names a buffer for them.
 */
moe_status_t moe_layer_forward(const moe_config_t* cfg, const moe_weights_t* w,
                               const void* x, const float* eps, const float* logits_in,
                               void* y, const moe_aux_t* aux, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/*
 * moe_layer_forward without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc.  The layer's intermediates live in a static
 * scratch array of MOE_NOALLOC_SCRATCH_BYTES (128 MiB) that the library holds
 * on every device it runs on until the process ends; the call itself
 * allocates and frees nothing.  The scratch of the CURRENT device is used, so
 * `stream` must belong to the current device.  Every argument means what it
 * means for moe_layer_forward; inputs and outputs (x, y, eps, logits_in and
 * any aux buffers) are still the caller's.  Buffers named in `aux` take their
 * part out of the scratch, so they raise the largest layer that fits.
 * Returns MOE_ERR_WORKSPACE_TOO_SMALL, before anything is enqueued, when the
 * layer needs more than the scratch holds (a decode batch of the Mixtral
 * shape needs about 39 MiB, the Switch-shaped layer about 102 MiB; prefill
 * shapes do not fit).  All calls on one device share its scratch: calls that
 * overlap on one device (on different streams, or from several host threads
 * without ordering) race and give undefined results.  Nothing in the scratch
 * needs to start at zero; it keeps the last call's contents.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
moe_status_t moe_layer_forward_noalloc(const moe_config_t* cfg, const moe_weights_t* w,
                                       const void* x, const float* eps,
                                       const float* logits_in, void* y, const moe_aux_t* aux,
                                       hipStream_t stream);

/*
 * ---- Backward pass (token choice) ----------------------------------------------
 *
 * The pages train these layers but print no backward ([MoE&SMS] Mathematical
 * Formulation: the router learns through the gate values and L_aux through
 * P_i, f_i being a hard count; [MoEM] Level 2: routing decisions are
 * discrete).  The objective differentiated is
 *     L = <dy, y> + g_aux * L_aux + g_z * L_z
 * with dy [T,d] float32 the upstream gradient of the layer output, L_aux the
 * load-balancing loss of moe_combine's statistics and L_z the z-loss of
 * moe_router_diagnostics.  Held fixed (no gradient): the top-k set, capacity
 * drops, re-routing and the counts f_i.  The float32 rounding of the logits
 * is taken as the identity.  Gradients flow through
 *   - the gates (softmax over the selected logits; a dropped slot's own gate
 *     gradient is 0, and its logit still receives gradient through the other
 *     gates, which were not renormalised),
 *   - P_i:   dL_aux/dH[t,j] = (E/T) p_tj (f_j - sum_i f_i p_ti),
 *   - L_z:   dL_z/dH[t,j]   = (2/T) lse_t p_tj,
 *   - softplus of the noise: d/d(x W_noise^T) = dH * eps * sigmoid(x W_noise^T),
 *   - the expert FFNs (shared experts with weight 1) and the router weights.
 * Every gradient is float32; dW = sum over rows in float32 from config-dtype
 * operands (bf16 layers: bf16 MFMA products of bf16-rounded dy, gated rows
 * and activations).  Deterministic (no atomics).
 */
typedef struct moe_grads {
  float* dx;        /* [T,d]    required                                        */
  float* dw_g;      /* [E,d]    required                                        */
  float* db_g;      /* [E]      required when router_bias                       */
  float* dw_noise;  /* [E,d]    required when router_noise                      */
  float* dw1;       /* [E,h,d]  required                                        */
  float* dw3;       /* [E,h,d]  required for SwiGLU                             */
  float* dw2;       /* [E,d,h]  required                                        */
  float* db1;       /* [E,h]    required when ffn_bias                          */
  float* db2;       /* [E,d]    required when ffn_bias                          */
  float* dws1;      /* [S,h,d]  required when n_shared > 0                      */
  float* dws3;      /* [S,h,d]  required when n_shared > 0 and SwiGLU           */
  float* dws2;      /* [S,d,h]  required when n_shared > 0                      */
} moe_grads_t;

/* (host) Workspace bytes for moe_layer_backward; 0 for an invalid config. */
size_t moe_backward_workspace_bytes(const moe_config_t* cfg);

/*
 * Backward of moe_layer_forward, token choice (drop or re-route) or expert
 * choice.  With expert choice the scores are the full softmax of the logits,
 * so the logits receive its backward of dS[t,e] = dy_t . (expert e's output
 * for t) over the pairs an expert took; every expert holds C' rows, so
 * f = 1/E and L_aux adds no logit gradient.
 *   x, eps       the forward's inputs (eps: [T,E] when router_noise)
 *   dy           [T,d] float32 upstream gradient of y
 *   g_aux, g_z   weights of L_aux and of the z-loss in L (0 disables each)
 *   saved        what moe_layer_forward wrote for this batch; required members:
 *                logits, counts, offsets, row_token, hidden, pre, y_rows, and
 *                topk_idx, topk_gate, dest (token choice; the final offsets
 *                and dest when re-routing, the router's counts) or scores,
 *                slot (expert choice)
 *   grads        outputs, every member float32, overwritten (not accumulated)
 * The weights must be the ones the forward used.  Workspace: at least
 * moe_backward_workspace_bytes(cfg).  MOE_ERR_UNSUPPORTED when a bf16
 * intermediate would exceed 2^30 elements, or when E + n_shared > 512.
 */
moe_status_t moe_layer_backward(const moe_config_t* cfg, const moe_weights_t* w,
                                const void* x, const float* eps, const float* dy,
                                float g_aux, float g_z, const moe_aux_t* saved,
                                const moe_grads_t* grads, void* ws, size_t ws_bytes,
                                hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
