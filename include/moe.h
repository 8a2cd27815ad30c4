/*
 * moe.h -- C ABI of libmoe_mi355x.so: the forward pass (and its backward
 * pass, for training) of a sparse mixture-of-experts feed-forward layer on
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (sources: "Mixture of experts", Inside the Model guide ch. 14,
 * section "The computation", equation block; "Mixture of Experts", LLM
 * tutorial ch. 11, sections "The mathematics" and "The routing decision"):
 *
 *     s   = W_r x (+ o)                    router scores, one per expert
 *     S   = TopK(q, k),  q = a(s) + b      ordered top-k of the selection key
 *     g_i = normalize(s)_i, i in S         gates over the kept experts
 *     y   = sum_{i in S, kept} g_i Expert_i(x)  +  sum_shared Shared_j(x)
 *
 * with an optional Switch-style expert capacity (LLM tutorial ch. 11,
 * "Expert capacity and dropped tokens"): a slot beyond its expert's capacity
 * is dropped and contributes 0, so the token's residual carries it.  y is the
 * MoE branch only; the caller adds the residual.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensors are dense, row-major, contiguous, in device memory unless
 *   stated otherwise, and 16-byte aligned.  "dtype" is cfg->dtype (fp32 or
 *   bf16) and applies to x, all weights, y and the intermediate activations.
 *   Scores, offsets, biases and gates are fp32; indices and counts are int32.
 * - Weight layouts follow the pages' expert arrays ("Mixture of Experts", LLM
 *   tutorial ch. 11, "The mathematics", numpy forward pass):
 *     w_router [E, d];  w1, w3 [E, d_ff, d];  w2 [E, d, d_ff];
 *     ws1, ws3 [S, d_ff_shared, d];  ws2 [S, d, d_ff_shared]
 *   (S = cfg->num_shared).  Expert e computes
 *     relu/gelu:  w2[e] . act(w1[e] . x)
 *     swiglu:     w2[e] . (silu(w1[e] . x) * (w3[e] . x))
 *   with no biases anywhere.
 * - The caller owns every buffer.  The library never allocates device memory;
 *   calls that need scratch space take a caller-provided workspace whose size
 *   moe_workspace_size() returns.
 * - Every call enqueues work on `stream` (a hipStream_t; NULL = the legacy
 *   default stream) and returns without synchronising.  Errors detected on
 *   the host are returned before anything is enqueued; a fault inside a kernel
 *   surfaces at the caller's next synchronisation, as usual for HIP.
 * - T = 0 is valid: the call validates cfg and enqueues nothing; pointer
 *   arguments are not inspected (empty tensors may have NULL data).
 * - Results are deterministic: no floating-point atomics; the same inputs give
 *   the same bits on every run.
 * - The library never prints and never aborts.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types (cfg->dtype) */
#define MOE_F32  0
#define MOE_BF16 1

/* expert nonlinearity (cfg->act).  GeLU is the exact erf form. */
#define MOE_ACT_RELU   0
#define MOE_ACT_GELU   1
#define MOE_ACT_SWIGLU 2

/* gating (cfg->gating)
 *  SOFTMAX_TOPK : key q = s (+ b); gates = softmax over the k kept scores
 *                 ("Mixture of Experts", LLM tutorial ch. 11, "The routing
 *                 decision").
 *  SIGMOID_TOPK : key q = sigmoid(s) (+ b); gates = sigmoid(s_i) divided by
 *                 the sum over the kept experts ("Mixture of experts", Inside
 *                 the Model ch. 14, "The computation" and "Auxiliary-loss-free
 *                 balancing"; the bias b picks experts only).
 *  SOFTMAX_FULL : key q = s (+ b); gate = the full-softmax probability of each
 *                 kept expert (the Switch top-1 variant, LLM tutorial ch. 11,
 *                 "Top-1 vs top-2"). */
#define MOE_GATE_SOFTMAX_TOPK 0
#define MOE_GATE_SIGMOID_TOPK 1
#define MOE_GATE_SOFTMAX_FULL 2

/* which slots claim expert capacity first (cfg->capacity_priority)
 *  TOKEN : ascending token, a token's slots in choice order -- the first C
 *          assignments of each expert are kept ("Mixture of Experts", LLM
 *          tutorial ch. 11, "Expert capacity and dropped tokens": the excess
 *          is dropped).
 *  SLOT  : every token's first choice (ascending token), then every token's
 *          second choice, ...: a token loses its first choice only if C
 *          other first choices precede it (GShard-style priority).
 * Each expert's rows in expert_offsets / perm_src follow the same order.
 * Without a capacity limit nothing is dropped and only the row order differs. */
#define MOE_PRIORITY_TOKEN 0
#define MOE_PRIORITY_SLOT  1

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* null required pointer, misaligned pointer,
                               k < 1, k > E, T < 0, bad enum value        */
  MOE_ERR_UNSUPPORTED = 2,  /* valid but not built: see moe_config_t       */
  MOE_ERR_WORKSPACE = 3,    /* ws_bytes below moe_workspace_size()         */
  MOE_ERR_HIP = 4           /* a HIP runtime call or launch failed         */
} moe_status_t;

/* Problem statement ("Mixture of experts", Inside the Model ch. 14, "The
 * computation": d, E, k; "Fine-grained and shared experts"; LLM tutorial
 * ch. 11, "Expert capacity and dropped tokens": capacity factor).
 *
 * Supported: 1 <= k <= E <= 256, k <= 16; d and d_ff (and d_ff_shared when
 * num_shared > 0) positive multiples of 64 for bf16, of 4 for fp32;
 * num_shared in [0, 8], shared experts are SwiGLU and need dtype bf16 or fp32
 * like the rest.  Enum fields are int32 so the struct has one layout in every
 * language (44 bytes, no padding). */
typedef struct moe_config {
  int32_t d;                /* model width                                  */
  int32_t num_experts;      /* E, routed experts                            */
  int32_t top_k;            /* k, experts per token                         */
  int32_t d_ff;             /* hidden width of a routed expert              */
  int32_t act;              /* MOE_ACT_*                                    */
  int32_t gating;           /* MOE_GATE_*                                   */
  int32_t dtype;            /* MOE_F32 | MOE_BF16                           */
  float   capacity_factor;  /* rho; <= 0 means no capacity limit            */
  int32_t num_shared;       /* always-on shared SwiGLU experts (0 = none)   */
  int32_t d_ff_shared;      /* their hidden width                           */
  int32_t capacity_priority;  /* MOE_PRIORITY_*                             */
} moe_config_t;

/* Human-readable name of a status code (static storage; never NULL). */
const char* moe_status_str(moe_status_t status);

/* Validate cfg for T tokens without touching the GPU. */
moe_status_t moe_check_config(const moe_config_t* cfg, int64_t T);

/* Bytes of workspace moe_forward() needs for T tokens; the same amount
 * suffices for moe_permute() and moe_expert_ffn().  Host only. */
moe_status_t moe_workspace_size(const moe_config_t* cfg, int64_t T,
                                size_t* bytes);

/* Expert capacity C = floor(((rho * k) * T) / E), computed in IEEE double
 * from the float rho ("Mixture of experts", Inside the Model ch. 14,
 * "Auxiliary loss": tokens per batch / N x capacity factor; "Mixture of
 * Experts", LLM tutorial ch. 11, Exercise 4 truncates it to an integer; with
 * k slots per token the fair share is k T / E).  *capacity = -1 when rho <= 0
 * (no limit).  Host only. */
moe_status_t moe_capacity(const moe_config_t* cfg, int64_t T,
                          int64_t* capacity);

/* Router and gating ("Mixture of experts", Inside the Model ch. 14, "The
 * computation"; LLM tutorial ch. 11, "The routing decision" and "Training
 * instability": router math in FP32).
 *   x            [T, d]     dtype
 *   w_router     [E, d]     dtype
 *   logit_offset [E] fp32 or NULL: added to every token's score (it enters
 *                both the selection and the gates)
 *   select_bias  [E] fp32 or NULL: added to the selection key only
 *   logits       [T, E] fp32 out, or NULL: s = x . w_router^T (+ offset),
 *                products exact, fp32 accumulation
 *   topk_idx     [T, k] int32 out: experts in descending key order, ties to
 *                the lower index, -0.0 == +0.0
 *   topk_gate    [T, k] fp32 out: gates in the same order
 *   workspace    optional device scratch (NULL allowed, 256-byte aligned).
 *                With T <= 16 (bf16) and ws_bytes >= moe_workspace_size(),
 *                the scores are computed split over K by many workgroups and
 *                reduced in a fixed order; with T > 16, E > 64 (bf16) and no
 *                logits output it holds the scores between the two kernels
 *                below; otherwise it is not used.
 * One fused kernel: MFMA score GEMM, then per-token top-k with wavefront
 * shuffles and the gates, from the scores held in LDS (small batches with a
 * workspace: a split-K score kernel plus one reduce-and-select kernel; E > 64
 * with logits or a workspace: the score GEMM in expert slices, then a
 * select kernel).  The results do not depend on which path runs. */
moe_status_t moe_route(const moe_config_t* cfg, int64_t T, const void* x,
                       const void* w_router, const float* logit_offset,
                       const float* select_bias, float* logits,
                       int32_t* topk_idx, float* topk_gate, void* workspace,
                       size_t ws_bytes, void* stream);

/* Capacity, histogram, scan and the stable permutation (LLM tutorial ch. 11,
 * "Expert capacity and dropped tokens" and Exercise 4; "Chapter 33 -- Mixture
 * of Experts (MoE)", "Simple MoE Layer Implementation": rows grouped per
 * expert, replacing its per-expert mask loop with one gather).
 *   topk_idx       [T, k] int32 in (from moe_route)
 *   x              [T, d] dtype in; may be NULL when x_perm is NULL
 *   expert_counts  [E] int32 out or NULL: slots per expert before capacity
 *   expert_offsets [E+1] int32 out: exclusive scan of kept = min(count, C)
 *   perm_src       [T*k] int32 out: flat slot t*k+j of permuted row p for
 *                  p < expert_offsets[E]; -1 for the rows after that.  Rows of
 *                  one expert are in ascending token order; experts ascend.
 *   slot_pos       [T*k] int32 out: permuted row of slot t*k+j, -1 = dropped.
 *                  Slots are kept first-come in token order.
 *   num_dropped    [1] int32 out or NULL: sum_e max(0, count_e - C)
 *   x_perm         [T*k, d] dtype out or NULL: x_perm[p] = x[perm_src[p]/k];
 *                  rows past expert_offsets[E] are left untouched
 *   workspace      device scratch of ws_bytes >= moe_workspace_size() */
moe_status_t moe_permute(const moe_config_t* cfg, int64_t T,
                         const int32_t* topk_idx, const void* x,
                         int32_t* expert_counts, int32_t* expert_offsets,
                         int32_t* perm_src, int32_t* slot_pos,
                         int32_t* num_dropped, void* x_perm, void* workspace,
                         size_t ws_bytes, void* stream);

/* The experts on their routed rows, and the shared experts on all tokens
 * ("Mixture of experts", Inside the Model ch. 14, "The computation": each
 * expert a gated MLP, only the selected ones run; "Fine-grained and shared
 * experts"; LLM tutorial ch. 11, "The mathematics").
 *   x              [T, d] dtype, read only by the shared experts (NULL if none)
 *   x_perm         [T*k, d] dtype: rows grouped per expert (moe_permute)
 *   expert_offsets [E+1] int32 (device): rows of expert e are
 *                  [expert_offsets[e], expert_offsets[e+1])
 *   w1, w3, w2     routed expert weights (w3 only for SwiGLU, else NULL)
 *   ws1, ws3, ws2  shared expert weights, or NULL when num_shared == 0
 *   expert_out     [T*k, d] dtype out: Expert_e(x_perm[p]) for the kept rows
 *   shared_out     [S, T, d] dtype out (NULL when num_shared == 0)
 * Ragged grouped GEMMs on bf16 MFMA with fp32 accumulation and a fused
 * activation / SwiGLU epilogue; the hidden activations are rounded to dtype.
 * When T*k <= MOE_DECODE_MAX_ROWS a small-batch variant is used that reads
 * each active expert's weights once and skips idle experts. */
#define MOE_DECODE_MAX_ROWS 64
moe_status_t moe_expert_ffn(const moe_config_t* cfg, int64_t T,
                            const void* x, const void* x_perm,
                            const int32_t* expert_offsets, const void* w1,
                            const void* w3, const void* w2, const void* ws1,
                            const void* ws3, const void* ws2, void* expert_out,
                            void* shared_out, void* workspace,
                            size_t ws_bytes, void* stream);

/* Gate-weighted sum ("Mixture of experts", Inside the Model ch. 14, "The
 * computation": y = sum g_i Expert_i(x); "Mixture-of-Experts", Neural
 * Networks Visually ch. 15, "Show the math": unselected experts add exactly
 * zero).  For each token, in slot order j = 0..k-1 and then shared expert
 * s = 0..S-1, in fp32, rounded once to dtype:
 *   y[t] = sum_{j: slot_pos[t*k+j] >= 0} topk_gate[t,j] * expert_out[slot_pos]
 *          + sum_s shared_out[s, t]
 * Dropped slots add 0 and the remaining gates are not renormalised.
 *   shared_out may be NULL (then nothing is added). */
moe_status_t moe_combine(const moe_config_t* cfg, int64_t T,
                         const void* expert_out, const int32_t* slot_pos,
                         const float* topk_gate, const void* shared_out,
                         void* y, void* stream);

/* The whole layer, y = sum_{i in S} g_i Expert_i(x) (+ shared experts), as
 * the equation block of "Mixture of experts" (Inside the Model guide ch. 14,
 * "The computation") states it and the numpy forward pass of "Mixture of
 * Experts" (LLM tutorial ch. 11, "The mathematics") computes it token by
 * token: moe_route, moe_permute, moe_expert_ffn, moe_combine on one stream,
 * with the row gather folded into the first expert GEMM's loads and, for
 * T <= 16, the routing and the permutation in two launches.
 *   y [T, d] dtype out.  topk_idx [T,k], topk_gate [T,k], expert_counts [E]
 *   and num_dropped [1] are optional outputs (NULL = keep them in the
 *   workspace).  The other arguments are as above; y's bits are those of the
 *   stepwise calls. */
moe_status_t moe_forward(const moe_config_t* cfg, int64_t T, const void* x,
                         const void* w_router, const float* logit_offset,
                         const float* select_bias, const void* w1,
                         const void* w3, const void* w2, const void* ws1,
                         const void* ws3, const void* ws2, void* y,
                         int32_t* topk_idx, float* topk_gate,
                         int32_t* expert_counts, int32_t* num_dropped,
                         void* workspace, size_t ws_bytes, void* stream);

/* moe_forward without a workspace argument, for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  The layer's scratch memory (tile plans and queue
 * words, router parts, the first GEMM's hidden activations, the expert
 * outputs) is a device array of MOE_NOALLOC_SCRATCH_BYTES that the library
 * holds on each GPU it runs on until the process ends.  Arguments, results
 * and bits are those of moe_forward (which this call shares every kernel
 * with); nothing is allocated (keep moe_profile_enable off: the event
 * profiler creates events).
 *   Limit: T such that moe_workspace_size(cfg, T) <= MOE_NOALLOC_SCRATCH_BYTES
 *   (256 MiB: a Mixtral-shape layer, d = 4096, d_ff = 14336, top-2, up to
 *   3638 tokens; a DeepSeek-V3-shape layer up to 1604; any decode batch);
 *   beyond it the call returns MOE_ERR_WORKSPACE before touching the GPU.
 *   Every call on one GPU uses that GPU's one array: calls that overlap on a
 *   GPU (two streams, two host threads) race and must be serialised by the
 *   caller.  Nothing in the array needs to start at zero. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
moe_status_t moe_forward_noalloc(const moe_config_t* cfg, int64_t T, const void* x,
                                 const void* w_router, const float* logit_offset,
                                 const float* select_bias, const void* w1,
                                 const void* w3, const void* w2, const void* ws1,
                                 const void* ws3, const void* ws2, void* y,
                                 int32_t* topk_idx, float* topk_gate,
                                 int32_t* expert_counts, int32_t* num_dropped,
                                 void* stream);

/* Routing statistics of one batch: the balance signals a routing pass yields
 * (sources: "Mixture of experts", Inside the Model guide ch. 14, sections
 * "Auxiliary loss" (balance-loss equation) and "Auxiliary-loss-free
 * balancing"; "Mixture of Experts", LLM tutorial ch. 11, "The auxiliary loss"
 * and Exercise 4):
 *     f_i       = count_i / T                 fraction of tokens sent to i
 *     P_i       = (1/T) sum_t softmax(s_t)_i  mean router probability of i
 *                 (softmax over all E scores, for every gating)
 *     loss      = alpha * E * sum_i f_i P_i   Switch balance loss
 *     drop_rate = num_dropped / (T k)
 *     bias_i'   = bias_i - gamma  if count_i * E > T k  (overloaded)
 *                 bias_i + gamma  if count_i * E < T k  (underloaded)
 *                 bias_i          otherwise
 * With k > 1 a token counts once per expert it is sent to (sum f = k).
 *   logits         [T, E] fp32 in: the scores s (+ offset), as moe_route
 *                  writes them
 *   expert_counts  [E] int32 in: assignments per expert before capacity, as
 *                  moe_permute / moe_forward write them
 *   num_dropped    [1] int32 in; needed only for drop_rate
 *   select_bias    [E] fp32 in; needed only for bias_out
 *   gamma, alpha   host scalars >= 0 (bias step, loss weight)
 *   f, P           [E] fp32 out
 *   loss           [1] fp32 out
 *   drop_rate      [1] fp32 out, or NULL
 *   bias_out       [E] fp32 out, or NULL; may be select_bias itself
 *                  (in-place update)
 *   workspace      device scratch of ws_bytes >= moe_workspace_size()
 * fp32 throughout; sums run in a fixed order.  T = 0 enqueues nothing (the
 * statistics of an empty batch are undefined).  Errors: MOE_ERR_INVALID_ARG
 * for a missing required pointer, drop_rate without num_dropped, bias_out
 * without select_bias, or negative / NaN gamma or alpha; MOE_ERR_WORKSPACE. */
moe_status_t moe_routing_stats(const moe_config_t* cfg, int64_t T,
                               const float* logits, const int32_t* expert_counts,
                               const int32_t* num_dropped, const float* select_bias,
                               float gamma, float alpha, float* f, float* P,
                               float* loss, float* drop_rate, float* bias_out,
                               void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------ training ---
 * The backward pass of the same layer (sources: "Mixture of Experts", LLM
 * tutorial ch. 11, "The routing decision", last paragraph, and "Training
 * instability"; "Mixture of experts", Inside the Model ch. 14, "Auxiliary
 * loss" and "Check yourself").  Given dy = dLoss/dy it returns the gradients
 * of <dy, y> (+ the balance loss alpha E sum_i f_i P_i when aux_alpha > 0)
 * with respect to x, w_router and every expert weight.  The routing is held
 * fixed: top-k selection and the capacity cut are discrete and pass no
 * gradient; the router learns through the gate values (all three gatings)
 * and, with the balance loss, through P (f is a count and carries none).
 * select_bias and logit_offset receive no gradient.  bf16 only
 * (MOE_ERR_UNSUPPORTED otherwise).
 *
 * Two calls: moe_forward_train() is moe_forward() that keeps what the
 * backward needs (routing, router scores, gathered rows, expert
 * pre-activations, hidden activations, expert outputs) in a caller-owned
 * `saved` buffer; moe_backward() reads it.  The saved buffer must not be
 * written between the two calls; it may be reused for the next step. */

/* Bytes of the saved buffer of moe_forward_train() for T tokens.  Host only. */
moe_status_t moe_train_workspace_size(const moe_config_t* cfg, int64_t T,
                                      size_t* bytes);

/* The forward pass of moe_forward() (same arguments and the same y bits),
 * keeping in `saved` (saved_bytes >= moe_train_workspace_size(), 256-byte
 * aligned) the routing, the router scores, the permuted input rows and, per
 * kept row, the first GEMM's pre-activations (W1 x, and W3 x for SwiGLU,
 * rounded to bf16), the hidden activations and the expert outputs; the
 * shared experts' likewise. */
moe_status_t moe_forward_train(const moe_config_t* cfg, int64_t T,
                               const void* x, const void* w_router,
                               const float* logit_offset,
                               const float* select_bias, const void* w1,
                               const void* w3, const void* w2, const void* ws1,
                               const void* ws3, const void* ws2, void* y,
                               void* saved, size_t saved_bytes, void* stream);

/* Device pointers into a saved buffer (host arithmetic only, nothing is
 * enqueued): the router scores [T, E] fp32, topk_idx [T, k], topk_gate [T, k],
 * expert_counts [E], num_dropped [1], expert_offsets [E+1], slot_pos [T*k], as
 * moe_forward_train() wrote them.  Any output pointer may be NULL. */
moe_status_t moe_saved_routing(const moe_config_t* cfg, int64_t T, void* saved,
                               float** logits, int32_t** topk_idx,
                               float** topk_gate, int32_t** expert_counts,
                               int32_t** num_dropped, int32_t** expert_offsets,
                               int32_t** slot_pos);

/* Bytes of the workspace moe_backward() needs for T tokens.  Host only. */
moe_status_t moe_backward_workspace_size(const moe_config_t* cfg, int64_t T,
                                         size_t* bytes);

/* Gradients of one layer.
 *   x, w_router, w1, w3, w2, ws1, ws3, ws2   as given to moe_forward_train()
 *   saved      the buffer moe_forward_train() filled (saved_bytes as there)
 *   dy         [T, d] bf16: gradient of the loss with respect to y
 *   aux_alpha  host scalar >= 0: weight of the balance loss (0 = none)
 *   dx         [T, d] bf16 out
 *   dw_router  [E, d] fp32 out (router math in FP32)
 *   dw1, dw3   [E, d_ff, d] bf16 out (dw3 only for SwiGLU, else NULL)
 *   dw2        [E, d, d_ff] bf16 out
 *   dws1, dws3 [S, d_ff_shared, d], dws2 [S, d, d_ff_shared] bf16 out (NULL
 *              when num_shared == 0)
 *   d_gate     [T, k] fp32 out or NULL: dLoss/dg (0 on dropped slots)
 *   d_logits   [T, E] fp32 out or NULL: dLoss/ds, the router score gradient
 *   workspace  device scratch, ws_bytes >= moe_backward_workspace_size()
 * Every output is overwritten (an expert with no kept row gets zero weight
 * gradients).  Per kept slot: dg = <dy, Expert(x)>, the expert's output
 * gradient g dy (rounded to bf16); then dH = (g dy) W2, the activation's
 * derivative from the saved pre-activations, dX, dW1, dW2, dW3 on bf16 MFMA
 * with fp32 accumulation over the expert's rows, each rounded once to bf16;
 * dx sums the kept slots' dX, the shared experts' dX and ds . w_router in
 * fp32 and rounds once.  Deterministic (no atomics). */
moe_status_t moe_backward(const moe_config_t* cfg, int64_t T, const void* x,
                          const void* w_router, const void* w1, const void* w3,
                          const void* w2, const void* ws1, const void* ws3,
                          const void* ws2, const void* saved,
                          size_t saved_bytes, const void* dy, float aux_alpha,
                          void* dx, float* dw_router, void* dw1, void* dw3,
                          void* dw2, void* dws1, void* dws3, void* dws2,
                          float* d_gate, float* d_logits, void* workspace,
                          size_t ws_bytes, void* stream);

/* Per-kernel timing with HIP events, for measurement tools.
 * moe_profile_enable(1) clears the record and brackets every later launch by
 * this library with a pair of events on the launch's stream;
 * moe_profile_enable(0) stops recording.  moe_profile_read() waits for the
 * recorded events and reports, per kernel name (at most max_names of them),
 * the total elapsed milliseconds and the number of launches; it returns the
 * number of names written, or -1 on a HIP error.  names[i] point to static
 * strings.  Not meant for use from several threads at once. */
moe_status_t moe_profile_enable(int32_t on);
int32_t moe_profile_read(const char** names, double* total_ms,
                         int32_t* launches, int32_t max_names);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
