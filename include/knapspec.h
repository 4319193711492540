/*
 * knapspec.h -- C ABI of the MI355X (gfx950) KnapSpec layer-selection library.
 *
 * What it computes.  KnapSpec (Cha, Kim, Han, Yang, Han; arXiv 2602.20217, described on the
 * pith.science review page) treats each Attention and each MLP block of a decoder as a 0/1
 * knapsack item.  An item's weight is its latency (Attention grows linearly with the context
 * length, MLP is flat: review, "The reading"); its value is how close the hidden state stays
 * to the full model's, measured by cosine similarity.  A dynamic program over items x latency
 * budgets keeps, at every item and budget, whichever of "execute" or "skip" gives the higher
 * cosine to the full model's state at that depth (review, "What carries the argument";
 * referee major comment 1: Section 3.4, Eq. 8, Algorithm 1), giving one candidate layer set
 * per budget.  A grid over the draft length gamma then maximises Tokens-per-Time,
 *     TPT(S, gamma) = ((1 - a^(gamma+1)) / (1 - a)) / (gamma * t_draft(S) + t_target)
 * (review, "What carries the argument", Eq. 4), where a is the acceptance estimate of S.
 *
 * Conventions used by every call:
 *   - Items i = 0 .. 2L-1: item 2l is the Attention block of layer l, item 2l+1 its MLP.
 *   - Budget b = 0 .. n_budgets-1 is the USED integer weight sum over executed items.  The
 *     paper indexes by skipped weight j; the two are related by b = P_i - j with P_i the
 *     weight prefix sum through item i (review, referee minor comment 2).
 *   - Weights: Delta = (sum of item latencies) / (n_budgets - 1) and
 *     w_i = max(1, round-half-even(t_i / Delta)) (review, referee major comment 4: w = t/Delta).
 *   - The decoder is a Llama-style pre-norm block: RMSNorm (unit gain) -> q|k|v projection
 *     -> rotate-half RoPE at position ctx_len -> grouped-query softmax attention over the
 *     ctx_len cached positions plus the token's own k/v -> output projection + residual;
 *     RMSNorm -> gate|up projection -> silu(gate)*up -> down projection + residual.
 *   - Exact cosine ties keep "skip"; a NaN cosine counts as minus infinity.
 *
 * Error behaviour: every int-returning call returns KNAPSPEC_OK (0) or a negative code and
 * never throws or aborts; the message of the last failure on the calling thread is
 * available from knapspec_last_error().  On failure, outputs are left untouched.
 * Threading: a model handle must not be used by two threads at once.
 */
#ifndef KNAPSPEC_H
#define KNAPSPEC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KNAPSPEC_ABI_VERSION 3

#define KNAPSPEC_OK 0
#define KNAPSPEC_EINVAL (-1)       /* bad argument, shape or pointer */
#define KNAPSPEC_ENOMEM (-2)       /* a device or pinned-host allocation failed */
#define KNAPSPEC_EHIP (-3)         /* HIP runtime or kernel launch error */
#define KNAPSPEC_EUNSUPPORTED (-4) /* a shape the compiled kernels do not cover */

#define KNAPSPEC_F32 0  /* weights and KV cache in float32 */
#define KNAPSPEC_BF16 1 /* weights and KV cache in bfloat16 */

#define KNAPSPEC_RETURN_DECISIONS 1 /* fill knapspec_result.decisions */
#define KNAPSPEC_RETURN_MARGINS 2   /* fill knapspec_result.margins */
#define KNAPSPEC_ALPHA_LM_HEAD 4    /* TPT acceptance from the LM head (knapspec_set_lm_head) */
#define KNAPSPEC_KEEP_PRUNED_ROWS 8 /* keep pruned budgets' rows (see knapspec_solve) */

#define KNAPSPEC_WINDOW_MAX 16 /* largest r of an r-token window */
#define KNAPSPEC_BEAM_MAX 8   /* largest beam width of the beam variant of the DP */

typedef struct knapspec_model knapspec_model; /* opaque */

/* Decoder shape and the limits the library sizes its device workspace for. */
typedef struct {
  int32_t n_layers;    /* L; the DP has 2L items */
  int32_t d_model;     /* hidden size d (a multiple of 4; bf16: of 64) */
  int32_t n_q_heads;   /* hq */
  int32_t n_kv_heads;  /* hkv, divides hq; query head h reads KV head h / (hq/hkv) */
  int32_t head_dim;    /* dh: 64 or 128 */
  int32_t d_ff;        /* SwiGLU inner size */
  int32_t dtype;       /* KNAPSPEC_F32 or KNAPSPEC_BF16 */
  float rms_eps;       /* RMSNorm epsilon */
  float rope_theta;    /* RoPE base: angle_j = pos * theta^(-2j/dh) */
  int32_t max_budgets; /* largest n_budgets a solve may use (2..1024) */
  int32_t max_seqs;    /* largest n_seqs a solve may use */
  int32_t max_ctx;     /* largest ctx_len a solve may use */
  int32_t max_window;  /* largest r a sequence may use (0 or 1: single-token states;
                          <= KNAPSPEC_WINDOW_MAX); the workspace scales with it */
  int32_t max_beam;    /* largest beam a solve may use (0 or 1: the one-state DP only;
                          <= KNAPSPEC_BEAM_MAX); the workspace scales with it */
} knapspec_model_desc;

/* Device pointers of one layer's weights, row-major [out][in], in desc.dtype:
 *   w_qkv     [(hq + 2*hkv) * dh][d]   rows: q heads, then k heads, then v heads
 *   w_o       [d][hq * dh]
 *   w_gate_up [2 * d_ff][d]            rows: gate, then up
 *   w_down    [d][d_ff]
 * Borrowed: the caller keeps them alive and unchanged until knapspec_free_model. */
typedef struct {
  const void *w_qkv, *w_o, *w_gate_up, *w_down;
} knapspec_layer_weights;

/* Validates the shape, records the weight pointers and allocates the device workspace
 * (sized from max_budgets, max_seqs and max_ctx) and pinned host staging.  hip_stream is
 * the stream used for set-up work (NULL = default stream).  *out receives the handle. */
int knapspec_load_model(const knapspec_model_desc* desc, const knapspec_layer_weights* layers,
                        void* hip_stream, knapspec_model** out);

/* Per-item latency model (one-time profile; review, "Editorial extensions": profiling once,
 * re-solving on the fly).  t_attn(n) = attn_base + attn_per_token * n, t_mlp = mlp, and
 * `fixed` is added once to every pass (draft and target).  per_item, when not NULL, points to
 * 2L host doubles that replace the linear model for every sequence (copied).  All values must
 * be finite and >= 0, with a positive total.  Until this is called, solves fail (EINVAL). */
typedef struct {
  double attn_base, attn_per_token, mlp, fixed;
  const double* per_item;
} knapspec_latency_model;

int knapspec_set_latency_model(knapspec_model* model, const knapspec_latency_model* lat);

/* One sequence to solve for.  All pointers are device pointers borrowed for the call.
 *   k_cache[l], v_cache[l]: layer l's cache, [hkv][ctx_capacity][dh] in desc.dtype, holding
 *     positions 0 .. ctx_len-1 already rotated.
 *   x0: float32 [window][d], the input hidden states of the window's tokens, token t at
 *     position ctx_len + t.
 *   window: r, the tokens per DP state (0 counts as 1; <= desc.max_window).  The review
 *     gives the DP table as (2L+1) x (K+1) x r x d (referee major comment 4) over a window
 *     of recent tokens (free parameter m).  Reading: the r tokens pass through each item as
 *     one causal block (each attends to the cache and to window tokens 0..t), and states
 *     are compared by the cosine of the flattened r x d matrices. */
typedef struct {
  int32_t ctx_len;      /* 0 .. max_ctx */
  int32_t ctx_capacity; /* positions per KV head in the buffers, >= ctx_len */
  const void* const* k_cache; /* host array of n_layers device pointers */
  const void* const* v_cache; /* host array of n_layers device pointers */
  const float* x0;
  int32_t window;
} knapspec_seq;

typedef struct {
  int32_t n_seqs;             /* 1 .. max_seqs; sequences are solved together, independently */
  const knapspec_seq* seqs;   /* host array [n_seqs] */
  int32_t n_budgets;          /* B, 2 .. max_budgets */
  int32_t gamma_min, gamma_max; /* TPT grid, 1 <= gamma_min <= gamma_max <= 64 */
  float tau;                  /* prune a cell whose kept cosine < tau; -INFINITY disables */
  int32_t max_skip_weight;    /* prune cells whose skipped weight P_i - b exceeds it; <0 off */
  int32_t flags;              /* KNAPSPEC_RETURN_DECISIONS | KNAPSPEC_RETURN_MARGINS |
                                 KNAPSPEC_ALPHA_LM_HEAD | KNAPSPEC_KEEP_PRUNED_ROWS */
  void* hip_stream;           /* stream the work is enqueued on (NULL = default stream) */
  int32_t beam;               /* states kept per (item, budget) cell: 0 or 1 = the one-state
                                 DP; k in 2..desc.max_beam = the beam variant (review,
                                 "Reading between the lines": an exact or beam-search variant
                                 measures the greedy rule's headroom).  Each cell keeps the k
                                 candidates -- its k skip states and the item applied to the k
                                 states of b - w_i -- with the highest cosine (ties: skip slots,
                                 then execute slots, each in slot order); results report each
                                 budget's best set.  Decisions and margins are those of the
                                 one-state DP: with beam > 1 their flags are EINVAL. */
} knapspec_solve_args;

/* Caller-allocated HOST arrays; "W" = knapspec_mask_words(n_layers), L2 = 2 * n_layers. */
typedef struct {
  uint64_t* masks;      /* [n_seqs][n_budgets][W]; bit i of word i/64 set = item i executed */
  float* cos;           /* [n_seqs][n_budgets] cosine to the full model after item 2L-1; NaN
                           where invalid */
  uint8_t* valid;       /* [n_seqs][n_budgets] 1 = budget holds a candidate set */
  double* t_draft;      /* [n_seqs][n_budgets] fixed + sum of t_i over executed items */
  int32_t* item_weight; /* [n_seqs][L2] integer weights used */
  int32_t* best_budget; /* [n_seqs] argmax budget of the TPT grid, -1 if none valid */
  int32_t* best_gamma;  /* [n_seqs] its gamma, -1 if none valid */
  double* best_tpt;     /* [n_seqs] its TPT, NaN if none valid */
  uint8_t* decisions;   /* nullable [n_seqs][L2][n_budgets]: 0 skip, 1 execute, 255 invalid */
  float* margins;       /* nullable [n_seqs][L2][n_budgets]: |c_exec - c_skip|, +inf when one
                           option exists, NaN when none */
  float* alpha;         /* nullable [n_seqs][n_budgets]: the acceptance estimate the TPT grid
                           used (clamp(cos, 0, 1), or the LM-head estimate); 0 if invalid */
  int32_t* tokens;      /* nullable: per sequence in order, (n_budgets + 1) x window_q
                           entries: with KNAPSPEC_ALPHA_LM_HEAD, the greedy token of each
                           window token of each budget's final state (budget n_budgets: the
                           full model); -1 for invalid budgets and without the flag */
} knapspec_result;

/* Runs the whole DP for every sequence on the GPU: per item, one batched GEMM over all live
 * budget rows of all sequences (plus each sequence's full-model reference row), attention that
 * streams each layer's KV cache once per sequence for all rows, and the per-budget
 * cosine/select.  Enqueues on args->hip_stream, synchronises once, copies the per-budget
 * results to `result` and runs the TPT grid on the host with a = clamp(cos, 0, 1).
 * Rows are planned from budget reachability.  With tau or the skip cap on (one-state DP, up to
 * 64 sequences) the rows of every item after the first are rebuilt on the device from the
 * previous item's valid flags, so budgets pruned so far leave the attention (and, above 512
 * rows, the MLP GEMMs) -- review, Figure 4 caption: pruning cuts the optimisation work.
 * KNAPSPEC_KEEP_PRUNED_ROWS keeps the reachability plan instead (results agree within
 * floating-point reordering of the attention's context splits; bit-identical when nothing is
 * pruned).
 * The acceptance proxy a = clamp(cos) stands in for the paper's history estimate (Eq. 9),
 * which the pages do not print.  With KNAPSPEC_ALPHA_LM_HEAD (needs knapspec_set_lm_head)
 * the grid instead uses, per budget, the fraction of the window's tokens whose greedy token
 * -- argmax over the LM head of the RMSNorm'd final state, float32 logits, ties to the lower
 * index -- equals the full model's (review, free parameters: the window is used "for DP and
 * acceptance estimation"; reading of Eq. 9).
 * Environment: KNAPSPEC_GRAPHS=0 (read at every solve) launches every kernel eagerly instead
 * of replaying a captured HIP graph; KNAPSPEC_GEMM_AREG (read once per process) selects the
 * GEMM of the K-split projections with 65..256 rows: 3 (default) or 4 stages of activation
 * loads in flight on the register-activation kernel, 0 the LDS-ring kernel (results differ
 * only by the order in which K is summed). */
int knapspec_solve(knapspec_model* model, const knapspec_solve_args* args,
                   knapspec_result* result);

/* knapspec_solve for callers that cannot allocate device memory (code under HIP graph capture
 * of its surroundings, tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * results and errors as knapspec_solve, and the same kernels; the difference is where the
 * per-solve device buffers live (DP states, activation rows, GEMM and attention partial
 * results, decisions, row maps): in one static device array of the library, 64 MiB per GPU,
 * held from the first model load on that GPU until the process ends, instead of the model's
 * workspace.  The call allocates nothing (no hipMalloc / hipFree, no events or graph
 * instantiation; work is launched eagerly on hip_stream).
 * Limits and errors: EINVAL when the model's per-solve buffers (sized at load from
 * max_budgets, max_seqs, max_ctx, max_window, max_beam and the decoder shape) exceed 64 MiB --
 * e.g. a 28-layer, d 2048 decoder loaded for 128 budgets fits, a Llama-3-8B shape for 256
 * budgets does not -- or when profiling is enabled.  Nothing in the array needs to start at
 * zero: every value a solve uses is written earlier in the same solve (launch rows past the
 * live rows of a pruned solve may compute on an earlier call's data; nothing reads their
 * results).  All calls on one GPU
 * share the array: calls that overlap on one GPU (several threads, streams or models) race
 * and must be serialised by the caller. */
int knapspec_solve_static(knapspec_model* model, const knapspec_solve_args* args,
                          knapspec_result* result);

/* LM head for the acceptance estimate: w [vocab][d_model] in desc.dtype, a borrowed device
 * pointer kept alive and unchanged until the model is freed or the head replaced.  The
 * first call allocates the device buffers the estimate needs (a running argmax per row);
 * EINVAL for a NULL pointer or vocab outside [1, 2^24], ENOMEM when allocation fails. */
int knapspec_set_lm_head(knapspec_model* model, const void* w, int32_t vocab);

/* One self-speculative step with a chosen layer set, for measuring its speed (review, "The
 * reading": the draft runs the selected items and the target verifies).  Drafts gamma tokens
 * greedily through the items whose bit is set in mask (ceil(2L/64) words, bit i = item i),
 * each token on one row: executed Attention items append the token's key/value to seq's
 * caches at position ctx_len + t, the LM head gives the greedy token (float32 logits, ties to
 * the lower index) and its LM-head row is the next token's input (tied embeddings).  Then
 * verifies: every item on [x0, e(y_0), .., e(y_{gamma-1})] at positions ctx_len .. ctx_len +
 * gamma as one causal block over the cache 0 .. ctx_len-1 (appending the block's keys/values
 * at those positions), and the LM head's greedy tokens z_0 .. z_gamma.
 * seq: x0 is the current token's input [d] (window <= 1); the caches must hold ctx_len +
 * gamma + 1 positions and are WRITTEN at positions ctx_len .. ctx_len + gamma.  Needs
 * knapspec_set_lm_head; 1 <= gamma <= KNAPSPEC_WINDOW_MAX - 1.
 * Outputs (host): draft_tokens[gamma], verify_tokens[gamma + 1], *accepted = the number of
 * leading t with y_t == z_t, and the device time of the draft and of the verification (HIP
 * events on hip_stream, microseconds).  Synchronises hip_stream.  Uses the model's workspace
 * (do not overlap with a solve on the same model). */
int knapspec_draft_verify(knapspec_model* model, const knapspec_seq* seq, const uint64_t* mask,
                          int32_t gamma, void* hip_stream, int32_t* draft_tokens,
                          int32_t* verify_tokens, int32_t* accepted, double* draft_us,
                          double* verify_us);

/* Host-only TPT grid for caller-supplied acceptance estimates alpha[b] (any a in [0,1]).
 * Ties keep the smaller budget, then the smaller gamma.  Writes -1/-1/NaN when no budget is
 * valid.  Needs no GPU. */
int knapspec_tpt_select(const float* alpha, const double* t_draft, const uint8_t* valid,
                        int32_t n_budgets, double t_target, int32_t gamma_min,
                        int32_t gamma_max, int32_t* best_budget, int32_t* best_gamma,
                        double* best_tpt);

/* Host-only: the launch plan knapspec_solve uses for one GEMM of an item -- `rows` rows,
 * output columns n_cols (2 * d_ff for the SwiGLU gate|up GEMM, swiglu != 0), inner size k,
 * room for cap_floats partial sums (the model's workspace holds max(16 * min(R, 256), R) x
 * the widest N) -- for bf16 (bf16 != 0) or float32 weights.  plan[0..7]: 64-column groups per
 * tile of the LDS-ring kernel (0: another kernel), 32-row blocks per tile, m-tiles, n-tiles, K
 * splits, K per split, activation stages in flight of the register-activation kernel (0: not
 * that kernel), 0.  The KNAPSPEC_GEMM_AREG environment variable (see knapspec_solve) applies.
 * Returns KNAPSPEC_EINVAL on a NULL plan or sizes < 1, KNAPSPEC_EUNSUPPORTED for bf16 sizes
 * that are not multiples of 64 (shapes knapspec_load_model and knapspec_set_lm_head refuse).
 * Needs no GPU. */
int knapspec_gemm_plan(int32_t bf16, int32_t rows, int32_t n_cols, int32_t k, int32_t swiglu,
                       int32_t d_ff, int64_t cap_floats, int32_t* plan);

/* Host-only: the latencies t_i and integer weights w_i one solve uses for a sequence at
 * context length ctx_len (t: 2L doubles, w: 2L int32; either may be NULL).  Needs no GPU. */
int knapspec_item_weights(const knapspec_latency_model* lat, int32_t n_layers, int32_t ctx_len,
                          int32_t n_budgets, double* t, int32_t* w);

/* Device latency profile of the draft pass's items, the measured item latencies the weights
 * come from (review, "The reading": an item's weight is its latency, Attention's growing
 * linearly with the context length and MLP's flat; the paper profiles them once per model).
 * Times one decode token (M = 1 row) through an Attention item -- q|k|v GEMM, RoPE, attention
 * over ctx positions of `seq`'s cache plus its own, O GEMM, residual -- at each context length
 * ctx_lens[0 .. n_ctx-1], and through an MLP item -- gate|up GEMM with SwiGLU, down GEMM,
 * residual -- each `reps` times, bracketed by HIP events on hip_stream.  Repetition r uses
 * layer r mod n_layers, so consecutive repetitions stream different weights.
 * seq: x0 and caches as for knapspec_solve, ctx_capacity >= max(ctx_lens) (ctx_len ignored).
 * Writes attn_us[n_ctx] and *mlp_us: medians over the repetitions, in microseconds.  Uses the
 * model's workspace (do not overlap with a solve on the same model).  1 <= n_ctx <= 1024,
 * 1 <= reps <= 10000; EINVAL for bad arguments, ENOMEM / EHIP for runtime failures. */
int knapspec_profile_items(knapspec_model* model, const knapspec_seq* seq,
                           const int32_t* ctx_lens, int32_t n_ctx, int32_t reps,
                           void* hip_stream, double* attn_us, double* mlp_us);

/* Host-only least-squares line t = a + b*n through (n[i], t[i]), i < count, and its R^2
 * (1 when every t[i] is equal), e.g. to turn knapspec_profile_items' attention latencies into
 * the attn_base / attn_per_token of knapspec_latency_model.  Needs count >= 2 points with at
 * least two distinct n and finite t; EINVAL otherwise. */
int knapspec_fit_latency(const int32_t* n, const double* t, int32_t count, double* a,
                         double* b, double* r2);

/* Measurement hook.  With profiling enabled, knapspec_solve brackets every kernel launch with
 * a pair of HIP events on the solve stream and, after its synchronisation, adds the elapsed
 * time to one of the kernel classes below.  Enabling (enable = 1) resets the counters;
 * knapspec_get_kernel_times copies them (n_classes entries, at most KNAPSPEC_KERNEL_CLASSES).
 * Profiling adds two event records per launch and does not change any result. */
#define KNAPSPEC_KERNEL_CLASSES 10
#define KNAPSPEC_K_INIT 0
#define KNAPSPEC_K_GEMM_QKV 1
#define KNAPSPEC_K_QKV_ROPE 2
#define KNAPSPEC_K_ATTENTION 3
#define KNAPSPEC_K_COMBINE 4
#define KNAPSPEC_K_GEMM_O 5
#define KNAPSPEC_K_GEMM_GATE_UP 6
#define KNAPSPEC_K_GEMM_DOWN 7
#define KNAPSPEC_K_SELECT 8 /* split/residual reduce + cosine select + next-item RMSNorm */
#define KNAPSPEC_K_LM_HEAD 9 /* LM-head GEMM + greedy-token reduction (acceptance estimate) */
int knapspec_set_profiling(knapspec_model* model, int32_t enable);
int knapspec_get_kernel_times(const knapspec_model* model, double* total_ms, int64_t* launches,
                              int32_t n_classes);

int32_t knapspec_mask_words(int32_t n_layers); /* ceil(2L / 64) */
void knapspec_free_model(knapspec_model* model); /* NULL is a no-op */
const char* knapspec_last_error(void);          /* thread-local; "" when none */
int32_t knapspec_abi_version(void);             /* KNAPSPEC_ABI_VERSION */

#ifdef __cplusplus
}
#endif

#endif /* KNAPSPEC_H */
