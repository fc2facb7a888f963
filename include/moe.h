/*
 * moe.h -- C ABI of libmoe, the forward and backward passes of the
 * sparsely-gated noisy top-k Mixture-of-Experts layer on one AMD Instinct
 * MI355X (gfx950).
 *
 * The layer, as the pages on Shazeer et al. 2017 describe it:
 *   - "MoE:稀疏门控混合专家" (nengyongai.cn), section 二: one MoE layer is
 *     y = sum_i G(x)_i E_i(x) over n experts; an expert is a one-hidden-layer
 *     FFN (512 -> 1024 -> 512); experts with gate 0 are not evaluated.
 *   - same page, section 三: scores x W_g (one table column per expert),
 *     KeepTopK sets all but the k best scores to -inf, softmax turns the kept
 *     scores into weights summing to 1; with thousands of experts the gate
 *     picks groups first, then experts inside the chosen groups ("-h").
 *   - same page, section 四: noisy scores
 *     H(x)_i = (x W_g)_i + eps * softplus((x W_noise)_i), eps redrawn per call.
 *   - "Outrageously Large Neural Networks ... 中文验证版" (ai-papers.xuzou.cn),
 *     section 瓶颈: each expert receives about k*b/n rows (the sub-batch that
 *     routing builds); section 方法适配: importance and load losses.
 *   - "MoE 混合专家：参数大、计算省" (transformer.xph.ink), section 核心概念:
 *     the Mixtral-style top-2 layer whose SwiGLU expert variant is provided.
 *
 * Conventions for every entry point:
 *   - Every pointer is a DEVICE pointer to caller-owned memory (or NULL where
 *     a parameter says "nullable").  The library never allocates, frees,
 *     copies to the host or synchronizes; all work is enqueued on `stream`
 *     (a hipStream_t; NULL = the default stream) and results are valid once
 *     the stream has reached that point.
 *   - Scratch memory is the caller's workspace `ws` of `ws_bytes` bytes,
 *     256-byte aligned, at least moe_workspace_size(cfg) bytes.  Its contents
 *     need no initialization and are clobbered.
 *   - Arguments are validated before anything is enqueued.  On error the
 *     call returns a negative moe_status, writes no output and enqueues
 *     nothing; moe_last_error() describes the problem (thread-local).
 *   - Results are deterministic: repeated calls with the same inputs give
 *     bitwise identical outputs (no floating-point atomics).
 *   - Layouts are row-major.  T = tokens, d = d_model, E = n_experts,
 *     h = d_hidden, k = top_k, A = T*k assignments (a = t*k + s for slot s of
 *     token t), G = n_groups, Eg = E/G.
 *   - Element type of x, gate tables and expert tables is cfg->dtype
 *     (MOE_F32 or MOE_BF16).  Gates, scores, noise and bias are float32.
 *
 * Limits: 1 <= k <= 8, k <= E; bf16 needs d % 64 == 0 and h % 64 == 0;
 * tokens < 2^31 / 8.  Anything else returns MOE_ERR_UNSUPPORTED.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, negative size, k > E, ... */
  MOE_ERR_UNSUPPORTED = -2, /* valid layer the library does not implement */
  MOE_ERR_WORKSPACE = -3,   /* ws too small or misaligned */
  MOE_ERR_HIP = -4          /* a HIP launch failed */
} moe_status;

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum moe_ffn {
  MOE_FFN_RELU = 0,  /* E(x) = max(x W1, 0) W2                 */
  MOE_FFN_SWIGLU = 1 /* E(x) = (silu(x W1) * (x W3)) W2        */
} moe_ffn;

typedef struct moe_config {
  int64_t tokens;      /* T >= 0 */
  int32_t d_model;     /* d */
  int32_t n_experts;   /* E */
  int32_t d_hidden;    /* h */
  int32_t top_k;       /* k; for the hierarchy k = k_groups * k_per_group */
  int32_t n_groups;    /* 0 = flat gate; else G groups of E/G experts */
  int32_t k_groups;    /* groups kept per token (hierarchy only) */
  int32_t k_per_group; /* experts kept inside each kept group */
  int32_t noisy;       /* 1 = noisy gating (noise tables and eps given) */
  int32_t ffn;         /* moe_ffn */
  int32_t dtype;       /* moe_dtype */
  int32_t capacity;    /* 0 = none; else rows an expert takes at most: the
                          first `capacity` assignments in token order are
                          kept and the rest dropped (a capacity factor with
                          overflow drop, "MoE 混合专家：参数大、计算省",
                          section 核心概念).  A dropped assignment adds nothing
                          to y; gates are not renormalized; the balance
                          statistics stay those of the gate's choice. */
} moe_config;

/* Gate and expert parameters.  Tables hold one ROW per output unit (the
 * pages' d x n gate table is stored transposed, [E][d]).
 *   w_gate    [E][d]    clean score table W_g
 *   w_noise   [E][d]    noise scale table W_noise (NULL unless noisy)
 *   bias      [E] f32   per-expert score bias added to x W_g (nullable)
 *   w_gate_p  [G][d]    primary (group) score table (hierarchy only)
 *   w_noise_p [G][d]    primary noise table (hierarchy and noisy only)
 *   w1        [E][h][d] first expert layer (ReLU: in; SwiGLU: gate)
 *   w3        [E][h][d] SwiGLU up projection (NULL for ReLU)
 *   w2        [E][d][h] second expert layer (out / down)
 *   w_packed  nullable: w1 and w2 repacked by moe_pack_experts; when given,
 *             the expert stage reads it instead of w1 / w2 (which may then
 *             be NULL).  Same values, laid out in the order the expert
 *             kernel streams them.
 *   w_gate_packed  nullable: w_gate and w_noise repacked by moe_pack_gate;
 *             when given, the gate and smooth-load kernels read it instead
 *             of w_gate / w_noise (which must still be given: the
 *             validation and the fp32 paths use them).  Same values.
 * For the hierarchy, rows g*Eg .. g*Eg+Eg-1 of w_gate / w_noise are the
 * secondary tables of group g. */
typedef struct moe_params {
  const void* w_gate;
  const void* w_noise;
  const float* bias;
  const void* w_gate_p;
  const void* w_noise_p;
  const void* w1;
  const void* w3;
  const void* w2;
  const void* w_packed;
  const void* w_gate_packed;
} moe_params;

/* Noise draws, float32 ~ N(0,1), supplied by the caller (NULL = no noise),
 * or drawn inside the kernels:
 *   eps    flat: [T][E];  hierarchy: [T][G][Eg], only the slices of the
 *          groups a token keeps are read
 *   eps_p  hierarchy: [T][G] primary noise
 *   in_kernel  1: eps / eps_p are not read; every kernel that needs a draw
 *          makes it from a counter-based generator keyed by `seed`:
 *          Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random
 *          Numbers: As Easy as 1, 2, 3", SC 2011).  Element j of the noise
 *          row of token t takes counter (j/4, t, g, stream) (g: the group of
 *          the hierarchy's secondary noise, else 0; stream 1 for eps_p, else
 *          0); output words (0,1) serve elements 4q, 4q+1 and (2,3) elements
 *          4q+2, 4q+3 through Box-Muller, r = sqrt(-2 ln u_a) times
 *          cos(2 pi u_b) (even j) or sin(2 pi u_b) (odd j), with
 *          u = (top 23 bits + 1/2) / 2^23.  moe_draw_noise writes the same
 *          draws out.  A fresh seed per call gives the fresh draw the lesson
 *          page's section 四 asks for. */
typedef struct moe_noise {
  const float* eps;
  const float* eps_p;
  uint64_t seed;
  int32_t in_kernel;
} moe_noise;

/* The generator's draws for `seed` written out: eps [T][E] (flat) or
 * [T][G][Eg] (hierarchy) and eps_p [T][G] (hierarchy), either nullable. */
moe_status moe_draw_noise(const moe_config* cfg, uint64_t seed, float* eps, float* eps_p,
                          void* stream);

/* Bytes of workspace needed by any entry point for this configuration. */
size_t moe_workspace_size(const moe_config* cfg);

/* Gate: noisy scores, KeepTopK and softmax over the kept scores
 * (nengyongai.cn lesson, sections 三 and 四).
 *   x         [T][d]
 *   topk_idx  [T][k] int32 out: kept experts, ascending expert index
 *   topk_gate [T][k] f32 out: their gates (softmax over the kept scores)
 *   thr       [T][2] f32 out, nullable, flat gate only: the k-th and
 *             (k+1)-th largest noisy score (-inf when k == E)
 * Ties between equal scores go to the lower expert index.  The hierarchy
 * keeps k_groups groups by the primary scores, then k_per_group experts in
 * each kept group; a gate is the product of the primary and secondary
 * softmax weights.  A NaN score (from a NaN in x or the tables) ranks as
 * -inf, so every row keeps k experts in [0, E); its gates are then NaN.
 * noise must be non-NULL when cfg->noisy (MOE_ERR_INVALID_ARG otherwise,
 * whatever the token count). */
moe_status moe_gate(const moe_config* cfg, const void* x, const moe_params* p,
                    const moe_noise* noise, int32_t* topk_idx, float* topk_gate,
                    float* thr, void* ws, size_t ws_bytes, void* stream);

/* Route: group the A assignments by expert (the per-expert sub-batch of the
 * paper card, section 瓶颈).
 *   topk_idx  [T][k] int32 in
 *   counts    [E] int32 out: rows per expert
 *   offsets   [E+1] int32 out: exclusive prefix sum of counts
 *   perm      [A] int32 out: perm[p] = assignment placed at position p;
 *             positions are expert-contiguous, tokens ascending inside each
 *             expert (stable)
 *   inv       [A] int32 out: inv[a] = position of assignment a
 *   x, x_sorted  nullable pair: when both are given, x_sorted[p] = x[perm[p]/k]
 * With cfg->capacity > 0: counts and offsets count the kept rows only,
 * inv[a] = -1 for a dropped assignment, and perm[p] = 0 for the positions
 * p >= offsets[E] that no kept assignment takes.  An expert id outside
 * [0, E) in topk_idx is dropped the same way: it takes no row, its inv is -1
 * and it adds nothing downstream. */
moe_status moe_route(const moe_config* cfg, const int32_t* topk_idx,
                     int32_t* counts, int32_t* offsets, int32_t* perm,
                     int32_t* inv, const void* x, void* x_sorted, void* ws,
                     size_t ws_bytes, void* stream);

/* Expert FFNs over the routed rows (lesson page, section 二): for every
 * position p of expert e, y_sorted[p] = E_e(row p), where row p is
 * x[perm[p]/k] when perm is given, else x[p] (x is then the x_sorted of
 * moe_route, [A][d]).  Experts with no rows cost nothing.
 *   offsets   [E+1] int32 from moe_route
 *   y_sorted  [A][d] out (cfg dtype)
 * bf16: products exact in fp32, fp32 accumulation, hidden activations
 * rounded to bf16 before the second layer, outputs rounded to bf16. */
moe_status moe_expert_ffn(const moe_config* cfg, const void* x,
                          const int32_t* perm, const int32_t* offsets,
                          const moe_params* p, void* y_sorted, void* ws,
                          size_t ws_bytes, void* stream);

/* Bytes of the packed expert tables for cfg, or 0 when the configuration
 * has no packed form (packing applies to bf16 ReLU experts with
 * d_model == 512 and d_hidden % 256 == 0). */
size_t moe_packed_experts_size(const moe_config* cfg);

/* Repack p->w1 and p->w2 into `packed` (moe_packed_experts_size bytes,
 * 16-byte aligned) in the fragment order the expert kernel consumes, so
 * that each of its wave-wide weight loads reads 1 KB of contiguous memory.
 * A one-time transform of the parameters; the values are unchanged.
 * Returns MOE_ERR_UNSUPPORTED when the configuration has no packed form. */
moe_status moe_pack_experts(const moe_config* cfg, const moe_params* p, void* packed,
                            void* stream);

/* Bytes of the packed gate tables for cfg, or 0 when the configuration has
 * no packed form (packing applies to bf16 gates with d_model <= 1024). */
size_t moe_packed_gate_size(const moe_config* cfg);

/* Repack p->w_gate (and p->w_noise when cfg->noisy) into `packed`
 * (moe_packed_gate_size bytes, 16-byte aligned) in the fragment order the
 * gate kernels consume, so that each of their wave-wide table loads reads
 * 1 KB of contiguous memory instead of 32 B from each of 32 rows.  A
 * one-time transform of the parameters; the values are unchanged and the
 * gate's results are bitwise those of the unpacked tables.  Layout: per
 * table group g (the hierarchy's groups, else one), per block of 32 experts
 * (the last one padded by repeating its last expert), per 64 columns, per
 * table (gate, then noise), four 1 KB pieces.  Returns MOE_ERR_UNSUPPORTED
 * when the configuration has no packed form. */
moe_status moe_pack_gate(const moe_config* cfg, const moe_params* p, void* packed, void* stream);

/* Combine: y[t] = sum over slots s (ascending) of
 * topk_gate[t][s] * y_sorted[inv[t*k+s]], accumulated in fp32
 * (lesson page, section 二); slots with inv = -1 (dropped by a capacity)
 * add nothing.  y [T][d] out (cfg dtype). */
moe_status moe_combine(const moe_config* cfg, const void* y_sorted,
                       const int32_t* inv, const float* topk_gate, void* y,
                       void* stream);

/* Balance statistics (reading note page, sections 核心想法 / 方法怎么做;
 * paper card, section 方法适配):
 *   importance[e] = sum_t G(x_t)_e
 *   load[e]       = flat noisy gate: sum_t Phi((clean[t,e] - theta[t,e]) /
 *                   softplus(x_t W_noise)_e), clean = x W_g + bias, theta =
 *                   thr[t][1] if e is kept by token t else thr[t][0];
 *                   otherwise (no noise, or hierarchy): counts[e]
 *   out[0] = CV^2(importance), out[1] = CV^2(load),
 *   out[2] = w_importance * out[0] + w_load * out[1]
 * CV^2 = population variance / mean^2 (0 when the mean is 0).
 * Inputs: x, p (w_gate, w_noise, bias) and thr are used only for the smooth
 * load; perm/offsets from moe_route without a capacity (the statistics
 * describe the gate's choice); topk_idx/topk_gate/thr from moe_gate.
 * importance, load [E] f32 out; out [3] f32 out. */
moe_status moe_balance_loss(const moe_config* cfg, const void* x,
                            const moe_params* p, const int32_t* topk_idx,
                            const float* topk_gate, const float* thr,
                            const int32_t* perm, const int32_t* offsets,
                            float w_importance, float w_load, float* importance,
                            float* load, float* out, void* ws, size_t ws_bytes,
                            void* stream);

/* Outputs of moe_forward.  y is required; the rest are nullable (the
 * library then keeps them in the workspace).  The last five are what
 * moe_backward reads back (see moe_saved). */
typedef struct moe_outputs {
  void* y;            /* [T][d] */
  int32_t* topk_idx;  /* [T][k] */
  float* topk_gate;   /* [T][k] */
  int32_t* counts;    /* [E] */
  float* importance;  /* [E]; balance statistics are computed only when */
  float* load;        /* [E]; `balance` is non-NULL */
  float* balance;     /* [3]: cv2 importance, cv2 load, weighted loss */
  float* thr;         /* [T][2] flat gate: k-th and (k+1)-th noisy score */
  int32_t* offsets;   /* [E+1] routing offsets */
  int32_t* perm;      /* [A] routing permutation */
  int32_t* inv;       /* [A] its inverse */
  void* y_sorted;     /* [A][d] expert outputs in routed order */
} moe_outputs;

/* The whole layer: gate -> route -> experts -> combine (-> balance).
 * Streams: the work is ordered on `stream`.  For a flat noisy gate with more
 * than 256 experts and the balance statistics on, the smooth load's
 * recompute and the balance reduction run on the device's second stream
 * (the one moe_backward uses for its expert side), forked from `stream`
 * after the gate and joined back to it with events before the call returns,
 * on error paths too. */
moe_status moe_forward(const moe_config* cfg, const void* x,
                       const moe_params* p, const moe_noise* noise,
                       float w_importance, float w_load, moe_outputs* out,
                       void* ws, size_t ws_bytes, void* stream);

/* ---- Forward pass that allocates nothing --------------------------------
 * For callers that cannot allocate: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  moe_forward_static is
 * moe_forward (same arguments without ws / ws_bytes, same kernels, bitwise
 * the same results) with its scratch in a static device array of
 * MOE_FORWARD_STATIC_SCRATCH_BYTES inside the library: each GPU the library
 * runs on holds one such array until the process ends.  It calls no
 * allocating routine.  The array of the current device is used, so `stream`
 * must belong to the current device.
 *   - Returns MOE_ERR_WORKSPACE, enqueueing nothing, when the layer needs more
 *     scratch than that (moe_workspace_size(cfg) > the limit; for example the
 *     8192-token, 256-expert, d_model 512 layer needs about 34 MiB).
 *   - Every call on one GPU shares that GPU's array: calls that overlap on
 *     one GPU (on different streams, or from several threads without
 *     ordering) race and give wrong results.  Calls ordered on one stream are
 *     safe.  The array needs no initialization; each call overwrites what it
 *     uses.
 *   - The first call on a device looks the array's address up (thread-safe)
 *     and keeps it; a failure there returns MOE_ERR_HIP. */
#define MOE_FORWARD_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

moe_status moe_forward_static(const moe_config* cfg, const void* x,
                              const moe_params* p, const moe_noise* noise,
                              float w_importance, float w_load, moe_outputs* out,
                              void* stream);

/* ---- Per-batch equal-size expert mask ------------------------------------
 * In place of KeepTopK, the flat layer's experts choose their tokens
 * ("Outrageously Large Neural Networks: The Sparsely-Gated Mixture-of-Experts
 * Layer - 中文验证版", ai-papers.xuzou.cn, section 方法适配: in some
 * translation runs a per-batch mask gives every expert the same batch size in
 * training, and per-expert thresholds approximate that mask at inference):
 *   batch mask (thresholds == NULL): expert e keeps the rows_per_expert = m
 *     tokens of the batch with the largest noisy scores H[:, e] (ties: the
 *     lower token), so every expert receives exactly m rows;
 *   threshold mask (thresholds [E] f32 given): expert e keeps every token
 *     with H[t, e] >= thresholds[e]; the first m of them in token order take
 *     rows, later ones are dropped and add nothing to y.
 * A token's gates are the softmax over the scores of the experts that kept
 * it; a token kept by no expert gets y = 0.  The balance statistics are
 * importance[e] = sum of e's gates over the batch and load[e] = the number of
 * tokens e kept (before the cap), CV^2 and the weighted loss as in
 * moe_balance_loss.  H, the projections and the noise are those of moe_gate
 * (same tables, bias, noise and packed tables).  Flat gate only
 * (cfg->n_groups == 0); cfg->capacity must be 0 (m sets the rows);
 * cfg->top_k is not used.  1 <= m <= tokens (any m >= 1 for an empty batch).
 * A NaN score ranks as -inf.  Rows: at most R = E * m. */
typedef struct moe_mask_outputs {
  void* y;                 /* [T][d], required when T > 0 */
  int32_t* counts;         /* [E] rows of each expert (nullable, as all below) */
  int32_t* offsets;        /* [E+1] exclusive prefix sum of counts */
  int32_t* perm;           /* [R] token of each row: expert-contiguous, tokens
                              ascending inside an expert; rows past offsets[E]
                              hold 0 */
  int32_t* tok_offsets;    /* [T+1] token t's slots are [tok_offsets[t],
                              tok_offsets[t+1]) */
  int32_t* slot_expert;    /* [R] expert of each slot, ascending in a token */
  float* slot_gate;        /* [R] its gate */
  int32_t* slot_row;       /* [R] its row (position in expert order) */
  float* importance;       /* [E]; the statistics are computed only when */
  float* load;             /* [E]; `balance` is non-NULL */
  float* balance;          /* [3]: cv2 importance, cv2 load, weighted loss */
} moe_mask_outputs;

/* Bytes of workspace moe_forward_mask needs (0 for an invalid request). */
size_t moe_mask_workspace_size(const moe_config* cfg, int32_t rows_per_expert);

moe_status moe_forward_mask(const moe_config* cfg, const void* x, const moe_params* p,
                            const moe_noise* noise, int32_t rows_per_expert,
                            const float* thresholds, float w_importance, float w_load,
                            moe_mask_outputs* out, void* ws, size_t ws_bytes, void* stream);

/* ---- Backward pass -------------------------------------------------------
 * Gradients of L = sum(dy * y) + w_importance * CV^2(importance) +
 * w_load * CV^2(load) for the flat gate or the hierarchy, ReLU or SwiGLU
 * experts, bf16 or fp32.  dy is the gradient flowing into y from above; the
 * balance losses are those moe_balance_loss defines, added to the objective
 * with the given weights.  The choice of kept experts has no gradient (the
 * reading note "Outrageously Large Neural Networks — MoE 怎样让模型“很大但
 * 不每次全算”", section 问题是什么): the kept set and the experts ranked k-th
 * and (k+1)-th are held fixed, and gradients flow through the softmax over the
 * kept scores, the noisy scores (section 方法怎么做: the learnable noise), the
 * smooth load estimate (whose threshold passes its gradient to the score it
 * was read from) and the experts.  Hidden activations are recomputed, not
 * saved (paper card, section 瓶颈: activation recomputation).  In the
 * hierarchy a kept gate is the product of the primary (group) and secondary
 * (expert) softmax weights; the product passes its gradient to both levels,
 * each of which then differentiates like a flat gate over its kept scores.
 * The hierarchy's load is a hard count, so w_load adds no gradient there, and
 * the secondary tables' gradients cover every kept (token, expert) pair of
 * the gate's choice, dropped by a capacity or not.
 *
 * Tensors saved from the forward pass of the same inputs (moe_forward with
 * the matching moe_outputs fields, or the staged calls). */
typedef struct moe_saved {
  const int32_t* topk_idx;  /* [T][k] */
  const float* topk_gate;   /* [T][k] */
  const float* thr;         /* [T][2]; needed when noisy and w_load != 0 */
  const int32_t* offsets;   /* [E+1] */
  const int32_t* perm;      /* [A] */
  const int32_t* inv;       /* [A] */
  const void* y_sorted;     /* [A][d] */
  const float* importance;  /* [E]; needed when w_importance != 0 */
  const float* load;        /* [E]; needed when noisy and w_load != 0 */
} moe_saved;

/* Gradient outputs.  dx is required; the others are nullable (not
 * computed).  Element type: cfg dtype, except dbias (float32).  Experts
 * that receive no rows get zero table gradients. */
typedef struct moe_grads {
  void* dx;        /* [T][d] */
  void* dw_gate;   /* [E][d] */
  void* dw_noise;  /* [E][d] (noisy only) */
  float* dbias;    /* [E] (flat gate only) */
  void* dw1;       /* [E][h][d] */
  void* dw3;       /* [E][h][d] (SwiGLU only) */
  void* dw2;       /* [E][d][h] */
  void* dw_gate_p;   /* [G][d] (hierarchy only) */
  void* dw_noise_p;  /* [G][d] (hierarchy and noisy only) */
} moe_grads;

/* Bytes of workspace moe_backward needs for this configuration (0 for an
 * invalid configuration). */
size_t moe_backward_workspace_size(const moe_config* cfg);

/* The backward pass.  x, p (w_gate, w_noise, bias, w1, w2, w3, and for the
 * hierarchy w_gate_p, w_noise_p; the unpacked w1 / w2 / w3 are required, and
 * the packed tables are optional: w_gate_packed for the gate, w_packed for
 * the W1 reads of the ReLU hidden layer's recompute at d_model 512), noise
 * (eps, and eps_p for the hierarchy, when noisy) and `saved` are the
 * forward's inputs and saved tensors (thr is not needed by the hierarchy);
 * dy [T][d] is in the cfg dtype.  Returns MOE_ERR_UNSUPPORTED for fp32
 * layers whose d_model or d_hidden is not a multiple of 4.  The hierarchy's
 * gate side runs in fp32 arithmetic for both dtypes.  bf16: products on MFMA
 * with fp32 accumulation; fp32 operands (score gradients) and gate-scaled
 * output gradients are rounded to bf16 as they enter a product, the hidden
 * activation and its gradients are rounded to bf16 between products.
 * Streams: the work is ordered on `stream`.  The expert-side products run on
 * a second stream of the current device (created by the device's first call,
 * non-blocking, default priority, kept until the process ends), forked from
 * `stream` and joined back to it with events before the call's last kernel,
 * on error paths too; calls on one device share that stream, so their
 * expert sides run one after another. */
moe_status moe_backward(const moe_config* cfg, const void* x, const moe_params* p,
                        const moe_noise* noise, const moe_saved* saved, const void* dy,
                        float w_importance, float w_load, moe_grads* grads, void* ws,
                        size_t ws_bytes, void* stream);

/* Static text for a status code. */
const char* moe_status_string(int status);

/* Detail of the last error returned on this thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
