/*
 * libmoe — Mixture-of-Experts layer forward on one AMD Instinct MI355X (gfx950).
 *
 * The layer is the token-choice MoE block of the Qwen3 family as the pages
 * state it:
 *   - Qwen3-Omni issue #115 ("Training: Extremely Slow Deepspeed Engine
 *     initialization ..."), SpeedupMoeSparseMoeBlock.forward: gate -> float32
 *     softmax -> top-k -> optional renormalisation (norm_topk_prob); and
 *     SpeedupMoeExperts: concatenated experts gate_up_proj [E, H, 2I] (gate in
 *     columns [0, I), up in [I, 2I)) and down_proj [E, I, H], SwiGLU
 *     up * silu(gate), outputs weighted by the routing weights and added into
 *     the token rows;
 *   - MindSpore hyper-parallel moe.py page: TokenChoiceTopKRouter.forward
 *     (returns routing weights, expert ids, tokens per expert),
 *     MoE.permutation (stable token-major -> expert-major order),
 *     GroupedExperts / _run_experts_for_loop (per-expert SwiGLU over rows in
 *     expert-major order split by counts), MoE.unpermutation (add back);
 *   - transformers PR "Qwen3 moe", Ep2DpParallel._token_dispatch: the rows one
 *     expert-parallel rank receives come grouped by source rank and must be
 *     reshuffled to expert-major order before the grouped experts.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers to row-major, contiguous
 *     buffers, 16-byte aligned, allocated and owned by the caller.  The
 *     library allocates nothing, frees nothing and never synchronises the
 *     host; all work is enqueued on `stream` in order.
 *   - Every argument is validated before anything is enqueued.  On error the
 *     call returns a negative status (below) and enqueues nothing.  A status of
 *     MOE_ERR_HIP means a launch failed after validation.
 *   - T = 0 (or N = 0) is a valid no-op apart from zero-filling outputs that
 *     are defined for every expert (counts, offsets).
 *   - Device-side contents (expert ids, counts, offsets) cannot be validated
 *     on the host; kernels clamp every index they derive from them, so
 *     inconsistent contents give unspecified values but never out-of-bounds
 *     accesses.
 *   - dtype MOE_BF16: hidden states, weights, expert outputs and the layer
 *     output are bfloat16; router logits and routing weights are float32;
 *     all accumulation is float32.  dtype MOE_F32: everything float32.
 *   - Shape limits: 1 <= top_k <= E <= 256; H a multiple of 128 and I a
 *     multiple of 64 (the router alone needs only H a multiple of 64);
 *     routed rows N <= 2^30; rank-major mode R * E <= 4096.
 *   - Calls are stateless and may be made from several host threads on
 *     different streams (moe_layer_forward_noalloc excepted: its calls on
 *     one GPU share a static scratch buffer; see there).
 */
#ifndef LIBMOE_H
#define LIBMOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
  MOE_ERR_DTYPE = -3,       /* unknown dtype */
  MOE_ERR_WORKSPACE = -4,   /* workspace missing or smaller than moe_workspace_size() */
  MOE_ERR_UNSUPPORTED = -5, /* valid request this build does not handle */
  MOE_ERR_HIP = -6,         /* a HIP launch failed */
  MOE_ERR_ALIGN = -7,       /* a pointer is not 16-byte aligned */
  MOE_ERR_SCRATCH = -8      /* moe_layer_forward_noalloc: the request needs more
                               than MOE_STATIC_SCRATCH_BYTES of workspace */
};

/* Workspace queries: `op` names the entry point. */
enum {
  MOE_OP_ROUTE = 0,
  MOE_OP_PERMUTE = 1,
  MOE_OP_GATE_UP = 2,
  MOE_OP_DOWN = 3,
  MOE_OP_GROUPED_SWIGLU = 4,
  MOE_OP_LAYER = 5,
  MOE_OP_SHARED = 6,
  MOE_OP_LAYER_BACKWARD = 7
};

/* Bytes of device workspace entry point `op` needs for these sizes.
 * N is the number of routed rows (T * top_k for token choice; for the
 * rank-major permutation and the grouped calls, the caller's row count).
 * R is the number of source ranks for the rank-major permutation; for
 * MOE_OP_LAYER it is the shared expert's intermediate size (0: none); else 0.
 * For MOE_OP_SHARED, I is the shared expert's intermediate size.
 * Returns 0 if the op needs none, (size_t)-1 for invalid sizes. */
size_t moe_workspace_size(int op, int T, int H, int I, int E, int top_k, int R,
                          int N, moe_dtype dt);

/* Human-readable text for a status code (static storage). */
const char* moe_status_string(int status);

/* Library ABI version (increments on any signature change). */
int moe_version(void);

/*
 * moe_route — router GEMM, float32 softmax, top-k, renormalisation.
 * Qwen3-Omni issue #115, SpeedupMoeSparseMoeBlock.forward; MindSpore moe.py,
 * TokenChoiceTopKRouter.forward (softmax scoring).
 *
 *   router_logits[t, e] = sum_h hidden_states[t, h] * router_weight[e, h]
 *                         + router_bias[e]                      (float32)
 *   topk_ids[t, 0..k-1]  = the k experts with the largest logits, in order of
 *                          decreasing logit; equal logits (-0 == +0) go to the
 *                          lower expert id.
 *   topk_weights[t, j]   = softmax(router_logits[t, :])[topk_ids[t, j]],
 *                          divided by the sum over j when norm_topk_prob != 0.
 *   num_tokens_per_expert[e] = number of (t, j) with topk_ids[t, j] == e.
 *
 * hidden_states [T, H] dt; router_weight [E, H] dt (nn.Linear(H, E) layout);
 * router_bias [E] float32 or NULL (no bias); router_logits [T, E] float32 or
 * NULL (not written); topk_ids [T, k] int32; topk_weights [T, k] float32;
 * num_tokens_per_expert [E] int32 or NULL.  No workspace.
 */
int moe_route(const void* hidden_states, const void* router_weight,
              const float* router_bias, int T, int H, int E, int top_k,
              int norm_topk_prob, moe_dtype dt, float* router_logits,
              int32_t* topk_ids, float* topk_weights,
              int32_t* num_tokens_per_expert, hipStream_t stream);

/*
 * moe_permute — expert histogram, offsets and the expert-major permutation.
 * MindSpore moe.py, MoE.permutation (stable argsort of the flattened expert
 * ids, token = flat index // top_k, bincount); transformers PR "Qwen3 moe",
 * Ep2DpParallel._token_dispatch (rank-major received rows).
 *
 * Token-choice mode (topk_ids != NULL, rank_major_counts == NULL):
 *   N = T * top_k flat slots i = t * top_k + j with expert topk_ids[t, j].
 *   Expert-major order lists, for e = 0..E-1, the slots with expert e in
 *   ascending i.  For expert-major position p:
 *     sorted_slot_ids[p]  = i,   sorted_token_ids[p] = i / top_k,
 *     slot_pos[i] = p.
 * Rank-major mode (topk_ids == NULL, rank_major_counts != NULL):
 *   N received rows laid out as blocks (source rank r = 0..R-1, local expert
 *   e = 0..E-1) of rank_major_counts[r, e] rows (int32 [R, E], device).
 *   Expert-major order lists blocks (e, r) with each block's order kept.
 *     sorted_slot_ids[p] = sorted_token_ids[p] = received row i,
 *     slot_pos[i] = p.   Sum of rank_major_counts must equal N.
 * Both modes: num_tokens_per_expert [E] int32, expert_offsets [E + 1] int32
 * (exclusive prefix sum, expert_offsets[E] = N); sorted_token_ids,
 * sorted_slot_ids, slot_pos [N] int32.  sorted_slot_ids may be NULL.
 * Workspace: moe_workspace_size(MOE_OP_PERMUTE, ...).  Deterministic.
 */
int moe_permute(const int32_t* topk_ids, int T, int top_k,
                const int32_t* rank_major_counts, int R, int N, int E,
                int32_t* num_tokens_per_expert, int32_t* expert_offsets,
                int32_t* sorted_token_ids, int32_t* sorted_slot_ids,
                int32_t* slot_pos, void* workspace, size_t workspace_bytes,
                hipStream_t stream);

/*
 * moe_gather_rows — x_perm[p, :] = x[row_index[p], :] (MindSpore moe.py,
 * MoE.forward: routed_x = x_flat[token_indices]).  Optional: the grouped
 * GEMMs gather rows on load and never need x_perm.
 * x [x_rows, H] dt; row_index [N] int32 (clamped to [0, x_rows)); x_perm
 * [N, H] dt.
 */
int moe_gather_rows(const void* x, int x_rows, const int32_t* row_index, int N,
                    int H, moe_dtype dt, void* x_perm, hipStream_t stream);

/*
 * moe_grouped_gate_up_swiglu — first grouped GEMM with the SwiGLU fused.
 * Qwen3-Omni issue #115, SpeedupMoeExperts.forward (gate_up = state @
 * gate_up_proj[e]; gate, up = chunk(2); up * silu(gate)); MindSpore moe.py,
 * _run_experts_for_loop.
 *   For each expert e and expert-major row p in [expert_offsets[e],
 *   expert_offsets[e+1]):  g = x[row(p)] @ gate_up[e]  (float32 accumulate),
 *   h[p, n] = silu(g[n]) * g[I + n]  for n < I, rounded to dt.
 *   row(p) = row_index[p], or p when row_index is NULL.
 * x [x_rows, H] dt (row indices are clamped to [0, x_rows)); expert_offsets
 * [E + 1] int32 (device); gate_up [E, H, 2I] dt;
 * h [N, I] dt.  Empty experts are skipped.  Workspace:
 * moe_workspace_size(MOE_OP_GATE_UP, ...).
 */
int moe_grouped_gate_up_swiglu(const void* x, int x_rows, const int32_t* row_index,
                               const int32_t* expert_offsets, int N, int H,
                               int I, int E, const void* gate_up, moe_dtype dt,
                               void* h, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * moe_grouped_down — second grouped GEMM (Qwen3-Omni issue #115,
 * SpeedupMoeExperts.forward: expert_out = gated_output @ down_proj[e]).
 *   y[dst(p), :] = h[p, :] @ down[e]   for p in expert e's rows,
 *   dst(p) = out_index[p], or p when out_index is NULL (expert-major y).
 * h [N, I] dt; down [E, I, H] dt; y [N, H] dt.  out_index must be a
 * permutation of [0, N).  Workspace: moe_workspace_size(MOE_OP_DOWN, ...).
 */
int moe_grouped_down(const void* h, const int32_t* expert_offsets,
                     const int32_t* out_index, int N, int H, int I, int E,
                     const void* down, moe_dtype dt, void* y, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/*
 * moe_grouped_swiglu — both grouped GEMMs: y[dst(p)] = SwiGLU_e(x[row(p)]).
 * Intermediate h lives in the workspace
 * (moe_workspace_size(MOE_OP_GROUPED_SWIGLU, ...)).  With row_index =
 * out_index = the rank-major permutation's sorted_token_ids this is one
 * expert-parallel rank's reshuffle -> experts -> reverse reshuffle, with the
 * row moves fused into the GEMM loads and stores.
 */
int moe_grouped_swiglu(const void* x, int x_rows, const int32_t* row_index,
                       const int32_t* out_index, const int32_t* expert_offsets,
                       int N, int H, int I, int E, const void* gate_up,
                       const void* down, moe_dtype dt, void* y, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/*
 * moe_combine — weighted un-permute (Qwen3-Omni issue #115: expert_out *
 * routing_weights, index_add_ into the token rows; MindSpore moe.py,
 * MoE.unpermutation).
 *   out[t, :] = sum_{j = 0..k-1} w[t, j] * y[src(t, j), :]
 * accumulated in float32 in ascending j, rounded once to dt; no atomics, so
 * bitwise deterministic.  src(t, j) = slot_pos[t * k + j], or t * k + j when
 * slot_pos is NULL (y already in flat-slot order).  w = topk_weights [T, k]
 * float32, or 1 when NULL (plain un-permute).  y [N, H] dt; out [T, H] dt.
 */
int moe_combine(const void* y, const int32_t* slot_pos,
                const float* topk_weights, int T, int top_k, int H,
                moe_dtype dt, void* out, hipStream_t stream);

/*
 * moe_layer_forward — the whole layer: moe_route, moe_permute (token
 * choice), the two grouped GEMMs (rows gathered on load, outputs stored in
 * flat-slot order) and moe_combine.  Qwen3-Omni issue #115,
 * SpeedupMoeSparseMoeBlock.forward returns (out, router_logits).
 * out [T, H] dt; router_logits [T, E] float32, topk_ids [T, k] int32,
 * topk_weights [T, k] float32 and num_tokens_per_expert [E] int32 are written
 * when non-NULL (the workspace holds them otherwise).  Workspace:
 * moe_workspace_size(MOE_OP_LAYER, ...).
 * stage_events: NULL, or an array of 6 caller-created HIP events recorded on
 * `stream` before the router, the permutation, the first GEMM, the second
 * GEMM and the combine, and after the combine (for per-stage timing; NULL
 * entries are skipped).  The library neither creates nor destroys them.
 */
int moe_layer_forward(const void* hidden_states, const void* router_weight,
                      const float* router_bias, const void* gate_up,
                      const void* down, int T, int H, int I, int E, int top_k,
                      int norm_topk_prob, moe_dtype dt, void* out,
                      float* router_logits, int32_t* topk_ids,
                      float* topk_weights, int32_t* num_tokens_per_expert,
                      void* workspace, size_t workspace_bytes,
                      hipEvent_t* stage_events, hipStream_t stream);

/*
 * Router variants — MindSpore hyper-parallel moe.py page,
 * TokenChoiceTopKRouter.forward and _get_node_limited_routing_scores
 * (auxiliary-loss-free load balancing: MoE.update_expert_bias).
 *
 *   score[t, e] = score_func(router_logits[t, e]) * route_scale, where
 *                 score_func is a sigmoid, or a softmax over the experts;
 *   with num_expert_groups = G > 0 the experts form G contiguous groups of
 *   E / G, a group's score is its largest expert score, and only the
 *   num_limited_groups groups with the largest group scores (equal scores:
 *   lower group first) stay selectable for the token;
 *   topk_ids[t, :]   = the top_k selectable experts by score + expert_bias
 *                      (bias for selection only; equal keys: lower id first),
 *                      in decreasing key order; keys are float32;
 *   topk_weights     = the unbiased scores of those experts, divided by
 *                      their sum when norm_topk_prob != 0;
 *   tokens_per_expert (float [E], optional) += selections per expert.
 *
 * All pointers in the struct are device pointers (or NULL); expert_bias and
 * tokens_per_expert have E entries.  Requirements: score_func is one of the
 * two constants, route_scale is finite, and with G > 0: E % G == 0,
 * 1 <= num_limited_groups <= G and top_k <= num_limited_groups * E / G.
 * Violations return MOE_ERR_SHAPE (or MOE_ERR_UNSUPPORTED for an unknown
 * score_func) before anything is enqueued.
 */
enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 };

typedef struct moe_router_config {
  int score_func;
  float route_scale;
  const float* expert_bias;
  int num_expert_groups;
  int num_limited_groups;
  float* tokens_per_expert;
} moe_router_config;

/* moe_route with a router variant.  cfg == NULL is exactly moe_route (the
 * softmax router that ranks the logits).  router_bias is added to the
 * logits (it is part of router_logits); cfg->expert_bias only steers
 * selection. */
int moe_route_cfg(const void* hidden_states, const void* router_weight,
                  const float* router_bias, int T, int H, int E, int top_k,
                  int norm_topk_prob, moe_dtype dt, const moe_router_config* cfg,
                  float* router_logits, int32_t* topk_ids, float* topk_weights,
                  int32_t* num_tokens_per_expert, hipStream_t stream);

/* moe_layer_forward with a router variant (cfg == NULL: moe_layer_forward).
 * The combine weights each expert output by topk_weights as above. */
int moe_layer_forward_cfg(const void* hidden_states, const void* router_weight,
                          const float* router_bias, const void* gate_up,
                          const void* down, int T, int H, int I, int E, int top_k,
                          int norm_topk_prob, moe_dtype dt, const moe_router_config* cfg,
                          void* out, float* router_logits, int32_t* topk_ids,
                          float* topk_weights, int32_t* num_tokens_per_expert,
                          void* workspace, size_t workspace_bytes,
                          hipEvent_t* stage_events, hipStream_t stream);

/*
 * moe_update_expert_bias — one auxiliary-loss-free bias step (MindSpore
 * moe.py, MoE.update_expert_bias), in place on device float arrays of E
 * entries (1 <= E <= 256):
 *   load = tokens_per_expert / num_recomputations   (when it is > 1)
 *   step[e] = lr * sign(mean(load) - load[e]);  step -= mean(step)
 *   expert_bias += step;  tokens_per_expert = 0
 * Sums are float32 in a fixed order.  MOE_ERR_NULL / MOE_ERR_SHAPE on bad
 * arguments.
 */
int moe_update_expert_bias(float* expert_bias, float* tokens_per_expert, int E, float lr,
                           int num_recomputations, hipStream_t stream);

/*
 * Shared expert — MindSpore moe.py, FeedForward (a SwiGLU feed-forward that
 * every token passes through) and MoE.forward (its output is added to the
 * unpermuted routed output, without a routing weight).
 *
 * With nn.Linear weights w1, w3 [Is, H] and w2 [H, Is], FeedForward is
 *   shared(x) = w2(silu(w1 x) * w3 x).
 * The library takes them transposed, in the routed experts' layout:
 *   gate_up [H, 2 * Is] dt: columns [0, Is) are w1^T (gate), [Is, 2 * Is)
 *                           are w3^T (up);
 *   down    [Is, H] dt:     w2^T.
 * Is (intermediate_size) must be a positive multiple of 64.
 */
typedef struct moe_shared_expert {
  const void* gate_up;
  const void* down;
  int intermediate_size;
} moe_shared_expert;

/* The shared expert alone on T tokens: out [T, H] dt = shared(x) for each
 * row, the hidden h [T, Is] rounded to dt between the two GEMMs (as the
 * routed experts do), float32 accumulation.  Workspace:
 * moe_workspace_size(MOE_OP_SHARED, T, H, Is, 1, 1, 0, T, dt). */
int moe_shared_expert_forward(const void* hidden_states, const void* gate_up,
                              const void* down, int T, int H, int Is, moe_dtype dt,
                              void* out, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* moe_layer_forward_cfg plus an optional shared expert (shared == NULL: no
 * shared expert, exactly moe_layer_forward_cfg).  With one,
 *   out[t, :] = sum_j w[t, j] * y[t * k + j, :] + shared(x[t, :])
 * where shared(x) is rounded to dt and joins the combine's float32 sum last,
 * before the single rounding of out.  Workspace:
 * moe_workspace_size(MOE_OP_LAYER, T, H, I, E, top_k, Is, T * top_k, dt).
 * For bf16 with Is a multiple of 128 the shared expert's GEMMs run inside
 * the two grouped launches (stage events 2-3 and 3-4); otherwise they run
 * on their own between stage events 4 and 5, before the combine. */
int moe_layer_forward_ex(const void* hidden_states, const void* router_weight,
                         const float* router_bias, const void* gate_up,
                         const void* down, int T, int H, int I, int E, int top_k,
                         int norm_topk_prob, moe_dtype dt, const moe_router_config* cfg,
                         const moe_shared_expert* shared, void* out, float* router_logits,
                         int32_t* topk_ids, float* topk_weights,
                         int32_t* num_tokens_per_expert, void* workspace,
                         size_t workspace_bytes, hipEvent_t* stage_events,
                         hipStream_t stream);

/*
 * moe_layer_forward_noalloc — moe_layer_forward_ex for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It takes no workspace argument and
 * calls no allocating routine (hipMalloc, hipFree or any library that
 * allocates); its workspace is a static device array of
 * MOE_STATIC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends.  Arguments, outputs and results are those of
 * moe_layer_forward_ex (bit-identical for the same inputs).  The caller still
 * passes (and owns) every input and output.
 *   - The array of the CURRENT device is used: the stream must belong to the
 *     device that is current when the call is made.
 *   - A request whose moe_workspace_size(MOE_OP_LAYER, ...) exceeds
 *     MOE_STATIC_SCRATCH_BYTES returns MOE_ERR_SCRATCH and enqueues nothing
 *     (at the Qwen3-30B-A3B expert shape, H = 2048, I = 768, top-8, that is
 *     above 1,344 tokens; 1,208 with a 768-wide shared expert).
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents.  Calls that overlap on one GPU (on several streams,
 *     or from several host threads without ordering) race on it; serialise
 *     them on one stream.
 *   - The first call on a device looks up the array's device address
 *     (hipGetSymbolAddress); a failure there returns MOE_ERR_HIP.
 */
#define MOE_STATIC_SCRATCH_BYTES (64u << 20)

int moe_layer_forward_noalloc(const void* hidden_states, const void* router_weight,
                              const float* router_bias, const void* gate_up,
                              const void* down, int T, int H, int I, int E, int top_k,
                              int norm_topk_prob, moe_dtype dt, const moe_router_config* cfg,
                              const moe_shared_expert* shared, void* out, float* router_logits,
                              int32_t* topk_ids, float* topk_weights,
                              int32_t* num_tokens_per_expert, hipEvent_t* stage_events,
                              hipStream_t stream);

/*
 * moe_layer_workspace_offset — where the layer forward keeps its own
 * permutation and expert outputs inside its workspace, for callers that
 * inspect them after the call (the layer's stream must have reached the end
 * of the call).  These are the values moe_permute would return for the
 * call's topk_ids (MindSpore moe.py, MoE.permutation) and the second grouped
 * GEMM's outputs before the combine (Qwen3-Omni issue #115,
 * SpeedupMoeExperts.forward, expert_out before it is weighted):
 *   MOE_LAYER_WS_OFFSETS       int32 [E + 1] expert_offsets
 *   MOE_LAYER_WS_SORTED_TOKEN  int32 [T*k]   sorted_token_ids
 *   MOE_LAYER_WS_SORTED_SLOT   int32 [T*k]   sorted_slot_ids
 *   MOE_LAYER_WS_SLOT_POS      int32 [T*k]   slot_pos
 *   MOE_LAYER_WS_EXPERT_OUT    dt [T*k, H]   expert outputs, row t*k + j
 *                                            (not written by the training
 *                                            forward, which puts them in
 *                                            moe_train_saved.expert_out)
 * Arguments as moe_workspace_size(MOE_OP_LAYER, T, H, I, E, top_k, shared_I,
 * T*top_k, dt).  Returns the byte offset from the start of the workspace
 * (256-byte aligned), or (size_t)-1 for an unknown piece or invalid sizes.
 * Pure host computation; enqueues nothing.
 */
enum {
  MOE_LAYER_WS_OFFSETS = 0,
  MOE_LAYER_WS_SORTED_TOKEN = 1,
  MOE_LAYER_WS_SORTED_SLOT = 2,
  MOE_LAYER_WS_SLOT_POS = 3,
  MOE_LAYER_WS_EXPERT_OUT = 4
};

size_t moe_layer_workspace_offset(int piece, int T, int H, int I, int E, int top_k,
                                  int shared_I, moe_dtype dt);

/*
 * Training: the layer forward that keeps what its backward needs, and the
 * backward.  The pages train this layer through autograd (Qwen3-Omni issue
 * #115, SpeedupMoeExperts' per-expert training loop and
 * SpeedupMoeSparseMoeBlock's softmax routing weights; MindSpore moe.py,
 * MoE.forward, MoE.unpermutation and FeedForward); the backward is the
 * gradient of sum(dout * out) for the layer with the default router
 * (softmax, optionally renormalised, optional router_bias) or a router
 * variant (cfg: sigmoid or softmax scores times route_scale; the expert bias
 * and the group limit steer the selection only), with or without a shared
 * expert.  The top-k choice is piecewise constant: gradients flow through
 * the routing weights' values.
 * bf16 only, I and Is multiples of 128 (else MOE_ERR_UNSUPPORTED).
 *
 * moe_layer_forward_train: moe_layer_forward_ex (router variant cfg and
 * shared expert optional) that also keeps, in the caller's buffers of
 * moe_train_saved:
 *   gate_up_out        [T*k, 2I] dt: the gate/up pre-activations x.gate_up[e]
 *                      of every routed row, rows in the expert-major order of
 *                      moe_permute (stable in the flat slot index), gate in
 *                      columns [0, I), up in [I, 2I);
 *   expert_out         [T*k, H] dt: each slot's expert output, row t*k + j
 *                      (the combine's input; the backward does not read it);
 *   shared_gate_up_out [T, 2Is] dt: the shared expert's pre-activations
 *                      (only with a shared expert; Is a multiple of 128).
 * router_logits, topk_ids and topk_weights are required (the backward reads
 * them).  Pass the same cfg and shared expert to the backward.  Workspace:
 * moe_workspace_size(MOE_OP_LAYER, T, H, I, E, top_k, Is, T*top_k, dt).
 */
typedef struct moe_train_saved {
  void* gate_up_out;
  void* expert_out;
  void* shared_gate_up_out;
} moe_train_saved;

int moe_layer_forward_train(const void* hidden_states, const void* router_weight,
                            const float* router_bias, const void* gate_up,
                            const void* down, int T, int H, int I, int E, int top_k,
                            int norm_topk_prob, moe_dtype dt, const moe_router_config* cfg,
                            const moe_shared_expert* shared, void* out,
                            float* router_logits, int32_t* topk_ids,
                            float* topk_weights, int32_t* num_tokens_per_expert,
                            const moe_train_saved* saved, void* workspace,
                            size_t workspace_bytes, hipEvent_t* stage_events,
                            hipStream_t stream);

/*
 * moe_layer_backward — from dout [T, H] dt and the training forward's
 * router_logits, topk_ids, topk_weights and saved activations:
 *   d_topk_weights[t, j] = <dout[t], y[t, j]>            float32 [T, k], or NULL
 *       (evaluated as <dout[t] down[e]^T, h[t, j]>, the first dgrad's
 *       product against the recomputed h, so y is not re-read)
 *   dL (router logits): the routing weights' Jacobian applied to d_w —
 *       softmax, renormalised:  w (d_w - <d_w, w>) on the selection, else 0
 *       softmax, plain:         p (route_scale g - <d_w, w>), p = softmax,
 *                               g = d_w scattered to the ids
 *       sigmoid, renormalised:  w (1 - sg) (d_w - <d_w, w>) on the selection
 *       sigmoid, plain:         d_w w (1 - sg) on the selection
 *   per expert e on its rows, dY = w dout[token]:
 *     d_down[e]    = h^T dY        [E, I, H] dt   (h = silu(g) * u)
 *     dH = dY down[e]^T;  du = dH silu(g);  dg = dH u silu'(g)
 *     d_gate_up[e] = X^T [dg | du] [E, H, 2I] dt  (experts without rows: 0)
 *   shared expert (weight 1 on every token), in its transposed layout:
 *     d_shared_down [Is, H] dt = h_s^T dout; d_shared_gate_up [H, 2Is] dt
 *   dx = sum_j [dg | du] gate_up[e]^T (per slot) + dL router_weight
 *        (+ the shared expert's input gradient)                   [T, H] dt
 *   d_router_weight = dL^T x  [E, H] float32;  d_router_bias = sum_t dL  [E]
 *   float32 or NULL.
 * Every sum is float32 in a fixed order: deterministic.  Weight gradients
 * overwrite their buffers (no accumulation).  Workspace:
 * moe_workspace_size(MOE_OP_LAYER_BACKWARD, T, H, I, E, top_k, Is, T*top_k, dt).
 * stage_events: NULL, or 7 caller-created events recorded before the
 * permutation, before the first dgrad GEMM, before the second dgrad GEMM
 * (after d_topk_weights and dL), before the first wgrad GEMM (after the
 * shared expert's dgrads and dx), before the second wgrad GEMM, before the
 * router's weight gradient (then the shared expert's wgrads), and at the end
 * (NULL entries are skipped).  saved->expert_out may be NULL here.
 */
typedef struct moe_layer_grads {
  void* dx;
  float* d_router_weight;
  float* d_router_bias;
  void* d_gate_up;
  void* d_down;
  float* d_topk_weights;
  void* d_shared_gate_up;
  void* d_shared_down;
} moe_layer_grads;

int moe_layer_backward(const void* hidden_states, const void* router_weight,
                       const void* gate_up, const void* down, int T, int H, int I, int E,
                       int top_k, int norm_topk_prob, moe_dtype dt,
                       const moe_router_config* cfg, const moe_shared_expert* shared,
                       const float* router_logits, const int32_t* topk_ids,
                       const float* topk_weights, const moe_train_saved* saved,
                       const void* dout, const moe_layer_grads* grads, void* workspace,
                       size_t workspace_bytes, hipEvent_t* stage_events, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBMOE_H */
