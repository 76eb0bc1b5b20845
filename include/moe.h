/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE layer forward library, libmoe.so.
 *
 * The layer is route + pack + compute + combine:
 *   route    router projection, softmax, top-k (optionally renormalised over
 *            the k selected experts), lowest expert index first on ties;
 *   pack     counting-sort permute that duplicates token rows and groups them
 *            by expert, with optional capacity C = ceil(phi*T*k/E) and
 *            dropping of overflow routes in arrival (token) order;
 *   compute  per-expert SwiGLU FFN, run as variable-size grouped GEMMs;
 *   combine  gate-weighted un-permute that restores token order, plus an
 *            optional always-on shared expert.
 * Definitions follow these pages:
 *   "271,104 Routes: What I Missed About Mixture-of-Experts" (michaelml.dev),
 *      section 1 "The MoE Block" (y = sum_i p_i(x) E_i(x)), section 2
 *      "The Router" (topk then softmax of the selected logits), section 3
 *      "Dispatch: Turning Routes Into GPU Work" (stable argsort, bincount +
 *      cumsum, index_select, restore).
 *   "Mixture of Experts: Routing, Dispatch, and Load Balancing"
 *      (int8ai.pages.dev), section 1 (router x W + b), sections 2-4.
 *   "MoE Inference Visualized" (infra.bea.ai), "The Router" and
 *      "Expert Execution" (gate/up/down SwiGLU expert; top-1 output scaled by
 *      its softmax probability).
 *   "Session 19: Mixture-of-Experts: routing and capacity"
 *      (cours.spawnkit.ai), "Top-k and mixture" (renormalisation, shared
 *      expert), "Capacity" and "Worked case -- full trace" (C, drops).
 *   "Mixture-of-experts routing" (understandingdata.com), "The maths"
 *      (gate, capacity and imbalance formulas).
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless marked "host".  Tensors are
 *    row-major and contiguous; x, weights, packed rows and outputs must be
 *    16-byte aligned.  Weights use the [out, in] storage of a linear layer.
 *  - Element type of x, weights, packed rows, hidden rows and y is the
 *    shape's dtype (fp32 or bf16).  Accumulation is always fp32.  Router
 *    bias, logits and gates are fp32; ids, counts and indices int32.
 *  - Ownership: the caller allocates and owns every buffer, including the
 *    workspace (moe_workspace_bytes).  The library never allocates or frees
 *    device memory, keeps no state between calls and is reentrant.
 *  - Every call is asynchronous on the given HIP stream (NULL = the null
 *    stream); none synchronises or reads device memory on the host.
 *  - Errors: every call validates its arguments on the host before any
 *    launch and returns a moe_status.  On error nothing is launched and no
 *    output is touched.  A failed launch returns MOE_ERR_HIP; faults inside
 *    kernels surface at the caller's next synchronisation.  No C++
 *    exception crosses this interface.
 *  - Supported range: T >= 0, T*k < 2^31, 1 <= E <= 256, 1 <= k <= min(E, 8),
 *    d, d_ff (and d_ff_shared when non-zero) positive multiples of 8 and
 *    below 2^22; x [T, d] and each expert's (and the shared expert's) weight
 *    matrix below 2^31 bytes; packed, hidden and output rows of any count
 *    (beyond these, MOE_ERR_UNSUPPORTED).  The fixed-shape buffer, expert
 *    choice and the queue policy add limits of their own (below).
 *    NaN or infinite inputs give unspecified (but memory-safe) results.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null required pointer, bad size, misalignment */
  MOE_ERR_UNSUPPORTED = 2, /* outside the supported range or unknown mode  */
  MOE_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required   */
  MOE_ERR_HIP = 4          /* a kernel launch failed                       */
} moe_status;

#define MOE_DTYPE_F32 0
#define MOE_DTYPE_BF16 1
#define MOE_TIE_LOWEST_INDEX 0

/* Problem description (host struct, passed by pointer). */
typedef struct moe_shape {
  int64_t T;           /* tokens                                           */
  int64_t d;           /* model width                                      */
  int64_t E;           /* routed experts                                   */
  int64_t k;           /* experts selected per token                       */
  int64_t d_ff;        /* routed-expert SwiGLU hidden width                */
  int64_t d_ff_shared; /* shared-expert hidden width, 0 = no shared expert */
  int32_t dtype;       /* MOE_DTYPE_F32 or MOE_DTYPE_BF16                  */
  int32_t renormalize; /* 1: gates = softmax over the k selected logits;
                          0: gates = full softmax probabilities over all E */
  int32_t tie_break;   /* MOE_TIE_LOWEST_INDEX (only supported rule)       */
  int32_t reserved;    /* must be 0                                        */
  double phi;          /* capacity factor; <= 0 means no capacity limit    */
} moe_shape;

/* Human-readable name of a status code (static string). */
const char* moe_status_string(int status);

/* Host only.  Capacity and packed-row bound.
 * C = ceil(phi * (double)(T*k) / (double)E) when phi > 0, else -1 (no
 * limit) -- "Mixture-of-experts routing", "Capacity"; the spawnkit trace
 * gives C = ceil(8*2/4*1.25) = 5.  R_max = T*k without a limit, else
 * min(T*k, E*C): the number of rows every packed buffer must hold.
 * Either output pointer may be NULL. */
int moe_capacity(const moe_shape* s, int64_t* C_out /*host*/, int64_t* R_max_out /*host*/);

/* Host only.  Bytes of device workspace that moe_route, moe_permute,
 * moe_expert_ffn and moe_layer_forward need for shape s (one size serves
 * all of them; 0 is never returned for a valid shape).  The workspace must be 256-byte
 * aligned. */
int moe_workspace_bytes(const moe_shape* s, size_t* bytes_out /*host*/);

/* Route: logits = x W_router^T + b ("Mixture of Experts: Routing, Dispatch,
 * and Load Balancing", section 1), fp32, each dot product summed in the
 * fixed order R64 (the pages leave the order open): hidden index i belongs
 * to granule i/8, granule q to partial sum q mod 64, each partial sum a
 * chain of fused multiply-adds in increasing i from +0; the 64 partial sums
 * are folded by halving, p[l] += p[l+s] for l < s, s = 32, ..., 1; the bias
 * is added last.  top-k by (logit descending, expert index ascending) ("271,104
 * Routes", section 2); gates per shape->renormalize (see moe_shape).
 *   x           [T, d]   dtype
 *   w_router    [E, d]   dtype
 *   b_router    [E]      fp32, may be NULL (no bias)
 *   logits      [T, E]   fp32 output, may be NULL (not written)
 *   expert_ids  [T, k]   int32 output, slot j = j-th largest logit
 *   gates       [T, k]   fp32 output
 * Workspace: moe_workspace_bytes (holds the logits when logits is NULL). */
int moe_route(const moe_shape* s, const void* x, const void* w_router, const float* b_router,
              float* logits, int32_t* expert_ids, float* gates, void* ws, size_t ws_bytes,
              hipStream_t stream);

/* Pack: stable counting sort of the T*k routes r = t*k + j by expert
 * ("271,104 Routes", section 3: argsort(stable) + bincount.cumsum), with
 * capacity: route r is kept iff its arrival slot (number of earlier routes
 * to the same expert) is < C; overflow routes are dropped ("Session 19",
 * "Capacity" and the full trace).
 *   x           [T, d]     dtype
 *   expert_ids  [T, k]     int32, each in [0, E); a token lists an expert at
 *                          most once (as moe_route produces)
 *   counts      [E]        int32 output: demand n_e before capacity
 *   kept_counts [E]        int32 output: m_e = min(n_e, C)
 *   offsets     [E+1]      int32 output: exclusive prefix of m_e
 *   route_pos   [T, k]     int32 output: packed row of route r, -1 if dropped
 *   row_token   [R_max]    int32 output: source token of packed row p
 *   x_packed    [R_max, d] dtype output: x_packed[p] = x[row_token[p]]
 * Rows at or past offsets[E] of row_token / x_packed are left unwritten.
 * Workspace: moe_workspace_bytes. */
int moe_permute(const moe_shape* s, const void* x, const int32_t* expert_ids, int32_t* counts,
                int32_t* kept_counts, int32_t* offsets, int32_t* route_pos, int32_t* row_token,
                void* x_packed, void* ws, size_t ws_bytes, hipStream_t stream);

/* Compute: for every expert e and packed row p in [offsets[e], offsets[e+1]):
 *   y_packed[p] = W_down[e] (SiLU(W_gate[e] x_p) * (W_up[e] x_p))
 * ("MoE Inference Visualized", "Expert Execution"), as two grouped GEMMs on
 * bf16 MFMA (fp32 accumulation; the hidden activations are rounded to dtype
 * between the two GEMMs).
 *   x_packed    [R_max, d]       dtype
 *   offsets     [E+1]            int32 (device; never read on the host)
 *   w_gate      [E, d_ff, d]     dtype
 *   w_up        [E, d_ff, d]     dtype
 *   w_down      [E, d, d_ff]     dtype
 *   y_packed    [R_max, d]       dtype output (rows past offsets[E] unwritten)
 * offsets[E] must be <= R_max of the shape.  A dense FFN (such as a shared
 * expert) is the case E = 1, k = 1 with offsets = {0, T}.
 * Workspace: moe_workspace_bytes. */
int moe_expert_ffn(const moe_shape* s, const void* x_packed, const int32_t* offsets,
                   const void* w_gate, const void* w_up, const void* w_down, void* y_packed,
                   void* ws, size_t ws_bytes, hipStream_t stream);

/* Combine: y[t] = sum_{j<k, route_pos[t,j] >= 0} gates[t,j] * y_packed[route_pos[t,j]]
 *                 (+ y_shared[t])
 * summed in fp32 with j ascending, shared output added last, rounded once to
 * dtype ("271,104 Routes", sections 1 and 3; "Session 19", "Top-k and
 * mixture": the shared expert is outside the gate normalisation; dropped
 * routes contribute nothing and the other gates are not renormalised).
 *   y_packed  [R_max, d]  dtype
 *   route_pos [T, k]      int32
 *   gates     [T, k]      fp32
 *   y_shared  [T, d]      dtype, may be NULL
 *   y         [T, d]      dtype output
 * No workspace. */
int moe_combine(const moe_shape* s, const void* y_packed, const int32_t* route_pos,
                const float* gates, const void* y_shared, void* y, hipStream_t stream);

/* The whole layer: route -> pack -> compute (routed experts, and the shared
 * expert when d_ff_shared > 0) -> combine, all stream-ordered with no host
 * synchronisation.  The packed copy of x is not materialised: the first
 * grouped GEMM reads token rows through the route table.  No residual add
 * (the caller adds x).
 *   x, w_router, b_router (nullable)       as in moe_route
 *   w_gate, w_up, w_down                   as in moe_expert_ffn
 *   ws_gate [d_ff_shared, d], ws_up [d_ff_shared, d], ws_down [d, d_ff_shared]
 *                                          dtype; required iff d_ff_shared > 0
 *   y          [T, d]  dtype output
 *   expert_ids [T, k], gates [T, k], counts [E], route_pos [T, k]:
 *              optional outputs (NULL = not returned)
 * Workspace: moe_workspace_bytes. */
int moe_layer_forward(const moe_shape* s, const void* x, const void* w_router,
                      const float* b_router, const void* w_gate, const void* w_up,
                      const void* w_down, const void* ws_gate, const void* ws_up,
                      const void* ws_down, void* y, int32_t* expert_ids, float* gates,
                      int32_t* counts, int32_t* route_pos, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/* moe_layer_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, semantics and output
 * bits as moe_layer_forward (the same kernels run); the workspace is a
 * fixed array of MOE_NOALLOC_SCRATCH_BYTES inside the library, one per GPU,
 * held from the library's load until the process ends.  The call allocates
 * nothing.
 *   - Shapes whose moe_workspace_bytes exceeds MOE_NOALLOC_SCRATCH_BYTES
 *     (64 MiB: enough for, e.g., Switch T=4096 d=768 d_ff=3072, Granite
 *     T=1412 k=8 of 32 experts d=1024, Mixtral decode T=16 d=4096
 *     d_ff=14336) return MOE_ERR_UNSUPPORTED before any launch.
 *   - The array's address on the current device is looked up on the first
 *     call there (MOE_ERR_HIP if that fails).
 *   - Every call on one GPU shares that GPU's array: calls that overlap on
 *     one GPU (on different streams, or from different threads without
 *     ordering) race and give wrong results.  Calls ordered on one stream
 *     are safe.  The layer needs no part of the array cleared between
 *     calls (every value it reads there it wrote earlier in the same call). */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_layer_forward_noalloc(const moe_shape* s, const void* x, const void* w_router,
                              const float* b_router, const void* w_gate, const void* w_up,
                              const void* w_down, const void* ws_gate, const void* ws_up,
                              const void* ws_down, void* y, int32_t* expert_ids, float* gates,
                              int32_t* counts, int32_t* route_pos, hipStream_t stream);

/* Fixed-shape dispatch buffer [E, C, d] ("Session 19: Mixture-of-Experts:
 * routing and capacity", "Capacity": capacity is a tensor dimension, and the
 * slot table of "Visual support -- Capacity"; "271,104 Routes", section 3
 * "When one expert gets too many tokens": fixed expert buffers make shapes
 * regular at the cost of padding).  The same counting-sort dispatch as
 * moe_permute, written into the fixed buffer instead of packed rows:
 *   route_pos[T*k]     row e*C + slot of the buffer for a kept route (slot =
 *                      its arrival rank at expert e), -1 if dropped
 *   x_padded[E*C][d]   x_padded[e*C + c] = x[token seated in slot c of e];
 *                      empty slots are zero rows
 *   counts, kept_counts as in moe_permute.
 * Needs a capacity (phi > 0): otherwise MOE_ERR_INVALID_ARG.  E*C rows must
 * fit 32-bit buffer offsets (else MOE_ERR_UNSUPPORTED). */
int moe_permute_padded(const moe_shape* s, const void* x, const int32_t* expert_ids,
                       int32_t* counts, int32_t* kept_counts, int32_t* route_pos, void* x_padded,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_layer_forward over the fixed-shape buffer: the expert FFNs run on all
 * E*C rows of [E, C, d] (empty slots included -- the padding the pages
 * price: E*C - sum_e m_e rows of work), then the same combine.  The output
 * equals moe_layer_forward's for every kept route (padding rows are zero
 * and never read back).  The optional route_pos output receives the
 * buffer's rows e*C + slot.  Same arguments and errors as moe_layer_forward,
 * plus those of moe_permute_padded. */
int moe_layer_forward_padded(const moe_shape* s, const void* x, const void* w_router,
                             const float* b_router, const void* w_gate, const void* w_up,
                             const void* w_down, const void* ws_gate, const void* ws_up,
                             const void* ws_down, void* y, int32_t* expert_ids, float* gates,
                             int32_t* counts, int32_t* route_pos, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/* Overflow policy "reroute" ("Session 19: Mixture-of-Experts: routing and
 * capacity", "Overflow policies": the overflowing route is handled by the
 * token's next-best expert, the router decision overridden; "271,104
 * Routes", section 3: an overflowing expert's routes are dropped, rerouted,
 * given more room or handled dynamically).  Routes keep the seats of the drop
 * policy (moe_permute); then the dropped routes, in arrival order r = t*k + j,
 * each take the best-ranked expert of token t (logit descending, lower index
 * first on ties) that t does not already hold and that still has room (<= C
 * seats); without one the route stays dropped.  Gates are not changed.
 * Inputs: logits [T][E] and expert_ids [T][k] from moe_route.
 * Outputs: expert_ids_out [T][k] the expert of every route after rerouting;
 *   counts [E] demand of the router's choices (before capacity); filled [E]
 *   seats used per expert; offsets [E+1] their exclusive prefix; route_pos
 *   [T][k] packed row (an expert's kept routes first, then its rerouted
 *   ones, each in arrival order), -1 if dropped; row_token [R_max];
 *   x_packed [R_max][d] as in moe_permute.
 * expert_ids must lie in [0, E), as moe_route writes them.  Up to 64
 * experts the dropped routes are placed by parallel rounds (deferred
 * acceptance under token-order priority, which ends in the same assignment
 * as the arrival-order greedy) while the per-expert token bitmaps fit 144
 * KiB of LDS (T <= 65535 at E <= 16, T <= 35744 at E = 32, T <= 18144 at
 * E = 64), else by one wave walking them in arrival order; beyond 64
 * experts always by the walk (four experts per lane).  The workspace of
 * moe_workspace_bytes covers each. */
int moe_permute_reroute(const moe_shape* s, const void* x, const float* logits,
                        const int32_t* expert_ids, int32_t* expert_ids_out, int32_t* counts,
                        int32_t* filled, int32_t* offsets, int32_t* route_pos,
                        int32_t* row_token, void* x_packed, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* moe_layer_forward with the reroute overflow policy (moe_permute_reroute
 * in place of moe_permute).  expert_ids receives the experts after
 * rerouting, counts the demand of the router's choices, route_pos the
 * rerouted packed rows. */
int moe_layer_forward_reroute(const moe_shape* s, const void* x, const void* w_router,
                              const float* b_router, const void* w_gate, const void* w_up,
                              const void* w_down, const void* ws_gate, const void* ws_up,
                              const void* ws_down, void* y, int32_t* expert_ids, float* gates,
                              int32_t* counts, int32_t* route_pos, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/* Forward-only routing statistics of one batch of routes, from the outputs
 * of moe_route (logits must have been requested) and moe_permute (counts).
 *   "Mixture of Experts: Routing, Dispatch, and Load Balancing", section 4:
 *     the Switch auxiliary load-balancing loss alpha * N * sum_i f_i P_i,
 *     f_i the share of routes sent to expert i (before capacity), P_i the
 *     mean over tokens of its full softmax probability (N = E).
 *   "Mixture-of-experts routing", load imbalance: max_e D_e / mean D, D the
 *     demand before capacity.
 *   "271,104 Routes", section 4: selection share, largest selected weight,
 *     normalised routing entropy, Jensen-Shannon distance of load vectors.
 *   "MoE Inference Visualized", "Router Confidence": the softmax probability
 *     of the chosen expert.
 * Inputs (device): logits [T][E] fp32, gates [T][k] fp32, counts [E] int32
 * (demand, as moe_permute writes it).  alpha: loss coefficient (the Switch
 * Transformer value is 1e-2).  n_bins in [1, 256].
 * Outputs (device):
 *   stats [6 + 2E] fp32:
 *     [0] aux loss  [1] load imbalance  [2] mean largest selected gate
 *     [3] mean normalised entropy of the selected gates (each token's k
 *         gates normalised to sum 1, entropy / ln k; 0 when k = 1)
 *     [4] Jensen-Shannon distance (base 2) of the route shares to the
 *         uniform load  [5] mean router confidence
 *     [6, 6+E) route shares f  [6+E, 6+2E) mean probabilities P
 *   hist [n_bins] int32: tokens by router confidence (the largest softmax
 *     probability) in equal bins on [0, 1].
 * Sums run in a fixed order in fp32 (repeat calls give identical results).
 * T = 0 gives zeros.  Uses the workspace of moe_workspace_bytes. */
int moe_routing_stats(const moe_shape* s, const float* logits, const float* gates,
                      const int32_t* counts, double alpha, int32_t n_bins, float* stats,
                      int32_t* hist, void* ws, size_t ws_bytes, hipStream_t stream);

/* Expert-choice routing ("MoE Inference Visualized", "Why MoE Matters for
 * Infrastructure": against load imbalance the experts pick the tokens
 * instead of the tokens picking experts; the page names the idea only).
 * Reading: score[t][e] = softmax of token t's router logits over all E
 * experts; expert e keeps the Ce = min(C, T) tokens of largest score (C =
 * moe_capacity's), the lower token index first among equal scores; a kept
 * pair's gate is its score.  Every expert holds exactly Ce rows; a token may
 * be kept by any number of experts, none included (it then gets only the
 * shared expert).  The choice is made on the fp32 scores written out.
 * Inputs: x [T][d]; logits [T][E] fp32 from moe_route.
 * Outputs:
 *   scores      [T][E] fp32
 *   route_pos   [T][E] int32: row e*Ce + i when expert e kept token t as its
 *               i-th token in increasing index, else -1
 *   offsets     [E+1] int32: e*Ce
 *   row_token   [E*Ce] int32: source token of every row
 *   x_packed    [E*Ce][d]: x_packed[r] = x[row_token[r]]
 * shape->k only sets C = ceil(phi*T*k/E).  Needs phi > 0 and renormalize = 0
 * (else MOE_ERR_INVALID_ARG) and E*T < 2^29 (the [E][T] key and route
 * tables below 2 GiB; else MOE_ERR_UNSUPPORTED).
 * Uses the workspace of moe_workspace_bytes. */
int moe_permute_expert_choice(const moe_shape* s, const void* x, const float* logits,
                              float* scores, int32_t* route_pos, int32_t* offsets,
                              int32_t* row_token, void* x_packed, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/* moe_layer_forward under expert-choice routing: router logits, the choice of
 * moe_permute_expert_choice, the expert FFNs on the E*Ce rows, then
 * y[t] = sum over the experts e that kept t, in increasing e, of
 * score[t][e] * E_e(x_t), plus the shared expert.  scores and route_pos
 * ([T][E]) are optional outputs (NULL: kept in the workspace).  Same
 * requirements as moe_permute_expert_choice. */
int moe_layer_forward_expert_choice(const moe_shape* s, const void* x, const void* w_router,
                                    const float* b_router, const void* w_gate, const void* w_up,
                                    const void* w_down, const void* ws_gate, const void* ws_up,
                                    const void* ws_down, void* y, float* scores,
                                    int32_t* route_pos, void* ws, size_t ws_bytes,
                                    hipStream_t stream);

/* Measurement variant of moe_layer_forward (same arguments without the
 * optional routing outputs): additionally records events[i] on the stream at
 * the stage boundaries, so that elapsed times between them are the stage
 * times ("271,104 Routes", "The next experiment": one trace that lines up
 * router, permutation and packing, expert matmuls and combine):
 *   events[0] before route          events[1] before the permute
 *   events[2] before grouped GEMM 1 events[3] before grouped GEMM 2
 *   events[4] before the shared expert (equal to events[5] without one)
 *   events[5] before combine        events[6] after combine
 *   events     host array of 7 hipEvent_t created by the caller; a NULL
 *              entry is skipped.  The array itself must not be NULL.
 *   layout     0: packed rows (moe_layer_forward); 1: the fixed-shape
 *              [E, C, d] buffer (moe_layer_forward_padded); 2: the reroute
 *              overflow policy (moe_layer_forward_reroute); 3: expert-choice
 *              routing (moe_layer_forward_expert_choice; events[1] is then
 *              before the choice). */
int moe_layer_forward_timed(const moe_shape* s, const void* x, const void* w_router,
                            const float* b_router, const void* w_gate, const void* w_up,
                            const void* w_down, const void* ws_gate, const void* ws_up,
                            const void* ws_down, void* y, void* ws, size_t ws_bytes,
                            hipStream_t stream, hipEvent_t* events /*host*/, int32_t layout);

/* Overflow policy "queue to the next micro-batch" ("Session 19:
 * Mixture-of-Experts: routing and capacity", "Overflow policies": the
 * overflowing route is processed in the next micro-batch, at the price of an
 * extra exchange and a saw-tooth latency).  A route that finds its expert
 * full is neither lost nor moved: it waits, with its expert and gate, in a
 * queue the caller keeps and passes to the next call.  In that call the
 * waiting routes arrive first, in queue order, and the call's own routes
 * after them in the order r = t*k + j (arrival a < q_n is queued route a,
 * arrival q_n + r is route r).  Each expert seats its first C arrivals, C =
 * ceil(phi*T*k/E) of this call's batch (no limit when phi <= 0); every
 * later arrival, queued or new, joins the outgoing queue, in arrival order.
 * The library keeps no state: the queue lives in the caller's buffers.
 *   q_n          routes waiting from the previous call (host, >= 0)
 *   q_x [q_n, d] their token rows (dtype); q_ids [q_n] int32 experts;
 *   q_gates [q_n] fp32 gates; q_tags [q_n] int64 (opaque to the library,
 *                returned with the route)
 *   tag_base     tag of this batch's token t is tag_base + t
 *   y [T, d]     this batch: its seated routes' gated expert outputs plus
 *                the shared expert
 *   y_late [q_n, d]  row a: queued route a's gate times its expert output
 *                if it was seated in this call, else a zero row (the caller
 *                adds it to the output of the token its tag names)
 *   out_n        device int32: routes in the outgoing queue
 *   out_x [q_n + T*k, d], out_ids, out_gates, out_tags: the outgoing queue
 *                (first *out_n entries), same layout as the q_ arguments;
 *                out_x must not alias q_x or x
 *   expert_ids, gates [T, k], counts [E] (demand over all arrivals): optional
 *   route_pos [q_n + T*k]: optional, packed row of every arrival, -1 if it
 *                waits
 * Workspace: moe_workspace_bytes_queued(s, q_n).  Errors as
 * moe_layer_forward; MOE_ERR_UNSUPPORTED when q_n + T*k, the queued rows
 * [q_n, d] or the packed rows leave the 32-bit ranges. */
int moe_workspace_bytes_queued(const moe_shape* s, int64_t q_n, size_t* bytes_out /*host*/);
int moe_layer_forward_queued(const moe_shape* s, const void* x, const void* w_router,
                             const float* b_router, const void* w_gate, const void* w_up,
                             const void* w_down, const void* ws_gate, const void* ws_up,
                             const void* ws_down, int64_t q_n, const void* q_x,
                             const int32_t* q_ids, const float* q_gates, const int64_t* q_tags,
                             int64_t tag_base, void* y, void* y_late, int32_t* out_n, void* out_x,
                             int32_t* out_ids, float* out_gates, int64_t* out_tags,
                             int32_t* expert_ids, float* gates, int32_t* counts,
                             int32_t* route_pos, void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_layer_forward_queued (tag_base 0, no optional outputs) with the
 * stage-boundary events of moe_layer_forward_timed (events[1] before the
 * arrivals' dispatch and the outgoing queue; the late rows follow
 * events[6]).  For measurement only. */
int moe_layer_forward_queued_timed(const moe_shape* s, const void* x, const void* w_router,
                                   const float* b_router, const void* w_gate, const void* w_up,
                                   const void* w_down, const void* ws_gate, const void* ws_up,
                                   const void* ws_down, int64_t q_n, const void* q_x,
                                   const int32_t* q_ids, const float* q_gates,
                                   const int64_t* q_tags, void* y, void* y_late, int32_t* out_n,
                                   void* out_x, int32_t* out_ids, float* out_gates,
                                   int64_t* out_tags, void* ws, size_t ws_bytes,
                                   hipStream_t stream, hipEvent_t* events /*host*/);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
