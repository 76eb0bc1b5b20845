/*
 * oracle.h -- plain CPU oracle for the MoE layer forward pass
 * (route + pack + compute + combine).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * (the HIP library and its Python binding) never calls it and shares no code,
 * header, table or helper with it.
 *
 * Sources (the pages this follows; every function below cites its passage):
 *   [MML]  "271,104 Routes: What I Missed About Mixture-of-Experts"
 *          (michaelml.dev), sections 1 "The MoE Block", 2 "The Router",
 *          3 "Dispatch: Turning Routes Into GPU Work".
 *   [INT8] "Mixture of Experts: Routing, Dispatch, and Load Balancing"
 *          (int8ai.pages.dev), section 1 (router), section 3 (minimal
 *          example), section 4 (capacity, overflow, load imbalance).
 *   [BEA]  "MoE Inference Visualized" (infra.bea.ai), "The Router" and
 *          "Expert Execution: Gather -> Compute -> Scale -> Scatter".
 *   [SPK]  "Session 19: Mixture-of-Experts: routing and capacity"
 *          (cours.spawnkit.ai), slides "Top-k and mixture", "Capacity",
 *          "Worked case -- full trace".
 *   [UD]   "Mixture-of-experts routing" (understandingdata.com),
 *          "The maths": the gate, capacity and load-imbalance formulas.
 *
 * Precision.  Router logits are fp32 (the [MML] Granite experiment casts the
 * router logits to float before top-k), accumulated in one fixed order, R64
 * (see oracle_router_logits); that order is a reading of ours, because the
 * pages leave it open and the selected expert ids depend on it at near ties.
 * Gates, expert FFNs and the combine are computed in double precision.
 *
 * Element types: dtype 0 = IEEE binary32, dtype 1 = bfloat16 (raw 16-bit
 * patterns, the upper half of a binary32).  All arrays are row-major and
 * contiguous.  Weights use the [out, in] storage of a linear layer:
 * w_router[E][d], w_gate[E][d_ff][d], w_up[E][d_ff][d], w_down[E][d][d_ff].
 *
 * Parity status per function is stated beside each declaration.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* Expert capacity C = ceil(phi * T * k / E) ([UD] "Capacity"; [SPK]
 * "Capacity" and the full trace).  Evaluated in IEEE double as
 * ceil(phi * (double)(T*k) / (double)E).  phi <= 0 means "no capacity
 * limit" and returns -1.  Pinned by the [SPK] trace (C = 5, 4, 8, 6, 3) and
 * the [INT8] overflow case (C = 2). */
int64_t oracle_capacity(int64_t T, int64_t E, int64_t k, double phi);

/* Router logits, fp32: logits[t][e] = sum_i x[t][i] * w[e][i] (+ b[e])
 * ([INT8] section 1: x @ W_router + b_router; [BEA] "The Router": one
 * 768-wide dot product per expert row).  b may be NULL.
 * Summation order R64: hidden index i lies in granule q = i / 8 (eight
 * consecutive elements); granule q is accumulated into partial sum
 * l = q mod 64, each partial sum a chain of fmaf over its elements in
 * increasing i, starting from +0; then for s = 32, 16, 8, 4, 2, 1 the
 * partial sums are folded, p[l] = p[l] + p[l + s] for l < s; the logit is
 * p[0], and the bias is added last.
 * Pinned against fp64 dot products within the fp32 error bound, and by
 * hand-derived sums whose rounding depends on the order (a 2^24 term with
 * unit terms in chosen granules). */
void oracle_router_logits(int64_t T, int64_t d, int64_t E, int dtype,
                          const void* x, const void* w, const float* b,
                          float* logits);

/* The same dot products in double precision (exact products, double sums),
 * for the near-tie report.  Not used for decisions. */
void oracle_router_logits_f64(int64_t T, int64_t d, int64_t E, int dtype,
                              const void* x, const void* w, const float* b,
                              double* logits);

/* Top-k selection and gates ([MML] section 2: logits.topk then softmax over
 * the selected logits; [UD] "The gate"; [SPK] "Top-k and mixture":
 * renormalise the selected probabilities by their sum; [BEA] "Expert
 * Execution": top-1 scaled by its softmax probability).
 * Selection: the k largest logits, slot j = j-th largest; equal logits are
 * ordered by lower expert index first.
 * renorm = 1: g_j = exp(l_j - m) / sum_{selected} exp(l_i - m)
 * renorm = 0: g_j = exp(l_j - m) / sum_{all e} exp(l_e - m)
 * with m the largest logit; computed in double, rounded once to float.
 * Pinned by the [SPK] worked example, the gate-sum invariant and brute-force
 * sorting. */
void oracle_topk_gates(int64_t T, int64_t E, int64_t k, int renorm,
                       const float* logits, int32_t* expert_ids, float* gates);

/* Counting-sort dispatch with optional capacity ([MML] section 3: flatten
 * routes r = t*k + j, stable argsort by expert, bincount + cumsum;
 * [SPK] "Capacity" and trace: arrivals beyond C are dropped in arrival
 * order; [INT8] section 4 overflow case).
 *   counts[e]      demand n_e (routes choosing e, before capacity)
 *   kept[e]        m_e = min(n_e, C)
 *   offsets[E+1]   exclusive prefix of m_e
 *   route_pos[r]   row of route r in the expert-grouped layout, -1 if dropped
 *   row_token[p]   source token of packed row p, p < offsets[E]
 * C < 0 means no capacity limit.  Pinned by the [MML] and [SPK]/[INT8]
 * worked cases. */
void oracle_dispatch(int64_t T, int64_t E, int64_t k, int64_t C,
                     const int32_t* expert_ids, int32_t* counts, int32_t* kept,
                     int32_t* offsets, int32_t* route_pos, int32_t* row_token);

/* The fixed-shape dispatch buffer [E, C, d] ("Session 19", "Capacity":
 * capacity is a tensor dimension; "Visual support -- Capacity" slot table;
 * "271,104 Routes", section 3 "When one expert gets too many tokens": fixed
 * expert buffers).  From a dispatch with capacity C >= 1 (route_pos and
 * offsets of oracle_dispatch):
 *   pad_pos[r]       e*C + slot of route r (slot = its arrival rank at e),
 *                    -1 if dropped
 *   slot_token[e*C + c]  token seated in slot c of expert e, -1 if empty
 * Pinned by the slot table of the "Session 19" trace (15 filled, 5 empty). */
void oracle_dispatch_padded(int64_t T, int64_t E, int64_t k, int64_t C,
                            const int32_t* expert_ids, const int32_t* route_pos,
                            const int32_t* offsets, int32_t* pad_pos,
                            int32_t* slot_token);

/* Overflow policy "reroute" ("Session 19", "Overflow policies": the
 * overflowing route is handled by the token's next-best expert; the router
 * decision is overridden).  Reading: routes keep the seats the drop policy
 * gives them (oracle_dispatch); then the dropped routes, in arrival order
 * r = t*k + j, each move to the best-ranked expert of token t (logit
 * descending, lower index first on ties) that t does not already hold and
 * that still has room, taking its next free slot; with no such expert the
 * route stays dropped.  Its gate is unchanged.
 *   ids_out[T*k]     the expert of every route after rerouting
 *   counts[E]        demand of the original choices (before capacity)
 *   filled[E]        seats used per expert (kept + rerouted, <= C)
 *   offsets[E+1]     exclusive prefix of filled
 *   route_pos[T*k]   packed row: kept routes first in each expert (arrival
 *                    order), then its rerouted routes (arrival order); -1
 *                    if dropped after all
 *   row_token[p]     source token of packed row p
 *   n_rerouted       (out) routes moved
 * Pinned by the trace (t6 at E1 goes to its third choice) and by invariants
 * of the greedy order (no expert over C; every expert a rerouted route
 * preferred, and every expert a dropped route could take, is full). */
void oracle_dispatch_reroute(int64_t T, int64_t E, int64_t k, int64_t C,
                             const float* logits, const int32_t* ids_in,
                             int32_t* ids_out, int32_t* counts, int32_t* filled,
                             int32_t* offsets, int32_t* route_pos,
                             int32_t* row_token, int64_t* n_rerouted);

/* Overflow policy "queue to the next micro-batch" ("Session 19", "Overflow
 * policies": the overflowing route is processed in the next micro-batch, at
 * the cost of an extra exchange and a saw-tooth latency).  Reading: a route
 * that finds its expert full is neither lost nor moved; it waits, with its
 * expert and its gate, for the next call.  In that call the waiting routes
 * arrive first, in their queue order, and the call's own routes after them
 * in the order r = t*k + j: arrival a = 0..Q-1 is queued route a, arrival
 * a = Q + r is route r.  Each expert seats its first C arrivals (C of the
 * call's own batch); every later arrival, queued or new, waits again, and
 * the new queue lists them in arrival order.  That is the drop policy of
 * oracle_dispatch over the arrival sequence, the drops kept.
 *   q_ids[Q], ids[T*k]   experts of the queued routes and of the call's routes
 *   counts[E], kept[E], offsets[E+1]   as oracle_dispatch, over the arrivals
 *   pos[Q + T*k]         packed row of arrival a, -1 if it waits again
 *   row_arrival[p]       the arrival seated in packed row p
 *   out_arrival[]        the arrivals that wait again, in arrival order
 * Returns their number.  Pinned by the trace (t6's route at E1 waits, then
 * takes the first seat of E1 in the next batch), by invariants over a run of
 * batches (each route seated once; queued routes ahead of new ones; no
 * expert over C) and, through the layer, by a dense brute force over that
 * run. */
int64_t oracle_dispatch_queue(int64_t T, int64_t E, int64_t k, int64_t C, int64_t Q,
                              const int32_t* q_ids, const int32_t* ids, int32_t* counts,
                              int32_t* kept, int32_t* offsets, int32_t* pos,
                              int32_t* row_arrival, int32_t* out_arrival);

/* Expert-choice routing ("MoE Inference Visualized", "Why MoE Matters for
 * Infrastructure": the experts pick the tokens instead of the tokens picking
 * experts -- named only).  Reading: score[t][e] = full softmax probability
 * of the router logits (stored as fp32; the choice is made on that value);
 * expert e takes the Ce = min(C, T) tokens of largest score, lower token
 * index first among equal scores (C < 0: Ce = T, every expert takes every
 * token).  Every expert thus holds exactly Ce rows; a token may be taken by
 * any number of experts, none included.
 *   scores[T][E]      the scores = the gates of the chosen pairs
 *   route_pos[T][E]   row e*Ce + i if expert e took token t as its i-th
 *                     token in increasing token order, else -1
 *   row_token[E*Ce]   source token of every row (may be NULL)
 * Pinned by a worked example with closed-form scores, the tie rule on equal
 * scores, the ranking invariant on random inputs and the C >= T case (the
 * full soft mixture). */
void oracle_expert_choice(int64_t T, int64_t E, int64_t C, const float* logits,
                          float* scores, int32_t* route_pos, int32_t* row_token);

/* Row duplication: packed[p][:] = x[row_token[p]][:] for p < n_rows, a bit
 * copy of elem_bytes-sized elements ([MML] section 3: index_select). */
void oracle_gather_rows(int64_t n_rows, int64_t d, int64_t elem_bytes,
                        const void* x, const int32_t* row_token, void* packed);

/* Expert SwiGLU FFN of one expert on n rows, in double:
 *   a = x Wg^T, b = x Wu^T, h = SiLU(a) * b, y = h Wd^T
 * ([BEA] "Expert Execution": down_proj(SiLU(gate_proj(x)) * up_proj(x))).
 * x: [n][d] (dtype), wg, wu: [d_ff][d], wd: [d][d_ff] (dtype), y: [n][d].
 * Pinned against a torch fp64 dense MLP. */
void oracle_swiglu_rows(int64_t n, int64_t d, int64_t d_ff, int dtype,
                        const void* x, const void* wg, const void* wu,
                        const void* wd, double* y);

/* Expert FFN over expert-grouped rows: rows [offsets[e], offsets[e+1]) of
 * x_packed run through expert e ([MML] section 3: grouped expert matmuls).
 * y_packed: [offsets[E]][d] double. */
void oracle_expert_ffn(int64_t E, int64_t d, int64_t d_ff, int dtype,
                       const int32_t* offsets, const void* x_packed,
                       const void* w_gate, const void* w_up,
                       const void* w_down, double* y_packed);

/* Gate-weighted combine ([MML] section 1: y = sum_i p_i E_i(x), section 3:
 * restore token order; [SPK] "Top-k and mixture": + shared expert outside
 * the renormalisation; [SPK] trace: a dropped route contributes nothing and
 * the remaining gates are not renormalised).
 * y[t] = sum_{j < k, route_pos[t*k+j] >= 0} g[t][j] * y_packed[route_pos]
 *        + y_shared[t]
 * y_packed and y_shared are given in ypdtype (0 f32, 1 bf16, 2 f64);
 * y_shared may be NULL.  Output in double. */
void oracle_combine(int64_t T, int64_t k, int64_t d, int ypdtype,
                    const void* y_packed, const int32_t* route_pos,
                    const float* gates, const void* y_shared, double* y);

/* Forward-only routing statistics of one batch of routes.
 *   out[0]  aux     Switch auxiliary load-balancing loss value
 *                   alpha * E * sum_e f_e * P_e ([INT8] section 4, after
 *                   Switch Transformer), f_e = counts[e] / (T*k) the share of
 *                   routes sent to e (demand, before capacity), P_e the mean
 *                   over tokens of the full softmax probability of e
 *   out[1]  imbalance  max_e counts[e] / (T*k/E) ([UD] load imbalance,
 *                   measured on demand)
 *   out[2]  mean over tokens of the largest selected gate ([MML] section 4
 *                   "largest selected weight")
 *   out[3]  mean over tokens of the normalised routing entropy: the k
 *                   selected gates normalised to sum 1, entropy / ln k
 *                   (0 when k = 1) ([MML] section 4)
 *   out[4]  Jensen-Shannon distance, base 2, between the route shares f and
 *                   the uniform load 1/E ([MML] section 4 compares load
 *                   vectors with it)
 *   out[5]  mean over tokens of the router confidence: the softmax
 *                   probability of the chosen (largest-logit) expert ([BEA]
 *                   "Router Confidence")
 *   share[E] = f, mean_prob[E] = P
 *   hist[n_bins]: tokens by router confidence in n_bins equal bins on
 *                   [0, 1] (bin b holds [b/n_bins, (b+1)/n_bins); 1.0 goes
 *                   to the last bin)
 * Everything in double from the fp32 logits; T = 0 gives zeros.  Pinned by
 * closed forms (uniform logits, balanced routing gives aux = alpha, a hot
 * expert gives E/k) and scipy's entropy and Jensen-Shannon routines. */
void oracle_routing_stats(int64_t T, int64_t E, int64_t k, const float* logits,
                          const float* gates, const int32_t* counts,
                          double alpha, int32_t n_bins, double* out,
                          double* share, double* mean_prob, int64_t* hist);

/* Whole layer forward: logits -> top-k gates -> dispatch with capacity ->
 * expert FFN per kept route -> gate-weighted sum (+ shared expert).
 * Routing (ids, gates, counts, route_pos) is computed for all T tokens;
 * the output rows are computed for the n_sel tokens listed in sel (all T
 * tokens in order when sel is NULL), y: [n_sel][d] double.
 * d_ff_shared = 0 means no shared expert (ws_* may be NULL).
 * Any of ids/gates/counts/route_pos may be NULL.
 * Returns 0, or -1 on bad arguments. */
int oracle_layer_forward(int64_t T, int64_t d, int64_t E, int64_t k,
                         int64_t d_ff, int64_t d_ff_shared, int dtype,
                         int renorm, double phi, const void* x,
                         const void* w_router, const float* b_router,
                         const void* w_gate, const void* w_up,
                         const void* w_down, const void* ws_gate,
                         const void* ws_up, const void* ws_down,
                         int64_t n_sel, const int32_t* sel, double* y,
                         int32_t* ids, float* gates, int32_t* counts,
                         int32_t* route_pos);

/* Whole layer under expert-choice routing: router logits as
 * oracle_router_logits, choice as oracle_expert_choice with capacity C,
 * y[t] = sum over the experts e that took t (increasing e) of
 * score[t][e] * E_e(x_t), plus the shared expert when d_ff_shared > 0.
 * y holds the tokens in sel (all when sel is NULL), in double.  scores_out
 * and route_pos_out ([T][E]) may be NULL.  Returns 0, or -1 on bad sizes. */
int oracle_layer_forward_expert_choice(int64_t T, int64_t d, int64_t E,
                                       int64_t d_ff, int64_t d_ff_shared,
                                       int dtype, int64_t C, const void* x,
                                       const void* w_router,
                                       const float* b_router,
                                       const void* w_gate, const void* w_up,
                                       const void* w_down, const void* ws_gate,
                                       const void* ws_up, const void* ws_down,
                                       int64_t n_sel, const int32_t* sel,
                                       double* y, float* scores_out,
                                       int32_t* route_pos_out);

#ifdef __cplusplus
}
#endif
#endif
