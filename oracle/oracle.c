/*
 * oracle.c -- plain, slow, obviously correct CPU oracle for the MoE layer
 * forward pass.  TEST INFRASTRUCTURE ONLY (see oracle.h): only tests, the
 * smoke check and the benchmark's CPU-baseline leg use it.
 *
 * Every loop follows the definition on the pages directly: per token, per
 * selected expert, per element.  Token loops carry an OpenMP "parallel for"
 * (independent tokens; no arithmetic is reordered by it).
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC
 * (no contraction, so every a*b+c below is two roundings unless written as
 * fmaf/fma explicitly).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* bfloat16 is the upper 16 bits of an IEEE binary32 value. */
static float bf16_to_float(uint16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Element idx of an array of the given element type, as float (exact). */
static float elem_f(const void* base, int dtype, int64_t idx) {
  if (dtype == ORACLE_F32) return ((const float*)base)[idx];
  return bf16_to_float(((const uint16_t*)base)[idx]);
}

/* ypdtype 2 = double. */
static double elem_d(const void* base, int dtype, int64_t idx) {
  if (dtype == 2) return ((const double*)base)[idx];
  return (double)elem_f(base, dtype, idx);
}

int64_t oracle_capacity(int64_t T, int64_t E, int64_t k, double phi) {
  /* [UD] "Capacity": C = ceil(phi * T * k / E); [SPK] trace:
   * C = ceil(8*2/4 * 1.25) = 5.  No limit when phi <= 0. */
  if (!(phi > 0.0)) return -1;
  double c = ceil(phi * (double)(T * k) / (double)E);
  return (int64_t)c;
}

void oracle_router_logits(int64_t T, int64_t d, int64_t E, int dtype,
                          const void* x, const void* w, const float* b,
                          float* logits) {
  /* [INT8] section 1: scores = x @ W_router + b_router, W stored [E][d].
   * fp32 accumulation ([MML] section 4 casts the router logits to float)
   * in the fixed order of oracle.h ("R64"): the hidden index i belongs to
   * granule i / 8 and granule q to partial sum q mod 64; each partial sum
   * is a chain of fmaf in increasing i from +0; the 64 partial sums are
   * folded by halving (sum l += sum l+s for l < s, s = 32, 16, ..., 1);
   * the bias is added to the result. */
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; t++) {
    for (int64_t e = 0; e < E; e++) {
      float part[64];
      for (int l = 0; l < 64; l++) part[l] = 0.0f;
      for (int64_t i = 0; i < d; i++) {
        const int l = (int)((i / 8) % 64);
        part[l] = fmaf(elem_f(x, dtype, t * d + i), elem_f(w, dtype, e * d + i),
                       part[l]);
      }
      for (int s = 32; s >= 1; s /= 2) {
        for (int l = 0; l < s; l++) part[l] = part[l] + part[l + s];
      }
      float acc = part[0];
      if (b) acc = acc + b[e];
      logits[t * E + e] = acc;
    }
  }
}

void oracle_router_logits_f64(int64_t T, int64_t d, int64_t E, int dtype,
                              const void* x, const void* w, const float* b,
                              double* logits) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; t++) {
    for (int64_t e = 0; e < E; e++) {
      double acc = 0.0;
      for (int64_t i = 0; i < d; i++) {
        acc += (double)elem_f(x, dtype, t * d + i) *
               (double)elem_f(w, dtype, e * d + i);
      }
      if (b) acc += (double)b[e];
      logits[t * E + e] = acc;
    }
  }
}

void oracle_topk_gates(int64_t T, int64_t E, int64_t k, int renorm,
                       const float* logits, int32_t* expert_ids,
                       float* gates) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; t++) {
    const float* l = logits + t * E;
    unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
    int32_t* ids = expert_ids + t * k;
    /* [MML] section 2: logits.topk(k) -- the k largest, largest first.
     * Scanning e upward with a strict ">" keeps the lowest index on ties. */
    for (int64_t j = 0; j < k; j++) {
      int64_t best = -1;
      for (int64_t e = 0; e < E; e++) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e;
      }
      taken[best] = 1;
      ids[j] = (int32_t)best;
    }
    free(taken);
    /* Gates.  renorm: softmax over the selected logits ([MML] section 2,
     * [UD] "The gate"), identical to dividing the selected softmax
     * probabilities by their sum ([SPK] "Top-k and mixture", [INT8]
     * section 3).  No renorm: the full softmax probability ([BEA]). */
    double m = (double)l[ids[0]];
    double denom = 0.0;
    if (renorm) {
      for (int64_t j = 0; j < k; j++) denom += exp((double)l[ids[j]] - m);
    } else {
      for (int64_t e = 0; e < E; e++) denom += exp((double)l[e] - m);
    }
    for (int64_t j = 0; j < k; j++) {
      gates[t * k + j] = (float)(exp((double)l[ids[j]] - m) / denom);
    }
  }
}

void oracle_dispatch(int64_t T, int64_t E, int64_t k, int64_t C,
                     const int32_t* expert_ids, int32_t* counts, int32_t* kept,
                     int32_t* offsets, int32_t* route_pos,
                     int32_t* row_token) {
  int64_t R = T * k;
  int64_t* slot = (int64_t*)malloc((size_t)(R > 0 ? R : 1) * sizeof(int64_t));
  /* Demand count and arrival slot: walk routes in flat order r = t*k + j
   * ([MML] section 3: expert_ids.flatten(), stable argsort).  slot(r) is the
   * number of earlier routes to the same expert = the route's position
   * inside its expert batch. */
  for (int64_t e = 0; e < E; e++) counts[e] = 0;
  for (int64_t r = 0; r < R; r++) {
    int32_t e = expert_ids[r];
    slot[r] = counts[e];
    counts[e] += 1;
  }
  /* Capacity: the first C arrivals are kept ([SPK] trace: the 6th arrival
   * at E1 is dropped when C = 5). */
  for (int64_t e = 0; e < E; e++) {
    kept[e] = (C < 0 || counts[e] <= C) ? counts[e] : (int32_t)C;
  }
  /* bincount(...).cumsum(0) ([MML] section 3) over the kept rows, stored as
   * an exclusive prefix with a leading 0. */
  offsets[0] = 0;
  for (int64_t e = 0; e < E; e++) offsets[e + 1] = offsets[e] + kept[e];
  for (int64_t r = 0; r < R; r++) {
    int32_t e = expert_ids[r];
    if (C < 0 || slot[r] < C) {
      int32_t p = (int32_t)(offsets[e] + slot[r]);
      route_pos[r] = p;
      if (row_token) row_token[p] = (int32_t)(r / k);
    } else {
      route_pos[r] = -1;
    }
  }
  free(slot);
}

void oracle_dispatch_padded(int64_t T, int64_t E, int64_t k, int64_t C,
                            const int32_t* expert_ids, const int32_t* route_pos,
                            const int32_t* offsets, int32_t* pad_pos,
                            int32_t* slot_token) {
  for (int64_t p = 0; p < E * C; p++) slot_token[p] = -1;
  for (int64_t r = 0; r < T * k; r++) {
    if (route_pos[r] < 0) {
      pad_pos[r] = -1;
      continue;
    }
    int32_t e = expert_ids[r];
    int64_t slot = route_pos[r] - offsets[e]; /* arrival rank among kept */
    pad_pos[r] = (int32_t)(e * C + slot);
    slot_token[e * C + slot] = (int32_t)(r / k);
  }
}

void oracle_dispatch_reroute(int64_t T, int64_t E, int64_t k, int64_t C,
                             const float* logits, const int32_t* ids_in,
                             int32_t* ids_out, int32_t* counts, int32_t* filled,
                             int32_t* offsets, int32_t* route_pos,
                             int32_t* row_token, int64_t* n_rerouted) {
  int64_t R = T * k;
  size_t nR = (size_t)(R > 0 ? R : 1);
  int32_t* kept = (int32_t*)malloc((size_t)E * sizeof(int32_t));
  int32_t* offs0 = (int32_t*)malloc((size_t)(E + 1) * sizeof(int32_t));
  int32_t* pos0 = (int32_t*)malloc(nR * sizeof(int32_t));
  int64_t* slot = (int64_t*)malloc(nR * sizeof(int64_t));
  /* pass 1: the drop policy */
  oracle_dispatch(T, E, k, C, ids_in, counts, kept, offs0, pos0, NULL);
  for (int64_t e = 0; e < E; e++) filled[e] = kept[e];
  for (int64_t r = 0; r < R; r++) {
    ids_out[r] = ids_in[r];
    slot[r] = pos0[r] >= 0 ? pos0[r] - offs0[ids_in[r]] : -1;
  }
  /* pass 2: dropped routes in arrival order take the best expert with room */
  int64_t moved = 0;
  for (int64_t r = 0; r < R; r++) {
    if (slot[r] >= 0) continue;
    int64_t t = r / k;
    const float* l = logits + t * E;
    int64_t best = -1;
    for (int64_t e = 0; e < E; e++) {
      if (C >= 0 && filled[e] >= C) continue; /* no room */
      int held = 0;
      for (int64_t j = 0; j < k; j++) held |= (ids_out[t * k + j] == e);
      if (held) continue;
      if (best < 0 || l[e] > l[best]) best = e; /* strict >: lower index on ties */
    }
    if (best < 0) continue; /* stays dropped */
    ids_out[r] = (int32_t)best;
    slot[r] = filled[best];
    filled[best] += 1;
    moved += 1;
  }
  offsets[0] = 0;
  for (int64_t e = 0; e < E; e++) offsets[e + 1] = offsets[e] + filled[e];
  for (int64_t r = 0; r < R; r++) {
    if (slot[r] < 0) {
      route_pos[r] = -1;
      continue;
    }
    int32_t p = (int32_t)(offsets[ids_out[r]] + slot[r]);
    route_pos[r] = p;
    if (row_token) row_token[p] = (int32_t)(r / k);
  }
  if (n_rerouted) *n_rerouted = moved;
  free(kept);
  free(offs0);
  free(pos0);
  free(slot);
}

/* Queue to the next micro-batch ("Session 19", "Overflow policies"): the
 * drop policy over the arrival sequence (queued routes first, then the
 * call's routes), with the routes past capacity listed for the next call
 * instead of being lost. */
int64_t oracle_dispatch_queue(int64_t T, int64_t E, int64_t k, int64_t C, int64_t Q,
                              const int32_t* q_ids, const int32_t* ids, int32_t* counts,
                              int32_t* kept, int32_t* offsets, int32_t* pos,
                              int32_t* row_arrival, int32_t* out_arrival) {
  int64_t N = Q + T * k;
  int32_t* seq = (int32_t*)malloc((size_t)(N > 0 ? N : 1) * sizeof(int32_t));
  for (int64_t a = 0; a < Q; a++) seq[a] = q_ids[a];
  for (int64_t r = 0; r < T * k; r++) seq[Q + r] = ids[r];
  /* one route per arrival: k = 1 over the sequence */
  oracle_dispatch(N, E, 1, C, seq, counts, kept, offsets, pos, row_arrival);
  int64_t n_out = 0;
  for (int64_t a = 0; a < N; a++)
    if (pos[a] < 0) out_arrival[n_out++] = (int32_t)a;
  free(seq);
  return n_out;
}

/* Expert-choice routing ("MoE Inference Visualized", "Why MoE Matters for
 * Infrastructure": against load imbalance the experts can pick the tokens
 * instead of the tokens picking experts).  The page names the idea only.
 * Reading: the score of (t, e) is the full softmax probability of the
 * router logits; each expert takes the Ce = min(C, T) tokens of largest
 * score (C < 0: no limit, Ce = T); a token's gate for an expert that took it
 * is that score. */
typedef struct {
  float s;
  int32_t t;
} ec_item;

/* larger score first; the lower token index first among equal scores */
static int ec_order(const void* a, const void* b) {
  const ec_item* x = (const ec_item*)a;
  const ec_item* y = (const ec_item*)b;
  if (x->s != y->s) return x->s > y->s ? -1 : 1;
  return x->t < y->t ? -1 : (x->t > y->t ? 1 : 0);
}

void oracle_expert_choice(int64_t T, int64_t E, int64_t C, const float* logits,
                          float* scores, int32_t* route_pos, int32_t* row_token) {
  const int64_t Ce = (C < 0 || C > T) ? T : C;
  /* scores: softmax over all E logits of the token, in double, stored as
   * the fp32 gate (the decision below is taken on this stored value) */
  for (int64_t t = 0; t < T; t++) {
    const float* l = logits + t * E;
    double m = (double)l[0];
    for (int64_t e = 1; e < E; e++)
      if ((double)l[e] > m) m = (double)l[e];
    double denom = 0.0;
    for (int64_t e = 0; e < E; e++) denom += exp((double)l[e] - m);
    for (int64_t e = 0; e < E; e++)
      scores[t * E + e] = (float)(exp((double)l[e] - m) / denom);
  }
  ec_item* items = (ec_item*)malloc((size_t)(T > 0 ? T : 1) * sizeof(ec_item));
  unsigned char* chosen = (unsigned char*)malloc((size_t)(T > 0 ? T : 1));
  for (int64_t e = 0; e < E; e++) {
    /* expert e ranks every token by its score and keeps the first Ce */
    for (int64_t t = 0; t < T; t++) {
      items[t].s = scores[t * E + e];
      items[t].t = (int32_t)t;
    }
    qsort(items, (size_t)T, sizeof(ec_item), ec_order);
    memset(chosen, 0, (size_t)(T > 0 ? T : 1));
    for (int64_t i = 0; i < Ce; i++) chosen[items[i].t] = 1;
    /* its rows: Ce of them from row e*Ce, its tokens in increasing index */
    int64_t n = 0;
    for (int64_t t = 0; t < T; t++) {
      if (chosen[t]) {
        route_pos[t * E + e] = (int32_t)(e * Ce + n);
        if (row_token) row_token[e * Ce + n] = (int32_t)t;
        n++;
      } else {
        route_pos[t * E + e] = -1;
      }
    }
  }
  free(items);
  free(chosen);
}

void oracle_gather_rows(int64_t n_rows, int64_t d, int64_t elem_bytes,
                        const void* x, const int32_t* row_token,
                        void* packed) {
  /* [MML] section 3: packed = x.index_select(0, token_ids[order]). */
  size_t row_bytes = (size_t)(d * elem_bytes);
  for (int64_t p = 0; p < n_rows; p++) {
    memcpy((char*)packed + (size_t)p * row_bytes,
           (const char*)x + (size_t)row_token[p] * row_bytes, row_bytes);
  }
}

/* One row through a SwiGLU expert, in double ([BEA] "Expert Execution":
 * down_proj(SiLU(gate_proj(x)) * up_proj(x)); SiLU(a) = a * sigmoid(a)).
 * xrow: element offset x_off into x; weights already offset to the expert. */
static void swiglu_row(int64_t d, int64_t d_ff, int dtype, const void* x,
                       int64_t x_off, const void* wg, int64_t wg_off,
                       const void* wu, int64_t wu_off, const void* wd,
                       int64_t wd_off, double* h, double* yrow) {
  for (int64_t f = 0; f < d_ff; f++) {
    double a = 0.0, bb = 0.0;
    for (int64_t i = 0; i < d; i++) {
      double xi = (double)elem_f(x, dtype, x_off + i);
      a += xi * (double)elem_f(wg, dtype, wg_off + f * d + i);
      bb += xi * (double)elem_f(wu, dtype, wu_off + f * d + i);
    }
    double silu = a / (1.0 + exp(-a));
    h[f] = silu * bb;
  }
  for (int64_t i = 0; i < d; i++) {
    double acc = 0.0;
    for (int64_t f = 0; f < d_ff; f++) {
      acc += h[f] * (double)elem_f(wd, dtype, wd_off + i * d_ff + f);
    }
    yrow[i] = acc;
  }
}

void oracle_swiglu_rows(int64_t n, int64_t d, int64_t d_ff, int dtype,
                        const void* x, const void* wg, const void* wu,
                        const void* wd, double* y) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t p = 0; p < n; p++) {
    double* h = (double*)malloc((size_t)d_ff * sizeof(double));
    swiglu_row(d, d_ff, dtype, x, p * d, wg, 0, wu, 0, wd, 0, h, y + p * d);
    free(h);
  }
}

void oracle_expert_ffn(int64_t E, int64_t d, int64_t d_ff, int dtype,
                       const int32_t* offsets, const void* x_packed,
                       const void* w_gate, const void* w_up,
                       const void* w_down, double* y_packed) {
  int64_t n = offsets[E];
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t p = 0; p < n; p++) {
    int64_t e = 0;
    while (!(p >= offsets[e] && p < offsets[e + 1])) e++;
    double* h = (double*)malloc((size_t)d_ff * sizeof(double));
    swiglu_row(d, d_ff, dtype, x_packed, p * d, w_gate, e * d_ff * d, w_up,
               e * d_ff * d, w_down, e * d * d_ff, h, y_packed + p * d);
    free(h);
  }
}

void oracle_combine(int64_t T, int64_t k, int64_t d, int ypdtype,
                    const void* y_packed, const int32_t* route_pos,
                    const float* gates, const void* y_shared, double* y) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; t++) {
    for (int64_t i = 0; i < d; i++) {
      double acc = 0.0;
      for (int64_t j = 0; j < k; j++) {
        int32_t p = route_pos[t * k + j];
        if (p < 0) continue; /* dropped: contributes nothing */
        acc += (double)gates[t * k + j] *
               elem_d(y_packed, ypdtype, (int64_t)p * d + i);
      }
      if (y_shared) acc += elem_d(y_shared, ypdtype, t * d + i);
      y[t * d + i] = acc;
    }
  }
}

void oracle_routing_stats(int64_t T, int64_t E, int64_t k, const float* logits,
                          const float* gates, const int32_t* counts,
                          double alpha, int32_t n_bins, double* out,
                          double* share, double* mean_prob, int64_t* hist) {
  for (int i = 0; i < 6; i++) out[i] = 0.0;
  for (int64_t e = 0; e < E; e++) {
    share[e] = 0.0;
    mean_prob[e] = 0.0;
  }
  for (int32_t b = 0; b < n_bins; b++) hist[b] = 0;
  if (T <= 0) return;
  /* route shares f_e and the demand imbalance */
  double R = (double)T * (double)k;
  double cmax = 0.0;
  for (int64_t e = 0; e < E; e++) {
    share[e] = (double)counts[e] / R;
    if ((double)counts[e] > cmax) cmax = (double)counts[e];
  }
  out[1] = cmax / (R / (double)E);
  /* per token: softmax over all experts, confidence, gates */
  double sum_max_gate = 0.0, sum_entropy = 0.0, sum_conf = 0.0;
  for (int64_t t = 0; t < T; t++) {
    const float* l = logits + t * E;
    double m = (double)l[0];
    for (int64_t e = 1; e < E; e++)
      if ((double)l[e] > m) m = (double)l[e];
    double z = 0.0;
    for (int64_t e = 0; e < E; e++) z += exp((double)l[e] - m);
    for (int64_t e = 0; e < E; e++) mean_prob[e] += exp((double)l[e] - m) / z;
    double conf = 1.0 / z; /* probability of the largest logit */
    sum_conf += conf;
    int32_t b = (int32_t)floor(conf * (double)n_bins);
    if (b >= n_bins) b = n_bins - 1;
    if (b < 0) b = 0;
    hist[b] += 1;
    const float* g = gates + t * k;
    double gmax = (double)g[0], gsum = 0.0;
    for (int64_t j = 0; j < k; j++) {
      if ((double)g[j] > gmax) gmax = (double)g[j];
      gsum += (double)g[j];
    }
    sum_max_gate += gmax;
    if (k > 1 && gsum > 0.0) {
      double h = 0.0;
      for (int64_t j = 0; j < k; j++) {
        double q = (double)g[j] / gsum;
        if (q > 0.0) h -= q * log(q);
      }
      sum_entropy += h / log((double)k);
    }
  }
  for (int64_t e = 0; e < E; e++) mean_prob[e] /= (double)T;
  double aux = 0.0;
  for (int64_t e = 0; e < E; e++) aux += share[e] * mean_prob[e];
  out[0] = alpha * (double)E * aux;
  out[2] = sum_max_gate / (double)T;
  out[3] = sum_entropy / (double)T;
  /* Jensen-Shannon divergence (base 2) of f and the uniform load */
  double js = 0.0, u = 1.0 / (double)E;
  for (int64_t e = 0; e < E; e++) {
    double mid = 0.5 * (share[e] + u);
    if (share[e] > 0.0) js += 0.5 * share[e] * log2(share[e] / mid);
    js += 0.5 * u * log2(u / mid);
  }
  out[4] = sqrt(js > 0.0 ? js : 0.0);
  out[5] = sum_conf / (double)T;
}

int oracle_layer_forward(int64_t T, int64_t d, int64_t E, int64_t k,
                         int64_t d_ff, int64_t d_ff_shared, int dtype,
                         int renorm, double phi, const void* x,
                         const void* w_router, const float* b_router,
                         const void* w_gate, const void* w_up,
                         const void* w_down, const void* ws_gate,
                         const void* ws_up, const void* ws_down,
                         int64_t n_sel, const int32_t* sel, double* y,
                         int32_t* ids_out, float* gates_out,
                         int32_t* counts_out, int32_t* route_pos_out) {
  if (T < 0 || d <= 0 || E <= 0 || k <= 0 || k > E || d_ff <= 0) return -1;
  if (d_ff_shared > 0 && (!ws_gate || !ws_up || !ws_down)) return -1;
  int64_t R = T * k;
  size_t nR = (size_t)(R > 0 ? R : 1);
  float* logits = (float*)malloc((size_t)(T > 0 ? T : 1) * E * sizeof(float));
  int32_t* ids = (int32_t*)malloc(nR * sizeof(int32_t));
  float* gates = (float*)malloc(nR * sizeof(float));
  int32_t* counts = (int32_t*)malloc((size_t)E * sizeof(int32_t));
  int32_t* kept = (int32_t*)malloc((size_t)E * sizeof(int32_t));
  int32_t* offsets = (int32_t*)malloc((size_t)(E + 1) * sizeof(int32_t));
  int32_t* route_pos = (int32_t*)malloc(nR * sizeof(int32_t));

  /* route */
  oracle_router_logits(T, d, E, dtype, x, w_router, b_router, logits);
  oracle_topk_gates(T, E, k, renorm, logits, ids, gates);
  /* pack (the slot bookkeeping; rows are read straight from x below, which
   * is the same bits as the packed copy) */
  int64_t C = oracle_capacity(T, E, k, phi);
  oracle_dispatch(T, E, k, C, ids, counts, kept, offsets, route_pos, NULL);

  /* compute + combine, one output token at a time ([MML] section 1 loop:
   * for each token, for each selected slot, y += g * E_id(x)). */
  int64_t n_out = sel ? n_sel : T;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t s = 0; s < n_out; s++) {
    int64_t t = sel ? sel[s] : s;
    int64_t hmax = d_ff > d_ff_shared ? d_ff : d_ff_shared;
    double* h = (double*)malloc((size_t)hmax * sizeof(double));
    double* ye = (double*)malloc((size_t)d * sizeof(double));
    double* yt = y + s * d;
    for (int64_t i = 0; i < d; i++) yt[i] = 0.0;
    for (int64_t j = 0; j < k; j++) {
      if (route_pos[t * k + j] < 0) continue; /* dropped route */
      int64_t e = ids[t * k + j];
      swiglu_row(d, d_ff, dtype, x, t * d, w_gate, e * d_ff * d, w_up,
                 e * d_ff * d, w_down, e * d * d_ff, h, ye);
      double g = (double)gates[t * k + j];
      for (int64_t i = 0; i < d; i++) yt[i] += g * ye[i];
    }
    if (d_ff_shared > 0) {
      /* always-on shared expert, outside the gate normalisation */
      swiglu_row(d, d_ff_shared, dtype, x, t * d, ws_gate, 0, ws_up, 0,
                 ws_down, 0, h, ye);
      for (int64_t i = 0; i < d; i++) yt[i] += ye[i];
    }
    free(h);
    free(ye);
  }

  if (ids_out) memcpy(ids_out, ids, (size_t)R * sizeof(int32_t));
  if (gates_out) memcpy(gates_out, gates, (size_t)R * sizeof(float));
  if (counts_out) memcpy(counts_out, counts, (size_t)E * sizeof(int32_t));
  if (route_pos_out) memcpy(route_pos_out, route_pos, (size_t)R * sizeof(int32_t));
  free(logits);
  free(ids);
  free(gates);
  free(counts);
  free(kept);
  free(offsets);
  free(route_pos);
  return 0;
}

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
                                       int32_t* route_pos_out) {
  if (T < 0 || d <= 0 || E <= 0 || d_ff <= 0) return -1;
  if (d_ff_shared > 0 && (!ws_gate || !ws_up || !ws_down)) return -1;
  size_t nTE = (size_t)(T > 0 ? T : 1) * (size_t)E;
  float* logits = (float*)malloc(nTE * sizeof(float));
  float* scores = (float*)malloc(nTE * sizeof(float));
  int32_t* route_pos = (int32_t*)malloc(nTE * sizeof(int32_t));
  oracle_router_logits(T, d, E, dtype, x, w_router, b_router, logits);
  oracle_expert_choice(T, E, C, logits, scores, route_pos, NULL);
  /* [MML] section 1: y = sum over the experts that hold the token of
   * gate * E_e(x), here over the experts that chose it, in expert order */
  int64_t n_out = sel ? n_sel : T;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t s = 0; s < n_out; s++) {
    int64_t t = sel ? sel[s] : s;
    int64_t hmax = d_ff > d_ff_shared ? d_ff : d_ff_shared;
    double* h = (double*)malloc((size_t)hmax * sizeof(double));
    double* ye = (double*)malloc((size_t)d * sizeof(double));
    double* yt = y + s * d;
    for (int64_t i = 0; i < d; i++) yt[i] = 0.0;
    for (int64_t e = 0; e < E; e++) {
      if (route_pos[t * E + e] < 0) continue; /* expert e did not take t */
      swiglu_row(d, d_ff, dtype, x, t * d, w_gate, e * d_ff * d, w_up,
                 e * d_ff * d, w_down, e * d * d_ff, h, ye);
      double g = (double)scores[t * E + e];
      for (int64_t i = 0; i < d; i++) yt[i] += g * ye[i];
    }
    if (d_ff_shared > 0) {
      swiglu_row(d, d_ff_shared, dtype, x, t * d, ws_gate, 0, ws_up, 0,
                 ws_down, 0, h, ye);
      for (int64_t i = 0; i < d; i++) yt[i] += ye[i];
    }
    free(h);
    free(ye);
  }
  if (scores_out) memcpy(scores_out, scores, (size_t)(T * E) * sizeof(float));
  if (route_pos_out)
    memcpy(route_pos_out, route_pos, (size_t)(T * E) * sizeof(int32_t));
  free(logits);
  free(scores);
  free(route_pos);
  return 0;
}
