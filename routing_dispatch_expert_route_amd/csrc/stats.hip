// stats.hip -- forward-only routing statistics of one batch of routes.
//
// "Mixture of Experts: Routing, Dispatch, and Load Balancing", section 4:
// the Switch auxiliary load-balancing loss alpha * N * sum_i f_i P_i (f_i the
// share of tokens dispatched to expert i, P_i its mean routing probability).
// "Mixture-of-experts routing", load imbalance: max demand over mean demand,
// measured before capacity.  "271,104 Routes", section 4: selection share,
// largest selected weight, normalised routing entropy, Jensen-Shannon
// distance between load vectors.  "MoE Inference Visualized", "Router
// Confidence": the softmax probability of the chosen expert.
//
// Two kernels, no atomics on floating point (every sum has a fixed order):
//   stats_partial_kernel  64 tokens per block: softmax of each token's
//       logits (sequential over experts), its confidence bin, largest gate
//       and gate entropy; then per expert the block's sum of probabilities
//       over its tokens in token order.  Writes one partial row per block.
//   stats_final_kernel    one block: sums the partial rows (each column's
//       rows in interleaved slices, each slice in row order, then the slices
//       in order) and forms the statistics.
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kStatTok = 64;  // tokens per block

__global__ __launch_bounds__(256) void stats_partial_kernel(const float* __restrict__ logits,
                                                            const float* __restrict__ gates,
                                                            int T, int E, int k, int n_bins,
                                                            float* __restrict__ part,
                                                            int32_t* __restrict__ hpart) {
  __shared__ float s_l[kStatTok * 257];  // the block's logits, row stride E + 1
  __shared__ float s_m[kStatTok], s_iz[kStatTok];
  __shared__ float s_tok[3][kStatTok];
  __shared__ float s_scr[256];
  __shared__ int s_hist[kMaxStatBins];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kStatTok;
  const int nt = min(kStatTok, T - t0);
  const int ls = E + 1;
  for (int i = tid; i < nt * E; i += 256) s_l[(i / E) * ls + i % E] = logits[(size_t)t0 * E + i];
  for (int b = tid; b < n_bins; b += 256) s_hist[b] = 0;
  __syncthreads();
  if (tid < kStatTok) {
    float gmax = 0.0f, ent = 0.0f, conf = 0.0f;
    if (tid < nt) {
      const float* l = s_l + tid * ls;
      float m = l[0];
      for (int e = 1; e < E; ++e) m = fmaxf(m, l[e]);
      float z = 0.0f;
      for (int e = 0; e < E; ++e) z += __expf(l[e] - m);
      const float iz = 1.0f / z;
      s_m[tid] = m;
      s_iz[tid] = iz;
      conf = iz;  // probability of the largest logit
      int b = (int)(conf * (float)n_bins);
      b = b < n_bins ? b : n_bins - 1;
      atomicAdd(&s_hist[b], 1);  // integer counts: any order gives the same result
      const float* g = gates + (size_t)(t0 + tid) * k;
      float gs = 0.0f;
      gmax = g[0];
      for (int j = 0; j < k; ++j) {
        gmax = fmaxf(gmax, g[j]);
        gs += g[j];
      }
      if (k > 1 && gs > 0.0f) {
        float h = 0.0f;
        for (int j = 0; j < k; ++j) {
          const float q = g[j] / gs;
          if (q > 0.0f) h -= q * __logf(q);
        }
        ent = h / __logf((float)k);
      }
    }
    s_tok[0][tid] = gmax;
    s_tok[1][tid] = ent;
    s_tok[2][tid] = conf;
  }
  __syncthreads();
  const size_t row = (size_t)blockIdx.x * (E + 3);
  {
    // per expert, its probabilities summed over the block's tokens: token t
    // in slice t mod S, one thread per (expert, slice) in token order, then
    // the slices in order (up to 8 slices when the experts are few)
    int w = 1;
    while (w < E && w < 256) w *= 2;
    const int S = 256 / w < 8 ? 256 / w : 8;
    const int G = 256 / S;
    const int cl = tid % G, sl = tid / G;
    for (int e0 = 0; e0 < E; e0 += G) {
      const int e = e0 + cl;
      float acc = 0.0f;
      if (e < E)
        for (int t = sl; t < nt; t += S) acc += __expf(s_l[t * ls + e] - s_m[t]) * s_iz[t];
      s_scr[tid] = acc;
      __syncthreads();
      if (sl == 0 && e < E) {
        float v = s_scr[cl];
        for (int j = 1; j < S; ++j) v += s_scr[j * G + cl];
        part[row + e] = v;
      }
      __syncthreads();
    }
  }
  if (tid < 3) {
    float acc = 0.0f;
    for (int t = 0; t < kStatTok; ++t) acc += s_tok[tid][t];
    part[row + E + tid] = acc;
  }
  for (int b = tid; b < n_bins; b += 256) hpart[(size_t)blockIdx.x * n_bins + b] = s_hist[b];
}

// Column sums of a row-major [nblk][ld] array, columns 0 .. nc-1, into
// out[0 .. nc).  Row r belongs to slice r mod S; one thread sums a column's
// slice in row order with sixteen loads in flight, then the S slice sums are
// added in slice order -- a fixed order, so repeat calls agree.  The fewer
// the columns, the more slices (up to 8), so that a few columns still keep
// the block's 256 threads loading.  Every thread of the block calls it.
template <typename V>
__device__ void block_column_sums(const V* __restrict__ a, int nblk, int ld, int nc,
                                  V* __restrict__ out, V* __restrict__ s_scr /*[256]*/) {
  int w = 1;
  while (w < nc && w < 256) w *= 2;
  const int S = 256 / w < 8 ? 256 / w : 8;  // slices
  const int G = 256 / S;                    // columns per pass
  const int tid = threadIdx.x;
  const int cl = tid % G, sl = tid / G;
  for (int c0 = 0; c0 < nc; c0 += G) {
    const int c = c0 + cl;
    V acc = 0;
    if (c < nc) {
      for (int r0 = sl; r0 < nblk; r0 += 16 * S) {
        V v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int r = r0 + u * S;
          v[u] = r < nblk ? a[(size_t)r * ld + c] : V(0);
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) acc += v[u];
      }
    }
    s_scr[tid] = acc;
    __syncthreads();
    if (sl == 0 && c < nc) {
      V t = s_scr[cl];
      for (int j = 1; j < S; ++j) t += s_scr[j * G + cl];
      out[c] = t;
    }
    __syncthreads();
  }
}

// stats: [0] aux loss, [1] load imbalance, [2] mean largest gate, [3] mean
// normalised entropy, [4] JS distance of the shares to uniform (base 2),
// [5] mean confidence, [6, 6+E) shares, [6+E, 6+2E) mean probabilities.
__global__ __launch_bounds__(256) void stats_final_kernel(const float* __restrict__ part,
                                                          const int32_t* __restrict__ hpart,
                                                          int nblk, const int32_t* __restrict__ counts,
                                                          int T, int E, int k, int n_bins,
                                                          float alpha, float* __restrict__ stats,
                                                          int32_t* __restrict__ hist) {
  __shared__ float s_f[256], s_p[256];
  __shared__ float s_col[256 + 3];
  __shared__ float s_scrf[256];
  __shared__ int32_t s_scri[256];
  const int tid = threadIdx.x;
  const float inv_t = T > 0 ? 1.0f / (float)T : 0.0f;
  const float R = (float)T * (float)k;
  block_column_sums(part, nblk, E + 3, E + 3, s_col, s_scrf);
  block_column_sums(hpart, nblk, n_bins, n_bins, hist, s_scri);
  for (int e = tid; e < E; e += 256) {
    const float p = s_col[e] * inv_t;
    const float f = T > 0 ? (float)counts[e] / R : 0.0f;
    s_f[e] = f;
    s_p[e] = p;
    stats[6 + e] = f;
    stats[6 + E + e] = p;
  }
  __syncthreads();
  if (tid < kWave) {
    // wave 0: lane l takes experts l, l + 64, ... in order, then the lanes'
    // terms are folded by halving (a fixed order)
    float aux = 0.0f, cmax = 0.0f, js = 0.0f;
    const float u = 1.0f / (float)E;
    for (int e = tid; e < E; e += kWave) {
      aux += s_f[e] * s_p[e];
      cmax = fmaxf(cmax, (float)counts[e]);
      const float mid = 0.5f * (s_f[e] + u);
      if (s_f[e] > 0.0f) js += 0.5f * s_f[e] * __log2f(s_f[e] / mid);
      js += 0.5f * u * __log2f(u / mid);
    }
    for (int sh = kWave / 2; sh >= 1; sh /= 2) {
      aux += __shfl_xor(aux, sh, kWave);
      js += __shfl_xor(js, sh, kWave);
      cmax = fmaxf(cmax, __shfl_xor(cmax, sh, kWave));
    }
    if (tid == 0) {
      const bool any = T > 0;
      stats[0] = any ? alpha * (float)E * aux : 0.0f;
      stats[1] = any ? cmax / (R / (float)E) : 0.0f;
      stats[2] = s_col[E] * inv_t;
      stats[3] = s_col[E + 1] * inv_t;
      stats[4] = any ? sqrtf(fmaxf(js, 0.0f)) : 0.0f;
      stats[5] = s_col[E + 2] * inv_t;
    }
  }
}

int stats_blocks(long T) { return (int)((T + kStatTok - 1) / kStatTok); }

hipError_t launch_routing_stats(const float* logits, const float* gates, const int32_t* counts,
                                int T, int E, int k, int n_bins, float alpha, float* part,
                                int32_t* hpart, float* stats, int32_t* hist, hipStream_t st) {
  const int nblk = stats_blocks(T);
  if (nblk > 0) {
    hipLaunchKernelGGL(stats_partial_kernel, dim3(nblk), dim3(256), 0, st, logits, gates, T, E, k,
                       n_bins, part, hpart);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(256), 0, st, part, hpart, nblk, counts, T, E,
                     k, n_bins, alpha, stats, hist);
  return hipGetLastError();
}

}  // namespace moe
