// choice.hip -- expert-choice routing: the experts pick their tokens.
//
// "MoE Inference Visualized", "Why MoE Matters for Infrastructure": against
// load imbalance the experts can choose the tokens instead of the tokens
// choosing experts; every expert then receives the same number of rows.
// The page names the idea only.  Reading used here: the score of (t, e) is
// the full softmax probability of the router logits; expert e keeps the
// Ce = min(C, T) tokens of largest score, the lower token index first among
// equal scores; a kept pair's gate is its score; a token may be kept by any
// number of experts, none included.
//
// ec_scores_kernel  softmax of each token's logits -> scores [T][E] (when
//                   asked for) and keys [E][T] (the score's bits,
//                   expert-major so that one expert's column is contiguous;
//                   scores are >= +0, so their bits order like the values;
//                   read back as floats they are also the gates).
// ec_select_kernel  one block per expert: the Ce-th largest key of its
//                   column by radix passes (exact LDS histograms), then
//                   seating -- the keys above it and the first Ce -
//                   count(key > thr) equal to it in token order -- so expert
//                   e's rows e*Ce .. e*Ce+Ce-1 list its tokens in increasing
//                   index; the route table is written expert-major [E][T]
//                   (coalesced).  The result is unique and does not depend
//                   on timing (the histogram atomics add integers).
// ec_transpose_kernel  the [T][E] route table for callers that ask for it.
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kScoreTok = 32;   // tokens per block of the score kernel
constexpr int kScoreLanes = 8;  // threads per token

__global__ __launch_bounds__(256) void ec_scores_kernel(const float* __restrict__ logits, int T,
                                                        int E, float* __restrict__ scores,
                                                        uint32_t* __restrict__ keys) {
  extern __shared__ float s_l[];  // [kScoreTok][E+1]
  const int t0 = blockIdx.x * kScoreTok;
  const int nt = min(kScoreTok, T - t0);
  const int stride = E + 1;
  const int n = nt * E;
  const float* src = logits + (size_t)t0 * E;
  for (int i = threadIdx.x; i < n; i += blockDim.x) s_l[(i / E) * stride + i % E] = src[i];
  __syncthreads();
  const int j = threadIdx.x / kScoreLanes;  // token of this thread
  const int q = threadIdx.x % kScoreLanes;  // its share of the experts
  if (j < nt) {
    float* row = s_l + j * stride;
    float m = -INFINITY;
    for (int e = q; e < E; e += kScoreLanes) m = fmaxf(m, row[e]);
#pragma unroll
    for (int o = 1; o < kScoreLanes; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kScoreLanes));
    float sum = 0.0f;
    for (int e = q; e < E; e += kScoreLanes) {
      const float v = expf(row[e] - m);
      row[e] = v;
      sum += v;
    }
#pragma unroll
    for (int o = 1; o < kScoreLanes; o <<= 1) sum += __shfl_xor(sum, o, kScoreLanes);
    const float inv = 1.0f / sum;
    for (int e = q; e < E; e += kScoreLanes) row[e] *= inv;
  }  // the shuffles stay inside groups of kScoreLanes lanes, all on one token
  __syncthreads();
  if (scores) {
    float* dst = scores + (size_t)t0 * E;
    for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = s_l[(i / E) * stride + i % E];
  }
  // expert-major keys: consecutive threads take consecutive tokens
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int e = i / nt, jj = i % nt;
    keys[(size_t)e * T + t0 + jj] = __float_as_uint(s_l[jj * stride + e]);
  }
}

// One block of NT threads per expert, its column of keys read from memory
// (L2) in every pass.  The Ce-th largest key comes from four radix passes of
// 8 bits (largest digit first): each pass counts, in an LDS histogram, the
// digit of the keys that match the digits chosen so far (integer atomics:
// exact counts), and one wave picks the digit where the count of keys at or
// above it reaches the keys still needed.  Seating gives each wave a
// contiguous range of tokens: one pass counts every wave's keys above and
// equal to thr, one barrier, and a second pass walks each range 64 tokens at
// a time with running counts (ballots), so an expert's rows list its tokens
// in increasing index.
template <int NT>
__global__ __launch_bounds__(NT) void ec_select_kernel(const uint32_t* __restrict__ keys,
                                                            int T, int E, int Ce,
                                                            int32_t* __restrict__ pos_et,
                                                            int32_t* __restrict__ row_token,
                                                            int32_t* __restrict__ offsets) {
  constexpr int NW = NT / 64;
  __shared__ uint32_t s_h[256];
  __shared__ int s_sel[2];
  __shared__ uint32_t s_tot[NW][2];
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const uint32_t* col = keys + (size_t)e * T;
  uint32_t prefix = 0, pmask = 0;
  int need = Ce;  // keys still to take among those matching prefix under pmask
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += NT) s_h[i] = 0u;
    __syncthreads();
    for (int t = tid; t < T; t += NT) {
      const uint32_t k = col[t];
      if ((k & pmask) == prefix) atomicAdd(&s_h[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wid == 0) {
      // lane l holds digits 4l .. 4l+3; above = keys with a digit past them
      uint32_t b[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) b[q] = s_h[4 * lane + q];
      const uint32_t lsum = b[0] + b[1] + b[2] + b[3];
      uint32_t sfx = lsum;  // sum over lanes >= this one
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = __shfl_down(sfx, o, 64);
        if (lane + o < 64) sfx += v;
      }
      uint32_t ge = sfx - lsum;  // count of keys with a digit above 4l+3
      // the digit d with count(>= d) >= need and (d = 255 or count(> d) <
      // need): unique, since count(>= d) grows as d falls
#pragma unroll
      for (int q = 3; q >= 0; --q) {
        const uint32_t gt = ge;
        ge += b[q];
        const int d = 4 * lane + q;
        if ((int)ge >= need && (d == 255 || (int)gt < need)) {
          s_sel[0] = d;
          s_sel[1] = need - (int)gt;
        }
      }
    }
    __syncthreads();
    prefix |= (uint32_t)s_sel[0] << shift;
    pmask |= 255u << shift;
    need = s_sel[1];
  }
  const uint32_t thr = prefix;  // the Ce-th largest key (Ce > 0)
  // need = keys equal to thr to seat, in token order
  const int per = ((T + NW - 1) / NW + 63) / 64 * 64;
  const int w0 = min(T, wid * per), w1 = min(T, w0 + per);
  uint32_t cgt = 0, ceq = 0;
  for (int t0 = w0; t0 < w1; t0 += 64) {
    const int t = t0 + lane;
    const bool valid = t < w1;
    const uint32_t k = valid ? col[t] : 0u;
    cgt += (uint32_t)__popcll(__ballot(valid && k > thr));
    ceq += (uint32_t)__popcll(__ballot(valid && k == thr));
  }
  if (lane == 0) {
    s_tot[wid][0] = cgt;
    s_tot[wid][1] = ceq;
  }
  __syncthreads();
  int bgt = 0, beq = 0;  // keys above / equal to thr before this wave's range
  for (int w = 0; w < wid; ++w) {
    bgt += (int)s_tot[w][0];
    beq += (int)s_tot[w][1];
  }
  const uint64_t below = (1ull << lane) - 1ull;
  for (int t0 = w0; t0 < w1; t0 += 64) {
    const int t = t0 + lane;
    const bool valid = t < w1;
    const uint32_t k = valid ? col[t] : 0u;
    const bool gt = valid && k > thr, eq = valid && k == thr;
    const uint64_t mg = __ballot(gt), me = __ballot(eq);
    const int gb = bgt + __popcll(mg & below);
    const int eb = beq + __popcll(me & below);
    const int pos = gb + min(eb, need);
    const bool sel = (gt || (eq && eb < need)) && pos < Ce;
    if (valid) pos_et[(size_t)e * T + t] = sel ? e * Ce + pos : -1;
    if (sel) row_token[e * Ce + pos] = t;
    bgt += __popcll(mg);
    beq += __popcll(me);
  }
  if (tid == 0) {
    offsets[e] = e * Ce;
    if (e == E - 1) offsets[E] = E * Ce;
  }
}

// route_pos[t][e] = pos_et[e][t], through a tile of kTrTok tokens in LDS
// (E * (kTrTok + 1) ints: 33 KiB at E = 256).
constexpr int kTrTok = 32;
__global__ __launch_bounds__(256) void ec_transpose_kernel(const int32_t* __restrict__ pos_et,
                                                           int T, int E,
                                                           int32_t* __restrict__ route_pos) {
  extern __shared__ int32_t s_t[];  // [E][kTrTok + 1]
  const int t0 = blockIdx.x * kTrTok;
  const int nt = min(kTrTok, T - t0);
  for (int i = threadIdx.x; i < E * kTrTok; i += blockDim.x) {
    const int e = i / kTrTok, j = i % kTrTok;
    if (j < nt) s_t[e * (kTrTok + 1) + j] = pos_et[(size_t)e * T + t0 + j];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nt * E; i += blockDim.x) {
    const int j = i / E, e = i % E;
    route_pos[(size_t)(t0 + j) * E + e] = s_t[e * (kTrTok + 1) + j];
  }
}

hipError_t launch_expert_choice(const float* logits, int T, int E, int Ce, float* scores,
                                uint32_t* keys, int32_t* pos_et, int32_t* route_pos,
                                int32_t* row_token, int32_t* offsets, hipStream_t st) {
  // T = 0: no scores; the select blocks still write offsets (all zero)
  if (T > 0) {
    const size_t lds = (size_t)kScoreTok * (E + 1) * sizeof(float);
    hipLaunchKernelGGL(ec_scores_kernel, dim3(ceil_div(T, kScoreTok)),
                       dim3(kScoreTok * kScoreLanes), lds, st, logits, T, E, scores, keys);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL((ec_select_kernel<1024>), dim3(E), dim3(1024), 0, st, keys, T, E, Ce, pos_et,
                     row_token, offsets);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !route_pos || T == 0) return err;
  hipLaunchKernelGGL(ec_transpose_kernel, dim3(ceil_div(T, kTrTok)), dim3(256),
                     (size_t)E * (kTrTok + 1) * sizeof(int32_t), st, pos_et, T, E, route_pos);
  return hipGetLastError();
}

}  // namespace moe
