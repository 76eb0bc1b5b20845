// route.hip -- router projection, softmax and top-k.
//
// "Mixture of Experts: Routing, Dispatch, and Load Balancing", section 1:
// the router is a linear projection x W^T + b to one logit per expert,
// followed by softmax.  "271,104 Routes", section 2: topk on the logits, then
// softmax over the k selected logits (the renormalised gate); "MoE Inference
// Visualized", "Expert Execution": the top-1 output is scaled by its full
// softmax probability (no renormalisation).
//
// Two kernels:
//   router_logits_kernel  one lane per (token, group of EL experts): each
//       logit is a sequential fp32 fused multiply-add over the hidden index
//       in increasing order, bias added after the sum.  That fixed order is
//       what makes the logits -- and so the selected expert ids at near
//       ties -- bit-reproducible.  The lane's token row streams through
//       16-byte vector loads; the expert rows are wave-uniform, so the
//       compiler fetches them with scalar loads shared by the 64 lanes.
//   topk_gates_kernel  one lane per token over an LDS copy of its logits:
//       a single insertion pass keeps the k best by (logit desc, index asc),
//       then the gates.
#include "common.h"
#include "launch.h"

namespace moe {

template <bool BF16>
struct Granule;
template <>
struct Granule<true> {
  static constexpr int N = 8;  // 8 bf16 per 16 bytes
  __device__ __forceinline__ static void load(const void* p, float* v) {
    u32x4_t u = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = bf16lo(u[q]);
      v[2 * q + 1] = bf16hi(u[q]);
    }
  }
};
template <>
struct Granule<false> {
  static constexpr int N = 4;  // 4 fp32 per 16 bytes
  __device__ __forceinline__ static void load(const void* p, float* v) {
    f32x4_t u = *reinterpret_cast<const f32x4_t*>(p);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = u[q];
  }
};

template <bool BF16, int EL>
__global__ __launch_bounds__(256) void router_logits_kernel(
    const void* __restrict__ x, const void* __restrict__ w, const float* __restrict__ b, int T,
    int d, int E, float* __restrict__ logits) {
  using G = Granule<BF16>;
  constexpr int esz = BF16 ? 2 : 4;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int t = blockIdx.x * kWave + lane;
  const int e0 = (blockIdx.y * (blockDim.x / kWave) + wave) * EL;
  if (e0 >= E) return;  // whole wave
  const int tc = t < T ? t : T - 1;  // clamped row: loads stay in bounds
  const char* xr = reinterpret_cast<const char*>(x) + (size_t)tc * d * esz;
  const char* wr[EL];
#pragma unroll
  for (int j = 0; j < EL; ++j) {
    const int e = e0 + j < E ? e0 + j : E - 1;
    wr[j] = reinterpret_cast<const char*>(w) + (size_t)e * d * esz;
  }
  float acc[EL];
#pragma unroll
  for (int j = 0; j < EL; ++j) acc[j] = 0.0f;
  for (int i = 0; i < d; i += G::N) {
    float xv[G::N];
    G::load(xr + (size_t)i * esz, xv);
#pragma unroll
    for (int j = 0; j < EL; ++j) {
      float wv[G::N];
      G::load(wr[j] + (size_t)i * esz, wv);
#pragma unroll
      for (int q = 0; q < G::N; ++q) acc[j] = __builtin_fmaf(xv[q], wv[q], acc[j]);
    }
  }
  if (t >= T) return;
#pragma unroll
  for (int j = 0; j < EL; ++j) {
    const int e = e0 + j;
    if (e < E) {
      float v = acc[j];
      if (b) v = v + b[e];
      logits[(size_t)t * E + e] = v;
    }
  }
}

// (a, ia) precedes (b, ib) in the selection order: larger logit first, lower
// expert index first among equal logits.
__device__ __forceinline__ bool precedes(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}

__global__ __launch_bounds__(64) void topk_gates_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int renorm,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ gates) {
  extern __shared__ float s_log[];  // [blockDim.x][E+1]
  const int lane = threadIdx.x;
  const int tpb = blockDim.x;  // tokens per block
  const int t0 = blockIdx.x * tpb;
  const int nt = min(tpb, T - t0);
  const int stride = E + 1;
  for (int idx = lane; idx < nt * E; idx += tpb) {
    s_log[(idx / E) * stride + idx % E] = logits[(size_t)t0 * E + idx];
  }
  __syncthreads();
  if (lane >= nt) return;
  const float* row = s_log + lane * stride;
  constexpr int KMAX = 8;
  float bv[KMAX];
  int bi[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    bv[j] = 0.0f;
    bi[j] = 0;
  }
  int filled = 0;
  for (int e = 0; e < E; ++e) {
    float cv = row[e];
    int ci = e;
    // branch-free insertion: the displaced entry moves one slot down
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const bool take = (j < k) & ((j >= filled) | precedes(cv, ci, bv[j], bi[j]));
      const float ov = bv[j];
      const int oi = bi[j];
      bv[j] = take ? cv : ov;
      bi[j] = take ? ci : oi;
      cv = take ? ov : cv;
      ci = take ? oi : ci;
    }
    filled = filled < k ? filled + 1 : k;
  }
  const float m = bv[0];
  float ex[KMAX];
  float denom = 0.0f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    ex[j] = j < k ? expf(bv[j] - m) : 0.0f;
    if (renorm) denom += ex[j];
  }
  if (!renorm) {
    for (int e = 0; e < E; ++e) denom += expf(row[e] - m);
  }
  const int t = t0 + lane;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      ids[(size_t)t * k + j] = bi[j];
      gates[(size_t)t * k + j] = ex[j] / denom;
    }
  }
}

hipError_t launch_route(bool bf16, const void* x, const void* w, const float* b, int T, int d,
                        int E, int k, int renorm, float* logits, int32_t* ids, float* gates,
                        hipStream_t st) {
  if (T == 0) return hipSuccess;
  // experts per lane: enough waves to cover the chip when T*E is small,
  // more register reuse of the token row when it is large
  const long pairs = (long)T * E;
  int EL = 8;
  if (pairs <= 64L * 1024) EL = 1;
  else if (pairs <= 256L * 1024) EL = 4;
  dim3 grid(ceil_div(T, kWave), ceil_div(E, EL * 4));
  dim3 block(256);
#define RL(BF, EL_)                                                                     \
  hipLaunchKernelGGL((router_logits_kernel<BF, EL_>), grid, block, 0, st, x, w, b, T, d, E, \
                     logits)
  if (bf16) {
    if (EL == 1) RL(true, 1);
    else if (EL == 4) RL(true, 4);
    else RL(true, 8);
  } else {
    if (EL == 1) RL(false, 1);
    else if (EL == 4) RL(false, 4);
    else RL(false, 8);
  }
#undef RL
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int tpb = (E + 1) * 64 * (int)sizeof(float) <= 48 * 1024 ? 64 : 32;
  const size_t lds = (size_t)tpb * (E + 1) * sizeof(float);
  hipLaunchKernelGGL(topk_gates_kernel, dim3(ceil_div(T, tpb)), dim3(tpb), lds, st, logits, T, E,
                     k, renorm, ids, gates);
  return hipGetLastError();
}

}  // namespace moe
