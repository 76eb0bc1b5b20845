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
//   router_logits_kernel  one lane per (token, expert) chain: each logit is a
//       sequential fp32 fused multiply-add over the hidden index in
//       increasing order, bias added after the sum.  That fixed order is what
//       makes the logits -- and so the selected expert ids at near ties --
//       bit-reproducible.  Token and expert rows are staged through LDS as
//       fp32 tiles (see the kernel).
//   topk_gates_kernel  one lane per token over an LDS copy of its logits:
//       a single insertion pass keeps the k best by (logit desc, index asc),
//       then the gates.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "topk.h"

namespace moe {

// Calls f(integral_constant<int, I>) for I = B .. E-1 (compile-time unrolled).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Router logits.  Block = 64 tokens x (4 * EPW) experts; lane = token, wave
// w owns experts e0 + w*EPW + j.  The hidden dimension advances in chunks of
// RKC (128 when the chains are few and latency-bound, 64 when many blocks
// share a CU): the block stages the x tile [64][RKC] and the W tile
// [4*EPW][RKC] in LDS as fp32 (converted once per element), then every lane
// runs its EPW fused-multiply-add chains in increasing hidden index, reading
// its own x row and broadcast W rows.  Chunks are prefetched two ahead into
// two register sets while the current one is consumed.
template <bool BF16, int EPW, int RKC>
__global__ __launch_bounds__(256) void router_logits_kernel(
    const void* __restrict__ x, const void* __restrict__ w, const float* __restrict__ b, int T,
    int d, int E, float* __restrict__ logits) {
  constexpr int EB = 4 * EPW;             // experts per block
  constexpr int G = BF16 ? 8 : 4;         // elements per 16-byte chunk
  constexpr int CPR = RKC / G;            // 16-byte chunks per tile row
  constexpr int XPT = 64 * CPR / 256;     // x chunks per thread
  constexpr int WPT = (EB * CPR + 255) / 256;  // W chunks per thread (upper bound)
  constexpr int XS = RKC + 4;             // padded fp32 row (conflict-free b128 reads)
  __shared__ __attribute__((aligned(16))) float sx[64 * XS];
  __shared__ __attribute__((aligned(16))) float sw[EB * RKC];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t0 = blockIdx.x * 64;
  const int e0 = blockIdx.y * EB;
  const char* xb = reinterpret_cast<const char*>(x);
  const char* wb = reinterpret_cast<const char*>(w);
  constexpr int esz = BF16 ? 2 : 4;
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  u32x4_t rx[2][XPT], rw[2][WPT];
  auto fetch = [&](int set, int k0) {
#pragma unroll
    for (int q = 0; q < XPT; ++q) {
      const int c = q * 256 + tid;
      const int row = c / CPR, col = (c % CPR) * G;
      const int t = min(t0 + row, T - 1);
      rx[set][q] = (k0 + col < d)
                       ? *reinterpret_cast<const u32x4_t*>(xb + ((size_t)t * d + k0 + col) * esz)
                       : zero;
    }
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
      const int c = q * 256 + tid;
      const int row = c / CPR, col = (c % CPR) * G;
      const int e = min(e0 + row, E - 1);
      rw[set][q] = (c < EB * CPR && k0 + col < d)
                       ? *reinterpret_cast<const u32x4_t*>(wb + ((size_t)e * d + k0 + col) * esz)
                       : zero;
    }
  };
  auto put = [&](float* dst, const u32x4_t v) {
    if constexpr (BF16) {
      f32x4_t lo = {bf16lo(v[0]), bf16hi(v[0]), bf16lo(v[1]), bf16hi(v[1])};
      f32x4_t hi = {bf16lo(v[2]), bf16hi(v[2]), bf16lo(v[3]), bf16hi(v[3])};
      *reinterpret_cast<f32x4_t*>(dst) = lo;
      *reinterpret_cast<f32x4_t*>(dst + 4) = hi;
    } else {
      *reinterpret_cast<u32x4_t*>(dst) = v;
    }
  };
  auto stage = [&](int set) {
#pragma unroll
    for (int q = 0; q < XPT; ++q) {
      const int c = q * 256 + tid;
      put(sx + (c / CPR) * XS + (c % CPR) * G, rx[set][q]);
    }
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
      const int c = q * 256 + tid;
      if (c < EB * CPR) put(sw + (c / CPR) * RKC + (c % CPR) * G, rw[set][q]);
    }
  };

  float acc[EPW];
#pragma unroll
  for (int j = 0; j < EPW; ++j) acc[j] = 0.0f;
  const float* xr = sx + lane * XS;
  // One k step = 4 hidden indices: this lane's x values and each expert's
  // W values, then 4 FMAs per chain in increasing index.
  struct Step {
    f32x4_t x;
    f32x4_t w[EPW];
  };
  auto read_step = [&](int kk, Step& q) {
    q.x = *reinterpret_cast<const f32x4_t*>(xr + kk);
#pragma unroll
    for (int j = 0; j < EPW; ++j)
      q.w[j] = *reinterpret_cast<const f32x4_t*>(sw + (wave * EPW + j) * RKC + kk);
  };
  auto fma_step = [&](const Step& q) {
#pragma unroll
    for (int j = 0; j < EPW; ++j) {
      acc[j] = __builtin_fmaf(q.x[0], q.w[j][0], acc[j]);
      acc[j] = __builtin_fmaf(q.x[1], q.w[j][1], acc[j]);
      acc[j] = __builtin_fmaf(q.x[2], q.w[j][2], acc[j]);
      acc[j] = __builtin_fmaf(q.x[3], q.w[j][3], acc[j]);
    }
  };
  // A full chunk: the LDS reads run P steps ahead of the FMAs (a ring of P
  // register sets), so their latency hides behind (P-1) steps of FMAs even
  // with one or two waves per SIMD; the schedule keeps each step's FMAs
  // before the refill it allows.
  constexpr int P = EPW == 4 ? 3 : 8 / EPW;
  constexpr int NSTEP = RKC / 4;
  static_assert(P <= NSTEP, "read-ahead within a chunk");
  auto consume_full = [&]() {
    Step q[P];
    static_for<0, P>([&](auto i) { read_step(decltype(i)::value * 4, q[decltype(i)::value]); });
    static_for<0, NSTEP>([&](auto si) {
      constexpr int st = decltype(si)::value;
      fma_step(q[st % P]);
      if constexpr (st + P < NSTEP) {
        read_step((st + P) * 4, q[st % P]);
        __builtin_amdgcn_sched_group_barrier(0x002, 4 * EPW, 0);  // the FMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 1 + EPW, 0);  // then the refill
      }
    });
  };
  auto consume = [&](int k0) {
    const int kc = min(RKC, d - k0);  // a multiple of 8
    if (kc == RKC) {
      consume_full();
    } else {
      for (int kk = 0; kk < kc; kk += 4) {
        Step q;
        read_step(kk, q);
        fma_step(q);
      }
    }
  };
  const int nc = (d + RKC - 1) / RKC;
  fetch(0, 0);
  if (nc > 1) fetch(1, RKC);
  for (int c = 0; c < nc; c += 2) {
    __syncthreads();  // previous chunk fully consumed
    stage(0);
    if (c + 2 < nc) fetch(0, (c + 2) * RKC);
    __syncthreads();
    consume(c * RKC);
    if (c + 1 >= nc) break;
    __syncthreads();
    stage(1);
    if (c + 3 < nc) fetch(1, (c + 3) * RKC);
    __syncthreads();
    consume((c + 1) * RKC);
  }
  const int t = t0 + lane;
  if (t >= T) return;
#pragma unroll
  for (int j = 0; j < EPW; ++j) {
    const int e = e0 + wave * EPW + j;
    if (e < E) {
      float v = acc[j];
      if (b) v = v + b[e];
      logits[(size_t)t * E + e] = v;
    }
  }
}

// KMAX: slots kept by the insertion pass, the smallest power of two >= k
template <int KMAX>
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
  // coalesced staging, eight loads in flight per lane
  const int n = nt * E;
  for (int base = 0; base < n; base += 8 * tpb) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = base + u * tpb + lane;
      v[u] = idx < n ? logits[(size_t)t0 * E + idx] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = base + u * tpb + lane;
      if (idx < n) s_log[(idx / E) * stride + idx % E] = v[u];
    }
  }
  __syncthreads();
  if (lane >= nt) return;
  const float* row = s_log + lane * stride;
  int bi[KMAX];
  float gate[KMAX];
  topk_token<KMAX, 0>([&](int e) { return row[e]; }, E, k, renorm, bi, gate);
  const int t = t0 + lane;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      ids[(size_t)t * k + j] = bi[j];
      gates[(size_t)t * k + j] = gate[j];
    }
  }
}

hipError_t launch_route(bool bf16, const void* x, const void* w, const float* b, int T, int d,
                        int E, int k, int renorm, float* logits, int32_t* ids, float* gates,
                        hipStream_t st) {
  if (T == 0) return hipSuccess;
  // experts per wave: the most register reuse that still leaves about
  // 2048 waves (two per SIMD) of independent chains
  const long waves_at1 = (long)ceil_div(T, kWave) * E;
  int EPW = 1;
  if (waves_at1 >= 8192) EPW = 4;
  else if (waves_at1 >= 4096) EPW = 2;
  dim3 grid(ceil_div(T, kWave), ceil_div(E, 4 * EPW));
  dim3 block(256);
#define RL(BF, EPW_)                                                                            \
  hipLaunchKernelGGL((router_logits_kernel<BF, EPW_, (EPW_ == 4 ? 64 : 128)>), grid, block, 0, st, \
                     x, w, b, T, d, E, logits)
  if (bf16) {
    if (EPW == 1) RL(true, 1);
    else if (EPW == 2) RL(true, 2);
    else RL(true, 4);
  } else {
    if (EPW == 1) RL(false, 1);
    else if (EPW == 2) RL(false, 2);
    else RL(false, 4);
  }
#undef RL
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !ids) return err;  // logits only
  const int tpb = (E + 1) * 64 * (int)sizeof(float) <= 48 * 1024 ? 64 : 32;
  const size_t lds = (size_t)tpb * (E + 1) * sizeof(float);
  const dim3 tg(ceil_div(T, tpb)), tb(tpb);
  if (k <= 1)
    hipLaunchKernelGGL(topk_gates_kernel<1>, tg, tb, lds, st, logits, T, E, k, renorm, ids, gates);
  else if (k <= 2)
    hipLaunchKernelGGL(topk_gates_kernel<2>, tg, tb, lds, st, logits, T, E, k, renorm, ids, gates);
  else if (k <= 4)
    hipLaunchKernelGGL(topk_gates_kernel<4>, tg, tb, lds, st, logits, T, E, k, renorm, ids, gates);
  else
    hipLaunchKernelGGL(topk_gates_kernel<8>, tg, tb, lds, st, logits, T, E, k, renorm, ids, gates);
  return hipGetLastError();
}

}  // namespace moe
