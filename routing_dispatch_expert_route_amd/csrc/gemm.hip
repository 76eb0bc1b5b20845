// gemm.hip -- expert FFN as variable-size grouped GEMMs.
//
// "271,104 Routes", section 3: rows of one expert are packed into a batch so
// the expert runs one dense matmul; "Mixture-of-experts routing": dropless
// variable-size grouped matmuls; "MoE Inference Visualized", "Expert
// Execution": down_proj(SiLU(gate_proj(x)) * up_proj(x)).
//
// GEMM 1:  h[p, :]  = SiLU(A[p] Wg[e]^T) * (A[p] Wu[e]^T)   (SwiGLU epilogue)
// GEMM 2:  y[p, :]  = h[p] Wd[e]^T
// for every packed row p of expert e (rows [offsets[e], offsets[e+1])).
// Both operands are K-contiguous ([rows][K] activations, [N][K] weights), so
// every MFMA fragment is one 16-byte LDS read.
//
// Tile scheduling needs no host readback: the grid is an upper bound on the
// number of (row tile, column tile) pairs; each workgroup finds its expert by
// a wave-wide prefix scan over ceil(m_e / BM) read from the device offsets,
// and workgroups past the last tile exit at once.
//
// GEMM 1 can read its A rows through an index (a_rows[p] = source token), so
// the whole-layer path never materialises the packed copy of x.
#include "common.h"
#include "launch.h"

namespace moe {

struct GemmArgs {
  const void* A;          // [rows][K] activations (packed rows, or tokens via a_rows)
  const int32_t* a_rows;  // optional row index: A row of packed row p is a_rows[p]
  const int32_t* offsets; // [E+1] device offsets, or nullptr: one group of M_dense rows
  int E;
  int M_dense;
  const void* B0;  // gate (SwiGLU) or down weights [E][N][K]
  const void* B1;  // up weights [E][N][K] (SwiGLU only)
  int N;
  int K;
  void* C;            // [rows][N] in dtype, or fp32 partial planes [splits][R_max][N]
  long split_stride;  // elements between partial planes
  int n_tiles;        // column tiles
  int m_tiles;        // row tiles (an upper bound; tiles past the last group exit)
  int splits;         // K splits (partial-plane output when > 1)
  int k_chunk;        // K elements per split, a multiple of 64
  unsigned a_bytes;   // extent of A in bytes (< 2^31; buffer range of the activation loads)
};

// Find the (expert, first row, row count) of row-tile mt.  Executed by one
// wave; the lane that owns the tile writes the result to info[0..2]
// (info[0] stays -1 when mt is past the last tile).
template <int BM>
__device__ __forceinline__ void find_row_tile(const GemmArgs& a, int mt, int lane, int* info) {
  if (a.offsets == nullptr) {
    if (lane == 0) {
      const int r0 = mt * BM;
      if (r0 < a.M_dense) {
        info[0] = 0;
        info[1] = r0;
        info[2] = min(BM, a.M_dense - r0);
      } else {
        info[0] = -1;
      }
    }
    return;
  }
  if (lane == 0) info[0] = -1;
  int carry = 0;
  for (int e0 = 0; e0 < a.E; e0 += kWave) {
    const int e = e0 + lane;
    int m = 0, off = 0;
    if (e < a.E) {
      off = a.offsets[e];
      m = a.offsets[e + 1] - off;
    }
    const int tiles = (m + BM - 1) / BM;
    int incl = tiles;
#pragma unroll
    for (int s = 1; s < kWave; s <<= 1) {
      const int o = __shfl_up(incl, s, kWave);
      if (lane >= s) incl += o;
    }
    const int excl = carry + incl - tiles;
    if (e < a.E && mt >= excl && mt < excl + tiles) {
      const int local = mt - excl;
      info[0] = e;
      info[1] = off + local * BM;
      info[2] = min(BM, m - local * BM);
    }
    carry += __shfl(incl, kWave - 1, kWave);
  }
}

// Block -> (row tile, column tile, K split).  Workgroups are dispatched
// round-robin over the 8 XCDs (each with its own L2), so consecutive logical
// tiles are first gathered per XCD; tiles are then walked in groups of
// GM row tiles, column tile slowest inside a group, so the workgroups that
// run together on one XCD share both their weight and activation tiles.
__device__ __forceinline__ void tile_of_block(const GemmArgs& a, int& mt, int& nt, int& ks) {
  constexpr int NXCD = 8, GM = 8;
  const int nb = gridDim.x, bid = blockIdx.x;
  const int xcd = bid % NXCD, local = bid / NXCD;
  const int per = nb / NXCD, rem = nb % NXCD;
  int l = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + local;
  const int tiles = a.m_tiles * a.n_tiles;
  ks = l / tiles;
  l -= ks * tiles;
  const int group = l / (GM * a.n_tiles);
  const int first = group * GM;
  const int gsize = min(GM, a.m_tiles - first);
  const int within = l - group * GM * a.n_tiles;
  mt = first + within % gsize;
  nt = within / gsize;
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel, 256 threads = WM x WN waves.
//
// Operand roles.  The MFMA A operand is the weight tile (rows n), the B
// operand the activation tile (rows m), so the accumulator holds D[n][m]:
// lane l of a 32x32 tile owns column m = l%32 and rows n = 8*(v/4) +
// 4*(l/32) + v%4 -- four consecutive output columns of one token row per
// group of four accumulator registers, written as one 8-byte store.
//
// Pipeline.  K advances in stages of BK = 32 through a ring of four LDS
// stages filled by direct buffer->LDS loads (buffer_load_dwordx4 ... lds:
// each wave-level load writes 1 KB = 16 rows of 64 bytes; no staging
// registers; the K position is the scalar offset, so a lane's vector
// offset never changes).  Three stages are in flight while one feeds the
// MFMAs; a stage costs one s_waitcnt on the wave's own loads and one
// workgroup barrier.  Each ring slot is its own LDS object and every access
// names its slot statically (switch on kt % 4), so the compiler can tell a
// load into one slot from a read of another and inserts no extra waits.
//
// LDS layout.  A row holds 4 chunks of 16 bytes; logical chunk c of row r
// sits at c ^ f(r), f(r) = ((r >> 1) ^ (r >> 3)) & 3: the 8 or 16 lanes that
// read one chunk column of consecutive rows visit distinct bank groups
// whether the LDS has 32 or 64 four-byte banks.
//
// K tail (K not a multiple of 32): a chunk past the end gets a vector
// offset beyond the buffer, which the buffer unit returns as zero.
//
// SWIGLU: the weight tile stacks BNW/2 gate rows over the matching BNW/2 up
// rows; the epilogue writes SiLU(gate) * up.  PARTIAL: fp32 output into the
// K split's partial plane (summed later in a fixed order).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;
constexpr int kBufFlags = 0x00020000;  // raw buffer, 32-bit data format

template <int BM, int BNW, int WM, int WN, bool SWIGLU, bool GATHER, bool PARTIAL>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only emits the launch stub
  constexpr int BK = 32;
  constexpr int CH = BK / 8;       // 16-byte chunks per row
  constexpr int RPS = 64 / CH;     // rows per 1 KB wave-level load
  constexpr int NS = 4;            // ring slots
  constexpr int NREG = SWIGLU ? 2 : 1;
  constexpr int BNO = BNW / NREG;  // output columns per block
  constexpr int WTM = BM / WM, WTN = BNO / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int XS = BM / RPS / 4;   // activation loads per wave per stage
  constexpr int WS = BNW / RPS / 4;  // weight loads per wave per stage
  constexpr int PER = XS + WS;
  constexpr int STAGE = (BM + BNW) * CH;  // 16-byte units per stage
  static_assert(WM * WN == 4, "four waves");
  static_assert(TM >= 1 && TN >= 1 && XS >= 1 && WS >= 1, "tile shape");
  static_assert(!(SWIGLU && PARTIAL), "SwiGLU needs the full K sum");
  static_assert(PER * (NS - 1) < 64, "vmcnt range");

  __shared__ __attribute__((aligned(1024))) u32x4_t st0[STAGE];
  __shared__ __attribute__((aligned(1024))) u32x4_t st1[STAGE];
  __shared__ __attribute__((aligned(1024))) u32x4_t st2[STAGE];
  __shared__ __attribute__((aligned(1024))) u32x4_t st3[STAGE];
  __shared__ int s_info[3];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform values the compiler cannot prove uniform on its own (the
  // wave index, and the tile found by wave 0 and read back from LDS): they
  // feed buffer descriptors and LDS load destinations, which must be scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  int mt, nt, ks;
  tile_of_block(a, mt, nt, ks);

  if (wave == 0) find_row_tile<BM>(a, mt, lane, s_info);
  __syncthreads();
  const int e = __builtin_amdgcn_readfirstlane(s_info[0]);
  if (e < 0) return;
  const int row0 = __builtin_amdgcn_readfirstlane(s_info[1]);
  const int rows = __builtin_amdgcn_readfirstlane(s_info[2]);
  const int K = a.K, N = a.N;
  const int kb = ks * a.k_chunk;
  const int klen = min(K, kb + a.k_chunk) - kb;

  // Buffer resources: activations, and the expert's gate/up or down rows.
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.A), (short)0, (int)a.a_bytes, kBufFlags);
  __amdgpu_buffer_rsrc_t rw[NREG];
  const size_t wexp = (size_t)e * N * K * 2;
  rw[0] = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(reinterpret_cast<const char*>(a.B0) + wexp), (short)0, N * K * 2,
      kBufFlags);
  if constexpr (SWIGLU)
    rw[NREG - 1] = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(reinterpret_cast<const char*>(a.B1) + wexp), (short)0, N * K * 2,
        kBufFlags);

  // Lane i of wave-level load q writes row seg*RPS + i/CH (seg = wave*XS+q
  // for activations) at physical chunk i%CH, so it fetches logical chunk
  // (i%CH) ^ f(row).  Byte offsets, fixed for the whole K loop.
  unsigned xo[XS];
  int xc[XS];
#pragma unroll
  for (int q = 0; q < XS; ++q) {
    const int r = (wave * XS + q) * RPS + lane / CH;
    xc[q] = (lane % CH) ^ swz(r);
    const int p = row0 + (r < rows ? r : rows - 1);
    const int src = GATHER ? a.a_rows[p] : p;
    xo[q] = ((unsigned)src * (unsigned)K + (unsigned)(kb + xc[q] * 8)) * 2u;
  }
  unsigned wo[WS];
  int wc[WS];
#pragma unroll
  for (int q = 0; q < WS; ++q) {
    const int r = (wave * WS + q) * RPS + lane / CH;
    wc[q] = (lane % CH) ^ swz(r);
    int n = nt * BNO + (r % BNO);
    n = n < N ? n : N - 1;
    wo[q] = ((unsigned)n * (unsigned)K + (unsigned)(kb + wc[q] * 8)) * 2u;
  }

  // stage layout: BM activation rows, then BNW weight rows
  auto issue = [&](u32x4_t* stg, int kt) {
    const int k0 = kt * BK;
    const int soff = k0 * 2;
    const bool tail = k0 + BK > klen;  // includes padding stages past K
#pragma unroll
    for (int q = 0; q < XS; ++q) {
      // past-K chunk: an offset past every buffer extent reads zero
      const unsigned vo = (tail && xc[q] * 8 >= klen - k0) ? 0x80000000u : xo[q];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)(stg + (wave * XS + q) * 64), 16, vo,
                                               soff, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < WS; ++q) {
      const int reg = ((wave * WS + q) * RPS) / BNO;
      const unsigned vo = (tail && wc[q] * 8 >= klen - k0) ? 0x80000000u : wo[q];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw[reg],
                                               (lds_ptr_t)(stg + BM * CH + (wave * WS + q) * 64),
                                               16, vo, soff, 0, 0);
    }
  };

  f32x16_t acc[NREG][TN][TM];
#pragma unroll
  for (int g = 0; g < NREG; ++g)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[g][j][i][v] = 0.0f;

  // Fragment byte offsets inside a stage.  Row bases are multiples of 32,
  // so the swizzle of a fragment row depends on the lane's row (lane % 32)
  // only: one offset per (operand, 16-wide k step) covers every fragment,
  // the rest is a compile-time displacement.
  const int lrow = lane & 31;
  const int lk = lane >> 5;
  int xoff[2], woff[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int chunk = ((kk * 2 + lk) ^ swz(lrow)) * 16;
    xoff[kk] = (wm * WTM + lrow) * CH * 16 + chunk;
    woff[kk] = BM * CH * 16 + (wn * WTN + lrow) * CH * 16 + chunk;
  }
  auto compute = [&](const u32x4_t* stg) {
    // opaque copies: keeps the compiler from hoisting one set of addresses
    // per ring slot out of the loop (which would not fit in registers)
    int xo0 = xoff[0], xo1 = xoff[1], wo0 = woff[0], wo1 = woff[1];
    asm volatile("" : "+v"(xo0), "+v"(xo1), "+v"(wo0), "+v"(wo1));
    const char* base = reinterpret_cast<const char*>(stg);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int xo = kk ? xo1 : xo0;
      const int wo = kk ? wo1 : wo0;
      bf16x8_t bx[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        bx[i] = *reinterpret_cast<const bf16x8_t*>(base + xo + i * 32 * CH * 16);
#pragma unroll
      for (int g = 0; g < NREG; ++g) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const bf16x8_t aw =
              *reinterpret_cast<const bf16x8_t*>(base + wo + (g * BNO + j * 32) * CH * 16);
#pragma unroll
          for (int i = 0; i < TM; ++i)
            acc[g][j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, bx[i], acc[g][j][i], 0, 0, 0);
        }
      }
    }
  };

  // Stage count padded to a multiple of the ring size; stages past K (the
  // padding, and the refills issued during the last three stages) read
  // zeros -- every chunk offset is past the buffer -- so the loop body is
  // four straight-line steps and every refill is unconditional.  (A
  // conditional refill makes the compiler wait for all loads in flight
  // before the next LDS read, which would serialise the ring.)
  const int nk = ((klen + BK - 1) / BK + NS - 1) / NS * NS;
  constexpr int WAIT = 0x0F70 | ((2 * PER) & 15) | (((2 * PER) >> 4) << 14);  // vmcnt(2*PER)
  // stage kt: wait until only this wave's loads of stages kt+1, kt+2 are in
  // flight, barrier, refill the slot stage kt-1 used with stage kt+3, compute
  auto step = [&](u32x4_t* cur, u32x4_t* refill, int kt) {
    __builtin_amdgcn_s_waitcnt(WAIT);
    __builtin_amdgcn_s_barrier();
    issue(refill, kt + NS - 1);
    compute(cur);
  };
  issue(st0, 0);
  issue(st1, 1);
  issue(st2, 2);
  for (int kt = 0; kt < nk; kt += NS) {
    step(st0, st3, kt);
    step(st1, st0, kt + 1);
    step(st2, st1, kt + 2);
    step(st3, st2, kt + 3);
  }
  // the zero-reading refills past the end must land before the workgroup's
  // LDS is released
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // epilogue: four consecutive columns per store
#pragma unroll
  for (int j = 0; j < TN; ++j) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = wm * WTM + i * 32 + lrow;
      if (m >= rows) continue;
      const size_t p = (size_t)(row0 + m);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = nt * BNO + wn * WTN + j * 32 + 8 * q + 4 * lk;
        if (n >= N) continue;
        float o[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if constexpr (SWIGLU) {
            const float gv = acc[0][j][i][4 * q + t];
            const float uv = acc[1][j][i][4 * q + t];
            o[t] = __fdividef(gv, 1.0f + __expf(-gv)) * uv;
          } else {
            o[t] = acc[0][j][i][4 * q + t];
          }
        }
        if constexpr (PARTIAL) {
          float* Cp = reinterpret_cast<float*>(a.C) + (size_t)ks * a.split_stride;
          f32x4_t v = {o[0], o[1], o[2], o[3]};
          *reinterpret_cast<f32x4_t*>(Cp + p * N + n) = v;
        } else {
          bf16_t* Cp = reinterpret_cast<bf16_t*>(a.C);
          uint2 v;
          v.x = pack_bf16x2(o[0], o[1]);
          v.y = pack_bf16x2(o[2], o[3]);
          *reinterpret_cast<uint2*>(Cp + p * N + n) = v;
        }
      }
    }
  }
#endif
}

// ---------------------------------------------------------------------------
// fp32 kernel (plain fp32 FMA, one output element per thread, K ascending).
// Serves the fp32 dtype, whose shapes here are small.
// ---------------------------------------------------------------------------
template <bool SWIGLU, bool GATHER>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  constexpr int BM = 16, BNO = 16;
  __shared__ int s_info[3];
  const int tid = threadIdx.x;
  const int mt = blockIdx.x / a.n_tiles;
  const int nt = blockIdx.x % a.n_tiles;
  if (tid < 64) find_row_tile<BM>(a, mt, tid, s_info);
  __syncthreads();
  const int e = s_info[0];
  if (e < 0) return;
  const int row0 = s_info[1], rows = s_info[2];
  const int r = tid / BNO, c = tid % BNO;
  const int col = nt * BNO + c;
  if (r >= rows || col >= a.N) return;
  const int p = row0 + r;
  const int src = GATHER ? a.a_rows[p] : p;
  const float* Ar = reinterpret_cast<const float*>(a.A) + (size_t)src * a.K;
  const float* B0 = reinterpret_cast<const float*>(a.B0) + ((size_t)e * a.N + col) * a.K;
  float s0 = 0.0f, s1 = 0.0f;
  if constexpr (SWIGLU) {
    const float* B1 = reinterpret_cast<const float*>(a.B1) + ((size_t)e * a.N + col) * a.K;
    for (int kk = 0; kk < a.K; ++kk) {
      s0 = __builtin_fmaf(Ar[kk], B0[kk], s0);
      s1 = __builtin_fmaf(Ar[kk], B1[kk], s1);
    }
    s0 = s0 / (1.0f + expf(-s0)) * s1;
  } else {
    for (int kk = 0; kk < a.K; ++kk) s0 = __builtin_fmaf(Ar[kk], B0[kk], s0);
  }
  reinterpret_cast<float*>(a.C)[(size_t)p * a.N + col] = s0;
}

// Upper bound on the number of row tiles of size BM over all groups.
static long row_tile_bound(const GemmPlan& pl, int BM) {
  if (!pl.grouped) return (pl.M_dense + BM - 1) / BM;
  const long by_rows = (pl.R_max + (long)pl.E * (BM - 1)) / BM;
  const long by_cap = (long)pl.E * ((pl.m_cap + BM - 1) / BM);
  return by_rows < by_cap ? by_rows : by_cap;
}

// Tile shape: the largest row tile that still gives every CU work.  Tile
// counts are estimated from the row bound (each group wastes half a tile on
// average): 256-row tiles (128x128 per wave) when there are at least two
// per CU, else 128-row tiles when there is at least one, else 64.
enum TileCfg { TILE_L, TILE_M, TILE_S };
static long est_tiles(const GemmPlan& pl, int bm, int bno, int N) {
  const long mt = pl.grouped ? pl.R_max / bm + (pl.E + 1) / 2 : (pl.M_dense + bm - 1) / bm;
  return mt * ((N + bno - 1) / bno);
}
static TileCfg tile_cfg(const GemmPlan& pl, int N, bool swiglu) {
  const int bno = swiglu ? 128 : 256;
  if (est_tiles(pl, 256, bno, N) >= 512) return TILE_L;
  if (est_tiles(pl, 128, bno, N) >= 256) return TILE_M;
  return TILE_S;
}
static int cfg_bm(TileCfg c) { return c == TILE_L ? 256 : c == TILE_M ? 128 : 64; }

template <int BM, int BNW, int WM, int WN, bool SWIGLU, bool PARTIAL>
static hipError_t run_bf16(const GemmPlan& pl, GemmArgs a, hipStream_t st) {
  constexpr int BNO = SWIGLU ? BNW / 2 : BNW;
  a.n_tiles = (a.N + BNO - 1) / BNO;
  a.m_tiles = (int)row_tile_bound(pl, BM);
  const long blocks = (long)a.m_tiles * a.n_tiles * a.splits;
  if (blocks == 0) return hipSuccess;
  if (a.a_rows)
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BNW, WM, WN, SWIGLU, true, PARTIAL>),
                       dim3((unsigned)blocks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BNW, WM, WN, SWIGLU, false, PARTIAL>),
                       dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <bool SWIGLU, bool PARTIAL>
static hipError_t run_cfg(const GemmPlan& pl, GemmArgs a, hipStream_t st) {
  switch (tile_cfg(pl, a.N, SWIGLU)) {
    case TILE_L: return run_bf16<256, 256, 2, 2, SWIGLU, PARTIAL>(pl, a, st);
    case TILE_M: return run_bf16<128, 256, 2, 2, SWIGLU, PARTIAL>(pl, a, st);
    default: return run_bf16<64, 256, 1, 4, SWIGLU, PARTIAL>(pl, a, st);
  }
}

template <bool SWIGLU>
static hipError_t run_f32(const GemmPlan& pl, GemmArgs a, hipStream_t st) {
  a.n_tiles = (a.N + 15) / 16;
  const long blocks = row_tile_bound(pl, 16) * a.n_tiles;
  if (blocks == 0) return hipSuccess;
  if (a.a_rows)
    hipLaunchKernelGGL((gemm_f32_kernel<SWIGLU, true>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_f32_kernel<SWIGLU, false>), dim3((unsigned)blocks), dim3(256), 0, st,
                       a);
  return hipGetLastError();
}

int gemm_down_splits(const GemmPlan& pl, int N, int K) {
  if (!pl.bf16) return 1;
  const TileCfg c = tile_cfg(pl, N, false);
  const int bm = cfg_bm(c);
  const long mt = pl.grouped ? (pl.R_max + bm - 1) / bm + (pl.E + 1) / 2
                             : (pl.M_dense + bm - 1) / bm;
  const long blocks = mt * ((N + 255) / 256);
  const long want = 512;  // two workgroups per CU
  if (blocks == 0 || blocks >= want || K < 512) return 1;
  long s = (want + blocks - 1) / blocks;
  if (s > 8) s = 8;
  if (s > K / 256) s = K / 256;
  if (s < 1) s = 1;
  const int chunk = (int)(((K + s - 1) / s + 63) / 64 * 64);
  return (K + chunk - 1) / chunk;
}

hipError_t launch_gemm_swiglu(const GemmPlan& pl, const void* A, const int32_t* a_rows,
                              long a_nrows, const void* Wg, const void* Wu, int N, int K, void* H,
                              hipStream_t st) {
  GemmArgs a{A, a_rows, pl.offsets, pl.E, pl.M_dense, Wg, Wu, N, K, H, 0, 0, 0, 1, K,
             (unsigned)(a_nrows * K * 2)};
  if (!pl.bf16) return run_f32<true>(pl, a, st);
  return run_cfg<true, false>(pl, a, st);
}

hipError_t launch_gemm_down(const GemmPlan& pl, const void* H, const void* Wd, int N, int K,
                            void* Y, int splits, long split_stride, hipStream_t st) {
  const long h_rows = pl.grouped ? pl.R_max : pl.M_dense;
  GemmArgs a{H, nullptr, pl.offsets, pl.E, pl.M_dense, Wd, nullptr, N, K, Y, split_stride, 0, 0,
             1, K, (unsigned)(h_rows * K * 2)};
  if (!pl.bf16) return run_f32<false>(pl, a, st);
  if (splits <= 1) return run_cfg<false, false>(pl, a, st);
  a.splits = splits;
  a.k_chunk = (K + splits - 1) / splits;
  a.k_chunk = (a.k_chunk + 63) / 64 * 64;
  return run_cfg<false, true>(pl, a, st);
}

}  // namespace moe
