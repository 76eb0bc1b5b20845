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
#include <type_traits>

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
  int m_tiles;        // row tiles (an upper bound, host side; the kernel counts the real ones)
  int splits;         // K splits (partial-plane output when > 1)
  int k_chunk;        // K elements per split, a multiple of 64
  unsigned a_bytes;   // extent of A in bytes (< 2^31; buffer range of the activation loads)
  // Combine fused into the down projection (one route per token, no shared
  // expert; y_tok != nullptr): output row p is token y_tok[p]'s, scaled by
  // its gate y_gate[token] and written to row y_tok[p] of C ([T][N]) -- the
  // rounding of the separate combine kept: the row is rounded to bf16 first,
  // then gate * value (an FMA onto +0) is rounded again.  Workgroups from
  // main_blocks on write the zero rows of the tokens whose route was dropped
  // (y_pos[t] < 0).
  const int32_t* y_tok;
  const float* y_gate;
  const int32_t* y_pos;
  int y_T;
  int main_blocks;
};

// Tokens per zero-row workgroup of the fused combine.
constexpr int kZeroTok = 16;

// The zero rows of workgroup z of the fused combine: tokens [z*kZeroTok,
// (z+1)*kZeroTok) whose route was dropped, 16 bytes per thread and store.
__device__ __forceinline__ void zero_dropped_rows(const GemmArgs& a, int z) {
  const int cpr = a.N / 8;  // 16-byte chunks per row (N % 8 == 0)
  const int t0 = z * kZeroTok;
  const int nt = min(kZeroTok, a.y_T - t0);
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  for (int i = threadIdx.x; i < nt * cpr; i += blockDim.x) {
    const int t = t0 + i / cpr;
    if (a.y_pos[t] < 0)
      *reinterpret_cast<u32x4_t*>(reinterpret_cast<bf16_t*>(a.C) + (size_t)t * a.N +
                                  (size_t)(i % cpr) * 8) = zero;
  }
}

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

// Row tiles of size BM over all groups, from the device offsets (every lane
// of the calling wave gets the total).
template <int BM>
__device__ __forceinline__ int count_row_tiles(const GemmArgs& a, int lane) {
  if (a.offsets == nullptr) return (a.M_dense + BM - 1) / BM;
  int total = 0;
  for (int e0 = 0; e0 < a.E; e0 += kWave) {
    const int e = e0 + lane;
    int t = 0;
    if (e < a.E) t = (a.offsets[e + 1] - a.offsets[e] + BM - 1) / BM;
#pragma unroll
    for (int s = kWave / 2; s >= 1; s >>= 1) t += __shfl_xor(t, s, kWave);
    total += t;
  }
  return total;
}

// Block -> (row tile, column tile, K split) over the tiles that exist.  The
// grid is an upper bound (a multiple of 8) on the tile count; the real count
// comes from the device offsets.  Workgroups are dispatched round-robin over
// the 8 XCDs (each with its own L2), so XCD x takes the x-th contiguous
// eighth of the real tiles -- the work is spread evenly whatever the routing
// -- and blocks past its share exit.  Inside a share, tiles are walked in
// groups of GM row tiles, column tile slowest inside a group, so the
// workgroups that run together on one XCD share their weight and activation
// tiles.  Returns false for a block with no tile.
__device__ __forceinline__ bool tile_of_block(const GemmArgs& a, int m_real, int& mt, int& nt,
                                              int& ks) {
  constexpr int NXCD = 8, GM = 8;
  const int bid = blockIdx.x;
  const int xcd = bid % NXCD, local = bid / NXCD;
  const int tiles = m_real * a.n_tiles;
  const int n_real = tiles * a.splits;
  const int chunk = (n_real + NXCD - 1) / NXCD;
  if (local >= chunk) return false;
  int l = xcd * chunk + local;
  if (l >= n_real) return false;
  ks = l / tiles;
  l -= ks * tiles;
  const int group = l / (GM * a.n_tiles);
  const int first = group * GM;
  const int gsize = min(GM, m_real - first);
  const int within = l - group * GM * a.n_tiles;
  mt = first + within % gsize;
  nt = within / gsize;
  return true;
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel, WM x WN waves (four or eight).
//
// Operand roles.  The MFMA A operand is the weight tile (rows n), the B
// operand the activation tile (rows m), so the accumulator holds D[n][m]:
// lane l of a 32x32 tile owns column m = l%32 and rows n = 8*(v/4) +
// 4*(l/32) + v%4 -- four consecutive output columns of one token row per
// group of four accumulator registers, written as one 8-byte store.
//
// Pipeline.  K advances in stages of BK (32 or 64) through two LDS rings,
// NSX slots for the activation tile and NSW >= NSX for the weight tile
// (the weights, first touched in HBM, are fetched further ahead), filled by
// direct buffer->LDS loads (buffer_load_dwordx4 ... lds: each wave-level load
// writes 1 KB; no staging registers; the K position is the scalar offset, so
// a lane's vector offset never changes).  A stage costs one counted
// s_waitcnt on the wave's own loads and one workgroup barrier.  Each ring
// slot is its own LDS object and the loop body is unrolled over every
// combination of slots, so every access names its slot statically and the
// compiler inserts no extra waits.  MFMA fragments are double-buffered in
// registers and the schedule interleaves LDS reads, MFMAs and refills.
//
// LDS layout.  Logical 16-byte chunk c of row r sits at c ^ f(r) (swz<CH>),
// so the lanes that read one chunk column of consecutive rows visit
// distinct bank groups.
//
// K tail (K not a multiple of BK): a chunk past the end gets a vector
// offset beyond the buffer, which the buffer unit returns as zero.
//
// SWIGLU: the weight tile stacks BNW/2 gate rows over the matching BNW/2 up
// rows; the epilogue writes SiLU(gate) * up.  PARTIAL: fp32 output into the
// K split's partial plane (summed later in a fixed order).
// ---------------------------------------------------------------------------
// CH = 4 (64-byte rows): f(r) = (r ^ (r >> 2)) & 3, measured free of bank
// conflicts for the fragment reads below (the variant ((r >> 1) ^ (r >> 3))
// & 3 costs one conflict cycle per access cycle on gfx950).
// CH = 8 (128-byte rows): a 3-bit f that is a bijection on the low three
// row bits for any aligned 8 rows and on bits 1..3 for each row parity in
// any aligned 16 rows (also measured conflict-free).
template <int CH>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CH == 4) return (r ^ (r >> 2)) & 3;
  return ((((r >> 2) ^ (r >> 3)) & 1) << 2) | (r & 2) | ((r ^ (r >> 3)) & 1);
}

// Calls f(integral_constant<int, I>) for I = B .. E-1 (compile-time unrolled).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// LDS ring slot TAG of SIZE 16-byte units: one distinct LDS object per
// (TAG, SIZE), allocated in the kernels that use it.
template <int TAG, int SIZE>
__device__ __forceinline__ u32x4_t* lds_slot() {
  __shared__ __attribute__((aligned(1024))) u32x4_t buf[SIZE];
  return buf;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
constexpr int kBufFlags = 0x00020000;  // raw buffer, 32-bit data format

template <int BM, int BNW, int WM, int WN, int BK, int NSX, int NSW, int OCC, bool SWIGLU,
          bool GATHER, bool PARTIAL>
__global__ __launch_bounds__(64 * WM * WN, OCC) void gemm_bf16_kernel(GemmArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only emits the launch stub
  // BK: K elements per stage (32 or 64); NSX / NSW: ring slots of the
  // activation / weight tiles (2 to 4 each, NSW >= NSX: the weights, first
  // touched in HBM, may be fetched further ahead); OCC: waves per SIMD the
  // register budget must allow (2 = two workgroups per CU)
  constexpr int CH = BK / 8;       // 16-byte chunks per row
  constexpr int RPS = 64 / CH;     // rows per 1 KB wave-level load
  constexpr int NREG = SWIGLU ? 2 : 1;
  constexpr int BNO = BNW / NREG;  // output columns per block
  constexpr int WTM = BM / WM, WTN = BNO / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int NWV = WM * WN;          // waves per workgroup
  constexpr int XS = BM / RPS / NWV;   // activation loads per wave per stage
  constexpr int WS = BNW / RPS / NWV;  // weight loads per wave per stage
  constexpr int PER = XS + WS;
  constexpr int XSTAGE = BM * CH;   // 16-byte units per activation stage
  constexpr int WSTAGE = BNW * CH;  // 16-byte units per weight stage
  static_assert(NWV == 4 || NWV == 8, "four or eight waves");
  static_assert(TM >= 1 && TN >= 1 && XS >= 1 && WS >= 1, "tile shape");
  static_assert(!(SWIGLU && PARTIAL), "SwiGLU needs the full K sum");
  static_assert(XS * (NSX - 1) + WS * (NSW - 1) < 64, "vmcnt range");
  static_assert((BK == 32 || BK == 64) && NSX >= 2 && NSX <= NSW && NSW <= 4, "pipeline shape");

  // every ring slot is its own LDS object (only the slots in use exist), so
  // the compiler can tell a load into one slot from a read of another
  u32x4_t* const X0 = lds_slot<0, XSTAGE>();
  u32x4_t* const W0 = lds_slot<4, WSTAGE>();
  // the tile found by wave 0 is passed through the first ring slot, before
  // any load into it (a barrier separates the reads from the first refill)
  int* s_info = reinterpret_cast<int*>(X0);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform values the compiler cannot prove uniform on its own (the
  // wave index, and the tile found by wave 0 and read back from LDS): they
  // feed buffer descriptors and LDS load destinations, which must be scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  if constexpr (!SWIGLU && !PARTIAL) {
    if (a.y_tok && (int)blockIdx.x >= a.main_blocks) {  // whole workgroup, before any barrier
      zero_dropped_rows(a, (int)blockIdx.x - a.main_blocks);
      return;
    }
  }
  if (wave == 0) {
    int mt0 = 0, nt0 = 0, ks0 = 0;
    if (tile_of_block(a, count_row_tiles<BM>(a, lane), mt0, nt0, ks0)) {
      find_row_tile<BM>(a, mt0, lane, s_info);
      if (lane == 0) {
        s_info[3] = nt0;
        s_info[4] = ks0;
      }
    } else if (lane == 0) {
      s_info[0] = -1;
    }
  }
  __syncthreads();
  const int e = __builtin_amdgcn_readfirstlane(s_info[0]);
  if (e < 0) return;
  const int row0 = __builtin_amdgcn_readfirstlane(s_info[1]);
  const int rows = __builtin_amdgcn_readfirstlane(s_info[2]);
  const int nt = __builtin_amdgcn_readfirstlane(s_info[3]);
  const int ks = __builtin_amdgcn_readfirstlane(s_info[4]);
  __syncthreads();  // every wave has its tile before X0 is refilled
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
    xc[q] = (lane % CH) ^ swz<CH>(r);
    const int p = row0 + (r < rows ? r : rows - 1);
    const int src = GATHER ? a.a_rows[p] : p;
    xo[q] = ((unsigned)src * (unsigned)K + (unsigned)(kb + xc[q] * 8)) * 2u;
  }
  unsigned wo[WS];
  int wc[WS];
#pragma unroll
  for (int q = 0; q < WS; ++q) {
    const int r = (wave * WS + q) * RPS + lane / CH;
    wc[q] = (lane % CH) ^ swz<CH>(r);
    int n = nt * BNO + (r % BNO);
    n = n < N ? n : N - 1;
    wo[q] = ((unsigned)n * (unsigned)K + (unsigned)(kb + wc[q] * 8)) * 2u;
  }

  // one stage of the activation tile (BM rows) / of the weight tile (BNW rows)
  auto issue_x = [&](u32x4_t* xs, int kt) {
    const int k0 = kt * BK;
    const int soff = k0 * 2;
    const bool tail = k0 + BK > klen;  // includes padding stages past K
#pragma unroll
    for (int q = 0; q < XS; ++q) {
      // past-K chunk: an offset past every buffer extent reads zero
      const unsigned vo = (tail && xc[q] * 8 >= klen - k0) ? 0x80000000u : xo[q];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)(xs + (wave * XS + q) * 64), 16, vo,
                                               soff, 0, 0);
    }
  };
  auto issue_w = [&](u32x4_t* wsl, int kt) {
    const int k0 = kt * BK;
    const int soff = k0 * 2;
    const bool tail = k0 + BK > klen;
#pragma unroll
    for (int q = 0; q < WS; ++q) {
      const int reg = ((wave * WS + q) * RPS) / BNO;
      const unsigned vo = (tail && wc[q] * 8 >= klen - k0) ? 0x80000000u : wo[q];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw[reg], (lds_ptr_t)(wsl + (wave * WS + q) * 64), 16,
                                               vo, soff, 0, 0);
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
  constexpr int KS = BK / 16;  // 16-wide MFMA k steps per stage
  int xoff[KS], woff[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    const int chunk = ((kk * 2 + lk) ^ swz<CH>(lrow)) * 16;
    xoff[kk] = (wm * WTM + lrow) * CH * 16 + chunk;
    woff[kk] = (wn * WTN + lrow) * CH * 16 + chunk;
  }
  // Fragments of one 16-wide k step, double-buffered in registers: the
  // reads of step kk+1 are issued before the MFMAs of step kk, so the LDS
  // latency hides behind them.
  struct Frag {
    bf16x8_t bx[TM];
    bf16x8_t aw[NREG][TN];
  };
  auto read_frags = [&](const u32x4_t* xs, const u32x4_t* wsl, int kk, Frag& F) {
    // opaque copies: keeps the compiler from hoisting one set of addresses
    // per (ring slot, k step) out of the loop (which would not fit in
    // registers)
    int xo = xoff[kk], wo = woff[kk];
    asm volatile("" : "+v"(xo), "+v"(wo));
    const char* xb = reinterpret_cast<const char*>(xs);
    const char* wb = reinterpret_cast<const char*>(wsl);
#pragma unroll
    for (int i = 0; i < TM; ++i)
      F.bx[i] = *reinterpret_cast<const bf16x8_t*>(xb + xo + i * 32 * CH * 16);
#pragma unroll
    for (int g = 0; g < NREG; ++g)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        F.aw[g][j] = *reinterpret_cast<const bf16x8_t*>(wb + wo + (g * BNO + j * 32) * CH * 16);
  };
  auto mma = [&](const Frag& F) {
#pragma unroll
    for (int g = 0; g < NREG; ++g)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i)
          acc[g][j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.aw[g][j], F.bx[i], acc[g][j][i], 0, 0, 0);
  };

  // Stage count padded to a whole number of loop bodies (every combination
  // of the two rings' slots); stages past K (the padding, and the refills
  // issued during the last stages) read zeros -- every chunk offset is past
  // the buffer -- so the loop body is straight line and every refill is
  // unconditional.  (A conditional refill makes the compiler wait for all
  // loads in flight before the next LDS read, which would serialise the
  // ring.)
  constexpr int LB = NSX * NSW / (NSX == NSW ? NSX : (NSW % NSX == 0 ? NSX : 1));  // lcm
  const int nk = ((klen + BK - 1) / BK + LB - 1) / LB * LB;
  // The transition into stage t+1 (at the end of stage t) refills the
  // slots of stage t with x(t+NSX) and w(t+NSW), in that order.  Entering
  // it, x(t+1) and w(t+1) must have landed: the loads issued after x(t+1)
  // are w(t+NSX-1+...) of the same transition (when the weight ring is
  // deeper) and the NSX-2 transitions since.  Then its LDS reads must have
  // returned and every wave must be past the barrier (every wave's loads of
  // stage t+1 have landed, and every wave has read all it needs of stage t).
  constexpr int VM = (NSW > NSX ? WS : 0) + (NSX - 2) * PER;
  constexpr int WAIT = 0x0070 | (VM & 15) | ((VM >> 4) << 14);   // vmcnt(VM) lgkmcnt(0)
  constexpr int WAIT0 = 0x0F70 | (VM & 15) | ((VM >> 4) << 14);  // vmcnt(VM)
  auto xslot = [&](auto i) -> u32x4_t* {
    return lds_slot<decltype(i)::value % NSX, XSTAGE>();
  };
  auto wslot = [&](auto i) -> u32x4_t* {
    return lds_slot<4 + decltype(i)::value % NSW, WSTAGE>();
  };
  Frag F0, F1;
  // Instruction order (the scheduler otherwise sinks each LDS read to its
  // first use, which exposes the LDS latency on every k step): one LDS
  // read of the next step per MFMA of the current one, and after a barrier
  // one refill load per MFMA as well.
  constexpr int NDS = TM + NREG * TN;  // LDS reads per k step
  constexpr int NMF = NREG * TN * TM;  // MFMAs per k step
  auto order_kstep = [&]() {
#pragma unroll
    for (int u = 0; u < NMF; ++u) {
      if (u < NDS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // MFMA
    }
  };
  auto order_transition = [&]() {
#pragma unroll
    for (int u = 0; u < (NMF > PER ? NMF : PER); ++u) {
      if (u < PER) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
      if (u < NDS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      if (u < NMF) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    }
  };
  // Stage S of the loop body (kt = its stage index): k steps 0 .. KS-2 read
  // the next step's fragments first; the last step moves to the next stage
  // before its MFMAs, which only need registers.
  auto stage = [&](auto S, int kt) {
    constexpr int s = decltype(S)::value;
    u32x4_t* xc_ = xslot(std::integral_constant<int, s>{});
    u32x4_t* wc_ = wslot(std::integral_constant<int, s>{});
#pragma unroll
    for (int kk = 0; kk < KS - 1; ++kk) {
      if (kk % 2 == 0) {
        read_frags(xc_, wc_, kk + 1, F1);
        mma(F0);
      } else {
        read_frags(xc_, wc_, kk + 1, F0);
        mma(F1);
      }
      order_kstep();
    }
    __builtin_amdgcn_s_waitcnt(WAIT);
    __builtin_amdgcn_s_barrier();
    issue_x(xc_, kt + NSX);
    issue_w(wc_, kt + NSW);
    // KS is even: the last step used F1, the next stage starts in F0
    read_frags(xslot(std::integral_constant<int, s + 1>{}), wslot(std::integral_constant<int, s + 1>{}),
               0, F0);
    mma(F1);
    order_transition();
  };
  static_assert(BK / 16 % 2 == 0, "even number of k steps per stage");
  // prologue: the transitions before stage 0 (t = -NSW .. -1), the wait of
  // the last one in between
  static_for<0, NSW - 1>([&](auto tt) {
    constexpr int t = decltype(tt)::value - NSW;
    if constexpr (t + NSX >= 0) issue_x(xslot(std::integral_constant<int, t + NSX>{}), t + NSX);
    issue_w(wslot(std::integral_constant<int, t + NSW>{}), t + NSW);
  });
  __builtin_amdgcn_s_waitcnt(WAIT0);
  __builtin_amdgcn_s_barrier();
  issue_x(xslot(std::integral_constant<int, NSX - 1>{}), NSX - 1);
  issue_w(wslot(std::integral_constant<int, NSW - 1>{}), NSW - 1);
  read_frags(X0, W0, 0, F0);
  for (int kt = 0; kt < nk; kt += LB)
    static_for<0, LB>([&](auto S) { stage(S, kt + decltype(S)::value); });
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
        } else if (!SWIGLU && a.y_tok) {
          const int tk = a.y_tok[p];
          const float g = a.y_gate[tk];
          const uint32_t r0 = pack_bf16x2(o[0], o[1]), r1 = pack_bf16x2(o[2], o[3]);
          uint2 v;
          v.x = pack_bf16x2(__builtin_fmaf(g, bf16lo(r0), 0.0f), __builtin_fmaf(g, bf16hi(r0), 0.0f));
          v.y = pack_bf16x2(__builtin_fmaf(g, bf16lo(r1), 0.0f), __builtin_fmaf(g, bf16hi(r1), 0.0f));
          *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(a.C) + (size_t)tk * N + n) = v;
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

// Tile shape, from the shape alone (the routing is not known on the host;
// the row counts are bounded by R_max).  Measured on MI355X:
//   L  256-row tiles, one workgroup of eight waves per CU (two per SIMD,
//      so one wave's waits overlap the other's MFMAs): best when K is long
//      and every group has many rows (the K loop amortises the pipeline
//      fill); the gate/up projection already from K = 1024;
//   M  128-row tiles, two per CU: the default;
//   N  (gate/up only) 128-row tiles of 64 output columns with 64-wide K
//      stages: every row segment a load fetches is a whole 128-byte line
//      (32-wide stages fetch half lines, which the memory system serves at
//      about two thirds of the rate); worth its extra activation re-reads
//      up to about two rounds of M tiles;
//   S  64-row tiles: fewer idle slots in the last round for small problems
//      (the down projection below about two rounds of 128-row tiles, the
//      gate/up projection only for a few hundred rows in all).
// Tile counts are estimated from the row bound (each group wastes half a
// tile on average).
enum TileCfg { TILE_L, TILE_M, TILE_N, TILE_S };
static long est_tiles(const GemmPlan& pl, int bm, int bno, int N) {
  const long mt = pl.grouped ? pl.R_max / bm + (pl.E + 1) / 2 : (pl.M_dense + bm - 1) / bm;
  return mt * ((N + bno - 1) / bno);
}
static TileCfg tile_cfg(const GemmPlan& pl, int N, int K, bool swiglu) {
  const int bno = swiglu ? 128 : 256;
  const long per_group = pl.grouped ? pl.R_max / (pl.E > 0 ? pl.E : 1) : pl.M_dense;
  if (K >= (swiglu ? 1024 : 2048) && per_group >= 1024 && est_tiles(pl, 256, bno, N) >= 256)
    return TILE_L;
  // GEMM 1 keeps 128-row tiles unless the rows are very few (decode); the
  // down projection takes 64-row tiles below about two rounds
  const long est_m = est_tiles(pl, 128, bno, N);
  if (!swiglu) return est_m > 1024 ? TILE_M : TILE_S;
  if (est_m > 1024) return TILE_M;
  return est_m > 256 ? TILE_N : TILE_S;
}
// Down projection with a narrow output and a long K (the Switch shape): 64-
// row tiles of 128 output columns, a third weight slot in flight.  Twice
// the column tiles of the 256-wide S tile, so half the K splits (half the
// fp32 partial planes) fill the chip; measured 32 -> 27.5 us there, worse
// for a short K or a wide output.
static bool down_narrow(int N, int K) { return N <= 1024 && K >= 2048; }

static int cfg_bm(TileCfg c) { return c == TILE_L ? 256 : (c == TILE_M || c == TILE_N) ? 128 : 64; }

template <int BM, int BNW, int WM, int WN, int BK, int NSX, int NSW, int OCC, bool SWIGLU,
          bool PARTIAL>
static hipError_t run_bf16(const GemmPlan& pl, GemmArgs a, hipStream_t st) {
  constexpr int BNO = SWIGLU ? BNW / 2 : BNW;
  a.n_tiles = (a.N + BNO - 1) / BNO;
  a.m_tiles = (int)row_tile_bound(pl, BM);
  // an upper bound on the tiles, rounded up to whole rounds of the 8 XCDs
  const long blocks = ((long)a.m_tiles * a.n_tiles * a.splits + 7) / 8 * 8;
  a.main_blocks = (int)blocks;
  const long grid = blocks + (a.y_tok ? (a.y_T + kZeroTok - 1) / kZeroTok : 0);
  if (grid == 0) return hipSuccess;
  if (a.a_rows)
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BNW, WM, WN, BK, NSX, NSW, OCC, SWIGLU, true, PARTIAL>),
                       dim3((unsigned)grid), dim3(64 * WM * WN), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BNW, WM, WN, BK, NSX, NSW, OCC, SWIGLU, false, PARTIAL>),
                       dim3((unsigned)grid), dim3(64 * WM * WN), 0, st, a);
  return hipGetLastError();
}

template <bool SWIGLU, bool PARTIAL>
static hipError_t run_cfg(const GemmPlan& pl, GemmArgs a, hipStream_t st) {
  switch (tile_cfg(pl, a.N, a.K, SWIGLU)) {
    case TILE_L: return run_bf16<256, 256, 4, 2, 64, 2, 3, 1, SWIGLU, PARTIAL>(pl, a, st);
    case TILE_M: return run_bf16<128, 256, 2, 2, 32, 3, 3, 2, SWIGLU, PARTIAL>(pl, a, st);
    case TILE_N:
      if constexpr (SWIGLU) return run_bf16<128, 128, 2, 2, 64, 2, 3, 2, SWIGLU, PARTIAL>(pl, a, st);
      else return hipErrorInvalidValue;  // gate/up only
    default:
      // a long K loop per tile wants the deeper ring; short ones two
      // workgroups per CU
      if constexpr (!SWIGLU) {
        if (down_narrow(a.N, a.K)) return run_bf16<64, 128, 1, 4, 64, 2, 3, 2, SWIGLU, PARTIAL>(pl, a, st);
      }
      if (!SWIGLU && a.k_chunk >= 2048) return run_bf16<64, 256, 1, 4, 64, 3, 3, 1, SWIGLU, PARTIAL>(pl, a, st);
      return run_bf16<64, 256, 1, 4, 64, 2, 2, 2, SWIGLU, PARTIAL>(pl, a, st);
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
  const TileCfg c = tile_cfg(pl, N, K, false);
  const int bm = cfg_bm(c);
  const long mt = pl.grouped ? (pl.R_max + bm - 1) / bm + (pl.E + 1) / 2
                             : (pl.M_dense + bm - 1) / bm;
  const int bn = (c == TILE_S && down_narrow(N, K)) ? 128 : 256;  // output columns per tile
  const long blocks = mt * ((N + bn - 1) / bn);
  // split only when the tiles leave CUs idle: from one workgroup per CU on,
  // the fp32 partial planes cost the combine more than the split gains (the
  // Switch down projection: 30.0 us at one split, 29.7-30.3 at two)
  const long want = 512;  // two workgroups per CU
  if (blocks == 0 || blocks >= want / 2 || K < 512) return 1;
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

hipError_t launch_gemm_down_combine(const GemmPlan& pl, const void* H, const void* Wd, int N,
                                    int K, const int32_t* row_token, const float* gates,
                                    const int32_t* route_pos, int T, void* y, hipStream_t st) {
  if (!pl.bf16 || N % 8) return hipErrorInvalidValue;
  const long h_rows = pl.grouped ? pl.R_max : pl.M_dense;
  GemmArgs a{H, nullptr, pl.offsets, pl.E, pl.M_dense, Wd, nullptr, N, K, y, 0, 0, 0,
             1, K, (unsigned)(h_rows * K * 2), row_token, gates, route_pos, T, 0};
  return run_cfg<false, false>(pl, a, st);
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
