// moe_api.cpp -- the C ABI of libmoe (include/moe.h): argument validation,
// capacity and workspace arithmetic, and stream-ordered kernel launches.
// No allocation, no host synchronisation, no state.
#include "moe.h"

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "launch.h"

// Workspace of moe_layer_forward_noalloc: one fixed array per GPU, part of
// the library's code object (each device holds its copy from module load
// until the process ends).  Host code never names it after set-up: its
// device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int64_t kMaxE = 256;
constexpr int64_t kMaxK = 8;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(const moe_shape* s) { return s->dtype == MOE_DTYPE_BF16 ? 2 : 4; }

int validate(const moe_shape* s) {
  if (!s) return MOE_ERR_INVALID_ARG;
  if (s->reserved != 0) return MOE_ERR_INVALID_ARG;
  if (s->T < 0 || s->d <= 0 || s->E <= 0 || s->k <= 0 || s->d_ff <= 0 || s->d_ff_shared < 0)
    return MOE_ERR_INVALID_ARG;
  if (s->d % 8 || s->d_ff % 8 || s->d_ff_shared % 8) return MOE_ERR_INVALID_ARG;
  if (s->k > s->E) return MOE_ERR_INVALID_ARG;
  if (isnan(s->phi)) return MOE_ERR_INVALID_ARG;
  if (s->renormalize != 0 && s->renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (s->dtype != MOE_DTYPE_F32 && s->dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
  if (s->tie_break != MOE_TIE_LOWEST_INDEX) return MOE_ERR_UNSUPPORTED;
  if (s->E > kMaxE || s->k > kMaxK) return MOE_ERR_UNSUPPORTED;
  if (s->T * s->k >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  // a GEMM tile's rows (at most 256) must span less than 2^31 bytes: the
  // packed-row operands are addressed with 32-bit offsets from each tile's
  // first row, so their total size is free
  if (s->d >= (int64_t(1) << 22) || s->d_ff >= (int64_t(1) << 22) ||
      s->d_ff_shared >= (int64_t(1) << 22))
    return MOE_ERR_UNSUPPORTED;
  // token rows gathered by the first GEMM (x) and each expert's weight
  // matrices are addressed from their own base: each must span less than
  // 2^31 bytes
  const int64_t eb = s->dtype == MOE_DTYPE_BF16 ? 2 : 4;
  const int64_t lim = int64_t(1) << 31;
  if (s->T * s->d * eb >= lim || s->d * s->d_ff * eb >= lim || s->d * s->d_ff_shared * eb >= lim)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// C = ceil(phi * (double)(T*k) / (double)E), -1 without a limit; clamped to T*k.
int64_t capacity_of(const moe_shape* s) {
  if (!(s->phi > 0.0)) return -1;
  const double c = ceil(s->phi * (double)(s->T * s->k) / (double)s->E);
  const double lim = (double)(s->T * s->k);
  return (int64_t)(c < lim ? c : lim);
}

int64_t rmax_of(const moe_shape* s, int64_t C) {
  const int64_t R = s->T * s->k;
  if (C < 0) return R;
  const int64_t ec = s->E * C;
  return ec < R ? ec : R;
}

struct Layout {
  size_t logits, ids, gates, cnt, counts, kept, offsets, route_pos, row_token, h, yp, part, hs,
      ys, spart, shist, xpad, opad, ppos, ids2, slot, offs2, rpos0, pref, dast, eck, ecp, ecoff;
  // queue policy: packed rows of the arrivals, the outgoing queue's arrivals
  size_t xq, qarr;
  // fp32 scratch of the down GEMM's split last round (0 bytes when no plan
  // of this shape splits)
  size_t tail;
  long tail_floats;
  int splits;      // K splits of the routed down GEMM (fp32 partial planes when > 1)
  int splits_pad;  // the same for the fixed-shape [E, C] layout
  int splits_ec;   // the same for expert-choice rows
  size_t total;
};

// Plan of the routed-expert grouped GEMMs.  Each token picks an expert at
// most once, so with routes from moe_route no group exceeds min(T, C) rows;
// moe_expert_ffn takes caller offsets and only assumes offsets[E] <= R_max.
moe::GemmPlan routed_plan(const moe_shape* s, const int32_t* offsets, bool own_routes) {
  const int64_t C = capacity_of(s);
  const int64_t Rmax = rmax_of(s, C);
  long cap = (long)Rmax;
  if (own_routes) cap = (C >= 0 && C < s->T) ? (long)C : (long)s->T;
  return moe::GemmPlan{s->dtype == MOE_DTYPE_BF16, true, offsets, (int)s->E, 0, (long)Rmax, cap};
}

// Rows of the fixed-shape dispatch buffer [E, C, d] (0 without a capacity).
int64_t rpad_of(const moe_shape* s) {
  const int64_t C = capacity_of(s);
  return C > 0 ? s->E * C : 0;
}

// The fixed-shape [E, C, d] buffer needs a capacity, and its rows must stay
// within 32-bit buffer offsets like every other expert buffer.
int validate_padded(const moe_shape* s) {
  if (capacity_of(s) <= 0) return MOE_ERR_INVALID_ARG;
  const int64_t eb = elem_bytes(s);
  const int64_t wide = s->d > s->d_ff ? s->d : s->d_ff;
  if (rpad_of(s) * wide * eb >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Plan of the expert GEMMs over the fixed-shape buffer: E groups of C rows
// (device offsets e*C), every row computed, empty slots included.
moe::GemmPlan padded_plan(const moe_shape* s, const int32_t* offsets_pad) {
  const int64_t C = capacity_of(s);
  return moe::GemmPlan{s->dtype == MOE_DTYPE_BF16, true, offsets_pad, (int)s->E, 0,
                       (long)rpad_of(s), (long)(C > 0 ? C : 0)};
}

// Expert choice: every expert keeps Ce = min(C, T) tokens (C from phi > 0;
// 0 without a capacity, which validate_choice rejects).
int64_t ce_of(const moe_shape* s) {
  const int64_t C = capacity_of(s);
  if (C < 0) return 0;
  return C < s->T ? C : s->T;
}

// Expert choice needs a capacity (its rows are the fixed E*Ce; their extent
// is bounded like the fixed-shape buffer's), full softmax gates (a token's
// number of experts is not fixed, so there is no set to renormalise over)
// and its expert-major key and route tables ([E][T], 4 bytes each) below
// 2^31 bytes.
int validate_choice(const moe_shape* s) {
  if (!(s->phi > 0.0) || s->renormalize != 0) return MOE_ERR_INVALID_ARG;
  if (s->E * s->T >= (int64_t(1) << 29)) return MOE_ERR_UNSUPPORTED;
  const int64_t eb = elem_bytes(s);
  const int64_t wide = s->d > s->d_ff ? s->d : s->d_ff;
  if (s->E * ce_of(s) * wide * eb >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// E groups of exactly Ce rows (device offsets e*Ce).
moe::GemmPlan choice_plan(const moe_shape* s, const int32_t* offsets_ec) {
  const int64_t Ce = ce_of(s);
  return moe::GemmPlan{s->dtype == MOE_DTYPE_BF16, true, offsets_ec, (int)s->E, 0,
                       (long)(s->E * Ce), (long)Ce};
}

// Queue policy ("queue to the next micro-batch"): Q routes waiting from the
// previous call arrive ahead of this call's T*k routes, N = Q + T*k arrivals
// of one route each.  Packed rows: at most E*C (C of this call), else N.
int64_t rmax_queue(const moe_shape* s, int64_t Q) {
  const int64_t C = capacity_of(s);
  const int64_t N = Q + s->T * s->k;
  if (C < 0) return N;
  const int64_t ec = s->E * C;
  return ec < N ? ec : N;
}

// An expert seats at most C arrivals, and never more than every queued
// route plus each token once.
moe::GemmPlan queue_plan(const moe_shape* s, int64_t Q, const int32_t* offsets) {
  const int64_t C = capacity_of(s);
  const int64_t most = Q + s->T;
  const long cap = (long)(C >= 0 && C < most ? C : most);
  moe::GemmPlan pl{s->dtype == MOE_DTYPE_BF16, true, offsets, (int)s->E, 0,
                   (long)rmax_queue(s, Q), cap};
  // GEMM 1's tile for the rows a call seats in steady state, the drop
  // policy's bound min(T*k, E*C), not E*C (Switch phi 1.25: the 128x256
  // tile for E*C = 5120 rows against 2505 seated)
  pl.R_tile = (long)rmax_of(s, C);
  return pl;
}

// Q >= 0: the queue policy's layout for Q waiting routes (route-sized
// arrays span the N = Q + T*k arrivals; the other layouts' buffers are left
// out).  Q < 0: the layout every other entry point uses.
Layout layout_of(const moe_shape* s, int64_t Q = -1) {
  const bool queued = Q >= 0;
  const int64_t C = capacity_of(s);
  const int64_t Rmax = queued ? rmax_queue(s, Q) : rmax_of(s, C);
  const size_t R = (size_t)(s->T * s->k + (queued ? Q : 0));
  const size_t eb = (size_t)elem_bytes(s);
  const size_t nch = (size_t)moe::permute_nchunks((long)R);
  Layout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes > 0 ? bytes : 1);
    return at;
  };
  L.logits = take((size_t)s->T * s->E * sizeof(float));
  L.ids = take(R * sizeof(int32_t));
  L.gates = take(R * sizeof(float));
  L.cnt = take((size_t)s->E * nch * sizeof(int32_t));
  L.counts = take((size_t)s->E * sizeof(int32_t));
  L.kept = take((size_t)s->E * sizeof(int32_t));
  L.offsets = take((size_t)(s->E + 1) * sizeof(int32_t));
  L.route_pos = take(R * sizeof(int32_t));
  // expert rows: the packed layout's R_max rows, or the fixed-shape
  // buffer's E*C rows when there is a capacity (the larger of the two;
  // expert choice's E*Ce rows are at most E*C)
  const int64_t Rpad = queued ? 0 : rpad_of(s);
  const size_t Rbig = (size_t)(Rpad > Rmax ? Rpad : Rmax);
  L.row_token = take(Rbig * sizeof(int32_t));
  L.h = take(Rbig * s->d_ff * eb);
  L.yp = take(Rbig * s->d * eb);
  const moe::GemmPlan routed = queued ? queue_plan(s, Q, nullptr) : routed_plan(s, nullptr, false);
  L.splits = moe::gemm_down_splits(routed, (int)s->d, (int)s->d_ff);
  L.splits_pad = Rpad > 0 ? moe::gemm_down_splits(padded_plan(s, nullptr), (int)s->d, (int)s->d_ff)
                          : 1;
  L.splits_ec = Rpad > 0 ? moe::gemm_down_splits(choice_plan(s, nullptr), (int)s->d, (int)s->d_ff)
                         : 1;
  const size_t part_rows = (size_t)(L.splits > 1 ? L.splits * Rmax : 0);
  const size_t part_rows_pad = (size_t)(L.splits_pad > 1 ? L.splits_pad * Rpad : 0);
  const size_t part_rows_ec =
      (size_t)(L.splits_ec > 1 && Rpad > 0 ? L.splits_ec * s->E * ce_of(s) : 0);
  size_t part_max = part_rows > part_rows_pad ? part_rows : part_rows_pad;
  if (part_rows_ec > part_max) part_max = part_rows_ec;
  L.part = take(part_max * s->d * sizeof(float));
  L.xpad = take((size_t)Rpad * s->d * eb);
  L.opad = take((size_t)(s->E + 1) * sizeof(int32_t));
  const size_t Ro = queued ? 0 : R;  // routes of the other layouts' buffers
  L.ppos = take(Ro * sizeof(int32_t));
  // reroute policy: primary positions, final experts and seats
  L.ids2 = take(Ro * sizeof(int32_t));
  L.slot = take(Ro * sizeof(int32_t));
  L.offs2 = take((size_t)(s->E + 1) * sizeof(int32_t));
  L.rpos0 = take(Ro * sizeof(int32_t));
  // preference ranks of the dropped routes: a 64-byte row per route up to
  // 64 experts, a 256-byte row for the wide walk beyond
  L.pref = take(Ro * (s->E > 64 ? 256 : 64));
  // per-token state of the parallel reroute where it does not fit LDS
  L.dast = take(queued || s->E > 64 ? 0 : (size_t)moe::reroute_state_bytes((int)s->T, (int)s->E));
  // expert choice: expert-major keys (score bits) and route table, row groups
  const size_t TE = queued ? 0 : (size_t)s->T * s->E;
  L.eck = take(TE * sizeof(uint32_t));
  L.ecp = take(TE * sizeof(int32_t));
  L.ecoff = take((size_t)(s->E + 1) * sizeof(int32_t));
  L.hs = take((size_t)s->T * s->d_ff_shared * eb);
  L.ys = take(s->d_ff_shared > 0 ? (size_t)s->T * s->d * eb : 0);
  // routing statistics: one partial row per 64 tokens
  const size_t sblk = (size_t)moe::stats_blocks((long)s->T);
  L.spart = take(sblk * (size_t)(s->E + 3) * sizeof(float));
  L.shist = take(sblk * (size_t)moe::kMaxStatBins * sizeof(int32_t));
  // queue policy: the seated arrivals' rows, packed (from x or the carried
  // queued rows), and the arrivals of the outgoing queue
  L.xq = take(queued ? (size_t)Rmax * s->d * eb : 0);
  L.qarr = take(queued ? R * sizeof(int32_t) : 0);
  long tf = moe::gemm_tail_floats(routed, (int)s->d, (int)s->d_ff);
  if (Rpad > 0) {
    const long tp = moe::gemm_tail_floats(padded_plan(s, nullptr), (int)s->d, (int)s->d_ff);
    const long tc = moe::gemm_tail_floats(choice_plan(s, nullptr), (int)s->d, (int)s->d_ff);
    tf = tp > tf ? tp : tf;
    tf = tc > tf ? tc : tf;
  }
  if (s->d_ff_shared > 0) {
    const moe::GemmPlan ps{s->dtype == MOE_DTYPE_BF16, false, nullptr, 1, (int)s->T, (long)s->T,
                           (long)s->T};
    const long ts = moe::gemm_tail_floats(ps, (int)s->d, (int)s->d_ff_shared);
    tf = ts > tf ? ts : tf;
  }
  L.tail_floats = tf;
  L.tail = take((size_t)tf * sizeof(float));
  L.total = o;
  return L;
}

int check_ws(const moe_shape* s, void* ws, size_t ws_bytes) {
  if (!ws) return MOE_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return MOE_ERR_WORKSPACE;
  if (ws_bytes < layout_of(s).total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(ws) + off);
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// The plan with the workspace's tail scratch attached, for a down GEMM of
// width N over K that splits its last round.
moe::GemmPlan with_tail(moe::GemmPlan pl, const Layout& L, void* ws, int N, int K) {
  const long need = moe::gemm_tail_floats(pl, N, K);
  pl.tail = (need > 0 && need <= L.tail_floats) ? at<float>(ws, L.tail) : nullptr;
  return pl;
}

// Device address of `scratch` on the current device, looked up once per
// device with that device current (the first noalloc call there); nullptr
// when the lookup fails.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: outside the supported range";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: kernel launch failed";
    default: return "unknown moe status";
  }
}

int moe_capacity(const moe_shape* s, int64_t* C_out, int64_t* R_max_out) {
  const int v = validate(s);
  if (v != MOE_OK) return v;
  const int64_t C = capacity_of(s);
  if (C_out) *C_out = C;
  if (R_max_out) *R_max_out = rmax_of(s, C);
  return MOE_OK;
}

int moe_workspace_bytes(const moe_shape* s, size_t* bytes_out) {
  const int v = validate(s);
  if (v != MOE_OK) return v;
  if (!bytes_out) return MOE_ERR_INVALID_ARG;
  *bytes_out = layout_of(s).total;
  return MOE_OK;
}

int moe_route(const moe_shape* s, const void* x, const void* w_router, const float* b_router,
              float* logits, int32_t* expert_ids, float* gates, void* ws, size_t ws_bytes,
              hipStream_t stream) {
  int v = validate(s);
  if (v != MOE_OK) return v;
  const bool tok = s->T > 0;  // token-sized buffers may be NULL when T == 0
  if (!w_router || (tok && (!x || !expert_ids || !gates))) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router)) return MOE_ERR_INVALID_ARG;
  if (!logits) {
    v = check_ws(s, ws, ws_bytes);
    if (v != MOE_OK) return v;
    logits = at<float>(ws, layout_of(s).logits);
  }
  return hip_status(moe::launch_route(s->dtype == MOE_DTYPE_BF16, x, w_router, b_router, (int)s->T,
                                      (int)s->d, (int)s->E, (int)s->k, s->renormalize, logits,
                                      expert_ids, gates, stream));
}

int moe_permute(const moe_shape* s, const void* x, const int32_t* expert_ids, int32_t* counts,
                int32_t* kept_counts, int32_t* offsets, int32_t* route_pos, int32_t* row_token,
                void* x_packed, void* ws, size_t ws_bytes, hipStream_t stream) {
  int v = validate(s);
  if (v != MOE_OK) return v;
  const bool tok = s->T > 0;  // token- and row-sized buffers may be NULL when T == 0
  if (!counts || !kept_counts || !offsets ||
      (tok && (!x || !expert_ids || !route_pos || !row_token || !x_packed)))
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(x_packed)) return MOE_ERR_INVALID_ARG;
  v = check_ws(s, ws, ws_bytes);
  if (v != MOE_OK) return v;
  const Layout L = layout_of(s);
  const int64_t C = capacity_of(s);
  hipError_t e = moe::launch_permute_index(expert_ids, (int)s->T, (int)s->k, (int)s->E, (int)C,
                                           at<int32_t>(ws, L.cnt), counts, kept_counts, offsets,
                                           route_pos, row_token, stream);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(moe::launch_gather_rows(x, row_token, offsets, (int)s->E, rmax_of(s, C),
                                            s->d * elem_bytes(s), x_packed, stream));
}

int moe_permute_padded(const moe_shape* s, const void* x, const int32_t* expert_ids,
                       int32_t* counts, int32_t* kept_counts, int32_t* route_pos, void* x_padded,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
  int v = validate(s);
  if (v != MOE_OK) return v;
  if ((v = validate_padded(s)) != MOE_OK) return v;
  const bool tok = s->T > 0;
  if (!counts || !kept_counts || !x_padded || (tok && (!x || !expert_ids || !route_pos)))
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(x_padded)) return MOE_ERR_INVALID_ARG;
  v = check_ws(s, ws, ws_bytes);
  if (v != MOE_OK) return v;
  const Layout L = layout_of(s);
  const int64_t C = capacity_of(s);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* rpos = at<int32_t>(ws, L.route_pos);
  int32_t* row_token = at<int32_t>(ws, L.row_token);
  hipError_t e = moe::launch_permute_index(expert_ids, (int)s->T, (int)s->k, (int)s->E, (int)C,
                                           at<int32_t>(ws, L.cnt), counts, kept_counts, offsets,
                                           rpos, row_token, stream);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(moe::launch_padded(x, expert_ids, rpos, offsets, kept_counts, row_token,
                                       (int)s->T, (int)s->k, (int)s->E, (int)C,
                                       s->d * elem_bytes(s), route_pos, x_padded,
                                       at<int32_t>(ws, L.opad), stream));
}

int moe_permute_reroute(const moe_shape* s, const void* x, const float* logits,
                        const int32_t* expert_ids, int32_t* expert_ids_out, int32_t* counts,
                        int32_t* filled, int32_t* offsets, int32_t* route_pos,
                        int32_t* row_token, void* x_packed, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  int v = validate(s);
  if (v != MOE_OK) return v;
  const bool tok = s->T > 0;
  if (!counts || !filled || !offsets ||
      (tok && (!x || !logits || !expert_ids || !expert_ids_out || !route_pos || !row_token ||
               !x_packed)))
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(x_packed)) return MOE_ERR_INVALID_ARG;
  v = check_ws(s, ws, ws_bytes);
  if (v != MOE_OK) return v;
  const Layout L = layout_of(s);
  const int64_t C = capacity_of(s);
  const int T = (int)s->T, k = (int)s->k, E = (int)s->E;
  int32_t* offs0 = at<int32_t>(ws, L.offsets);
  hipError_t e = moe::launch_permute_index(expert_ids, T, k, E, (int)C, at<int32_t>(ws, L.cnt),
                                           counts, filled, offs0, at<int32_t>(ws, L.rpos0),
                                           row_token, stream);
  if (e != hipSuccess) return MOE_ERR_HIP;
  // kept counts (in filled) seed the walk, which turns them into seats
  e = moe::launch_reroute(logits, expert_ids, at<int32_t>(ws, L.rpos0), offs0, filled, T, k, E,
                          (int)C, expert_ids_out, at<int32_t>(ws, L.slot), offsets, route_pos,
                          row_token, at<uint8_t>(ws, L.pref), at<uint8_t>(ws, L.dast), stream);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = moe::launch_seats(offsets, E, filled, stream);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(moe::launch_gather_rows(x, row_token, offsets, E, rmax_of(s, C),
                                            s->d * elem_bytes(s), x_packed, stream));
}

int moe_permute_expert_choice(const moe_shape* s, const void* x, const float* logits,
                              float* scores, int32_t* route_pos, int32_t* offsets,
                              int32_t* row_token, void* x_packed, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  int v = validate(s);
  if (v != MOE_OK) return v;
  if ((v = validate_choice(s)) != MOE_OK) return v;
  const bool tok = s->T > 0;
  if (!offsets || (tok && (!x || !logits || !scores || !route_pos || !row_token || !x_packed)))
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(x_packed)) return MOE_ERR_INVALID_ARG;
  v = check_ws(s, ws, ws_bytes);
  if (v != MOE_OK) return v;
  const Layout L = layout_of(s);
  const int T = (int)s->T, E = (int)s->E;
  const int Ce = (int)ce_of(s);
  hipError_t e = moe::launch_expert_choice(logits, T, E, Ce, scores, at<uint32_t>(ws, L.eck),
                                           at<int32_t>(ws, L.ecp), route_pos, row_token, offsets,
                                           stream);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(moe::launch_gather_rows(x, row_token, offsets, E, (long)E * Ce,
                                            s->d * elem_bytes(s), x_packed, stream));
}

int moe_expert_ffn(const moe_shape* s, const void* x_packed, const int32_t* offsets,
                   const void* w_gate, const void* w_up, const void* w_down, void* y_packed,
                   void* ws, size_t ws_bytes, hipStream_t stream) {
  int v = validate(s);
  if (v != MOE_OK) return v;
  const bool tok = s->T > 0;  // row-sized buffers may be NULL when T == 0
  if (!offsets || !w_gate || !w_up || !w_down || (tok && (!x_packed || !y_packed)))
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_packed) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) ||
      !aligned16(y_packed))
    return MOE_ERR_INVALID_ARG;
  v = check_ws(s, ws, ws_bytes);
  if (v != MOE_OK) return v;
  const Layout L = layout_of(s);
  const moe::GemmPlan pl = with_tail(routed_plan(s, offsets, false), L, ws, (int)s->d, (int)s->d_ff);
  const bool bf16 = s->dtype == MOE_DTYPE_BF16;
  void* h = at<void>(ws, L.h);
  hipError_t e = moe::launch_gemm_swiglu(pl, x_packed, nullptr, pl.R_max, w_gate, w_up,
                                         (int)s->d_ff, (int)s->d, h, stream);
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (L.splits <= 1)
    return hip_status(moe::launch_gemm_down(pl, h, w_down, (int)s->d, (int)s->d_ff, y_packed, 1,
                                            0, stream));
  float* part = at<float>(ws, L.part);
  const long stride = pl.R_max * s->d;
  e = moe::launch_gemm_down(pl, h, w_down, (int)s->d, (int)s->d_ff, part, L.splits, stride,
                            stream);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(moe::launch_reduce_splits(bf16, part, L.splits, stride, offsets, (int)s->E,
                                              pl.R_max, (int)s->d, y_packed, stream));
}

int moe_combine(const moe_shape* s, const void* y_packed, const int32_t* route_pos,
                const float* gates, const void* y_shared, void* y, hipStream_t stream) {
  int v = validate(s);
  if (v != MOE_OK) return v;
  if (s->T > 0 && (!y_packed || !route_pos || !gates || !y)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(y_packed) || !aligned16(y) || (y_shared && !aligned16(y_shared)))
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_combine(s->dtype == MOE_DTYPE_BF16, y_packed, 1, 0, route_pos,
                                        gates, y_shared, (int)s->T, (int)s->k, (int)s->d, y,
                                        stream));
}

int moe_routing_stats(const moe_shape* s, const float* logits, const float* gates,
                      const int32_t* counts, double alpha, int32_t n_bins, float* stats,
                      int32_t* hist, void* ws, size_t ws_bytes, hipStream_t stream) {
  int v = validate(s);
  if (v != MOE_OK) return v;
  if (!counts || !stats || !hist || (s->T > 0 && (!logits || !gates))) return MOE_ERR_INVALID_ARG;
  if (n_bins < 1 || n_bins > moe::kMaxStatBins || isnan(alpha)) return MOE_ERR_INVALID_ARG;
  v = check_ws(s, ws, ws_bytes);
  if (v != MOE_OK) return v;
  const Layout L = layout_of(s);
  return hip_status(moe::launch_routing_stats(logits, gates, counts, (int)s->T, (int)s->E,
                                              (int)s->k, n_bins, (float)alpha,
                                              at<float>(ws, L.spart), at<int32_t>(ws, L.shist),
                                              stats, hist, stream));
}

// Expert GEMMs over the row groups of pl (activations A, gathered through
// a_rows when non-null; a_nrows rows of A), the shared expert (on x), and the
// combine over kslots slots per token (route table rpos, gates g, both
// [T][kslots], or [kslots][T] when slot_major).  splits: K splits of the
// down GEMM, whose fp32 planes hold `rows` rows each.  Records events 2..6 of
// the timed variant.
static int experts_and_combine(const moe_shape* s, const Layout& L, const moe::GemmPlan& pl_in,
                               const void* x, const void* A, const int32_t* a_rows, long a_nrows,
                               const void* w_gate, const void* w_up, const void* w_down,
                               const void* ws_gate, const void* ws_up, const void* ws_down,
                               int splits, long rows, const int32_t* rpos, const float* g,
                               int kslots, bool slot_major, void* y, void* ws, hipStream_t stream,
                               hipEvent_t* ev) {
  const bool bf16 = s->dtype == MOE_DTYPE_BF16;
  const int T = (int)s->T, d = (int)s->d, dff = (int)s->d_ff;
  const moe::GemmPlan pl = with_tail(pl_in, L, ws, d, dff);
  void* h = at<void>(ws, L.h);
  void* yp = at<void>(ws, L.yp);
  auto mark = [&](int i) {
    // a stage marker: a failed record loses a timing, never a result
    if (ev && ev[i]) (void)hipEventRecord(ev[i], stream);
  };
  hipError_t e;
  if (a_rows && moe::gemm_swiglu_prefers_packed(pl, dff, d)) {
    // The 256x256 GEMM 1 tile streams packed rows faster than it gathers
    // token rows (each of a tile's loads then takes a wave-uniform base), by
    // more than the gather costs at a wide d_ff: the dispatch packs the rows
    // (the pack of the permute step, before GEMM 1's stage marker) into
    // y_packed, which is free until the down GEMM writes it.
    e = moe::launch_gather_rows(A, a_rows, pl.offsets, pl.E, pl.R_max, (long)d * elem_bytes(s), yp,
                                stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
    mark(2);
    e = moe::launch_gemm_swiglu(pl, yp, nullptr, pl.R_max, w_gate, w_up, dff, d, h, stream);
  } else {
    mark(2);
    e = moe::launch_gemm_swiglu(pl, A, a_rows, a_nrows, w_gate, w_up, dff, d, h, stream);
  }
  if (e != hipSuccess) return MOE_ERR_HIP;
  mark(3);
  if (bf16 && splits <= 1 && s->d_ff_shared == 0 && kslots == 1 && !slot_major && a_rows) {
    // one route per token and nothing to add: the down GEMM writes y itself
    e = moe::launch_gemm_down_combine(pl, h, w_down, d, dff, a_rows, g, rpos, T, y, stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
    mark(4);
    mark(5);
    mark(6);
    return MOE_OK;
  }
  const void* yrows = yp;
  const long stride = rows * d;
  if (splits > 1) {
    yrows = at<float>(ws, L.part);
    e = moe::launch_gemm_down(pl, h, w_down, d, dff, at<float>(ws, L.part), splits, stride,
                              stream);
  } else {
    e = moe::launch_gemm_down(pl, h, w_down, d, dff, yp, 1, 0, stream);
  }
  if (e != hipSuccess) return MOE_ERR_HIP;
  mark(4);
  const void* ysh = nullptr;
  if (s->d_ff_shared > 0) {
    const moe::GemmPlan ps = with_tail(moe::GemmPlan{bf16, false, nullptr, 1, T, (long)T, (long)T},
                                       L, ws, d, (int)s->d_ff_shared);
    void* hs = at<void>(ws, L.hs);
    void* ys = at<void>(ws, L.ys);
    e = moe::launch_gemm_swiglu(ps, x, nullptr, T, ws_gate, ws_up, (int)s->d_ff_shared, d, hs,
                                stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
    e = moe::launch_gemm_down(ps, hs, ws_down, d, (int)s->d_ff_shared, ys, 1, 0, stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
    ysh = ys;
  }
  mark(5);
  e = slot_major ? moe::launch_combine_slot_major(bf16, yrows, splits, stride, rpos, g, ysh, T,
                                                  kslots, d, y, stream)
                 : moe::launch_combine(bf16, yrows, splits, stride, rpos, g, ysh, T, kslots, d, y,
                                       stream);
  if (e != hipSuccess) return MOE_ERR_HIP;
  mark(6);
  return MOE_OK;
}

static int layer_forward_impl(const moe_shape* s, const void* x, const void* w_router,
                              const float* b_router, const void* w_gate, const void* w_up,
                              const void* w_down, const void* ws_gate, const void* ws_up,
                              const void* ws_down, void* y, int32_t* expert_ids, float* gates,
                              int32_t* counts, int32_t* route_pos, void* ws, size_t ws_bytes,
                              hipStream_t stream, hipEvent_t* ev, int layout) {
  // layout 0: packed rows; 1: fixed-shape [E, C, d] buffer; 2: packed rows
  // after the reroute overflow policy; 3: expert-choice rows (gates and
  // route_pos are then [T][E], expert_ids and counts unused)
  const bool padded = layout == 1;
  const bool reroute = layout == 2;
  const bool choice = layout == 3;
  int v = validate(s);
  if (v != MOE_OK) return v;
  if (padded && (v = validate_padded(s)) != MOE_OK) return v;
  if (choice && (v = validate_choice(s)) != MOE_OK) return v;
  if (!w_router || !w_gate || !w_up || !w_down || (s->T > 0 && (!x || !y)))
    return MOE_ERR_INVALID_ARG;
  const bool shared = s->d_ff_shared > 0;
  if (shared && (!ws_gate || !ws_up || !ws_down)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(w_gate) || !aligned16(w_up) ||
      !aligned16(w_down) || !aligned16(y))
    return MOE_ERR_INVALID_ARG;
  if (shared && (!aligned16(ws_gate) || !aligned16(ws_up) || !aligned16(ws_down)))
    return MOE_ERR_INVALID_ARG;
  v = check_ws(s, ws, ws_bytes);
  if (v != MOE_OK) return v;

  const Layout L = layout_of(s);
  const bool bf16 = s->dtype == MOE_DTYPE_BF16;
  const int T = (int)s->T, d = (int)s->d, E = (int)s->E, k = (int)s->k;
  const int64_t C = capacity_of(s);
  const int64_t Rmax = rmax_of(s, C);
  // router choices (rerouting keeps them internal and reports the final
  // experts in expert_ids)
  int32_t* ids = (expert_ids && !reroute) ? expert_ids : at<int32_t>(ws, L.ids);
  int32_t* ids_final = expert_ids ? expert_ids : at<int32_t>(ws, L.ids2);
  float* g = gates ? gates : at<float>(ws, L.gates);
  int32_t* cnts = counts ? counts : at<int32_t>(ws, L.counts);
  // route positions: the caller's array receives the packed rows, or the
  // fixed-shape buffer's rows e*C + slot (the packed ones then stay internal)
  int32_t* rpos = (route_pos && !padded) ? route_pos : at<int32_t>(ws, L.route_pos);
  int32_t* ppos = route_pos ? route_pos : at<int32_t>(ws, L.ppos);
  const int64_t Rpad = rpad_of(s);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* row_token = at<int32_t>(ws, L.row_token);

  auto mark = [&](int i) {
    // a stage marker: a failed record loses a timing, never a result
    if (ev && ev[i]) (void)hipEventRecord(ev[i], stream);
  };
  mark(0);
  if (choice) {
    // expert choice: logits, each expert's top-Ce tokens, then the shared
    // GEMM, shared-expert and combine stages below with one slot per expert
    // the route table stays expert-major inside; the callers' [T][E] copies
    // of the scores and the table are written only when asked for
    const int Ce = (int)ce_of(s);
    uint32_t* keys = at<uint32_t>(ws, L.eck);
    int32_t* pos_et = at<int32_t>(ws, L.ecp);
    int32_t* ecoff = at<int32_t>(ws, L.ecoff);
    hipError_t e = moe::launch_route(bf16, x, w_router, b_router, T, d, E, k, 0,
                                     at<float>(ws, L.logits), nullptr, nullptr, stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
    mark(1);
    e = moe::launch_expert_choice(at<float>(ws, L.logits), T, E, Ce, gates, keys, pos_et,
                                  route_pos, row_token, ecoff, stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
    // gates: the score bits in the keys, read as floats, expert-major
    return experts_and_combine(s, L, choice_plan(s, ecoff), x, x, row_token, T, w_gate, w_up,
                               w_down, ws_gate, ws_up, ws_down, L.splits_ec, (long)E * Ce, pos_et,
                               reinterpret_cast<const float*>(keys), E, true, y, ws, stream, ev);
  }
  // few tokens and experts: top-k runs inside the single-workgroup permute
  // (one launch fewer; the route stage is then the projection alone)
  const bool fused = moe::topk_permute_fused(T, k, E);
  float* logits = at<float>(ws, L.logits);
  hipError_t e = moe::launch_route(bf16, x, w_router, b_router, T, d, E, k, s->renormalize, logits,
                                   fused ? nullptr : ids, g, stream);
  if (e != hipSuccess) return MOE_ERR_HIP;
  mark(1);
  int32_t* rp = reroute ? at<int32_t>(ws, L.rpos0) : rpos;
  e = fused ? moe::launch_topk_permute(logits, T, E, k, s->renormalize, (int)C, ids, g, cnts,
                                       at<int32_t>(ws, L.kept), offsets, rp, row_token, stream)
            : moe::launch_permute_index(ids, T, k, E, (int)C, at<int32_t>(ws, L.cnt), cnts,
                                        at<int32_t>(ws, L.kept), offsets, rp, row_token, stream);
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (reroute) {
    // the drop-policy seats stay; dropped routes move; packed rows follow
    // the final experts (offsets become the rerouted ones)
    e = moe::launch_reroute(at<float>(ws, L.logits), ids, at<int32_t>(ws, L.rpos0), offsets,
                            at<int32_t>(ws, L.kept), T, k, E, (int)C, ids_final,
                            at<int32_t>(ws, L.slot), at<int32_t>(ws, L.offs2), rpos, row_token,
                            at<uint8_t>(ws, L.pref), at<uint8_t>(ws, L.dast), stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
    offsets = at<int32_t>(ws, L.offs2);
  }
  if (padded) {
    e = moe::launch_padded(x, ids, rpos, offsets, at<int32_t>(ws, L.kept), row_token, T, k, E,
                           (int)C, (long)d * elem_bytes(s), ppos, at<void>(ws, L.xpad),
                           at<int32_t>(ws, L.opad), stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  const moe::GemmPlan pl =
      padded ? padded_plan(s, at<int32_t>(ws, L.opad)) : routed_plan(s, offsets, true);
  if (padded)
    return experts_and_combine(s, L, pl, x, at<void>(ws, L.xpad), nullptr, Rpad, w_gate, w_up,
                               w_down, ws_gate, ws_up, ws_down, L.splits_pad, Rpad, ppos, g, k,
                               false, y, ws, stream, ev);
  return experts_and_combine(s, L, pl, x, x, row_token, T, w_gate, w_up, w_down, ws_gate, ws_up,
                             ws_down, L.splits, Rmax, rpos, g, k, false, y, ws, stream, ev);
}

int moe_layer_forward(const moe_shape* s, const void* x, const void* w_router,
                      const float* b_router, const void* w_gate, const void* w_up,
                      const void* w_down, const void* ws_gate, const void* ws_up,
                      const void* ws_down, void* y, int32_t* expert_ids, float* gates,
                      int32_t* counts, int32_t* route_pos, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  return layer_forward_impl(s, x, w_router, b_router, w_gate, w_up, w_down, ws_gate, ws_up,
                            ws_down, y, expert_ids, gates, counts, route_pos, ws, ws_bytes,
                            stream, nullptr, 0);
}

int moe_layer_forward_noalloc(const moe_shape* s, const void* x, const void* w_router,
                              const float* b_router, const void* w_gate, const void* w_up,
                              const void* w_down, const void* ws_gate, const void* ws_up,
                              const void* ws_down, void* y, int32_t* expert_ids, float* gates,
                              int32_t* counts, int32_t* route_pos, hipStream_t stream) {
  const int v = validate(s);
  if (v != MOE_OK) return v;
  // the layout moe_layer_forward would take from the caller's workspace
  // must fit the fixed array; checked before anything touches the device
  if (layout_of(s).total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_UNSUPPORTED;
  void* ws = scratch_on_current_device();
  if (!ws) return MOE_ERR_HIP;
  return layer_forward_impl(s, x, w_router, b_router, w_gate, w_up, w_down, ws_gate, ws_up,
                            ws_down, y, expert_ids, gates, counts, route_pos, ws,
                            (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream, nullptr, 0);
}

int moe_layer_forward_padded(const moe_shape* s, const void* x, const void* w_router,
                             const float* b_router, const void* w_gate, const void* w_up,
                             const void* w_down, const void* ws_gate, const void* ws_up,
                             const void* ws_down, void* y, int32_t* expert_ids, float* gates,
                             int32_t* counts, int32_t* route_pos, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  return layer_forward_impl(s, x, w_router, b_router, w_gate, w_up, w_down, ws_gate, ws_up,
                            ws_down, y, expert_ids, gates, counts, route_pos, ws, ws_bytes,
                            stream, nullptr, 1);
}

int moe_layer_forward_reroute(const moe_shape* s, const void* x, const void* w_router,
                              const float* b_router, const void* w_gate, const void* w_up,
                              const void* w_down, const void* ws_gate, const void* ws_up,
                              const void* ws_down, void* y, int32_t* expert_ids, float* gates,
                              int32_t* counts, int32_t* route_pos, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  return layer_forward_impl(s, x, w_router, b_router, w_gate, w_up, w_down, ws_gate, ws_up,
                            ws_down, y, expert_ids, gates, counts, route_pos, ws, ws_bytes,
                            stream, nullptr, 2);
}

int moe_layer_forward_expert_choice(const moe_shape* s, const void* x, const void* w_router,
                                    const float* b_router, const void* w_gate, const void* w_up,
                                    const void* w_down, const void* ws_gate, const void* ws_up,
                                    const void* ws_down, void* y, float* scores,
                                    int32_t* route_pos, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
  return layer_forward_impl(s, x, w_router, b_router, w_gate, w_up, w_down, ws_gate, ws_up,
                            ws_down, y, nullptr, scores, nullptr, route_pos, ws, ws_bytes, stream,
                            nullptr, 3);
}

int moe_layer_forward_timed(const moe_shape* s, const void* x, const void* w_router,
                            const float* b_router, const void* w_gate, const void* w_up,
                            const void* w_down, const void* ws_gate, const void* ws_up,
                            const void* ws_down, void* y, void* ws, size_t ws_bytes,
                            hipStream_t stream, hipEvent_t* events, int32_t layout) {
  if (!events) return MOE_ERR_INVALID_ARG;
  if (layout < 0 || layout > 3) return MOE_ERR_INVALID_ARG;
  return layer_forward_impl(s, x, w_router, b_router, w_gate, w_up, w_down, ws_gate, ws_up,
                            ws_down, y, nullptr, nullptr, nullptr, nullptr, ws, ws_bytes, stream,
                            events, layout);
}

// Queue policy: the waiting routes of the previous call arrive first; the
// drop policy runs over the arrivals (one route each); the routes past
// capacity form the outgoing queue.  The seated rows are gathered from x and
// the carried queued rows into packed rows.
static int layer_forward_queued_impl(
    const moe_shape* s, const void* x, const void* w_router, const float* b_router,
    const void* w_gate, const void* w_up, const void* w_down, const void* ws_gate,
    const void* ws_up, const void* ws_down, int64_t q_n, const void* q_x, const int32_t* q_ids,
    const float* q_gates, const int64_t* q_tags, int64_t tag_base, void* y, void* y_late,
    int32_t* out_n, void* out_x, int32_t* out_ids, float* out_gates, int64_t* out_tags,
    int32_t* expert_ids, float* gates, int32_t* counts, int32_t* route_pos, void* ws,
    size_t ws_bytes, hipStream_t stream, hipEvent_t* ev) {
  int v = validate(s);
  if (v != MOE_OK) return v;
  if (q_n < 0) return MOE_ERR_INVALID_ARG;
  const int64_t Q = q_n, N = q_n + s->T * s->k;
  const int64_t eb = elem_bytes(s);
  const int64_t lim = int64_t(1) << 31;
  const int64_t wide = s->d > s->d_ff ? s->d : s->d_ff;
  if (N >= lim || Q * s->d * eb >= lim || rmax_queue(s, Q) * wide * eb >= lim)
    return MOE_ERR_UNSUPPORTED;
  if (!w_router || !w_gate || !w_up || !w_down || !out_n || (s->T > 0 && (!x || !y)) ||
      (Q > 0 && (!q_x || !q_ids || !q_gates || !q_tags || !y_late)) ||
      (N > 0 && (!out_x || !out_ids || !out_gates || !out_tags)))
    return MOE_ERR_INVALID_ARG;
  const bool shared = s->d_ff_shared > 0;
  if (shared && (!ws_gate || !ws_up || !ws_down)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(w_gate) || !aligned16(w_up) ||
      !aligned16(w_down) || !aligned16(y) || !aligned16(q_x) || !aligned16(y_late) ||
      !aligned16(out_x))
    return MOE_ERR_INVALID_ARG;
  if (shared && (!aligned16(ws_gate) || !aligned16(ws_up) || !aligned16(ws_down)))
    return MOE_ERR_INVALID_ARG;
  if (!ws || reinterpret_cast<uintptr_t>(ws) % kAlign) return MOE_ERR_WORKSPACE;
  const Layout L = layout_of(s, Q);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;

  const bool bf16 = s->dtype == MOE_DTYPE_BF16;
  const int T = (int)s->T, d = (int)s->d, E = (int)s->E, k = (int)s->k;
  const int64_t C = capacity_of(s);
  const int64_t Rmax = rmax_queue(s, Q);
  const size_t row_bytes = (size_t)d * eb;
  int32_t* ids_all = at<int32_t>(ws, L.ids);  // [Q queued experts; T*k router choices]
  float* g = gates ? gates : at<float>(ws, L.gates);
  int32_t* cnts = counts ? counts : at<int32_t>(ws, L.counts);
  int32_t* pos = route_pos ? route_pos : at<int32_t>(ws, L.route_pos);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* row_token = at<int32_t>(ws, L.row_token);  // arrival of each packed row
  void* xq = at<void>(ws, L.xq);
  auto mark = [&](int i) {
    // a stage marker: a failed record loses a timing, never a result
    if (ev && ev[i]) (void)hipEventRecord(ev[i], stream);
  };
  mark(0);
  // arrivals: the queued experts, then this batch's router choices
  if (Q > 0 && hipMemcpyAsync(ids_all, q_ids, (size_t)Q * sizeof(int32_t),
                              hipMemcpyDeviceToDevice, stream) != hipSuccess)
    return MOE_ERR_HIP;
  hipError_t e = moe::launch_route(bf16, x, w_router, b_router, T, d, E, k, s->renormalize,
                                   at<float>(ws, L.logits), ids_all + Q, g, stream);
  if (e != hipSuccess) return MOE_ERR_HIP;
  mark(1);
  if (expert_ids && T > 0 &&
      hipMemcpyAsync(expert_ids, ids_all + Q, (size_t)T * k * sizeof(int32_t),
                     hipMemcpyDeviceToDevice, stream) != hipSuccess)
    return MOE_ERR_HIP;
  // the drop policy over the arrivals, then the seated rows, packed
  e = moe::launch_permute_index(ids_all, (int)N, 1, E, (int)C, at<int32_t>(ws, L.cnt), cnts,
                                at<int32_t>(ws, L.kept), offsets, pos, row_token, stream);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = moe::launch_queue_gather(x, q_x, row_token, offsets + E, (int)Q, k, (long)Rmax,
                               (long)row_bytes, xq, stream);
  if (e != hipSuccess) return MOE_ERR_HIP;
  // the outgoing queue: arrivals past capacity, in arrival order, and their rows
  int32_t* qarr = at<int32_t>(ws, L.qarr);
  e = moe::launch_queue_compact(pos, (long)N, (int)Q, k, q_ids, q_gates, q_tags, ids_all + Q, g,
                                tag_base, out_n, qarr, out_ids, out_gates, out_tags, stream);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = moe::launch_queue_gather(x, q_x, qarr, out_n, (int)Q, k, (long)N, (long)row_bytes, out_x,
                               stream);
  if (e != hipSuccess) return MOE_ERR_HIP;
  // experts on the seated rows, shared expert, this batch's combine
  const moe::GemmPlan pl = queue_plan(s, Q, offsets);
  v = experts_and_combine(s, L, pl, x, xq, nullptr, (long)Rmax, w_gate, w_up, w_down, ws_gate,
                          ws_up, ws_down, L.splits, (long)Rmax, pos + Q, g, k, false, y, ws, stream,
                          ev);
  if (v != MOE_OK) return v;
  // late rows: each queued route's gated output (zero when it waits again)
  if (Q > 0) {
    const void* yrows = L.splits > 1 ? at<void>(ws, L.part) : at<void>(ws, L.yp);
    e = moe::launch_combine(bf16, yrows, L.splits, (long)Rmax * d, pos, q_gates, nullptr, (int)Q,
                            1, d, y_late, stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  return MOE_OK;
}

int moe_workspace_bytes_queued(const moe_shape* s, int64_t q_n, size_t* bytes_out) {
  int v = validate(s);
  if (v != MOE_OK) return v;
  if (!bytes_out || q_n < 0) return MOE_ERR_INVALID_ARG;
  *bytes_out = layout_of(s, q_n).total;
  return MOE_OK;
}

int moe_layer_forward_queued(const moe_shape* s, const void* x, const void* w_router,
                             const float* b_router, const void* w_gate, const void* w_up,
                             const void* w_down, const void* ws_gate, const void* ws_up,
                             const void* ws_down, int64_t q_n, const void* q_x,
                             const int32_t* q_ids, const float* q_gates, const int64_t* q_tags,
                             int64_t tag_base, void* y, void* y_late, int32_t* out_n, void* out_x,
                             int32_t* out_ids, float* out_gates, int64_t* out_tags,
                             int32_t* expert_ids, float* gates, int32_t* counts,
                             int32_t* route_pos, void* ws, size_t ws_bytes, hipStream_t stream) {
  return layer_forward_queued_impl(s, x, w_router, b_router, w_gate, w_up, w_down, ws_gate, ws_up,
                                   ws_down, q_n, q_x, q_ids, q_gates, q_tags, tag_base, y, y_late,
                                   out_n, out_x, out_ids, out_gates, out_tags, expert_ids, gates,
                                   counts, route_pos, ws, ws_bytes, stream, nullptr);
}

int moe_layer_forward_queued_timed(const moe_shape* s, const void* x, const void* w_router,
                                   const float* b_router, const void* w_gate, const void* w_up,
                                   const void* w_down, const void* ws_gate, const void* ws_up,
                                   const void* ws_down, int64_t q_n, const void* q_x,
                                   const int32_t* q_ids, const float* q_gates,
                                   const int64_t* q_tags, void* y, void* y_late, int32_t* out_n,
                                   void* out_x, int32_t* out_ids, float* out_gates,
                                   int64_t* out_tags, void* ws, size_t ws_bytes,
                                   hipStream_t stream, hipEvent_t* events) {
  if (!events) return MOE_ERR_INVALID_ARG;
  return layer_forward_queued_impl(s, x, w_router, b_router, w_gate, w_up, w_down, ws_gate, ws_up,
                                   ws_down, q_n, q_x, q_ids, q_gates, q_tags, 0, y, y_late, out_n,
                                   out_x, out_ids, out_gates, out_tags, nullptr, nullptr, nullptr,
                                   nullptr, ws, ws_bytes, stream, events);
}

}  // extern "C"
