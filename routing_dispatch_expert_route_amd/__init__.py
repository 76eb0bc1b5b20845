"""MI355X (gfx950) MoE layer forward: route + pack + compute + combine.

Thin Python binding over the C ABI of libmoe.so (include/moe.h).  Every step
of the layer runs in the library's HIP kernels; this module only checks
tensor arguments, allocates outputs with torch (device memory and streams are
torch's) and passes pointers.  There is no fallback: importing this package
fails when libmoe.so has not been built.

Entry points (same names as the C ABI, without the moe_ prefix):
    capacity, workspace_bytes, route, permute, expert_ffn, combine,
    layer_forward, layer_forward_timed, routing_stats, permute_padded,
    permute_reroute, permute_expert_choice, layer_forward_expert_choice,
    workspace_bytes_queued, layer_forward_queued, layer_forward_queued_timed,
    layer_forward_noalloc
    (layer_forward takes padded= / reroute= for the other layouts)
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libmoe.so is not built ({LIB_PATH}); run "
        "`python routing_dispatch_expert_route_amd/build.py` or __graft_entry__.build()")

_lib = ctypes.CDLL(LIB_PATH)

DTYPE_F32, DTYPE_BF16 = 0, 1
MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)

EXPORTS = ("moe_status_string", "moe_capacity", "moe_workspace_bytes", "moe_route",
           "moe_permute", "moe_expert_ffn", "moe_combine", "moe_layer_forward",
           "moe_layer_forward_timed", "moe_routing_stats", "moe_permute_padded",
           "moe_layer_forward_padded", "moe_permute_reroute", "moe_layer_forward_reroute",
           "moe_permute_expert_choice", "moe_layer_forward_expert_choice",
           "moe_workspace_bytes_queued", "moe_layer_forward_queued",
           "moe_layer_forward_queued_timed", "moe_layer_forward_noalloc")


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int64), ("E", ctypes.c_int64),
                ("k", ctypes.c_int64), ("d_ff", ctypes.c_int64), ("d_ff_shared", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("renormalize", ctypes.c_int32),
                ("tie_break", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("phi", ctypes.c_double)]


class MoeError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {_lib.moe_status_string(status).decode()}")


_vp, _sz, _i64p = ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(ctypes.c_int64)
_SP = ctypes.POINTER(MoeShape)
_lib.moe_status_string.restype = ctypes.c_char_p
_lib.moe_status_string.argtypes = [ctypes.c_int]
_lib.moe_capacity.argtypes = [_SP, _i64p, _i64p]
_lib.moe_workspace_bytes.argtypes = [_SP, ctypes.POINTER(_sz)]
_lib.moe_route.argtypes = [_SP] + [_vp] * 6 + [_vp, _sz, _vp]
_lib.moe_permute.argtypes = [_SP] + [_vp] * 8 + [_vp, _sz, _vp]
_lib.moe_expert_ffn.argtypes = [_SP] + [_vp] * 6 + [_vp, _sz, _vp]
_lib.moe_combine.argtypes = [_SP] + [_vp] * 5 + [_vp]
_lib.moe_layer_forward.argtypes = [_SP] + [_vp] * 14 + [_vp, _sz, _vp]
_lib.moe_layer_forward_noalloc.argtypes = [_SP] + [_vp] * 14 + [_vp]
_lib.moe_layer_forward_timed.argtypes = [_SP] + [_vp] * 10 + [_vp, _sz, _vp, _vp, ctypes.c_int32]
_lib.moe_permute_padded.argtypes = [_SP] + [_vp] * 6 + [_vp, _sz, _vp]
_lib.moe_layer_forward_padded.argtypes = [_SP] + [_vp] * 14 + [_vp, _sz, _vp]
_lib.moe_permute_reroute.argtypes = [_SP] + [_vp] * 10 + [_vp, _sz, _vp]
_lib.moe_layer_forward_reroute.argtypes = [_SP] + [_vp] * 14 + [_vp, _sz, _vp]
_lib.moe_permute_expert_choice.argtypes = [_SP] + [_vp] * 7 + [_vp, _sz, _vp]
_lib.moe_layer_forward_expert_choice.argtypes = [_SP] + [_vp] * 12 + [_vp, _sz, _vp]
_lib.moe_routing_stats.argtypes = [_SP, _vp, _vp, _vp, ctypes.c_double, ctypes.c_int32, _vp, _vp,
                                   _vp, _sz, _vp]
_i64 = ctypes.c_int64
_lib.moe_workspace_bytes_queued.argtypes = [_SP, _i64, ctypes.POINTER(_sz)]
_lib.moe_layer_forward_queued.argtypes = [_SP] + [_vp] * 9 + [_i64] + [_vp] * 4 + [_i64] + \
    [_vp] * 11 + [_vp, _sz, _vp]
_lib.moe_layer_forward_queued_timed.argtypes = [_SP] + [_vp] * 9 + [_i64] + [_vp] * 4 + \
    [_vp] * 7 + [_vp, _sz, _vp, _vp]
for _n in EXPORTS[1:]:
    getattr(_lib, _n).restype = ctypes.c_int


def shape(T, d, E, k, d_ff, d_ff_shared=0, dtype="bf16", renorm=1, phi=0.0):
    """Build the C moe_shape struct."""
    dt = {"bf16": DTYPE_BF16, torch.bfloat16: DTYPE_BF16, "f32": DTYPE_F32,
          torch.float32: DTYPE_F32}[dtype]
    return MoeShape(int(T), int(d), int(E), int(k), int(d_ff), int(d_ff_shared), dt,
                    int(renorm), 0, 0, float(phi))


def shape_of(w):
    """moe_shape of a workloads.Workload."""
    return shape(w.T, w.d, w.E, w.k, w.d_ff, w.d_ff_shared, w.dtype, w.renorm, w.phi)


def _tdtype(s):
    return torch.bfloat16 if s.dtype == DTYPE_BF16 else torch.float32


def _check(status, where):
    if status != MOE_OK:
        raise MoeError(status, where)


def _ptr(t, name, shp=None, dtype=None, device=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shp is not None and tuple(t.shape) != tuple(shp):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shp)}")
    if t.numel() == 0:
        return None
    return t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def capacity(s):
    """(C, R_max): C = -1 without a capacity limit."""
    C, R = ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.moe_capacity(ctypes.byref(s), ctypes.byref(C), ctypes.byref(R)), "moe_capacity")
    return C.value, R.value


def workspace_bytes(s):
    n = _sz()
    _check(_lib.moe_workspace_bytes(ctypes.byref(s), ctypes.byref(n)), "moe_workspace_bytes")
    return n.value


def workspace(s, device="cuda"):
    """A device byte tensor of moe_workspace_bytes (torch allocations are 256-byte aligned)."""
    return torch.empty(workspace_bytes(s), dtype=torch.uint8, device=device)


def _ws(s, ws, device):
    if ws is None:
        ws = workspace(s, device)
    _ptr(ws, "ws", dtype=torch.uint8)
    return ws


def route(s, x, w_router, b_router=None, logits=None, ws=None, stream=None, want_logits=False):
    """Router logits, top-k ids and gates.  Returns (expert_ids, gates, logits-or-None)."""
    dt = _tdtype(s)
    dev = x.device
    xp = _ptr(x, "x", (s.T, s.d), dt)
    wp = _ptr(w_router, "w_router", (s.E, s.d), dt)
    bp = _ptr(b_router, "b_router", (s.E,), torch.float32, optional=True)
    if logits is None and want_logits:
        logits = torch.empty(s.T, s.E, dtype=torch.float32, device=dev)
    lp = _ptr(logits, "logits", (s.T, s.E), torch.float32, optional=True)
    ids = torch.empty(s.T, s.k, dtype=torch.int32, device=dev)
    gates = torch.empty(s.T, s.k, dtype=torch.float32, device=dev)
    ws = _ws(s, ws, dev)
    _check(_lib.moe_route(ctypes.byref(s), xp, wp, bp, lp, ids.data_ptr() if ids.numel() else None,
                          gates.data_ptr() if gates.numel() else None, ws.data_ptr(), ws.numel(),
                          _stream(stream)), "moe_route")
    return ids, gates, logits


def permute(s, x, expert_ids, ws=None, stream=None):
    """Counting-sort dispatch.  Returns dict(counts, kept_counts, offsets,
    route_pos, row_token, x_packed); row_token / x_packed have R_max rows, of
    which the first offsets[E] are written."""
    dt = _tdtype(s)
    dev = x.device
    _, R_max = capacity(s)
    xp = _ptr(x, "x", (s.T, s.d), dt)
    ip = _ptr(expert_ids, "expert_ids", (s.T, s.k), torch.int32)
    out = dict(counts=torch.empty(s.E, dtype=torch.int32, device=dev),
               kept_counts=torch.empty(s.E, dtype=torch.int32, device=dev),
               offsets=torch.empty(s.E + 1, dtype=torch.int32, device=dev),
               route_pos=torch.empty(s.T, s.k, dtype=torch.int32, device=dev),
               row_token=torch.empty(max(R_max, 1), dtype=torch.int32, device=dev),
               x_packed=torch.empty(max(R_max, 1), s.d, dtype=dt, device=dev))
    ws = _ws(s, ws, dev)
    _check(_lib.moe_permute(ctypes.byref(s), xp, ip, out["counts"].data_ptr(),
                            out["kept_counts"].data_ptr(), out["offsets"].data_ptr(),
                            _ptr(out["route_pos"], "route_pos"), out["row_token"].data_ptr(),
                            out["x_packed"].data_ptr(), ws.data_ptr(), ws.numel(),
                            _stream(stream)), "moe_permute")
    return out


def permute_padded(s, x, expert_ids, ws=None, stream=None):
    """Dispatch into the fixed-shape buffer [E, C, d].  Returns dict(counts,
    kept_counts, route_pos (rows e*C + slot, -1 dropped), x_padded [E*C, d])."""
    dt = _tdtype(s)
    dev = x.device
    C, _ = capacity(s)
    if C <= 0:
        raise ValueError("the fixed-shape buffer needs a capacity (phi > 0)")
    xp = _ptr(x, "x", (s.T, s.d), dt)
    ip = _ptr(expert_ids, "expert_ids", (s.T, s.k), torch.int32)
    out = dict(counts=torch.empty(s.E, dtype=torch.int32, device=dev),
               kept_counts=torch.empty(s.E, dtype=torch.int32, device=dev),
               route_pos=torch.empty(s.T, s.k, dtype=torch.int32, device=dev),
               x_padded=torch.empty(s.E * C, s.d, dtype=dt, device=dev))
    ws = _ws(s, ws, dev)
    _check(_lib.moe_permute_padded(ctypes.byref(s), xp, ip, out["counts"].data_ptr(),
                                   out["kept_counts"].data_ptr(), _ptr(out["route_pos"], "route_pos"),
                                   out["x_padded"].data_ptr(), ws.data_ptr(), ws.numel(),
                                   _stream(stream)), "moe_permute_padded")
    return out


def permute_reroute(s, x, logits, expert_ids, ws=None, stream=None):
    """Dispatch with the reroute overflow policy.  Returns dict(expert_ids
    (after rerouting), counts (demand), filled, offsets, route_pos, row_token,
    x_packed)."""
    dt = _tdtype(s)
    dev = x.device
    _, R_max = capacity(s)
    xp = _ptr(x, "x", (s.T, s.d), dt)
    lp = _ptr(logits, "logits", (s.T, s.E), torch.float32)
    ip = _ptr(expert_ids, "expert_ids", (s.T, s.k), torch.int32)
    out = dict(expert_ids=torch.empty(s.T, s.k, dtype=torch.int32, device=dev),
               counts=torch.empty(s.E, dtype=torch.int32, device=dev),
               filled=torch.empty(s.E, dtype=torch.int32, device=dev),
               offsets=torch.empty(s.E + 1, dtype=torch.int32, device=dev),
               route_pos=torch.empty(s.T, s.k, dtype=torch.int32, device=dev),
               row_token=torch.empty(max(R_max, 1), dtype=torch.int32, device=dev),
               x_packed=torch.empty(max(R_max, 1), s.d, dtype=dt, device=dev))
    ws = _ws(s, ws, dev)
    _check(_lib.moe_permute_reroute(ctypes.byref(s), xp, lp, ip,
                                    _ptr(out["expert_ids"], "expert_ids_out"),
                                    out["counts"].data_ptr(), out["filled"].data_ptr(),
                                    out["offsets"].data_ptr(), _ptr(out["route_pos"], "route_pos"),
                                    out["row_token"].data_ptr(), out["x_packed"].data_ptr(),
                                    ws.data_ptr(), ws.numel(), _stream(stream)),
           "moe_permute_reroute")
    return out


def choice_capacity(s):
    """Tokens every expert keeps under expert-choice routing: min(C, T)."""
    C, _ = capacity(s)
    return max(0, min(C, s.T))


def permute_expert_choice(s, x, logits, ws=None, stream=None):
    """Expert-choice dispatch.  Returns dict(scores [T, E], route_pos [T, E],
    offsets [E+1], row_token [E*Ce], x_packed [E*Ce, d])."""
    dt = _tdtype(s)
    dev = x.device
    Ce = choice_capacity(s)
    xp = _ptr(x, "x", (s.T, s.d), dt)
    lp = _ptr(logits, "logits", (s.T, s.E), torch.float32)
    out = dict(scores=torch.empty(s.T, s.E, dtype=torch.float32, device=dev),
               route_pos=torch.empty(s.T, s.E, dtype=torch.int32, device=dev),
               offsets=torch.empty(s.E + 1, dtype=torch.int32, device=dev),
               row_token=torch.empty(max(s.E * Ce, 1), dtype=torch.int32, device=dev),
               x_packed=torch.empty(max(s.E * Ce, 1), s.d, dtype=dt, device=dev))
    ws = _ws(s, ws, dev)
    _check(_lib.moe_permute_expert_choice(ctypes.byref(s), xp, lp, _ptr(out["scores"], "scores"),
                                          _ptr(out["route_pos"], "route_pos"),
                                          out["offsets"].data_ptr(), out["row_token"].data_ptr(),
                                          out["x_packed"].data_ptr(), ws.data_ptr(), ws.numel(),
                                          _stream(stream)), "moe_permute_expert_choice")
    out["row_token"] = out["row_token"][:s.E * Ce]
    out["x_packed"] = out["x_packed"][:s.E * Ce]
    return out


def layer_forward_expert_choice(s, x, w_router, b_router, w_gate, w_up, w_down, ws_gate=None,
                                ws_up=None, ws_down=None, y=None, ws=None, stream=None,
                                return_routing=False):
    """Whole MoE layer under expert-choice routing.  Returns y, or (y,
    dict(scores [T, E], route_pos [T, E])) with return_routing."""
    dt = _tdtype(s)
    dev = x.device
    shp = s.d_ff_shared > 0
    args = (_ptr(x, "x", (s.T, s.d), dt), _ptr(w_router, "w_router", (s.E, s.d), dt),
            _ptr(b_router, "b_router", (s.E,), torch.float32, optional=True),
            _ptr(w_gate, "w_gate", (s.E, s.d_ff, s.d), dt),
            _ptr(w_up, "w_up", (s.E, s.d_ff, s.d), dt),
            _ptr(w_down, "w_down", (s.E, s.d, s.d_ff), dt),
            _ptr(ws_gate, "ws_gate", (s.d_ff_shared, s.d), dt, optional=not shp),
            _ptr(ws_up, "ws_up", (s.d_ff_shared, s.d), dt, optional=not shp),
            _ptr(ws_down, "ws_down", (s.d, s.d_ff_shared), dt, optional=not shp))
    if y is None:
        y = torch.empty(s.T, s.d, dtype=dt, device=dev)
    yo = _ptr(y, "y", (s.T, s.d), dt)
    routing = None
    scp = rpp = None
    if return_routing:
        routing = dict(scores=torch.empty(s.T, s.E, dtype=torch.float32, device=dev),
                       route_pos=torch.empty(s.T, s.E, dtype=torch.int32, device=dev))
        scp = _ptr(routing["scores"], "scores")
        rpp = _ptr(routing["route_pos"], "route_pos")
    ws = _ws(s, ws, dev)
    _check(_lib.moe_layer_forward_expert_choice(ctypes.byref(s), *args, yo, scp, rpp,
                                                ws.data_ptr(), ws.numel(), _stream(stream)),
           "moe_layer_forward_expert_choice")
    return (y, routing) if return_routing else y


def expert_ffn(s, x_packed, offsets, w_gate, w_up, w_down, y_packed=None, ws=None, stream=None):
    """Grouped SwiGLU expert FFN over packed rows.  Returns y_packed [R_max, d]."""
    dt = _tdtype(s)
    dev = x_packed.device
    xp = _ptr(x_packed, "x_packed", dtype=dt)
    if x_packed.dim() != 2 or x_packed.shape[1] != s.d:
        raise ValueError("x_packed must be [rows, d]")
    op = _ptr(offsets, "offsets", (s.E + 1,), torch.int32)
    gp = _ptr(w_gate, "w_gate", (s.E, s.d_ff, s.d), dt)
    up = _ptr(w_up, "w_up", (s.E, s.d_ff, s.d), dt)
    dp = _ptr(w_down, "w_down", (s.E, s.d, s.d_ff), dt)
    if y_packed is None:
        y_packed = torch.empty(x_packed.shape[0], s.d, dtype=dt, device=dev)
    yp = _ptr(y_packed, "y_packed", (x_packed.shape[0], s.d), dt)
    ws = _ws(s, ws, dev)
    _check(_lib.moe_expert_ffn(ctypes.byref(s), xp, op, gp, up, dp, yp, ws.data_ptr(), ws.numel(),
                               _stream(stream)), "moe_expert_ffn")
    return y_packed


def combine(s, y_packed, route_pos, gates, y_shared=None, y=None, stream=None):
    """Gate-weighted un-permute (+ shared expert rows).  Returns y [T, d]."""
    dt = _tdtype(s)
    dev = y_packed.device
    yp = _ptr(y_packed, "y_packed", dtype=dt)
    rp = _ptr(route_pos, "route_pos", (s.T, s.k), torch.int32)
    gp = _ptr(gates, "gates", (s.T, s.k), torch.float32)
    sp = _ptr(y_shared, "y_shared", (s.T, s.d), dt, optional=True)
    if y is None:
        y = torch.empty(s.T, s.d, dtype=dt, device=dev)
    op = _ptr(y, "y", (s.T, s.d), dt)
    _check(_lib.moe_combine(ctypes.byref(s), yp, rp, gp, sp, op, _stream(stream)), "moe_combine")
    return y


STAT_NAMES = ("aux_loss", "load_imbalance", "mean_max_gate", "mean_norm_entropy",
              "js_to_uniform", "mean_confidence")


def routing_stats(s, logits, gates, counts, alpha=1e-2, n_bins=20, ws=None, stream=None,
                  out=None):
    """moe_routing_stats.  Returns (stats [6 + 2E] fp32, hist [n_bins] int32)
    device tensors; stats_dict() turns them into named values."""
    dev = counts.device
    lp = _ptr(logits, "logits", (s.T, s.E), torch.float32, optional=s.T == 0)
    gp = _ptr(gates, "gates", (s.T, s.k), torch.float32, optional=s.T == 0)
    cp = _ptr(counts, "counts", (s.E,), torch.int32)
    if out is None:
        out = (torch.empty(6 + 2 * s.E, dtype=torch.float32, device=dev),
               torch.empty(int(n_bins), dtype=torch.int32, device=dev))
    st, hist = out
    ws = _ws(s, ws, dev)
    _check(_lib.moe_routing_stats(ctypes.byref(s), lp, gp, cp, float(alpha), int(n_bins),
                                  _ptr(st, "stats", (6 + 2 * s.E,), torch.float32),
                                  _ptr(hist, "hist", (int(n_bins),), torch.int32),
                                  ws.data_ptr(), ws.numel(), _stream(stream)), "moe_routing_stats")
    return st, hist


def stats_dict(s, stats, hist):
    """Named host copies of the routing_stats outputs."""
    v = stats.detach().cpu().double().numpy()
    res = dict(zip(STAT_NAMES, v[:6].tolist()))
    res.update(share=v[6:6 + s.E], mean_prob=v[6 + s.E:6 + 2 * s.E],
               hist=hist.detach().cpu().numpy().astype("int64"))
    return res


def layer_forward(s, x, w_router, b_router, w_gate, w_up, w_down, ws_gate=None, ws_up=None,
                  ws_down=None, y=None, ws=None, stream=None, return_routing=False, padded=False,
                  reroute=False):
    """Whole MoE layer.  Returns y, or (y, dict(expert_ids, gates, counts,
    route_pos)) with return_routing.  padded=True runs moe_layer_forward_padded
    (fixed-shape [E, C, d] buffer; route_pos then holds its rows e*C + slot);
    reroute=True runs moe_layer_forward_reroute (expert_ids then holds the
    experts after rerouting)."""
    dt = _tdtype(s)
    dev = x.device
    xp = _ptr(x, "x", (s.T, s.d), dt)
    rp = _ptr(w_router, "w_router", (s.E, s.d), dt)
    bp = _ptr(b_router, "b_router", (s.E,), torch.float32, optional=True)
    gp = _ptr(w_gate, "w_gate", (s.E, s.d_ff, s.d), dt)
    up = _ptr(w_up, "w_up", (s.E, s.d_ff, s.d), dt)
    dp = _ptr(w_down, "w_down", (s.E, s.d, s.d_ff), dt)
    shp = s.d_ff_shared > 0
    sg = _ptr(ws_gate, "ws_gate", (s.d_ff_shared, s.d), dt, optional=not shp)
    su = _ptr(ws_up, "ws_up", (s.d_ff_shared, s.d), dt, optional=not shp)
    sd = _ptr(ws_down, "ws_down", (s.d, s.d_ff_shared), dt, optional=not shp)
    if y is None:
        y = torch.empty(s.T, s.d, dtype=dt, device=dev)
    yo = _ptr(y, "y", (s.T, s.d), dt)
    routing = None
    ip = gtp = cp = rpp = None
    if return_routing:
        routing = dict(expert_ids=torch.empty(s.T, s.k, dtype=torch.int32, device=dev),
                       gates=torch.empty(s.T, s.k, dtype=torch.float32, device=dev),
                       counts=torch.empty(s.E, dtype=torch.int32, device=dev),
                       route_pos=torch.empty(s.T, s.k, dtype=torch.int32, device=dev))
        ip = _ptr(routing["expert_ids"], "expert_ids")
        gtp = _ptr(routing["gates"], "gates")
        cp = _ptr(routing["counts"], "counts")
        rpp = _ptr(routing["route_pos"], "route_pos")
    ws = _ws(s, ws, dev)
    name = ("moe_layer_forward_padded" if padded else
            "moe_layer_forward_reroute" if reroute else "moe_layer_forward")
    _check(getattr(_lib, name)(ctypes.byref(s), xp, rp, bp, gp, up, dp, sg, su, sd, yo, ip, gtp,
                               cp, rpp, ws.data_ptr(), ws.numel(), _stream(stream)), name)
    return (y, routing) if return_routing else y


NOALLOC_SCRATCH_BYTES = 64 << 20


def layer_forward_noalloc(s, x, w_router, b_router, w_gate, w_up, w_down, ws_gate=None,
                          ws_up=None, ws_down=None, y=None, stream=None, return_routing=False):
    """moe_layer_forward_noalloc: the layer with the library's fixed device
    array as its workspace (no workspace tensor; calls overlapping on one
    GPU race).  Outputs as layer_forward; y may be passed in."""
    dt = _tdtype(s)
    dev = x.device
    args = _layer_args(s, x, w_router, b_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down)
    if y is None:
        y = torch.empty(s.T, s.d, dtype=dt, device=dev)
    yo = _ptr(y, "y", (s.T, s.d), dt)
    routing = None
    extra = [None] * 4
    if return_routing:
        routing = dict(expert_ids=torch.empty(s.T, s.k, dtype=torch.int32, device=dev),
                       gates=torch.empty(s.T, s.k, dtype=torch.float32, device=dev),
                       counts=torch.empty(s.E, dtype=torch.int32, device=dev),
                       route_pos=torch.empty(s.T, s.k, dtype=torch.int32, device=dev))
        extra = [_ptr(routing[n], n) for n in ("expert_ids", "gates", "counts", "route_pos")]
    _check(_lib.moe_layer_forward_noalloc(ctypes.byref(s), *args, yo, *extra, _stream(stream)),
           "moe_layer_forward_noalloc")
    return (y, routing) if return_routing else y


def layer_forward_timed(s, x, w_router, b_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down,
                        y, ws, events, stream=None, padded=False, reroute=False, choice=False):
    """moe_layer_forward_timed: records the 7 stage-boundary hipEvents
    (`events`: sequence of raw hipEvent_t handles as ints).  padded, reroute
    and choice select the layout (fixed [E, C, d] buffer, reroute overflow
    policy, expert-choice routing)."""
    dt = _tdtype(s)
    arr = (ctypes.c_void_p * 7)(*[ctypes.c_void_p(e) for e in events])
    shp = s.d_ff_shared > 0
    _check(_lib.moe_layer_forward_timed(
        ctypes.byref(s), _ptr(x, "x", (s.T, s.d), dt), _ptr(w_router, "w_router", (s.E, s.d), dt),
        _ptr(b_router, "b_router", (s.E,), torch.float32, optional=True),
        _ptr(w_gate, "w_gate", (s.E, s.d_ff, s.d), dt), _ptr(w_up, "w_up", (s.E, s.d_ff, s.d), dt),
        _ptr(w_down, "w_down", (s.E, s.d, s.d_ff), dt),
        _ptr(ws_gate, "ws_gate", (s.d_ff_shared, s.d), dt, optional=not shp),
        _ptr(ws_up, "ws_up", (s.d_ff_shared, s.d), dt, optional=not shp),
        _ptr(ws_down, "ws_down", (s.d, s.d_ff_shared), dt, optional=not shp),
        _ptr(y, "y", (s.T, s.d), dt), ws.data_ptr(), ws.numel(), _stream(stream), arr,
        1 if padded else 2 if reroute else 3 if choice else 0),
        "moe_layer_forward_timed")
    return y


def workspace_bytes_queued(s, q_n):
    n = _sz()
    _check(_lib.moe_workspace_bytes_queued(ctypes.byref(s), int(q_n), ctypes.byref(n)),
           "moe_workspace_bytes_queued")
    return n.value


def queue_buffers(s, q_n, device="cuda"):
    """Device buffers of one queued call with q_n waiting routes: y, y_late,
    the outgoing queue (capacity q_n + T*k) and its length, and the
    workspace."""
    dt = _tdtype(s)
    n = int(q_n) + s.T * s.k
    return dict(y=torch.empty(s.T, s.d, dtype=dt, device=device),
                y_late=torch.empty(int(q_n), s.d, dtype=dt, device=device),
                out_n=torch.zeros(1, dtype=torch.int32, device=device),
                out_x=torch.empty(n, s.d, dtype=dt, device=device),
                out_ids=torch.empty(n, dtype=torch.int32, device=device),
                out_gates=torch.empty(n, dtype=torch.float32, device=device),
                out_tags=torch.empty(n, dtype=torch.int64, device=device),
                ws=torch.empty(workspace_bytes_queued(s, q_n), dtype=torch.uint8, device=device))


def _queue_args(s, queue, dt):
    if queue is None:
        return 0, None, None, None, None
    qn = int(queue["ids"].shape[0])
    return (qn, _ptr(queue["x"], "queue x", (qn, s.d), dt),
            _ptr(queue["ids"], "queue ids", (qn,), torch.int32),
            _ptr(queue["gates"], "queue gates", (qn,), torch.float32),
            _ptr(queue["tags"], "queue tags", (qn,), torch.int64))


def _layer_args(s, x, w_router, b_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down):
    dt = _tdtype(s)
    shp = s.d_ff_shared > 0
    return [_ptr(x, "x", (s.T, s.d), dt), _ptr(w_router, "w_router", (s.E, s.d), dt),
            _ptr(b_router, "b_router", (s.E,), torch.float32, optional=True),
            _ptr(w_gate, "w_gate", (s.E, s.d_ff, s.d), dt),
            _ptr(w_up, "w_up", (s.E, s.d_ff, s.d), dt),
            _ptr(w_down, "w_down", (s.E, s.d, s.d_ff), dt),
            _ptr(ws_gate, "ws_gate", (s.d_ff_shared, s.d), dt, optional=not shp),
            _ptr(ws_up, "ws_up", (s.d_ff_shared, s.d), dt, optional=not shp),
            _ptr(ws_down, "ws_down", (s.d, s.d_ff_shared), dt, optional=not shp)]


def _out_args(s, b, qn, dt):
    n = qn + s.T * s.k
    return [_ptr(b["y"], "y", (s.T, s.d), dt), _ptr(b["y_late"], "y_late", (qn, s.d), dt),
            _ptr(b["out_n"], "out_n", (1,), torch.int32),
            _ptr(b["out_x"], "out_x", (n, s.d), dt),
            _ptr(b["out_ids"], "out_ids", (n,), torch.int32),
            _ptr(b["out_gates"], "out_gates", (n,), torch.float32),
            _ptr(b["out_tags"], "out_tags", (n,), torch.int64)]


def layer_forward_queued(s, x, w_router, b_router, w_gate, w_up, w_down, ws_gate=None,
                         ws_up=None, ws_down=None, queue=None, tag_base=0, bufs=None,
                         stream=None, return_routing=False, sync=True):
    """moe_layer_forward_queued (overflow policy "queue to the next
    micro-batch").  queue: dict(x [Q, d], ids [Q] int32, gates [Q] fp32,
    tags [Q] int64) of the routes waiting from the previous call, or None.
    Returns (y, y_late, out_queue) -- out_queue in the same form, cut to its
    length (one host synchronisation; with sync=False the full buffers are
    returned with out_queue["n"], a device int32) -- plus, with
    return_routing, dict(expert_ids, gates, counts, route_pos [Q + T*k])."""
    dt = _tdtype(s)
    dev = x.device
    qn, qx, qi, qg, qt = _queue_args(s, queue, dt)
    if bufs is None:
        bufs = queue_buffers(s, qn, dev)
    routing = None
    extra = [None] * 4
    if return_routing:
        routing = dict(expert_ids=torch.empty(s.T, s.k, dtype=torch.int32, device=dev),
                       gates=torch.empty(s.T, s.k, dtype=torch.float32, device=dev),
                       counts=torch.empty(s.E, dtype=torch.int32, device=dev),
                       route_pos=torch.empty(qn + s.T * s.k, dtype=torch.int32, device=dev))
        extra = [_ptr(routing[n], n) for n in ("expert_ids", "gates", "counts", "route_pos")]
    ws = bufs["ws"]
    _ptr(ws, "ws", dtype=torch.uint8)
    args = _layer_args(s, x, w_router, b_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down)
    _check(_lib.moe_layer_forward_queued(ctypes.byref(s), *args, qn, qx, qi, qg, qt,
                                         int(tag_base), *_out_args(s, bufs, qn, dt), *extra,
                                         ws.data_ptr(), ws.numel(), _stream(stream)),
           "moe_layer_forward_queued")
    out = dict(x=bufs["out_x"], ids=bufs["out_ids"], gates=bufs["out_gates"],
               tags=bufs["out_tags"], n=bufs["out_n"])
    if sync:
        n = int(bufs["out_n"].item())
        out = dict(x=out["x"][:n], ids=out["ids"][:n], gates=out["gates"][:n],
                   tags=out["tags"][:n])
    res = (bufs["y"], bufs["y_late"], out)
    return res + (routing,) if return_routing else res


def layer_forward_queued_timed(s, x, w_router, b_router, w_gate, w_up, w_down, ws_gate, ws_up,
                               ws_down, queue, bufs, events, stream=None):
    """moe_layer_forward_queued_timed: the queued layer with the 7
    stage-boundary hipEvents of layer_forward_timed."""
    dt = _tdtype(s)
    qn, qx, qi, qg, qt = _queue_args(s, queue, dt)
    arr = (ctypes.c_void_p * 7)(*[ctypes.c_void_p(e) for e in events])
    ws = bufs["ws"]
    args = _layer_args(s, x, w_router, b_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down)
    _check(_lib.moe_layer_forward_queued_timed(ctypes.byref(s), *args, qn, qx, qi, qg, qt,
                                               *_out_args(s, bufs, qn, dt), ws.data_ptr(),
                                               ws.numel(), _stream(stream), arr),
           "moe_layer_forward_queued_timed")
    return bufs["y"]
