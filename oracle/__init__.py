"""Plain CPU oracle for the MoE layer forward pass (ctypes binding).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library (routing_dispatch_expert_route_amd) and does not import
it.  The arithmetic lives in oracle.c; this module only marshals arrays.

Arrays are numpy arrays: float32 for dtype "f32", uint16 bit patterns for
dtype "bf16" (torch bf16 tensors can be passed directly; they are viewed as
uint16 without conversion).

Parity status: every function is pinned by tests/test_oracle_pins.py against
the pages' worked values, closed forms, invariants, library routines or
brute force (see that file); none is "parity unpinned".
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_ORACLE_LIB names another build of oracle.c (the mutation check of the
# pins loads deliberately broken copies through it)
_LIB_PATH = os.environ.get("MOE_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16, F64 = 0, 1, 2

_i64 = ctypes.c_int64
_int = ctypes.c_int
_dbl = ctypes.c_double
_vp = ctypes.c_void_p


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from oracle import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_capacity.restype = _i64
        L.oracle_capacity.argtypes = [_i64, _i64, _i64, _dbl]
        L.oracle_router_logits.restype = None
        L.oracle_router_logits.argtypes = [_i64, _i64, _i64, _int, _vp, _vp, _vp, _vp]
        L.oracle_router_logits_f64.restype = None
        L.oracle_router_logits_f64.argtypes = [_i64, _i64, _i64, _int, _vp, _vp, _vp, _vp]
        L.oracle_topk_gates.restype = None
        L.oracle_topk_gates.argtypes = [_i64, _i64, _i64, _int, _vp, _vp, _vp]
        L.oracle_dispatch.restype = None
        L.oracle_dispatch.argtypes = [_i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]
        L.oracle_gather_rows.restype = None
        L.oracle_gather_rows.argtypes = [_i64, _i64, _i64, _vp, _vp, _vp]
        L.oracle_swiglu_rows.restype = None
        L.oracle_swiglu_rows.argtypes = [_i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp]
        L.oracle_expert_ffn.restype = None
        L.oracle_expert_ffn.argtypes = [_i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp]
        L.oracle_combine.restype = None
        L.oracle_combine.argtypes = [_i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp]
        L.oracle_dispatch_padded.restype = None
        L.oracle_dispatch_padded.argtypes = [_i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp]
        L.oracle_dispatch_reroute.restype = None
        L.oracle_dispatch_reroute.argtypes = [_i64, _i64, _i64, _i64] + [_vp] * 9
        L.oracle_dispatch_queue.restype = _i64
        L.oracle_dispatch_queue.argtypes = [_i64] * 5 + [_vp] * 8
        L.oracle_expert_choice.restype = None
        L.oracle_expert_choice.argtypes = [_i64, _i64, _i64, _vp, _vp, _vp, _vp]
        L.oracle_layer_forward_expert_choice.restype = _int
        L.oracle_layer_forward_expert_choice.argtypes = [_i64] * 5 + [_int, _i64] + [_vp] * 9 + \
            [_i64, _vp, _vp, _vp, _vp]
        L.oracle_routing_stats.restype = None
        L.oracle_routing_stats.argtypes = [_i64, _i64, _i64, _vp, _vp, _vp, _dbl, ctypes.c_int32,
                                           _vp, _vp, _vp, _vp]
        L.oracle_layer_forward.restype = _int
        L.oracle_layer_forward.argtypes = [_i64] * 6 + [_int, _int, _dbl] + [_vp] * 9 + \
            [_i64, _vp, _vp, _vp, _vp, _vp, _vp]
        _lib = L
    return _lib


def as_array(a):
    """Return (contiguous numpy array, dtype code) for a float32 / bf16 input.

    torch tensors are accepted (CPU); bf16 is passed as its raw 16-bit
    patterns.  float64 arrays get code F64 (only oracle_combine takes those).
    """
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous()
            if a.dtype == torch.bfloat16:
                return a.view(torch.int16).numpy().view(np.uint16), BF16
            a = a.numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    if a.dtype == np.float64:
        return a, F64
    raise TypeError(f"unsupported array dtype {a.dtype}")


def _p(a):
    return None if a is None else a.ctypes.data_as(_vp)


def capacity(T, E, k, phi):
    """C = ceil(phi*T*k/E), or -1 for no limit (phi <= 0)."""
    return int(lib().oracle_capacity(T, E, k, float(phi)))


def router_logits(x, w, b=None, f64=False):
    xa, dt = as_array(x)
    wa, dt2 = as_array(w)
    assert dt == dt2
    T, d = xa.shape
    E = wa.shape[0]
    ba = None if b is None else np.ascontiguousarray(as_array(b)[0], dtype=np.float32)
    out = np.empty((T, E), dtype=np.float64 if f64 else np.float32)
    fn = lib().oracle_router_logits_f64 if f64 else lib().oracle_router_logits
    fn(T, d, E, dt, _p(xa), _p(wa), _p(ba), _p(out))
    return out


def topk_gates(logits, k, renorm):
    la = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = la.shape
    ids = np.empty((T, k), dtype=np.int32)
    gates = np.empty((T, k), dtype=np.float32)
    lib().oracle_topk_gates(T, E, k, int(renorm), _p(la), _p(ids), _p(gates))
    return ids, gates


def dispatch(expert_ids, E, C):
    """Returns dict(counts, kept, offsets, route_pos, row_token)."""
    ids = np.ascontiguousarray(expert_ids, dtype=np.int32)
    T, k = ids.shape
    counts = np.empty(E, np.int32)
    kept = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    route_pos = np.empty(T * k, np.int32)
    row_token = np.full(max(T * k, 1), -1, np.int32)
    lib().oracle_dispatch(T, E, k, int(C), _p(ids), _p(counts), _p(kept), _p(offsets),
                          _p(route_pos), _p(row_token))
    n = int(offsets[E])
    return dict(counts=counts, kept=kept, offsets=offsets,
                route_pos=route_pos.reshape(T, k), row_token=row_token[:n].copy())


def dispatch_padded(expert_ids, E, C):
    """Dispatch into the fixed [E, C] slot buffer.  Returns dict(pad_pos [T, k],
    slot_token [E, C] (-1 = empty slot)) plus the packed dispatch's fields."""
    ids = np.ascontiguousarray(expert_ids, dtype=np.int32)
    T, k = ids.shape
    d = dispatch(ids, E, C)
    pad_pos = np.empty(T * k, np.int32)
    slot_token = np.empty(max(E * C, 1), np.int32)
    rp = np.ascontiguousarray(d["route_pos"].reshape(-1), dtype=np.int32)
    lib().oracle_dispatch_padded(T, E, k, int(C), _p(ids), _p(rp), _p(d["offsets"]),
                                 _p(pad_pos), _p(slot_token))
    d.update(pad_pos=pad_pos.reshape(T, k), slot_token=slot_token[:E * C].reshape(E, C))
    return d


def dispatch_reroute(logits, expert_ids, E, C):
    """Drop-then-reroute dispatch.  Returns dict(ids, counts, filled, offsets,
    route_pos [T, k], row_token, n_rerouted)."""
    la = np.ascontiguousarray(logits, dtype=np.float32)
    ids = np.ascontiguousarray(expert_ids, dtype=np.int32)
    T, k = ids.shape
    ids_out = np.empty_like(ids)
    counts = np.empty(E, np.int32)
    filled = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    route_pos = np.empty(T * k, np.int32)
    row_token = np.full(max(T * k, 1), -1, np.int32)
    moved = np.zeros(1, np.int64)
    lib().oracle_dispatch_reroute(T, E, k, int(C), _p(la), _p(ids), _p(ids_out), _p(counts),
                                  _p(filled), _p(offsets), _p(route_pos), _p(row_token),
                                  _p(moved))
    n = int(offsets[E])
    return dict(ids=ids_out, counts=counts, filled=filled, offsets=offsets,
                route_pos=route_pos.reshape(T, k), row_token=row_token[:n].copy(),
                n_rerouted=int(moved[0]))


def dispatch_queue(expert_ids, E, C, q_ids=None):
    """Queue-to-the-next-micro-batch dispatch (see oracle_dispatch_queue).
    expert_ids [T, k] of this batch, q_ids [Q] of the routes queued before.
    Returns dict(counts, kept, offsets, pos [Q + T*k] over the arrivals,
    row_arrival [offsets[E]], out_arrival [n_out]) -- arrival a < Q is queued
    route a, arrival Q + r is route r of this batch."""
    ids = np.ascontiguousarray(expert_ids, dtype=np.int32)
    T, k = ids.shape
    qa = np.ascontiguousarray(np.zeros(0) if q_ids is None else q_ids, dtype=np.int32).reshape(-1)
    Q = qa.shape[0]
    N = Q + T * k
    counts = np.empty(E, np.int32)
    kept = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    pos = np.empty(max(N, 1), np.int32)
    row_arrival = np.full(max(N, 1), -1, np.int32)
    out_arrival = np.empty(max(N, 1), np.int32)
    n_out = lib().oracle_dispatch_queue(T, E, k, int(C), Q, _p(qa), _p(ids), _p(counts),
                                        _p(kept), _p(offsets), _p(pos), _p(row_arrival),
                                        _p(out_arrival))
    n = int(offsets[E])
    return dict(counts=counts, kept=kept, offsets=offsets, pos=pos[:N].copy(),
                row_arrival=row_arrival[:n].copy(), out_arrival=out_arrival[:int(n_out)].copy())


def layer_forward_queued(x, w_router, b_router, w_gate, w_up, w_down, k, renorm, phi,
                         queue=None, tag_base=0, ws_gate=None, ws_up=None, ws_down=None):
    """The layer under the queue policy, composed from the oracle's steps:
    route this batch, dispatch the arrivals (queued routes first), run the
    experts on the seated rows (a queued route's row is its own token row,
    carried in the queue), combine this batch's routes (plus the shared
    expert) into y, and each seated queued route into its own row of y_late
    (gate times expert output; zero when it waits again).
    queue: dict(x [Q, d], ids [Q], gates [Q], tags [Q]) or None.  The tag
    of this batch's token t is tag_base + t.
    Returns dict(y [T, d], y_late [Q, d] (float64), ids, gates, counts,
    pos, out=dict(x, ids, gates, tags) in arrival order)."""
    xa, dt = as_array(x)
    T, d = xa.shape
    L = router_logits(x, w_router, b_router)
    E = L.shape[1]
    ids, gates = topk_gates(L, k, renorm)
    C = capacity(T, E, k, phi)
    if queue is None:
        qx = np.zeros((0, d), xa.dtype)
        qids = np.zeros(0, np.int32)
        qg = np.zeros(0, np.float32)
        qt = np.zeros(0, np.int64)
    else:
        qx = as_array(queue["x"])[0].reshape(-1, d)
        qids = np.ascontiguousarray(queue["ids"], np.int32).reshape(-1)
        qg = np.ascontiguousarray(queue["gates"], np.float32).reshape(-1)
        qt = np.ascontiguousarray(queue["tags"], np.int64).reshape(-1)
    Q = qids.shape[0]
    dq = dispatch_queue(ids, E, C, qids)
    rows = np.concatenate([xa, qx.astype(xa.dtype)], axis=0)       # token rows, then queued rows
    a = dq["row_arrival"].astype(np.int64)
    src = np.where(a < Q, T + a, (a - Q) // k)
    yp = expert_ffn(gather_rows(rows, src), dq["offsets"], w_gate, w_up, w_down)
    ysh = None if ws_gate is None else swiglu_rows(x, ws_gate, ws_up, ws_down)
    pos = dq["pos"]
    y = combine(yp, pos[Q:].reshape(T, k), gates, ysh)
    y_late = combine(yp, pos[:Q].reshape(Q, 1), qg.reshape(Q, 1)) if Q else np.zeros((0, d))
    # the routes that wait again, in arrival order
    n_out = dq["out_arrival"].shape[0]
    out = dict(x=np.empty((n_out, d), xa.dtype), ids=np.empty(n_out, np.int32),
               gates=np.empty(n_out, np.float32), tags=np.empty(n_out, np.int64))
    for i, a in enumerate(dq["out_arrival"].tolist()):
        if a < Q:
            out["x"][i], out["ids"][i], out["gates"][i], out["tags"][i] = \
                rows[T + a], qids[a], qg[a], qt[a]
        else:
            r = a - Q
            out["x"][i], out["ids"][i], out["gates"][i], out["tags"][i] = \
                rows[r // k], ids.reshape(-1)[r], gates.reshape(-1)[r], tag_base + r // k
    return dict(y=y, y_late=y_late, ids=ids, gates=gates, counts=dq["counts"], pos=pos, C=C,
                out=out)


def expert_choice(logits, C):
    """Expert-choice routing (see oracle_expert_choice).  Returns dict(scores
    [T, E] fp32, route_pos [T, E], row_token [E*Ce], Ce)."""
    la = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = la.shape
    Ce = T if (C < 0 or C > T) else int(C)
    scores = np.empty((T, E), np.float32)
    route_pos = np.empty((T, E), np.int32)
    row_token = np.full(max(E * Ce, 1), -1, np.int32)
    lib().oracle_expert_choice(T, E, int(C), _p(la), _p(scores), _p(route_pos), _p(row_token))
    return dict(scores=scores, route_pos=route_pos, row_token=row_token[:E * Ce].copy(), Ce=Ce)


def gather_rows(x, row_token):
    xa, dt = as_array(x)
    rt = np.ascontiguousarray(row_token, dtype=np.int32)
    out = np.empty((rt.shape[0], xa.shape[1]), dtype=xa.dtype)
    lib().oracle_gather_rows(rt.shape[0], xa.shape[1], xa.itemsize, _p(xa), _p(rt), _p(out))
    return out


def swiglu_rows(x, wg, wu, wd):
    xa, dt = as_array(x)
    ga, _ = as_array(wg)
    ua, _ = as_array(wu)
    da, _ = as_array(wd)
    n, d = xa.shape
    d_ff = ga.shape[0]
    y = np.empty((n, d), np.float64)
    lib().oracle_swiglu_rows(n, d, d_ff, dt, _p(xa), _p(ga), _p(ua), _p(da), _p(y))
    return y


def expert_ffn(x_packed, offsets, w_gate, w_up, w_down):
    xa, dt = as_array(x_packed)
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    ga, _ = as_array(w_gate)
    ua, _ = as_array(w_up)
    da, _ = as_array(w_down)
    E, d_ff, d = ga.shape
    y = np.empty((int(off[E]), d), np.float64)
    lib().oracle_expert_ffn(E, d, d_ff, dt, _p(off), _p(xa), _p(ga), _p(ua), _p(da), _p(y))
    return y


def combine(y_packed, route_pos, gates, y_shared=None):
    ya, dt = as_array(y_packed)
    rp = np.ascontiguousarray(route_pos, dtype=np.int32)
    g = np.ascontiguousarray(gates, dtype=np.float32)
    T, k = g.shape
    d = ya.shape[1]
    sa = None
    if y_shared is not None:
        sa, dts = as_array(y_shared)
        assert dts == dt
    y = np.empty((T, d), np.float64)
    lib().oracle_combine(T, k, d, dt, _p(ya), _p(rp), _p(g), _p(sa), _p(y))
    return y


STAT_NAMES = ("aux_loss", "load_imbalance", "mean_max_gate", "mean_norm_entropy",
              "js_to_uniform", "mean_confidence")


def routing_stats(logits, gates, counts, alpha=1e-2, n_bins=20):
    """Forward-only routing statistics (see oracle_routing_stats).  Returns
    dict with the six scalars by name, share[E], mean_prob[E], hist[n_bins]."""
    la = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = la.shape
    ga = np.ascontiguousarray(gates, dtype=np.float32)
    k = ga.shape[1] if ga.ndim == 2 else max(1, ga.size // max(T, 1))
    ca = np.ascontiguousarray(counts, dtype=np.int32)
    out = np.zeros(6)
    share = np.zeros(E)
    mean_prob = np.zeros(E)
    hist = np.zeros(n_bins, np.int64)
    lib().oracle_routing_stats(T, E, k, _p(la), _p(ga), _p(ca), float(alpha), int(n_bins),
                               _p(out), _p(share), _p(mean_prob), _p(hist))
    res = dict(zip(STAT_NAMES, out.tolist()))
    res.update(share=share, mean_prob=mean_prob, hist=hist)
    return res


def layer_forward(x, w_router, b_router, w_gate, w_up, w_down, k, renorm, phi,
                  ws_gate=None, ws_up=None, ws_down=None, sel=None):
    """Whole-layer oracle.  Returns dict(y, ids, gates, counts, route_pos).

    y holds the rows of the tokens listed in sel (all tokens when None),
    in float64.
    """
    xa, dt = as_array(x)
    T, d = xa.shape
    ra, _ = as_array(w_router)
    E = ra.shape[0]
    ba = None if b_router is None else np.ascontiguousarray(as_array(b_router)[0], np.float32)
    ga, _ = as_array(w_gate)
    ua, _ = as_array(w_up)
    da, _ = as_array(w_down)
    d_ff = ga.shape[1]
    d_ffs = 0
    sga = sua = sda = None
    if ws_gate is not None:
        sga, _ = as_array(ws_gate)
        sua, _ = as_array(ws_up)
        sda, _ = as_array(ws_down)
        d_ffs = sga.shape[0]
    sela = None if sel is None else np.ascontiguousarray(sel, dtype=np.int32)
    n_sel = T if sela is None else sela.shape[0]
    y = np.empty((n_sel, d), np.float64)
    ids = np.empty((T, k), np.int32)
    gates = np.empty((T, k), np.float32)
    counts = np.empty(E, np.int32)
    route_pos = np.empty((T, k), np.int32)
    rc = lib().oracle_layer_forward(T, d, E, k, d_ff, d_ffs, dt, int(renorm), float(phi),
                                    _p(xa), _p(ra), _p(ba), _p(ga), _p(ua), _p(da),
                                    _p(sga), _p(sua), _p(sda), n_sel, _p(sela), _p(y),
                                    _p(ids), _p(gates), _p(counts), _p(route_pos))
    if rc != 0:
        raise ValueError("oracle_layer_forward: bad arguments")
    return dict(y=y, ids=ids, gates=gates, counts=counts, route_pos=route_pos)


def layer_forward_expert_choice(x, w_router, b_router, w_gate, w_up, w_down, C,
                                ws_gate=None, ws_up=None, ws_down=None, sel=None):
    """Whole-layer oracle under expert-choice routing with capacity C (C < 0:
    every expert takes every token).  Returns dict(y, scores, route_pos)."""
    xa, dt = as_array(x)
    T, d = xa.shape
    ra, _ = as_array(w_router)
    E = ra.shape[0]
    ba = None if b_router is None else np.ascontiguousarray(as_array(b_router)[0], np.float32)
    ga, _ = as_array(w_gate)
    ua, _ = as_array(w_up)
    da, _ = as_array(w_down)
    d_ff = ga.shape[1]
    d_ffs = 0
    sga = sua = sda = None
    if ws_gate is not None:
        sga, _ = as_array(ws_gate)
        sua, _ = as_array(ws_up)
        sda, _ = as_array(ws_down)
        d_ffs = sga.shape[0]
    sela = None if sel is None else np.ascontiguousarray(sel, dtype=np.int32)
    n_sel = T if sela is None else sela.shape[0]
    y = np.empty((n_sel, d), np.float64)
    scores = np.empty((T, E), np.float32)
    route_pos = np.empty((T, E), np.int32)
    rc = lib().oracle_layer_forward_expert_choice(
        T, d, E, d_ff, d_ffs, dt, int(C), _p(xa), _p(ra), _p(ba), _p(ga), _p(ua), _p(da),
        _p(sga), _p(sua), _p(sda), n_sel, _p(sela), _p(y), _p(scores), _p(route_pos))
    if rc != 0:
        raise ValueError("oracle_layer_forward_expert_choice: bad arguments")
    return dict(y=y, scores=scores, route_pos=route_pos)
