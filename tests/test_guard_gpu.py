"""Overrun guards: every entry point of the C ABI, called on buffers that sit
at the front of larger allocations filled with a byte pattern.  After the
call the pattern must be intact

  - past the end of every output (y, y_late, ids, gates, logits, counts,
    offsets, route tables, packed rows, the outgoing queue, statistics),
  - past the end of the workspace,
  - in the rows of x_packed / row_token / y_packed at or past offsets[E]
    (the entry points leave those rows unwritten),

and, for moe_expert_ffn, the workspace bytes the call writes (found by
running it twice, over two different fill patterns: a byte it writes ends
equal in both runs, a byte it leaves keeps its fill) are exactly the hidden
rows below offsets[E] plus, when the down projection splits K, the same
rows of each fp32 partial plane.  The outputs themselves are checked
against the oracle elsewhere; here they only have to be finite where
written.
"""
import ctypes

import numpy as np
import pytest
import torch

from tests._gpu import say
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

PAT = 0x5A
PAT2 = 0xA5
GUARD = 4096  # bytes past every buffer


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU guard tests need a GPU"
    import routing_dispatch_expert_route_amd as m
    return m


class Guarded:
    """A device buffer of `shape` / `dtype` at the front of an allocation
    GUARD bytes longer, all of it filled with one byte value."""

    def __init__(self, shape, dtype, fill=PAT):
        n = int(np.prod(shape)) if len(shape) else 1
        self.nbytes = n * torch.empty(0, dtype=dtype).element_size()
        self.raw = torch.full((self.nbytes + GUARD,), fill, dtype=torch.uint8, device="cuda")
        self.fill = fill
        self.t = self.raw[:self.nbytes].view(dtype).view(shape)

    @property
    def ptr(self):
        return self.t.data_ptr()

    def tail_intact(self):
        return bool((self.raw[self.nbytes:] == self.fill).all().item())

    def rows_intact(self, first_row):
        """Bytes of rows [first_row, end) still hold the fill."""
        t = self.t
        per_row = self.nbytes // max(t.shape[0], 1)
        return bool((self.raw[first_row * per_row:self.nbytes] == self.fill).all().item())


def _lib(moe):
    return moe._lib


def _ws(moe, s, fill=PAT):
    return Guarded((moe.workspace_bytes(s),), torch.uint8, fill)


def _stream():
    return torch.cuda.current_stream().cuda_stream


CASES = {
    # capacity with drops, a shared expert, top-2
    "bf16_cap_shared": Workload("bf16_cap_shared", T=300, E=8, k=2, d=136, d_ff=72,
                                d_ff_shared=64, phi=0.8, bias="normal"),
    # top-1 without a shared expert: the down GEMM writes y itself
    "bf16_top1": Workload("bf16_top1", T=515, E=6, k=1, d=72, d_ff=40, renorm=0, phi=0.7,
                          bias="normal"),
    # few rows, long d_ff: the down projection splits K into fp32 planes
    "bf16_split": Workload("bf16_split", T=16, E=8, k=2, d=256, d_ff=2048, phi=1.0),
    "f32": Workload("f32", T=77, E=5, k=3, d=40, d_ff=24, dtype="f32", phi=0.8, bias="normal"),
    # beyond 64 experts (the reroute's wide walk, 256-byte rank rows)
    "bf16_e160": Workload("bf16_e160", T=400, E=160, k=4, d=64, d_ff=32, phi=0.8, bias="zipf"),
}


def _setup(moe, name):
    w = CASES[name]
    inp = make_inputs(w, seed=31)
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    return w, moe.shape_of(w), d


def _p(t):
    return None if t is None else t.data_ptr()


def _weights(d):
    return [_p(d[n]) for n in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")]


@pytest.mark.parametrize("name", list(CASES))
def test_route_permute_combine_guards(moe, name):
    w, s, d = _setup(moe, name)
    say(f"[guard route/permute/combine] {name}")
    L = _lib(moe)
    dt = w.torch_dtype
    T, E, k = w.T, w.E, w.k
    _, R_max = moe.capacity(s)
    ws = _ws(moe, s)
    logits = Guarded((T, E), torch.float32)
    ids = Guarded((T, k), torch.int32)
    gates = Guarded((T, k), torch.float32)
    st = L.moe_route(ctypes.byref(s), _p(d["x"]), _p(d["w_router"]), _p(d["b_router"]), logits.ptr,
                     ids.ptr, gates.ptr, ws.ptr, ws.nbytes, _stream())
    assert st == 0
    torch.cuda.synchronize()
    assert logits.tail_intact() and ids.tail_intact() and gates.tail_intact() and ws.tail_intact()

    counts = Guarded((E,), torch.int32)
    kept = Guarded((E,), torch.int32)
    offsets = Guarded((E + 1,), torch.int32)
    rpos = Guarded((T, k), torch.int32)
    rtok = Guarded((R_max,), torch.int32)
    xp = Guarded((R_max, w.d), dt)
    st = L.moe_permute(ctypes.byref(s), _p(d["x"]), ids.ptr, counts.ptr, kept.ptr, offsets.ptr,
                       rpos.ptr, rtok.ptr, xp.ptr, ws.ptr, ws.nbytes, _stream())
    assert st == 0
    torch.cuda.synchronize()
    n = int(offsets.t[-1].item())
    assert n <= R_max
    for g in (counts, kept, offsets, rpos, rtok, xp, ws):
        assert g.tail_intact()
    assert rtok.rows_intact(n) and xp.rows_intact(n), "rows past offsets[E] were written"

    # expert FFN on the packed rows: y_packed rows past offsets[E] untouched,
    # and the workspace bytes it writes are the hidden rows (+ partial planes)
    yps = []
    for fill in (PAT, PAT2):
        wsf = _ws(moe, s, fill)
        yp = Guarded((R_max, w.d), dt, fill)
        st = L.moe_expert_ffn(ctypes.byref(s), xp.ptr, offsets.ptr, *_weights(d)[:3], yp.ptr,
                              wsf.ptr, wsf.nbytes, _stream())
        assert st == 0
        torch.cuda.synchronize()
        assert yp.tail_intact() and wsf.tail_intact()
        assert yp.rows_intact(n), "y_packed rows past offsets[E] were written"
        yps.append((yp, wsf))
    same = int((yps[0][1].raw[:ws.nbytes] == yps[1][1].raw[:ws.nbytes]).sum().item())
    eb = torch.empty(0, dtype=dt).element_size()
    h_bytes = n * w.d_ff * eb
    extra = same - h_bytes
    plane = n * w.d * 4
    ok = extra == 0 or (plane > 0 and extra % plane == 0 and 2 <= extra // plane <= 8)
    assert ok, f"expert_ffn wrote {same} workspace bytes; hidden rows are {h_bytes}"
    assert torch.equal(yps[0][0].t[:n], yps[1][0].t[:n])  # independent of the workspace fill

    y = Guarded((T, w.d), dt)
    st = L.moe_combine(ctypes.byref(s), yps[0][0].ptr, rpos.ptr, gates.ptr, None, y.ptr, _stream())
    assert st == 0
    torch.cuda.synchronize()
    assert y.tail_intact()
    assert torch.isfinite(y.t.float()).all()
    say(f"   {name}: {n} of {R_max} packed rows, expert_ffn wrote {same} workspace bytes")


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("layout", ["packed", "padded", "reroute", "choice", "timed"])
def test_layer_guards(moe, name, layout):
    w, s, d = _setup(moe, name)
    if layout == "choice":
        w = w.with_(renorm=0)
        s = moe.shape_of(w)
    say(f"[guard layer] {name} {layout}")
    L = _lib(moe)
    dt = w.torch_dtype
    T, E, k = w.T, w.E, w.k
    ws = _ws(moe, s)
    y = Guarded((T, w.d), dt)
    args = [ctypes.byref(s), _p(d["x"]), _p(d["w_router"]), _p(d["b_router"])] + _weights(d)
    outs = []
    if layout == "choice":
        scores = Guarded((T, E), torch.float32)
        rpos = Guarded((T, E), torch.int32)
        outs = [scores, rpos]
        st = L.moe_layer_forward_expert_choice(*args, y.ptr, scores.ptr, rpos.ptr, ws.ptr,
                                               ws.nbytes, _stream())
    elif layout == "timed":
        arr = (ctypes.c_void_p * 7)()  # no events: every stage marker is skipped
        st = L.moe_layer_forward_timed(*args, y.ptr, ws.ptr, ws.nbytes, _stream(), arr, 0)
    else:
        ids = Guarded((T, k), torch.int32)
        gates = Guarded((T, k), torch.float32)
        counts = Guarded((E,), torch.int32)
        rpos = Guarded((T, k), torch.int32)
        outs = [ids, gates, counts, rpos]
        fn = {"packed": L.moe_layer_forward, "padded": L.moe_layer_forward_padded,
              "reroute": L.moe_layer_forward_reroute}[layout]
        st = fn(*args, y.ptr, ids.ptr, gates.ptr, counts.ptr, rpos.ptr, ws.ptr, ws.nbytes,
                _stream())
    assert st == 0, moe.MoeError(st, layout)
    torch.cuda.synchronize()
    for g in [y, ws] + outs:
        assert g.tail_intact(), f"{layout}: a write past the end of a buffer"
    assert torch.isfinite(y.t.float()).all()


@pytest.mark.parametrize("name", list(CASES))
def test_padded_reroute_choice_permute_guards(moe, name):
    w, s, d = _setup(moe, name)
    say(f"[guard permute variants] {name}")
    L = _lib(moe)
    dt = w.torch_dtype
    T, E, k = w.T, w.E, w.k
    C, R_max = moe.capacity(s)
    ws = _ws(moe, s)
    ids, gates, logits = moe.route(s, d["x"], d["w_router"], d["b_router"], want_logits=True)
    torch.cuda.synchronize()

    counts, kept = Guarded((E,), torch.int32), Guarded((E,), torch.int32)
    rpos = Guarded((T, k), torch.int32)
    xpad = Guarded((E * C, w.d), dt)
    st = L.moe_permute_padded(ctypes.byref(s), _p(d["x"]), _p(ids), counts.ptr, kept.ptr, rpos.ptr,
                              xpad.ptr, ws.ptr, ws.nbytes, _stream())
    assert st == 0
    torch.cuda.synchronize()
    for g in (counts, kept, rpos, xpad, ws):
        assert g.tail_intact()

    ids_out = Guarded((T, k), torch.int32)
    counts, filled = Guarded((E,), torch.int32), Guarded((E,), torch.int32)
    offsets, rpos = Guarded((E + 1,), torch.int32), Guarded((T, k), torch.int32)
    rtok, xp = Guarded((R_max,), torch.int32), Guarded((R_max, w.d), dt)
    st = L.moe_permute_reroute(ctypes.byref(s), _p(d["x"]), _p(logits), _p(ids), ids_out.ptr,
                               counts.ptr, filled.ptr, offsets.ptr, rpos.ptr, rtok.ptr, xp.ptr,
                               ws.ptr, ws.nbytes, _stream())
    assert st == 0
    torch.cuda.synchronize()
    n = int(offsets.t[-1].item())
    for g in (ids_out, counts, filled, offsets, rpos, rtok, xp, ws):
        assert g.tail_intact()
    assert rtok.rows_intact(n) and xp.rows_intact(n)

    wc = w.with_(renorm=0)
    sc = moe.shape_of(wc)
    Ce = moe.choice_capacity(sc)
    wsc = _ws(moe, sc)
    scores, rpos = Guarded((T, E), torch.float32), Guarded((T, E), torch.int32)
    offsets, rtok = Guarded((E + 1,), torch.int32), Guarded((E * Ce,), torch.int32)
    xp = Guarded((E * Ce, w.d), dt)
    st = L.moe_permute_expert_choice(ctypes.byref(sc), _p(d["x"]), _p(logits), scores.ptr,
                                     rpos.ptr, offsets.ptr, rtok.ptr, xp.ptr, wsc.ptr, wsc.nbytes,
                                     _stream())
    assert st == 0
    torch.cuda.synchronize()
    for g in (scores, rpos, offsets, rtok, xp, wsc):
        assert g.tail_intact()

    stats = Guarded((6 + 2 * E,), torch.float32)
    hist = Guarded((20,), torch.int32)
    st = L.moe_routing_stats(ctypes.byref(s), _p(logits), _p(gates), counts.ptr, 1e-2,
                             20, stats.ptr, hist.ptr, ws.ptr, ws.nbytes, _stream())
    assert st == 0
    torch.cuda.synchronize()
    assert stats.tail_intact() and hist.tail_intact() and ws.tail_intact()


@pytest.mark.parametrize("name", list(CASES))
def test_queued_guards(moe, name):
    w, s, d = _setup(moe, name)
    say(f"[guard queued] {name}")
    L = _lib(moe)
    dt = w.torch_dtype
    T, E, k = w.T, w.E, w.k
    # first call: no queue; its outgoing queue feeds the second call
    queue = None
    for call in range(2):
        qn = 0 if queue is None else int(queue["ids"].shape[0])
        N = qn + T * k
        wsq = Guarded((moe.workspace_bytes_queued(s, qn),), torch.uint8)
        y, y_late = Guarded((T, w.d), dt), Guarded((qn, w.d), dt)
        out_n = Guarded((1,), torch.int32)
        out_x, out_ids = Guarded((N, w.d), dt), Guarded((N,), torch.int32)
        out_g, out_t = Guarded((N,), torch.float32), Guarded((N,), torch.int64)
        ids, gates = Guarded((T, k), torch.int32), Guarded((T, k), torch.float32)
        counts, rpos = Guarded((E,), torch.int32), Guarded((N,), torch.int32)
        q = [None] * 4 if queue is None else [_p(queue[n]) for n in ("x", "ids", "gates", "tags")]
        st = L.moe_layer_forward_queued(
            ctypes.byref(s), _p(d["x"]), _p(d["w_router"]), _p(d["b_router"]), *_weights(d), qn,
            *q, 1000 * call, y.ptr, y_late.ptr if qn else None, out_n.ptr, out_x.ptr,
            out_ids.ptr, out_g.ptr, out_t.ptr, ids.ptr, gates.ptr, counts.ptr, rpos.ptr, wsq.ptr,
            wsq.nbytes, _stream())
        assert st == 0
        torch.cuda.synchronize()
        nq = int(out_n.t[0].item())
        for g in (wsq, y, y_late, out_n, out_x, out_ids, out_g, out_t, ids, gates, counts, rpos):
            assert g.tail_intact(), f"call {call}: a write past the end of a buffer"
        assert out_x.rows_intact(nq) and out_ids.rows_intact(nq), "queue rows past out_n written"
        queue = dict(x=out_x.t[:nq].clone(), ids=out_ids.t[:nq].clone(),
                     gates=out_g.t[:nq].clone(), tags=out_t.t[:nq].clone())
        say(f"   {name} call {call}: {qn} in, {nq} out")
