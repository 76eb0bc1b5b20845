"""GPU parity of expert-choice routing ("MoE Inference Visualized", "Why MoE
Matters for Infrastructure": the experts pick the tokens) --
moe_permute_expert_choice and moe_layer_forward_expert_choice -- against the
CPU oracle.

The choice is an integer result decided by fp32 scores that the two sides
compute with different exp and summation order (a few ulps apart).  So:
  - scores agree with the oracle's within 1e-6;
  - the GPU choice is exactly the top-Ce of the GPU's own scores, lower token
    first on equal scores (checked here with numpy's lexsort), Ce rows per
    expert in increasing token order, row_token / route_pos / x_packed
    consistent bit for bit;
  - it equals the oracle's choice, except for tokens whose oracle score lies
    within 2e-6 of that expert's boundary score (a near tie that rounding
    may order either way); such tokens are reported.
The layer output is held to the layer tolerances on the tokens whose choice
agrees with the oracle's (all of them when there is no near tie)."""
import numpy as np
import pytest
import torch

import oracle
from tests._gpu import bits, check_y, host_inputs, say, to_dev
from workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

NEAR = 2e-6


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    import routing_dispatch_expert_route_amd as m
    return m


def _np(t):
    return t if isinstance(t, np.ndarray) else t.detach().cpu().numpy()


def _dup_rows(inp, src=5, every=3):
    """x with every `every`-th row a copy of row `src`: identical logits, so
    identical scores on both sides -- exact ties that the rule must break."""
    out = dict(inp)
    x = inp["x"].clone()
    x[::every] = x[src]
    out["x"] = x
    return out


CASES = {
    "switch_phi1": (WORKLOADS["switch_phi1"], None),
    "switch_phi125": (WORKLOADS["switch_phi125"], None),
    "f32_ragged": (Workload("f32_ragged", T=77, E=5, k=3, d=40, d_ff=24, dtype="f32", phi=0.8,
                            renorm=0, bias="normal"), None),
    "full_capacity": (Workload("full_cap", T=100, E=4, k=2, d=64, d_ff=32, phi=10.0, renorm=0),
                      None),
    "cap_one": (Workload("cap_one", T=64, E=16, k=1, d=64, d_ff=64, phi=0.01, renorm=0), None),
    "dup_rows_ties": (Workload("dup_rows", T=300, E=8, k=2, d=64, d_ff=32, phi=1.0, renorm=0),
                      _dup_rows),
    "granite_1412": (WORKLOADS["granite_1412"].with_(name="granite_ec", renorm=0, phi=1.0), None),
    "e64_shared": (Workload("e64_shared", T=600, E=64, k=2, d=64, d_ff=32, d_ff_shared=48,
                            phi=1.25, renorm=0, bias="zipf"), None),
    "t16384_e32": (Workload("t16384", T=16384, E=32, k=8, d=64, d_ff=32, phi=1.0, renorm=0), None),
    "t32768_max": (Workload("t32768", T=32768, E=8, k=2, d=32, d_ff=16, phi=0.7, renorm=0,
                            bias="normal"), None),
    # long columns for the radix select: a ragged T, exact ties at the
    # boundary, a column of 131072 tokens
    "t32769_long": (Workload("t32769", T=32769, E=8, k=1, d=32, d_ff=16, phi=0.9, renorm=0,
                             bias="normal"), None),
    "dup_rows_long": (Workload("dup_long", T=40000, E=8, k=2, d=64, d_ff=32, phi=1.0, renorm=0),
                      _dup_rows),
    "t131072_e16": (Workload("t131072", T=131072, E=16, k=2, d=32, d_ff=16, phi=1.0, renorm=0,
                             bias="normal"), None),
    # the full-size MFMA-bound shapes under expert choice (the layer is
    # checked on sampled tokens)
    "granite_16384": (WORKLOADS["granite_16384"].with_(name="granite16k_ec", renorm=0, phi=1.0),
                      None),
    "mixtral_prefill": (WORKLOADS["mixtral_prefill"].with_(name="mixtral_ec", renorm=0, phi=1.0),
                        None),
}


def _inputs(name):
    w, fix = CASES[name]
    inp = host_inputs(name) if name in WORKLOADS else make_inputs(w, seed=23)
    if fix is not None:
        inp = fix(inp)
    return w, inp


def _ce(w):
    return min(oracle.capacity(w.T, w.E, w.k, w.phi), w.T)


def _check_choice(w, scores, route_pos, row_token, ref, name):
    """Returns the tokens whose choice differs from the oracle's (near ties)."""
    T, E = w.T, w.E
    Ce = _ce(w)
    S, P = _np(scores), _np(route_pos)
    assert np.max(np.abs(S - ref["scores"]), initial=0.0) <= 1e-6
    rt = _np(row_token)[:E * Ce]
    t_idx = np.arange(T)
    differ = set()
    for e in range(E):
        # the GPU's rows for e: Ce of them, increasing tokens, consistent tables
        taken = np.flatnonzero(P[:, e] >= 0)
        assert taken.size == Ce, (name, e, taken.size, Ce)
        assert P[taken, e].tolist() == list(range(e * Ce, (e + 1) * Ce))
        assert rt[e * Ce:(e + 1) * Ce].tolist() == taken.tolist()
        # exactly the top Ce of its own scores, lower token first on ties
        order = np.lexsort((t_idx, -S[:, e]))
        assert np.array_equal(np.sort(order[:Ce]), taken), (name, e)
        # against the oracle: equal but for near ties at the boundary
        mine = set(taken.tolist())
        theirs = set(np.flatnonzero(ref["route_pos"][:, e] >= 0).tolist())
        if mine != theirs:
            so = ref["scores"][:, e].astype(np.float64)
            thr = np.sort(so)[::-1][Ce - 1]
            for t in mine ^ theirs:
                assert abs(so[t] - thr) <= NEAR, (name, e, t, so[t], thr)
                differ.add(t)
    return differ


@pytest.mark.parametrize("name", list(CASES))
def test_permute_expert_choice_parity(moe, name):
    w, inp = _inputs(name)
    say(f"[permute expert choice] {name} T={w.T} E={w.E} Ce={_ce(w)}")
    d = to_dev(inp)
    s = moe.shape_of(w)
    _, _, logits = moe.route(s, d["x"], d["w_router"], d["b_router"], want_logits=True)
    out = moe.permute_expert_choice(s, d["x"], logits)
    torch.cuda.synchronize()
    L = oracle.router_logits(inp["x"], inp["w_router"], inp["b_router"])
    assert np.array_equal(bits(logits), L.view(np.int32))
    C = oracle.capacity(w.T, w.E, w.k, w.phi)
    ref = oracle.expert_choice(L, C)
    Ce = ref["Ce"]
    assert _np(out["offsets"]).tolist() == [e * Ce for e in range(w.E + 1)]
    differ = _check_choice(w, out["scores"], out["route_pos"], out["row_token"], ref, name)
    rt = _np(out["row_token"])
    assert np.array_equal(bits(out["x_packed"]), bits(inp["x"])[rt])
    say(f"   {name}: {len(differ)} near-tie tokens differ")


@pytest.mark.parametrize("name", [n for n in CASES
                                  if n not in ("t32768_max", "dup_rows_long", "t131072_e16")])
def test_layer_forward_expert_choice_parity(moe, name):
    w, inp = _inputs(name)
    say(f"[layer expert choice] {name}")
    d = to_dev(inp)
    s = moe.shape_of(w)
    y, rt = moe.layer_forward_expert_choice(s, d["x"], d["w_router"], d["b_router"], d["w_gate"],
                                            d["w_up"], d["w_down"], d["ws_gate"], d["ws_up"],
                                            d["ws_down"], return_routing=True)
    torch.cuda.synchronize()
    C = oracle.capacity(w.T, w.E, w.k, w.phi)
    L = oracle.router_logits(inp["x"], inp["w_router"], inp["b_router"])
    ref = oracle.expert_choice(L, C)
    Ce = ref["Ce"]
    rows = np.full(w.E * Ce, -1, np.int64)
    P = _np(rt["route_pos"])
    for e in range(w.E):
        rows[e * Ce:(e + 1) * Ce] = np.flatnonzero(P[:, e] >= 0)
    differ = _check_choice(w, rt["scores"], rt["route_pos"], rows, ref, name)
    rng = np.random.default_rng(3)
    # every token when the oracle's FFN work is small; else 512 seeded
    # tokens, the first and last, and every expert's first and last token
    if 6.0 * (w.E * Ce * w.d * w.d_ff + w.T * w.d * w.d_ff_shared) <= 100e9:
        sel = np.arange(w.T)
    else:
        firsts = np.concatenate([ref["row_token"][e * Ce:(e + 1) * Ce][[0, -1]]
                                 for e in range(w.E) if Ce > 0])
        sel = np.unique(np.concatenate([[0, w.T - 1], rng.choice(w.T, 512, replace=False),
                                        firsts]))
    sel = np.array([t for t in sel if t not in differ], np.int32)
    yref = oracle.layer_forward_expert_choice(inp["x"], inp["w_router"], inp["b_router"],
                                              inp["w_gate"], inp["w_up"], inp["w_down"], C,
                                              ws_gate=inp["ws_gate"], ws_up=inp["ws_up"],
                                              ws_down=inp["ws_down"], sel=sel)["y"]
    errs = check_y(y[torch.from_numpy(sel).long().to(y.device)], yref, w.dtype,
                   f"expert-choice layer {name}")
    # repeat calls give the same bits; the layer's routing is the permute's
    y2 = moe.layer_forward_expert_choice(s, d["x"], d["w_router"], d["b_router"], d["w_gate"],
                                         d["w_up"], d["w_down"], d["ws_gate"], d["ws_up"],
                                         d["ws_down"])
    torch.cuda.synchronize()
    assert np.array_equal(bits(y), bits(y2))
    say(f"   {name}: {sel.size} tokens, err {errs[0]:.3e} / {errs[1]:.3e}, "
        f"{len(differ)} near-tie tokens")


def test_expert_choice_empty_batch(moe):
    w = Workload("ec_empty", T=0, E=4, k=2, d=64, d_ff=32, phi=1.0, renorm=0)
    inp = to_dev(make_inputs(w, seed=1))
    s = moe.shape_of(w)
    y = moe.layer_forward_expert_choice(s, inp["x"], inp["w_router"], None, inp["w_gate"],
                                        inp["w_up"], inp["w_down"])
    logits = torch.empty(0, 4, dtype=torch.float32, device="cuda")
    out = moe.permute_expert_choice(s, inp["x"], logits)
    torch.cuda.synchronize()
    assert y.shape == (0, 64)
    assert _np(out["offsets"]).tolist() == [0] * 5


def test_expert_choice_timed_matches_layer(moe):
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    w, inp = _inputs("f32_ragged")
    d = to_dev(inp)
    s = moe.shape_of(w)
    y = moe.layer_forward_expert_choice(s, d["x"], d["w_router"], d["b_router"], d["w_gate"],
                                        d["w_up"], d["w_down"])
    evs = []
    for _ in range(7):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    y2 = torch.empty_like(y)
    moe.layer_forward_timed(s, d["x"], d["w_router"], d["b_router"], d["w_gate"], d["w_up"],
                            d["w_down"], None, None, None, y2, moe.workspace(s), evs, choice=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y), bits(y2))
    f = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(f), evs[0], evs[6]) == 0
    assert f.value > 0.0
    for e in evs:
        hip.hipEventDestroy(e)
