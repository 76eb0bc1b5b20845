"""GPU parity of the reroute overflow policy ("Session 19", "Overflow
policies") -- moe_permute_reroute and moe_layer_forward_reroute -- against the
CPU oracle.  Routing outputs (final experts, seats, offsets, packed rows) are
integers: bit for bit.  The layer output is held to the layer tolerances
against the oracle composed from its own pieces (rerouted dispatch, expert
FFN, combine)."""
import numpy as np
import pytest
import torch

import oracle
from tests._gpu import bits, check_y, host_inputs, say, to_dev
from workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    import routing_dispatch_expert_route_amd as m
    return m


def _np(t):
    return t.detach().cpu().numpy()


CASES = {
    "switch_phi1": WORKLOADS["switch_phi1"],
    "switch_phi125": WORKLOADS["switch_phi125"],
    "cap_one": Workload("cap_one", T=64, E=16, k=2, d=64, d_ff=64, phi=0.01),
    "f32_ragged": Workload("f32_ragged", T=77, E=5, k=3, d=40, d_ff=24, dtype="f32", phi=0.8,
                           bias="normal"),
    "shared_small": Workload("shared_small", T=130, E=4, k=1, d=128, d_ff=64, d_ff_shared=96,
                             renorm=0, phi=1.0, bias="zipf"),
    "granite_tight": WORKLOADS["granite_1412"].with_(name="granite_tight", phi=0.75, bias="normal"),
    "e64_k8_zipf": Workload("e64_k8", T=600, E=64, k=8, d=64, d_ff=32, phi=0.9, bias="zipf"),
    # the three reroute kernels: the parallel (deferred acceptance) kernel
    # with all its state in LDS (about 24 * T + (E + 1) * T / 8 bytes <= 144
    # KiB: the shapes above, k1_e64 and k8_e32_t3000), the same kernel with its
    # per-token state in the workspace ((E + 1) * T / 8 bytes of bitmaps <= 144
    # KiB, T <= 65535), and the sequential walk beyond
    "k1_e64_zipf": Workload("k1_e64", T=700, E=64, k=1, d=64, d_ff=32, renorm=0, phi=0.5,
                            bias="zipf"),
    "k1_state_ws": Workload("k1_ws", T=8000, E=8, k=1, d=64, d_ff=32, renorm=0, phi=1.0,
                            bias="normal"),
    "k8_e32_t3000": Workload("k8_t3000", T=3000, E=32, k=8, d=64, d_ff=32, phi=0.75,
                             bias="normal"),
    "k8_e40_t16384_ws": Workload("k8_e40_big", T=16384, E=40, k=8, d=64, d_ff=32, phi=0.75,
                                 bias="zipf"),
    "k1_t60000_ws": Workload("k1_t60000", T=60000, E=8, k=1, d=64, d_ff=32, renorm=0, phi=1.0,
                             bias="normal"),
    "k2_e64_t13000_ws": Workload("k2_t13000", T=13000, E=64, k=2, d=64, d_ff=32, phi=0.8,
                                 bias="normal"),
    "k2_e64_walk": Workload("k2_walk", T=20000, E=64, k=2, d=64, d_ff=32, phi=0.8,
                            bias="normal"),
    # beyond 64 experts: the walk with four experts per lane
    "e128_k8_zipf_wide": Workload("e128_k8", T=600, E=128, k=8, d=64, d_ff=32, phi=0.9,
                                  bias="zipf"),
    "e256_k2_wide": Workload("e256_k2", T=3000, E=256, k=2, d=64, d_ff=32, phi=0.7,
                             bias="normal"),
    "e65_k1_wide": Workload("e65_k1", T=900, E=65, k=1, d=64, d_ff=32, renorm=0, phi=0.6,
                            bias="zipf"),
}


def _inputs(name):
    w = CASES[name]
    return w, (host_inputs(name) if name in WORKLOADS else make_inputs(w, seed=17))


def _oracle(w, inp):
    L = oracle.router_logits(inp["x"], inp["w_router"], inp["b_router"])
    ids, gates = oracle.topk_gates(L, w.k, w.renorm)
    C = oracle.capacity(w.T, w.E, w.k, w.phi)
    return L, ids, gates, oracle.dispatch_reroute(L, ids, w.E, C)


@pytest.mark.parametrize("name", list(CASES))
def test_permute_reroute_parity(moe, name):
    w, inp = _inputs(name)
    say(f"[permute reroute] {name}")
    d = to_dev(inp)
    s = moe.shape_of(w)
    ids, _, logits = moe.route(s, d["x"], d["w_router"], d["b_router"], want_logits=True)
    out = moe.permute_reroute(s, d["x"], logits, ids)
    torch.cuda.synchronize()
    _, _, _, ref = _oracle(w, inp)
    assert np.array_equal(_np(out["expert_ids"]), ref["ids"])
    assert np.array_equal(_np(out["counts"]), ref["counts"])
    assert np.array_equal(_np(out["filled"]), ref["filled"])
    assert np.array_equal(_np(out["offsets"]), ref["offsets"])
    assert np.array_equal(_np(out["route_pos"]), ref["route_pos"])
    n = int(ref["offsets"][-1])
    assert np.array_equal(_np(out["row_token"])[:n], ref["row_token"])
    assert np.array_equal(bits(out["x_packed"])[:n], bits(inp["x"])[ref["row_token"]])
    say(f"   {name}: {ref['n_rerouted']} routes rerouted, {n} of {w.T * w.k} seated")


@pytest.mark.parametrize("name", list(CASES))
def test_layer_forward_reroute_parity(moe, name):
    w, inp = _inputs(name)
    say(f"[layer reroute] {name}")
    d = to_dev(inp)
    s = moe.shape_of(w)
    y, rt = moe.layer_forward(s, d["x"], d["w_router"], d["b_router"], d["w_gate"], d["w_up"],
                              d["w_down"], d["ws_gate"], d["ws_up"], d["ws_down"],
                              return_routing=True, reroute=True)
    torch.cuda.synchronize()
    _, _, gates, ref = _oracle(w, inp)
    assert np.array_equal(_np(rt["expert_ids"]), ref["ids"])
    assert np.array_equal(_np(rt["route_pos"]), ref["route_pos"])
    assert np.max(np.abs(_np(rt["gates"]) - gates), initial=0.0) <= 1e-6
    xp = oracle.gather_rows(inp["x"], ref["row_token"])
    yp = oracle.expert_ffn(xp, ref["offsets"], inp["w_gate"], inp["w_up"], inp["w_down"])
    ysh = None
    if w.d_ff_shared > 0:
        ysh = oracle.swiglu_rows(inp["x"], inp["ws_gate"], inp["ws_up"], inp["ws_down"])
    yref = oracle.combine(yp, ref["route_pos"], gates, ysh)
    errs = check_y(y, yref, w.dtype, f"reroute layer {name}")
    say(f"   {name}: err {errs[0]:.3e} / {errs[1]:.3e}")


@pytest.mark.parametrize("T,E,k,phi", [(2048, 16, 1, 0.5), (700, 64, 1, 0.4), (8000, 8, 1, 0.5),
                                       (1024, 16, 4, 0.5), (600, 64, 8, 0.3),
                                       (16384, 40, 8, 0.5), (13000, 64, 1, 0.5),
                                       (20000, 64, 1, 0.5), (1500, 200, 4, 0.5)])
def test_permute_reroute_common_order(moe, T, E, k, phi):
    """Every token has the same preference order (identical rows of x), so the
    dropped routes fill the experts one after another in that order: the
    longest chain of rejections the parallel kernel can meet (about one round
    per expert), with its per-token state in LDS or (T = 8000, 16384, 13000)
    in the workspace, and, at T = 20000 over 64 experts, the same inputs
    through the walk; over 200 experts, the wide walk."""
    w = Workload("common_order", T=T, E=E, k=k, d=64, d_ff=32, renorm=0, phi=phi, bias="zipf")
    inp = make_inputs(w, seed=5)
    inp["x"] = inp["x"][:1].repeat(T, 1).contiguous()
    say(f"[permute reroute common order] T={T} E={E} k={k} phi={phi}")
    d = to_dev(inp)
    s = moe.shape_of(w)
    ids, _, logits = moe.route(s, d["x"], d["w_router"], d["b_router"], want_logits=True)
    out = moe.permute_reroute(s, d["x"], logits, ids)
    torch.cuda.synchronize()
    _, _, _, ref = _oracle(w, inp)
    assert np.array_equal(_np(out["expert_ids"]), ref["ids"])
    assert np.array_equal(_np(out["offsets"]), ref["offsets"])
    assert np.array_equal(_np(out["route_pos"]), ref["route_pos"])
    n = int(ref["offsets"][-1])
    assert np.array_equal(_np(out["row_token"])[:n], ref["row_token"])
    C = oracle.capacity(T, E, k, phi)
    assert n == min(T * k, C * E)  # every expert full, or every route seated


@pytest.mark.parametrize("T,E,k,phi", [(300, 8, 1, 1.0), (500, 16, 2, 1.0), (400, 32, 8, 1.0),
                                       (8000, 8, 1, 1.25), (3000, 64, 2, 1.0),
                                       (20000, 64, 2, 1.0), (2000, 128, 4, 1.0),
                                       (1000, 256, 8, 1.0)])
def test_permute_reroute_exact_ties(moe, T, E, k, phi):
    """Integer-valued x and router rows in {-1, 0, 1} (and a bias of 3 on
    the first quarter of the experts, so they overflow) give integer logits,
    so many of a dropped route's free experts tie exactly: the reroute must
    take the lowest index among them ("Session 19", "Overflow policies", with
    the router's tie rule), on every reroute kernel (state in LDS, in the
    workspace at T = 8000, the walk at T = 20000 over 64 experts, and the
    wide walk over 128 and 256 experts)."""
    say(f"[permute reroute ties] T={T} E={E} k={k} phi={phi}")
    w = Workload("reroute_ties", T=T, E=E, k=k, d=64, d_ff=16, phi=phi)
    g = torch.Generator().manual_seed(T + E + k)
    x = torch.randint(-1, 2, (T, 64), generator=g).to(torch.bfloat16)
    wr = torch.randint(-1, 2, (E, 64), generator=g).to(torch.bfloat16)
    b = torch.zeros(E)
    b[:E // 4] = 3.0
    s = moe.shape_of(w)
    xd = x.cuda()
    ids, _, logits = moe.route(s, xd, wr.cuda(), b.cuda(), want_logits=True)
    out = moe.permute_reroute(s, xd, logits, ids)
    torch.cuda.synchronize()
    L = oracle.router_logits(x, wr, b)
    oids, _ = oracle.topk_gates(L, k, 1)
    assert np.array_equal(_np(logits), L) and np.array_equal(_np(ids), oids)
    ref = oracle.dispatch_reroute(L, oids, E, oracle.capacity(T, E, k, phi))
    assert np.array_equal(_np(out["expert_ids"]), ref["ids"])
    assert np.array_equal(_np(out["filled"]), ref["filled"])
    assert np.array_equal(_np(out["offsets"]), ref["offsets"])
    assert np.array_equal(_np(out["route_pos"]), ref["route_pos"])
    n = int(ref["offsets"][-1])
    assert np.array_equal(_np(out["row_token"])[:n], ref["row_token"])
    # the inputs really exercise the rule: count rerouted routes whose expert
    # tied with a higher-indexed expert the token did not hold
    tied = 0
    for t, j in zip(*np.nonzero(ref["ids"] != oids)):
        e1 = ref["ids"][t, j]
        held = set(ref["ids"][t].tolist())
        tied += any(L[t, e] == L[t, e1] and e not in held for e in range(e1 + 1, E))
    assert tied > 0, "no tie was broken"
    say(f"   {ref['n_rerouted']} rerouted, {tied} of them chosen among tied experts")
