"""GPU parity of the fixed-shape dispatch buffer [E, C, d] ("Session 19",
"Capacity": capacity as a tensor dimension) -- moe_permute_padded and
moe_layer_forward_padded -- against the CPU oracle.

Buffer rows and route positions are integer/byte results: bit for bit.  The
layer output is held to the same tolerances as the packed layer (1e-4 abs
fp32, 2e-2 rel bf16), against the oracle and against the packed path on the
same inputs (the padding rows are zeros that no route reads back).
"""
import numpy as np
import pytest
import torch

import oracle
from tests._gpu import bits, check_y, host_inputs, sample_tokens, say, to_dev
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
    "granite_phi2": WORKLOADS["granite_1412"].with_(name="granite_phi2", phi=2.0),
    "e256_phi1": Workload("e256_phi1", T=300, E=256, k=8, d=64, d_ff=32, phi=1.0),
}


def _inputs(name):
    w = CASES[name]
    return w, (host_inputs(name) if name in WORKLOADS else make_inputs(w, seed=13))


@pytest.mark.parametrize("name", list(CASES))
def test_permute_padded_parity(moe, name):
    w, inp = _inputs(name)
    say(f"[permute padded] {name}")
    d = to_dev(inp)
    s = moe.shape_of(w)
    ids, _, _ = moe.route(s, d["x"], d["w_router"], d["b_router"])
    out = moe.permute_padded(s, d["x"], ids)
    torch.cuda.synchronize()
    L = oracle.router_logits(inp["x"], inp["w_router"], inp["b_router"])
    oids, _ = oracle.topk_gates(L, w.k, w.renorm)
    C = oracle.capacity(w.T, w.E, w.k, w.phi)
    ref = oracle.dispatch_padded(oids, w.E, C)
    assert np.array_equal(_np(out["counts"]), ref["counts"])
    assert np.array_equal(_np(out["kept_counts"]), ref["kept"])
    assert np.array_equal(_np(out["route_pos"]), ref["pad_pos"])
    xb = bits(inp["x"])
    got = bits(out["x_padded"]).reshape(w.E, C, w.d)
    st = ref["slot_token"]
    filled = st >= 0
    assert np.array_equal(got[filled], xb[st[filled]])
    assert not got[~filled].any(), "empty slots must be zero rows"
    say(f"   {name}: {int(filled.sum())} of {w.E * C} slots filled")


@pytest.mark.parametrize("name", list(CASES))
def test_layer_forward_padded_parity(moe, name):
    w, inp = _inputs(name)
    say(f"[layer padded] {name}")
    d = to_dev(inp)
    s = moe.shape_of(w)
    args = (s, d["x"], d["w_router"], d["b_router"], d["w_gate"], d["w_up"], d["w_down"],
            d["ws_gate"], d["ws_up"], d["ws_down"])
    y_pad, rt = moe.layer_forward(*args, return_routing=True, padded=True)
    y_packed = moe.layer_forward(*args)
    torch.cuda.synchronize()
    L = oracle.router_logits(inp["x"], inp["w_router"], inp["b_router"])
    oids, _ = oracle.topk_gates(L, w.k, w.renorm)
    C = oracle.capacity(w.T, w.E, w.k, w.phi)
    disp = oracle.dispatch_padded(oids, w.E, C)
    assert np.array_equal(_np(rt["route_pos"]), disp["pad_pos"])
    sel = None
    if w.T > 256:
        sel = sample_tokens(w.T, disp["route_pos"], disp["offsets"], disp["row_token"], n_random=64)
    ref = oracle.layer_forward(inp["x"], inp["w_router"], inp["b_router"], inp["w_gate"],
                               inp["w_up"], inp["w_down"], w.k, w.renorm, w.phi,
                               inp["ws_gate"], inp["ws_up"], inp["ws_down"], sel=sel)
    idx = None if sel is None else torch.from_numpy(sel).long().cuda()
    got = y_pad if idx is None else y_pad[idx]
    errs = check_y(got, ref["y"], w.dtype, f"padded layer {name}")
    other = y_packed if idx is None else y_packed[idx]
    check_y(got, other.double().cpu().numpy(), w.dtype, f"padded vs packed {name}")
    say(f"   {name}: err {errs[0]:.3e} / {errs[1]:.3e}")
