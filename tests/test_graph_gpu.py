"""The layer under HIP graph capture: every entry point launches on the
caller's stream with no host synchronisation, no host reads of device data
and no memset nodes, so a captured step replays as recorded.  Each case
captures one call, then replays the graph several times with other eager
work and synchronisations between the replays, and checks every replay bit
for bit against the eager call (and the eager call against the oracle)."""
import numpy as np
import pytest
import torch

import oracle
from tests._gpu import bits, check_y, host_inputs, say, to_dev
from workloads import WORKLOADS

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    import routing_dispatch_expert_route_amd as m
    return m


def _run(moe, layout, s, d, y, ws, rt):
    if layout == "choice":
        moe.layer_forward_expert_choice(s, d["x"], d["w_router"], d["b_router"], d["w_gate"],
                                        d["w_up"], d["w_down"], d["ws_gate"], d["ws_up"],
                                        d["ws_down"], y=y, ws=ws)
        return
    moe.layer_forward(s, d["x"], d["w_router"], d["b_router"], d["w_gate"], d["w_up"],
                      d["w_down"], d["ws_gate"], d["ws_up"], d["ws_down"], y=y, ws=ws,
                      padded=layout == "padded", reroute=layout == "reroute")


@pytest.mark.parametrize("name,layout", [("switch_phi125", "packed"), ("switch_phi125", "reroute"),
                                         ("switch_phi125", "padded"), ("switch_phi1", "choice"),
                                         ("granite_1412", "packed"), ("mixtral_decode", "packed")])
def test_layer_replays_from_a_graph(moe, name, layout):
    w = WORKLOADS[name]
    if layout == "choice":
        w = w.with_(renorm=0)
    inp = host_inputs(name)
    d = to_dev(inp)
    s = moe.shape_of(w)
    ws = moe.workspace(s, "cuda")
    say(f"[graph] {name} {layout}")
    y_eager = torch.empty(w.T, w.d, dtype=w.torch_dtype, device="cuda")
    _run(moe, layout, s, d, y_eager, ws, None)
    torch.cuda.synchronize()
    ref = bits(y_eager)
    if layout == "packed":
        # the eager result itself against the oracle on sampled tokens
        sel = np.array(sorted({0, w.T - 1} | set(range(0, w.T, max(1, w.T // 64)))), np.int32)
        o = oracle.layer_forward(inp["x"], inp["w_router"], inp["b_router"], inp["w_gate"],
                                 inp["w_up"], inp["w_down"], w.k, w.renorm, w.phi,
                                 inp["ws_gate"], inp["ws_up"], inp["ws_down"], sel=sel)
        check_y(y_eager[torch.from_numpy(sel).long().cuda()], o["y"], w.dtype, f"{name} eager")
    y = torch.empty_like(y_eager)
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        _run(moe, layout, s, d, y, ws, None)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        _run(moe, layout, s, d, y, ws, None)
    for i in range(4):
        y.fill_(0)                 # eager work between replays
        ws.fill_(0x5A)             # the workspace scribbled over: the graph must rebuild it
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(y), ref), f"{name} {layout}: replay {i} differs"
    say(f"   {name} {layout}: 4 replays bit-identical")
