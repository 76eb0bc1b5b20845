"""GPU parity of every C-ABI entry point against the CPU oracle.

Integer outputs (expert ids, counts, offsets, route positions, row tokens,
drop masks) and byte copies (packed rows) must match bit for bit; router
logits too (both sides sum each dot product in the same fixed fp32 order,
R64: fused multiply-add chains over granules of eight elements, 64 partial
sums folded by halving, bias last).  Floating outputs are held to 1e-4 absolute (fp32) or
2e-2 relative (bf16).  Full-size workloads compare every routing output in
full; the layer output is compared on every token wherever the oracle's
FFN work is at most 1e11 flops (every workload but Granite T=16384, Mixtral
prefill and the shared-expert one), else on 512 seeded tokens plus the first
and last token and the owners of every expert's first and last packed row.
"""
import numpy as np
import pytest
import torch

import oracle
from tests._gpu import bits, check_y, host_inputs, sample_tokens, say, to_dev
from workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

ALL = list(WORKLOADS)
SMALL = ["tiny", "switch_phi1", "switch_phi125", "granite_1412"]

# The oracle computes the whole layer when its FFN work is at most this many
# flops (a few seconds on the host); above it, the layer output is checked on
# LAYER_SAMPLE seeded tokens plus the owners of every expert's first and last
# packed row (the integer outputs are always checked in full).
FULL_LAYER_FLOPS = 100e9
LAYER_SAMPLE = 512


def oracle_ffn_flops(w):
    return 6.0 * w.T * (w.k * w.d * w.d_ff + w.d * w.d_ff_shared)


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    import routing_dispatch_expert_route_amd as m
    return m


def _np(t):
    return t.detach().cpu().numpy()


def oracle_route(inp, w):
    L = oracle.router_logits(inp["x"], inp["w_router"], inp["b_router"])
    ids, gates = oracle.topk_gates(L, w.k, w.renorm)
    return L, ids, gates


# ------------------------------------------------------------------ route ---

@pytest.mark.parametrize("name", ALL)
def test_route_parity(moe, name):
    w = WORKLOADS[name]
    say(f"[route] {name}")
    inp = host_inputs(name, routing_only=True)
    dev = to_dev(inp)
    s = moe.shape_of(w)
    ids, gates, logits = moe.route(s, dev["x"], dev["w_router"], dev["b_router"], want_logits=True)
    torch.cuda.synchronize()
    L, oids, og = oracle_route(inp, w)
    assert np.array_equal(bits(logits), L.view(np.int32)), "logits differ"
    assert np.array_equal(_np(ids), oids)
    assert np.max(np.abs(_np(gates) - og)) <= 1e-6
    if w.renorm:
        assert np.max(np.abs(_np(gates).astype(np.float64).sum(-1) - 1.0)) <= 1e-6


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_route_worked_example(moe, dtype):
    """Router logits [2.1, 1.8, 0.2] -> softmax [0.529, 0.392, 0.079], top-2
    renormalised [0.574, 0.426] ("Session 19", worked case)."""
    say(f"[route worked] {dtype}")
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    x = torch.zeros(2, 8, dtype=dt)
    x[0, 0] = x[1, 1] = 1.0
    wr = torch.zeros(3, 8, dtype=dt)
    wr[:, 0] = torch.tensor([2.1, 1.8, 0.2])
    wr[:, 1] = torch.tensor([2.1, 1.8, 1.9])
    s3 = moe.shape(2, 8, 3, 3, 8, dtype=dtype, renorm=0)
    ids, g, _ = moe.route(s3, x.cuda(), wr.cuda())
    gl = _np(g)
    assert _np(ids)[0].tolist() == [0, 1, 2] and _np(ids)[1].tolist() == [0, 2, 1]
    tol = 5e-4 if dtype == "f32" else 5e-3   # bf16 stores 2.1 as 2.09375
    assert np.allclose(gl[0], [0.529, 0.392, 0.079], atol=tol)
    assert np.allclose(gl[1], [0.391, 0.320, 0.289], atol=tol)
    s2 = moe.shape(2, 8, 3, 2, 8, dtype=dtype, renorm=1)
    ids2, g2, _ = moe.route(s2, x.cuda(), wr.cuda())
    assert np.allclose(_np(g2)[0], [0.574, 0.426], atol=tol)
    assert sorted(_np(ids2)[1].tolist()) == [0, 2]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", ["A", "B", "C"])
def test_route_r64_hand_sums(moe, case, dtype):
    """Logits whose rounding depends on the summation order (a 2^24 term
    and unit terms in chosen granules; values derived by hand in
    tests/test_oracle_pins.py): the kernel's logit equals the hand value."""
    from tests.test_oracle_pins import r64_case
    say(f"[route R64 hand sums] {case} {dtype}")
    x, wr, b, want = r64_case(case, dtype)
    d = x.shape[1]
    s = moe.shape(1, d, 1, 1, 8, dtype=dtype, renorm=1)
    _, _, logits = moe.route(s, x.cuda(), wr.cuda(), None if b is None else b.cuda(),
                             want_logits=True)
    torch.cuda.synchronize()
    assert float(_np(logits)[0, 0]) == want
    # the same dot products among 70 tokens x 3 experts (other lanes and
    # groups of the launch): token 5, expert 1 carries the case
    xt = torch.zeros(70, d, dtype=x.dtype)
    xt[5] = x[0]
    wt = torch.zeros(3, d, dtype=x.dtype)
    wt[1] = wr[0]
    bt = None if b is None else torch.tensor([0.0, float(b[0]), 0.0])
    s3 = moe.shape(70, d, 3, 1, 8, dtype=dtype, renorm=1)
    _, _, L3 = moe.route(s3, xt.cuda(), wt.cuda(), None if bt is None else bt.cuda(),
                         want_logits=True)
    torch.cuda.synchronize()
    assert float(_np(L3)[5, 1]) == want
    if dtype == "bf16":
        # among 8192 tokens x 3 experts (a full-size launch: 2048 waves of 4
        # tokens each): token 5000, expert 1 carries the case
        xt = torch.zeros(8192, d, dtype=x.dtype)
        xt[5000] = x[0]
        sL = moe.shape(8192, d, 3, 1, 8, dtype=dtype, renorm=1)
        _, _, LL = moe.route(sL, xt.cuda(), wt.cuda(), None if bt is None else bt.cuda(),
                             want_logits=True)
        torch.cuda.synchronize()
        assert float(_np(LL)[5000, 1]) == want


def test_route_ties_take_lowest_index(moe):
    say("[route ties]")
    w = Workload("ties", T=300, E=16, k=5, d=64, d_ff=8, dtype="bf16")
    g = torch.Generator().manual_seed(3)
    x = torch.randint(-1, 2, (w.T, w.d), generator=g).to(torch.bfloat16)
    wr = torch.randint(-1, 2, (w.E, w.d), generator=g).to(torch.bfloat16)
    ids, gates, logits = moe.route(moe.shape_of(w), x.cuda(), wr.cuda(), want_logits=True)
    L = oracle.router_logits(x, wr)
    oids, og = oracle.topk_gates(L, w.k, 1)
    assert np.array_equal(_np(logits), L)
    assert np.array_equal(_np(ids), oids)
    for t in range(w.T):  # integer logits: many exact ties
        assert oids[t].tolist() == np.lexsort((np.arange(w.E), -L[t]))[:w.k].tolist()
    z = moe.route(moe.shape(5, 64, 8, 3, 8), torch.zeros(5, 64, dtype=torch.bfloat16).cuda(),
                  torch.zeros(8, 64, dtype=torch.bfloat16).cuda())[0]
    assert np.all(_np(z) == np.arange(3))


# ---------------------------------------------------------------- permute ---

PERMUTE_CASES = ALL + ["e256_k8", "ragged_cap"]


def _permute_case(name):
    if name == "e256_k8":
        return Workload(name, T=777, E=256, k=8, d=72, d_ff=40, phi=1.0)
    if name == "ragged_cap":
        return Workload(name, T=1001, E=7, k=3, d=24, d_ff=16, phi=0.6, bias="normal")
    return WORKLOADS[name]


@pytest.mark.parametrize("name", PERMUTE_CASES)
def test_permute_parity(moe, name):
    w = _permute_case(name)
    say(f"[permute] {name}")
    inp = host_inputs(name, routing_only=True) if name in WORKLOADS else \
        make_inputs(w, seed=1, routing_only=True)
    _, oids, _ = oracle_route(inp, w)
    C = oracle.capacity(w.T, w.E, w.k, w.phi)
    ref = oracle.dispatch(oids, w.E, C)
    s = moe.shape_of(w)
    out = moe.permute(s, inp["x"].cuda(), torch.from_numpy(oids).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(_np(out["counts"]), ref["counts"])
    assert np.array_equal(_np(out["kept_counts"]), ref["kept"])
    assert np.array_equal(_np(out["offsets"]), ref["offsets"])
    assert np.array_equal(_np(out["route_pos"]), ref["route_pos"])
    n = int(ref["offsets"][-1])
    assert np.array_equal(_np(out["row_token"])[:n], ref["row_token"])
    packed = oracle.gather_rows(inp["x"], ref["row_token"])
    assert np.array_equal(bits(out["x_packed"][:n]), packed.view(bits(out["x_packed"][:1]).dtype))
    assert int(ref["counts"].sum()) == w.T * w.k


def test_permute_capacity_trace(moe):
    """The "Session 19" trace: C = 5, E1 demand 6, t6 dropped; slot table."""
    say("[permute trace]")
    assign = np.array([[0, 1], [0, 2], [0, 1], [0, 3], [0, 2], [0, 1], [1, 3], [2, 3]], np.int32)
    x = torch.arange(8 * 8, dtype=torch.float32).reshape(8, 8)
    for phi, C, drops in ((1.25, 5, [10]), (1.0, 4, [8, 10]), (2.0, 8, []), (1.5, 6, [])):
        s = moe.shape(8, 8, 4, 2, 8, dtype="f32", phi=phi)
        assert moe.capacity(s)[0] == C
        out = moe.permute(s, x.cuda(), torch.from_numpy(assign).cuda())
        rp = _np(out["route_pos"]).reshape(-1)
        assert np.flatnonzero(rp < 0).tolist() == drops
        assert _np(out["counts"]).tolist() == [6, 4, 3, 3]
        if phi == 1.25:
            off = _np(out["offsets"])
            rt = _np(out["row_token"])
            assert rt[off[0]:off[1]].tolist() == [0, 1, 2, 3, 4]
            assert rt[off[1]:off[2]].tolist() == [0, 2, 5, 6]
            assert rt[off[2]:off[3]].tolist() == [1, 4, 7]
            assert rt[off[3]:off[4]].tolist() == [3, 6, 7]


def test_permute_out_of_range_ids_are_dropped(moe):
    say("[permute bad ids]")
    ids = torch.tensor([[0, 1], [9, 2], [-3, 1], [3, 0]], dtype=torch.int32)
    s = moe.shape(4, 8, 4, 2, 8, dtype="f32")
    out = moe.permute(s, torch.ones(4, 8).cuda(), ids.cuda())
    assert _np(out["counts"]).tolist() == [2, 2, 1, 1]
    rp = _np(out["route_pos"])
    assert rp[1, 0] == -1 and rp[2, 0] == -1 and np.all(rp[[0, 3]] >= 0)


# ---------------------------------------------------------------- combine ---

@pytest.mark.parametrize("dtype,k", [("f32", 1), ("f32", 2), ("bf16", 1), ("bf16", 2),
                                     ("bf16", 4), ("bf16", 8)])
def test_combine_round_trip_exact(moe, dtype, k):
    """permute then combine with gates 1/k returns x bit for bit ("271,104
    Routes", section 3: restored rows equal x[token_ids])."""
    say(f"[combine round trip] {dtype} k={k}")
    w = Workload("rt", T=333, E=16, k=k, d=200, d_ff=8, dtype=dtype)
    inp = make_inputs(w, seed=4, routing_only=True)
    s = moe.shape_of(w)
    x = inp["x"].cuda()
    ids, _, _ = moe.route(s, x, inp["w_router"].cuda())
    out = moe.permute(s, x, ids)
    gates = torch.full((w.T, k), 1.0 / k, dtype=torch.float32, device="cuda")
    y = moe.combine(s, out["x_packed"], out["route_pos"], gates)
    assert np.array_equal(bits(y), bits(inp["x"]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_combine_parity_with_drops_and_shared(moe, dtype):
    say(f"[combine parity] {dtype}")
    w = Workload("cmb", T=500, E=8, k=3, d=136, d_ff=8, dtype=dtype, phi=0.7, bias="normal")
    inp = make_inputs(w, seed=5, routing_only=True)
    s = moe.shape_of(w)
    _, oids, og = oracle_route(inp, w)
    ref = oracle.dispatch(oids, w.E, oracle.capacity(w.T, w.E, w.k, w.phi))
    assert np.any(ref["route_pos"] < 0)
    g = torch.Generator().manual_seed(6)
    n = int(ref["offsets"][-1])
    yp = torch.randn(n, w.d, generator=g).to(w.torch_dtype)
    ysh = torch.randn(w.T, w.d, generator=g).to(w.torch_dtype)
    y = moe.combine(s, yp.cuda(), torch.from_numpy(ref["route_pos"]).cuda(),
                    torch.from_numpy(og).cuda(), ysh.cuda())
    yref = oracle.combine(yp, ref["route_pos"], og, ysh)
    check_y(y, yref, dtype, "combine")
    if dtype == "bf16":  # one rounding of an fp32 sum: within 2 bf16 ulps
        assert np.max(np.abs(_np(y.float()) - yref) / (np.abs(yref) + 1e-3)) < 2 ** -7


# ------------------------------------------------------------- expert FFN ---

FFN_CASES = SMALL + ["ragged_ffn", "single_row_experts", "mixtral_decode", "shared64"]


def _ffn_case(name):
    if name == "ragged_ffn":
        return Workload(name, T=301, E=5, k=2, d=200, d_ff=72, phi=0.0, bias="normal")
    if name == "single_row_experts":
        return Workload(name, T=5, E=8, k=1, d=64, d_ff=96)
    return WORKLOADS[name]


@pytest.mark.parametrize("name", FFN_CASES)
def test_expert_ffn_parity(moe, name):
    w = _ffn_case(name)
    say(f"[expert_ffn] {name}")
    inp = host_inputs(name) if name in WORKLOADS else make_inputs(w, seed=2)
    _, oids, _ = oracle_route(inp, w)
    ref = oracle.dispatch(oids, w.E, oracle.capacity(w.T, w.E, w.k, w.phi))
    packed = oracle.gather_rows(inp["x"], ref["row_token"])
    n = int(ref["offsets"][-1])
    s = moe.shape_of(w)
    _, R_max = moe.capacity(s)
    xp = torch.zeros(max(R_max, 1), w.d, dtype=w.torch_dtype)
    xp[:n] = inp["x"][torch.from_numpy(ref["row_token"]).long()]
    assert np.array_equal(bits(xp[:n]), packed.view(bits(xp[:1]).dtype))
    d = to_dev(inp)
    yp = moe.expert_ffn(s, xp.cuda(), torch.from_numpy(ref["offsets"]).cuda(), d["w_gate"],
                        d["w_up"], d["w_down"])
    torch.cuda.synchronize()
    offs = ref["offsets"]
    if 6.0 * n * w.d * w.d_ff <= FULL_LAYER_FLOPS:
        rows = np.arange(n)
    else:
        rng = np.random.default_rng(0)
        rows = set(rng.choice(n, LAYER_SAMPLE, replace=False).tolist())
        for e in range(w.E):
            if offs[e + 1] > offs[e]:
                rows.update([int(offs[e]), int(offs[e + 1] - 1)])
        rows = np.array(sorted(rows))
    yref = np.empty((len(rows), w.d))
    for e in range(w.E):
        m = (rows >= offs[e]) & (rows < offs[e + 1])
        if m.any():
            yref[m] = oracle.swiglu_rows(xp[torch.from_numpy(rows[m]).long()], inp["w_gate"][e],
                                         inp["w_up"][e],
                                         inp["w_down"][e])
    check_y(yp[torch.from_numpy(rows).long().cuda()], yref, w.dtype, "y_packed")


def test_expert_ffn_dense_group(moe):
    """A dense SwiGLU MLP is the E = 1 case with offsets {0, T} (the shared
    expert's form); checked against torch fp64 matmuls."""
    say("[expert_ffn dense]")
    w = Workload("dense", T=257, E=1, k=1, d=256, d_ff=384)
    inp = make_inputs(w, seed=7)
    s = moe.shape_of(w)
    d = to_dev(inp)
    yp = moe.expert_ffn(s, d["x"], torch.tensor([0, w.T], dtype=torch.int32).cuda(), d["w_gate"],
                        d["w_up"], d["w_down"])
    X = inp["x"].double()
    ref = (torch.nn.functional.silu(X @ inp["w_gate"][0].double().T) *
           (X @ inp["w_up"][0].double().T)) @ inp["w_down"][0].double().T
    check_y(yp, ref.numpy(), "bf16", "dense")


# ------------------------------------------------------------ whole layer ---

def _layer_check(moe, w, inp, seed=0, n_random=LAYER_SAMPLE):
    d = to_dev(inp)
    s = moe.shape_of(w)
    y, rt = moe.layer_forward(s, d["x"], d["w_router"], d["b_router"], d["w_gate"], d["w_up"],
                              d["w_down"], d["ws_gate"], d["ws_up"], d["ws_down"],
                              return_routing=True)
    torch.cuda.synchronize()
    _, oids, og = oracle_route(inp, w)
    C = oracle.capacity(w.T, w.E, w.k, w.phi)
    disp = oracle.dispatch(oids, w.E, C)
    assert np.array_equal(_np(rt["expert_ids"]), oids)
    assert np.max(np.abs(_np(rt["gates"]) - og), initial=0.0) <= 1e-6
    assert np.array_equal(_np(rt["counts"]), disp["counts"])
    assert np.array_equal(_np(rt["route_pos"]), disp["route_pos"])
    if w.T == 0:
        return y
    sel = None
    if oracle_ffn_flops(w) > FULL_LAYER_FLOPS:
        sel = sample_tokens(w.T, disp["route_pos"], disp["offsets"], disp["row_token"],
                            n_random=n_random, seed=seed)
    ref = oracle.layer_forward(inp["x"], inp["w_router"], inp["b_router"], inp["w_gate"],
                               inp["w_up"], inp["w_down"], w.k, w.renorm, w.phi,
                               inp["ws_gate"], inp["ws_up"], inp["ws_down"], sel=sel)
    got = y if sel is None else y[torch.from_numpy(sel).long().cuda()]
    errs = check_y(got, ref["y"], w.dtype, f"layer {w.name}")
    say(f"   {w.name}: {'all' if sel is None else len(sel)} of {w.T} tokens, err {errs[0]:.3e}"
        f" / {errs[1]:.3e}, kept {int(disp['kept'].sum())} of {w.T * w.k} routes")
    return y


@pytest.mark.parametrize("name", ALL)
def test_layer_forward_parity(moe, name):
    w = WORKLOADS[name]
    say(f"[layer] {name}")
    _layer_check(moe, w, host_inputs(name))


EDGE = {
    "empty": Workload("empty", T=0, E=4, k=2, d=64, d_ff=64),
    "one_token": Workload("one_token", T=1, E=8, k=2, d=64, d_ff=64),
    "ragged_tails": Workload("ragged_tails", T=515, E=6, k=2, d=72, d_ff=40, bias="normal"),
    "e256_k8": Workload("e256_k8", T=300, E=256, k=8, d=64, d_ff=32),
    "cap_one": Workload("cap_one", T=64, E=16, k=2, d=64, d_ff=64, phi=0.01),
    "k_equals_E": Workload("k_equals_E", T=100, E=4, k=4, d=64, d_ff=64),
    "f32_ragged": Workload("f32_ragged", T=77, E=5, k=3, d=40, d_ff=24, dtype="f32",
                           phi=0.8, bias="normal"),
    "shared_small": Workload("shared_small", T=130, E=4, k=1, d=128, d_ff=64, d_ff_shared=96,
                             renorm=0, phi=1.0, bias="zipf"),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_layer_forward_edge_cases(moe, name):
    w = EDGE[name]
    say(f"[layer edge] {name}")
    _layer_check(moe, w, make_inputs(w, seed=11))


# Shapes that land on each grouped-GEMM tile with K tails (K not a multiple
# of the tile's K stage) and ragged output widths; the tile each one takes
# follows from the host heuristic in gemm.hip (shape only).
TILES = {
    # GEMM 1: 128x64-output tile (64-wide stages, K = 712 = 11*64 + 8); GEMM 2:
    # the narrow 64x128 down tile (N = 712, K = 3000) split into fp32 planes
    "narrow_tiles": Workload("narrow_tiles", T=2000, E=4, k=2, d=712, d_ff=3000, phi=1.1),
    # GEMM 1: 128x256 tile with 32-wide stages (K = 776 = 24*32 + 8)
    "m_tile_k_tail": Workload("m_tile_k_tail", T=8192, E=4, k=2, d=776, d_ff=1032),
    # GEMM 1: eight-wave 256-row tile (K = 1032, N = 2056 ragged); GEMM 2: 64x256
    "l_tile_gate_up": Workload("l_tile_gate_up", T=4096, E=2, k=1, d=1032, d_ff=2056,
                               renorm=0, bias="normal"),
    # both GEMMs on the eight-wave 256-row tile with K tails (4104, 2056)
    "l_tile_both": Workload("l_tile_both", T=8192, E=2, k=1, d=4104, d_ff=2056, renorm=0),
    # a wide d_ff on the 256-row tile with capacity drops: the dispatch packs
    # the rows before GEMM 1 (K = 1032 tail, N = 4104 ragged), and the down
    # GEMM (K = 4104) splits its partial last round along K
    "l_tile_packed_drops": Workload("l_tile_packed_drops", T=16384, E=8, k=2, d=1032, d_ff=4104,
                                    phi=0.9),
}


@pytest.mark.parametrize("name", list(TILES))
def test_layer_forward_tile_paths(moe, name):
    w = TILES[name]
    say(f"[layer tile path] {name}")
    _layer_check(moe, w, make_inputs(w, seed=13))


def test_layer_forward_packed_rows_beyond_2gib(moe):
    """Mixtral shape with T = 65536: 131072 packed rows, 3.8 GB of hidden
    rows and 1.1 GB of expert outputs, beyond 32-bit byte offsets (each GEMM
    tile addresses its rows from its own first row).  Routing outputs in
    full, the layer on 256 seeded tokens plus each expert's first and last
    row owners."""
    w = Workload("mixtral_t65536", T=65536, E=8, k=2, d=4096, d_ff=14336)
    say("[layer packed rows > 2 GiB] mixtral T=65536")
    _layer_check(moe, w, make_inputs(w, seed=29), n_random=256)


def test_forced_hot_expert_reaches_E_over_k(moe):
    say("[layer hot expert]")
    w = Workload("hot", T=512, E=32, k=8, d=64, d_ff=32, bias="normal")
    inp = make_inputs(w, seed=12)
    inp["b_router"] = torch.zeros(32)
    inp["b_router"][5] = 1e3
    _layer_check(moe, w, inp)
    s = moe.shape_of(w)
    d = to_dev(inp)
    _, rt = moe.layer_forward(s, d["x"], d["w_router"], d["b_router"], d["w_gate"], d["w_up"],
                              d["w_down"], return_routing=True)
    c = _np(rt["counts"]).astype(np.float64)
    assert c[5] == w.T and c.max() / c.mean() == w.E / w.k


def test_layer_forward_deterministic(moe):
    say("[layer determinism]")
    w = WORKLOADS["granite_1412"]
    d = to_dev(host_inputs("granite_1412"))
    s = moe.shape_of(w)
    runs = []
    for _ in range(2):
        y, rt = moe.layer_forward(s, d["x"], d["w_router"], d["b_router"], d["w_gate"], d["w_up"],
                                  d["w_down"], return_routing=True)
        runs.append((bits(y), {k_: _np(v) for k_, v in rt.items()}))
    assert np.array_equal(runs[0][0], runs[1][0])
    for k_ in runs[0][1]:
        assert np.array_equal(runs[0][1][k_], runs[1][1][k_])


def test_layer_dropped_route_keeps_only_other_gate(moe):
    """"Session 19" trace through the whole layer: t6 (logits equal to t1's)
    loses E1 at C = 5 and keeps 0.426 times E2's output."""
    say("[layer trace t6]")
    assign = [[0, 1], [0, 2], [0, 1], [0, 3], [0, 2], [0, 1], [1, 3], [2, 3]]
    w = Workload("trace", T=8, E=4, k=2, d=16, d_ff=24, dtype="f32", phi=1.25)
    inp = make_inputs(w, seed=13)
    x = torch.zeros(8, 16)
    x[torch.arange(8), torch.arange(8)] = 1.0
    wr = torch.full((4, 16), 0.0)
    wr[:, :8] = 0.2
    for t, (a, b) in enumerate(assign):
        wr[a, t], wr[b, t] = 2.1, 1.8
    inp["x"], inp["w_router"] = x, wr
    y = _layer_check(moe, w, inp)
    e2 = oracle.swiglu_rows(x[5:6], inp["w_gate"][1], inp["w_up"][1], inp["w_down"][1])[0]
    assert np.allclose(_np(y[5]), 0.4256 * e2, rtol=2e-3, atol=1e-6)


FUSED = {
    "switch_phi125": WORKLOADS["switch_phi125"],
    "switch_phi1": WORKLOADS["switch_phi1"],
    "k1_ragged_drops": Workload("k1_ragged", T=515, E=6, k=1, d=72, d_ff=40, renorm=0, phi=0.7,
                                bias="normal"),
    # the 256x256 down tile with a partial last round (about 300 tiles) and
    # K = 2048: that round is split along K into fp32 pieces, and the fix-up
    # kernel writes the gate-scaled token rows (and, with drops, the zero rows
    # come from the appended workgroups)
    "k1_tail_split": Workload("k1_tail", T=18432, E=8, k=1, d=1024, d_ff=2048, renorm=0,
                              bias="normal"),
    "k1_tail_split_drops": Workload("k1_tail_drops", T=18432, E=8, k=1, d=1024, d_ff=2048,
                                    renorm=0, phi=0.9),
    # the 256x256 down tile over whole K (K = 1024, 16 stages: no split) in
    # two rounds or more: its epilogue writes the gate-scaled token rows
    # (with drops, the appended workgroups write the zero rows)
    "k1_whole_k": Workload("k1_whole_k", T=16384, E=8, k=1, d=2048, d_ff=1024, renorm=0,
                           bias="normal"),
    "k1_whole_k_drops": Workload("k1_whole_k_drops", T=16384, E=8, k=1, d=2048, d_ff=1024,
                                 renorm=0, phi=0.9),
}


@pytest.mark.parametrize("name,reroute", [(n, False) for n in FUSED] + [("switch_phi125", True)])
def test_top1_layer_equals_its_pieces(moe, name, reroute):
    """With one route per token and no shared expert the layer's down GEMM
    writes y itself (gate-scaled rows, zero rows for dropped tokens).  Its
    output is the separate entry points' -- permute, expert_ffn, combine on
    the same routing -- bit for bit, a dropped token's row is zero, and the
    layer agrees with the oracle to the layer tolerance."""
    w = FUSED[name]
    inp = host_inputs(name) if name in WORKLOADS else make_inputs(w, seed=21)
    say(f"[top-1 layer vs pieces] {name} reroute={reroute}")
    d = to_dev(inp)
    s = moe.shape_of(w)
    y, rt = moe.layer_forward(s, d["x"], d["w_router"], d["b_router"], d["w_gate"], d["w_up"],
                              d["w_down"], return_routing=True, reroute=reroute)
    ids, gates, logits = moe.route(s, d["x"], d["w_router"], d["b_router"], want_logits=True)
    logits = logits.clone()
    out = (moe.permute_reroute(s, d["x"], logits, ids) if reroute
           else moe.permute(s, d["x"], ids))
    yp = moe.expert_ffn(s, out["x_packed"], out["offsets"], d["w_gate"], d["w_up"], d["w_down"])
    y2 = moe.combine(s, yp, out["route_pos"], gates)
    torch.cuda.synchronize()
    assert np.array_equal(_np(rt["route_pos"]), _np(out["route_pos"]))
    assert np.array_equal(bits(y), bits(y2)), f"{name}: fused layer differs from its pieces"
    dropped = _np(out["route_pos"]).reshape(-1) < 0
    assert not bits(y)[dropped].any()
    if not reroute:
        # and the layer itself against the oracle (every token)
        sel = None if oracle_ffn_flops(w) <= FULL_LAYER_FLOPS else sample_tokens(
            w.T, _np(out["route_pos"]), _np(out["offsets"]), _np(out["row_token"]),
            n_random=LAYER_SAMPLE)
        ref = oracle.layer_forward(inp["x"], inp["w_router"], inp["b_router"], inp["w_gate"],
                                   inp["w_up"], inp["w_down"], w.k, w.renorm, w.phi, sel=sel)
        got = y if sel is None else y[torch.from_numpy(sel).long().cuda()]
        check_y(got, ref["y"], w.dtype, f"top-1 layer {name}")
    say(f"   {name}: {int(dropped.sum())} dropped tokens, bit-identical")
