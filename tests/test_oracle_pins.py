"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test names the passage or the closed form it checks.  None of them
compares the oracle with itself: the references are the pages' printed
values (tests/golden/), library routines (numpy / scipy / torch fp64),
brute force and exact invariants.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from tests import _golden as G
from tests.bruteforce import dense_mask_layer, swiglu_dense
from workloads import WORKLOADS, Workload, make_inputs


def onehot_router(logit_rows, d=8):
    """x[t] = unit vector e_t, W_r[e][t] = logit -> the router's dot product
    returns the logit itself (one exact product, all other terms zero)."""
    L = np.asarray(logit_rows, dtype=np.float32)
    T, E = L.shape
    assert T <= d
    x = np.zeros((T, d), np.float32)
    x[np.arange(T), np.arange(T)] = 1.0
    w = np.zeros((E, d), np.float32)
    w[:, :T] = L.T
    return x, w


# ---------------------------------------------------------------- router ---

def test_worked_router_softmax_spk():
    g = G.load("spk_worked_router.txt")
    logits = G.nums(g["logits"])
    x, w = onehot_router([logits])
    L = oracle.router_logits(x, w)
    assert np.array_equal(L[0], np.float32(logits))
    # full softmax (k = E, no renormalisation) in descending order
    ids, gates = oracle.topk_gates(L, k=3, renorm=0)
    assert ids[0].tolist() == [0, 1, 2]
    assert np.allclose(gates[0], G.nums(g["softmax"]), atol=5e-4)
    # the printed exponentials: gate * sum(exp) = exp(l)
    assert np.allclose(gates[0] * float(g["exp_sum"]), G.nums(g["exp"]), atol=2e-3)
    # top-2 renormalised over the selected mass 0.921
    ids2, g2 = oracle.topk_gates(L, k=2, renorm=1)
    assert ids2[0].tolist() == G.nums(g["top2_ids"], int)
    assert np.allclose(g2[0], G.nums(g["top2_renorm"]), atol=5e-4)
    assert abs(gates[0][:2].sum() - float(g["selected_mass"])) < 1e-3
    assert np.allclose(g2[0], gates[0][:2] / gates[0][:2].sum(), atol=1e-7)
    # flipped third logit: E3 replaces E2 in the top-2
    fl = G.nums(g["flipped_logits"])
    x, w = onehot_router([fl])
    Lf = oracle.router_logits(x, w)
    idsf, gf = oracle.topk_gates(Lf, k=3, renorm=0)
    assert idsf[0].tolist() == [0, 2, 1]
    want = G.nums(g["flipped_softmax"])
    assert np.allclose(gf[0], [want[0], want[2], want[1]], atol=5e-4)
    ids2f, _ = oracle.topk_gates(Lf, k=2, renorm=1)
    assert sorted(ids2f[0].tolist()) == G.nums(g["flipped_top2_ids"], int)


def test_renormalised_equals_softmax_of_selected_logits():
    # 0.529/0.921 = 0.574 = 1/(1+exp(-0.3)): renormalising selected
    # probabilities is the softmax of the selected logits
    _, g2 = oracle.topk_gates(np.array([[2.1, 1.8, 0.2]], np.float32), 2, 1)
    l0, l1 = np.float32(2.1), np.float32(1.8)
    assert abs(g2[0, 0] - 1.0 / (1.0 + math.exp(float(l1) - float(l0)))) < 1e-7


@pytest.mark.parametrize("k", [1, 2, 8])
def test_gate_sum_invariant(k):
    # Granite check: renormalised gates sum to one within atol 1e-6
    rng = np.random.default_rng(1)
    L = rng.standard_normal((500, 32)).astype(np.float32) * 3
    ids, g = oracle.topk_gates(L, k, 1)
    assert np.max(np.abs(g.astype(np.float64).sum(-1) - 1.0)) <= 1e-6
    if k == 1:
        assert np.all(g == 1.0)


def test_k_equals_E_renorm_is_full_softmax():
    rng = np.random.default_rng(2)
    L = rng.standard_normal((64, 6)).astype(np.float32)
    ids, g = oracle.topk_gates(L, 6, 1)
    ref = scipy.special.softmax(L.astype(np.float64), axis=-1)
    assert np.allclose(g, np.take_along_axis(ref, ids, -1), atol=1e-7)
    ids0, g0 = oracle.topk_gates(L, 6, 0)
    assert np.array_equal(ids, ids0) and np.allclose(g, g0, atol=1e-7)


def test_top1_no_renorm_is_max_probability():
    rng = np.random.default_rng(3)
    L = rng.standard_normal((200, 8)).astype(np.float32)
    ids, g = oracle.topk_gates(L, 1, 0)
    ref = scipy.special.softmax(L.astype(np.float64), axis=-1)
    assert np.array_equal(ids[:, 0], ref.argmax(-1))
    assert np.allclose(g[:, 0], ref.max(-1), atol=1e-7)


@pytest.mark.parametrize("ties", [False, True])
def test_topk_against_full_sort(ties):
    rng = np.random.default_rng(4 + ties)
    E, k = 16, 5
    if ties:
        L = rng.integers(-2, 3, size=(400, E)).astype(np.float32)
    else:
        L = rng.standard_normal((400, E)).astype(np.float32)
    ids, _ = oracle.topk_gates(L, k, 1)
    for t in range(L.shape[0]):
        # order by (logit descending, index ascending)
        ref = np.lexsort((np.arange(E), -L[t]))[:k]
        assert ids[t].tolist() == ref.tolist()


def test_all_equal_logits_lowest_index():
    ids, g = oracle.topk_gates(np.zeros((3, 8), np.float32), 4, 1)
    assert np.all(ids == np.arange(4))
    assert np.allclose(g, 0.25)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_router_logits_within_fp32_bound(dtype):
    w = Workload("r", T=40, E=8, k=2, d=1000, d_ff=8, dtype=dtype, bias="normal")
    inp = make_inputs(w, seed=5)
    L = oracle.router_logits(inp["x"], inp["w_router"], inp["b_router"])
    L64 = oracle.router_logits(inp["x"], inp["w_router"], inp["b_router"], f64=True)
    # independent fp64 reference by library matmul
    X = inp["x"].double().numpy()
    Wr = inp["w_router"].double().numpy()
    ref = X @ Wr.T + inp["b_router"].double().numpy()
    assert np.allclose(L64, ref, rtol=0, atol=1e-12)
    # R64 order: every term passes through at most 8*ceil(d/512) fused
    # multiply-adds of its partial sum and 6 folds, so |err| <= gamma_n *
    # sum|x_i w_i| with n = 8*ceil(d/512) + 6, plus the bias rounding
    u = 2.0 ** -24
    n = 8 * -(-w.d // 512) + 6
    gam = n * u / (1 - n * u)
    bound = gam * (np.abs(X) @ np.abs(Wr).T) + 2 * u * (np.abs(ref) + 1)
    assert np.all(np.abs(L.astype(np.float64) - ref) <= bound)


# Hand-derived R64 sums.  x is 1 at the listed hidden indices (0 elsewhere)
# and the router row holds the listed weight there, so each product is one
# exact weight; 2^24 = 16777216 is where fp32 spacing becomes 2, so adding 1
# to it rounds (ties to even) and the result depends on the order.  Values:
#   A  d=512: 2^24 at i=0 and 1 at i=8l for l=1..63 (one unit in every other
#      partial sum).  Folds: s=32 2^24+1 -> 2^24, the rest 2; then +2, +4,
#      +8, +16, +32 exactly: 2^24 + 62 (exact sum 2^24+63; a sequential sum
#      gives 2^24).
#   B  d=512: 2^24 at i=0, 1 at i=256 and i=384 (partial sums 32 and 48), bias
#      2.  s=32: 2^24+1 -> 2^24 and p16 = 1; s=16: 2^24+1 -> 2^24; bias last:
#      2^24 + 2 (folding s=1 first gives 2^24+2 before the bias; the bias
#      added first gives 2^24+4).
#   C  d=1024: 2^24 at i=0, 1 at i=7 and i=512 (granules 0 and 64, both
#      partial sum 0), 1 at i=8 and i=520 (granules 1 and 65, partial sum 1).
#      p0: 2^24, +1 -> 2^24, +1 -> 2^24; p1 = 2; fold: 2^24 + 2 (granules of
#      one element instead of eight give 2^24+4, a sequential sum 2^24).
R64_CASES = {
    "A": (512, [(0, 2.0 ** 24)] + [(8 * l, 1.0) for l in range(1, 64)], None, 2 ** 24 + 62),
    "B": (512, [(0, 2.0 ** 24), (256, 1.0), (384, 1.0)], 2.0, 2 ** 24 + 2),
    "C": (1024, [(0, 2.0 ** 24), (7, 1.0), (512, 1.0), (8, 1.0), (520, 1.0)], None, 2 ** 24 + 2),
}


def r64_case(name, dtype):
    """(x [1, d], w_router [1, d], bias [1] or None, expected logit)."""
    d, terms, bias, want = R64_CASES[name]
    x = torch.zeros(1, d)
    w = torch.zeros(1, d)
    for i, v in terms:
        x[0, i] = 1.0
        w[0, i] = v
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    b = None if bias is None else torch.tensor([bias], dtype=torch.float32)
    return x.to(dt), w.to(dt), b, float(want)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name", list(R64_CASES))
def test_router_r64_order_hand_sums(name, dtype):
    x, w, b, want = r64_case(name, dtype)
    L = oracle.router_logits(x, w, b)
    assert float(L[0, 0]) == want, (name, float(L[0, 0]), want)


# -------------------------------------------------------------- dispatch ---

def test_permute_mml_example():
    g = G.load("mml_permute.txt")
    E = int(g["num_experts"])
    ids = np.array(G.rows(g["expert_ids"], int), np.int32)
    out = oracle.dispatch(ids, E, -1)
    ends = np.cumsum(out["counts"])
    assert ends.tolist() == G.nums(g["expert_ends"], int)
    assert out["offsets"].tolist() == [0] + G.nums(g["expert_ends"], int)
    for e in (2, 4, 7):
        lo, hi = out["offsets"][e], out["offsets"][e + 1]
        assert out["row_token"][lo:hi].tolist() == G.nums(g[f"group_{e}"], int)
    # round trip: packed rows restored to route order equal x[token_ids]
    x = np.array(G.rows(g["x"]), np.float32)
    packed = oracle.gather_rows(x, out["row_token"])
    restored = packed[out["route_pos"].reshape(-1)]
    assert np.array_equal(restored, x[np.repeat(np.arange(3), 2)])


def test_dispatch_matches_stable_argsort():
    # the page's formulation: stable argsort of the flat ids + bincount.cumsum
    rng = np.random.default_rng(6)
    T, E, k = 300, 12, 3
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    out = oracle.dispatch(ids, E, -1)
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")
    tok = np.repeat(np.arange(T), k)
    assert np.array_equal(out["row_token"], tok[order])
    assert np.array_equal(out["offsets"][1:], np.cumsum(np.bincount(flat, minlength=E)))
    inv = np.empty_like(order)
    inv[order] = np.arange(order.size)
    assert np.array_equal(out["route_pos"].reshape(-1), inv)


def _trace_variant(assign, E, phi, k):
    ids = np.array(assign, np.int32)[:, :k].copy()
    T = ids.shape[0]
    C = oracle.capacity(T, E, k, phi)
    return C, ids, oracle.dispatch(ids, E, C)


def test_capacity_trace_spk():
    g = G.load("spk_capacity_trace.txt")
    E, k = int(g["E"]), int(g["k"])
    assign = G.rows(g["assign"], int)
    variants = g["variant"]
    for v in variants:
        phi, C_want, dropped, used, reserved = v.split()
        C, ids, out = _trace_variant(assign, E, float(phi), k)
        assert C == int(C_want)
        assert out["counts"].tolist() == G.nums(g["counts"], int)
        assert int(out["counts"].sum()) == int(g["T"]) * k          # 16 = 8 x 2
        drops = sorted(f"{r // k}@{ids[r // k, r % k]}"
                       for r in np.flatnonzero(out["route_pos"].reshape(-1) < 0))
        want = [] if dropped == "-" else sorted(dropped.split(","))
        assert drops == want
        assert int(out["kept"].sum()) == int(used)
        assert E * C == int(reserved)
        if phi == "1.25":
            for e in range(E):
                lo, hi = out["offsets"][e], out["offsets"][e + 1]
                assert out["row_token"][lo:hi].tolist() == G.nums(g[f"slots_E{e}"], int)
    # k = 1: first choice of each pair, phi = 1.25
    C, ids, out = _trace_variant(assign, E, 1.25, 1)
    assert C == int(g["k1_C"])
    assert out["counts"].tolist() == G.nums(g["k1_loads"], int)
    assert np.flatnonzero(out["route_pos"].reshape(-1) < 0).tolist() == G.nums(g["k1_dropped"], int)


def test_capacity_trace_end_to_end_t6_keeps_only_second_gate():
    """Trace driven through the whole layer: each token's logits put its pair
    first (t6 shares t1's logits); with C = 5 t6 loses E1 and its output is
    the second gate (0.426) times E2's FFN output, not renormalised."""
    g = G.load("spk_capacity_trace.txt")
    assign = G.rows(g["assign"], int)
    T, E, k, d, d_ff = 8, 4, 2, 16, 24
    L = np.full((T, E), 0.2, np.float32)
    for t, (a, b) in enumerate(assign):
        L[t, a], L[t, b] = 2.1, 1.8
    x = np.zeros((T, d), np.float32)
    x[np.arange(T), np.arange(T)] = 1.0
    x += np.random.default_rng(7).standard_normal((T, d)).astype(np.float32) * 0  # keep one-hot
    wr = np.zeros((E, d), np.float32)
    wr[:, :T] = L.T
    rng = np.random.default_rng(8)
    wg = rng.standard_normal((E, d_ff, d)).astype(np.float32)
    wu = rng.standard_normal((E, d_ff, d)).astype(np.float32)
    wd = rng.standard_normal((E, d, d_ff)).astype(np.float32)
    out = oracle.layer_forward(x, wr, None, wg, wu, wd, k=k, renorm=1, phi=1.25)
    assert out["route_pos"][5, 0] == -1 and out["route_pos"][5, 1] >= 0
    X = torch.from_numpy(x).double()
    ffn_e2 = swiglu_dense(X[5:6], *(torch.from_numpy(w[1]).double() for w in (wg, wu, wd)))[0]
    gate = out["gates"][5, 1]
    assert abs(gate - float(g["t6_kept_gate"])) < 5e-4
    assert np.allclose(out["y"][5], gate * ffn_e2.numpy(), rtol=1e-12, atol=1e-12)


def test_overflow_int8():
    g = G.load("int8_overflow.txt")
    T, E, k, phi = int(g["T"]), int(g["E"]), int(g["k"]), float(g["phi"])
    ids = np.array(G.nums(g["assign"], int), np.int32).reshape(T, k)
    C = oracle.capacity(T, E, k, phi)
    assert C == int(g["C"])
    out = oracle.dispatch(ids, E, C)
    assert out["counts"].tolist() == G.nums(g["loads"], int)
    dropped = np.flatnonzero(out["route_pos"].reshape(-1) < 0)
    assert len(dropped) == int(g["dropped"])
    # arrival order: the last three arrivals at expert 0 are the dropped ones
    e0 = np.flatnonzero(ids[:, 0] == 0)
    assert dropped.tolist() == e0[2:].tolist()


def test_capacity_formula():
    assert oracle.capacity(8, 4, 2, 1.25) == 5
    assert oracle.capacity(8, 4, 1, 1.25) == 3
    assert oracle.capacity(4096, 8, 1, 1.0) == 512
    assert oracle.capacity(4096, 8, 1, 1.25) == 640
    assert oracle.capacity(10, 4, 1, 0.01) == 1
    assert oracle.capacity(8, 4, 2, 0.0) == -1
    assert oracle.capacity(8, 4, 2, -1.0) == -1


def test_route_count_granite_271104():
    """1,412 tokens x 24 layers x top-8 of 32 = 271,104 routes: the demand
    counts of 24 independently seeded router layers sum to that."""
    w = WORKLOADS["granite_1412"].with_(d_ff=8)
    total = 0
    for layer in range(24):
        inp = make_inputs(w.with_(E=32), seed=100 + layer)
        L = oracle.router_logits(inp["x"], inp["w_router"])
        ids, _ = oracle.topk_gates(L, w.k, 1)
        out = oracle.dispatch(ids, w.E, -1)
        assert int(out["counts"].sum()) == w.T * w.k == 11296
        assert int(out["offsets"][-1]) == 11296
        total += int(out["counts"].sum())
    assert total == 271104


def test_forced_expert_imbalance_reaches_E_over_k():
    """One expert in every token's top-k gives max/mean demand = E/k, the
    worst case (4 for 32 experts, top-8)."""
    w = Workload("imb", T=256, E=32, k=8, d=64, d_ff=8)
    inp = make_inputs(w, seed=9)
    b = np.zeros(32, np.float32)
    b[17] = 1e3
    L = oracle.router_logits(inp["x"], inp["w_router"], b)
    ids, _ = oracle.topk_gates(L, w.k, 1)
    counts = oracle.dispatch(ids, w.E, -1)["counts"]
    I = counts.max() / counts.mean()
    assert counts[17] == w.T and I == w.E / w.k == 4.0


# ------------------------------------------------------- FFN and layer ---

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_expert_is_dense_swiglu(dtype):
    w = Workload("dense", T=24, E=1, k=1, d=40, d_ff=56, dtype=dtype)
    inp = make_inputs(w, seed=10)
    out = oracle.layer_forward(inp["x"], inp["w_router"], None, inp["w_gate"], inp["w_up"],
                               inp["w_down"], k=1, renorm=1, phi=0)
    ref = swiglu_dense(inp["x"].double(), inp["w_gate"][0].double(), inp["w_up"][0].double(),
                       inp["w_down"][0].double())
    assert np.all(out["gates"] == 1.0)
    assert np.allclose(out["y"], ref.numpy(), rtol=1e-12, atol=1e-12)
    rows = oracle.swiglu_rows(inp["x"], inp["w_gate"][0], inp["w_up"][0], inp["w_down"][0])
    assert np.allclose(rows, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_shared_expert_alone_when_routed_outputs_zero():
    w = Workload("sh", T=16, E=4, k=2, d=32, d_ff=24, d_ff_shared=40, dtype="bf16")
    inp = make_inputs(w, seed=11, zero_routed=True)
    out = oracle.layer_forward(inp["x"], inp["w_router"], None, inp["w_gate"], inp["w_up"],
                               inp["w_down"], k=2, renorm=1, phi=0, ws_gate=inp["ws_gate"],
                               ws_up=inp["ws_up"], ws_down=inp["ws_down"])
    ref = swiglu_dense(inp["x"].double(), inp["ws_gate"].double(), inp["ws_up"].double(),
                       inp["ws_down"].double())
    assert np.allclose(out["y"], ref.numpy(), rtol=1e-12, atol=1e-12)


CASES = [
    dict(T=48, E=4, k=2, d=32, d_ff=48, dtype="f32", renorm=1, phi=0.0, bias=None),
    dict(T=40, E=8, k=1, d=24, d_ff=40, dtype="bf16", renorm=0, phi=1.0, bias="normal"),
    dict(T=40, E=8, k=1, d=24, d_ff=40, dtype="bf16", renorm=0, phi=1.25, bias="normal"),
    dict(T=30, E=6, k=3, d=16, d_ff=24, dtype="bf16", renorm=1, phi=0.75, bias=None),
    dict(T=32, E=16, k=2, d=32, d_ff=16, d_ff_shared=40, dtype="bf16", renorm=1, phi=0.0,
         bias="zipf"),
    dict(T=20, E=5, k=5, d=16, d_ff=16, dtype="f32", renorm=1, phi=0.0, bias=None),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_layer_matches_dense_mask_bruteforce(case):
    w = Workload("bf", **CASES[case])
    inp = make_inputs(w, seed=20 + case)
    sh = dict(ws_gate=inp["ws_gate"], ws_up=inp["ws_up"], ws_down=inp["ws_down"])
    out = oracle.layer_forward(inp["x"], inp["w_router"], inp["b_router"], inp["w_gate"],
                               inp["w_up"], inp["w_down"], k=w.k, renorm=w.renorm, phi=w.phi, **sh)
    ref = dense_mask_layer(inp["x"], inp["w_router"], inp["b_router"], inp["w_gate"],
                           inp["w_up"], inp["w_down"], w.k, w.renorm, w.phi, **sh)
    if ref["gap"] is not None:
        assert float(ref["gap"].min()) > 1e-4   # no near tie at these seeds
    assert np.array_equal(out["ids"], ref["ids"].numpy())
    scale = np.abs(ref["y"].numpy()).max()
    assert np.max(np.abs(out["y"] - ref["y"].numpy())) <= 1e-5 * scale
    # gates agree with the brute-force weights of the selected experts
    wsel = torch.gather(ref["weights"], 1, ref["ids"].long()).numpy()
    kept = out["route_pos"] >= 0
    assert np.allclose(out["gates"][kept], wsel[kept], atol=1e-6)


def test_token_permutation_equivariance_dropless():
    w = Workload("perm", T=32, E=8, k=2, d=32, d_ff=24, dtype="bf16")
    inp = make_inputs(w, seed=30)
    args = lambda x: (x, inp["w_router"], None, inp["w_gate"], inp["w_up"], inp["w_down"])
    y = oracle.layer_forward(*args(inp["x"]), k=2, renorm=1, phi=0)["y"]
    perm = torch.randperm(w.T, generator=torch.Generator().manual_seed(1))
    yp = oracle.layer_forward(*args(inp["x"][perm].contiguous()), k=2, renorm=1, phi=0)["y"]
    assert np.array_equal(yp, y[perm.numpy()])


def test_expert_relabelling_invariance():
    w = Workload("relab", T=32, E=8, k=2, d=32, d_ff=24, dtype="bf16", bias="normal")
    inp = make_inputs(w, seed=31)
    perm = torch.tensor([3, 7, 0, 5, 1, 6, 2, 4])
    base = oracle.layer_forward(inp["x"], inp["w_router"], inp["b_router"], inp["w_gate"],
                                inp["w_up"], inp["w_down"], k=2, renorm=1, phi=0)
    rel = oracle.layer_forward(inp["x"], inp["w_router"][perm].contiguous(),
                               inp["b_router"][perm].contiguous(), inp["w_gate"][perm].contiguous(),
                               inp["w_up"][perm].contiguous(), inp["w_down"][perm].contiguous(),
                               k=2, renorm=1, phi=0)
    assert np.array_equal(perm.numpy()[rel["ids"]], base["ids"])
    assert np.allclose(rel["y"], base["y"], rtol=1e-12, atol=1e-12)


def test_down_projection_scaling_is_exact():
    w = Workload("sc", T=16, E=4, k=2, d=32, d_ff=24, dtype="bf16")
    inp = make_inputs(w, seed=32)
    a = oracle.layer_forward(inp["x"], inp["w_router"], None, inp["w_gate"], inp["w_up"],
                             inp["w_down"], k=2, renorm=1, phi=0)["y"]
    b = oracle.layer_forward(inp["x"], inp["w_router"], None, inp["w_gate"], inp["w_up"],
                             inp["w_down"] * 2, k=2, renorm=1, phi=0)["y"]
    assert np.array_equal(b, 2 * a)


def test_combine_round_trip_with_uniform_gates():
    """Gates 1/k over packed copies of x return x exactly (k a power of
    two): checks that combine reads each route's own packed row."""
    for k in (1, 2, 4):
        w = Workload("rt", T=50, E=8, k=k, d=16, d_ff=8, dtype="bf16")
        inp = make_inputs(w, seed=33)
        L = oracle.router_logits(inp["x"], inp["w_router"])
        ids, _ = oracle.topk_gates(L, k, 1)
        disp = oracle.dispatch(ids, 8, -1)
        packed = oracle.gather_rows(inp["x"], disp["row_token"])
        gates = np.full((w.T, k), 1.0 / k, np.float32)
        y = oracle.combine(packed, disp["route_pos"], gates)
        assert np.array_equal(y, inp["x"].double().numpy())


def test_expert_ffn_and_combine_compose_to_layer():
    w = Workload("cmp", T=40, E=6, k=2, d=24, d_ff=32, d_ff_shared=16, dtype="bf16",
                 phi=1.0, bias="normal")
    inp = make_inputs(w, seed=34)
    out = oracle.layer_forward(inp["x"], inp["w_router"], inp["b_router"], inp["w_gate"],
                               inp["w_up"], inp["w_down"], k=2, renorm=1, phi=1.0,
                               ws_gate=inp["ws_gate"], ws_up=inp["ws_up"], ws_down=inp["ws_down"])
    C = oracle.capacity(w.T, w.E, w.k, 1.0)
    disp = oracle.dispatch(out["ids"], w.E, C)
    assert np.array_equal(disp["route_pos"], out["route_pos"])
    packed = oracle.gather_rows(inp["x"], disp["row_token"])
    yp = oracle.expert_ffn(packed, disp["offsets"], inp["w_gate"], inp["w_up"], inp["w_down"])
    ysh = oracle.swiglu_rows(inp["x"], inp["ws_gate"], inp["ws_up"], inp["ws_down"])
    y = oracle.combine(yp, disp["route_pos"], out["gates"], ysh)
    assert np.allclose(y, out["y"], rtol=1e-12, atol=1e-12)


def test_sampled_tokens_match_full_run_and_determinism():
    w = Workload("sel", T=30, E=4, k=2, d=16, d_ff=16, dtype="bf16", phi=1.0)
    inp = make_inputs(w, seed=35)
    args = (inp["x"], inp["w_router"], None, inp["w_gate"], inp["w_up"], inp["w_down"])
    full = oracle.layer_forward(*args, k=2, renorm=1, phi=1.0)
    again = oracle.layer_forward(*args, k=2, renorm=1, phi=1.0)
    for key in full:
        assert np.array_equal(full[key], again[key])
    sel = np.array([29, 0, 7, 7], np.int32)
    part = oracle.layer_forward(*args, k=2, renorm=1, phi=1.0, sel=sel)
    assert np.array_equal(part["y"], full["y"][sel])


def test_empty_batch():
    w = Workload("empty", T=0, E=4, k=2, d=16, d_ff=16, dtype="bf16")
    inp = make_inputs(w, seed=36)
    out = oracle.layer_forward(inp["x"], inp["w_router"], None, inp["w_gate"], inp["w_up"],
                               inp["w_down"], k=2, renorm=1, phi=1.0)
    assert out["y"].shape == (0, 16) and out["counts"].tolist() == [0, 0, 0, 0]


# ---------------------------------------------------------------------------
# Forward-only routing statistics ([INT8] section 4 aux loss; [UD] load
# imbalance; [MML] section 4 shares, largest weight, entropy, JS distance;
# [BEA] "Router Confidence").

def _routing(T, E, k, renorm, seed, scale=1.0, bias=None):
    rng = np.random.default_rng(seed)
    logits = (rng.standard_normal((T, E)) * scale).astype(np.float32)
    if bias is not None:
        logits = (logits + bias).astype(np.float32)
    ids, gates = oracle.topk_gates(logits, k, renorm)
    counts = np.bincount(ids.ravel(), minlength=E).astype(np.int32)
    return logits, ids, gates, counts


def test_stats_balanced_routing_gives_alpha():
    # f_e = 1/E for every expert => aux = alpha * E * sum_e P_e / E = alpha
    # whatever the probabilities (they sum to 1)
    T, E, k = 64, 8, 2
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    _, gates = oracle.topk_gates(logits, k, 1)
    counts = np.full(E, T * k // E, np.int32)
    st = oracle.routing_stats(logits, gates, counts, alpha=1e-2)
    assert st["aux_loss"] == pytest.approx(1e-2, rel=1e-12)
    assert st["load_imbalance"] == pytest.approx(1.0, rel=1e-12)
    assert st["js_to_uniform"] == pytest.approx(0.0, abs=1e-7)


def test_stats_uniform_logits():
    T, E, k, nb = 32, 8, 2, 20
    logits = np.zeros((T, E), np.float32)
    ids, gates = oracle.topk_gates(logits, k, 1)
    counts = np.bincount(ids.ravel(), minlength=E).astype(np.int32)
    st = oracle.routing_stats(logits, gates, counts, n_bins=nb)
    assert np.allclose(st["mean_prob"], 1.0 / E, rtol=0, atol=1e-15)
    assert st["mean_confidence"] == pytest.approx(1.0 / E, rel=1e-12)
    assert st["hist"][int(nb / E)] == T and st["hist"].sum() == T
    # all ties go to experts 0..k-1 ([UD]: the worst case is E/k)
    assert st["load_imbalance"] == pytest.approx(E / k, rel=1e-12)
    assert st["mean_norm_entropy"] == pytest.approx(1.0, rel=1e-12)
    assert st["mean_max_gate"] == pytest.approx(1.0 / k, rel=1e-7)


def test_stats_hot_expert_imbalance_is_E_over_k():
    T, E, k = 128, 32, 8
    bias = np.zeros(E, np.float32)
    bias[5] = 1e3
    logits, ids, gates, counts = _routing(T, E, k, 1, seed=4, bias=bias)
    st = oracle.routing_stats(logits, gates, counts)
    assert st["load_imbalance"] == pytest.approx(E / k, rel=1e-12)


@pytest.mark.parametrize("T,E,k,renorm", [(300, 8, 2, 1), (257, 32, 8, 1), (100, 8, 1, 0), (64, 64, 2, 1)])
def test_stats_against_scipy(T, E, k, renorm):
    from scipy.spatial.distance import jensenshannon
    from scipy.special import softmax
    from scipy.stats import entropy
    nb = 16
    logits, ids, gates, counts = _routing(T, E, k, renorm, seed=T + E, scale=2.0)
    st = oracle.routing_stats(logits, gates, counts, alpha=1e-2, n_bins=nb)
    p = softmax(logits.astype(np.float64), axis=1)
    share = counts / (T * k)
    assert np.allclose(st["share"], share, rtol=1e-14)
    assert np.allclose(st["mean_prob"], p.mean(axis=0), rtol=1e-12, atol=1e-15)
    assert st["aux_loss"] == pytest.approx(1e-2 * E * float(np.dot(share, p.mean(axis=0))), rel=1e-12)
    assert st["js_to_uniform"] == pytest.approx(float(jensenshannon(share, np.full(E, 1.0 / E), base=2)),
                                                rel=1e-9, abs=1e-12)
    g = gates.astype(np.float64)
    assert st["mean_max_gate"] == pytest.approx(float(g.max(axis=1).mean()), rel=1e-12)
    if k > 1:
        h = entropy(g / g.sum(axis=1, keepdims=True), axis=1) / np.log(k)
        assert st["mean_norm_entropy"] == pytest.approx(float(h.mean()), rel=1e-10)
    else:
        assert st["mean_norm_entropy"] == 0.0
    conf = p.max(axis=1)
    assert st["mean_confidence"] == pytest.approx(float(conf.mean()), rel=1e-12)
    ref_hist, _ = np.histogram(conf, bins=nb, range=(0.0, 1.0))
    assert np.array_equal(st["hist"], ref_hist)


def test_stats_empty_batch():
    st = oracle.routing_stats(np.zeros((0, 4), np.float32), np.zeros((0, 2), np.float32),
                              np.zeros(4, np.int32), n_bins=8)
    assert all(st[n] == 0.0 for n in oracle.STAT_NAMES)
    assert st["hist"].sum() == 0


def test_padded_slot_table_spk():
    """"Session 19", "Visual support -- Capacity": the [E, C, d] dispatch
    buffer for the trace with C = 5 -- slots in arrival order per expert,
    15 filled, 5 empty, t6 dropped at E1."""
    g = G.load("spk_capacity_trace.txt")
    E, k = int(g["E"]), int(g["k"])
    ids = np.array(G.rows(g["assign"], int), np.int32)
    C = oracle.capacity(int(g["T"]), E, k, 1.25)
    out = oracle.dispatch_padded(ids, E, C)
    st = out["slot_token"]
    assert st.shape == (E, 5)
    for e in range(E):
        seated = G.nums(g[f"slots_E{e}"], int)
        assert st[e, :len(seated)].tolist() == seated
        assert (st[e, len(seated):] == -1).all()
    assert int((st >= 0).sum()) == 15 and int((st < 0).sum()) == 5
    pp = out["pad_pos"]
    assert pp[5, 0] == -1                                  # t6 at E1 dropped
    for t in range(ids.shape[0]):
        for j in range(k):
            if pp[t, j] >= 0:
                e, c = divmod(int(pp[t, j]), C)
                assert e == ids[t, j] and st[e, c] == t


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_padded_positions_follow_arrival_order(seed):
    # brute force: slot = number of earlier kept routes to the same expert
    rng = np.random.default_rng(seed)
    T, E, k = 50, 6, 2
    ids = np.array([rng.choice(E, size=k, replace=False) for _ in range(T)], np.int32)
    C = oracle.capacity(T, E, k, 1.0)
    out = oracle.dispatch_padded(ids, E, C)
    seen = np.zeros(E, int)
    for r in range(T * k):
        t, j = divmod(r, k)
        e = ids[t, j]
        if seen[e] < C:
            assert out["pad_pos"][t, j] == e * C + seen[e]
            seen[e] += 1
        else:
            assert out["pad_pos"][t, j] == -1


def test_reroute_trace_spk():
    """"Session 19", "Overflow policies": with C = 5, t6 finds E1 full; under
    the reroute policy its route goes to its third-best expert (it already
    holds E2) -- E3 here -- and every one of the 16 routes is seated."""
    g = G.load("spk_capacity_trace.txt")
    assign = G.rows(g["assign"], int)
    T, E, k = 8, 4, 2
    L = np.full((T, E), 0.2, np.float32)
    for t, (a, b) in enumerate(assign):
        L[t, a], L[t, b] = 2.1, 1.8
    third = 2 if 2 not in assign[5] else 3
    L[5, third] = 0.9   # third-best of t6 (its pair comes first)
    ids = np.array(assign, np.int32)
    C = oracle.capacity(T, E, k, 1.25)
    out = oracle.dispatch_reroute(L, ids, E, C)
    assert out["n_rerouted"] == 1
    assert out["ids"][5].tolist() == [third, 1]
    assert out["filled"].tolist() == [5, 4, 4, 3]
    assert int(out["offsets"][E]) == 16
    # E3's seats: t2, t5, t8 kept, then t6 in the fourth slot
    lo = out["offsets"][third]
    assert out["row_token"][lo:lo + 4].tolist() == G.nums(g[f"slots_E{third}"], int) + [5]


def test_reroute_ties_take_lowest_index():
    """Ties in the reroute: among free experts with equal logits a dropped
    route takes the lowest index ("Session 19", "Overflow policies": the
    overflowing route goes to the token's next-best expert; ties broken by
    the lowest expert index, as in the router's own top-k).  Expected values
    derived by hand.

    Top-1, E = 4, T = 3, C = ceil(1.0 * 3 / 4) = 1, every token's logits
    [3, 1, 1, 0]: t0 takes E0; t1 overflows E0, E1 and E2 tie -> E1; t2
    overflows E0, E1 is now full -> E2 (its tie partner); E3 stays empty.
    Top-2, E = 5, T = 2, C = ceil(0.5 * 4 / 5) = 1, logits [4, 3, 1, 1, 1]:
    t0 holds E0, E1; t1 loses both, E2..E4 tie -> E2 then E3."""
    L = np.array([[3, 1, 1, 0]] * 3, np.float32)
    ids, _ = oracle.topk_gates(L, 1, 0)
    assert ids[:, 0].tolist() == [0, 0, 0]
    C = oracle.capacity(3, 4, 1, 1.0)
    assert C == 1
    out = oracle.dispatch_reroute(L, ids, 4, C)
    assert out["ids"][:, 0].tolist() == [0, 1, 2]
    assert out["filled"].tolist() == [1, 1, 1, 0]
    assert out["route_pos"][:, 0].tolist() == [0, 1, 2]
    assert out["n_rerouted"] == 2

    L2 = np.array([[4, 3, 1, 1, 1]] * 2, np.float32)
    ids2, _ = oracle.topk_gates(L2, 2, 1)
    assert ids2.tolist() == [[0, 1], [0, 1]]
    C2 = oracle.capacity(2, 5, 2, 0.5)
    assert C2 == 1
    out2 = oracle.dispatch_reroute(L2, ids2, 5, C2)
    assert out2["ids"].tolist() == [[0, 1], [2, 3]]
    assert out2["filled"].tolist() == [1, 1, 1, 1, 0]
    assert out2["route_pos"].tolist() == [[0, 1], [2, 3]]


def _reroute_invariants(L, ids, E, C, out, ref):
    T, k = ids.shape
    fids, rp = out["ids"], out["route_pos"]
    filled = out["filled"]
    assert (filled <= C).all()
    seated = rp >= 0
    assert np.array_equal(np.bincount(fids[seated], minlength=E), filled)
    for t in range(T):
        assert len(set(fids[t].tolist())) == k, "a token holds an expert twice"
    order = lambda t: sorted(range(E), key=lambda e: (-float(L[t, e]), e))
    for t in range(T):
        for j in range(k):
            e0, e1 = ids[t, j], fids[t, j]
            if ref["route_pos"][t, j] >= 0:
                # kept by the drop policy: same expert, same slot
                assert e1 == e0 and rp[t, j] - out["offsets"][e1] == ref["route_pos"][t, j] - ref["offsets"][e0]
                continue
            others = set(fids[t].tolist()) - {e1}
            if rp[t, j] >= 0:       # rerouted: every preferred free choice is full now
                assert e1 != e0
                for e in order(t):
                    if e == e1:
                        break
                    if e not in others and e != e0:
                        assert filled[e] == C, (t, j, e)
            else:                   # still dropped: nothing it could take has room
                for e in range(E):
                    if e not in others and e != e0:
                        assert filled[e] == C
    # packed rows: kept routes of an expert first, then its rerouted ones,
    # each group in arrival order
    for e in range(E):
        lo, hi = out["offsets"][e], out["offsets"][e + 1]
        rows = [(int(rp[t, j]), t * k + j, ref["route_pos"][t, j] >= 0)
                for t in range(T) for j in range(k) if fids[t, j] == e and rp[t, j] >= 0]
        rows.sort()
        assert [r[0] for r in rows] == list(range(lo, hi))
        flags = [r[2] for r in rows]
        assert flags == sorted(flags, reverse=True)
        kept_routes = [r[1] for r in rows if r[2]]
        moved_routes = [r[1] for r in rows if not r[2]]
        assert kept_routes == sorted(kept_routes) and moved_routes == sorted(moved_routes)
        for p, r, _ in rows:
            assert out["row_token"][p] == r // k


@pytest.mark.parametrize("T,E,k,phi,seed", [(40, 4, 2, 0.6, 0), (64, 8, 2, 0.5, 1),
                                            (50, 8, 1, 0.7, 2), (30, 16, 4, 0.3, 3),
                                            (25, 4, 4, 0.5, 4)])
def test_reroute_greedy_invariants(T, E, k, phi, seed):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((T, E)).astype(np.float32)
    L[:, 0] += 1.5                                  # a popular expert: many overflows
    L[rng.random((T, E)) < 0.1] = 0.25              # and some exact ties
    ids, _ = oracle.topk_gates(L, k, 1)
    C = oracle.capacity(T, E, k, phi)
    ref = oracle.dispatch(ids, E, C)
    out = oracle.dispatch_reroute(L, ids, E, C)
    assert np.array_equal(out["counts"], ref["counts"])
    _reroute_invariants(L, ids, E, C, out, ref)
    assert out["n_rerouted"] == int((ref["route_pos"] < 0).sum()) - int((out["route_pos"] < 0).sum())


def test_reroute_without_overflow_is_the_drop_policy():
    T, E, k = 32, 8, 2
    L = np.random.default_rng(9).standard_normal((T, E)).astype(np.float32)
    ids, _ = oracle.topk_gates(L, k, 1)
    C = oracle.capacity(T, E, k, 4.0)
    ref = oracle.dispatch(ids, E, C)
    out = oracle.dispatch_reroute(L, ids, E, C)
    assert out["n_rerouted"] == 0
    assert np.array_equal(out["route_pos"], ref["route_pos"])
    assert np.array_equal(out["ids"], ids)


# ---------------------------------------------------------------------------
# Overflow policy "queue to the next micro-batch" ([SPK] "Overflow policies":
# the overflowing route is processed in the next micro-batch).  Reading: it
# waits with its expert and gate; in the next call the waiting routes arrive
# before that call's routes and are seated first.

def test_queue_trace_spk():
    """The [SPK] trace (C = 5): t6's route at E1 is the one overflow; under the
    queue policy it waits instead of being lost.  Next micro-batch (the same
    eight assignments again): E1 now has 7 arrivals for 5 seats -- the waiting
    t6 route takes the first seat, then t1..t4; the new t5 and t6 routes to E1
    wait in their arrival order.  Derived by hand from the reading."""
    g = G.load("spk_capacity_trace.txt")
    ids = np.array(G.rows(g["assign"], int), np.int32)
    T, E, k = 8, 4, 2
    C = oracle.capacity(T, E, k, 1.25)
    b1 = oracle.dispatch_queue(ids, E, C)
    assert b1["out_arrival"].tolist() == [5 * k + 0]              # t6's first route (to E1)
    assert b1["kept"].tolist() == [5, 4, 3, 3]
    # batch 2: the queued E1 route arrives first
    q = ids.reshape(-1)[b1["out_arrival"]]
    assert q.tolist() == [0]
    b2 = oracle.dispatch_queue(ids, E, C, q)
    assert b2["counts"].tolist() == [7, 4, 3, 3]
    assert b2["kept"].tolist() == [5, 4, 3, 3]
    lo = int(b2["offsets"][0])
    assert b2["row_arrival"][lo:lo + 5].tolist() == [0] + [1 + t * k for t in range(4)]
    assert b2["pos"][0] == lo                                       # first seat of E1
    assert b2["out_arrival"].tolist() == [1 + 4 * k, 1 + 5 * k]     # t5, t6 of batch 2 at E1


def _queue_run(batches, E, k, phi):
    """Dispatch a run of batches (lists of [T, k] ids) under the queue policy;
    queued routes carry their (batch, route) name."""
    names = np.zeros((0, 2), np.int64)
    qids = np.zeros(0, np.int32)
    runs = []
    for b, ids in enumerate(batches):
        T = ids.shape[0]
        C = oracle.capacity(T, E, k, phi)
        out = oracle.dispatch_queue(ids, E, C, qids)
        Q = qids.shape[0]
        arr_names = np.concatenate([names, np.stack([np.full(T * k, b), np.arange(T * k)], 1)])
        arr_ids = np.concatenate([qids, ids.reshape(-1)]).astype(np.int32)
        runs.append(dict(out=out, Q=Q, C=C, names=arr_names, ids=arr_ids))
        names = arr_names[out["out_arrival"]]
        qids = arr_ids[out["out_arrival"]]
    return runs, names


@pytest.mark.parametrize("k,phi,seed", [(1, 0.6, 0), (2, 0.5, 1), (2, 0.9, 2), (4, 0.4, 3)])
def test_queue_run_invariants(k, phi, seed):
    """Over a run of micro-batches: no expert seats more than C per batch;
    each route is seated exactly once or is still waiting at the end; at each
    expert every seated queued route is ahead of every seated new route, and
    a new route is seated only when no queued route to that expert waits;
    the queue keeps arrival order; no overflow leaves the drop policy."""
    rng = np.random.default_rng(seed)
    E = 6
    batches = []
    for b in range(5):
        T = int(rng.integers(5, 40))
        L = rng.standard_normal((T, E)).astype(np.float32)
        L[:, 0] += 1.0
        batches.append(oracle.topk_gates(L, k, 1)[0])
    runs, left = _queue_run(batches, E, k, phi)
    seen = {}
    for b, run in enumerate(runs):
        out, Q, C = run["out"], run["Q"], run["C"]
        assert (out["kept"] <= C).all()
        pos = out["pos"]
        assert np.array_equal(np.bincount(run["ids"][pos >= 0], minlength=E), out["kept"])
        for a in np.flatnonzero(pos >= 0):
            key = tuple(run["names"][a])
            assert key not in seen
            seen[key] = b
        for e in range(E):
            arr = np.flatnonzero(run["ids"] == e)
            seated = arr[pos[arr] >= 0]
            waiting = arr[pos[arr] < 0]
            # seats go to the earliest arrivals: queued ones first
            assert (seated.size == 0 or waiting.size == 0) or seated.max() < waiting.min()
            assert np.array_equal(pos[seated], out["offsets"][e] + np.arange(seated.size))
        assert np.array_equal(out["out_arrival"], np.flatnonzero(pos < 0))
    total = sum(ids.size for ids in batches)
    assert len(seen) + left.shape[0] == total
    for key in map(tuple, left):
        assert key not in seen
    # no overflow: every batch is the drop policy's, nothing waits
    runs2, left2 = _queue_run(batches, E, k, 8.0)
    assert left2.shape[0] == 0
    for ids, run in zip(batches, runs2):
        ref = oracle.dispatch(ids, E, run["C"])
        assert np.array_equal(run["out"]["pos"], ref["route_pos"].reshape(-1))


def test_queue_layer_run_against_dense_brute_force():
    """A run of fp32 micro-batches with overflow, then one call with no batch
    and no capacity that seats every waiting route.  Each token's output in
    its own batch plus the late rows of its queued routes equals the dense
    fp64 mixture of all its k routes (no capacity) plus the shared expert."""
    rng = np.random.default_rng(11)
    E, k, d, d_ff, d_ffs = 4, 2, 16, 24, 8
    wr = rng.standard_normal((E, d)).astype(np.float32) * 0.5
    br = np.array([1.5, 0.0, -0.5, -1.0], np.float32)
    wg, wu = (rng.standard_normal((E, d_ff, d)).astype(np.float32) / 4 for _ in range(2))
    wd = rng.standard_normal((E, d, d_ff)).astype(np.float32) / 5
    sg, su = (rng.standard_normal((d_ffs, d)).astype(np.float32) / 4 for _ in range(2))
    sd = rng.standard_normal((d, d_ffs)).astype(np.float32) / 3
    xs = [rng.standard_normal((T, d)).astype(np.float32) for T in (12, 9, 15)] + \
        [np.zeros((0, d), np.float32)]
    total = {}
    queue = None
    for b, x in enumerate(xs):
        last = b == len(xs) - 1
        out = oracle.layer_forward_queued(x, wr, br, wg, wu, wd, k, 1, 0.0 if last else 0.6,
                                          queue=queue, tag_base=1000 * b,
                                          ws_gate=None if last else sg, ws_up=None if last else su,
                                          ws_down=None if last else sd)
        for t in range(x.shape[0]):
            total[1000 * b + t] = out["y"][t].copy()
        if queue is not None:
            for q, tag in enumerate(queue["tags"].tolist()):
                total[tag] += out["y_late"][q]
        if not last:
            assert out["out"]["ids"].size > 0 or b > 0    # the run does overflow
        queue = out["out"]
    assert queue["ids"].size == 0                       # the last call seats everyone
    for b, x in enumerate(xs[:-1]):
        ref = dense_mask_layer(torch.from_numpy(x), torch.from_numpy(wr), torch.from_numpy(br),
                               torch.from_numpy(wg), torch.from_numpy(wu), torch.from_numpy(wd),
                               k, 1, 0.0, torch.from_numpy(sg), torch.from_numpy(su),
                               torch.from_numpy(sd))["y"].numpy()
        got = np.stack([total[1000 * b + t] for t in range(x.shape[0])])
        assert np.allclose(got, ref, rtol=1e-5, atol=1e-5), np.abs(got - ref).max()


# ---------------------------------------------------------------------------
# Expert-choice routing ([BEA] "Why MoE Matters for Infrastructure": experts
# pick tokens).  Reading: score = full softmax probability, expert e keeps
# its Ce = min(C, T) best tokens (lower index first on equal scores), gate =
# score.

def _logits_from_p0(p0):
    """Two experts with softmax probabilities (p0, 1 - p0): logits
    (0, ln((1 - p0) / p0)) in closed form."""
    p0 = np.asarray(p0, np.float64)
    L = np.zeros((p0.size, 2), np.float32)
    L[:, 1] = np.log((1.0 - p0) / p0)
    return L


def test_expert_choice_closed_form():
    # expert 0 sees (0.25, 0.5, 0.9, 0.1) -> keeps tokens 2 and 1; expert 1
    # sees (0.75, 0.5, 0.1, 0.9) -> keeps tokens 3 and 0; rows list each
    # expert's tokens in increasing index
    out = oracle.expert_choice(_logits_from_p0([0.25, 0.5, 0.9, 0.1]), 2)
    assert out["Ce"] == 2
    np.testing.assert_allclose(out["scores"][:, 0], [0.25, 0.5, 0.9, 0.1], rtol=1e-6)
    assert out["route_pos"].tolist() == [[-1, 2], [0, -1], [1, -1], [-1, 3]]
    assert out["row_token"].tolist() == [1, 2, 0, 3]


def test_expert_choice_equal_scores_take_lower_tokens():
    out = oracle.expert_choice(np.zeros((5, 2), np.float32), 3)
    assert (out["scores"] == 0.5).all()
    assert out["route_pos"].tolist() == [[0, 3], [1, 4], [2, 5], [-1, -1], [-1, -1]]
    # one expert: every score is 1, so the first Ce tokens are taken
    one = oracle.expert_choice(np.random.default_rng(0).standard_normal((10, 1)).astype(np.float32), 4)
    assert one["route_pos"][:, 0].tolist() == [0, 1, 2, 3, -1, -1, -1, -1, -1, -1]


@pytest.mark.parametrize("T,E,C,seed", [(50, 4, 13, 0), (97, 8, 25, 1), (64, 16, 64, 2),
                                        (33, 3, 40, 3), (200, 32, 7, 4)])
def test_expert_choice_ranking_invariant(T, E, C, seed):
    rng = np.random.default_rng(seed)
    L = (rng.standard_normal((T, E)) * 2.0).astype(np.float32)
    L[rng.integers(0, T, T // 5), :] = 0.0  # whole rows of equal scores (ties)
    out = oracle.expert_choice(L, C)
    S, P = out["scores"], out["route_pos"]
    ref = torch.softmax(torch.from_numpy(L).double(), dim=-1).numpy()
    np.testing.assert_allclose(S, ref, rtol=2e-7, atol=1e-12)
    Ce = min(C, T)
    assert out["Ce"] == Ce
    for e in range(E):
        taken = np.flatnonzero(P[:, e] >= 0)
        assert taken.size == Ce  # every expert holds exactly Ce tokens
        # rows e*Ce .. e*Ce+Ce-1 in increasing token order
        assert P[taken, e].tolist() == list(range(e * Ce, (e + 1) * Ce))
        assert out["row_token"][e * Ce:(e + 1) * Ce].tolist() == taken.tolist()
        left = np.flatnonzero(P[:, e] < 0)
        if taken.size and left.size:
            s_in, s_out = S[taken, e], S[left, e]
            worst_in = s_in.min()
            assert worst_in >= s_out.max()
            # among tokens at the boundary score, the taken ones come first
            tie_in = taken[s_in == worst_in]
            tie_out = left[s_out == worst_in]
            if tie_out.size:
                assert tie_in.max() < tie_out.min()


def test_expert_choice_full_capacity_is_the_soft_mixture():
    # C >= T: every expert takes every token, so y = sum_e p_e E_e(x) + shared,
    # the dense soft mixture -- the brute-force dense-mask layer with k = E
    # and no renormalisation
    w = Workload("ec_dense", T=24, E=4, k=4, d=16, d_ff=24, d_ff_shared=8, dtype="f32",
                 bias="normal")
    inp = make_inputs(w, seed=41)
    out = oracle.layer_forward_expert_choice(inp["x"], inp["w_router"], inp["b_router"],
                                             inp["w_gate"], inp["w_up"], inp["w_down"], C=-1,
                                             ws_gate=inp["ws_gate"], ws_up=inp["ws_up"],
                                             ws_down=inp["ws_down"])
    assert (out["route_pos"] >= 0).all()
    ref = dense_mask_layer(inp["x"], inp["w_router"], inp["b_router"], inp["w_gate"], inp["w_up"],
                           inp["w_down"], k=4, renorm=0, phi=0.0, ws_gate=inp["ws_gate"],
                           ws_up=inp["ws_up"], ws_down=inp["ws_down"])["y"].numpy()
    scale = np.abs(ref).max()
    # the oracle's gates are the fp32 scores (relative rounding 2^-24)
    np.testing.assert_allclose(out["y"], ref, rtol=1e-6, atol=1e-6 * scale)


@pytest.mark.parametrize("dtype,phi", [("bf16", 1.0), ("f32", 0.5)])
def test_expert_choice_layer_against_dense_products(dtype, phi):
    w = Workload("ec_layer", T=40, E=6, k=2, d=24, d_ff=32, d_ff_shared=16, dtype=dtype,
                 bias="normal")
    inp = make_inputs(w, seed=42)
    C = oracle.capacity(w.T, w.E, w.k, phi)
    out = oracle.layer_forward_expert_choice(inp["x"], inp["w_router"], inp["b_router"],
                                             inp["w_gate"], inp["w_up"], inp["w_down"], C,
                                             ws_gate=inp["ws_gate"], ws_up=inp["ws_up"],
                                             ws_down=inp["ws_down"])
    # the choice is the pinned expert_choice of the router logits
    L = oracle.router_logits(inp["x"], inp["w_router"], inp["b_router"])
    ch = oracle.expert_choice(L, C)
    assert np.array_equal(out["route_pos"], ch["route_pos"])
    assert np.array_equal(out["scores"], ch["scores"])
    # y from fp64 library matmuls: every expert on every token, masked
    X = inp["x"].double()
    mask = torch.from_numpy((ch["route_pos"] >= 0).astype(np.float64))
    g = torch.from_numpy(ch["scores"].astype(np.float64)) * mask
    y = swiglu_dense(X, inp["ws_gate"].double(), inp["ws_up"].double(), inp["ws_down"].double())
    for e in range(w.E):
        y = y + g[:, e:e + 1] * swiglu_dense(X, inp["w_gate"][e].double(),
                                             inp["w_up"][e].double(), inp["w_down"][e].double())
    np.testing.assert_allclose(out["y"], y.numpy(), rtol=1e-10, atol=1e-12)
    # a token no expert took gets only the shared expert
    none = np.flatnonzero((ch["route_pos"] < 0).all(axis=1))
    if none.size:
        ysh = swiglu_dense(X, inp["ws_gate"].double(), inp["ws_up"].double(),
                           inp["ws_down"].double()).numpy()
        np.testing.assert_allclose(out["y"][none], ysh[none], rtol=1e-10, atol=1e-12)


def test_expert_choice_empty_batch():
    out = oracle.expert_choice(np.zeros((0, 4), np.float32), 3)
    assert out["Ce"] == 0 and out["row_token"].size == 0 and out["route_pos"].shape == (0, 4)
