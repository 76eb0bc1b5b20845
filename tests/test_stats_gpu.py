"""GPU parity of moe_routing_stats (forward-only routing statistics) against
the CPU oracle.

Each side routes on its own (the logits and expert ids match bit for bit,
which test_parity_gpu checks); the statistics are sums in fp32 on the GPU
and in double in the oracle: scalars and per-expert vectors agree within
fp32 reduction error.  The confidence histogram is integer, but its bins are
decided by a floating-point probability: tokens whose probability lies
within 1e-4 of a bin edge may fall on either side, nothing else may differ.
"""
import numpy as np
import pytest
import torch

import oracle
from tests._gpu import host_inputs, say, to_dev
from workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

NB = 20


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    import routing_dispatch_expert_route_amd as m
    return m


def _gpu_stats(moe, w, inp, alpha, nb):
    d = to_dev(inp)
    s = moe.shape_of(w)
    ws = moe.workspace(s, "cuda")
    ids, gates, logits = moe.route(s, d["x"], d["w_router"], d["b_router"], ws=ws, want_logits=True)
    per = moe.permute(s, d["x"], ids, ws=ws)
    st, hist = moe.routing_stats(s, logits, gates, per["counts"], alpha=alpha, n_bins=nb, ws=ws)
    st2, hist2 = moe.routing_stats(s, logits, gates, per["counts"], alpha=alpha, n_bins=nb, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(st, st2) and torch.equal(hist, hist2), "repeat call differs"
    return moe.stats_dict(s, st, hist)


def _oracle_stats(w, inp, alpha, nb):
    L = oracle.router_logits(inp["x"], inp["w_router"], inp["b_router"])
    ids, gates = oracle.topk_gates(L, w.k, w.renorm)
    counts = np.bincount(ids.ravel(), minlength=w.E).astype(np.int32)
    ref = oracle.routing_stats(L, gates, counts, alpha=alpha, n_bins=nb)
    z = np.exp(L.astype(np.float64) - L.max(axis=1, keepdims=True)).sum(axis=1)
    conf = 1.0 / z
    edge = np.abs(conf * nb - np.round(conf * nb)) < 1e-4
    return ref, int(edge.sum())


def _compare(got, ref, near_edge):
    for n in oracle.STAT_NAMES:
        assert got[n] == pytest.approx(ref[n], rel=1e-4, abs=2e-6), n
    assert np.max(np.abs(got["share"] - ref["share"])) <= 1e-6
    assert np.max(np.abs(got["mean_prob"] - ref["mean_prob"])) <= 2e-6
    assert got["hist"].sum() == ref["hist"].sum()
    assert int(np.abs(got["hist"] - ref["hist"]).sum()) <= 2 * near_edge


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_routing_stats_parity(moe, name):
    w = WORKLOADS[name]
    say(f"[stats] {name}")
    inp = host_inputs(name, routing_only=True)
    got = _gpu_stats(moe, w, inp, 1e-2, NB)
    ref, near = _oracle_stats(w, inp, 1e-2, NB)
    _compare(got, ref, near)


@pytest.mark.parametrize("case", ["empty", "one_token", "e256_k8", "hot", "k1_norenorm"])
def test_routing_stats_edge_cases(moe, case):
    say(f"[stats edge] {case}")
    w = {"empty": Workload("empty", T=0, E=4, k=2, d=64, d_ff=64),
         "one_token": Workload("one_token", T=1, E=8, k=2, d=64, d_ff=64),
         "e256_k8": Workload("e256_k8", T=300, E=256, k=8, d=64, d_ff=32),
         "hot": Workload("hot", T=512, E=32, k=8, d=64, d_ff=32, bias="normal"),
         "k1_norenorm": Workload("k1", T=777, E=16, k=1, d=64, d_ff=32, renorm=0, bias="zipf")}[case]
    inp = make_inputs(w, seed=21, routing_only=True)
    if case == "hot":
        inp["b_router"] = torch.zeros(w.E)
        inp["b_router"][3] = 1e3
    got = _gpu_stats(moe, w, inp, 0.5, 7)
    ref, near = _oracle_stats(w, inp, 0.5, 7)
    _compare(got, ref, near)
    if case == "hot":
        assert got["load_imbalance"] == pytest.approx(w.E / w.k, rel=1e-6)
