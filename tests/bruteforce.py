"""Independent fp64 dense-mask reference for tiny shapes (torch CPU).

Used only to pin the oracle.  It is written from the layer's definition in a
different form than the oracle: every expert runs on every token, the
routing is a 0/1 mask, gates come from the full softmax divided by the
selected mass ("Mixture of Experts: Routing, Dispatch, and Load Balancing",
section 3: normalise by total weight), capacity slots come from a cumulative
sum over route one-hots, and all matrix products are library matmuls.
"""
import math

import torch


def _f64(t):
    return None if t is None else t.detach().to(torch.float64)


def swiglu_dense(X, Wg, Wu, Wd):
    """down(SiLU(gate(x)) * up(x)) for all rows of X, float64 matmuls."""
    return (torch.nn.functional.silu(X @ Wg.T) * (X @ Wu.T)) @ Wd.T


def dense_mask_layer(x, w_router, b_router, w_gate, w_up, w_down, k, renorm, phi,
                     ws_gate=None, ws_up=None, ws_down=None):
    X = _f64(x)
    Wr = _f64(w_router)
    T, d = X.shape
    E = Wr.shape[0]
    logits = X @ Wr.T
    if b_router is not None:
        logits = logits + _f64(b_router)
    probs = torch.softmax(logits, dim=-1)
    # full stable sort of the negated logits: ties keep the lower expert index first
    order = torch.sort(-logits, dim=-1, stable=True).indices
    sel = order[:, :k]                                   # [T, k] slot order
    mask = torch.zeros(T, E, dtype=torch.float64)
    mask.scatter_(1, sel, 1.0)
    weights = probs * mask
    if renorm:
        weights = weights / weights.sum(dim=-1, keepdim=True)
    # capacity: slot of a route = number of earlier routes (flat order t*k+j) to its expert
    if phi > 0:
        C = math.ceil(phi * T * k / E)
        onehot = torch.zeros(T * k, E, dtype=torch.float64)
        onehot[torch.arange(T * k), sel.reshape(-1)] = 1.0
        slot = (torch.cumsum(onehot, dim=0) - 1.0)[torch.arange(T * k), sel.reshape(-1)]
        keep = (slot < C).to(torch.float64).reshape(T, k)
        keep_mask = torch.zeros(T, E, dtype=torch.float64)
        keep_mask.scatter_(1, sel, keep)
        weights = weights * keep_mask
    y = torch.zeros(T, d, dtype=torch.float64)
    for e in range(E):
        Ye = swiglu_dense(X, _f64(w_gate[e]), _f64(w_up[e]), _f64(w_down[e]))
        y += weights[:, e:e + 1] * Ye
    if ws_gate is not None:
        y += swiglu_dense(X, _f64(ws_gate), _f64(ws_up), _f64(ws_down))
    gap = None
    if k < E:
        srt = torch.sort(logits, dim=-1, descending=True).values
        gap = (srt[:, :k] - srt[:, 1:k + 1]).min(dim=-1).values
    return dict(y=y, ids=sel.to(torch.int32), weights=weights, logits=logits, gap=gap)
