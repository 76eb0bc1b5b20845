"""Helpers for the GPU parity tests: device inputs, sampled tokens and the
tolerances the layer is held to (fp32: max abs error 1e-4; bf16: relative
error 2e-2, both as max|d|/max|ref| and as ||d||_2/||ref||_2)."""
import functools
import sys

import numpy as np
import torch

from workloads import WORKLOADS, make_inputs


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=2)
def host_inputs(name, seed=0, routing_only=False):
    return make_inputs(WORKLOADS[name], seed=seed, routing_only=routing_only)


def to_dev(inp):
    return {k: (None if v is None else v.cuda()) for k, v in inp.items()}


def check_y(got, ref, dtype, what="y"):
    """got: torch tensor (any device), ref: float64 numpy array."""
    g = got.detach().float().cpu().double().numpy()
    ref = np.asarray(ref, np.float64)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    if g.size == 0:
        return 0.0, 0.0
    diff = np.abs(g - ref)
    assert np.all(np.isfinite(g)), what
    if dtype == "f32":
        m = float(diff.max())
        assert m <= 1e-4, f"{what}: max abs err {m:.3e} > 1e-4"
        return m, m
    scale = float(np.abs(ref).max())
    max_rel = float(diff.max()) / max(scale, 1e-30)
    l2_rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-30))
    assert max_rel <= 2e-2 and l2_rel <= 2e-2, f"{what}: max_rel {max_rel:.3e} l2_rel {l2_rel:.3e}"
    return max_rel, l2_rel


def sample_tokens(T, route_pos, offsets, row_token, n_random=96, seed=0):
    """First and last tokens, a seeded random set, and the tokens owning the
    first and last packed row of every non-empty expert."""
    rng = np.random.default_rng(seed)
    sel = {0, T - 1}
    sel.update(rng.choice(T, size=min(n_random, T), replace=False).tolist())
    E = len(offsets) - 1
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            sel.add(int(row_token[lo]))
            sel.add(int(row_token[hi - 1]))
    return np.array(sorted(sel), np.int32)


def bits(t):
    """Raw bits of a tensor as a numpy integer array (bit-exact comparisons)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy()
    return t.numpy()
