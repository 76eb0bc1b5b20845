"""Seeded synthetic inputs for the MoE layer workloads.

This module only draws inputs; it holds none of the layer's arithmetic.  It
is shared by the tests, the smoke check and the benchmark, and feeds the
same bytes to the HIP library and to the CPU oracle.

Workloads (shapes from the pages' model families; no checkpoint or prompt
set is available, so seeded random tensors of the same shapes stand in):

  tiny            E=4  k=2 T=64    d=128  d_ff=256   fp32, renormalised, no capacity
  switch_phi1     E=8  k=1 T=4096  d=768  d_ff=3072  bf16, bias ~ N(0,1), phi = 1.0,
                  gate = full softmax probability (top-1, no renormalisation)
  switch_phi125   as above with phi = 1.25
  granite_1412    E=32 k=8 T=1412  d=1024 d_ff=512   bf16, renormalised, dropless
  granite_16384   as above with T=16384
  mixtral_decode  E=8  k=2 T=16    d=4096 d_ff=14336 bf16, renormalised, dropless
  mixtral_prefill as above with T=8192
  shared64        E=64 k=2 T=8192  d=2048 d_ff=1408, shared expert d_ff=2816, bf16,
                  router bias b_e = -ln(e+1) (Zipf s=1 popularity), renormalised, dropless

Recipe: one torch CPU generator seeded with `seed` (default 0).  Draw order:
x[T,d]; W_router[E,d]; the router bias (switch only); then per expert e:
W_gate[e], W_up[e], W_down[e]; then the shared W_gate, W_up, W_down.  Every
draw is torch.randn in float32.  x stays N(0,1); every weight matrix is
scaled by 1/sqrt(d) (variance 1/d); bf16 workloads then round to bf16
(round-to-nearest-even).  The router bias stays float32.
"""
from dataclasses import dataclass, field, replace
import math
from typing import Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    E: int
    k: int
    d: int
    d_ff: int
    d_ff_shared: int = 0
    dtype: str = "bf16"          # "f32" or "bf16"
    renorm: int = 1
    phi: float = 0.0             # <= 0: no capacity limit
    bias: Optional[str] = None   # None, "normal", "zipf"
    note: str = ""

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", T=64, E=4, k=2, d=128, d_ff=256, dtype="f32", renorm=1),
    "switch_phi1": Workload("switch_phi1", T=4096, E=8, k=1, d=768, d_ff=3072,
                            renorm=0, phi=1.0, bias="normal"),
    "switch_phi125": Workload("switch_phi125", T=4096, E=8, k=1, d=768, d_ff=3072,
                              renorm=0, phi=1.25, bias="normal"),
    "granite_1412": Workload("granite_1412", T=1412, E=32, k=8, d=1024, d_ff=512),
    "granite_16384": Workload("granite_16384", T=16384, E=32, k=8, d=1024, d_ff=512),
    "mixtral_decode": Workload("mixtral_decode", T=16, E=8, k=2, d=4096, d_ff=14336),
    "mixtral_prefill": Workload("mixtral_prefill", T=8192, E=8, k=2, d=4096, d_ff=14336),
    "shared64": Workload("shared64", T=8192, E=64, k=2, d=2048, d_ff=1408,
                         d_ff_shared=2816, bias="zipf"),
}


def make_inputs(w: Workload, seed: int = 0, device: str = "cpu", zero_routed: bool = False,
                routing_only: bool = False):
    """Draw the workload's inputs on the CPU (then move them to `device`).

    Returns a dict with x, w_router, b_router (or None), w_gate, w_up,
    w_down, ws_gate, ws_up, ws_down (None without a shared expert).
    routing_only stops after the router tensors (the same x, W_router and
    bias as a full draw, since those come first); expert weights are None.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    dt = w.torch_dtype
    scale = 1.0 / math.sqrt(w.d)

    def draw(*shape, scaled=True):
        t = torch.randn(*shape, generator=g, dtype=torch.float32)
        if scaled:
            t.mul_(scale)
        return t.to(dt)

    x = draw(w.T, w.d, scaled=False)
    w_router = draw(w.E, w.d)
    b_router = None
    if w.bias == "normal":
        b_router = torch.randn(w.E, generator=g, dtype=torch.float32)
    elif w.bias == "zipf":
        # log-prior proportional to 1/rank: expert 0 most popular
        b_router = -torch.log(torch.arange(1, w.E + 1, dtype=torch.float64)).to(torch.float32)
    if routing_only:
        out = dict(x=x, w_router=w_router, b_router=b_router, w_gate=None, w_up=None,
                   w_down=None, ws_gate=None, ws_up=None, ws_down=None)
        if device != "cpu":
            out = {k_: (None if v is None else v.to(device)) for k_, v in out.items()}
        return out
    w_gate = torch.empty(w.E, w.d_ff, w.d, dtype=dt)
    w_up = torch.empty(w.E, w.d_ff, w.d, dtype=dt)
    w_down = torch.empty(w.E, w.d, w.d_ff, dtype=dt)
    for e in range(w.E):
        w_gate[e] = draw(w.d_ff, w.d)
        w_up[e] = draw(w.d_ff, w.d)
        w_down[e] = draw(w.d, w.d_ff)
    if zero_routed:
        w_down.zero_()
    ws_gate = ws_up = ws_down = None
    if w.d_ff_shared > 0:
        ws_gate = draw(w.d_ff_shared, w.d)
        ws_up = draw(w.d_ff_shared, w.d)
        ws_down = draw(w.d, w.d_ff_shared)
    out = dict(x=x, w_router=w_router, b_router=b_router, w_gate=w_gate, w_up=w_up,
               w_down=w_down, ws_gate=ws_gate, ws_up=ws_up, ws_down=ws_down)
    if device != "cpu":
        out = {k_: (None if v is None else v.to(device)) for k_, v in out.items()}
    return out

