"""moe_layer_forward_noalloc (the layer with the library's fixed device
array as its workspace, for callers that cannot allocate) against
moe_layer_forward (the caller-workspace entry point it shares its kernels
with): two calls in a row, the second on a smaller batch, each bit-identical
to moe_layer_forward on the same inputs -- y and every routing output.  A
shape whose workspace exceeds the array is rejected on the host."""
import numpy as np
import pytest
import torch

from tests._gpu import bits, say
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import routing_dispatch_expert_route_amd as m
    return m


def _run_both(moe, w, seed):
    inp = make_inputs(w, seed=seed)
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    s = moe.shape_of(w)
    assert moe.workspace_bytes(s) <= moe.NOALLOC_SCRATCH_BYTES
    args = (s, d["x"], d["w_router"], d["b_router"], d["w_gate"], d["w_up"], d["w_down"],
            d["ws_gate"], d["ws_up"], d["ws_down"])
    y0, r0 = moe.layer_forward_noalloc(*args, return_routing=True)
    y1, r1 = moe.layer_forward(*args, return_routing=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y0), bits(y1)), f"{w.name}: y differs"
    for k in r1:
        assert np.array_equal(bits(r0[k]), bits(r1[k])), f"{w.name}: {k} differs"
    assert torch.isfinite(y0.float()).all()
    return y0


@pytest.mark.parametrize("first,second", [
    # capacity with drops and a shared expert, then a smaller batch
    (Workload("noalloc_a", T=1000, E=8, k=2, d=512, d_ff=1024, d_ff_shared=256, phi=1.0,
              bias="normal"),
     Workload("noalloc_b", T=300, E=8, k=2, d=512, d_ff=1024, d_ff_shared=256, phi=1.0,
              bias="normal")),
    # the Switch shape (top-1, the down GEMM writes y), then fewer tokens
    (Workload("noalloc_switch", T=4096, E=8, k=1, d=768, d_ff=3072, renorm=0, phi=1.25,
              bias="normal"),
     Workload("noalloc_switch_small", T=515, E=8, k=1, d=768, d_ff=3072, renorm=0, phi=1.25,
              bias="normal")),
])
def test_noalloc_matches_layer_forward_twice(moe, first, second):
    say(f"[noalloc] {first.name} then {second.name}")
    y_first = _run_both(moe, first, seed=41)
    _run_both(moe, second, seed=42)
    assert y_first.shape[0] == first.T


def test_noalloc_rejects_shapes_beyond_the_array(moe):
    say("[noalloc] too large")
    w = Workload("noalloc_big", T=8192, E=8, k=2, d=4096, d_ff=14336)
    s = moe.shape_of(w)
    assert moe.workspace_bytes(s) > moe.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(1, device="cuda")  # never read: rejected before any launch
    with pytest.raises(moe.MoeError) as ei:
        moe._check(moe._lib.moe_layer_forward_noalloc(
            moe.ctypes.byref(s), *([x.data_ptr()] * 6), None, None, None, x.data_ptr(),
            None, None, None, None, None), "moe_layer_forward_noalloc")
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
