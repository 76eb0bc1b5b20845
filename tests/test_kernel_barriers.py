"""Every HIP kernel of the library, compiled for gfx950 as the build compiles
it, has no workgroup barrier inside a loop the compiler made divergent (the
scan in tests/_asm_scan.py).  Such a loop lets one wave meet a barrier a
different number of times than the others: a hang on the GPU, caught here on
the host from the assembly alone.

The scan itself is pinned on two small kernels with the same round structure
(per-route loop, block-wide OR, barrier, per-route loop): with per-lane loop
bounds the compiler builds a divergent round loop around the barriers, with
wave-uniform bounds and a scalar exit it does not."""
import concurrent.futures as cf
import importlib.util
import os
import shutil
import subprocess

import pytest

from tests._asm_scan import divergent_barrier_loops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "routing_dispatch_expert_route_amd", "csrc")

pytestmark = pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="needs hipcc")


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "moe_build", os.path.join(ROOT, "routing_dispatch_expert_route_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _asm(src, out, extra=()):
    b = _build_module()
    cmd = [b.HIPCC] + b.COMMON + b.DEVICE_ONLY + list(extra) + ["--cuda-device-only", "-S",
                                                                src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return f.read()


ROUNDS = r"""
#include <hip/hip_runtime.h>
__global__ __launch_bounds__(1024) void rounds_per_lane_bound(int* p, int n) {
  __shared__ unsigned char s[4096];
  __shared__ int t[64];
  for (int j = threadIdx.x; j < n; j += 1024) s[j] = 0;
  if (threadIdx.x < 64) t[threadIdx.x] = 0;
  __syncthreads();
  for (;;) {
    int any = 0;
    for (int j = threadIdx.x; j < n; j += 1024) {
      if (s[j] < 3) { s[j] = s[j] + 1; atomicAdd(&t[j & 63], 1); any = 1; }
    }
    if (!__syncthreads_or(any)) break;
    if (threadIdx.x < 64) t[threadIdx.x] >>= 1;
    __syncthreads();
    for (int j = threadIdx.x; j < n; j += 1024)
      if (t[j & 63] & 1) s[j] = s[j] + 1;
  }
  for (int j = threadIdx.x; j < n; j += 1024) p[j] = s[j];
}
__global__ __launch_bounds__(1024) void rounds_uniform_bound(int* p, int n) {
  __shared__ unsigned char s[4096];
  __shared__ int t[64];
  for (int j = threadIdx.x; j < n; j += 1024) s[j] = 0;
  if (threadIdx.x < 64) t[threadIdx.x] = 0;
  __syncthreads();
  for (;;) {
    int any = 0;
    for (int j0 = 0; j0 < n; j0 += 1024) {
      const int j = j0 + threadIdx.x;
      if (j < n && s[j] < 3) { s[j] = s[j] + 1; atomicAdd(&t[j & 63], 1); any = 1; }
    }
    if (!__builtin_amdgcn_readfirstlane(__syncthreads_or(any))) break;
    if (threadIdx.x < 64) t[threadIdx.x] >>= 1;
    __syncthreads();
    for (int j0 = 0; j0 < n; j0 += 1024) {
      const int j = j0 + threadIdx.x;
      if (j < n && (t[j & 63] & 1)) s[j] = s[j] + 1;
    }
  }
  for (int j = threadIdx.x; j < n; j += 1024) p[j] = s[j];
}
"""


def test_scan_flags_a_divergent_round_loop(tmp_path):
    src = tmp_path / "rounds.hip"
    src.write_text(ROUNDS)
    text = _asm(str(src), str(tmp_path / "rounds.s"))
    kernels = {k for k, _ in divergent_barrier_loops(text)}
    assert any("rounds_per_lane_bound" in k for k in kernels), kernels
    assert not any("rounds_uniform_bound" in k for k in kernels), kernels


def test_no_barrier_in_a_divergent_loop(tmp_path):
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    assert srcs
    workers = min(len(srcs), max(1, (os.cpu_count() or 2) // 2))
    with cf.ThreadPoolExecutor(workers) as ex:
        texts = dict(zip(srcs, ex.map(
            lambda f: _asm(os.path.join(CSRC, f), str(tmp_path / (f + ".s"))), srcs)))
    bad = {f: divergent_barrier_loops(t) for f, t in texts.items()}
    bad = {f: v for f, v in bad.items() if v}
    assert not bad, bad
    shutil.rmtree(tmp_path, ignore_errors=True)
