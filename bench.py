"""Benchmark of the MoE layer forward (route + pack + compute + combine) on one
MI355X.

A step is one moe_layer_forward call over one batch of seeded synthetic
input, inputs resident in HBM.  By default each step uses the next of
several device copies of the expert weights (enough copies to exceed the
256 MB last-level cache), as consecutive MoE layers of a model would: the
weights are read cold from HBM every step.

Prints ONE JSON line:
  value          whole-step tokens/s: T / (wall time of the K timed steps / K),
                 the steps bracketed by device synchronisations
  step_us        p10 / median / p90 of the same K steps' GPU time, from
                 hipEvents recorded on the library's stream at the start and
                 end of every timed step
  roofline       dominant kernel (grouped GEMM 1, gate+up+SwiGLU) against
                 the MI355X bf16 dense MFMA peak or the HBM peak, timed with
                 hipEvents recorded on the library's stream around it in
                 every timed step; traffic = HBM bytes per launch from the
                 committed rocprofv3 counter summary (null when absent or
                 taken on another version of the GEMM source)
  cpu_baseline   the CPU oracle on a bounded sample of the same workload
  stages_us      mean per-stage times of a second, fully event-marked pass
                 (stage_step_us_percentiles: that pass's per-step times)
  routing_stats  forward-only routing statistics of the batch (Switch
                 aux-loss value with alpha 1e-2, demand imbalance, ...) and
                 the time of one moe_routing_stats call

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Counter support (HBM traffic of GEMM 1):
  --copy-calibration MIB   after the run, copy a MIB-MiB device buffer
                           three times (plain blit copies of known size, the
                           scale for FETCH_SIZE / WRITE_SIZE)
  --traffic-from F W       read two rocprofv3 --pmc csv output folders (F:
                           FETCH_SIZE pass, W: WRITE_SIZE pass, both of
                           `bench.py --copy-calibration ...`) and write the
                           per-launch traffic summary of GEMM 1 (no GPU use)
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 (vector)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
MALL_BYTES = 256 << 20
# The largest configuration that fits one GPU: Mixtral-like prefill (E=8,
# top-2, d=4096, d_ff=14336, T=8192; 5.77 TFLOP per step, MFMA-bound).
DEFAULT_WORKLOAD = "mixtral_prefill"
METRIC = "MoE layer tokens/s at 1 GPU; % of MFMA peak (large T) / HBM BW (small T)"
STAGES = ["route", "permute", "gemm1_gate_up_swiglu", "gemm2_down", "shared_expert", "combine"]


def _hip():
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


def gemm1_model(w, kept_rows, active_experts):
    """Algorithmic flops and bytes of grouped GEMM 1 (gate + up + SwiGLU):
    flops = kept * 4*d*d_ff; bytes = active experts' gate+up weights + the
    kept token rows read + the hidden rows written."""
    eb = 2 if w.dtype == "bf16" else 4
    flops = kept_rows * 4.0 * w.d * w.d_ff
    byts = active_experts * 2.0 * w.d * w.d_ff * eb + kept_rows * (w.d + w.d_ff) * eb
    return flops, byts


def layer_model(w, kept_rows, active_experts):
    """Algorithmic flops and bytes of the whole layer ("Measurement"):
    F = kept*6*d*d_ff + T*6*d*d_ffs + 2*T*d*E (kept routes only, no padding);
    B = active experts' weights + the shared expert's + router weights + x
    read + y written + 12 bytes of route metadata per route."""
    eb = 2 if w.dtype == "bf16" else 4
    flops = (kept_rows * 6.0 * w.d * w.d_ff + w.T * 6.0 * w.d * w.d_ff_shared
             + 2.0 * w.T * w.d * w.E)
    byts = (active_experts * 3.0 * w.d * w.d_ff * eb + 3.0 * w.d * w.d_ff_shared * eb
            + w.E * w.d * eb + 2.0 * w.T * w.d * eb + w.T * w.k * 12.0)
    return flops, byts


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


GEMM_SRC = os.path.join(ROOT, "routing_dispatch_expert_route_amd", "csrc", "gemm.hip")
N_CAL = 3  # calibration copies at the end of a --copy-calibration run


def _gemm_sha():
    return hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"gemm1_{workload}_traffic.json")


def traffic_from_profile(workload):
    """HBM bytes per GEMM-1 launch from the committed rocprofv3 counter
    summary, or None when absent or taken on a different gemm.hip."""
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("gemm_hip_sha256") != _gemm_sha():
        return None
    return rec["traffic_bytes_per_launch"]


def _is_gemm1(name, shared=False):
    # gemm_bf16_kernel<tile and pipeline sizes..., SWIGLU, GATHER, PARTIAL> or
    # gemm_pp_kernel<SWIGLU, GATHER>: GEMM 1 of the whole-layer path is the
    # SwiGLU instance that gathers token rows -- or, on the 256x256 tile with
    # a wide d_ff, the one that reads the rows packed first (the same name as
    # a shared expert's GEMM 1 on that tile, so only without a shared expert)
    if "gemm_pp_kernel<" in name:
        args = [a.strip() for a in name.split("<", 1)[1].split(">", 1)[0].split(",")]
        return args == ["true", "true"] or (args == ["true", "false"] and not shared)
    if "gemm_bf16_kernel<" not in name:
        return False
    args = [a.strip() for a in name.split("<", 1)[1].split(">", 1)[0].split(",")]
    return len(args) >= 3 and args[-3] == "true" and args[-2] == "true"


def _counter_rows(folder, counter):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)):
        rows += [r for r in csv.DictReader(open(f)) if r["Counter_Name"] == counter]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    if not rows:
        raise SystemExit(f"no {counter} rows under {folder}")
    return rows


def traffic_summary(fetch_dir, write_dir, workload, cal_mib, out_path):
    """Per-launch HBM bytes of GEMM 1 from two counter passes, each counter
    scaled by what it reads for the calibration copies (known bytes)."""
    from workloads import WORKLOADS
    res = {"workload": workload, "gemm_hip_sha256": _gemm_sha(), "calibration_mib": cal_mib}
    known = cal_mib * 1024.0  # KiB read (and written) by one calibration copy
    for key, folder, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = _counter_rows(folder, counter)
        shared = WORKLOADS[workload].d_ff_shared > 0 if workload in WORKLOADS else True
        g1 = [float(r["Counter_Value"]) for r in rows if _is_gemm1(r["Kernel_Name"], shared)]
        cal = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]][-N_CAL:]
        if not g1 or len(cal) < N_CAL:
            raise SystemExit(f"{counter}: {len(g1)} GEMM-1 and {len(cal)} calibration dispatches")
        res[f"{key}_kib"] = sum(g1) / len(g1)
        res[f"{key}_dispatches"] = len(g1)
        res[f"{key}_copy_kib"] = sum(cal) / len(cal)
        res[f"{key}_scale"] = known / res[f"{key}_copy_kib"]
    res["traffic_bytes_per_launch"] = 1024.0 * (res["fetch_kib"] * res["fetch_scale"]
                                                 + res["write_kib"] * res["write_scale"])
    with open(out_path, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(res))


def cpu_baseline(w, inp, seconds, choice=False):
    import numpy as np
    import oracle
    cores = int(os.environ.get("OMP_NUM_THREADS") or len(os.sched_getaffinity(0)))

    def run(n):
        sel = np.arange(n, dtype=np.int32)
        t0 = time.perf_counter()
        if choice:
            oracle.layer_forward_expert_choice(
                inp["x"], inp["w_router"], inp["b_router"], inp["w_gate"], inp["w_up"],
                inp["w_down"], oracle.capacity(w.T, w.E, w.k, w.phi), inp["ws_gate"],
                inp["ws_up"], inp["ws_down"], sel=sel)
        else:
            oracle.layer_forward(inp["x"], inp["w_router"], inp["b_router"], inp["w_gate"],
                                 inp["w_up"], inp["w_down"], w.k, w.renorm, w.phi, inp["ws_gate"],
                                 inp["ws_up"], inp["ws_down"], sel=sel)
        return time.perf_counter() - t0

    t_route = run(0)                      # routing of all T tokens, no FFN
    # grow the FFN sample geometrically until it takes a quarter of the
    # budget, then extrapolate to the budget (the whole run stays within
    # about 1.5x the budget however slow a token is)
    n = min(w.T, max(1, cores))
    while True:
        t = run(n)
        if n == w.T or t >= seconds / 4:
            break
        n = min(w.T, 4 * n)
    grow = (seconds - t_route) / max(t - t_route, 1e-3)
    if grow > 1.25 and n < w.T:
        n = int(min(w.T, n * grow))
        t = run(n)
    reps = 1
    if n == w.T:                          # the whole workload fits: repeat it
        while t < seconds:
            t += run(n)
            reps += 1
    what = (f"all {w.T} tokens of {w.name} (full layer), {reps} passes" if n == w.T else
            f"first {n} of {w.T} tokens of {w.name} (routing of all {w.T} tokens, "
            f"expert FFN + combine of the {n})")
    return {"value": n * reps / t, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{what}, {t:.1f} s wall", "cpu_model": _cpu_model()}


def blas_reference(w, kept, steps, dev):
    """The expert GEMMs' shapes on the vendor library (torch.nn.functional.linear
    in bf16, i.e. hipBLASLt): for every active expert e, its m_e rows times
    [W_gate; W_up][e]^T (one GEMM of 2*d_ff outputs), then m_e rows times
    W_down[e]^T.  A dense-GEMM reference for this GPU's reachable MFMA rate on
    the same per-expert shapes -- no SwiGLU, no gather, one launch per expert
    -- timed with events around the gate/up and the down launches of each
    pass.  Not part of the MoE path."""
    import torch
    import torch.nn.functional as F
    g = torch.Generator(device="cpu").manual_seed(1)
    act = [int(m) for m in kept.tolist() if m > 0]
    wgu = [torch.randn(2 * w.d_ff, w.d, generator=g).to(torch.bfloat16).to(dev) for _ in act]
    wd = [torch.randn(w.d, w.d_ff, generator=g).to(torch.bfloat16).to(dev) for _ in act]
    xs = [torch.randn(m, w.d, generator=g).to(torch.bfloat16).to(dev) for m in act]
    hs = [torch.randn(m, w.d_ff, generator=g).to(torch.bfloat16).to(dev) for m in act]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * steps)]

    def one_pass():
        for x_, wg_ in zip(xs, wgu):
            F.linear(x_, wg_)

    def down_pass():
        for h_, wd_ in zip(hs, wd):
            F.linear(h_, wd_)

    for _ in range(2):
        one_pass()
        down_pass()
    torch.cuda.synchronize()
    for i in range(steps):
        ev[3 * i].record()
        one_pass()
        ev[3 * i + 1].record()
        down_pass()
        ev[3 * i + 2].record()
    torch.cuda.synchronize()
    t1 = sorted(ev[3 * i].elapsed_time(ev[3 * i + 1]) for i in range(steps))[steps // 2]
    t2 = sorted(ev[3 * i + 1].elapsed_time(ev[3 * i + 2]) for i in range(steps))[steps // 2]
    rows = sum(act)
    f1 = 2.0 * rows * w.d * 2 * w.d_ff
    f2 = 2.0 * rows * w.d_ff * w.d

    # The gate/up shapes again with nothing in between: the per-expert passes
    # back to back, and one dense GEMM over all the rows (one weight matrix)
    # back to back -- what the library sustains when the MFMA units stay busy
    # for milliseconds, as the grouped GEMM 1 does.
    def back_to_back(fn):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        fn()
        torch.cuda.synchronize()
        evs[0].record()
        for i in range(steps):
            fn()
            evs[i + 1].record()
        torch.cuda.synchronize()
        return sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))[steps // 2]

    t_seq = back_to_back(one_pass)
    x_all = torch.cat(xs)
    t_dense = back_to_back(lambda: F.linear(x_all, wgu[0]))
    return {"library": "torch.nn.functional.linear bf16 (hipBLASLt)", "experts": len(act),
            "rows": rows, "gate_up_ms": round(t1, 4), "gate_up_tflops": round(f1 / t1 / 1e9, 1),
            "down_ms": round(t2, 4), "down_tflops": round(f2 / t2 / 1e9, 1),
            "gate_up_back_to_back_ms": round(t_seq, 4),
            "gate_up_back_to_back_tflops": round(f1 / t_seq / 1e9, 1),
            "gate_up_dense_ms": round(t_dense, 4),
            "gate_up_dense_tflops": round(f1 / t_dense / 1e9, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--weight-sets", type=int, default=0,
                    help="device copies of the weights cycled per step (0 = enough to exceed the LLC)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-stages", action="store_true")
    ap.add_argument("--padded", action="store_true",
                    help="fixed-shape [E, C, d] dispatch buffer instead of packed rows")
    ap.add_argument("--reroute", action="store_true",
                    help="reroute overflow policy (dropped routes move to the next-best expert with room)")
    ap.add_argument("--choice", action="store_true",
                    help="expert-choice routing (each expert keeps its top-C tokens; full softmax "
                         "gates, capacity factor 1 when the workload has none)")
    ap.add_argument("--queue", action="store_true",
                    help="queue-to-the-next-micro-batch overflow policy: each step processes the "
                         "batch plus the routes one earlier batch left waiting")
    ap.add_argument("--phi", type=float, default=None,
                    help="override the workload's capacity factor (0: no capacity); the line's "
                         "config names the value, and no committed traffic figure applies")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay timing (graph_ms_per_step)")
    ap.add_argument("--blas-reference", action="store_true",
                    help="also time the expert GEMMs' per-expert shapes on hipBLASLt "
                         "(blas_reference: a dense-GEMM reference, not the MoE path)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--traffic-out", default=None)
    args = ap.parse_args()

    if args.traffic_from:
        traffic_summary(args.traffic_from[0], args.traffic_from[1], args.workload,
                        args.copy_calibration or 256,
                        args.traffic_out or traffic_path(args.workload))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import routing_dispatch_expert_route_amd as moe
    from workloads import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    if args.phi is not None:
        w = w.with_(phi=args.phi)
    if args.choice:  # expert choice needs a capacity and full softmax gates
        w = w.with_(renorm=0, phi=w.phi if w.phi > 0 else 1.0)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_inputs(w, seed=0)
    d = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    s = moe.shape_of(w)
    eb = 2 if w.dtype == "bf16" else 4
    wbytes = (w.E * 3 * w.d * w.d_ff + 3 * w.d * w.d_ff_shared) * eb
    nsets = args.weight_sets or max(1, -(-2 * MALL_BYTES // max(wbytes, 1)))
    nsets = min(nsets, max(1, int(torch.cuda.mem_get_info()[0] * 0.6 // max(wbytes, 1))))
    sets = [d] + [{k: (v.clone() if (v is not None and k.startswith("w")) else v)
                   for k, v in d.items()} for _ in range(nsets - 1)]
    ws = moe.workspace(s, dev)
    y = torch.empty(w.T, w.d, dtype=w.torch_dtype, device=dev)
    stream = torch.cuda.current_stream()

    # queue policy: the routes one earlier batch (the same tokens) left waiting
    # arrive with every step's batch
    queue = qbufs = None
    if args.queue:
        _, _, queue = moe.layer_forward_queued(s, d["x"], d["w_router"], d["b_router"],
                                               d["w_gate"], d["w_up"], d["w_down"], d["ws_gate"],
                                               d["ws_up"], d["ws_down"])
        qbufs = moe.queue_buffers(s, queue["ids"].shape[0], dev)

    def timed(p, events):
        if args.queue:
            moe.layer_forward_queued_timed(s, p["x"], p["w_router"], p["b_router"], p["w_gate"],
                                           p["w_up"], p["w_down"], p["ws_gate"], p["ws_up"],
                                           p["ws_down"], queue, qbufs, events, stream=stream)
            return
        moe.layer_forward_timed(s, p["x"], p["w_router"], p["b_router"], p["w_gate"], p["w_up"],
                                p["w_down"], p["ws_gate"], p["ws_up"], p["ws_down"], y, ws,
                                events, stream=stream, padded=args.padded, reroute=args.reroute,
                                choice=args.choice)

    def step(i):
        p = sets[i % nsets]
        if args.queue:
            timed(p, [None] * 7)
            return
        if args.choice:
            moe.layer_forward_expert_choice(s, p["x"], p["w_router"], p["b_router"], p["w_gate"],
                                            p["w_up"], p["w_down"], p["ws_gate"], p["ws_up"],
                                            p["ws_down"], y=y, ws=ws)
            return
        moe.layer_forward(s, p["x"], p["w_router"], p["b_router"], p["w_gate"], p["w_up"],
                          p["w_down"], p["ws_gate"], p["ws_up"], p["ws_down"], y=y, ws=ws,
                          padded=args.padded, reroute=args.reroute)

    # routing statistics for the work model
    _, rt = moe.layer_forward(s, d["x"], d["w_router"], d["b_router"], d["w_gate"], d["w_up"],
                              d["w_down"], d["ws_gate"], d["ws_up"], d["ws_down"],
                              return_routing=True)
    if args.reroute:
        _, rt_r = moe.layer_forward(s, d["x"], d["w_router"], d["b_router"], d["w_gate"],
                                    d["w_up"], d["w_down"], d["ws_gate"], d["ws_up"],
                                    d["ws_down"], return_routing=True, reroute=True)
    counts = rt["counts"].cpu().long()
    C, _ = moe.capacity(s)
    kept = counts.clamp(max=C) if C >= 0 else counts
    if args.reroute:  # seated rows per expert after rerouting
        seated = rt_r["route_pos"].cpu().flatten() >= 0
        kept = torch.bincount(rt_r["expert_ids"].cpu().flatten().long()[seated], minlength=w.E)
    if args.choice:  # every expert holds exactly Ce rows
        kept = torch.full((w.E,), moe.choice_capacity(s), dtype=torch.long)
    n_wait = None
    if args.queue:  # seated arrivals per expert (queued routes first)
        _, _, q_out, rt_q = moe.layer_forward_queued(
            s, d["x"], d["w_router"], d["b_router"], d["w_gate"], d["w_up"], d["w_down"],
            d["ws_gate"], d["ws_up"], d["ws_down"], queue=queue, return_routing=True)
        arr_ids = torch.cat([queue["ids"], rt_q["expert_ids"].flatten()]).cpu().long()
        seated = rt_q["route_pos"].cpu() >= 0
        kept = torch.bincount(arr_ids[seated], minlength=w.E)
        n_wait = int(q_out["ids"].shape[0])
    kept_rows = int(kept.sum())
    active = int((kept > 0).sum())

    hip = _hip()

    def new_events(n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert hip.hipEventCreate(ctypes.byref(e)) == 0
            evs.append(e.value)
        return evs

    def elapsed_us(a, b):
        f = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(f), a, b) == 0
        return f.value * 1e3

    # timed region: K steps, each bracketed by hipEvents on the library's
    # stream, and GEMM 1 inside it too (the other stage boundaries are not
    # marked here)
    K = args.steps
    ev = new_events(4 * K)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        e4 = ev[4 * i:4 * i + 4]
        timed(sets[i % nsets], [e4[0], None, e4[1], e4[2], None, None, e4[3]])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / K
    value = w.T / (ms / 1e3)
    g1_us = sum(elapsed_us(ev[4 * i + 1], ev[4 * i + 2]) for i in range(K)) / K
    step_us = sorted(elapsed_us(ev[4 * i], ev[4 * i + 3]) for i in range(K))
    for e in ev:
        hip.hipEventDestroy(e)

    def pct(v, q):
        return round(v[min(len(v) - 1, int(q * len(v)))], 2)

    step_ev = {"p10": pct(step_us, 0.1), "median": pct(step_us, 0.5), "p90": pct(step_us, 0.9)}

    # the same steps replayed from a HIP graph (one captured step per weight
    # set, replayed until K steps ran): the launch sequence without the host,
    # reported beside the eager value
    graph_ms = None
    if not args.no_graph and not args.queue:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(nsets):
                step(i)
        reps = max(1, -(-K // nsets))
        g.replay()
        torch.cuda.synchronize()
        tg0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - tg0) * 1e3 / (reps * nsets)
        del g

    # per-stage times: a second pass with every stage boundary marked
    stages = None
    step_pct = None
    warm_ms = None
    if not args.no_stages:
        evs = new_events(K * 7)
        torch.cuda.synchronize()
        for i in range(K):
            timed(sets[i % nsets], evs[7 * i:7 * i + 7])
        torch.cuda.synchronize()
        acc = [0.0] * 6
        per_step = []
        for i in range(K):
            for j in range(6):
                acc[j] += elapsed_us(evs[7 * i + j], evs[7 * i + j + 1])
            per_step.append(elapsed_us(evs[7 * i], evs[7 * i + 6]))
        for e in evs:
            hip.hipEventDestroy(e)
        stages = {n: round(a / K, 2) for n, a in zip(STAGES, acc)}
        per_step.sort()
        step_pct = {"p10": pct(per_step, 0.1), "p50": pct(per_step, 0.5),
                    "p90": pct(per_step, 0.9)}

        # warm caches: the same K steps on one weight set (MALL-resident
        # when the weights fit), labelled as such
        torch.cuda.synchronize()
        tw0 = time.perf_counter()
        for i in range(K):
            timed(sets[0], [None] * 7)
        torch.cuda.synchronize()
        warm_ms = (time.perf_counter() - tw0) * 1e3 / K

    # forward-only routing statistics of the bench batch: one extra pass over
    # the route outputs (router logits requested from moe_route)
    rstats = None
    if not args.no_stages:
        ids_, gates_, logits_ = moe.route(s, d["x"], d["w_router"], d["b_router"], ws=ws,
                                          want_logits=True)
        counts_ = moe.permute(s, d["x"], ids_, ws=ws)["counts"]
        outs = moe.routing_stats(s, logits_, gates_, counts_, alpha=1e-2, n_bins=20, ws=ws)
        ev = new_events(2)
        torch.cuda.synchronize()
        hip_rec = hip.hipEventRecord
        hip_rec.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        # the calls are short next to their host-side marshalling: keep the
        # GPU busy while they are queued, so the events time the GPU only
        torch.cuda._sleep(int(K * 2e5))
        hip_rec(ev[0], ctypes.c_void_p(stream.cuda_stream))
        for _ in range(K):
            moe.routing_stats(s, logits_, gates_, counts_, alpha=1e-2, n_bins=20, ws=ws, out=outs)
        hip_rec(ev[1], ctypes.c_void_p(stream.cuda_stream))
        torch.cuda.synchronize()
        named = moe.stats_dict(s, *outs)
        rstats = {n: round(float(named[n]), 6) for n in moe.STAT_NAMES}
        rstats["us_per_call"] = round(elapsed_us(ev[0], ev[1]) / K, 2)
        for e in ev:
            hip.hipEventDestroy(e)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(N_CAL):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    roof = None
    if g1_us > 0:
        flops, byts = gemm1_model(w, kept_rows, active)
        peak_c = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
        t_c = flops / (peak_c * 1e12)
        t_m = byts / (PEAK_HBM_GBS * 1e9)
        if t_c >= t_m:
            ach = flops / (g1_us * 1e-6) / 1e12
            roof = {"bound": "mfma" if w.dtype == "bf16" else "alu", "achieved": round(ach, 1),
                    "peak": peak_c, "unit": "TFLOP/s", "frac": round(ach / peak_c, 4)}
        else:
            ach = byts / (g1_us * 1e-6) / 1e9
            roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4)}
        roof["kernel"] = "grouped GEMM 1 (gate+up+SwiGLU)"
        roof["us_per_launch"] = round(g1_us, 2)
        roof["algorithmic_flops"] = flops
        roof["algorithmic_bytes"] = byts
        roof["traffic"] = (None if (args.padded or args.reroute or args.choice or args.queue
                                    or args.phi is not None)
                           else traffic_from_profile(w.name))

    layer_roof = None
    if ms > 0:
        lf, lb = layer_model(w, kept_rows, active)
        peak_c = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
        t = ms * 1e-3
        fm = lf / t / (peak_c * 1e12)
        fh = lb / t / (PEAK_HBM_GBS * 1e9)
        layer_roof = {"algorithmic_flops": lf, "algorithmic_bytes": lb,
                      "tflops": round(lf / t / 1e12, 1), "gbs": round(lb / t / 1e9, 1),
                      "frac_mfma": round(fm, 4), "frac_hbm": round(fh, 4),
                      "frac": round(max(fm, fh), 4)}

    blas = None
    if args.blas_reference and w.dtype == "bf16":
        blas = blas_reference(w, kept, max(5, min(K, 20)), dev)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w, inp, args.cpu_seconds, choice=args.choice)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded randn, no checkpoint)",
        "config": {"workload": w.name, "T": w.T, "E": w.E, "k": w.k, "d": w.d, "d_ff": w.d_ff,
                   "d_ff_shared": w.d_ff_shared, "phi": w.phi, "renormalize": w.renorm,
                   "kept_routes": kept_rows, "weight_sets": nsets,
                   "layout": "padded [E, C, d]" if args.padded else "packed",
                   "overflow": ("reroute" if args.reroute else "queue to the next micro-batch"
                                if args.queue else "drop"),
                   "queued_in": int(queue["ids"].shape[0]) if args.queue else None,
                   "queued_out": n_wait,
                   "routing": "expert choice" if args.choice else "token choice (top-k)",
                   "padded_rows": (w.E * C) if (args.padded and C > 0) else None,
                   "capacity": C if C >= 0 else None,
                   "dropped_routes": ((w.T * w.k - kept_rows) if not (args.choice or args.queue)
                                      else None),
                   "fill": round(kept_rows / (w.E * C), 4) if C > 0 else None,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "layer_roofline": layer_roof,
        "step_us": step_ev,
        "stage_step_us_percentiles": step_pct,
        "warm_ms_per_step": round(warm_ms, 5) if warm_ms else None,
        "graph_ms_per_step": round(graph_ms, 5) if graph_ms else None,
        "cpu_baseline": cpu,
        "stages_us": stages,
        "routing_stats": rstats,
    }
    if blas is not None:
        out["blas_reference"] = blas
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
