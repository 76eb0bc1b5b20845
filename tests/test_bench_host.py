"""Host logic of bench.py that needs no GPU: the GEMM-1 kernel-name filter
and the counter-based traffic summary (FETCH_SIZE / WRITE_SIZE scaled by the
calibration copies)."""
import csv
import json
import os

import pytest

import bench

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
G1 = "void moe::gemm_bf16_kernel<128, 256, 2, 2, 32, 3, 3, 2, true, true, false>(moe::GemmArgs)"
G2 = "void moe::gemm_bf16_kernel<64, 256, 1, 4, 64, 2, 2, 2, false, false, true>(moe::GemmArgs)"
SHARED1 = "void moe::gemm_bf16_kernel<256, 256, 4, 2, 64, 2, 3, 1, true, false, false>(moe::GemmArgs)"
COPY = "__amd_rocclr_copyBuffer"


PP1 = "void moe::gemm_pp_kernel<true, true>(moe::GemmArgs)"
PP2 = "void moe::gemm_pp_kernel<false, false>(moe::GemmArgs)"
PPS = "void moe::gemm_pp_kernel<true, false>(moe::GemmArgs)"


def test_gemm1_filter():
    assert bench._is_gemm1(PP1)
    assert not bench._is_gemm1(PP2)
    # the packed GEMM 1 on the 256x256 tile counts unless a shared expert's
    # GEMM 1 could have the same name
    assert bench._is_gemm1(PPS) and not bench._is_gemm1(PPS, shared=True)
    assert bench._is_gemm1(G1)
    assert not bench._is_gemm1(G2)
    assert not bench._is_gemm1(SHARED1)  # the shared expert's GEMM 1 reads x directly
    assert not bench._is_gemm1(COPY)


def _write(folder, counter, rows):
    os.makedirs(os.path.join(folder, "host"), exist_ok=True)
    with open(os.path.join(folder, "host", "run_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, FIELDS)
        wr.writeheader()
        for i, (name, v) in enumerate(rows):
            wr.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter,
                         "Counter_Value": v})


def test_traffic_summary(tmp_path):
    mib = 4
    # an early copy (weight clone) that must not count as calibration, two
    # GEMM-1 launches, a GEMM 2, then the three calibration copies
    _write(tmp_path / "f", "FETCH_SIZE",
           [(COPY, 99.0), (G1, 1000.0), (G2, 5.0), (G1, 1200.0),
            (COPY, 2048.0), (COPY, 2048.0), (COPY, 2048.0)])
    _write(tmp_path / "w", "WRITE_SIZE",
           [(COPY, 7.0), (G1, 300.0), (G2, 5.0), (G1, 300.0),
            (COPY, 8192.0), (COPY, 8192.0), (COPY, 8192.0)])
    out = tmp_path / "t.json"
    bench.traffic_summary(str(tmp_path / "f"), str(tmp_path / "w"), "wl", mib, str(out))
    rec = json.load(open(out))
    assert rec["fetch_kib"] == pytest.approx(1100.0)
    assert rec["fetch_scale"] == pytest.approx(4096.0 / 2048.0)
    assert rec["write_scale"] == pytest.approx(4096.0 / 8192.0)
    assert rec["traffic_bytes_per_launch"] == pytest.approx(1024.0 * (1100.0 * 2.0 + 300.0 * 0.5))
    assert rec["gemm_hip_sha256"] == bench._gemm_sha()


def test_traffic_summary_needs_calibration(tmp_path):
    _write(tmp_path / "f", "FETCH_SIZE", [(G1, 1000.0), (COPY, 10.0)])
    _write(tmp_path / "w", "WRITE_SIZE", [(G1, 1000.0), (COPY, 10.0)])
    with pytest.raises(SystemExit):
        bench.traffic_summary(str(tmp_path / "f"), str(tmp_path / "w"), "wl", 1,
                              str(tmp_path / "t.json"))


def test_multi_gpu_refused():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_layer_model_matches_the_work_table():
    # Mixtral decode: T=16, E=8, k=2, d=4096, d_ff=14336, bf16, all 32 routes
    # kept on all 8 experts -> F = 11.3 GFLOP, B = 2.82 GB (the measurement
    # table's algorithmic work: kept routes, active experts' weights)
    from workloads import WORKLOADS
    w = WORKLOADS["mixtral_decode"]
    f, b = bench.layer_model(w, kept_rows=32, active_experts=8)
    assert f == pytest.approx(32 * 6 * 4096 * 14336 + 2 * 16 * 4096 * 8)
    assert f == pytest.approx(11.27e9, rel=1e-3)
    assert b == pytest.approx(2.818e9, rel=1e-3)
    # Granite T=16384 dropless: F = 413 GFLOP
    g = WORKLOADS["granite_16384"]
    f2, _ = bench.layer_model(g, kept_rows=16384 * 8, active_experts=32)
    assert f2 == pytest.approx(413e9, rel=2e-3)
