"""Host logic of bench.py: the algorithmic work model, the roofline record, the
traffic record's source check, and the one-GPU guard.  No GPU is used."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from test_rnn_layer_ttt_amd.build import source_digest
from test_rnn_layer_ttt_amd.inputs import make_case, make_update_mask

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_forward_bytes_scale_with_tokens_and_input_width():
    a = make_case(2, 3, 32, 64, seed=0)
    b = make_case(2, 3, 64, 64, seed=0)
    c = make_case(2, 3, 32, 64, seed=0, in_bf16=True)
    n_a, by_a, fl_a = bench.algorithmic_work(a)
    n_b, by_b, fl_b = bench.algorithmic_work(b)
    n_c, by_c, _ = bench.algorithmic_work(c)
    assert (n_a, n_b) == (2 * 3 * 32, 2 * 3 * 64)
    # per token-head: q, k, v, gate (d each) and eta in, out (d fp32) written
    assert by_b - by_a == (n_b - n_a) * ((4 * 64 + 1) * 4 + 4 * 64)
    assert by_a - by_c == n_a * (4 * 64 + 1) * 2
    assert fl_b == 2 * fl_a


def test_mask_counts_skipped_chunks_as_cheaper():
    x = make_case(2, 2, 64, 64, seed=1, dual=True, chunk=16, in_bf16=True)
    none = make_update_mask(2, 2, 64, 16, 0.0, seed=2)     # every chunk skipped
    every = make_update_mask(2, 2, 64, 16, 1.0, seed=2)    # every chunk updated
    _, by0, fl0 = bench.algorithmic_work(x)
    _, by_all, fl_all = bench.algorithmic_work(x, every)
    _, by_none, fl_none = bench.algorithmic_work(x, none)
    assert by_all == by0 + every.size and fl_all == fl0
    assert by_none < by_all and fl_none < fl_all


def test_roofline_fraction_is_achieved_over_the_binding_peak():
    # fp32 inputs: 1284 B and 6 d^2 flops per token-head; the HBM time is the larger
    x = make_case(1, 2, 48, 64, seed=3)
    _, nbytes, flops = bench.algorithmic_work(x)
    assert nbytes / 8e12 > flops / 157.3e12
    name, roof = bench.roofline(x, kernel_ms=1e-6, traffic=None, kernel="scan_mfma")
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s"
    assert roof["achieved"] == pytest.approx(nbytes / 1e-9 / 1e9, rel=1e-3)
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], rel=1e-3)
    assert roof["frac_hbm"] == roof["frac"]
    assert roof["frac_compute"] == pytest.approx(flops / 1e-9 / 157.3e12, rel=1e-3)
    # bf16 inputs halve the input bytes: the fp32 arithmetic is then the binding roof
    xb = make_case(1, 2, 2048, 64, seed=3, in_bf16=True)   # long enough that W0 is minor
    _, nb, fb = bench.algorithmic_work(xb)
    _, rb = bench.roofline(xb, kernel_ms=1e-3, traffic=None, kernel="scan_mfma",
                           hbm_measured_gbs=5000.0)
    assert rb["bound"] == "alu" and rb["unit"] == "TFLOP/s" and rb["peak"] == 157.3
    assert rb["frac"] == rb["frac_compute"]
    assert rb["frac_hbm"] == pytest.approx(nb / 1e-6 / 8e12, rel=1e-3)
    assert rb["frac_hbm_measured"] == pytest.approx(nb / 1e-6 / 5e12, rel=1e-3)
    assert rb["t_compute_us"] > rb["t_hbm_us"]
    # the dual form's contractions are priced on the bf16 matrix cores: HBM binds
    xd = make_case(1, 2, 2048, 64, seed=3, in_bf16=True, dual=True, chunk=16)
    _, rd = bench.roofline(xd, kernel_ms=1e-3, traffic=None, kernel="scan_mfma")
    assert rd["bound"] == "hbm" and rd["compute_peak_tflops"] == 2500.0
    _, rt = bench.roofline(x, kernel_ms=2.0, traffic=123, train=True)
    assert rt["traffic"] == 123 and rt["bound"] == "hbm"


def test_headline_workload_ceilings():
    # the 256-scan per-token workload: 815,800,320 algorithmic bytes (102.0 us at
    # 8 TB/s) and 25.77 GFLOP (163.8 us at 157.3 TFLOP/s), so fp32 arithmetic binds
    from test_rnn_layer_ttt_amd.inputs import WORKLOADS
    cfg = WORKLOADS["h1024_T4096_bf16"]
    x = make_case(cfg["B"], cfg["H"], 16, cfg["d"], seed=0, in_bf16=True)
    B, H, d, T = cfg["B"], cfg["H"], cfg["d"], cfg["T"]
    nbytes = B * H * T * ((4 * d + 1) * 2 + 4 * d) + B * H * 8 * d * d + H * 8 * d
    assert nbytes == 815_800_320
    assert 6 * d * d * B * H * T / 157.3e12 * 1e6 == pytest.approx(163.8, abs=0.1)
    del x


def test_traffic_is_reported_only_for_the_measured_source(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"scan_mfma|wl": {"source_digest": source_digest("scan_mfma"), "traffic_bytes": 7},
           "bwd_mfma|wl/backward": {"source_digest": "0" * 16, "traffic_bytes": 9}}
    (prof / "traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_traffic("scan_mfma", "wl") == 7
    assert bench.load_traffic("bwd_mfma", "wl/backward") is None      # changed since
    assert bench.load_traffic("scan_mfma", "other") is None


def test_digest_follows_one_kernel_source():
    assert source_digest("scan_mfma") != source_digest("bwd_mfma")
    assert len(source_digest()) == 16


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_projection_work_and_its_matrix_roofline():
    a = make_case(2, 4, 32, 64, seed=4, in_bf16=True)
    b = make_case(2, 4, 64, 64, seed=4, in_bf16=True)
    c = make_case(2, 4, 32, 64, seed=4)
    _, by_a, fl_a = bench.projection_work(a)
    _, by_b, fl_b = bench.projection_work(b)
    _, by_c, _ = bench.projection_work(c)
    hidden, rows = 4 * 64, 4 * (4 * 64 + 1)
    assert fl_b == 2 * fl_a == 2 * (2 * 2 * 32 * hidden * rows)
    # 32 more tokens of 2 batches: their x rows in and their results out (bf16)
    assert by_b - by_a == 2 * 32 * (hidden * 2 + rows * 2)
    assert by_c - by_a == 2 * 32 * rows * 2          # fp32 results are twice as wide
    # hidden 256 is below the bf16 ridge: the weights' and results' bytes bind
    name, roof = bench.roofline(a, kernel_ms=1e-3, traffic=None, project=True)
    assert name == "proj_mfma" and roof["bound"] == "hbm"
    assert roof["frac_compute"] == pytest.approx(fl_a / 1e-6 / 1e12 / 2500.0, abs=1e-4)
    # hidden 1024 over 4096 tokens: the matrix cores bind
    big = make_case(2, 16, 2048, 64, seed=4, in_bf16=True)
    _, _, fl_big = bench.projection_work(big)
    name, roof = bench.roofline(big, kernel_ms=1e-3, traffic=None, project=True)
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s"
    assert roof["peak"] == bench.BF16_MATRIX_PEAK_TFLOPS
    assert roof["achieved"] == pytest.approx(fl_big / 1e-6 / 1e12, rel=1e-3)


def test_peak_probe_library_exports_and_flop_counts():
    # the throughput probes bench.py measures its compute ceilings with: a
    # separate library beside the scan's, with these four symbols; the flop
    # counts follow the probes' loops (8 fp32 FMA chains per thread; 4
    # 16x16x32 products per wave per iteration)
    import ctypes

    from test_rnn_layer_ttt_amd.build import PEAKS_LIB
    if not os.path.exists(PEAKS_LIB):
        pytest.skip("probe library not built")
    out = subprocess.run(["nm", "-D", "--defined-only", PEAKS_LIB], capture_output=True,
                         text=True, check=True).stdout
    names = {l.split()[-1] for l in out.splitlines() if l.strip()}
    assert {"ttt_peak_fp32", "ttt_peak_bf16_mfma", "ttt_peak_bf16_mfma32", "ttt_peak_fp32_flops",
            "ttt_peak_bf16_mfma_flops", "ttt_peak_bf16_mfma32_flops"} <= names
    lib = ctypes.CDLL(PEAKS_LIB)
    for fn in (lib.ttt_peak_fp32_flops, lib.ttt_peak_bf16_mfma_flops,
               lib.ttt_peak_bf16_mfma32_flops):
        fn.restype = ctypes.c_double
        fn.argtypes = [ctypes.c_int32, ctypes.c_int32]
    assert lib.ttt_peak_fp32_flops(1024, 100) == 2 * 8 * 256 * 1024 * 100
    assert lib.ttt_peak_bf16_mfma_flops(1024, 100) == 4 * 16384 * 4 * 1024 * 100
    assert lib.ttt_peak_bf16_mfma32_flops(1024, 100) == 2 * 32768 * 4 * 1024 * 100


def test_roofline_reports_measured_compute_ceiling():
    x = make_case(2, 3, 64, 64, seed=0, in_bf16=True)
    peaks = {"fp32_vector": 80.0, "bf16_mfma": 2000.0}
    _, r = bench.roofline(x, kernel_ms=0.01, traffic=None, peaks=peaks, kernel="scan_mfma")
    assert r["compute_measured_tflops"] == 80.0
    assert r["frac_compute_measured"] == pytest.approx(r["frac_compute"] * 157.3 / 80.0, rel=1e-3)
    xd = make_case(2, 3, 64, 64, seed=0, in_bf16=True, dual=True, chunk=16)
    _, rd = bench.roofline(xd, kernel_ms=0.01, traffic=None, peaks=peaks, kernel="scan_mfma")
    assert rd["compute_measured_tflops"] == 2000.0
