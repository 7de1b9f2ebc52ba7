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


def test_roofline_fraction_is_achieved_over_peak():
    x = make_case(1, 2, 48, 64, seed=3, in_bf16=True)
    _, nbytes, _ = bench.algorithmic_work(x)
    name, roof = bench.roofline(x, kernel_ms=1e-6, traffic=None)   # ~1e5 GB/s: rounding is small
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s"
    assert roof["achieved"] == pytest.approx(nbytes / 1e-9 / 1e9, rel=1e-3)
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], rel=1e-3)
    _, rt = bench.roofline(x, kernel_ms=2.0, traffic=123, train=True)
    assert rt["traffic"] == 123 and rt["bound"] == "hbm"


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
    name, roof = bench.roofline(a, kernel_ms=1e-3, traffic=None, project=True)
    assert name == "proj_mfma" and roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s"
    assert roof["peak"] == bench.BF16_MATRIX_PEAK_TFLOPS
    assert roof["achieved"] == pytest.approx(fl_a / 1e-6 / 1e12, rel=1e-3)
