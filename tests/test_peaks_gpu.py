"""The throughput probes behind the roofline's measured compute ceilings, on
the GPU: they run and land in a plausible range of the published peaks
(fp32 vector 157.3 TFLOP/s counts packed instructions, which the kernels are
built without, so about half of it is reachable; dense bf16 MFMA 2.5 PFLOP/s)."""
import sys

import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def test_measured_peaks_plausible():
    import bench
    print("case peak probes", file=sys.stderr, flush=True)
    peaks = bench.measure_peaks(torch.cuda.current_stream())
    assert peaks is not None, "probe library not built"
    print(f"    measured {peaks}", file=sys.stderr, flush=True)
    assert 20.0 < peaks["fp32_vector"] < 170.0
    assert 300.0 < peaks["bf16_mfma"] < 2700.0
