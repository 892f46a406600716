"""The measurement probes (libfa355_probe.so) run and return plausible
numbers on the GPU: a matrix-core rate below the part's published dense bf16
peak, an engine clock between 0.5 and 3 GHz, and a streaming read rate below
the published HBM bandwidth.  These numbers put the roofline fractions in
context; they are not part of the attention path."""

import pytest

pytestmark = pytest.mark.gpu


def test_mfma_probe_and_clock():
    from exact_io_aware_15_amd import probe
    print("probe: mfma loop", flush=True)
    tflops, ghz, sec = probe.mfma_bf16(iters=2000, waves_per_simd=2)
    assert 100.0 < tflops < 2600.0, tflops
    assert 0.5 < ghz < 3.0, ghz
    assert sec > 0.0


def test_read_probe():
    from exact_io_aware_15_amd import probe
    print("probe: streaming read", flush=True)
    gbs = probe.read_bw(64 << 20, 2)
    assert 100.0 < gbs < 9000.0, gbs
