"""The two measurement probes on the GPU: the streaming-read rate and the
matrix-core rate that the roofline fractions are read against.  They only
have to land between a clearly broken value and the published peak (8 TB/s
HBM; 2.5 PFLOP/s dense bf16 and fp16 on MI355X)."""

from __future__ import annotations

import sys

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import shared_prefix_kv_amd as fca  # noqa: E402

HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fca.lib()


def test_read_probe_within_published_peak():
    say("read probe: two 1 GiB buffers")
    bufs = [torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(i + 1) for i in range(2)]
    g = fca.measure_read_bandwidth(bufs, repeats=2)
    say(f"read probe: {g:.0f} GB/s")
    assert 0.25 * HBM_PEAK_GBPS < g < 1.05 * HBM_PEAK_GBPS


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_mfma_probe_within_published_peak(dtype):
    say(f"MFMA probe {dtype}")
    t = fca.measure_mfma_rate(dtype, iters=2000)
    say(f"MFMA probe {dtype}: {t:.0f} TFLOP/s")
    assert 0.25 * MFMA_PEAK_TFLOPS < t < 1.05 * MFMA_PEAK_TFLOPS
