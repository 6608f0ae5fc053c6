"""The FP8 MFMA throughput probe (mqa_mfma_peak) that bench.py reads the scan's
MFMA fraction against: it runs through the C ABI, writes finite sums, and
reports a rate between a tenth of the MI355X dense FP8 peak (5.0 PFLOP/s) and
that peak plus 10%."""
import pytest

import fp8_mqa_logits_amd as mqa


@pytest.mark.gpu
def test_mfma_peak_probe_rate():
    import torch

    torch.cuda.set_device(0)
    rate = mqa.mfma_peak_tflops(workgroups=512, iters=1024, repeats=2)
    print(f"measured FP8 MFMA rate {rate:.0f} TFLOP/s", flush=True)
    assert 500.0 < rate < 5500.0
