"""The MFMA-rate diagnostic (fp8bs_mfma_rate): exact results, and a rate
between the FP16 MFMA's plausible at-clock floor and its 2.5 PFLOP/s spec
peak, so the ceiling the benchmark prices its GEMMs against is real."""
import pytest
import torch

import fp8_block_scaled_03_amd as fp8

pytestmark = pytest.mark.gpu


def test_mfma_rate_values_are_exact():
    for blocks, iters, v in ((1, 0, 0.5), (3, 1, 0.125), (256, 7, 0.25), (1024, 30, 0.0625)):
        out = fp8.fp8bs_mfma_rate(blocks, iters, v)
        torch.cuda.synchronize()
        expect = 16384 * v * v * iters
        print(f"mfma_rate blocks={blocks} iters={iters} v={v}", flush=True)
        assert out.shape == (blocks * 256,)
        assert bool((out == expect).all()), (out.min().item(), out.max().item(), expect)


def test_mfma_rate_is_plausible():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 8 * cus, 200
    out = fp8.fp8bs_mfma_rate(blocks, iters)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    fp8.fp8bs_mfma_rate(blocks, iters, out=out)
    e1.record()
    torch.cuda.synchronize()
    tflops = blocks * 4 * iters * 128 * 16384 / (e0.elapsed_time(e1) / 1e3) / 1e12
    print(f"mfma_rate {tflops:.0f} TFLOP/s on {cus} CUs", flush=True)
    assert 1000 < tflops < 2600
