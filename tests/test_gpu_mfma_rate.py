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


@pytest.mark.parametrize("n", [0, 5, 4096, 4096 * 37 + 23])
def test_hbm_rate_kernel_moves_the_bytes(n):
    """The streaming probe writes the high byte (and, with two outputs, the
    low byte) of every input value, including a ragged tail."""
    print(f"hbm rate n={n}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(n)
    x = torch.randint(-32768, 32767, (n,), dtype=torch.int16, device="cuda", generator=g)
    y0, y1 = fp8.fp8bs_hbm_rate(x, two_outputs=True)
    z0, z1 = fp8.fp8bs_hbm_rate(x)
    torch.cuda.synchronize()
    u = x.to(torch.int32) & 0xFFFF
    assert torch.equal(y0.to(torch.int32), u >> 8)
    assert torch.equal(y1.to(torch.int32), u & 0xFF)
    assert z1 is None and torch.equal(z0, y0)


def test_launch_past_the_grid_limit_is_a_shape_error():
    """2^24 + 1 workgroups of 256 threads need more than 2^32 - 1 work-items
    in one grid dimension: the call is refused with FP8BS_ERR_SHAPE before
    anything is enqueued.  The output buffer is still sized for the whole
    grid (16 GiB), so that even a launch would stay inside it."""
    blocks = (1 << 24) + 1
    out = torch.full((blocks * 256,), -1.0, dtype=torch.float32, device="cuda")
    print(f"mfma_rate refused blocks={blocks}", flush=True)
    with pytest.raises(fp8.Fp8bsError) as err:
        fp8.fp8bs_mfma_rate(blocks, 0, out=out)
    torch.cuda.synchronize()
    assert err.value.status == 2
    assert bool((out[:1024] == -1.0).all()) and bool((out[-1024:] == -1.0).all())
    del out
    torch.cuda.empty_cache()
