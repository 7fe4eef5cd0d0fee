"""fp8_quantize_block_many through the C ABI: every weight's codes, transposed
codes and scales equal, byte for byte, what fp8_quantize_block gives for it
alone (itself bit-exact with the oracle), over more jobs than one launch
takes, with empty jobs and jobs without transposed codes mixed in; one weight
is also checked against the oracle directly."""
import numpy as np
import pytest
import torch

import oracle
import fp8_block_scaled_03_amd as fp8
from fp8_block_scaled_03_amd import inputs
from helpers import to_dev_bf16, to_np

pytestmark = pytest.mark.gpu


def test_block_many_equals_single_calls():
    shapes = [(4096, 2048), (2048, 2048), (12288, 2048), (2048, 6144), (128, 128), (384, 640),
              (256, 128), (128, 1024)] * 2 + [(512, 384), (640, 256), (128, 256), (256, 256)]
    ws = [to_dev_bf16(inputs.normal((150, i, N, K), (N, K), 0.02)) for i, (N, K) in enumerate(shapes)]
    flags = [i % 3 != 1 for i in range(len(ws))]
    print(f"{len(ws)} weights in one call", flush=True)
    outs = fp8.fp8_quantize_block_many(ws, with_transpose=flags)
    for i, (w, t) in enumerate(zip(ws, flags)):
        q, qt, s = fp8.fp8_quantize_block(w, with_transpose=t)
        mq, mqt, ms = outs[i]
        assert torch.equal(q, mq) and torch.equal(s.view(torch.int32), ms.view(torch.int32)), i
        assert (qt is None and mqt is None) or torch.equal(qt, mqt), i
    torch.cuda.synchronize()
    wb = inputs.normal((150, 2, 12288, 2048), (12288, 2048), 0.02)
    oq, oqt, os_ = oracle.quantize_block(wb)
    q, qt, s = outs[2]
    assert np.array_equal(to_np(q), oq) and np.array_equal(to_np(qt), oqt)
    assert np.array_equal(to_np(s).view(np.uint32), os_.view(np.uint32))


def test_block_many_skips_empty_jobs():
    ws = [torch.empty((0, 256), dtype=torch.bfloat16, device="cuda"),
          to_dev_bf16(inputs.normal((151, 256, 384), (256, 384), 0.02)),
          torch.empty((128, 0), dtype=torch.bfloat16, device="cuda")]
    outs = fp8.fp8_quantize_block_many(ws)
    q, qt, s = fp8.fp8_quantize_block(ws[1])
    torch.cuda.synchronize()
    assert torch.equal(outs[1][0], q) and torch.equal(outs[1][1], qt)
    assert torch.equal(outs[1][2].view(torch.int32), s.view(torch.int32))
    assert fp8.fp8_quantize_block_many([]) == []
