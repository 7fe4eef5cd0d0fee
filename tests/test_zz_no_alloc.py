"""fp8_gemm_wgrad_noalloc (split-K slices in the library's static device
scratch, no allocation) against fp8_gemm_wgrad with a caller workspace, on
two calls in a row with the second smaller than the first (the scratch then
still holds the first call's slices), and the rejection of a shape whose
split would need more than the static maximum."""
import pytest
import torch

import fp8_block_scaled_03_amd as fp8
from fp8_block_scaled_03_amd import _binding as B

pytestmark = pytest.mark.gpu


def _operands(M, N, K, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    dytq = torch.randint(0, 0x7F, (N, M), dtype=torch.uint8, device="cuda", generator=g)
    xtq = torch.randint(0, 0x7F, (K, M), dtype=torch.uint8, device="cuda", generator=g)
    dytq[dytq == 0x7F] = 0x7E                       # no NaN codes
    xtq[xtq == 0x7F] = 0x7E
    sign = torch.randint(0, 2, (N, M), dtype=torch.uint8, device="cuda", generator=g) << 7
    dytq |= sign
    dyts = torch.rand(N, M // 128, device="cuda", generator=g) * 1e-3 + 1e-4
    xts = torch.rand(K, M // 128, device="cuda", generator=g) * 1e-2 + 1e-3
    return dytq, dyts, xtq, xts


def _bits(t):
    return t.view(torch.int32)


def test_noalloc_matches_workspace_wgrad_twice():
    # 2048 x 2048 over 16384 tokens splits into four pieces (three 16 MiB
    # slices); 1024 x 1024 over 4096 tokens into eight (seven 4 MiB slices)
    for (M, N, K), seed in (((16384, 2048, 2048), 1), ((4096, 1024, 1024), 2)):
        print(f"noalloc wgrad M={M} N={N} K={K}", flush=True)
        assert 0 < fp8.fp8_gemm_wgrad_workspace_bytes(M, N, K) <= B.NOALLOC_SCRATCH_BYTES
        ops = _operands(M, N, K, seed)
        want = fp8.fp8_gemm_wgrad(*ops, workspace="auto")
        got = torch.full((N, K), float("nan"), device="cuda")
        torch.cuda.synchronize()
        fp8.fp8_gemm_wgrad_noalloc(*ops, dw=got)
        torch.cuda.synchronize()
        assert torch.equal(_bits(got), _bits(want)), f"M={M} N={N} K={K}"
        assert torch.isfinite(got).all()


def test_noalloc_rejects_a_split_beyond_the_scratch():
    M, N, K = 4096, 12288, 3072        # two pieces: one 144 MiB slice
    print(f"noalloc wgrad M={M} N={N} K={K}: larger than the scratch", flush=True)
    need = fp8.fp8_gemm_wgrad_workspace_bytes(M, N, K)
    assert need > B.NOALLOC_SCRATCH_BYTES
    ops = _operands(M, N, K, 3)
    dw = torch.full((N, K), 7.0, device="cuda")
    with pytest.raises(fp8.Fp8bsError) as e:
        fp8.fp8_gemm_wgrad_noalloc(*ops, dw=dw)
    assert e.value.status == 5                     # FP8BS_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((dw == 7.0).all())                 # nothing was launched


def test_noalloc_unsplit_shape_needs_no_scratch():
    M, N, K = 512, 128, 256            # a single piece: no slices at all
    print(f"noalloc wgrad M={M} N={N} K={K}: no split", flush=True)
    ops = _operands(M, N, K, 4)
    want = fp8.fp8_gemm_wgrad(*ops)
    got = torch.empty((N, K), device="cuda")
    fp8.fp8_gemm_wgrad_noalloc(*ops, dw=got)
    torch.cuda.synchronize()
    assert torch.equal(_bits(got), _bits(want))
