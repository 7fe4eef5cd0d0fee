"""GPU parity at the full Qwen3-1.7B-like configurations, launched as the
benchmark launches them (activations and gradients through the dual-axis
quantizer, weights through the block quantizer, wgrad with its split-K
workspace).

Every GEMM whose output is BF16 (fprop, dgrad) is run twice on the same
quantized operands: with BF16 output, checked within one BF16 ulp of the
rounded oracle value, and with FP32 output, checked at relF <= 1e-5 and the
per-element bound; the BF16 result must also be the round-to-nearest-even of
the FP32 one, bit for bit.

- QKV, MLP pair and down-projection backward (8192 tokens): sampled rows, and
  in a second test every output element.
- The 28-layer linear set (16,384 tokens): the eight shared activations and
  gradients quantized along both axes, compared in full; then, for every one
  of the 28 layers, its four weights' codes, scales and transposed codes in
  full and 16 sampled output rows (plus the first and last) of each of its 12
  GEMMs.

Row tiles and weight blocks are local, so the oracle quantizes only what the
sampled rows need."""
import numpy as np
import pytest
import torch

import oracle
import fp8_block_scaled_03_amd as fp8
from fp8_block_scaled_03_amd import inputs
from helpers import check_bf16, check_bf16_is_rne_of_f32, check_f32, to_dev_bf16, to_np

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def sample_rows(n, k=48, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=min(k, n), replace=False)]))


def _rows_to_host(t: torch.Tensor, rows: np.ndarray) -> np.ndarray:
    """Only the sampled rows leave the device."""
    return to_np(t[torch.as_tensor(rows, device=t.device)])


def check_output(kind, run, rows, ref, ad, bd, out):
    """run(out_dtype) -> device output.  BF16 outputs: the BF16 gate, the FP32
    gate on the same kernel with FP32 output, and BF16 == RNE(FP32)."""
    if out == "f32":
        check_f32(_rows_to_host(run("f32"), rows), ref, ad, bd, kind)
        return
    got16 = _rows_to_host(run("bf16"), rows)
    got32 = _rows_to_host(run("f32"), rows)
    check_f32(got32, ref, ad, bd, kind + " (FP32 output)")
    check_bf16(got16, ref, ad, bd, kind + " (BF16 output)")
    check_bf16_is_rne_of_f32(got16, got32, kind)


def gemm_case(kind, abits, bbits, out, rows, dev=None, ora=None):
    """Run one GEMM of a configuration on the GPU (full size) and the oracle
    on the sampled rows.  abits is the row-side operand [M, .] for fprop /
    dgrad and dY [M, N] for wgrad (rows then index dW's rows = dY channels).
    dev / ora: optional caches of device-quantized and oracle-quantized
    operands, keyed by the operands' identities."""
    dev = {} if dev is None else dev
    ora = {} if ora is None else ora

    def dual(bits):
        k = ("dual", id(bits))
        if k not in dev:
            dev[k] = fp8.fp8_quantize_dual(to_dev_bf16(bits))
        return dev[k]

    def block(bits):
        k = ("block", id(bits))
        if k not in dev:
            dev[k] = fp8.fp8_quantize_block(to_dev_bf16(bits))
        return dev[k]

    def oblock(bits):
        k = ("block", id(bits))
        if k not in ora:
            ora[k] = oracle.quantize_block(bits)
        return ora[k]

    def otrans(bits):
        k = ("trans", id(bits))
        if k not in ora:
            ora[k] = oracle.quantize_transposed(bits)
        return ora[k]

    if kind == "fprop":
        aq, as_, _, _ = dual(abits)
        bq, _, bs = block(bbits)
        run = lambda o: fp8.fp8_gemm_fprop(aq, as_, bq, bs, out_dtype=o)
        oq, os_ = oracle.quantize_rowtile(np.ascontiguousarray(abits[rows]))
        wq, _, ws = oblock(bbits)
        ref = oracle.gemm_fprop(oq, os_, wq, ws)
        ad, bd = oracle.dequantize_rows(oq, os_), oracle.dequantize_block(wq, ws)
    elif kind == "dgrad":
        aq, as_, _, _ = dual(abits)
        _, bqt, bs = block(bbits)
        run = lambda o: fp8.fp8_gemm_dgrad(aq, as_, bqt, bs, out_dtype=o)
        oq, os_ = oracle.quantize_rowtile(np.ascontiguousarray(abits[rows]))
        wq, wqt, ws = oblock(bbits)
        ref = oracle.gemm_dgrad(oq, os_, wqt, ws)
        ad, bd = oracle.dequantize_rows(oq, os_), oracle.dequantize_block(wq, ws).T
    else:
        _, _, atq, ats = dual(abits)
        _, _, btq, bts = dual(bbits)
        run = lambda o: fp8.fp8_gemm_wgrad(atq, ats, btq, bts, workspace="auto")
        oq, os_ = oracle.quantize_transposed(np.ascontiguousarray(abits[:, rows]))
        xq, xs = otrans(bbits)
        ref = oracle.gemm_wgrad(oq, os_, xq, xs)
        ad, bd = oracle.dequantize_rows(oq, os_), oracle.dequantize_rows(xq, xs)
    check_output(kind, run, rows, ref, ad, bd, out)


@pytest.mark.parametrize("cfg", ["tiny", "qkv", "mlp", "down_bwd"])
def test_config_gemms_sampled(cfg):
    c = inputs.CONFIGS[cfg]
    dev, ora = {}, {}
    bits = {n: inputs.tensor(cfg, n) for n in c.tensors}
    for g in c.gemms:
        _say(f"config {cfg} {g.name} M={g.M} N={g.N} K={g.K} out={g.out}")
        n_rows = g.M if g.kind != "wgrad" else g.N
        rows = np.arange(n_rows) if cfg == "tiny" else sample_rows(n_rows, seed=c.key)
        gemm_case(g.kind, bits[g.a], bits[g.b], g.out, rows, dev, ora)


@pytest.mark.parametrize("cfg", ["qkv", "mlp", "down_bwd"])
def test_config_gemms_every_element(cfg):
    """Every output element, not a sample, of the QKV fprop (8192 x 4096 x
    2048), the MLP pair (gate/up 8192 x 12288 x 2048, down 8192 x 2048 x 6144)
    and the down-projection backward (dgrad and wgrad, 8192 tokens, 2048 x
    6144) against the oracle, BF16 outputs also with FP32 output."""
    c = inputs.CONFIGS[cfg]
    dev, ora = {}, {}
    bits = {n: inputs.tensor(cfg, n) for n in c.tensors}
    for g in c.gemms:
        _say(f"config {cfg} {g.name} M={g.M} N={g.N} K={g.K} out={g.out}: every element")
        n_rows = g.M if g.kind != "wgrad" else g.N
        gemm_case(g.kind, bits[g.a], bits[g.b], g.out, np.arange(n_rows), dev, ora)


# ----------------------------------------------------- the 28-layer linear set
_C5 = {}


def _c5_shared():
    """Host bits of the shared activations and gradients, their device dual
    quantization, and the oracle's token-axis quantization of the wgrad B
    operands (X_qkv, X_o, X_mlp, H), computed once per process."""
    if not _C5:
        c = inputs.CONFIGS["linear_set"]
        shared = [n for n in c.tensors if n not in c.per_layer]
        _say("linear_set: drawing the shared activations and gradients")
        _C5["bits"] = {n: inputs.tensor("linear_set", n) for n in shared}
        _C5["dev"] = {}
        _C5["ora"] = {}
        for n in shared:
            b = _C5["bits"][n]
            _C5["dev"][("dual", id(b))] = fp8.fp8_quantize_dual(to_dev_bf16(b))
        for g in c.gemms:
            if g.kind == "wgrad":
                b = _C5["bits"][g.b]
                if ("trans", id(b)) not in _C5["ora"]:
                    _C5["ora"][("trans", id(b))] = oracle.quantize_transposed(b)
        torch.cuda.synchronize()
    return _C5


def test_linear_set_activations_quantized_in_full():
    """The eight shared tensors of the 16,384-token linear set (X_qkv, X_o,
    X_mlp, H, dY_qkv, dY_o, dY_gu, dY_d), dual-quantized as the benchmark
    step does, against the oracle's row-tile and token-axis quantizers on
    every element."""
    s = _c5_shared()
    for n, b in s["bits"].items():
        _say(f"linear_set {n} {b.shape}: both axes, every element")
        q, sc, qt, st = (to_np(t) for t in s["dev"][("dual", id(b))])
        oq, osc = oracle.quantize_rowtile(b)
        assert np.array_equal(q, oq), n
        assert np.array_equal(sc.view(np.uint32), osc.view(np.uint32)), n
        del oq, osc
        if ("trans", id(b)) in s["ora"]:
            oqt, ost = s["ora"][("trans", id(b))]
        else:
            oqt, ost = oracle.quantize_transposed(b)
        assert np.array_equal(qt, oqt), n
        assert np.array_equal(st.view(np.uint32), ost.view(np.uint32)), n


@pytest.mark.parametrize("layer", list(range(inputs.LAYERS)))
def test_linear_set_layer(layer):
    """Layer `layer` of the 28-layer, 16,384-token linear set: its four
    weights' block quantization (codes, scales, transposed codes) in full,
    and 16 sampled output rows of all 12 GEMMs, on the seeded weights of
    that layer."""
    c = inputs.CONFIGS["linear_set"]
    s = _c5_shared()
    wbits = {n: inputs.tensor("linear_set", n, layer=layer) for n in c.per_layer}
    dev = dict(s["dev"])
    ora = dict(s["ora"])
    for n, b in wbits.items():
        _say(f"linear_set layer {layer} {n} {b.shape}: block quantization, every element")
        q, qt, sc = fp8.fp8_quantize_block(to_dev_bf16(b))
        dev[("block", id(b))] = (q, qt, sc)
        oq, oqt, osc = oracle.quantize_block(b)
        ora[("block", id(b))] = (oq, oqt, osc)
        assert np.array_equal(to_np(q), oq), n
        assert np.array_equal(to_np(qt), oqt), n
        assert np.array_equal(to_np(sc).view(np.uint32), osc.view(np.uint32)), n
    bits = {**s["bits"], **wbits}
    for g in c.gemms:
        _say(f"linear_set layer {layer} {g.name} M={g.M} N={g.N} K={g.K} out={g.out}")
        n_rows = g.M if g.kind != "wgrad" else g.N
        rows = sample_rows(n_rows, k=16, seed=1000 + layer)
        gemm_case(g.kind, bits[g.a], bits[g.b], g.out, rows, dev, ora)
