"""Host logic of bench.py that needs no GPU: the comparison of a layer's GPU
results with the oracle's (fed here with the oracle's own results, then with
one planted difference each), the kernel-name classification of profiler
output, and the refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import numpy as np

import bench
import oracle
from fp8_block_scaled_03_amd import inputs


def _layer(M=256, N=384, K=256, fraction=2):
    """A small layer (fprop, dgrad, wgrad of one linear) in the structure
    cpu_baseline builds, and the 'GPU' results that match it exactly."""
    x = inputs.normal((50,), (M, K))
    w = inputs.normal((51,), (N, K), 0.02)
    dy = inputs.student_t((52,), (M, N), 3.0, 1e-3)
    G = inputs.Gemm
    gemms = [G("l.fprop", "fprop", "X", "W", M, N, K, "bf16"),
             G("l.dgrad", "dgrad", "dY", "W", M, N, K, "bf16"),
             G("l.wgrad", "wgrad", "dY", "X", M, N, K, "f32")]
    rq = {"X": oracle.quantize_rowtile(x), "dY": oracle.quantize_rowtile(dy)}
    tq = {"X": oracle.quantize_transposed(x), "dY": oracle.quantize_transposed(dy)}
    wq = {"W": oracle.quantize_block(w)}
    out = {"l.fprop": oracle.f32_to_bf16(oracle.gemm_fprop(*rq["X"], wq["W"][0], wq["W"][2])),
           "l.dgrad": oracle.f32_to_bf16(oracle.gemm_dgrad(*rq["dY"], wq["W"][1], wq["W"][2])),
           "l.wgrad": oracle.gemm_wgrad(*tq["dY"], *tq["X"])}
    results = []
    for g in gemms:
        if g.kind == "fprop":
            rows = np.arange(0, M, fraction)
            qa = oracle.quantize_rowtile(np.ascontiguousarray(x[rows]))
            y = oracle.gemm_fprop(*qa, wq["W"][0], wq["W"][2])
            results.append((g, rows, qa, wq["W"], y))
        elif g.kind == "dgrad":
            rows = np.arange(0, M, fraction)
            qa = oracle.quantize_rowtile(np.ascontiguousarray(dy[rows]))
            y = oracle.gemm_dgrad(*qa, wq["W"][1], wq["W"][2])
            results.append((g, rows, qa, wq["W"], y))
        else:
            rows = np.arange(0, N, fraction)
            qa = oracle.quantize_transposed(np.ascontiguousarray(dy[:, rows]))
            y = oracle.gemm_wgrad(*qa, *tq["X"])
            results.append((g, rows, qa, tq["X"], y))
    gpu = {"rq": rq, "tq": tq, "wq": wq, "out": out}
    copy = lambda v: tuple(a.copy() for a in v) if isinstance(v, tuple) else v.copy()
    return {k: {n: copy(v) for n, v in d.items()} for k, d in gpu.items()}, results


def test_parity_report_passes_on_matching_results():
    gpu, results = _layer()
    rep = bench._parity_against_oracle(np, oracle, gpu, results)
    assert rep["codes_and_scales_bit_exact"] and rep["all_gemms_within_gate"], rep
    assert rep["gemms"]["l.wgrad"]["relF"] == 0.0


def test_parity_report_catches_each_planted_difference():
    gpu, results = _layer()
    gpu["wq"]["W"][0][3, 5] ^= 1                                  # one weight code
    assert not bench._parity_against_oracle(np, oracle, gpu, results)["codes_and_scales_bit_exact"]
    gpu, results = _layer()
    gpu["tq"]["X"][1][0, 0] = np.nextafter(gpu["tq"]["X"][1][0, 0], np.float32(1))   # one scale
    assert not bench._parity_against_oracle(np, oracle, gpu, results)["codes_and_scales_bit_exact"]
    gpu, results = _layer()
    gpu["out"]["l.fprop"][4, 7] += np.uint16(2)                   # two BF16 ulps off
    rep = bench._parity_against_oracle(np, oracle, gpu, results)
    assert rep["codes_and_scales_bit_exact"] and not rep["gemms"]["l.fprop"]["within_gate"]
    gpu, results = _layer()
    gpu["out"]["l.wgrad"][2, 9] *= np.float32(1.001)              # one FP32 output 1e-3 off
    rep = bench._parity_against_oracle(np, oracle, gpu, results)
    assert not rep["gemms"]["l.wgrad"]["within_gate"] and rep["gemms"]["l.dgrad"]["within_gate"]


def test_kernel_names_map_to_library_calls():
    assert bench.kernel_kind("fp8bs::gemm_bs_fp8_big_kernel<2, false, false>(...)") == ("gemm_wgrad", True)
    assert bench.kernel_kind("fp8bs::gemm_bs_fp8_kernel<0, true>(...)") == ("gemm_fprop", True)
    assert bench.kernel_kind("fp8bs::splitk_reduce_kernel(...)") == ("gemm_wgrad", False)
    assert bench.kernel_kind("fp8bs::quant_dual_kernel<false>(...)") == ("quant_transposed", True)
    assert bench.kernel_kind("fp8bs::quant_dual_kernel<true>(...)") == ("quant_dual", True)
    assert bench.kernel_kind("fp8bs::mfma_rate_kernel(float*, int, float)") == (None, False)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2 and "one GPU" in r.stdout


def test_sclk_parsing_of_both_smi_tools():
    amd = ('[{"gpu": 0, "clock": {"gfx_0": {"clk": {"value": 2100, "unit": "MHz"}, '
           '"min_clk": {"value": 500, "unit": "MHz"}}, "gfx_1": {"clk": {"value": 2095, '
           '"unit": "MHz"}}, "mem_0": {"clk": {"value": 1900, "unit": "MHz"}}}}]')
    assert bench.parse_sclk_json(amd) == [2100.0, 2095.0]
    rocm = 'WARNING: x\n{"card0": {"sclk clock speed:": "(2400Mhz)", "mclk clock speed:": "(1900Mhz)"}}'
    assert bench.parse_sclk_json(rocm) == [2400.0]
    assert bench.parse_sclk_json("no json here") is None
    assert bench.parse_sclk_json('{"card0": {"fclk clock speed:": "(1000Mhz)"}}') is None


def test_cpu_model_is_a_string():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()


def _pmc_csv(path, counter, rows):
    import csv
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, grid, kib) in enumerate(rows):
            w.writerow([i, grid, name, counter, kib])


def test_traffic_record_scales_by_the_copy_and_groups_calls(tmp_path):
    copy = ("__amd_rocclr_copyBuffer", "131072")
    wg = ("fp8bs::gemm_bs_fp8_big_kernel<2, false, false>(unsigned char const*)", "131072")
    red = ("fp8bs::splitk_reduce_kernel(float const*)", "1048576")
    # the copy moves 1 GiB = 1048576 KiB; fetch reads half of it, write all of it
    _pmc_csv(str(tmp_path / "f"), "FETCH_SIZE", [(*copy, 524288), (*wg, 1000), (*red, 300),
                                                 (*wg, 1200), (*red, 300)])
    _pmc_csv(str(tmp_path / "w"), "WRITE_SIZE", [(*copy, 1048576), (*wg, 400), (*red, 100),
                                                 (*wg, 400), (*red, 100)])
    out = tmp_path / "traffic.json"
    bench.record_traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(out))
    rec = json.loads(out.read_text())["gemm_wgrad"]
    assert rec["launches"] == 2
    # per call: fetch 2 x (1100 + 300) KiB, write 400 + 100 KiB, in bytes
    assert rec["bytes_per_launch"] == (2 * (1100 + 300) + (400 + 100)) * 1024
    assert rec["source_sha256_16"] == bench.source_digest("gemm_wgrad")


def test_smi_tools_run_without_an_env_hop(monkeypatch, tmp_path):
    script = tmp_path / "amd-smi"
    script.write_text("#!/usr/bin/env python3\nprint('{}')\n")
    script.chmod(0o755)
    monkeypatch.setenv("PATH", str(tmp_path) + os.pathsep + os.environ.get("PATH", ""))
    cmd = bench._smi_command("amd-smi", ["metric"])
    assert cmd == [sys.executable, str(script), "metric"]
    monkeypatch.setenv("LD_PRELOAD", "/opt/rocm/lib/librocprofiler-sdk-tool.so")
    assert bench.under_profiler() and bench._sclk_from_smi() is None
