#!/usr/bin/env python3
"""Benchmark of the FP8 block-scaled linear-layer path on one MI355X.

One step is one pass of the whole path over the linear layers of a 28-layer
Qwen3-1.7B-like decoder micro-batch (4 x 4096 tokens, hidden 2048, FFN 6144,
16 query / 8 key-value heads of width 128): per layer and per linear (QKV, O,
gate/up, down) the row-tile quantization of the input and of the output
gradient, the block quantization of the weight (with its transposed codes),
the token-axis quantization of both wgrad operands, and the fprop, dgrad and
wgrad GEMMs.  Inputs are seeded synthetic tensors already resident in HBM;
weights are distinct per layer, activations and gradients are shared.

Prints one JSON line: GEMM TFLOP/s of the whole step (quantizers included in
the time), the dominant kernel's roofline, and the CPU oracle's throughput on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 block-scaled GEMM TFLOP/s at Qwen3-1.7B-like shapes; % of FP8 MFMA peak"
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense FP8 MFMA
PEAK_F16_TFLOPS = 2500.0       # MI355X dense FP16 / BF16 MFMA
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "gemm": ["gemm.hip", "gemm_common.h", "device_common.h", "internal.h"],
    "quant": ["quantize.hip", "device_common.h", "internal.h"],
}


def _code_only(text: str) -> str:
    """C++ source without comments and blank lines (a comment edit does not
    change a kernel).  String literals in these sources hold no comment
    markers."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(l.rstrip() for l in text.splitlines() if l.strip())


def source_digest(kind: str) -> str:
    """Digest of the code (comments stripped) of the sources a kernel kind is
    built from: counter records taken on other code are stale."""
    import hashlib
    h = hashlib.sha256()
    for fn in KERNEL_SOURCES["gemm" if kind.startswith("gemm") else "quant"]:
        with open(os.path.join(ROOT, "fp8_block_scaled_03_amd", "csrc", fn), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def kernel_kind(name: str):
    """(kind, counts_as_call) of a device kernel name: the library call it
    belongs to, and whether each of its launches is one call of that kind
    (the split-K reduction is part of a wgrad call, not a call of its own)."""
    import re
    if "splitk_reduce_kernel" in name:
        return "gemm_wgrad", False
    m = re.search(r"gemm_bs_fp8(?:_big)?_kernel<(\d)", name)
    if m:
        return ("gemm_fprop", "gemm_dgrad", "gemm_wgrad")[int(m.group(1))], True
    if "quant_dual_kernel<false>" in name:          # the token-axis-only instance
        return "quant_transposed", True
    for k in ("quant_rowtile", "quant_block", "quant_transposed", "quant_dual"):
        if k + "_kernel" in name:
            return k, True
    return None, False


def recorded_traffic(kind: str):
    """HBM bytes per launch of `kind` from the committed counter runs, or None
    when none were taken or the kernel source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kind)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256_16") != source_digest(kind):
        return None
    return rec


def summarize_rocprof(d: str) -> None:
    """Text summary of a rocprofv3 run (-f csv): kernel stats, or per-kernel
    counter averages per dispatch when counters were collected."""
    import csv
    import glob
    stats = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    for path in stats:
        print(f"# {os.path.relpath(path, d)}")
        print(f"{'kernel':64s} {'calls':>6s} {'avg_us':>10s} {'total_ms':>10s} {'pct':>6s}")
        for r in csv.DictReader(open(path)):
            name = r["Name"].split("(")[0].replace("void ", "")[:64]
            print(f"{name:64s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                  f"{float(r['TotalDurationNs']) / 1e6:10.3f} {float(r['Percentage']):6.2f}")
        per_kind = {}
        for r in csv.DictReader(open(path)):
            kind, is_call = kernel_kind(r["Name"])
            if kind:
                k = per_kind.setdefault(kind, [0.0, 0])
                k[0] += float(r["TotalDurationNs"])
                k[1] += int(r["Calls"]) if is_call else 0
        print("# per library call (split-K reductions counted with their wgrad call)")
        print(f"{'kind':20s} {'calls':>6s} {'avg_us_per_call':>16s} {'total_ms':>10s}")
        for kind, (ns, calls) in sorted(per_kind.items(), key=lambda kv: -kv[1][0]):
            print(f"{kind:20s} {calls:6d} {ns / max(calls, 1) / 1e3:16.2f} {ns / 1e6:10.3f}")
    pmc = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    for path in pmc:
        agg = {}
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"].split("(")[0].replace("void ", "")
            key = (name, r["Grid_Size"])
            a = agg.setdefault(key, {"dispatches": set()})
            a["dispatches"].add(r["Dispatch_Id"])
            a[r["Counter_Name"]] = a.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        print(f"# {os.path.relpath(path, d)} (per-dispatch averages)")
        ratios = []
        for (name, grid), a in sorted(agg.items()):
            n = len(a.pop("dispatches"))
            vals = " ".join(f"{c}={v / n:.6g}" for c, v in sorted(a.items()))
            print(f"{name[:64]:64s} grid={grid:>9s} n={n:4d} {vals}")
            r = []
            if a.get("SQ_BUSY_CU_CYCLES") and "SQ_VALU_MFMA_BUSY_CYCLES" in a:
                r.append(f"mfma_busy={a['SQ_VALU_MFMA_BUSY_CYCLES'] / (4 * a['SQ_BUSY_CU_CYCLES']):.3f}")
            if a.get("SQ_LDS_IDX_ACTIVE") and "SQ_LDS_BANK_CONFLICT" in a:
                r.append(f"lds_conflict={a['SQ_LDS_BANK_CONFLICT'] / a['SQ_LDS_IDX_ACTIVE']:.3f}")
            if a.get("SQ_WAVE_CYCLES") and "SQ_WAIT_INST_ANY" in a:
                r.append(f"wave_wait={a['SQ_WAIT_INST_ANY'] / a['SQ_WAVE_CYCLES']:.3f}")
            if r:
                ratios.append(f"{name[:64]:64s} grid={grid:>9s} " + " ".join(r))
        if ratios:
            print("# ratios: mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs x SQ_BUSY_CU_CYCLES); "
                  "lds_conflict = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; "
                  "wave_wait = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES")
            print("\n".join(ratios))


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle leg (for profiler runs)")
    ap.add_argument("--cpu-fraction", type=int, default=6,
                    help="the CPU sample computes 1/N of layer 0's output rows")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before warmup, run one plain device copy of this many MiB (a "
                         "known-size kernel for scaling HBM byte counters)")
    ap.add_argument("--quantizer", choices=("fused", "separate"), default="fused",
                    help="fused: one dual-axis pass per activation/gradient tensor; separate: "
                         "row-tile and token-axis kernels called one after the other")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip the measurements of the layer-level comparisons that follow the "
                         "step (for profiler runs, whose kernel statistics should hold the step "
                         "alone)")
    ap.add_argument("--summarize-rocprof", metavar="DIR",
                    help="print a text summary of rocprofv3 CSV output in DIR and exit")
    return ap.parse_args()


class Plan:
    """Preallocated buffers and the ordered list of library calls of one step."""

    def __init__(self, torch, fp8, inputs):
        self.torch = torch
        cfg = inputs.CONFIGS["linear_set"]
        self.cfg = cfg
        dev = torch.device("cuda")
        L = fp8.capi()
        self.L = L

        def bf16(bits):
            return torch.from_numpy(bits.view("int16")).view(torch.bfloat16).to(dev)

        t0 = time.perf_counter()
        shared = [n for n in cfg.tensors if n not in cfg.per_layer]
        self.act = {n: bf16(inputs.tensor("linear_set", n)) for n in shared}
        self.w = [{n: bf16(inputs.tensor("linear_set", n, layer=l)) for n in cfg.per_layer}
                  for l in range(cfg.layers)]
        torch.cuda.synchronize()
        self.gen_seconds = time.perf_counter() - t0

        u8, f32 = torch.uint8, torch.float32
        E = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
        self.rq, self.tq, self.wq = {}, {}, {}
        for n, x in self.act.items():
            M, C = x.shape
            self.rq[n] = (E((M, C), u8), E((M, C // 128), f32))
            self.tq[n] = (E((C, M), u8), E((C, M // 128), f32))
        for n in cfg.per_layer:
            N, K = self.w[0][n].shape
            self.wq[n] = (E((N, K), u8), E((K, N), u8), E((N // 128, K // 128), f32))
        self.out = {}
        self.ws = {}
        for g in cfg.gemms:
            if g.kind == "fprop":
                self.out[g.name] = E((g.M, g.N), torch.bfloat16)
            elif g.kind == "dgrad":
                self.out[g.name] = E((g.M, g.K), torch.bfloat16)
            else:
                self.out[g.name] = E((g.N, g.K), f32)
                nb = int(L.fp8_gemm_wgrad_workspace_bytes(g.M, g.N, g.K))
                self.ws[g.name] = E((max(nb, 1),), u8) if nb else None

    def ops(self, stream, fused: bool):
        """[(kind, callable, args, algorithmic units)] for one step; units are
        bytes for quantizers and flops for GEMMs.  With fused, each activation
        (forward) and output gradient (backward) is quantized along both axes
        in one pass; otherwise by the row-tile kernel where its GEMM needs it
        and by the token-axis kernel before each wgrad."""
        L, cfg = self.L, self.cfg
        ops = []

        def rowtile(name):
            x = self.act[name]
            M, K = x.shape
            q, s = self.rq[name]
            ops.append(("quant_rowtile", L.fp8_quantize_rowtile,
                        (x.data_ptr(), M, K, q.data_ptr(), s.data_ptr(), stream),
                        M * K * 3 + M * (K // 128) * 4))

        def transposed(name):
            x = self.act[name]
            M, C = x.shape
            tq, ts = self.tq[name]
            ops.append(("quant_transposed", L.fp8_quantize_transposed,
                        (x.data_ptr(), M, C, tq.data_ptr(), ts.data_ptr(), stream),
                        M * C * 3 + C * (M // 128) * 4))

        def dual(name):
            x = self.act[name]
            M, C = x.shape
            q, s = self.rq[name]
            tq, ts = self.tq[name]
            ops.append(("quant_dual", L.fp8_quantize_dual,
                        (x.data_ptr(), M, C, q.data_ptr(), s.data_ptr(), tq.data_ptr(),
                         ts.data_ptr(), stream),
                        M * C * 4 + M * (C // 128) * 4 + C * (M // 128) * 4))

        for layer in range(cfg.layers):
            W = self.w[layer]
            fwd = [g for g in cfg.gemms if g.kind == "fprop"]
            for g in fwd:                                # forward
                (dual if fused else rowtile)(g.a)
                w = W[g.b]
                N, K2 = w.shape
                wq, wqt, ws = self.wq[g.b]
                ops.append(("quant_block", L.fp8_quantize_block,
                            (w.data_ptr(), N, K2, wq.data_ptr(), wqt.data_ptr(), ws.data_ptr(),
                             stream), N * K2 * 4 + (N // 128) * (K2 // 128) * 4))
                q, s = self.rq[g.a]
                ops.append(("gemm_fprop", L.fp8_gemm_fprop,
                            (q.data_ptr(), s.data_ptr(), wq.data_ptr(), ws.data_ptr(),
                             self.out[g.name].data_ptr(), 1, g.M, g.N, g.K, stream), g.flops))
            for g in fwd[::-1]:                           # backward, last linear first
                lin = g.name.split(".")[0]
                gd = next(x for x in cfg.gemms if x.name == lin + ".dgrad")
                gw = next(x for x in cfg.gemms if x.name == lin + ".wgrad")
                (dual if fused else rowtile)(gd.a)
                dq, ds = self.rq[gd.a]
                wq, wqt, ws = self.wq[gd.b]
                ops.append(("gemm_dgrad", L.fp8_gemm_dgrad,
                            (dq.data_ptr(), ds.data_ptr(), wqt.data_ptr(), ws.data_ptr(),
                             self.out[gd.name].data_ptr(), 1, gd.M, gd.N, gd.K, stream),
                            gd.flops))
                if not fused:
                    transposed(gw.a)
                    transposed(gw.b)
                dyt, dyts = self.tq[gw.a]
                xt, xts = self.tq[gw.b]
                wsb = self.ws[gw.name]
                ops.append(("gemm_wgrad", L.fp8_gemm_wgrad,
                            (dyt.data_ptr(), dyts.data_ptr(), xt.data_ptr(), xts.data_ptr(),
                             self.out[gw.name].data_ptr(), gw.M, gw.N, gw.K,
                             None if wsb is None else wsb.data_ptr(),
                             0 if wsb is None else wsb.numel(), stream), gw.flops))
        return ops

    def standalone_quant_ops(self, stream):
        """One row-tile and one token-axis quantization of every shared
        tensor: the single-axis kernels, timed outside the step when the step
        uses the fused one."""
        L = self.L
        ops = []
        for name, x in self.act.items():
            M, C = x.shape
            q, s = self.rq[name]
            tq, ts = self.tq[name]
            ops.append(("quant_rowtile", L.fp8_quantize_rowtile,
                        (x.data_ptr(), M, C, q.data_ptr(), s.data_ptr(), stream),
                        M * C * 3 + M * (C // 128) * 4))
            ops.append(("quant_transposed", L.fp8_quantize_transposed,
                        (x.data_ptr(), M, C, tq.data_ptr(), ts.data_ptr(), stream),
                        M * C * 3 + C * (M // 128) * 4))
        return ops


def accumulate_kinds(kinds, ops, events):
    for i, (kind, _, _, units) in enumerate(ops):
        ms = events[i].elapsed_time(events[i + 1])
        k = kinds.setdefault(kind, {"ms": 0.0, "units": 0, "launches": 0})
        k["ms"] += ms
        k["units"] += units
        k["launches"] += 1


def kind_summary(kinds, steps):
    out = {}
    for kind, k in sorted(kinds.items(), key=lambda kv: -kv[1]["ms"]):
        sec = k["ms"] / 1e3
        is_gemm = kind.startswith("gemm")
        rate = k["units"] / sec / (1e12 if is_gemm else 1e9)
        peak = PEAK_F16_TFLOPS if is_gemm else PEAK_HBM_GBS
        out[kind] = {
            "ms_per_step": round(k["ms"] / steps, 3),
            "launches_per_step": k["launches"] // steps,
            "avg_launch_us": round(k["ms"] / k["launches"] * 1e3, 2),
            "rate": round(rate, 2), "unit": "TFLOP/s" if is_gemm else "GB/s",
            "frac": round(rate / peak, 4)}
    return out


def run_step(ops, events=None):
    for i, (kind, fn, args, _) in enumerate(ops):
        if events is not None:
            events[i].record()
        rc = fn(*args)
        if rc != 0:
            raise RuntimeError(f"{kind} returned status {rc}")
    if events is not None:
        events[len(ops)].record()


def cpu_baseline(fraction: int, gpu=None):
    """The oracle, as it stands, on layer 0 of the same workload: each of the
    12 GEMMs on 1/fraction of its output rows, with the quantization those
    rows need (row tiles of the sampled rows, whole weight blocks, token-axis
    tiles of the sampled gradient channels and of the whole other operand).
    With gpu (host copies of the GPU's layer-0 codes, scales and outputs, see
    gpu_layer0), the oracle's results are then compared with them, outside
    the timed part: (baseline, parity)."""
    import numpy as np

    import oracle
    from fp8_block_scaled_03_amd import inputs

    cfg = inputs.CONFIGS["linear_set"]
    cores = len(os.sched_getaffinity(0))
    host = {n: inputs.tensor("linear_set", n, layer=0) for n in cfg.tensors}
    flops = 0
    results = []
    t0 = time.perf_counter()
    for g in cfg.gemms:
        a, b = host[g.a], host[g.b]
        if g.kind in ("fprop", "dgrad"):
            rows = np.arange(0, g.M, fraction)
            aq, as_ = oracle.quantize_rowtile(np.ascontiguousarray(a[rows]), threads=cores)
            wq, wqt, ws = oracle.quantize_block(b, with_transpose=(g.kind == "dgrad"),
                                                threads=cores)
            if g.kind == "fprop":
                y = oracle.gemm_fprop(aq, as_, wq, ws, threads=cores)
            else:
                y = oracle.gemm_dgrad(aq, as_, wqt, ws, threads=cores)
            flops += 2 * len(rows) * g.N * g.K
            results.append((g, rows, (aq, as_), (wq, wqt, ws), y))
        else:
            rows = np.arange(0, g.N, fraction)
            dq, ds = oracle.quantize_transposed(np.ascontiguousarray(a[:, rows]), threads=cores)
            xq, xs = oracle.quantize_transposed(b, threads=cores)
            y = oracle.gemm_wgrad(dq, ds, xq, xs, threads=cores)
            flops += 2 * len(rows) * g.K * g.M
            results.append((g, rows, (dq, ds), (xq, xs), y))
    secs = time.perf_counter() - t0
    baseline = {"value": round(flops / secs / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
                "kind": "oracle",
                "sample": f"layer 0 of the 28-layer linear set: all 12 GEMMs on 1/{fraction} of "
                          f"their output rows ({flops / 1e9:.1f} GFLOP) plus the quantization "
                          f"those rows need; {secs:.1f} s wall"}
    if gpu is None:
        return baseline, None
    return baseline, _parity_against_oracle(np, oracle, gpu, results)


def _parity_against_oracle(np, oracle, gpu, results):
    """Codes and scales must match bit for bit; FP32 outputs relF <= 1e-5 and
    |err| <= 1e-4 ||a_i|| ||b_j|| (dequantized contraction vectors); BF16
    outputs within one BF16 ulp of the rounded oracle value, or within that
    bound plus half an ulp."""
    codes_ok = True
    gemms = {}
    for g, rows, qa, qb, y in results:
        if g.kind in ("fprop", "dgrad"):
            rq, rs = gpu["rq"][g.a]
            codes_ok &= np.array_equal(rq[rows], qa[0]) and np.array_equal(
                rs[rows].view(np.uint32), qa[1].view(np.uint32))
            wq, wqt, ws = gpu["wq"][g.b]
            codes_ok &= np.array_equal(wq, qb[0]) and np.array_equal(
                ws.view(np.uint32), qb[2].view(np.uint32))
            a_deq = oracle.dequantize_rows(*qa)
            w_deq = oracle.dequantize_block(qb[0], qb[2])
            if g.kind == "dgrad":
                codes_ok &= np.array_equal(wqt, qb[1])
                w_deq = np.ascontiguousarray(w_deq.T)
            out = gpu["out"][g.name][rows]
            ref_bits = oracle.f32_to_bf16(y)
            got = oracle.bf16_to_f32(out).astype(np.float64)
            ref = oracle.bf16_to_f32(ref_bits).astype(np.float64)
            mag = np.maximum(np.abs(ref), np.finfo(np.float32).tiny)
            ulp = np.exp2(np.floor(np.log2(mag)) - 7)
            bound = 1e-4 * np.outer(np.linalg.norm(a_deq, axis=1), np.linalg.norm(w_deq, axis=1))
            err = np.abs(got - ref)
            ok = (err <= ulp) | (err <= bound + 0.5 * ulp)
            gemms[g.name] = {"out": "bf16", "elements": int(ok.size),
                             "within_gate": bool(ok.all()),
                             "relF_vs_fp32_oracle": float(f"{oracle.rel_frobenius(got, y):.3e}")}
        else:
            tq, ts = gpu["tq"][g.a]
            codes_ok &= np.array_equal(tq[rows], qa[0]) and np.array_equal(
                ts[rows].view(np.uint32), qa[1].view(np.uint32))
            xq, xs = gpu["tq"][g.b]
            codes_ok &= np.array_equal(xq, qb[0]) and np.array_equal(
                xs.view(np.uint32), qb[1].view(np.uint32))
            out = gpu["out"][g.name][rows]
            rel = oracle.rel_frobenius(out, y)
            ratio = oracle.elementwise_bound_ratio(out, y, oracle.dequantize_rows(*qa),
                                                   oracle.dequantize_rows(*qb), 1e-4)
            gemms[g.name] = {"out": "f32", "elements": int(out.size),
                             "within_gate": bool(rel <= 1e-5 and ratio <= 1.0),
                             "relF": float(f"{rel:.3e}"),
                             "max_err_over_bound": float(f"{ratio:.3e}")}
    return {"layer": 0, "codes_and_scales_bit_exact": bool(codes_ok),
            "all_gemms_within_gate": all(v["within_gate"] for v in gemms.values()),
            "gemms": gemms}


def gpu_layer0(torch, plan, ops):
    """Run layer 0's launches of the step once more and copy what they wrote
    (codes, scales, outputs) to the host, for the oracle comparison."""
    per_layer = len(ops) // plan.cfg.layers
    run_step(ops[:per_layer])
    torch.cuda.synchronize()

    def host(t):
        t = t.cpu()
        return t.view(torch.int16).numpy().view("uint16") if t.dtype == torch.bfloat16 else t.numpy()

    return {"rq": {n: tuple(host(t) for t in v) for n, v in plan.rq.items()},
            "tq": {n: tuple(host(t) for t in v) for n, v in plan.tq.items()},
            "wq": {n: tuple(host(t) for t in v) for n, v in plan.wq.items()},
            "out": {n: host(t) for n, t in plan.out.items()}}


LAYER_LINEARS = [("qkv", 2048, 4096), ("o", 2048, 2048), ("gate_up", 2048, 12288),
                 ("down", 6144, 2048)]


def _time_events(torch, fn, reps):
    fn()
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def mfma_ceiling(torch, fp8, reps=5):
    """Attainable FP16 MFMA rate of this GPU in TFLOP/s: the library's MFMA-only
    diagnostic kernel (8 workgroups of 256 threads per CU, ~3 ms a launch),
    best of reps, after checking its exact output."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters, v = 8 * cus, 400, 0.125
    flop = blocks * 4 * iters * 128 * 16384
    out = fp8.fp8bs_mfma_rate(blocks, iters, v)
    torch.cuda.synchronize()
    expect = 16384 * v * v * iters
    if not bool((out == expect).all()):
        raise RuntimeError("MFMA-rate kernel returned wrong values")
    best = min(_time_events(torch, lambda: fp8.fp8bs_mfma_rate(blocks, iters, v, out=out), 1)
               for _ in range(reps))
    return flop / (best / 1e3) / 1e12


def bf16_comparison(torch, fp8, cfg, fp8_ms_per_layer, reps=5):
    """The 12 GEMMs of one layer in TN form on BF16 operands: this library's
    BF16 kernel and torch's BF16 matmul (the vendor BLAS), against the FP8
    GEMMs' device time per layer in the step."""
    gen = torch.Generator(device="cuda").manual_seed(1)
    own = blas = 0.0
    flops = 0
    for g in cfg.gemms:
        if g.kind == "fprop":
            I, J, K = g.M, g.N, g.K
        elif g.kind == "dgrad":
            I, J, K = g.M, g.K, g.N
        else:
            I, J, K = g.N, g.K, g.M
        out = torch.float32 if g.kind == "wgrad" else torch.bfloat16
        a = torch.randn(I, K, device="cuda", generator=gen).bfloat16()
        b = torch.randn(J, K, device="cuda", generator=gen).bfloat16()
        c = torch.empty(I, J, device="cuda", dtype=out)
        own += _time_events(torch, lambda: fp8.bf16_gemm_tn(a, b, out_dtype=out, c=c), reps)
        blas += _time_events(torch, lambda: torch.matmul(a, b.t(), out=c) if out == torch.bfloat16
                             else torch.matmul(a, b.t()), reps)
        flops += g.flops
        del a, b, c
    return {"f2_bf16_gemm": {
        "workload": "one layer's 12 GEMMs of the linear set (16384 tokens) in TN form on BF16 "
                    "operands, FP32 accumulation, BF16 out (FP32 for wgrad)",
        "bf16_ms_per_layer": round(own, 3), "bf16_tflops": round(flops / own / 1e9, 1),
        "fp8_ms_per_layer": round(fp8_ms_per_layer, 3),
        "fp8_tflops": round(flops / fp8_ms_per_layer / 1e9, 1),
        "fp8_speedup_vs_own_bf16": round(own / fp8_ms_per_layer, 3),
        "torch_bf16_ms_per_layer": round(blas, 3), "torch_bf16_tflops": round(flops / blas / 1e9, 1)}}


def dgrad_epilogue_quantization(torch, fp8, cfg, reps=5):
    """One layer's four dgrad GEMMs at 16,384 tokens: dgrad with BF16 output
    followed by the row-tile quantizer on dX, against the same with the
    quantizer fused into the dgrad epilogue (BF16 dX kept, or codes only)."""
    gen = torch.Generator(device="cuda").manual_seed(2)
    sep = fused = codes_only = 0.0
    for g in cfg.gemms:
        if g.kind != "dgrad":
            continue
        dy = (torch.randn(g.M, g.N, device="cuda", generator=gen) * 1e-3).bfloat16()
        w = (torch.randn(g.N, g.K, device="cuda", generator=gen) * 0.02).bfloat16()
        dyq, dys = fp8.fp8_quantize_rowtile(dy)
        _, wqt, ws = fp8.fp8_quantize_block(w)
        dx = torch.empty(g.M, g.K, device="cuda", dtype=torch.bfloat16)
        q = torch.empty(g.M, g.K, device="cuda", dtype=torch.uint8)
        s = torch.empty(g.M, g.K // 128, device="cuda", dtype=torch.float32)

        def separate():
            fp8.fp8_gemm_dgrad(dyq, dys, wqt, ws, dx=dx)
            fp8.fp8_quantize_rowtile(dx, q, s)

        sep += _time_events(torch, separate, reps)
        fused += _time_events(torch, lambda: fp8.fp8_gemm_dgrad_quantized(
            dyq, dys, wqt, ws, dx=dx, dxq=q, dxs=s), reps)
        codes_only += _time_events(torch, lambda: fp8.fp8_gemm_dgrad_quantized(
            dyq, dys, wqt, ws, with_bf16=False, dxq=q, dxs=s), reps)
        del dy, w, dyq, dys, wqt, ws, dx, q, s
    return {"f3_dgrad_quantize_on_produce": {
        "workload": "one layer's four dgrad GEMMs of the linear set (16384 tokens), each "
                    "followed by 1x128 row-tile quantization of dX",
        "separate_ms_per_layer": round(sep, 3), "fused_ms_per_layer": round(fused, 3),
        "fused_codes_only_ms_per_layer": round(codes_only, 3),
        "fused_speedup": round(sep / fused, 3)}}


def fp8_linear_comparison(torch, fp8, reps=5):
    """One decoder layer's four linears at 16,384 tokens, forward + backward:
    through Fp8Linear (the FP8 block-scaled path) and through torch's BF16
    linear (the vendor BLAS), on the same shapes."""
    T = 16384
    gen = torch.Generator(device="cuda").manual_seed(0)
    mods, bf_w, xs, dys = [], [], [], []
    for _, d_in, d_out in LAYER_LINEARS:
        m = fp8.Fp8Linear(d_in, d_out, device="cuda")
        mods.append(m)
        bf_w.append(m.weight.detach().clone().requires_grad_(True))
        xs.append(torch.randn(T, d_in, device="cuda", generator=gen).bfloat16().requires_grad_(True))
        dys.append((torch.randn(T, d_out, device="cuda", generator=gen) * 1e-3).bfloat16())

    def fp8_layer():
        for m, x, dy in zip(mods, xs, dys):
            x.grad = None
            m.weight.grad = None
            m(x).backward(dy)

    def bf16_layer():
        for w, x, dy in zip(bf_w, xs, dys):
            x.grad = None
            w.grad = None
            torch.nn.functional.linear(x, w).backward(dy)

    flops = sum(3 * 2 * T * d_in * d_out for _, d_in, d_out in LAYER_LINEARS)
    ms8 = _time_events(torch, fp8_layer, reps)
    ms16 = _time_events(torch, bf16_layer, reps)
    return {"f4_fp8_linear_layer": {
        "workload": "one decoder layer's QKV, O, gate/up and down linears at 16384 tokens, "
                    "forward + backward (dual quantization of X and dY, block quantization of "
                    "W, fprop, dgrad, wgrad)",
        "fp8_ms": round(ms8, 3), "fp8_tflops": round(flops / ms8 / 1e9, 1),
        "torch_bf16_ms": round(ms16, 3), "torch_bf16_tflops": round(flops / ms16 / 1e9, 1),
        "fp8_speedup_vs_torch_bf16": round(ms16 / ms8, 3)}}


def main():
    args = parse()
    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the path is "
                          "measured on one MI355X and has no multi-GPU mode",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch

    import fp8_block_scaled_03_amd as fp8
    from fp8_block_scaled_03_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fp8.capi()                                   # fails loudly if the library is missing
    plan = Plan(torch, fp8, inputs)
    stream = torch.cuda.current_stream()
    fused = args.quantizer == "fused"
    ops = plan.ops(stream.cuda_stream, fused)
    print(f"# setup: {len(ops)} launches per step, inputs generated in "
          f"{plan.gen_seconds:.1f} s", file=sys.stderr, flush=True)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        run_step(ops)
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        run_step(ops, events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-kind device time from the events bracketing every launch
    kinds = {}
    for s in range(args.steps):
        accumulate_kinds(kinds, ops, events[s])
    standalone = {}
    if fused:
        sops = plan.standalone_quant_ops(stream.cuda_stream)
        sev = [torch.cuda.Event(enable_timing=True) for _ in range(len(sops) + 1)]
        run_step(sops)
        torch.cuda.synchronize()
        run_step(sops, sev)
        torch.cuda.synchronize()
        accumulate_kinds(standalone, sops, sev)
    step_ms = wall / args.steps * 1e3
    gemm_flops = sum(g.flops for g in plan.cfg.gemms) * plan.cfg.layers
    value = gemm_flops / (wall / args.steps) / 1e12

    breakdown = kind_summary(kinds, args.steps)
    dom = next(iter(breakdown))
    d = breakdown[dom]
    dom_is_gemm = dom.startswith("gemm")
    roofline = {
        "kernel": dom,
        "bound": "mfma" if dom_is_gemm else "hbm",
        "achieved": d["rate"],
        "peak": PEAK_F16_TFLOPS if dom_is_gemm else PEAK_HBM_GBS,
        "unit": d["unit"],
        "frac": d["frac"],
        "traffic": None,
        "traffic_source": None,
        "note": ("contraction runs on FP16 MFMA (E4M3 widened exactly in registers); "
                 "gfx950 FP8 MFMA truncates within 8-product groups and misses FP32 "
                 "accumulation parity") if dom_is_gemm else "",
    }

    if dom_is_gemm:
        # the same kernel's rate against what the matrix cores sustain on this
        # GPU at the clock they hold under load (measured after the timed steps)
        ceiling = mfma_ceiling(torch, fp8)
        roofline["peak_at_clock"] = round(ceiling, 1)
        roofline["frac_at_clock"] = round(d["rate"] / ceiling, 4)
    rec = recorded_traffic(dom)
    if rec:
        roofline["traffic"] = rec["bytes_per_launch"]
        roofline["traffic_source"] = rec["profile"]
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 operands on f16 mfma, f32 accumulation",
        "data": "synthetic",
        "config": {"workload": "linear_set: 28-layer Qwen3-1.7B-like decoder micro-batch, "
                               "4x4096 tokens, hidden 2048, FFN 6144, QKV 4096; per layer "
                               "fprop+dgrad+wgrad of QKV, O, gate/up, down with all quantizers",
                   "tokens": 16384, "layers": 28, "gemm_tflop_per_step": round(gemm_flops / 1e12, 3),
                   "launches_per_step": len(ops), "quantizer": args.quantizer},
        "pct_fp8_peak": round(100 * value / PEAK_FP8_TFLOPS, 2),
        "roofline": roofline,
        "kernels": breakdown,
    }
    if standalone:
        result["kernels_outside_step"] = kind_summary(standalone, 1)
    # the GPU's own layer-0 results, compared with the oracle's in the cpu_baseline leg
    layer0 = None if args.no_cpu_baseline else gpu_layer0(torch, plan, ops)
    if not args.no_next_rows:
        cfg_obj, cfg_layers = plan.cfg, plan.cfg.layers
        del plan, ops, events
        torch.cuda.empty_cache()
        fp8_gemm_ms = sum(v["ms_per_step"] for k, v in breakdown.items()
                          if k.startswith("gemm")) / cfg_layers
        result["next_rows"] = {**bf16_comparison(torch, fp8, cfg_obj, fp8_gemm_ms),
                               **dgrad_epilogue_quantization(torch, fp8, cfg_obj),
                               **fp8_linear_comparison(torch, fp8)}
    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["parity_sample"] = cpu_baseline(args.cpu_fraction, layer0)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
