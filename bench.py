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
    "gemm_mfma8": ["gemm_mfma8.hip", "gemm.hip", "gemm_common.h", "device_common.h", "internal.h"],
    "quant": ["quantize.hip", "device_common.h", "internal.h"],
}


def _source_set(kind: str) -> str:
    """Which sources a kernel kind is built from (the FP8-MFMA GEMMs' split-K
    reduction lives in gemm.hip)."""
    if kind.startswith("gemm"):
        return "gemm_mfma8" if kind.endswith("_mfma8") else "gemm"
    return "quant"


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
    for fn in KERNEL_SOURCES[_source_set(kind)]:
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
    if "rmsnorm_rstd_kernel" in name:               # the first launch of an RMSNorm call
        return "rmsnorm_dual", False
    for k in ("rmsnorm_dual", "swiglu_bwd_dual", "swiglu_dual"):
        if k + "_kernel" in name:
            return k, True
    m = re.search(r"gemm_bs_fp8(?:_big)?_kernel<(\d)", name)
    if m:
        return ("gemm_fprop", "gemm_dgrad", "gemm_wgrad")[int(m.group(1))], True
    m = re.search(r"gemm_mfma8_kernel<(\d)", name)
    if m:
        return ("gemm_fprop_mfma8", "gemm_dgrad_mfma8", "gemm_wgrad_mfma8")[int(m.group(1))], True
    if "quant_block_many_kernel" in name:           # a layer's weights in one launch
        return "quant_block", True
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
            name = r["Name"].replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")[:64]
            print(f"{name:64s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                  f"{float(r['TotalDurationNs']) / 1e6:10.3f} {float(r['Percentage']):6.2f}")
        per_kind = {}
        trace = os.path.join(os.path.dirname(path), os.path.basename(path).replace(
            "kernel_stats.csv", "kernel_trace.csv"))
        if os.path.exists(trace):
            # dispatch order: a split-K reduction belongs to the wgrad call before it
            last_wgrad = "gemm_wgrad"
            rows = sorted(csv.DictReader(open(trace)), key=lambda r: int(r["Dispatch_Id"]))
            for r in rows:
                kind, is_call = kernel_kind(r["Kernel_Name"])
                if kind and kind.startswith("gemm_wgrad") and is_call:
                    last_wgrad = kind
                elif kind and not is_call and kind.startswith("gemm_wgrad"):
                    kind = last_wgrad
                if kind:
                    k = per_kind.setdefault(kind, [0.0, 0])
                    k[0] += float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
                    k[1] += 1 if is_call else 0
        else:
            for r in csv.DictReader(open(path)):
                kind, is_call = kernel_kind(r["Name"])
                if kind:
                    k = per_kind.setdefault(kind, [0.0, 0])
                    k[0] += float(r["TotalDurationNs"])
                    k[1] += int(r["Calls"]) if is_call else 0
        print("# per library call (split-K reductions counted with the wgrad call they follow)")
        print(f"{'kind':20s} {'calls':>6s} {'avg_us_per_call':>16s} {'total_ms':>10s}")
        for kind, (ns, calls) in sorted(per_kind.items(), key=lambda kv: -kv[1][0]):
            print(f"{kind:20s} {calls:6d} {ns / max(calls, 1) / 1e3:16.2f} {ns / 1e6:10.3f}")
    pmc = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    for path in pmc:
        agg = {}
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
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


def _pmc_dispatches(d: str, counter: str):
    """[(kernel name, grid, value)] of one counter, one entry per dispatch,
    from a rocprofv3 --pmc run (-f csv) under d."""
    import csv
    import glob
    out = {}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = (path, r["Dispatch_Id"])
            name = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
            prev = out.get(key, (name, r["Grid_Size"], 0.0))
            out[key] = (name, r["Grid_Size"], prev[2] + float(r["Counter_Value"]))
    return list(out.values())


def record_traffic(fetch_dir: str, write_dir: str, out_path: str | None = TRAFFIC_FILE) -> None:
    """HBM bytes per library call from two counter runs of the step (FETCH_SIZE
    and WRITE_SIZE, KiB per dispatch, each run made with --copy-calibration-mib
    1024).  Each counter is scaled by what it reads for that plain 1 GiB
    device copy; a wgrad call's bytes include its split-K reduction.  Writes
    the per-kind records (keyed to the kernel sources' digest; not with out_path
    None) and prints the per-kernel lines."""
    fetch = _pmc_dispatches(fetch_dir, "FETCH_SIZE")
    write = _pmc_dispatches(write_dir, "WRITE_SIZE")
    gib_kib = float(1 << 20)

    def factor(rows):
        copies = [v for n, g, v in rows if "copyBuffer" in n]
        return gib_kib / max(copies) if copies and max(copies) > 0 else 1.0

    ff, fw = factor(fetch), factor(write)
    print(f"# scale: the 1 GiB device copy reads {max(v for n, g, v in fetch if 'copyBuffer' in n):.0f} "
          f"KiB of FETCH_SIZE and {max(v for n, g, v in write if 'copyBuffer' in n):.0f} KiB of "
          f"WRITE_SIZE; factors applied: FETCH x{ff:.4f}, WRITE x{fw:.4f}")
    per_kernel = {}
    for rows, f, col in ((fetch, ff, 0), (write, fw, 1)):
        for n, g, v in rows:
            e = per_kernel.setdefault((n, g), [[], []])
            e[col].append(v * f * 1024)
    kinds = {}
    for (n, g), (fb, wb) in sorted(per_kernel.items()):
        nd = max(len(fb), len(wb))
        mf = sum(fb) / max(len(fb), 1) / 1e6
        mw = sum(wb) / max(len(wb), 1) / 1e6
        print(f"{n[:60]:60s} grid={g:>9s} n={nd:4d} fetch_MB={mf:10.2f} write_MB={mw:10.2f}")
        kind, is_call = kernel_kind(n)
        if kind:
            k = kinds.setdefault(kind, [0.0, 0])
            k[0] += sum(fb) / max(len(fb), 1) * nd + sum(wb) / max(len(wb), 1) * nd
            k[1] += nd if is_call else 0
    rec = {}
    for kind, (b, calls) in kinds.items():
        if calls:
            rec[kind] = {"bytes_per_launch": int(b / calls), "launches": calls,
                         "profile": "profiles/linear_set_hbm_bytes.txt",
                         "source_sha256_16": source_digest(kind)}
    if out_path:
        with open(out_path, "w") as f:
            json.dump(rec, f, indent=1)
    print("# per library call (a wgrad call includes its split-K reduction)")
    for kind, r in sorted(rec.items()):
        print(f"{kind:20s} calls={r['launches']:5d} bytes_per_call={r['bytes_per_launch'] / 1e6:10.2f} MB")


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
    ap.add_argument("--no-mfma8", action="store_true",
                    help="skip the step with the FP8-MFMA GEMMs (fp8_gemm_*_mfma8)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration measurements of configurations 1-4")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from a FETCH_SIZE and a WRITE_SIZE "
                         "rocprofv3 run of the step and print the per-kernel bytes, then exit")
    ap.add_argument("--producers", action="store_true",
                    help="measure only the quantize-on-produce calls (RMSNorm, SwiGLU and its "
                         "backward at 16384 tokens), print them as one JSON line and exit (for "
                         "profiler runs of those kernels)")
    ap.add_argument("--traffic-print-only", action="store_true",
                    help="with --record-traffic: print the per-kernel bytes but leave "
                         "profiles/traffic.json (which holds the step's records) as it is")
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
                nb = max(int(L.fp8_gemm_wgrad_workspace_bytes(g.M, g.N, g.K)),
                         int(L.fp8_gemm_wgrad_mfma8_workspace_bytes(g.M, g.N, g.K)))
                self.ws[g.name] = E((max(nb, 1),), u8) if nb else None

    def ops(self, stream, fused: bool, mfma8: bool = False):
        """[(kind, callable, args, algorithmic units)] for one step; units are
        bytes for quantizers and flops for GEMMs.  With fused, each activation
        (forward) and output gradient (backward) is quantized along both axes
        in one pass; otherwise by the row-tile kernel where its GEMM needs it
        and by the token-axis kernel before each wgrad.  With mfma8 the GEMMs
        are the fp8_gemm_*_mfma8 calls (block sums on the FP8 matrix core)."""
        L, cfg = self.L, self.cfg
        fprop = L.fp8_gemm_fprop_mfma8 if mfma8 else L.fp8_gemm_fprop
        dgrad = L.fp8_gemm_dgrad_mfma8 if mfma8 else L.fp8_gemm_dgrad
        wgrad = L.fp8_gemm_wgrad_mfma8 if mfma8 else L.fp8_gemm_wgrad
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

        import ctypes

        from fp8_block_scaled_03_amd._binding import BlockJob
        self._jobs = getattr(self, "_jobs", [])      # the job tables must outlive the ops
        for layer in range(cfg.layers):
            W = self.w[layer]
            fwd = [g for g in cfg.gemms if g.kind == "fprop"]
            # the layer's four weights through the block quantizer in one launch
            jobs = (BlockJob * len(fwd))()
            wbytes = 0
            for i, g in enumerate(fwd):
                w = W[g.b]
                N, K2 = w.shape
                wq, wqt, ws = self.wq[g.b]
                jobs[i] = BlockJob(w.data_ptr(), N, K2, wq.data_ptr(), wqt.data_ptr(), ws.data_ptr())
                wbytes += N * K2 * 4 + (N // 128) * (K2 // 128) * 4
            self._jobs.append(jobs)
            ops.append(("quant_block", L.fp8_quantize_block_many,
                        (ctypes.cast(jobs, ctypes.c_void_p), len(fwd), stream), wbytes))
            for g in fwd:                                # forward
                (dual if fused else rowtile)(g.a)
                wq, wqt, ws = self.wq[g.b]
                q, s = self.rq[g.a]
                ops.append(("gemm_fprop", fprop,
                            (q.data_ptr(), s.data_ptr(), wq.data_ptr(), ws.data_ptr(),
                             self.out[g.name].data_ptr(), 1, g.M, g.N, g.K, stream), g.flops))
            for g in fwd[::-1]:                           # backward, last linear first
                lin = g.name.split(".")[0]
                gd = next(x for x in cfg.gemms if x.name == lin + ".dgrad")
                gw = next(x for x in cfg.gemms if x.name == lin + ".wgrad")
                (dual if fused else rowtile)(gd.a)
                dq, ds = self.rq[gd.a]
                wq, wqt, ws = self.wq[gd.b]
                ops.append(("gemm_dgrad", dgrad,
                            (dq.data_ptr(), ds.data_ptr(), wqt.data_ptr(), ws.data_ptr(),
                             self.out[gd.name].data_ptr(), 1, gd.M, gd.N, gd.K, stream),
                            gd.flops))
                if not fused:
                    transposed(gw.a)
                    transposed(gw.b)
                dyt, dyts = self.tq[gw.a]
                xt, xts = self.tq[gw.b]
                wsb = self.ws[gw.name]
                ops.append(("gemm_wgrad", wgrad,
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


def cpu_baseline(fraction: int, gpu=None, gpu_mfma8=None):
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
                "cpu": cpu_model(), "kind": "oracle",
                "sample": f"layer 0 of the 28-layer linear set: all 12 GEMMs on 1/{fraction} of "
                          f"their output rows ({flops / 1e9:.1f} GFLOP) plus the quantization "
                          f"those rows need; {secs:.1f} s wall"}
    parity = None if gpu is None else _parity_against_oracle(np, oracle, gpu, results)
    parity8 = None if gpu_mfma8 is None else _parity_mfma8(np, oracle, gpu_mfma8, results)
    return baseline, parity, parity8


def bf16_gate(np, oracle, out_bits, ref_f32, a_deq, b_deq):
    """Per-element pass mask of BF16 outputs: within one BF16 ulp of the
    rounded oracle value; only where the oracle value is itself no larger
    than the FP32 bound 1e-4 ||a_i|| ||b_j|| may it differ by that bound plus
    one ulp of the larger value (an FP32-level difference spans many ulps of
    so small a value)."""
    got = oracle.bf16_to_f32(out_bits).astype(np.float64)
    r = oracle.bf16_to_f32(oracle.f32_to_bf16(ref_f32)).astype(np.float64)
    tiny = np.finfo(np.float32).tiny
    ulp = lambda v: np.exp2(np.floor(np.log2(np.maximum(np.abs(v), tiny))) - 7)
    bound = 1e-4 * np.outer(np.linalg.norm(a_deq, axis=1), np.linalg.norm(b_deq, axis=1))
    err = np.abs(got - r)
    near_zero = np.abs(np.asarray(ref_f32, np.float64)) <= bound
    return (err <= ulp(r)) | (near_zero & (err <= bound + ulp(np.maximum(np.abs(r), np.abs(got)))))


def _parity_against_oracle(np, oracle, gpu, results):
    """Codes and scales must match bit for bit; FP32 outputs relF <= 1e-5 and
    |err| <= 1e-4 ||a_i|| ||b_j|| (dequantized contraction vectors); BF16
    outputs as bf16_gate."""
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
            got = oracle.bf16_to_f32(out).astype(np.float64)
            ok = bf16_gate(np, oracle, out, y, a_deq, w_deq)
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


MFMA8_ELEM_C = 2.0 ** -9 + 2.0 ** -16    # per element, times ||a_i|| ||b_j||
MFMA8_RELF = 1e-4


def _parity_mfma8(np, oracle, gpu, results):
    """The FP8-MFMA GEMMs against the exact oracle: the matrix core's
    window bounds each block sum's error by 2^-9 times the sum of its
    products' magnitudes, so |err| <= (2^-9 + 2^-16) ||a_i|| ||b_j|| per
    element (plus one BF16 ulp for BF16 outputs), and relF <= 1e-4 for FP32
    outputs."""
    gemms = {}
    for g, rows, qa, qb, y in results:
        if g.kind in ("fprop", "dgrad"):
            a_deq = oracle.dequantize_rows(*qa)
            w_deq = oracle.dequantize_block(qb[0], qb[2])
            b_deq = np.ascontiguousarray(w_deq.T) if g.kind == "dgrad" else w_deq
            got = oracle.bf16_to_f32(gpu["out"][g.name][rows]).astype(np.float64)
            ref = np.asarray(y, np.float64)
            bound = MFMA8_ELEM_C * np.outer(np.linalg.norm(a_deq, axis=1),
                                            np.linalg.norm(b_deq, axis=1))
            tiny = np.finfo(np.float32).tiny
            ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref) + bound, tiny))) - 7)
            ok = np.abs(got - ref) <= bound + ulp
            gemms[g.name] = {"out": "bf16", "elements": int(ok.size), "within_gate": bool(ok.all()),
                             "relF_vs_fp32_oracle": float(f"{oracle.rel_frobenius(got, y):.3e}")}
        else:
            out = gpu["out"][g.name][rows]
            rel = oracle.rel_frobenius(out, y)
            ratio = oracle.elementwise_bound_ratio(out, y, oracle.dequantize_rows(*qa),
                                                   oracle.dequantize_rows(*qb), MFMA8_ELEM_C)
            gemms[g.name] = {"out": "f32", "elements": int(out.size),
                             "within_gate": bool(rel <= MFMA8_RELF and ratio <= 1.0),
                             "relF": float(f"{rel:.3e}"), "max_err_over_bound": float(f"{ratio:.3e}")}
    return {"layer": 0, "gate": "per element (2^-9 + 2^-16) ||a_i|| ||b_j|| (+1 BF16 ulp); "
                                "FP32 outputs also relF <= 1e-4",
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

FLUSH_BYTES = 512 << 20       # > the 256 MB last-level cache


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def parse_sclk_json(text: str):
    """Graphics clocks (MHz) found in amd-smi ("gfx_N" clock entries) or
    rocm-smi ("sclk clock speed") JSON output, or None."""
    import re
    start = min((i for i in (text.find("{"), text.find("[")) if i >= 0), default=-1)
    if start < 0:
        return None
    try:
        data = json.loads(text[start:])
    except ValueError:
        return None
    found = []

    def walk(o, path):
        if isinstance(o, dict):
            for k, v in o.items():
                walk(v, path + [str(k).lower()])
        elif isinstance(o, list):
            for v in o:
                walk(v, path)
        else:
            key = " ".join(path)
            if (re.search(r"\bgfx_\d+ clk value$", key) or "sclk clock speed" in key):
                m = re.search(r"(\d+(?:\.\d+)?)", str(o))
                if m:
                    found.append(float(m.group(1)))

    walk(data, [])
    return found or None


def under_profiler() -> bool:
    """True inside a rocprofv3 run (its library is preloaded into every
    process, which then counts as using the GPU)."""
    return any("rocprof" in os.environ.get(k, "") for k in ("LD_PRELOAD", "HSA_TOOLS_LIB"))


def _smi_command(tool: str, args):
    """argv for an SMI tool.  Both are Python scripts started through
    /usr/bin/env; running the script with this interpreter avoids env
    replacing itself with python3 in a child of a process that uses the GPU."""
    import shutil
    path = shutil.which(tool) or os.path.join("/opt/rocm/bin", tool)
    try:
        with open(path, "rb") as f:
            first = f.readline()
    except OSError:
        return None
    if first.startswith(b"#!") and b"python" in first:
        return [sys.executable, path, *args]
    return [path, *args]


def _sclk_from_smi():
    """Current graphics clocks in MHz reported by amd-smi or rocm-smi (a list,
    one per GPU), or None when neither answers (or under a profiler)."""
    import subprocess
    if under_profiler():
        return None
    for tool, args in (("amd-smi", ["metric", "--clock", "--json"]),
                       ("rocm-smi", ["--showclocks", "--json"])):
        cmd = _smi_command(tool, args)
        if cmd is None:
            continue
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=20)
        except (OSError, subprocess.SubprocessError):
            continue
        if r.returncode == 0:
            v = parse_sclk_json(r.stdout)
            if v:
                return v
    return None


class SclkSampler:
    """Samples the graphics clock from the SMI tools in a background thread
    (the tool runs as a child process; the GIL is released while waiting)."""

    def __init__(self, period_s: float = 0.5):
        import threading
        self.period = period_s
        self.samples = []
        self.stop = threading.Event()
        self.thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        while not self.stop.is_set():
            v = _sclk_from_smi()
            if v is None:
                return
            self.samples.append(max(v))
            self.stop.wait(self.period)

    def __enter__(self):
        self.thread.start()
        return self

    def __exit__(self, *exc):
        self.stop.set()
        self.thread.join(timeout=30)

    def summary(self):
        if not self.samples:
            return None
        v = sorted(self.samples)
        return {"samples": len(v), "min_mhz": v[0], "median_mhz": v[len(v) // 2], "max_mhz": v[-1]}


class Timer:
    """Median kernel time of fn over reps iterations, each preceded by a
    write of a 512 MiB scratch buffer (outside the timed events) so the
    last-level cache holds nothing of the inputs; events are recorded on the
    current stream, the one the library calls are enqueued on."""

    def __init__(self, torch):
        self.torch = torch
        self.flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")

    def median_ms(self, fn, reps=25, warmup=3):
        torch = self.torch
        for _ in range(warmup):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for i, (a, b) in enumerate(ev):
            self.flush.fill_(i & 0xFF)
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) for a, b in ev)
        return t[len(t) // 2]


def hbm_ceiling(torch, fp8, timer, n: int, two_outputs: bool) -> float:
    """GB/s of the library's streaming probe moving the quantizers' bytes
    (2 read + 1 or 2 written per element) for n elements, cache flushed."""
    x = torch.empty(n, dtype=torch.int16, device="cuda").fill_(0x3F80)
    y0 = torch.empty(n, dtype=torch.uint8, device="cuda")
    y1 = torch.empty(n, dtype=torch.uint8, device="cuda") if two_outputs else None
    ms = timer.median_ms(lambda: fp8.fp8bs_hbm_rate(x, y0, y1), reps=15)
    return n * (4 if two_outputs else 3) / (ms / 1e3) / 1e9


def _config_ops(torch, fp8, cfg_name, inputs):
    """(name, kind, fn, units) for every kernel a configuration runs, on
    device tensors of its seeded inputs (units: bytes or flops)."""
    c = inputs.CONFIGS[cfg_name]
    dev = {n: torch.from_numpy(inputs.tensor(cfg_name, n).view("int16")).view(torch.bfloat16)
           .to("cuda") for n in c.tensors}
    ops = []
    done = set()
    for g in c.gemms:
        a, b = dev[g.a], dev[g.b]
        if g.kind in ("fprop", "dgrad"):
            M, L = a.shape
            q, s = fp8.fp8_quantize_rowtile(a)
            if ("row", g.a) not in done:
                ops.append((f"{g.a}.rowtile", "quant_rowtile",
                            lambda a=a, q=q, s=s: fp8.fp8_quantize_rowtile(a, q, s),
                            M * L * 3 + M * (L // 128) * 4))
                done.add(("row", g.a))
            N, K = b.shape
            wq, wqt, ws = fp8.fp8_quantize_block(b, with_transpose=(g.kind == "dgrad"))
            if ("block", g.b, g.kind) not in done:
                ops.append((f"{g.b}.block", "quant_block",
                            lambda b=b, wq=wq, wqt=wqt, ws=ws: fp8.fp8_quantize_block(
                                b, wq, wqt, ws, with_transpose=wqt is not None),
                            N * K * (4 if g.kind == "dgrad" else 3) + (N // 128) * (K // 128) * 4))
                done.add(("block", g.b, g.kind))
            out = torch.float32 if g.out == "f32" else torch.bfloat16
            if g.kind == "fprop":
                y = torch.empty(g.M, g.N, dtype=out, device="cuda")
                fn = lambda q=q, s=s, wq=wq, ws=ws, y=y, o=out: fp8.fp8_gemm_fprop(q, s, wq, ws, o, y)
            else:
                y = torch.empty(g.M, g.K, dtype=out, device="cuda")
                fn = lambda q=q, s=s, wqt=wqt, ws=ws, y=y, o=out: fp8.fp8_gemm_dgrad(q, s, wqt, ws, o, y)
            ops.append((g.name, "gemm_" + g.kind, fn, g.flops))
        else:
            tq = {}
            for nm, x in ((g.a, a), (g.b, b)):
                M, C = x.shape
                qt, st = fp8.fp8_quantize_transposed(x)
                tq[nm] = (qt, st)
                ops.append((f"{nm}.transposed", "quant_transposed",
                            lambda x=x, qt=qt, st=st: fp8.fp8_quantize_transposed(x, qt, st),
                            M * C * 3 + C * (M // 128) * 4))
            dyt, dyts = tq[g.a]
            xt, xts = tq[g.b]
            dw = torch.empty(g.N, g.K, dtype=torch.float32, device="cuda")
            nb = fp8.fp8_gemm_wgrad_workspace_bytes(g.M, g.N, g.K)
            wsp = torch.empty(nb, dtype=torch.uint8, device="cuda") if nb else None
            ops.append((g.name, "gemm_wgrad",
                        lambda dyt=dyt, dyts=dyts, xt=xt, xts=xts, dw=dw, wsp=wsp:
                        fp8.fp8_gemm_wgrad(dyt, dyts, xt, xts, dw, wsp), g.flops))
    return ops


def _oracle_config_seconds(cfg_name, inputs, cores):
    """Wall seconds of the oracle computing a configuration in full (its
    quantizations and every GEMM), on `cores` threads."""
    import oracle
    c = inputs.CONFIGS[cfg_name]
    host = {n: inputs.tensor(cfg_name, n) for n in c.tensors}
    t0 = time.perf_counter()
    for g in c.gemms:
        a, b = host[g.a], host[g.b]
        if g.kind in ("fprop", "dgrad"):
            q, s = oracle.quantize_rowtile(a, threads=cores)
            wq, wqt, ws = oracle.quantize_block(b, with_transpose=(g.kind == "dgrad"), threads=cores)
            if g.kind == "fprop":
                oracle.gemm_fprop(q, s, wq, ws, threads=cores)
            else:
                oracle.gemm_dgrad(q, s, wqt, ws, threads=cores)
        else:
            dq, ds = oracle.quantize_transposed(a, threads=cores)
            xq, xs = oracle.quantize_transposed(b, threads=cores)
            oracle.gemm_wgrad(dq, ds, xq, xs, threads=cores)
    return time.perf_counter() - t0


def config_measurements(torch, fp8, inputs, timer, ceilings, with_oracle: bool):
    """Configurations 1-4 (Tiny, QKV, MLP pair, down backward), each kernel
    timed alone with the cache flushed before every iteration (median of 25),
    and the oracle's time for the whole configuration on all host cores."""
    cores = len(os.sched_getaffinity(0))
    out = {}
    for cfg_name in ("tiny", "qkv", "mlp", "down_bwd"):
        ops = _config_ops(torch, fp8, cfg_name, inputs)
        torch.cuda.synchronize()
        kern = {}
        gemm_ms = quant_ms = 0.0
        flops = qbytes = 0
        for name, kind, fn, units in ops:
            ms = timer.median_ms(fn)
            e = {"kind": kind, "us": round(ms * 1e3, 2)}
            if kind.startswith("gemm"):
                tf = units / (ms / 1e3) / 1e12
                e.update(tflops=round(tf, 1), frac_f16_peak=round(tf / PEAK_F16_TFLOPS, 4),
                         pct_fp8_peak=round(100 * tf / PEAK_FP8_TFLOPS, 2))
                gemm_ms += ms
                flops += units
            else:
                gbs = units / (ms / 1e3) / 1e9
                ceil = ceilings["write1"]
                e.update(gbs=round(gbs, 1), frac_hbm_peak=round(gbs / PEAK_HBM_GBS, 4),
                         frac_of_probe=round(gbs / ceil, 4))
                quant_ms += ms
                qbytes += units
            kern[name] = e
        line = {"kernels": kern,
                "gemm_tflops": round(flops / (gemm_ms / 1e3) / 1e12, 1),
                "gemm_frac_f16_peak": round(flops / (gemm_ms / 1e3) / 1e12 / PEAK_F16_TFLOPS, 4),
                "quant_gbs": round(qbytes / (quant_ms / 1e3) / 1e9, 1),
                "quant_frac_hbm_peak": round(qbytes / (quant_ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4)}
        if cfg_name == "tiny":
            line["note"] = "67 MFLOP and 0.4 MB per call: launch-bound, exempt from the roofline gates"
        if with_oracle:
            secs = _oracle_config_seconds(cfg_name, inputs, cores)
            gpu_s = (gemm_ms + quant_ms) / 1e3
            line["oracle"] = {"seconds": round(secs, 2), "cores": cores, "cpu": cpu_model(),
                              "gflops": round(flops / secs / 1e9, 2),
                              "gpu_speedup": round(secs / gpu_s, 1)}
        out[cfg_name] = line
        del ops
        torch.cuda.empty_cache()
    return out


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


def bf16_comparison(torch, fp8, cfg, fp8_ms_per_layer, mfma8_ms_per_layer=None, reps=5):
    """The 12 GEMMs of one layer in TN form on BF16 operands: this library's
    BF16 kernel and torch's BF16 matmul (the vendor BLAS), against the FP8
    GEMMs' device time per layer in the step (and, when given, the FP8-MFMA
    GEMMs' in their step)."""
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
    res = {
        "workload": "one layer's 12 GEMMs of the linear set (16384 tokens) in TN form on BF16 "
                    "operands, FP32 accumulation, BF16 out (FP32 for wgrad)",
        "bf16_ms_per_layer": round(own, 3), "bf16_tflops": round(flops / own / 1e9, 1),
        "fp8_ms_per_layer": round(fp8_ms_per_layer, 3),
        "fp8_tflops": round(flops / fp8_ms_per_layer / 1e9, 1),
        "fp8_speedup_vs_own_bf16": round(own / fp8_ms_per_layer, 3),
        "torch_bf16_ms_per_layer": round(blas, 3), "torch_bf16_tflops": round(flops / blas / 1e9, 1),
        "fp8_speedup_vs_best_bf16": round(min(own, blas) / fp8_ms_per_layer, 3)}
    if mfma8_ms_per_layer:
        res["fp8_mfma8_ms_per_layer"] = round(mfma8_ms_per_layer, 3)
        res["fp8_mfma8_tflops"] = round(flops / mfma8_ms_per_layer / 1e9, 1)
        res["fp8_mfma8_speedup_vs_best_bf16"] = round(min(own, blas) / mfma8_ms_per_layer, 3)
    return {"f2_bf16_gemm": res}


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


def swiglu_quantization(torch, fp8, reps=5):
    """The MLP's SwiGLU at 16,384 tokens (gate/up [16384, 12288] -> H [16384,
    6144]) followed by both quantizations of H that the down projection needs:
    torch's BF16 SwiGLU then fp8_quantize_dual, against
    fp8_swiglu_quantize_dual (H never stored, or stored as well)."""
    T, F = 16384, 6144
    gen = torch.Generator(device="cuda").manual_seed(3)
    gu = torch.randn(T, 2 * F, device="cuda", generator=gen).bfloat16()
    q = torch.empty(T, F, device="cuda", dtype=torch.uint8)
    s = torch.empty(T, F // 128, device="cuda", dtype=torch.float32)
    qt = torch.empty(F, T, device="cuda", dtype=torch.uint8)
    st = torch.empty(F, T // 128, device="cuda", dtype=torch.float32)
    h = torch.empty(T, F, device="cuda", dtype=torch.bfloat16)

    def separate():
        torch.mul(torch.nn.functional.silu(gu[:, :F]), gu[:, F:], out=h)
        fp8.fp8_quantize_dual(h, q, s, qt, st)

    sep = _time_events(torch, separate, reps)
    fused = _time_events(torch, lambda: fp8.fp8_swiglu_quantize_dual(gu, q, s, qt, st), reps)
    fused_h = _time_events(torch, lambda: fp8.fp8_swiglu_quantize_dual(gu, q, s, qt, st, h=h),
                           reps)
    # read gate and up (4 B per element of H), write both code sets (2 B) and both
    # scale sets (2 x 4 B per 128 elements)
    algo = T * F * (4 + 2 + 8 / 128)
    rate = algo / (fused * 1e-3) / 1e9
    del q, s, qt, st, h
    # backward: dH [T, F] and gate/up -> the gate/up gradient [T, 2F], both quantizations
    dh = (torch.randn(T, F, device="cuda", generator=gen) * 1e-3).bfloat16()
    q = torch.empty(T, 2 * F, device="cuda", dtype=torch.uint8)
    s = torch.empty(T, 2 * F // 128, device="cuda", dtype=torch.float32)
    qt = torch.empty(2 * F, T, device="cuda", dtype=torch.uint8)
    st = torch.empty(2 * F, T // 128, device="cuda", dtype=torch.float32)
    dgu = torch.empty(T, 2 * F, device="cuda", dtype=torch.bfloat16)

    def separate_bwd():
        g, u = gu[:, :F].float(), gu[:, F:].float()
        sg = torch.sigmoid(g)
        d = dh.float()
        dgu[:, :F] = d * u * (sg * (1 + g * (1 - sg)))
        dgu[:, F:] = d * (g * sg)
        fp8.fp8_quantize_dual(dgu, q, s, qt, st)

    sep_b = _time_events(torch, separate_bwd, reps)
    fused_b = _time_events(torch, lambda: fp8.fp8_swiglu_backward_quantize_dual(
        dh, gu, q, s, qt, st), reps)
    # read dH, gate and up once (3 B per element of the gradient), write both code
    # sets and scale sets (2 + 8/128 B)
    algo_b = T * 2 * F * (3 + 2 + 8 / 128)
    rate_b = algo_b / (fused_b * 1e-3) / 1e9
    del gu, dh, q, s, qt, st, dgu
    torch.cuda.empty_cache()
    return {"f3_swiglu_quantize_on_produce": {
        "workload": "the MLP's SwiGLU at 16384 tokens (gate/up [16384, 12288] bf16 -> H "
                    "[16384, 6144]) with H's row-tile and token-axis quantization",
        "separate_ms": round(sep, 4), "fused_ms": round(fused, 4),
        "fused_with_bf16_h_ms": round(fused_h, 4), "fused_speedup": round(sep / fused, 3),
        "fused_algorithmic_bytes": int(algo), "fused_gbs": round(rate, 1),
        "fused_frac_hbm": round(rate / PEAK_HBM_GBS, 4),
        "backward": {
            "workload": "its backward: dH [16384, 6144] and gate/up -> the gate/up gradient "
                        "[16384, 12288] with both of its quantizations",
            "separate_ms": round(sep_b, 4), "fused_ms": round(fused_b, 4),
            "fused_speedup": round(sep_b / fused_b, 3), "fused_algorithmic_bytes": int(algo_b),
            "fused_gbs": round(rate_b, 1), "fused_frac_hbm": round(rate_b / PEAK_HBM_GBS, 4)}}}


def rmsnorm_quantization(torch, fp8, reps=5):
    """The RMSNorm in front of the QKV and MLP input projections at 16,384
    tokens (X [16384, 2048]) with both quantizations of its output: torch's
    BF16 rms_norm then fp8_quantize_dual, against fp8_rmsnorm_quantize_dual."""
    T, C, eps = 16384, 2048, 1e-6
    gen = torch.Generator(device="cuda").manual_seed(4)
    x = torch.randn(T, C, device="cuda", generator=gen).bfloat16()
    gamma = (torch.rand(C, device="cuda", generator=gen) + 0.5).bfloat16()
    q = torch.empty(T, C, device="cuda", dtype=torch.uint8)
    s = torch.empty(T, C // 128, device="cuda", dtype=torch.float32)
    qt = torch.empty(C, T, device="cuda", dtype=torch.uint8)
    st = torch.empty(C, T // 128, device="cuda", dtype=torch.float32)
    r = torch.empty(T, device="cuda", dtype=torch.float32)

    def separate():
        y = torch.nn.functional.rms_norm(x, (C,), weight=gamma, eps=eps)
        fp8.fp8_quantize_dual(y, q, s, qt, st)

    sep = _time_events(torch, separate, reps)
    fused = _time_events(torch, lambda: fp8.fp8_rmsnorm_quantize_dual(
        x, gamma, eps, q, s, qt, st, r), reps)
    # read x once (2 B per element), write both code sets and scale sets (2 + 8/128 B)
    # and r (4 B per row); the fused form reads x twice (r first, then the tiles)
    algo = T * C * (2 + 2 + 8 / 128) + 4 * T
    rate = algo / (fused * 1e-3) / 1e9
    del x, gamma, q, s, qt, st, r
    torch.cuda.empty_cache()
    return {"f3_rmsnorm_quantize_on_produce": {
        "workload": "the RMSNorm of the QKV / MLP input at 16384 tokens (X [16384, 2048] bf16) "
                    "with its output's row-tile and token-axis quantization",
        "separate_ms": round(sep, 4), "fused_ms": round(fused, 4),
        "fused_speedup": round(sep / fused, 3), "fused_algorithmic_bytes": int(algo),
        "fused_gbs": round(rate, 1), "fused_frac_hbm": round(rate / PEAK_HBM_GBS, 4)}}


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

    def fp8_mfma8_layer():
        for m, x, dy in zip(mods, xs, dys):
            x.grad = None
            m.weight.grad = None
            m.mfma8 = True
            m(x).backward(dy)
            m.mfma8 = False

    def bf16_layer():
        for w, x, dy in zip(bf_w, xs, dys):
            x.grad = None
            w.grad = None
            torch.nn.functional.linear(x, w).backward(dy)

    flops = sum(3 * 2 * T * d_in * d_out for _, d_in, d_out in LAYER_LINEARS)
    ms8 = _time_events(torch, fp8_layer, reps)
    ms8m = _time_events(torch, fp8_mfma8_layer, reps)
    ms16 = _time_events(torch, bf16_layer, reps)
    return {"f4_fp8_linear_layer": {
        "workload": "one decoder layer's QKV, O, gate/up and down linears at 16384 tokens, "
                    "forward + backward (dual quantization of X and dY, block quantization of "
                    "W, fprop, dgrad, wgrad)",
        "fp8_ms": round(ms8, 3), "fp8_tflops": round(flops / ms8 / 1e9, 1),
        "torch_bf16_ms": round(ms16, 3), "torch_bf16_tflops": round(flops / ms16 / 1e9, 1),
        "fp8_speedup_vs_torch_bf16": round(ms16 / ms8, 3),
        "fp8_mfma8_ms": round(ms8m, 3), "fp8_mfma8_tflops": round(flops / ms8m / 1e9, 1),
        "fp8_mfma8_speedup_vs_torch_bf16": round(ms16 / ms8m, 3)}}


def fp8_mlp_comparison(torch, fp8, reps=5):
    """The decoder's MLP at 16,384 tokens (hidden 2048, FFN 6144), forward +
    backward: Fp8SwiGLUMLP (both projections on the FP8 path, the SwiGLU and
    its backward quantizing on produce) against torch's BF16 linear layers and
    SwiGLU under autograd."""
    T, d, F = 16384, 2048, 6144
    gen = torch.Generator(device="cuda").manual_seed(5)
    mlp = fp8.Fp8SwiGLUMLP(d, F, device="cuda")
    wgu = mlp.weight_gate_up.detach().clone().requires_grad_(True)
    wd = mlp.weight_down.detach().clone().requires_grad_(True)
    x = torch.randn(T, d, device="cuda", generator=gen).bfloat16().requires_grad_(True)
    dy = (torch.randn(T, d, device="cuda", generator=gen) * 1e-3).bfloat16()

    def fp8_mlp(mfma8):
        def run():
            x.grad = None
            mlp.weight_gate_up.grad = mlp.weight_down.grad = None
            mlp.mfma8 = mfma8
            mlp(x).backward(dy)
            mlp.mfma8 = False
        return run

    def bf16_mlp():
        x.grad = wgu.grad = wd.grad = None
        gu = torch.nn.functional.linear(x, wgu)
        h = torch.nn.functional.silu(gu[:, :F]) * gu[:, F:]
        torch.nn.functional.linear(h, wd).backward(dy)

    flops = 3 * 2 * T * d * (3 * F)
    ms8 = _time_events(torch, fp8_mlp(False), reps)
    ms8m = _time_events(torch, fp8_mlp(True), reps)
    ms16 = _time_events(torch, bf16_mlp, reps)
    del mlp, wgu, wd, x, dy
    torch.cuda.empty_cache()
    return {"f4_fp8_swiglu_mlp": {
        "workload": "the decoder's MLP at 16384 tokens (hidden 2048, FFN 6144: gate/up "
                    "projection, SwiGLU, down projection), forward + backward",
        "fp8_ms": round(ms8, 3), "fp8_tflops": round(flops / ms8 / 1e9, 1),
        "torch_bf16_ms": round(ms16, 3), "torch_bf16_tflops": round(flops / ms16 / 1e9, 1),
        "fp8_speedup_vs_torch_bf16": round(ms16 / ms8, 3),
        "fp8_mfma8_ms": round(ms8m, 3), "fp8_mfma8_tflops": round(flops / ms8m / 1e9, 1),
        "fp8_mfma8_speedup_vs_torch_bf16": round(ms16 / ms8m, 3)}}


def mfma8_step(torch, plan, stream, fused, args, exact_value, layer0_fn):
    """The same step with the GEMMs whose block sums come from the FP8 matrix
    core (fp8_gemm_*_mfma8): their limited accumulation precision inside each
    128-wide block is the pages' FP8 tensor-core arithmetic, not the exact
    block sums of the headline path, so the headline value stays the exact
    path's and this is reported beside it."""
    ops8 = plan.ops(stream.cuda_stream, fused, mfma8=True)
    run_step(ops8)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(ops8) + 1)]
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        run_step(ops8, ev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kinds = {}
    for s in range(args.steps):
        accumulate_kinds(kinds, ops8, ev[s])
    breakdown = kind_summary(kinds, args.steps)
    for kind, v in breakdown.items():
        if kind.startswith("gemm"):
            v["frac_fp8_peak"] = round(v["rate"] / PEAK_FP8_TFLOPS, 4)
    gemm_flops = sum(g.flops for g in plan.cfg.gemms) * plan.cfg.layers
    value = gemm_flops / (wall / args.steps) / 1e12
    dom = next(k for k in breakdown if k.startswith("gemm"))
    roofline = {"kernel": dom, "bound": "mfma", "achieved": breakdown[dom]["rate"],
                "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": round(breakdown[dom]["rate"] / PEAK_FP8_TFLOPS, 4)}
    out = {"what": "the headline step with fp8_gemm_fprop/dgrad/wgrad_mfma8: each 128-wide "
                   "block's sum of products formed by the FP8 MFMA (v_mfma_f32_16x16x128_f8f6f4, "
                   "fixed-point window of ~14 bits per 8 products), folded into FP32 as in the "
                   "exact path; it does not meet the exact path's relF 1e-5 gate",
           "value": round(value, 2), "unit": "TFLOP/s", "ms_per_step": round(wall / args.steps * 1e3, 3),
           "pct_fp8_peak": round(100 * value / PEAK_FP8_TFLOPS, 2),
           "speedup_vs_exact_step": round(value / exact_value, 3),
           "roofline": roofline, "kernels": breakdown}
    layer0 = layer0_fn(torch, plan, ops8) if layer0_fn else None
    return out, layer0


def main():
    args = parse()
    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof)
        return
    if args.record_traffic:
        record_traffic(*args.record_traffic,
                       out_path=None if args.traffic_print_only else TRAFFIC_FILE)
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
    if args.producers:
        if args.copy_calibration_mib:
            n = args.copy_calibration_mib << 20
            src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
            torch.empty_like(src).copy_(src)
            torch.cuda.synchronize()
            del src
        print(json.dumps({**rmsnorm_quantization(torch, fp8), **swiglu_quantization(torch, fp8)}),
              flush=True)
        return
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
    with SclkSampler() as sclk:
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
    # the quantizers' own ceiling: the library's streaming probe moving the
    # same bytes per element (2 read, 1 or 2 written) over the largest tensor
    # of the step, cache flushed
    timer = Timer(torch)
    n_big = max(x.numel() for x in plan.act.values())
    ceilings = {"write1": hbm_ceiling(torch, fp8, timer, n_big, False),
                "write2": hbm_ceiling(torch, fp8, timer, n_big, True)}
    for kind, v in breakdown.items():
        if not kind.startswith("gemm"):
            c = ceilings["write2" if kind == "quant_dual" else "write1"]
            v["frac_of_probe"] = round(v["rate"] / c, 4)
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
        for kind, v in result["kernels_outside_step"].items():
            v["frac_of_probe"] = round(v["rate"] / ceilings["write1"], 4)
    result["hbm_probe"] = {
        "what": "fp8bs_hbm_rate: 2 bytes read and 1 (write1) or 2 (write2) bytes written per "
                "element in 16-byte accesses, %d elements, last-level cache flushed, median" % n_big,
        "write1_gbs": round(ceilings["write1"], 1), "write2_gbs": round(ceilings["write2"], 1),
        "write1_frac_hbm_peak": round(ceilings["write1"] / PEAK_HBM_GBS, 4),
        "write2_frac_hbm_peak": round(ceilings["write2"] / PEAK_HBM_GBS, 4)}
    result["sclk"] = sclk.summary()
    if roofline.get("peak_at_clock"):
        # the clock the MFMA-only kernel implies: 2.5 PFLOP/s is the spec at 2.4 GHz
        result["sclk_from_mfma_rate_mhz"] = round(roofline["peak_at_clock"] / PEAK_F16_TFLOPS * 2400)
    if not args.no_configs:
        result["configs"] = config_measurements(torch, fp8, inputs, timer, ceilings,
                                                not args.no_cpu_baseline)
    # the GPU's own layer-0 results, compared with the oracle's in the cpu_baseline leg
    layer0 = None if args.no_cpu_baseline else gpu_layer0(torch, plan, ops)
    layer0_8 = None
    mfma8_gemm_ms = None
    if not args.no_mfma8:
        step8, layer0_8 = mfma8_step(torch, plan, stream, fused, args, value,
                                     None if args.no_cpu_baseline else gpu_layer0)
        result["fp8_mfma_step"] = step8
        mfma8_gemm_ms = sum(v["ms_per_step"] for k, v in step8["kernels"].items()
                            if k.startswith("gemm")) / plan.cfg.layers
    del timer
    if not args.no_next_rows:
        cfg_obj, cfg_layers = plan.cfg, plan.cfg.layers
        del plan, ops, events
        torch.cuda.empty_cache()
        fp8_gemm_ms = sum(v["ms_per_step"] for k, v in breakdown.items()
                          if k.startswith("gemm")) / cfg_layers
        result["next_rows"] = {**bf16_comparison(torch, fp8, cfg_obj, fp8_gemm_ms, mfma8_gemm_ms),
                               **dgrad_epilogue_quantization(torch, fp8, cfg_obj),
                               **swiglu_quantization(torch, fp8),
                               **rmsnorm_quantization(torch, fp8),
                               **fp8_linear_comparison(torch, fp8),
                               **fp8_mlp_comparison(torch, fp8)}
    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["parity_sample"], parity8 = cpu_baseline(
            args.cpu_fraction, layer0, layer0_8)
        if parity8 is not None:
            result["fp8_mfma_step"]["parity_sample"] = parity8
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
