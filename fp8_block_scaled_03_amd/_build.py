"""Build libfp8bs.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfp8bs.so")
SOURCES = ["quantize.hip", "gemm.hip", "gemm_mfma8.hip", "gemm_bf16.hip", "noalloc.hip", "capi.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # scalar FP32 only: the compiler may not form packed FP32 instructions (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
    # every symbol resolved at link time: a kernel whose host launch stub the
    # compiler failed to emit is a link error here, not a load error later
    "-Wl,-z,defs",
]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the same
# sources (the argument checks of the C ABI run under them; device code is
# built as usual).  Loaded only by the C-ABI CPU tests, with clang's ASan
# runtime preloaded.
ASAN_LIB = os.path.join(PKG, "libfp8bs_asan.so")
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-shared-libsan",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    out = ASAN_LIB if sanitize else LIB
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *(SANITIZE_FLAGS if sanitize else []), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
