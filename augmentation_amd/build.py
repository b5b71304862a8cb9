"""Build libfn.so (HIP, gfx950) in place with hipcc.

Flags:
  -ffp-contract=off     the sampler's fp32 operations stay separately
                        rounded; the pixel pass writes its fma explicitly.
  -fhip-fp32-correctly-rounded-divide-sqrt
                        fp32 '/' and sqrtf are IEEE correctly rounded (the
                        sampler's decisions depend on it).
  -Xclang -target-feature -Xclang -packed-fp32-ops
                        no packed fp32 instructions are generated.
  -fvisibility=hidden   only the extern "C" entry points are exported.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
SOURCES = [os.path.join(HERE, "csrc", "fn_api.hip")]
HEADERS = [os.path.join(HERE, "csrc", h) for h in ("fn_device.hpp", "fn_kernels.hpp",
                                                   "exp2_table.inc")] + [
    os.path.join(ROOT, "include", "fn.h")]
LIB_PATH = os.path.join(HERE, "libfn.so")
# the instrumented build: the tiles kernel records per-tile clock stamps
# (fn_test_timeline); a measurement tool, never the product library
TIMELINE_LIB_PATH = os.path.join(HERE, "libfn_timeline.so")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", f"-I{os.path.join(ROOT, 'include')}",
]


CPU_SOURCES = [os.path.join(HERE, "cpu", "fn_cpu.cpp")]
CPU_LIB_PATH = os.path.join(HERE, "libfn_cpu.so")
# the page's host method: SSE4.1 (with its SSSE3 byte shuffle) + F16C;
# -ffp-contract=off keeps its product and difference separately rounded
CPU_FLAGS = ["-std=c++17", "-O3", "-msse4.1", "-mf16c", "-ffp-contract=off", "-fPIC", "-shared",
             "-fvisibility=hidden", "-Wall", "-Wextra", f"-I{os.path.join(ROOT, 'include')}"]


def build_cpu(verbose: bool = False) -> str:
    """Compile the host SSE4.1/F16C library (always recompiles)."""
    tmp = CPU_LIB_PATH + ".tmp"
    cmd = ["g++", *CPU_FLAGS, *CPU_SOURCES, "-o", tmp, "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("g++ failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, CPU_LIB_PATH)
    return CPU_LIB_PATH


def build(verbose: bool = False, timeline: bool = False) -> str:
    """Compile the library (always recompiles) and return its path;
    timeline: the instrumented build libfn_timeline.so instead."""
    path = TIMELINE_LIB_PATH if timeline else LIB_PATH
    tmp = path + ".tmp"
    cmd = [HIPCC, *FLAGS, *(["-DFN_TIMELINE=1"] if timeline else []), *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"  # the host pass does not know the target feature: harmless
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln and ln.strip()]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, path)
    return path


if __name__ == "__main__":
    print(build(verbose=True))
    print(build(verbose=True, timeline=True))
    print(build_cpu(verbose=True))
