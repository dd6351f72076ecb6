"""Build the LeapQuant HIP library (gfx950) in-tree with hipcc.

    python -m linear_attention_recurrent_kda_amd.build

writes linear_attention_recurrent_kda_amd/_lib/libleapquant.so. hipcc
cross-compiles for gfx950, so the build needs no GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libleapquant.so")
SOURCES = ["abi.hip", "decode_step.hip", "window_close.hip", "fp32_baseline.hip", "prefill.hip", "snapshot.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU instructions stay off: scalar fp32 FMA only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the window close keeps its fp32
    # state in registers that the vector ALU reads directly
    "-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm toolchain required to build the HIP library)")
    return exe


def build(verbose: bool = False) -> str:
    """Compile every HIP source into one shared library; returns its path."""
    os.makedirs(LIBDIR, exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    t0 = time.time()
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    # every kernel launch stub must resolve: a host pass that silently drops a
    # kernel instantiation leaves an undefined symbol that only dlopen reports
    undefined = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True).stdout
    stubs = [ln for ln in undefined.splitlines() if "__device_stub__" in ln]
    if stubs:
        raise RuntimeError("kernel launch stubs missing from the host pass:\n" + "\n".join(stubs))
    os.replace(tmp, LIB)
    if verbose:
        if res.stderr.strip():
            print(res.stderr, flush=True)
        print(f"built {LIB} in {time.time() - t0:.1f}s", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
