"""Build libw4a8.so (the HIP kernels + C ABI) in-tree with hipcc for gfx950.

Usage: ``python -m bit_codebook_quantized_amd.build`` (or ``__graft_entry__.build()``).
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libw4a8.so")
SOURCES = ["w4a8_api.cpp", "rotate_quant.hip", "decode.hip", "gemv.hip", "gemm.hip", "quantize.hip", "regrid.hip", "grad.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # the epilogue's separately rounded multiply and add must not be fused
    "-ffp-contract=off",
    # keep the compiler from emitting packed fp32 math (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


# Kernels whose main loop loads into registers with inline asm (the compiler sees those
# registers as written at once): a spill of them would store stale data, so they must not
# use scratch memory at all.
NO_SCRATCH = {"gemm.hip": "gemm_kernel"}


def check_no_scratch(hipcc: str) -> None:
    """Compile each NO_SCRATCH source to gfx950 assembly and fail if a listed kernel
    uses private (scratch) memory."""
    import re
    import tempfile
    for src, kernel in NO_SCRATCH.items():
        with tempfile.TemporaryDirectory() as td:
            asm = os.path.join(td, "k.s")
            cmd = [hipcc, *[f for f in HIPCC_FLAGS if f not in ("-fPIC", "-shared")], "-S", "--cuda-device-only",
                   "-o", asm, os.path.join(CSRC, src)]
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError(f"hipcc -S {src} failed:\n{res.stderr}")
            text = open(asm).read()
        found = 0
        for block in text.split("  - .agpr_count:")[1:]:
            name = re.search(r"\.name:\s+(\S+)", block)
            priv = re.search(r"\.private_segment_fixed_size:\s+(\d+)", block)
            if name and kernel in name.group(1):
                found += 1
                if priv is None or int(priv.group(1)) != 0:
                    raise RuntimeError(f"{name.group(1)} uses scratch memory; its asm-loaded registers must not spill")
        if not found:
            raise RuntimeError(f"no {kernel} found in the assembly of {src}")


def build(verbose: bool = False) -> str:
    """Compile every source into libw4a8.so next to this file; returns its path."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-o", tmp, *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"   # host pass: harmless unknown-feature warning
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    check_no_scratch(hipcc)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
