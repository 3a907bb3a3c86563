"""Build the HIP library ``libkdaconv.so`` in-tree for gfx950.

All device code is compiled for gfx950 only, with packed-fp32 instruction
selection disabled.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkdaconv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wshadow", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs: the state pass post-processes
    # its MFMA results with vector ALU ops every chunk, and AGPR results would
    # have to be copied over first
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-o", tmp] + sources()
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is harmless
    err = "\n".join(line for line in res.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if res.returncode != 0:
        sys.stderr.write(err)
        raise RuntimeError("hipcc failed building libkdaconv.so")
    if verbose and err.strip():
        sys.stderr.write(err + "\n")
    os.replace(tmp, LIB)
    return LIB


def kernel_resources() -> dict:
    """Per-kernel register and scratch use as the compiler reports it.

    Compiles the device code only (nothing is written in-tree) and returns
    {mangled kernel name: {"VGPRs": n, "SGPRs": n, "ScratchSize": bytes/lane,
    "Occupancy": waves/SIMD}}.
    """
    out = {}
    for src in sources():
        cmd = ([HIPCC] + [f for f in FLAGS if f not in ("-shared", "-fPIC")] +
               ["--cuda-device-only", "-c", "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage", src])
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stderr)
            raise RuntimeError("hipcc failed on " + src)
        name = None
        for line in res.stderr.splitlines():
            if "remark:" not in line:
                continue
            body = line.split("remark:", 1)[1].split("[-Rpass")[0].strip()
            key, _, val = body.partition(":")
            val = val.strip()
            if key == "Function Name":
                name = val
                out[name] = {}
            elif name is not None and key in ("VGPRs", "TotalSGPRs", "ScratchSize [bytes/lane]",
                                              "Occupancy [waves/SIMD]"):
                out[name][key.split(" ")[0].replace("Total", "")] = int(val)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
