"""Builds libpuro.so (all HIP kernels + the C ABI) for gfx950 with hipcc, in-tree.

Usage: ``python -m blockwise_fp8_gemm_x128_amd.build`` (also called by ``__graft_entry__.build``).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO_DIR, "include")
LIB_PATH = os.path.join(PKG_DIR, "libpuro.so")
SOURCES = ["abi.hip", "quant.hip", "gemm.hip", "optim.hip", "debug.hip"]
# The matrix-core microbenchmark that bench.py --ceiling runs; a library of its own, outside the
# GEMM path.
PROBE_PATH = os.path.join(PKG_DIR, "libpuro_probe.so")
PROBE_SOURCES = ["ceiling.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # Packed FP32 ALU ops stay off: every fp32 operation is a plain single-lane instruction.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Let MFMA results land in VGPRs, where the fp32 promotion reads them directly.
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def _hipcc(sources, out: str, verbose: bool) -> str:
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-I" + INCLUDE, "-I" + CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; that is harmless.
    noise = [l for l in res.stderr.splitlines() if l.strip() and "packed-fp32-ops" not in l]
    if res.returncode != 0:
        sys.stderr.write(res.stderr)
        raise RuntimeError("hipcc failed building " + os.path.basename(out))
    if noise and verbose:
        sys.stderr.write("\n".join(noise) + "\n")
    os.replace(tmp, out)
    return out


def build(verbose: bool = True) -> str:
    _hipcc(PROBE_SOURCES, PROBE_PATH, verbose)
    return _hipcc(SOURCES, LIB_PATH, verbose)


if __name__ == "__main__":
    print(build())
