"""Host-side model of the hardware range check on the GEMM tiles' LDS-DMA loads: compiles
tests/dma_range_model.cpp (which uses the kernels' own offset functions from
csrc/dma_offsets.hpp) with the host compiler and runs it over ragged shapes and every tile
plan. No GPU involved."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "blockwise_fp8_gemm_x128_amd", "csrc")


def test_dma_offsets_stay_in_range(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "dma_range_model")
    # built with AddressSanitizer and UndefinedBehaviorSanitizer: the model's own arithmetic
    # (offsets in 32 bits, products of tile sizes and pitches) must not overflow
    subprocess.check_call([cxx, "-std=c++17", "-O1", "-Wall", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined", "-I" + CSRC,
                           os.path.join(HERE, "dma_range_model.cpp"), "-o", exe])
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and res.stdout.strip().endswith("ok"), res.stdout + res.stderr
