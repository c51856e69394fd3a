"""Host-side checks of the C ABI (no GPU needed): libpuro.so loads, exports every function
declared in include/puro.h, and its validation rejects bad arguments before touching the
device. None of these calls reaches a kernel launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "puro.h")


@pytest.fixture(scope="module")
def L():
    from blockwise_fp8_gemm_x128_amd import _lib
    from blockwise_fp8_gemm_x128_amd.build import LIB_PATH, build
    if not os.path.exists(LIB_PATH):
        build(verbose=False)
    return _lib.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(puro_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_six_entry_points():
    names = declared_functions()
    for n in ("puro_quant_act_1x128", "puro_quant_w_128x128", "puro_quant_transpose",
              "puro_fp8_gemm_fwd", "puro_fp8_gemm_dgrad", "puro_fp8_gemm_wgrad"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    from blockwise_fp8_gemm_x128_amd._lib import SIGNATURES
    for name in declared_functions():
        assert hasattr(L, name), name
        assert name in SIGNATURES, name


def test_version_and_status_strings(L):
    assert L.puro_abi_version() == 1
    assert L.puro_status_string(0) == b"PURO_OK"
    for code in range(1, 6):
        assert L.puro_status_string(code).startswith(b"PURO_ERR_")
    assert L.puro_status_string(99) == b"unknown puro_status"


FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation first
MIS = 0x10001   # misaligned


POW2 = ["", "_pow2"]


def test_every_entry_point_has_a_pow2_twin():
    names = set(declared_functions())
    bases = [n for n in names if n.startswith(("puro_quant_", "puro_fp8_gemm_"))
             and not n.endswith("_pow2")]
    assert len(bases) == 8
    for n in bases:
        assert n + "_pow2" in names, n


@pytest.mark.parametrize("fn", ["puro_quant_act_1x128", "puro_quant_w_128x128",
                                "puro_quant_transpose"])
@pytest.mark.parametrize("sfx", POW2)
def test_quant_validation(L, fn, sfx):
    fn = fn + sfx
    f = getattr(L, fn)
    assert f(FAKE, 100, 128, FAKE, FAKE, None) == 2          # ragged rows
    assert f(FAKE, 128, 200, FAKE, FAKE, None) == 2          # ragged cols
    assert f(FAKE, -128, 128, FAKE, FAKE, None) == 2         # negative
    assert f(FAKE, 1 << 25, 128, FAKE, FAKE, None) == 2      # beyond the size limit
    assert f(None, 128, 128, FAKE, FAKE, None) == 1          # NULL input
    assert f(FAKE, 128, 128, None, FAKE, None) == 1          # NULL payload
    assert f(FAKE, 128, 128, FAKE, None, None) == 1          # NULL scales
    assert f(MIS, 128, 128, FAKE, FAKE, None) == 3           # misaligned
    assert f(FAKE, 128, 128, FAKE, MIS, None) == 3
    assert f(None, 0, 128, None, None, None) == 0            # empty: nothing to do
    assert f(None, 256, 0, None, None, None) == 0


@pytest.mark.parametrize("sfx", POW2)
def test_dual_quant_validation(L, sfx):
    f = getattr(L, "puro_quant_dual_1x128" + sfx)
    assert f(FAKE, 100, 128, FAKE, FAKE, FAKE, FAKE, None) == 2    # ragged rows
    assert f(FAKE, 128, 200, FAKE, FAKE, FAKE, FAKE, None) == 2    # ragged cols
    assert f(FAKE, 1 << 25, 128, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert f(None, 128, 128, FAKE, FAKE, FAKE, FAKE, None) == 1    # NULL input
    assert f(FAKE, 128, 128, FAKE, FAKE, None, FAKE, None) == 1    # NULL transposed payload
    assert f(FAKE, 128, 128, FAKE, FAKE, FAKE, None, None) == 1    # NULL transposed scales
    assert f(FAKE, 128, 128, FAKE, FAKE, FAKE, MIS, None) == 3     # misaligned
    assert f(None, 0, 128, None, None, None, None, None) == 0      # empty: nothing to do


@pytest.mark.parametrize("sfx", POW2)
def test_w_group_validation(L, sfx):
    from blockwise_fp8_gemm_x128_amd._lib import PuroWItem
    f = getattr(L, "puro_quant_w_128x128_group" + sfx)
    items = (PuroWItem * 9)()
    for i in range(9):
        items[i] = PuroWItem(FAKE, 128, 256, FAKE, FAKE)
    assert f(items, -1, None) == 5                         # count out of range
    assert f(items, 9, None) == 5
    assert f(None, 1, None) == 1                           # NULL item array
    assert f(None, 0, None) == 0                           # nothing to do
    items[1] = PuroWItem(FAKE, 128, 200, FAKE, FAKE)
    assert f(items, 2, None) == 2                          # ragged entry
    items[1] = PuroWItem(None, 128, 256, FAKE, FAKE)
    assert f(items, 2, None) == 1                          # NULL input of an entry
    items[1] = PuroWItem(FAKE, 128, 256, FAKE, MIS)
    assert f(items, 2, None) == 3                          # misaligned scales
    items[0] = PuroWItem(None, 0, 256, None, None)         # empty entries are skipped
    items[1] = PuroWItem(None, 128, 0, None, None)
    assert f(items, 2, None) == 0


@pytest.mark.parametrize("sfx", POW2)
def test_gemm_validation(L, sfx):
    fwd, dgrad, wgrad = (getattr(L, "puro_fp8_gemm_" + k + sfx) for k in ("fwd", "dgrad", "wgrad"))
    for f in (fwd, dgrad):
        assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 130, 128, 128, None) == 2
        assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 128, 128, 64, None) == 2
        assert f(None, FAKE, FAKE, FAKE, FAKE, 128, 128, 128, None) == 1
        assert f(FAKE, FAKE, FAKE, FAKE, None, 128, 128, 128, None) == 1
        assert f(FAKE, FAKE, MIS, FAKE, FAKE, 128, 128, 128, None) == 3
        assert f(None, None, None, None, None, 0, 128, 128, None) == 0
    assert fwd(None, None, None, None, None, 128, 0, 128, None) == 0
    assert dgrad(None, None, None, None, None, 128, 128, 0, None) == 0
    assert wgrad(FAKE, FAKE, FAKE, FAKE, FAKE, 128, 128, 128, 2, None) == 5
    assert wgrad(FAKE, FAKE, FAKE, FAKE, FAKE, 128, 96, 128, 0, None) == 2
    assert wgrad(FAKE, FAKE, FAKE, FAKE, None, 128, 128, 128, 0, None) == 1
    assert wgrad(None, None, None, None, None, 128, 0, 128, 1, None) == 0


def test_optim_validation(L):
    from blockwise_fp8_gemm_x128_amd._lib import OPT_WORKSPACE_BYTES, PuroAdamWParams
    assert OPT_WORKSPACE_BYTES == 8 * 2048 + 256
    text = open(HEADER).read()
    assert "#define PURO_OPT_MAX_BLOCKS 2048" in text
    norm, hb, adamw = L.puro_frobenius_norm, L.puro_hyperball_step, L.puro_adamw_step
    assert norm(FAKE, 6, FAKE, FAKE, None) == 2            # numel not a multiple of 4
    assert norm(FAKE, -4, FAKE, FAKE, None) == 2
    assert norm(None, 8, FAKE, FAKE, None) == 1
    assert norm(FAKE, 8, None, FAKE, None) == 1            # NULL output
    assert norm(FAKE, 8, FAKE, None, None) == 1            # NULL workspace
    assert norm(FAKE, 8, FAKE, MIS, None) == 3             # misaligned workspace
    assert hb(FAKE, FAKE, 6, 0.1, FAKE, FAKE, FAKE, None) == 2
    assert hb(FAKE, None, 8, 0.1, FAKE, FAKE, FAKE, None) == 1
    assert hb(FAKE, FAKE, 8, 0.1, None, FAKE, FAKE, None) == 1    # NULL radius
    assert hb(FAKE, FAKE, 8, 0.1, FAKE, FAKE, None, None) == 1    # NULL workspace
    assert hb(FAKE, FAKE, 8, 0.1, FAKE, MIS, FAKE, None) == 3     # misaligned bf16 output
    assert hb(FAKE, FAKE, 8, float("nan"), FAKE, FAKE, FAKE, None) == 5
    assert hb(None, None, 0, 0.1, None, None, None, None) == 0    # empty: nothing to do
    ok = PuroAdamWParams(1e-3, 0.9, 0.95, 1e-8, 0.1, 1)
    assert adamw(FAKE, FAKE, FAKE, FAKE, 6, ctypes.byref(ok), None, None) == 2
    assert adamw(FAKE, FAKE, FAKE, FAKE, 8, None, None, None) == 1
    assert adamw(FAKE, FAKE, None, FAKE, 8, ctypes.byref(ok), None, None) == 1
    assert adamw(FAKE, FAKE, FAKE, FAKE, 8, ctypes.byref(ok), MIS, None) == 3
    for bad in (PuroAdamWParams(1e-3, 0.9, 0.95, 1e-8, 0.1, 0),      # step 0
                PuroAdamWParams(1e-3, 1.0, 0.95, 1e-8, 0.1, 1),      # beta1 = 1
                PuroAdamWParams(1e-3, 0.9, -0.1, 1e-8, 0.1, 1),      # beta2 < 0
                PuroAdamWParams(1e-3, 0.9, 0.95, 0.0, 0.1, 1),       # eps = 0
                PuroAdamWParams(float("inf"), 0.9, 0.95, 1e-8, 0.1, 1)):
        assert adamw(FAKE, FAKE, FAKE, FAKE, 8, ctypes.byref(bad), None, None) == 5
    assert adamw(None, None, None, None, 0, ctypes.byref(ok), None, None) == 0


def test_gemm_kernel_names(L):
    # the kernel each GEMM entry point picks for the Qwen3-1.7B-shaped layer at M = 8192 on a
    # 256-CU part (no device here: the shape picker assumes 256 compute units)
    name = lambda op, M, N, K, p=0: (L.puro_gemm_kernel_name(op, M, N, K, p) or b"").decode()  # noqa: E731
    for K, N in ((2048, 4096), (2048, 2048), (2048, 12288), (6144, 2048)):
        assert name(0, 8192, N, K) == "gemm_fwd_256x256"
        assert name(1, 8192, N, K) == "gemm_dgrad_256x256"
        assert name(0, 8192, N, K, 1) == "gemm_fwd_256x256_pow2"
    assert name(2, 8192, 4096, 2048) == "gemm_wgrad_128x128"
    assert name(2, 8192, 2048, 2048) == "gemm_wgrad_128x128_k2"
    assert name(2, 8192, 12288, 2048) == "gemm_wgrad_192x256"
    assert name(2, 8192, 2048, 6144) == "gemm_wgrad_256x192"
    assert name(2, 8192, 4096, 4096) == "gemm_wgrad_256x256"
    assert name(0, 256, 256, 256) == "gemm_fwd_128x128"
    assert name(1, 256, 256, 256, 1) == "gemm_dgrad_128x128_pow2"
    assert name(0, 0, 256, 256) == "" and name(0, 130, 256, 256) == "" and name(3, 128, 128, 128) == ""
    assert name(0, 128, 128, 128, 2) == ""


def test_noalloc_validation(L):
    # invalid arguments are rejected before the device is touched
    f = L.puro_hyperball_step_noalloc
    assert f(FAKE, FAKE, 6, 0.1, FAKE, FAKE, None) == 2           # numel not a multiple of 4
    assert f(FAKE, FAKE, (1 << 40) + 4, 0.1, FAKE, FAKE, None) == 2   # beyond the size limit
    assert f(FAKE, None, 8, 0.1, FAKE, FAKE, None) == 1           # NULL direction
    assert f(FAKE, FAKE, 8, 0.1, None, FAKE, None) == 1           # NULL radius
    assert f(FAKE, FAKE, 8, 0.1, FAKE, MIS, None) == 3            # misaligned bf16 output
    assert f(FAKE, FAKE, 8, float("inf"), FAKE, FAKE, None) == 5  # non-finite learning rate
    assert f(None, None, 0, 0.1, None, None, None) == 0           # empty: nothing to do


def test_launch_failure_maps_to_err_launch(L):
    # With no HIP device the runtime rejects every launch: calls whose arguments pass validation
    # must then report PURO_ERR_LAUNCH (4) rather than succeed or crash. On a machine with a
    # device these arguments would reach a kernel, so the test only runs where there is none.
    import torch
    if torch.cuda.is_available():
        pytest.skip("a HIP device is present: these fake pointers would be dereferenced")
    assert L.puro_quant_act_1x128(FAKE, 128, 128, FAKE, FAKE, None) == 4
    assert L.puro_quant_dual_1x128(FAKE, 128, 128, FAKE, FAKE, FAKE, FAKE, None) == 4
    assert L.puro_fp8_gemm_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 128, 128, 128, None) == 4
    assert L.puro_fp8_gemm_wgrad(FAKE, FAKE, FAKE, FAKE, FAKE, 8192, 2048, 2048, 0, None) == 4
    assert L.puro_hyperball_step_noalloc(FAKE, FAKE, 8, 0.1, FAKE, FAKE, None) == 4


def test_probe_library_validation():
    """The matrix-core microbenchmark (libpuro_probe.so, bench.py --ceiling) loads, exports its
    one function and rejects bad arguments before any launch."""
    from blockwise_fp8_gemm_x128_amd.build import PROBE_PATH, build
    if not os.path.exists(PROBE_PATH):
        build(verbose=False)
    P = ctypes.CDLL(PROBE_PATH)
    fn = P.puro_probe_mfma
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                   ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.c_void_p]
    p = 1 << 16  # a fake, 64-byte aligned address: validation never dereferences it
    good = (p, 4096, 1, 8, 1, 0, p, p, p, None)
    for i, bad in ((0, None), (1, 4000), (1, 4100), (0, p + 32), (2, 0), (3, 17), (3, 0),
                   (4, 0), (5, 3), (5, -1), (6, None), (7, None), (8, None)):
        args = list(good)
        args[i] = bad
        assert fn(*args) == 1, (i, bad)


def test_debug_level(L):
    """The debug level is host state: settable, clamped at 0, and read from PURO_DEBUG."""
    import subprocess
    import sys
    before = L.puro_debug_level()
    try:
        L.puro_set_debug(2)
        assert L.puro_debug_level() == 2
        L.puro_set_debug(-5)
        assert L.puro_debug_level() == 0
    finally:
        L.puro_set_debug(before)
    code = ("import sys; sys.path.insert(0, %r); from blockwise_fp8_gemm_x128_amd import _lib; "
            "print(_lib.lib().puro_debug_level())" % ROOT)
    for env, want in (("3", "3"), ("0", "0"), ("", "0")):
        out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                             env={**os.environ, "PURO_DEBUG": env}, timeout=120)
        assert out.stdout.strip() == want, (env, out.stdout, out.stderr)
