"""ctypes loader for libpuro.so. The library must have been built (see build.py); there is no
fallback of any kind: a missing or unloadable library raises."""
from __future__ import annotations

import ctypes
import os
import threading

from .build import LIB_PATH

_lock = threading.Lock()
_lib = None

# Every symbol declared in include/puro.h, with its ctypes signature.
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
W_GROUP_MAX = 8  # PURO_W_GROUP_MAX


class PuroWItem(ctypes.Structure):
    """puro_w_item: one weight matrix of a grouped 128x128 quantisation."""
    _fields_ = [("w", ctypes.c_void_p), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("q", ctypes.c_void_p), ("s", ctypes.c_void_p)]

class PuroAdamWParams(ctypes.Structure):
    """puro_adamw_params: AdamW hyperparameters of one step."""
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("step", ctypes.c_int64)]


OPT_MAX_BLOCKS = 2048  # PURO_OPT_MAX_BLOCKS
OPT_WORKSPACE_BYTES = 8 * OPT_MAX_BLOCKS + 256  # PURO_OPT_WORKSPACE_BYTES

SIGNATURES = {
    "puro_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "puro_abi_version": ([], ctypes.c_int),
    "puro_set_debug": ([ctypes.c_int], None),
    "puro_debug_level": ([], ctypes.c_int),
    "puro_quant_act_1x128": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "puro_quant_w_128x128": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "puro_quant_transpose": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "puro_quant_dual_1x128": ([_P, _I64, _I64, _P, _P, _P, _P, _P], ctypes.c_int),
    "puro_quant_w_128x128_group": ([ctypes.POINTER(PuroWItem), ctypes.c_int, _P], ctypes.c_int),
    "puro_fp8_gemm_fwd": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "puro_fp8_gemm_dgrad": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "puro_fp8_gemm_wgrad": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, ctypes.c_int, _P],
                            ctypes.c_int),
    "puro_gemm_kernel_name": ([ctypes.c_int, _I64, _I64, _I64, ctypes.c_int], ctypes.c_char_p),
}
SIGNATURES.update({
    "puro_frobenius_norm": ([_P, _I64, _P, _P, _P], ctypes.c_int),
    "puro_hyperball_step": ([_P, _P, _I64, ctypes.c_float, _P, _P, _P, _P], ctypes.c_int),
    "puro_hyperball_step_noalloc": ([_P, _P, _I64, ctypes.c_float, _P, _P, _P], ctypes.c_int),
    "puro_adamw_step": ([_P, _P, _P, _P, _I64, ctypes.POINTER(PuroAdamWParams), _P, _P],
                        ctypes.c_int),
})
# The power-of-two-scale variants take the same arguments as their standard counterparts.
POW2_BASES = ("puro_quant_act_1x128", "puro_quant_w_128x128", "puro_quant_w_128x128_group",
              "puro_quant_transpose", "puro_quant_dual_1x128", "puro_fp8_gemm_fwd",
              "puro_fp8_gemm_dgrad", "puro_fp8_gemm_wgrad")
SIGNATURES.update({b + "_pow2": SIGNATURES[b] for b in POW2_BASES})


class PuroError(RuntimeError):
    """A libpuro call returned a nonzero status (or the library is unavailable)."""


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise PuroError(
                    "libpuro.so is not built (%s); run `python -m "
                    "blockwise_fp8_gemm_x128_amd.build`" % LIB_PATH)
            try:  # make torch's HIP runtime the one libpuro binds to (one runtime per process)
                import torch  # noqa: F401
            except ImportError:  # pragma: no cover
                pass
            L = ctypes.CDLL(LIB_PATH)
            for name, (args, res) in SIGNATURES.items():
                fn = getattr(L, name)
                fn.argtypes = args
                fn.restype = res
            _lib = L
    return _lib


def check(status: int) -> None:
    if status != 0:
        raise PuroError(lib().puro_status_string(status).decode())
