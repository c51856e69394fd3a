"""Blockwise-FP8 linear-layer GEMMs and quantisers for AMD Instinct MI355X (gfx950).

The compute lives in ``libpuro.so`` (HIP kernels behind the C ABI in ``include/puro.h``);
this package is its thin binding (``binding``), the hipcc build step (``build``) and the seeded
synthetic-input recipes (``synth``).
"""
from ._lib import PuroError  # noqa: F401

__all__ = [
    "PuroError",
    "puro_quant_act_1x128",
    "puro_quant_w_128x128",
    "puro_quant_transpose",
    "puro_fp8_gemm_fwd",
    "puro_fp8_gemm_dgrad",
    "puro_fp8_gemm_wgrad",
    "puro_quant_dual_1x128",
    "puro_quant_w_128x128_group",
    "puro_quant_act_1x128_pow2",
    "puro_quant_w_128x128_pow2",
    "puro_quant_w_128x128_group_pow2",
    "puro_quant_transpose_pow2",
    "puro_quant_dual_1x128_pow2",
    "puro_fp8_gemm_fwd_pow2",
    "puro_fp8_gemm_dgrad_pow2",
    "puro_fp8_gemm_wgrad_pow2",
]


def __getattr__(name):
    # The torch-facing binding is imported lazily so that the build step and the C-ABI checks
    # work without initialising torch.
    if name in __all__[1:]:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
