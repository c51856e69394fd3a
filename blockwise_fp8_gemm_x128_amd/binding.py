"""Python binding of libpuro's C ABI: same names, argument marshalling only.

Each function takes torch tensors that live on a HIP device, checks dtype / shape / contiguity
/ device, allocates missing outputs with torch (device memory is PyTorch's job here), and calls
the C entry point with raw device pointers on the current torch stream. Every step of the
computation runs in libpuro's HIP kernels; there is no other code path.
"""
from __future__ import annotations

import ctypes

import torch

from ._lib import (OPT_WORKSPACE_BYTES, W_GROUP_MAX, PuroAdamWParams, PuroError, PuroWItem,
                   check, lib)

FP8 = torch.uint8  # E4M3 codes travel as raw bytes


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _need(t: torch.Tensor, name: str, dtype, shape, dev) -> None:
    if not isinstance(t, torch.Tensor):
        raise PuroError(f"{name}: expected a torch.Tensor")
    if t.dtype != dtype:
        raise PuroError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise PuroError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise PuroError(f"{name}: must be contiguous")
    if t.device != dev:
        raise PuroError(f"{name}: on {t.device}, expected {dev}")


def _dev(t: torch.Tensor) -> torch.device:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise PuroError("inputs must be torch tensors on a HIP device")
    return t.device


def _out(t, name, dtype, shape, dev):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    _need(t, name, dtype, shape, dev)
    return t


def puro_quant_act_1x128(x: torch.Tensor, q=None, s=None, _fn="puro_quant_act_1x128"):
    """x bf16 [rows, cols] -> (q uint8 E4M3 [rows, cols], s fp32 [cols/128, rows])."""
    dev = _dev(x)
    rows, cols = x.shape
    _need(x, "x", torch.bfloat16, (rows, cols), dev)
    q = _out(q, "q", FP8, (rows, cols), dev)
    s = _out(s, "s", torch.float32, (cols // 128, rows), dev)
    check(getattr(lib(), _fn)(x.data_ptr(), rows, cols, q.data_ptr(), s.data_ptr(),
                              _stream(dev)))
    return q, s


def puro_quant_w_128x128(w: torch.Tensor, q=None, s=None, _fn="puro_quant_w_128x128"):
    """w bf16 [n, k] -> (q uint8 E4M3 [n, k], s fp32 [n/128, k/128])."""
    dev = _dev(w)
    n, k = w.shape
    _need(w, "w", torch.bfloat16, (n, k), dev)
    q = _out(q, "q", FP8, (n, k), dev)
    s = _out(s, "s", torch.float32, (n // 128, k // 128), dev)
    check(getattr(lib(), _fn)(w.data_ptr(), n, k, q.data_ptr(), s.data_ptr(), _stream(dev)))
    return q, s


def w_group_items(ws, qs, ss):
    """ctypes array of puro_w_item for weights ws [n, k] and outputs qs, ss (checked)."""
    if len(ws) > W_GROUP_MAX:
        raise PuroError(f"at most {W_GROUP_MAX} matrices per grouped call")
    if not (len(ws) == len(qs) == len(ss)):
        raise PuroError("ws, qs and ss must have the same length")
    items = (PuroWItem * max(len(ws), 1))()
    for i, (w, q, s) in enumerate(zip(ws, qs, ss)):
        dev = _dev(w)
        n, k = w.shape
        _need(w, f"w[{i}]", torch.bfloat16, (n, k), dev)
        _need(q, f"q[{i}]", FP8, (n, k), dev)
        _need(s, f"s[{i}]", torch.float32, (n // 128, k // 128), dev)
        items[i] = PuroWItem(w.data_ptr(), n, k, q.data_ptr(), s.data_ptr())
    return items


def puro_quant_w_128x128_group(ws, qs=None, ss=None, _fn="puro_quant_w_128x128_group"):
    """Several bf16 weights [n, k] quantised in one launch -> (list of q, list of s), each as
    from puro_quant_w_128x128."""
    if not ws:
        return [], []
    dev = _dev(ws[0])
    qs = qs or [torch.empty(w.shape, dtype=FP8, device=dev) for w in ws]
    ss = ss or [torch.empty((w.shape[0] // 128, w.shape[1] // 128), dtype=torch.float32,
                            device=dev) for w in ws]
    items = w_group_items(ws, qs, ss)
    check(getattr(lib(), _fn)(items, len(ws), _stream(dev)))
    return qs, ss


def puro_quant_transpose(x: torch.Tensor, qt=None, st=None, _fn="puro_quant_transpose"):
    """x bf16 [rows, cols] -> (qt uint8 E4M3 [cols, rows], st fp32 [rows/128, cols])."""
    dev = _dev(x)
    rows, cols = x.shape
    _need(x, "x", torch.bfloat16, (rows, cols), dev)
    qt = _out(qt, "qt", FP8, (cols, rows), dev)
    st = _out(st, "st", torch.float32, (rows // 128, cols), dev)
    check(getattr(lib(), _fn)(x.data_ptr(), rows, cols, qt.data_ptr(), st.data_ptr(),
                              _stream(dev)))
    return qt, st


def puro_quant_dual_1x128(x: torch.Tensor, q=None, s=None, qt=None, st=None,
                          _fn="puro_quant_dual_1x128"):
    """x bf16 [rows, cols] -> (q [rows, cols], s [cols/128, rows], qt [cols, rows],
    st [rows/128, cols]): the outputs of puro_quant_act_1x128 and puro_quant_transpose from one
    read of x."""
    dev = _dev(x)
    rows, cols = x.shape
    _need(x, "x", torch.bfloat16, (rows, cols), dev)
    q = _out(q, "q", FP8, (rows, cols), dev)
    s = _out(s, "s", torch.float32, (cols // 128, rows), dev)
    qt = _out(qt, "qt", FP8, (cols, rows), dev)
    st = _out(st, "st", torch.float32, (rows // 128, cols), dev)
    check(getattr(lib(), _fn)(x.data_ptr(), rows, cols, q.data_ptr(), s.data_ptr(),
                              qt.data_ptr(), st.data_ptr(), _stream(dev)))
    return q, s, qt, st


def puro_fp8_gemm_fwd(xq, sx, wq, sw, y=None, _fn="puro_fp8_gemm_fwd"):
    """Y bf16 [M, N] from xq [M, K], sx [K/128, M], wq [N, K], sw [N/128, K/128]."""
    dev = _dev(xq)
    M, K = xq.shape
    N = wq.shape[0]
    _need(xq, "xq", FP8, (M, K), dev)
    _need(sx, "sx", torch.float32, (K // 128, M), dev)
    _need(wq, "wq", FP8, (N, K), dev)
    _need(sw, "sw", torch.float32, (N // 128, K // 128), dev)
    y = _out(y, "y", torch.bfloat16, (M, N), dev)
    check(getattr(lib(), _fn)(xq.data_ptr(), sx.data_ptr(), wq.data_ptr(), sw.data_ptr(),
                              y.data_ptr(), M, N, K, _stream(dev)))
    return y


def puro_fp8_gemm_dgrad(dyq, sdy, wq, sw, dx=None, _fn="puro_fp8_gemm_dgrad"):
    """dX bf16 [M, K] from dyq [M, N], sdy [N/128, M], wq [N, K], sw [N/128, K/128]."""
    dev = _dev(dyq)
    M, N = dyq.shape
    K = wq.shape[1]
    _need(dyq, "dyq", FP8, (M, N), dev)
    _need(sdy, "sdy", torch.float32, (N // 128, M), dev)
    _need(wq, "wq", FP8, (N, K), dev)
    _need(sw, "sw", torch.float32, (N // 128, K // 128), dev)
    dx = _out(dx, "dx", torch.bfloat16, (M, K), dev)
    check(getattr(lib(), _fn)(dyq.data_ptr(), sdy.data_ptr(), wq.data_ptr(), sw.data_ptr(),
                              dx.data_ptr(), M, N, K, _stream(dev)))
    return dx


def puro_fp8_gemm_wgrad(dytq, sdyt, xtq, sxt, dw=None, accumulate: bool = False,
                        _fn="puro_fp8_gemm_wgrad"):
    """dW fp32 [N, K] (= or +=) from dytq [N, M], sdyt [M/128, N], xtq [K, M], sxt [M/128, K]."""
    dev = _dev(dytq)
    N, M = dytq.shape
    K = xtq.shape[0]
    _need(dytq, "dytq", FP8, (N, M), dev)
    _need(sdyt, "sdyt", torch.float32, (M // 128, N), dev)
    _need(xtq, "xtq", FP8, (K, M), dev)
    _need(sxt, "sxt", torch.float32, (M // 128, K), dev)
    if accumulate and dw is None:
        raise PuroError("accumulate=True needs an existing dw")
    dw = _out(dw, "dw", torch.float32, (N, K), dev)
    check(getattr(lib(), _fn)(dytq.data_ptr(), sdyt.data_ptr(), xtq.data_ptr(),
                              sxt.data_ptr(), dw.data_ptr(), M, N, K, 1 if accumulate else 0,
                              _stream(dev)))
    return dw


def optim_workspace(dev) -> torch.Tensor:
    """Device workspace for the optimizer-step entry points (PURO_OPT_WORKSPACE_BYTES)."""
    return torch.empty(OPT_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)


def puro_frobenius_norm(w: torch.Tensor, norm=None, workspace=None):
    """||w||_F of an fp32 tensor -> fp32 device tensor of shape (1,)."""
    dev = _dev(w)
    _need(w, "w", torch.float32, tuple(w.shape), dev)
    norm = _out(norm, "norm", torch.float32, (1,), dev)
    ws = optim_workspace(dev) if workspace is None else workspace
    check(lib().puro_frobenius_norm(w.data_ptr(), w.numel(), norm.data_ptr(), ws.data_ptr(),
                                    _stream(dev)))
    return norm


def puro_hyperball_step(w: torch.Tensor, u: torch.Tensor, lr: float, radius: torch.Tensor,
                        w_bf16=None, workspace=None):
    """In place: w <- (w - lr*u) * radius / ||w - lr*u||_F; returns the bf16 copy of w."""
    dev = _dev(w)
    n = w.numel()
    _need(w, "w", torch.float32, tuple(w.shape), dev)
    _need(u, "u", torch.float32, tuple(w.shape), dev)
    _need(radius, "radius", torch.float32, (1,), dev)
    w_bf16 = _out(w_bf16, "w_bf16", torch.bfloat16, tuple(w.shape), dev)
    ws = optim_workspace(dev) if workspace is None else workspace
    check(lib().puro_hyperball_step(w.data_ptr(), u.data_ptr(), n, float(lr), radius.data_ptr(),
                                    w_bf16.data_ptr(), ws.data_ptr(), _stream(dev)))
    return w_bf16


def puro_hyperball_step_noalloc(w: torch.Tensor, u: torch.Tensor, lr: float,
                                radius: torch.Tensor, w_bf16: torch.Tensor):
    """puro_hyperball_step with the library's own scratch instead of a workspace; the bf16
    output is required (this path allocates nothing)."""
    dev = _dev(w)
    _need(w, "w", torch.float32, tuple(w.shape), dev)
    _need(u, "u", torch.float32, tuple(w.shape), dev)
    _need(radius, "radius", torch.float32, (1,), dev)
    _need(w_bf16, "w_bf16", torch.bfloat16, tuple(w.shape), dev)
    check(lib().puro_hyperball_step_noalloc(w.data_ptr(), u.data_ptr(), w.numel(), float(lr),
                                            radius.data_ptr(), w_bf16.data_ptr(), _stream(dev)))
    return w_bf16


def adamw_params(lr, beta1, beta2, eps, weight_decay, step) -> PuroAdamWParams:
    return PuroAdamWParams(lr, beta1, beta2, eps, weight_decay, int(step))


def puro_adamw_step(p, g, m, v, lr, beta1, beta2, eps, weight_decay, step, p_bf16=None,
                    want_bf16: bool = False):
    """In place AdamW step on fp32 p, m, v with gradient g; returns the bf16 copy of p if
    p_bf16 is given or want_bf16 is set, else None."""
    dev = _dev(p)
    shape = tuple(p.shape)
    for t, name in ((p, "p"), (g, "g"), (m, "m"), (v, "v")):
        _need(t, name, torch.float32, shape, dev)
    if p_bf16 is None and want_bf16:
        p_bf16 = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    if p_bf16 is not None:
        _need(p_bf16, "p_bf16", torch.bfloat16, shape, dev)
    hp = adamw_params(lr, beta1, beta2, eps, weight_decay, step)
    check(lib().puro_adamw_step(p.data_ptr(), g.data_ptr(), m.data_ptr(), v.data_ptr(),
                                p.numel(), ctypes.byref(hp),
                                None if p_bf16 is None else p_bf16.data_ptr(), _stream(dev)))
    return p_bf16


def _pow2_variant(base):
    name = base.__name__ + "_pow2"

    def f(*args, **kwargs):
        return base(*args, _fn=name, **kwargs)

    f.__name__ = name
    f.__doc__ = (base.__doc__ or "") + "\n\n    Power-of-two scales (the library's E8M0 variant)."
    return f


puro_quant_act_1x128_pow2 = _pow2_variant(puro_quant_act_1x128)
puro_quant_w_128x128_pow2 = _pow2_variant(puro_quant_w_128x128)
puro_quant_w_128x128_group_pow2 = _pow2_variant(puro_quant_w_128x128_group)
puro_quant_transpose_pow2 = _pow2_variant(puro_quant_transpose)
puro_quant_dual_1x128_pow2 = _pow2_variant(puro_quant_dual_1x128)
puro_fp8_gemm_fwd_pow2 = _pow2_variant(puro_fp8_gemm_fwd)
puro_fp8_gemm_dgrad_pow2 = _pow2_variant(puro_fp8_gemm_dgrad)
puro_fp8_gemm_wgrad_pow2 = _pow2_variant(puro_fp8_gemm_wgrad)


def puro_set_debug(level: int) -> None:
    """Debug level of the library (0: off; 1 or more: every quantiser and GEMM call checks its
    inputs on the device first and raises PuroError with PURO_ERR_INPUT on data outside the
    contract)."""
    lib().puro_set_debug(int(level))


def puro_debug_level() -> int:
    """Current debug level (initially the PURO_DEBUG environment variable, else 0)."""
    return int(lib().puro_debug_level())


def puro_gemm_kernel_name(op: str, M: int, N: int, K: int, pow2: bool = False) -> str:
    """Name of the kernel function puro_fp8_gemm_<op> (op: 'fwd', 'dgrad' or 'wgrad') launches
    for these sizes on the current device, or '' if it would launch nothing."""
    code = {"fwd": 0, "dgrad": 1, "wgrad": 2}[op]
    res = lib().puro_gemm_kernel_name(code, M, N, K, int(bool(pow2)))
    return res.decode() if res else ""


def prepare(name: str, *args, stream=None):
    """Pre-marshalled call of a C entry point for hot loops: tensors become raw device
    pointers, `stream` (a torch.cuda.Stream; default the current torch stream) is bound, and the
    returned zero-argument callable only crosses into the C ABI (which still validates) and
    checks the status."""
    fn = getattr(lib(), name)
    dev = None
    conv = []
    for a in args:
        if isinstance(a, torch.Tensor):
            dev = dev or a.device
            conv.append(a.data_ptr())
        else:
            conv.append(a)
    conv.append(stream.cuda_stream if stream is not None else _stream(dev))

    keep = tuple(args)  # tensors and ctypes arrays the raw arguments point into

    def call():
        # `keep` holds the tensors: their device memory must outlive every launch of this call
        # (including replays of a captured graph), not just the moment of preparation.
        st = fn(*conv)
        if st != 0:
            check(st)

    call.tensors = keep
    return call
