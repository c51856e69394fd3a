"""CPU oracle for the blockwise-FP8 quantisers and GEMMs — TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg may
import this package. The GPU library never does, and nothing here imports the GPU library.

Thin ctypes/numpy wrapper over ``oracle.c`` (plain C, IEEE binary32/64 arithmetic, OpenMP over
independent groups/rows). The method it follows is stated in the page "Paper walkthrough:
Puro-2B" (ta-paperlens.web.app), section "Lever 2: use blockwise FP8 from step zero": the
linear-layer GEMMs alone take FP8 operands, each with an fp32 scale per local group (a run of
128 along the GEMM's reduction for X and dY, a 128x128 block for W).

Inputs are bf16 tensors given as numpy ``uint16`` bit patterns (or torch bf16 CPU tensors);
quantised payloads are ``uint8`` E4M3 codes; scales are ``float32``; GEMM results ``float64``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
             "-fno-fast-math", "-Wall"]


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            I64 = ctypes.c_int64
            L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
            L.oracle_bf16_to_f32.restype = ctypes.c_float
            L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
            L.oracle_e4m3_decode.restype = ctypes.c_double
            L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
            L.oracle_e4m3_encode.restype = ctypes.c_uint8
            L.oracle_e4m3_encode_array.argtypes = [P, I64, P]
            L.oracle_quant_group.argtypes = [P, I64, I64, P, I64, P, ctypes.c_int]
            for name in ("oracle_quant_act_1x128", "oracle_quant_w_128x128",
                         "oracle_quant_transpose"):
                getattr(L, name).argtypes = [P, I64, I64, P, P, ctypes.c_int]
                getattr(L, name).restype = None
            for name in ("oracle_gemm_fwd", "oracle_gemm_dgrad", "oracle_gemm_wgrad"):
                getattr(L, name).argtypes = [P, P, P, P, I64, I64, I64, P, I64, P]
                getattr(L, name).restype = None
            L.oracle_num_threads.restype = ctypes.c_int
            D = ctypes.c_double
            L.oracle_frobenius_norm.argtypes = [P, I64]
            L.oracle_frobenius_norm.restype = D
            L.oracle_hyperball_update.argtypes = [P, P, I64, D, D, P]
            L.oracle_hyperball_update.restype = None
            L.oracle_adamw.argtypes = [P, P, P, P, I64, D, D, D, D, D, I64, P, P, P]
            L.oracle_adamw.restype = None
            _lib = L
    return _lib


def _u16(x) -> np.ndarray:
    """bf16 data as a C-contiguous uint16 array of bit patterns."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            assert x.dtype == torch.bfloat16
            x = x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    assert x.dtype == np.uint16, x.dtype
    return x


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def bf16_to_f32(h: int) -> float:
    return float(lib().oracle_bf16_to_f32(int(h)))


def e4m3_decode(code: int) -> float:
    return float(lib().oracle_e4m3_decode(int(code)))


def e4m3_decode_array(codes) -> np.ndarray:
    table = np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(t: float) -> int:
    return int(lib().oracle_e4m3_encode(float(t)))


def e4m3_encode_array(t) -> np.ndarray:
    t = np.ascontiguousarray(t, dtype=np.float32)
    out = np.empty(t.shape, dtype=np.uint8)
    lib().oracle_e4m3_encode_array(_ptr(t), t.size, _ptr(out))
    return out


def quant_group(x, pow2: bool = False) -> tuple[np.ndarray, float]:
    """Quantise one group (any length) of bf16 bit patterns. ``pow2`` selects power-of-two
    scales (the smallest 2^e, e >= -127, with 448 * 2^e >= amax) instead of amax/448."""
    x = _u16(x).reshape(-1)
    q = np.empty(x.size, dtype=np.uint8)
    s = np.empty(1, dtype=np.float32)
    lib().oracle_quant_group(_ptr(x), x.size, 1, _ptr(q), 1, _ptr(s), int(bool(pow2)))
    return q, float(s[0])


def quant_act_1x128(x, pow2: bool = False) -> tuple[np.ndarray, np.ndarray]:
    """x[rows, cols] bf16 -> (q[rows, cols] uint8, s[cols/128, rows] float32)."""
    x = _u16(x)
    rows, cols = x.shape
    assert cols % 128 == 0
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty((cols // 128, rows), dtype=np.float32)
    lib().oracle_quant_act_1x128(_ptr(x), rows, cols, _ptr(q), _ptr(s), int(bool(pow2)))
    return q, s


def quant_w_128x128(w, pow2: bool = False) -> tuple[np.ndarray, np.ndarray]:
    """w[n, k] bf16 -> (q[n, k] uint8, s[n/128, k/128] float32)."""
    w = _u16(w)
    n, k = w.shape
    assert n % 128 == 0 and k % 128 == 0
    q = np.empty((n, k), dtype=np.uint8)
    s = np.empty((n // 128, k // 128), dtype=np.float32)
    lib().oracle_quant_w_128x128(_ptr(w), n, k, _ptr(q), _ptr(s), int(bool(pow2)))
    return q, s


def quant_transpose(x, pow2: bool = False) -> tuple[np.ndarray, np.ndarray]:
    """x[rows, cols] bf16 -> (qt[cols, rows] uint8, st[rows/128, cols] float32)."""
    x = _u16(x)
    rows, cols = x.shape
    assert rows % 128 == 0
    qt = np.empty((cols, rows), dtype=np.uint8)
    st = np.empty((rows // 128, cols), dtype=np.float32)
    lib().oracle_quant_transpose(_ptr(x), rows, cols, _ptr(qt), _ptr(st), int(bool(pow2)))
    return qt, st


def _rows(rows, total):
    if rows is None:
        return None, total
    r = np.ascontiguousarray(rows, dtype=np.int64)
    assert r.ndim == 1 and (r.size == 0 or (r.min() >= 0 and r.max() < total))
    return r, r.size


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


def gemm_fwd(xq, sx, wq, sw, rows=None) -> np.ndarray:
    """Y[m, n] = sum_kb sx[kb, m] * sw[n/128, kb] * sum_{k in kb} xq[m, k] * wq[n, k]."""
    xq, wq = _c(xq, np.uint8), _c(wq, np.uint8)
    sx, sw = _c(sx, np.float32), _c(sw, np.float32)
    M, K = xq.shape
    N = wq.shape[0]
    assert wq.shape == (N, K) and sx.shape == (K // 128, M) and sw.shape == (N // 128, K // 128)
    r, nr = _rows(rows, M)
    out = np.empty((nr, N), dtype=np.float64)
    lib().oracle_gemm_fwd(_ptr(xq), _ptr(sx), _ptr(wq), _ptr(sw), M, N, K,
                          None if r is None else _ptr(r), nr, _ptr(out))
    return out


def gemm_dgrad(dyq, sdy, wq, sw, rows=None) -> np.ndarray:
    """dX[m, k] = sum_nb sdy[nb, m] * sw[nb, k/128] * sum_{n in nb} dyq[m, n] * wq[n, k]."""
    dyq, wq = _c(dyq, np.uint8), _c(wq, np.uint8)
    sdy, sw = _c(sdy, np.float32), _c(sw, np.float32)
    M, N = dyq.shape
    K = wq.shape[1]
    assert wq.shape == (N, K) and sdy.shape == (N // 128, M) and sw.shape == (N // 128, K // 128)
    r, nr = _rows(rows, M)
    out = np.empty((nr, K), dtype=np.float64)
    lib().oracle_gemm_dgrad(_ptr(dyq), _ptr(sdy), _ptr(wq), _ptr(sw), M, N, K,
                            None if r is None else _ptr(r), nr, _ptr(out))
    return out


def gemm_wgrad(dytq, sdyt, xtq, sxt, rows=None) -> np.ndarray:
    """dW[n, k] = sum_mb sdyt[mb, n] * sxt[mb, k] * sum_{m in mb} dytq[n, m] * xtq[k, m]."""
    dytq, xtq = _c(dytq, np.uint8), _c(xtq, np.uint8)
    sdyt, sxt = _c(sdyt, np.float32), _c(sxt, np.float32)
    N, M = dytq.shape
    K = xtq.shape[0]
    assert xtq.shape == (K, M) and sdyt.shape == (M // 128, N) and sxt.shape == (M // 128, K)
    r, nr = _rows(rows, N)
    out = np.empty((nr, K), dtype=np.float64)
    lib().oracle_gemm_wgrad(_ptr(dytq), _ptr(sdyt), _ptr(xtq), _ptr(sxt), M, N, K,
                            None if r is None else _ptr(r), nr, _ptr(out))
    return out


def dequant_act(q, s) -> np.ndarray:
    """Exact dequantisation of a 1x128-grouped tensor: q[r, c] -> dec(q) * s[c/128, r]."""
    v = e4m3_decode_array(q)
    return v * np.repeat(s.T.astype(np.float64), 128, axis=1)


def dequant_w(q, s) -> np.ndarray:
    """Exact dequantisation of a 128x128-blocked tensor."""
    v = e4m3_decode_array(q)
    return v * np.kron(s.astype(np.float64), np.ones((128, 128)))


def _f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == np.float32, a.dtype
    return a


def frobenius_norm(w) -> float:
    """sqrt(sum w^2) of an fp32 array, in binary64."""
    w = _f32(w)
    return float(lib().oracle_frobenius_norm(_ptr(w), w.size))


def hyperball_update(w, u, lr: float, radius: float) -> np.ndarray:
    """(w - lr*u) scaled to Frobenius norm `radius` (binary64, shape of w)."""
    w, u = _f32(w), _f32(u)
    assert w.shape == u.shape
    out = np.empty(w.shape, dtype=np.float64)
    lib().oracle_hyperball_update(_ptr(w), _ptr(u), w.size, float(lr), float(radius), _ptr(out))
    return out


def adamw(p, g, m, v, lr, beta1, beta2, eps, weight_decay, step):
    """One AdamW step on fp32 state -> (p, m, v) in binary64."""
    p, g, m, v = _f32(p), _f32(g), _f32(m), _f32(v)
    assert p.shape == g.shape == m.shape == v.shape and step >= 1
    outs = [np.empty(p.shape, dtype=np.float64) for _ in range(3)]
    lib().oracle_adamw(_ptr(p), _ptr(g), _ptr(m), _ptr(v), p.size, float(lr), float(beta1),
                       float(beta2), float(eps), float(weight_decay), int(step),
                       *[_ptr(o) for o in outs])
    return tuple(outs)
