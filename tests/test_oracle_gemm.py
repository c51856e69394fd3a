"""Pins of the oracle GEMMs: exact rational brute force on tiny non-square shapes (catches a
dropped chunk, a wrong scale index, a transposed operand or a sign), the numpy float64 matmul
of exactly dequantised operands (library special case), and a lossless-quantisation case in
which quantise-then-multiply must reproduce the plain double matmul of the bf16 inputs."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from helpers import bf16_bits_to_f32, f32_to_bf16_bits, torch_e4m3_decode

DEC = torch_e4m3_decode(np.arange(256, dtype=np.uint8))


def _rand_bf16(shape, seed, std=1.0):
    g = torch.Generator().manual_seed(seed)
    t = (torch.randn(shape, generator=g) * std).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _exact_dot(a_vals, a_scales, b_vals, b_scales):
    """sum_l (dec(a_l) * sa_l) * (dec(b_l) * sb_l) in exact rationals."""
    tot = Fraction(0)
    mag = Fraction(0)
    for av, asc, bv, bsc in zip(a_vals, a_scales, b_vals, b_scales):
        term = Fraction(float(av)) * Fraction(float(asc)) * Fraction(float(bv)) * Fraction(float(bsc))
        tot += term
        mag += abs(term)
    return tot, mag


def _check(out, exact, mag):
    assert abs(Fraction(float(out)) - exact) <= Fraction(1, 10 ** 14) * mag + Fraction(1, 10 ** 300)


def test_fwd_brute_force(oracle):
    M, N, K = 3, 128, 256
    x = _rand_bf16((M, K), 21)
    w = _rand_bf16((N, K), 22, 0.02)
    xq, sx = oracle.quant_act_1x128(x)
    wq, sw = oracle.quant_w_128x128(w)
    y = oracle.gemm_fwd(xq, sx, wq, sw)
    assert y.shape == (M, N)
    rng = np.random.default_rng(0)
    for m, n in [(0, 0), (2, 127)] + [tuple(p) for p in rng.integers(0, [M, N], size=(6, 2))]:
        ex, mag = _exact_dot(DEC[xq[m]], [sx[k // 128, m] for k in range(K)],
                             DEC[wq[n]], [sw[n // 128, k // 128] for k in range(K)])
        _check(y[m, n], ex, mag)


def test_dgrad_brute_force(oracle):
    M, N, K = 3, 256, 128
    dy = _rand_bf16((M, N), 23, 1e-3)
    w = _rand_bf16((N, K), 24, 0.02)
    dyq, sdy = oracle.quant_act_1x128(dy)
    wq, sw = oracle.quant_w_128x128(w)
    dx = oracle.gemm_dgrad(dyq, sdy, wq, sw)
    assert dx.shape == (M, K)
    for m, k in [(0, 0), (2, 127), (1, 64), (0, 5)]:
        ex, mag = _exact_dot(DEC[dyq[m]], [sdy[n // 128, m] for n in range(N)],
                             DEC[wq[:, k]], [sw[n // 128, k // 128] for n in range(N)])
        _check(dx[m, k], ex, mag)


def test_wgrad_brute_force(oracle):
    M, N, K = 256, 3, 5
    dy = _rand_bf16((M, N), 25, 1e-3)
    x = _rand_bf16((M, K), 26)
    dytq, sdyt = oracle.quant_transpose(dy)
    xtq, sxt = oracle.quant_transpose(x)
    dw = oracle.gemm_wgrad(dytq, sdyt, xtq, sxt)
    assert dw.shape == (N, K)
    for n in range(N):
        for k in range(K):
            ex, mag = _exact_dot(DEC[dytq[n]], [sdyt[m // 128, n] for m in range(M)],
                                 DEC[xtq[k]], [sxt[m // 128, k] for m in range(M)])
            _check(dw[n, k], ex, mag)


def test_row_subset_matches_full(oracle):
    x = _rand_bf16((40, 256), 27)
    w = _rand_bf16((256, 256), 28, 0.02)
    xq, sx = oracle.quant_act_1x128(x)
    wq, sw = oracle.quant_w_128x128(w)
    full = oracle.gemm_fwd(xq, sx, wq, sw)
    rows = np.array([39, 0, 17])
    assert np.array_equal(oracle.gemm_fwd(xq, sx, wq, sw, rows=rows), full[rows])


def _frob_rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def test_numpy_dequant_matmul(oracle):
    M, N, K = 64, 256, 384
    x = _rand_bf16((M, K), 31)
    w = _rand_bf16((N, K), 32, 0.02)
    dy = _rand_bf16((M, N), 33, 1e-3)
    xq, sx = oracle.quant_act_1x128(x)
    wq, sw = oracle.quant_w_128x128(w)
    dyq, sdy = oracle.quant_act_1x128(dy)
    xd = DEC[xq] * np.repeat(sx.T.astype(np.float64), 128, axis=1)
    wd = DEC[wq] * np.kron(sw.astype(np.float64), np.ones((128, 128)))
    dyd = DEC[dyq] * np.repeat(sdy.T.astype(np.float64), 128, axis=1)
    assert _frob_rel(oracle.gemm_fwd(xq, sx, wq, sw), xd @ wd.T) < 1e-13
    assert _frob_rel(oracle.gemm_dgrad(dyq, sdy, wq, sw), dyd @ wd) < 1e-13
    M2 = 384
    x2 = _rand_bf16((M2, 256), 34)
    dy2 = _rand_bf16((M2, 128), 35, 1e-3)
    xtq, sxt = oracle.quant_transpose(x2)
    dytq, sdyt = oracle.quant_transpose(dy2)
    xtd = DEC[xtq] * np.repeat(sxt.T.astype(np.float64), 128, axis=1)
    dytd = DEC[dytq] * np.repeat(sdyt.T.astype(np.float64), 128, axis=1)
    assert _frob_rel(oracle.gemm_wgrad(dytq, sdyt, xtq, sxt), dytd @ xtd.T) < 1e-13


def _lossless_rows(rows, cols, seed):
    """bf16 rows whose every 1x128 group is (E4M3 values) * 2^j with one element = +-448 * 2^j,
    so quantisation is exact with s = 2^j."""
    rng = np.random.default_rng(seed)
    finite = DEC[np.r_[0:0x7F, 0x80:0xFF]]
    vals = rng.choice(finite, size=(rows, cols))
    for r in range(rows):
        for g in range(cols // 128):
            vals[r, g * 128 + rng.integers(128)] = rng.choice([448.0, -448.0])
            vals[r, g * 128:(g + 1) * 128] *= 2.0 ** int(rng.integers(-3, 4))
    return vals.astype(np.float32)


def test_lossless_quantisation_reproduces_plain_matmul(oracle):
    M, N, K = 5, 128, 384
    xv = _lossless_rows(M, K, 41)
    # weights: one scale per 128x128 block, so build each block from one power of two
    rng = np.random.default_rng(42)
    finite = DEC[np.r_[0:0x7F, 0x80:0xFF]]
    wv = rng.choice(finite, size=(N, K)).astype(np.float64)
    for bj in range(K // 128):
        wv[rng.integers(N), bj * 128 + rng.integers(128)] = 448.0
        wv[:, bj * 128:(bj + 1) * 128] *= 2.0 ** int(rng.integers(-3, 4))
    wv = wv.astype(np.float32)
    x, w = f32_to_bf16_bits(xv), f32_to_bf16_bits(wv)
    xq, sx = oracle.quant_act_1x128(x)
    wq, sw = oracle.quant_w_128x128(w)
    assert np.array_equal(DEC[xq] * np.repeat(sx.T.astype(np.float64), 128, axis=1), xv)
    y = oracle.gemm_fwd(xq, sx, wq, sw)
    ref = bf16_bits_to_f32(x).astype(np.float64) @ bf16_bits_to_f32(w).astype(np.float64).T
    assert _frob_rel(y, ref) < 1e-14


def test_zero_reduction_chunks_contribute_nothing(oracle):
    # an all-zero 1x128 group quantises to s = 1 and zero codes; its chunk adds exactly 0
    x = _rand_bf16((4, 256), 51)
    x[:, 128:] = 0
    w = _rand_bf16((128, 256), 52, 0.02)
    xq, sx = oracle.quant_act_1x128(x)
    wq, sw = oracle.quant_w_128x128(w)
    assert np.all(sx[1] == 1.0) and np.all(xq[:, 128:] == 0)
    full = oracle.gemm_fwd(xq, sx, wq, sw)
    half = oracle.gemm_fwd(np.ascontiguousarray(xq[:, :128]), np.ascontiguousarray(sx[:1]),
                           np.ascontiguousarray(wq[:, :128]), np.ascontiguousarray(sw[:, :1]))
    assert np.array_equal(full, half)
