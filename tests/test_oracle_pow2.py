"""Pins of the oracle's power-of-two-scale quantisers (a variant of this library; the pages fix
one fp32 scale per group and no formula). A nonzero group's scale is s = 2^e for the least
integer e with 448 * 2^e >= amax (e raised to -127 when smaller), its payload E4M3_RNE(x * 2^-e).

The pins do not retype the oracle: the exponent is found here by exact rational search
(fractions.Fraction), the payload by torch's float8_e4m3fn cast of the exactly scaled value, the
hand cases come from tests/golden/quant_pow2_hand.txt, and the standard rule is cross-checked on
groups where both rules must agree."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from helpers import (bf16_bits_to_f32, f32_to_bf16_bits, read_quant_hand, torch_e4m3_decode,
                     torch_e4m3_encode)


def _group_from_case(case):
    vals = np.zeros(128, np.float32)
    for i, v in case["values"].items():
        vals[i] = v
    return f32_to_bf16_bits(vals)


@pytest.mark.parametrize("case", read_quant_hand("quant_pow2_hand.txt"), ids=lambda c: c["name"])
def test_pow2_hand_golden(oracle, case):
    x = _group_from_case(case)
    q, s = oracle.quant_group(x, pow2=True)
    assert np.float32(s).view(np.uint32) == np.float32(case["scale"]).view(np.uint32)
    want = np.zeros(128, np.uint8)
    for i, c in case["codes"].items():
        want[i] = c
    assert np.array_equal(q, want), [hex(v) for v in q[:8]]


def _rand_bf16(shape, seed, std=1.0):
    g = torch.Generator().manual_seed(seed)
    t = (torch.randn(shape, generator=g) * std).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _least_exponent(amax: float) -> int:
    """Least integer e with 448 * 2^e >= amax, by exact rational comparison over a range wide
    enough for every finite bf16 amax, then raised to -127."""
    a = Fraction(amax)
    for e in range(-200, 200):
        if Fraction(448) * Fraction(2) ** e >= a:
            return max(e, -127)
    raise AssertionError("no exponent found")


@pytest.mark.parametrize("std,seed", [(1.0, 1), (0.02, 2), (1e-3, 3), (300.0, 4), (1e-20, 5),
                                      (1e30, 6), (1e-37, 7), (1e-39, 8)])
def test_pow2_brute_force(oracle, std, seed):
    x = _rand_bf16((48, 128), seed, std)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    for g in range(x.shape[0]):
        q, s = oracle.quant_group(x[g], pow2=True)
        amax = float(np.max(np.abs(xf[g])))
        if amax == 0.0:
            assert s == 1.0
            continue
        e = _least_exponent(amax)
        assert s == 2.0 ** e
        # exact scaling in binary64, then torch's round-to-nearest-even cast
        t = np.ldexp(xf[g], -e)
        assert np.all(np.abs(t) <= 448.0)
        assert np.array_equal(q, torch_e4m3_encode(t.astype(np.float32)))


def test_pow2_range_of_the_largest_element(oracle):
    """Away from the bottom clamp, amax / s lies in (224, 448]: the largest element's payload
    uses the top binade of E4M3 (or its upper neighbour 448)."""
    x = _rand_bf16((64, 128), 21, 3.0)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    dec = torch_e4m3_decode(np.arange(256, dtype=np.uint8))
    for g in range(64):
        q, s = oracle.quant_group(x[g], pow2=True)
        amax = np.max(np.abs(xf[g]))
        assert 224.0 < amax / s <= 448.0
        i = int(np.argmax(np.abs(xf[g])))
        assert 224.0 <= abs(dec[q[i]]) <= 448.0
        # dequantisation error: half an E4M3 ulp of x / s, times s (x / s is exact)
        t = np.abs(xf[g]) / s
        ulp = np.where(t < 2.0 ** -6, 2.0 ** -9,
                       2.0 ** (np.floor(np.log2(np.maximum(t, 1e-300))) - 3))
        assert np.all(np.abs(dec[q] * s - xf[g]) <= 0.5 * ulp * s)


@pytest.mark.parametrize("j", [-20, -1, 0, 3, 40])
def test_pow2_agrees_with_standard_rule_at_448_times_power_of_two(oracle, j):
    """When amax = 448 * 2^j both rules give s = 2^j and identical bytes (448/amax = 2^-j is
    exact, so the standard rule's product is the same exact scaling)."""
    x = _rand_bf16((8, 128), 30 + j, 50.0)
    xf = bf16_bits_to_f32(x).copy()
    xf = np.clip(xf, -447.0, 447.0)
    xf[:, 5] = 448.0
    xf *= np.float32(2.0 ** j)
    xb = f32_to_bf16_bits(xf)
    for g in range(8):
        q0, s0 = oracle.quant_group(xb[g])
        q1, s1 = oracle.quant_group(xb[g], pow2=True)
        assert s0 == s1 == 2.0 ** j
        assert np.array_equal(q0, q1)


@pytest.mark.parametrize("j", [-60, -7, 1, 5, 60])
def test_pow2_power_of_two_equivariance(oracle, j):
    x = _rand_bf16((8, 128), 11)
    xs = f32_to_bf16_bits(bf16_bits_to_f32(x) * np.float32(2.0 ** j))
    for g in range(8):
        q0, s0 = oracle.quant_group(x[g], pow2=True)
        q1, s1 = oracle.quant_group(xs[g], pow2=True)
        assert np.array_equal(q0, q1)
        assert s1 == s0 * 2.0 ** j


def test_pow2_sign_symmetry_and_zero(oracle):
    x = _rand_bf16((8, 128), 12)
    xn = x ^ np.uint16(0x8000)
    for g in range(8):
        q0, s0 = oracle.quant_group(x[g], pow2=True)
        q1, s1 = oracle.quant_group(xn[g], pow2=True)
        assert s0 == s1 and np.array_equal(q1, q0 ^ np.uint8(0x80))
    z = f32_to_bf16_bits(np.array([0.0, -0.0] * 64, np.float32))
    q, s = oracle.quant_group(z, pow2=True)
    assert s == 1.0 and np.array_equal(q, np.array([0x00, 0x80] * 64, np.uint8))


def test_pow2_layouts(oracle):
    """The act, weight-block and transposed quantisers apply the group rule to the groups their
    layouts define, in power-of-two mode too."""
    x = _rand_bf16((256, 384), 40)
    q, s = oracle.quant_act_1x128(x, pow2=True)
    for r in (0, 77, 255):
        for c in range(3):
            qg, sg = oracle.quant_group(x[r, c * 128:(c + 1) * 128], pow2=True)
            assert np.array_equal(q[r, c * 128:(c + 1) * 128], qg) and s[c, r] == sg
    qt, st = oracle.quant_transpose(x, pow2=True)
    qa, sa = oracle.quant_act_1x128(np.ascontiguousarray(x.T), pow2=True)
    assert np.array_equal(qt, qa) and np.array_equal(st, sa)
    qw, sw = oracle.quant_w_128x128(x, pow2=True)
    for bi in range(2):
        for bj in range(3):
            blk = x[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
            qg, sg = oracle.quant_group(blk.reshape(-1), pow2=True)
            assert sw[bi, bj] == sg
            assert np.array_equal(qw[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128],
                                  qg.reshape(128, 128))
    # power-of-two scales: every scale's significand is exactly 1
    for arr in (s, st, sw):
        m, _ = np.frexp(arr.astype(np.float64))
        assert np.all(m == 0.5)


def test_pow2_gemm_matches_exact_dequantised_product(oracle):
    """With power-of-two scales every dequantised element is exact in binary64, so the GEMM
    oracle on pow2 operands equals a float64 matmul of the dequantised matrices up to the
    matmul's own rounding."""
    M, N, K = 128, 256, 384
    x = _rand_bf16((M, K), 50)
    w = _rand_bf16((N, K), 51, 0.02)
    xq, sx = oracle.quant_act_1x128(x, pow2=True)
    wq, sw = oracle.quant_w_128x128(w, pow2=True)
    y = oracle.gemm_fwd(xq, sx, wq, sw)
    xd = oracle.dequant_act(xq, sx)
    wd = oracle.dequant_w(wq, sw)
    ref = xd @ wd.T
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
