"""Pins of the oracle's quantisers: hand-derived golden groups, the invariants the contract
fixes (amax maps to +-448, |q| <= 448, error bound, all-zero groups), exact equivariances
(powers of two, sign, permutation), scale isolation, and the layout identities between the
three quantisers."""
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


@pytest.mark.parametrize("case", read_quant_hand(), ids=lambda c: c["name"])
def test_quant_group_hand_golden(oracle, case):
    x = _group_from_case(case)
    q, s = oracle.quant_group(x)
    assert np.float32(s).view(np.uint32) == np.float32(case["scale"]).view(np.uint32)
    want = np.zeros(128, np.uint8)
    for i, c in case["codes"].items():
        want[i] = c
    assert np.array_equal(q, want), [hex(v) for v in q[:8]]


def _rand_bf16(shape, seed, std=1.0):
    g = torch.Generator().manual_seed(seed)
    t = (torch.randn(shape, generator=g) * std).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _nearest_f32_is(q: Fraction, f: float) -> bool:
    """True iff binary32 f is a correctly rounded (nearest) representation of rational q."""
    f32 = np.float32(f)
    lo = np.nextafter(f32, np.float32(-np.inf))
    hi = np.nextafter(f32, np.float32(np.inf))
    d = abs(Fraction(float(f32)) - q)
    return d <= abs(Fraction(float(lo)) - q) and d <= abs(Fraction(float(hi)) - q)


@pytest.mark.parametrize("std,seed", [(1.0, 1), (0.02, 2), (1e-3, 3), (300.0, 4), (1e-20, 5)])
def test_group_invariants(oracle, std, seed):
    x = _rand_bf16((64, 128), seed, std)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    dec = torch_e4m3_decode(np.arange(256, dtype=np.uint8))
    for g in range(x.shape[0]):
        q, s = oracle.quant_group(x[g])
        amax = np.max(np.abs(xf[g]))
        # scale is the correctly rounded fp32 of amax / 448
        assert _nearest_f32_is(Fraction(float(amax)) / 448, s)
        v = dec[q]
        assert not np.any(np.isnan(v)) and np.all(np.abs(v) <= 448.0)
        # every element of maximal magnitude encodes to +-448 exactly
        at_max = np.abs(xf[g]) == amax
        assert np.all(np.abs(v[at_max]) == 448.0)
        assert np.all((q[at_max] & 0x7F) == 0x7E)
        # dequantisation error: half an E4M3 ulp of x*r, times s, plus fp32 slack
        r = 448.0 / amax
        t = np.abs(xf[g]) * r
        ulp = np.where(t < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(t, 1e-300))) - 3))
        err = np.abs(v * s - xf[g])
        assert np.all(err <= 0.5 * ulp * s + 2.0 ** -21 * np.abs(xf[g]))
        # signs are kept (zero codes carry the input's sign)
        assert np.array_equal(np.signbit(v), np.signbit(xf[g]))


def test_all_zero_group(oracle):
    x = f32_to_bf16_bits(np.array([0.0, -0.0] * 64, np.float32))
    q, s = oracle.quant_group(x)
    assert s == 1.0
    assert np.array_equal(q, np.array([0x00, 0x80] * 64, np.uint8))


@pytest.mark.parametrize("j", [-60, -7, 1, 5, 60])
def test_power_of_two_equivariance(oracle, j):
    x = _rand_bf16((8, 128), 11)
    xs = f32_to_bf16_bits(bf16_bits_to_f32(x) * np.float32(2.0 ** j))
    for g in range(8):
        q0, s0 = oracle.quant_group(x[g])
        q1, s1 = oracle.quant_group(xs[g])
        assert np.array_equal(q0, q1)
        assert s1 == s0 * 2.0 ** j


def test_sign_symmetry(oracle):
    x = _rand_bf16((8, 128), 12)
    xn = x ^ np.uint16(0x8000)
    for g in range(8):
        q0, s0 = oracle.quant_group(x[g])
        q1, s1 = oracle.quant_group(xn[g])
        assert s0 == s1
        assert np.array_equal(q1, q0 ^ np.uint8(0x80))


def test_permutation_equivariance(oracle):
    x = _rand_bf16((4, 128), 13)
    rng = np.random.default_rng(0)
    for g in range(4):
        perm = rng.permutation(128)
        q0, s0 = oracle.quant_group(x[g])
        q1, s1 = oracle.quant_group(x[g][perm])
        assert s0 == s1 and np.array_equal(q1, q0[perm])


def test_act_layout_and_scale_isolation(oracle):
    x = _rand_bf16((96, 384), 14)
    q, s = oracle.quant_act_1x128(x)
    assert q.shape == (96, 384) and s.shape == (3, 96)
    for r in (0, 5, 95):
        for c in range(3):
            qg, sg = oracle.quant_group(x[r, c * 128:(c + 1) * 128])
            assert np.array_equal(q[r, c * 128:(c + 1) * 128], qg) and s[c, r] == sg
    # perturb one group by a large outlier: only that group's bytes and scale change
    x2 = x.copy()
    x2[7, 130] = f32_to_bf16_bits(np.array([8192.0], np.float32))[0]
    q2, s2 = oracle.quant_act_1x128(x2)
    changed_q = np.argwhere(q2 != q)
    assert changed_q.size and np.all(changed_q[:, 0] == 7) and np.all(changed_q[:, 1] // 128 == 1)
    changed_s = np.argwhere(s2 != s)
    assert changed_s.tolist() == [[1, 7]]


def test_weight_blocks(oracle):
    w = _rand_bf16((256, 384), 15, std=0.02)
    q, s = oracle.quant_w_128x128(w)
    assert s.shape == (2, 3)
    for bi in range(2):
        for bj in range(3):
            blk = w[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
            qg, sg = oracle.quant_group(blk.reshape(-1))
            assert s[bi, bj] == sg
            assert np.array_equal(q[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128],
                                  qg.reshape(128, 128))
    # a x50 block changes only its own scale; codes of a block are invariant to a power-of-two
    w2 = f32_to_bf16_bits(bf16_bits_to_f32(w).copy())
    w2[128:256, 0:128] = f32_to_bf16_bits(bf16_bits_to_f32(w[128:256, 0:128]) * np.float32(64.0))
    q2, s2 = oracle.quant_w_128x128(w2)
    assert np.array_equal(q2, q)
    assert s2[1, 0] == s[1, 0] * 64 and np.array_equal(np.delete(s2.ravel(), 3), np.delete(s.ravel(), 3))


def test_transpose_equals_act_of_transpose(oracle):
    x = _rand_bf16((384, 256), 16)
    qt, st = oracle.quant_transpose(x)
    qa, sa = oracle.quant_act_1x128(np.ascontiguousarray(x.T))
    assert np.array_equal(qt, qa)
    assert np.array_equal(st, sa)


@pytest.mark.parametrize("std,seed", [(1.0, 21), (0.02, 22), (1e-3, 23)])
def test_payload_against_numpy_and_torch_cast(oracle, std, seed):
    # The standard rule rebuilt from library arithmetic on 16384 seeded groups: numpy's fp32
    # division and multiply (each one correctly rounded operation) for the factor and the scaled
    # value, torch's float8_e4m3fn cast for the encoding. A few percent of N(0,1) groups hold an
    # element whose exact scaled value is an E4M3 midpoint, where a different factor rule
    # (x/s, x * fl32(1/s)) would give another byte.
    x = _rand_bf16((16384, 128), seed, std)
    xf = bf16_bits_to_f32(x)
    amax = np.max(np.abs(xf), axis=1, keepdims=True)
    r = np.where(amax > 0, np.float32(448.0) / np.where(amax > 0, amax, 1), np.float32(1.0))
    t = np.clip((xf * r.astype(np.float32)).astype(np.float32), -448.0, 448.0)
    want = torch_e4m3_encode(t)
    q, s = oracle.quant_act_1x128(x)
    assert np.array_equal(q, want)
    assert np.array_equal(s[0], np.where(amax[:, 0] > 0, amax[:, 0] / np.float32(448.0), 1.0).astype(np.float32))
    # the midpoint cases are present in this sample: the alternatives differ somewhere
    s32 = (amax / np.float32(448.0)).astype(np.float32)
    alt_d = torch_e4m3_encode(np.clip((xf / s32).astype(np.float32), -448, 448))
    alt_i = torch_e4m3_encode(np.clip((xf * (np.float32(1.0) / s32)).astype(np.float32), -448, 448))
    assert np.any(alt_d != want) and np.any(alt_i != want)
