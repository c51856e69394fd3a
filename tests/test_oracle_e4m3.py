"""Pins of the oracle's E4M3 codec to things other than itself: the format definition (hand
golden cases), torch's float8_e4m3fn (a library cast), and structural properties of
round-to-nearest-even (idempotence on representable values, monotonicity, tie behaviour)."""
import numpy as np
import pytest
import torch

from helpers import read_e4m3_hand, torch_e4m3_decode, torch_e4m3_encode


def test_decode_all_codes_match_torch(oracle):
    ours = np.array([oracle.e4m3_decode(c) for c in range(256)])
    lib = torch_e4m3_decode(np.arange(256, dtype=np.uint8))
    nan_ours, nan_lib = np.isnan(ours), np.isnan(lib)
    assert np.array_equal(nan_ours, nan_lib)
    assert sorted(np.nonzero(nan_ours)[0].tolist()) == [0x7F, 0xFF]
    assert np.array_equal(ours[~nan_ours], lib[~nan_lib])
    # signs of zero
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_decode_closed_forms(oracle):
    assert oracle.e4m3_decode(0x7E) == 448.0
    assert oracle.e4m3_decode(0x01) == 2.0 ** -9
    assert oracle.e4m3_decode(0x07) == 7 * 2.0 ** -9
    assert oracle.e4m3_decode(0x08) == 2.0 ** -6
    assert oracle.e4m3_decode(0x38) == 1.0
    assert oracle.e4m3_decode(0xB8) == -1.0
    # every finite code is a multiple of 2^-9 and the values are strictly increasing in code
    pos = [oracle.e4m3_decode(c) for c in range(0x7F)]
    assert all(b > a for a, b in zip(pos, pos[1:]))
    assert all(float(v * 512).is_integer() for v in pos)


@pytest.mark.parametrize("value,code,why", read_e4m3_hand())
def test_encode_hand_golden(oracle, value, code, why):
    assert oracle.e4m3_encode(value) == code, why


def test_encode_idempotent_on_representable(oracle):
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.e4m3_encode(oracle.e4m3_decode(c)) == c


def _sweep_values(seed=0):
    """fp32 inputs in [-448, 448]: every exponent, every top-10 mantissa pattern, several
    low-bit patterns (exact, sticky, all-ones), plus random bit patterns."""
    e = np.arange(0, 136, dtype=np.uint32)  # up to 2^8 binade
    top = np.arange(1024, dtype=np.uint32) << 13
    low = np.array([0, 1, 0x0FFF, 0x1000, 0x1001, 0x1FFF], dtype=np.uint32)
    bits = (e[:, None, None] << 23) | top[None, :, None] | low[None, None, :]
    bits = bits.reshape(-1)
    rng = np.random.default_rng(seed)
    rnd = rng.integers(0, 1 << 31, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    bits = np.concatenate([bits, rnd])
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= 448.0)]
    return np.concatenate([vals, -vals]).astype(np.float32)


def test_encode_matches_torch_sweep(oracle):
    vals = _sweep_values()
    ours = oracle.e4m3_encode_array(vals)
    lib = torch_e4m3_encode(vals)
    bad = np.nonzero(ours != lib)[0]
    assert bad.size == 0, [(float(vals[i]).hex(), hex(ours[i]), hex(lib[i])) for i in bad[:10]]


def test_encode_ties_to_even_at_every_midpoint(oracle):
    # midpoints between consecutive non-negative codes, and one fp32 ulp either side
    for c in range(0x7E):
        lo, hi = oracle.e4m3_decode(c), oracle.e4m3_decode(c + 1)
        mid = np.float32((lo + hi) / 2)  # exact: e4m3 values have few significant bits
        assert float(mid) == (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(float(mid)) == even
        assert oracle.e4m3_encode(float(np.nextafter(mid, np.float32(0)))) == c
        assert oracle.e4m3_encode(float(np.nextafter(mid, np.float32(1e9)))) == c + 1
        # the negative side mirrors with the sign bit
        assert oracle.e4m3_encode(-float(mid)) == even | 0x80


def test_encode_monotone(oracle):
    vals = np.sort(_sweep_values(seed=1))
    codes = oracle.e4m3_encode_array(vals)
    dec = np.array([oracle.e4m3_decode(c) for c in range(256)])[codes]
    assert np.all(np.diff(dec) >= 0)


def test_negative_underflow_keeps_sign(oracle):
    for v in (-1e-30, -(2.0 ** -11), -(2.0 ** -10), -1e-45):
        assert oracle.e4m3_encode(v) == 0x80
    assert oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(0.0) == 0x00
    # torch agrees on the sign of zero for negative underflow
    assert int(torch_e4m3_encode(np.array([-(2.0 ** -11)], np.float32))[0]) == 0x80


def test_bf16_widening_is_exact(oracle):
    for h in (0x0000, 0x8000, 0x3F80, 0x43E0, 0x0001, 0x7F7F, 0xFF7F, 0x3C00):
        f = np.array([h], np.uint16).astype(np.uint32) << 16
        assert np.float32(oracle.bf16_to_f32(h)).view(np.uint32) == f.view(np.uint32)[0]
