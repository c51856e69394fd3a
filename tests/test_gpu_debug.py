"""Debug mode (puro_set_debug / PURO_DEBUG): with the level set, every quantiser and GEMM entry
point scans its inputs on the device first and returns PURO_ERR_INPUT on data outside the
contract, enqueueing nothing more; valid data gives the same bytes as with the checks off; with
the level at 0 nothing is checked. Every kernel here runs on in-bounds data and ends normally:
the bad values are ordinary bf16 / E4M3 / fp32 bit patterns."""
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TINY = 2.0 ** -121  # a nonzero magnitude below 2^-119, exact in bf16


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture
def dbg(puro):
    puro.puro_set_debug(1)
    yield puro
    puro.puro_set_debug(0)


def bf16(rows, cols, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((rows, cols), generator=g).to(torch.bfloat16).to(DEV)


def rejects(fn, *args):
    with pytest.raises(Exception) as e:
        fn(*args)
    torch.cuda.synchronize()
    assert "PURO_ERR_INPUT" in str(e.value), str(e.value)


def test_valid_data_same_bytes(dbg):
    say("debug: valid data through every quantiser and GEMM")
    x, w, dy = bf16(256, 384, 1), bf16(256, 384, 2), bf16(256, 256, 3)
    outs = {}
    for level in (0, 1):
        dbg.puro_set_debug(level)
        xq, sx, xtq, sxt = dbg.puro_quant_dual_1x128(x)
        wq, sw = dbg.puro_quant_w_128x128(w)
        dyq, sdy, dytq, sdyt = dbg.puro_quant_dual_1x128(dy)
        y = dbg.puro_fp8_gemm_fwd(xq, sx, wq, sw)
        dx = dbg.puro_fp8_gemm_dgrad(dyq, sdy, wq, sw)
        dw = dbg.puro_fp8_gemm_wgrad(dytq, sdyt, xtq, sxt)
        a, s = dbg.puro_quant_act_1x128(x)
        t, st = dbg.puro_quant_transpose(x)
        torch.cuda.synchronize()
        outs[level] = [xq, sx, xtq, sxt, wq, sw, y, dx, dw, a, s, t, st]
    assert dbg.puro_debug_level() == 1
    for u, v in zip(outs[0], outs[1]):
        assert torch.equal(u.view(torch.uint8), v.view(torch.uint8))


@pytest.mark.parametrize("pow2", [False, True])
def test_quantisers_reject_non_finite(dbg, pow2):
    sfx = "_pow2" if pow2 else ""
    for bad in (float("nan"), float("inf"), float("-inf")):
        say("debug: quantisers on", bad, "pow2" if pow2 else "")
        x = bf16(256, 256, 4)
        x[130, 200] = bad
        rejects(getattr(dbg, "puro_quant_act_1x128" + sfx), x)
        rejects(getattr(dbg, "puro_quant_transpose" + sfx), x)
        rejects(getattr(dbg, "puro_quant_dual_1x128" + sfx), x)
        rejects(getattr(dbg, "puro_quant_w_128x128" + sfx), x)
        rejects(getattr(dbg, "puro_quant_w_128x128_group" + sfx), [bf16(128, 128, 5), x])


def test_tiny_groups_by_shape(dbg):
    say("debug: tiny groups")
    # one 1x128 row group of tiny values (the rest of its column groups and its block normal)
    x = bf16(256, 256, 6)
    x[3, 128:256] = TINY
    rejects(dbg.puro_quant_act_1x128, x)
    rejects(dbg.puro_quant_dual_1x128, x)
    dbg.puro_quant_transpose(x)    # every column group still holds normal values
    dbg.puro_quant_w_128x128(x)    # so does every block
    # one 128x1 column group of tiny values
    x = bf16(256, 256, 7)
    x[128:256, 5] = TINY
    rejects(dbg.puro_quant_transpose, x)
    rejects(dbg.puro_quant_dual_1x128, x)
    dbg.puro_quant_act_1x128(x)
    dbg.puro_quant_w_128x128(x)
    # one 128x128 block of tiny values
    x = bf16(256, 256, 8)
    x[0:128, 128:256] = TINY
    rejects(dbg.puro_quant_w_128x128, x)
    rejects(dbg.puro_quant_act_1x128, x)
    # an all-zero group is in contract, and the power-of-two rule has no lower bound
    x = bf16(256, 256, 9)
    x[0:128, 128:256] = 0.0
    dbg.puro_quant_w_128x128(x)
    dbg.puro_quant_dual_1x128(x)
    x[0:128, 128:256] = TINY
    dbg.puro_quant_w_128x128_pow2(x)
    dbg.puro_quant_dual_1x128_pow2(x)
    torch.cuda.synchronize()


def test_gemms_reject_nan_codes_and_bad_scales(dbg):
    x, w, dy = bf16(256, 256, 10), bf16(256, 256, 11), bf16(256, 256, 12)
    xq, sx, xtq, sxt = dbg.puro_quant_dual_1x128(x)
    wq, sw = dbg.puro_quant_w_128x128(w)
    dyq, sdy, dytq, sdyt = dbg.puro_quant_dual_1x128(dy)
    for code in (0x7F, 0xFF):
        say("debug: GEMMs with code", hex(code))
        bad = xq.clone()
        bad.view(torch.uint8)[17, 99] = code
        rejects(dbg.puro_fp8_gemm_fwd, bad, sx, wq, sw)
        badw = wq.clone()
        badw.view(torch.uint8)[200, 3] = code
        rejects(dbg.puro_fp8_gemm_dgrad, dyq, sdy, badw, sw)
        badt = xtq.clone()
        badt.view(torch.uint8)[255, 255] = code
        rejects(dbg.puro_fp8_gemm_wgrad, dytq, sdyt, badt, sxt)
    for val in (0.0, -1.0, float("inf"), float("nan")):
        say("debug: GEMMs with scale", val)
        s = sx.clone()
        s.view(-1)[5] = val
        rejects(dbg.puro_fp8_gemm_fwd, xq, s, wq, sw)
        s = sw.clone()
        s.view(-1)[0] = val
        rejects(dbg.puro_fp8_gemm_dgrad, dyq, sdy, wq, s)
        s = sdyt.clone()
        s.view(-1)[-1] = val
        rejects(dbg.puro_fp8_gemm_wgrad, dytq, s, xtq, sxt)
        rejects(dbg.puro_fp8_gemm_fwd_pow2, xq, sx, wq, s.new_full(sw.shape, val))


def test_level_zero_checks_nothing(dbg):
    say("debug: level 0")
    dbg.puro_set_debug(0)
    x = bf16(128, 128, 13)
    x[0, 0] = float("nan")
    dbg.puro_quant_act_1x128(x)  # garbage in, garbage out, but no error
    torch.cuda.synchronize()
