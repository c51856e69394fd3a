"""GPU parity of the three GEMMs (and their power-of-two-scale variants) against the oracle,
element by element, under the acceptance
rule |gpu - oracle| <= 2^-7 |oracle| + 1e-3 rms(oracle). The oracle quantises the same bf16
inputs itself (its quantised operands are bit-identical to the GPU's, which the quantiser
tests check separately) and computes exact chunk products with double accumulation.

Small shapes are compared in full; the full-size layer shapes (M = 4096, 8192, 16384) on
seeded samples of output rows (all columns), which the oracle computes one row at a time."""
import sys

import numpy as np
import pytest
import torch

from blockwise_fp8_gemm_x128_amd import synth
from helpers import bf16_np, gemm_tolerance_violations

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_to_np64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def sample_rows(total, n, seed):
    if n >= total:
        return np.arange(total)
    rng = np.random.default_rng(seed)
    pick = rng.choice(np.arange(1, total - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, total - 1], pick]))


def check(gpu, ref, what):
    nbad, worst = gemm_tolerance_violations(gpu, ref)
    assert nbad == 0, f"{what}: {nbad} elements out of tolerance (worst err/bound {worst:.3g})"
    return worst


def fn(puro, name, pow2):
    return getattr(puro, name + ("_pow2" if pow2 else ""))


def run_fwd(puro, oracle, x, w, rows=None, what="fwd", pow2=False):
    M, K = x.shape
    N = w.shape[0]
    say(what, "fwd M,N,K =", M, N, K, "pow2" if pow2 else "")
    xq, sx = fn(puro, "puro_quant_act_1x128", pow2)(x.cuda())
    wq, sw = fn(puro, "puro_quant_w_128x128", pow2)(w.cuda())
    y = fn(puro, "puro_fp8_gemm_fwd", pow2)(xq, sx, wq, sw)
    torch.cuda.synchronize()
    oxq, osx = oracle.quant_act_1x128(bf16_np(x), pow2=pow2)
    owq, osw = oracle.quant_w_128x128(bf16_np(w), pow2=pow2)
    ref = oracle.gemm_fwd(oxq, osx, owq, osw, rows=rows)
    got = bf16_to_np64(y if rows is None else y[torch.as_tensor(rows).cuda()])
    return check(got, ref, what)


def run_dgrad(puro, oracle, dy, w, rows=None, what="dgrad", pow2=False):
    M, N = dy.shape
    K = w.shape[1]
    say(what, "dgrad M,N,K =", M, N, K, "pow2" if pow2 else "")
    dyq, sdy = fn(puro, "puro_quant_act_1x128", pow2)(dy.cuda())
    wq, sw = fn(puro, "puro_quant_w_128x128", pow2)(w.cuda())
    dx = fn(puro, "puro_fp8_gemm_dgrad", pow2)(dyq, sdy, wq, sw)
    torch.cuda.synchronize()
    odyq, osdy = oracle.quant_act_1x128(bf16_np(dy), pow2=pow2)
    owq, osw = oracle.quant_w_128x128(bf16_np(w), pow2=pow2)
    ref = oracle.gemm_dgrad(odyq, osdy, owq, osw, rows=rows)
    got = bf16_to_np64(dx if rows is None else dx[torch.as_tensor(rows).cuda()])
    return check(got, ref, what)


def run_wgrad(puro, oracle, dy, x, rows=None, what="wgrad", dw0=None, pow2=False):
    M, N = dy.shape
    K = x.shape[1]
    say(what, "wgrad M,N,K =", M, N, K, "pow2" if pow2 else "")
    dytq, sdyt = fn(puro, "puro_quant_transpose", pow2)(dy.cuda())
    xtq, sxt = fn(puro, "puro_quant_transpose", pow2)(x.cuda())
    dw_in = None if dw0 is None else dw0.clone().cuda()
    dw = fn(puro, "puro_fp8_gemm_wgrad", pow2)(dytq, sdyt, xtq, sxt, dw=dw_in,
                                               accumulate=dw0 is not None)
    torch.cuda.synchronize()
    odytq, osdyt = oracle.quant_transpose(bf16_np(dy), pow2=pow2)
    oxtq, osxt = oracle.quant_transpose(bf16_np(x), pow2=pow2)
    ref = oracle.gemm_wgrad(odytq, osdyt, oxtq, osxt, rows=rows)
    if dw0 is not None:
        base = dw0.numpy().astype(np.float64)
        ref = ref + (base if rows is None else base[rows])
    got = dw.cpu().numpy().astype(np.float64)
    if rows is not None:
        got = got[rows]
    return check(got, ref, what)


@pytest.mark.parametrize("pow2", [False, True])
def test_tiny_forward(puro, oracle, pow2):
    x, w = synth.tiny_forward_inputs()
    run_fwd(puro, oracle, x, w, what="tiny 256^3", pow2=pow2)


SMALL = [(128, 128, 128), (384, 640, 384), (256, 384, 1152), (640, 256, 256), (1024, 768, 512)]


@pytest.mark.parametrize("M,N,K", SMALL)
@pytest.mark.parametrize("pow2", [False, True])
def test_small_all_three(puro, oracle, M, N, K, pow2):
    seed = M * 7 + N * 3 + K
    x = synth.randn_bf16((M, K), 1.0, seed)
    w = synth.randn_bf16((N, K), 0.02, seed + 1)
    dy = synth.randn_bf16((M, N), 1e-3, seed + 2)
    run_fwd(puro, oracle, x, w, what=f"fwd {M}x{N}x{K}", pow2=pow2)
    run_dgrad(puro, oracle, dy, w, what=f"dgrad {M}x{N}x{K}", pow2=pow2)
    run_wgrad(puro, oracle, dy, x, what=f"wgrad {M}x{N}x{K}", pow2=pow2)


@pytest.mark.parametrize("pow2", [False, True])
def test_wgrad_accumulate(puro, oracle, pow2):
    M, N, K = 512, 256, 384
    x = synth.randn_bf16((M, K), 1.0, 71)
    dy = synth.randn_bf16((M, N), 1e-3, 72)
    dw0 = torch.randn((N, K), generator=torch.Generator().manual_seed(73)) * 1e-2
    run_wgrad(puro, oracle, dy, x, dw0=dw0, what="wgrad accumulate", pow2=pow2)


# Weight-gradient outputs chosen so that each tile shape the library picks from is used on a
# 256-CU part: the split-reduction 128x128 tile (a 128 x 384 output; a 2048 x 2048 output over
# 9 chunks, so one group multiplies out one chunk more than the other), the four-wave 128x128
# tile (a 4096 x 2048 output: one round of two blocks per CU), 256x192 (a 2048 x 4608 output:
# one round instead of two), 192x256 (a 12288 x 2048 output: two rounds of 512 tiles), 256x256
# (a 4096 x 4096 output: one round; its fp32 epilogue goes through LDS in two passes); sampled
# output rows, overwrite and accumulate.
WGRAD_SHAPES = [(256, 128, 384), (1152, 2048, 2048), (256, 4096, 2048), (256, 2048, 4608),
                (256, 12288, 2048), (256, 4096, 4096)]


@pytest.mark.parametrize("M,N,K", WGRAD_SHAPES)
@pytest.mark.parametrize("acc,pow2", [(False, False), (True, False), (True, True)])
def test_wgrad_tile_shapes(puro, oracle, M, N, K, acc, pow2):
    x = synth.randn_bf16((M, K), 1.0, 101 + N + K)
    dy = synth.randn_bf16((M, N), 1e-3, 102 + N + K)
    dw0 = (torch.randn((N, K), generator=torch.Generator().manual_seed(103)) * 1e-2
           if acc else None)
    run_wgrad(puro, oracle, dy, x, rows=sample_rows(N, 24, N + K), dw0=dw0,
              what=f"wgrad tiles {M}x{N}x{K} acc={acc}", pow2=pow2)


@pytest.mark.parametrize("pow2", [False, True])
def test_big_tiles_with_ragged_edge(puro, oracle, pow2):
    # 16512 = 64.5 x 256 rows and 1152 = 4.5 x 256 columns: enough 256x256 tiles for the
    # big-tile kernels, whose last tile row and last tile column are half outside the output
    # (there half of the waves store nothing); the sampled rows include the half tile row.
    M, N, K = 16512, 1152, 256
    x = synth.randn_bf16((M, K), 1.0, 111)
    w = synth.randn_bf16((N, K), 0.02, 112)
    dy = synth.randn_bf16((M, N), 1e-3, 113)
    rows = np.unique(np.concatenate([sample_rows(M, 16, 114), np.arange(M - 130, M)]))
    run_fwd(puro, oracle, x, w, rows=rows, what="fwd ragged big tiles", pow2=pow2)
    w2 = synth.randn_bf16((N, 1152), 0.02, 115)
    run_dgrad(puro, oracle, dy, w2, rows=rows, what="dgrad ragged big tiles", pow2=pow2)


@pytest.mark.parametrize("pow2", [False, True])
def test_big_tile_edges_write_nothing_outside(puro, pow2):
    # The ragged 256x256 forward and data-gradient outputs are written into the front of a
    # buffer followed by 256 sentinel rows: the waves of the half-outside tiles (last tile row
    # and last tile column) must store nothing, so the sentinels survive, and the output equals
    # that of a call into a buffer of its own.
    M, N, K = 16512, 1152, 256
    sentinel = 0x7FC1  # a bf16 NaN the kernels never produce
    x = synth.randn_bf16((M, K), 1.0, 121).cuda()
    w = synth.randn_bf16((N, K), 0.02, 122).cuda()
    dy = synth.randn_bf16((M, N), 1e-3, 123).cuda()
    w2 = synth.randn_bf16((N, 1152), 0.02, 124).cuda()
    xq, sx = fn(puro, "puro_quant_act_1x128", pow2)(x)
    wq, sw = fn(puro, "puro_quant_w_128x128", pow2)(w)
    dyq, sdy = fn(puro, "puro_quant_act_1x128", pow2)(dy)
    w2q, sw2 = fn(puro, "puro_quant_w_128x128", pow2)(w2)
    for what, call, cols in (
            ("fwd", lambda out: fn(puro, "puro_fp8_gemm_fwd", pow2)(xq, sx, wq, sw, out), N),
            ("dgrad", lambda out: fn(puro, "puro_fp8_gemm_dgrad", pow2)(dyq, sdy, w2q, sw2, out),
             1152)):
        say("edges", what, "M, cols =", M, cols, "pow2" if pow2 else "")
        buf = torch.empty((M + 256, cols), dtype=torch.bfloat16, device="cuda")
        buf.view(torch.int16).fill_(sentinel)
        call(buf[:M])
        ref = call(None)
        torch.cuda.synchronize()
        tail = buf[M:].view(torch.int16)
        assert bool((tail == sentinel).all()), f"{what}: a store landed past the output"
        assert torch.equal(buf[:M].view(torch.int16), ref.view(torch.int16)), what


# The 8-wave tiles alternate each chunk's DMA between the two halves of the block by chunk
# parity, and the last chunk of an odd count takes its own path through the pipeline: odd
# chunk counts (1, 3, 9) on shapes that use the 256x256 (forward, data gradient) and 256x192
# (weight gradient, 2048 x 6144 output) tiles.
@pytest.mark.parametrize("chunks", [1, 3, 9])
@pytest.mark.parametrize("pow2", [False, True])
def test_big_tiles_odd_chunks(puro, oracle, chunks, pow2):
    R = 128 * chunks
    seed = 130 + chunks
    x = synth.randn_bf16((4096, R), 1.0, seed)
    w = synth.randn_bf16((4096, R), 0.02, seed + 1)
    run_fwd(puro, oracle, x, w, rows=sample_rows(4096, 12, seed), what=f"fwd {chunks} chunks",
            pow2=pow2)
    dy = synth.randn_bf16((4096, R), 1e-3, seed + 2)
    w2 = synth.randn_bf16((R, 4096), 0.02, seed + 3)
    run_dgrad(puro, oracle, dy, w2, rows=sample_rows(4096, 12, seed + 4),
              what=f"dgrad {chunks} chunks", pow2=pow2)
    xw = synth.randn_bf16((R, 6144), 1.0, seed + 5)
    dyw = synth.randn_bf16((R, 2048), 1e-3, seed + 6)
    run_wgrad(puro, oracle, dyw, xw, rows=sample_rows(2048, 8, seed + 7),
              what=f"wgrad {chunks} chunks", pow2=pow2)


# Seeded random shapes (every dimension a multiple of 128): small ones, which the 128x128 and
# split-reduction kernels take, and large outputs with short reductions, which the 8-wave
# kernels take; all three GEMMs against the oracle on sampled rows, both scale rules.
def _random_shapes():
    rng = np.random.default_rng(2024)
    small = [tuple(int(v) * 128 for v in rng.integers(1, 17, size=3)) for _ in range(5)]
    large = [(int(rng.integers(24, 65)) * 128, int(rng.integers(24, 65)) * 128,
              int(rng.integers(1, 10)) * 128) for _ in range(4)]
    return small + large


@pytest.mark.parametrize("M,N,K", _random_shapes())
@pytest.mark.parametrize("pow2", [False, True])
def test_random_shapes(puro, oracle, M, N, K, pow2):
    seed = 7 * M + 5 * N + 3 * K + int(pow2)
    x = synth.randn_bf16((M, K), 1.0, seed)
    w = synth.randn_bf16((N, K), 0.02, seed + 1)
    dy = synth.randn_bf16((M, N), 1e-3, seed + 2)
    run_fwd(puro, oracle, x, w, rows=sample_rows(M, 10, seed), what="random fwd", pow2=pow2)
    run_dgrad(puro, oracle, dy, w, rows=sample_rows(M, 10, seed + 3), what="random dgrad",
              pow2=pow2)
    run_wgrad(puro, oracle, dy, x, rows=sample_rows(N, 8, seed + 4), what="random wgrad",
              pow2=pow2)


def test_zero_reduction(puro):
    say("zero reduction")
    xq = torch.empty((256, 0), dtype=torch.uint8, device="cuda")
    sx = torch.empty((0, 256), dtype=torch.float32, device="cuda")
    wq = torch.empty((384, 0), dtype=torch.uint8, device="cuda")
    sw = torch.empty((3, 0), dtype=torch.float32, device="cuda")
    y = torch.full((256, 384), 7.0, dtype=torch.bfloat16, device="cuda")
    puro.puro_fp8_gemm_fwd(xq, sx, wq, sw, y=y)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0
    # wgrad with M = 0: overwrite gives zeros, accumulate leaves dW unchanged
    dytq = torch.empty((256, 0), dtype=torch.uint8, device="cuda")
    sdyt = torch.empty((0, 256), dtype=torch.float32, device="cuda")
    xtq = torch.empty((128, 0), dtype=torch.uint8, device="cuda")
    sxt = torch.empty((0, 128), dtype=torch.float32, device="cuda")
    dw = torch.full((256, 128), 3.0, dtype=torch.float32, device="cuda")
    puro.puro_fp8_gemm_wgrad(dytq, sdyt, xtq, sxt, dw=dw, accumulate=True)
    torch.cuda.synchronize()
    assert torch.all(dw == 3.0)
    puro.puro_fp8_gemm_wgrad(dytq, sdyt, xtq, sxt, dw=dw, accumulate=False)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dw).item() == 0


@pytest.mark.parametrize("pow2", [False, True])
def test_zero_groups_and_scale_isolation(puro, oracle, pow2):
    # rows with all-zero 1x128 tiles and one outlier block: exercises the s = 1 path inside GEMMs
    M, N, K = 384, 256, 512
    x = synth.randn_bf16((M, K), 1.0, 81).float()
    x[5, 128:256] = 0
    x[100:228, 384:] = 0
    x[7, :] *= 1000.0
    x = x.to(torch.bfloat16)
    w = synth.randn_bf16((N, K), 0.02, 82).float()
    w[128:, 256:384] *= 50.0
    w = w.to(torch.bfloat16)
    run_fwd(puro, oracle, x, w, what="fwd zero/outlier", pow2=pow2)


def test_deterministic(puro):
    M, N, K = 512, 512, 1024
    x = synth.randn_bf16((M, K), 1.0, 91).cuda()
    w = synth.randn_bf16((N, K), 0.02, 92).cuda()
    xq, sx = puro.puro_quant_act_1x128(x)
    wq, sw = puro.puro_quant_w_128x128(w)
    y1 = puro.puro_fp8_gemm_fwd(xq, sx, wq, sw)
    y2 = puro.puro_fp8_gemm_fwd(xq, sx, wq, sw)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("li", range(4))
def test_layer_forward_m4096(puro, oracle, li):
    name, K, N = synth.LINEARS[li]
    x, w, _ = synth.linear_inputs(1, li, 4096, K, N)
    run_fwd(puro, oracle, x, w, rows=sample_rows(4096, 48, li), what=f"{name} fwd M=4096")


@pytest.mark.parametrize("M", [8192, 16384])
@pytest.mark.parametrize("li", range(4))
def test_layer_fwd_bwd(puro, oracle, M, li):
    name, K, N = synth.LINEARS[li]
    config = 2 if M == 16384 else 4
    x, w, dy = synth.linear_inputs(config, li, M, K, N)
    run_fwd(puro, oracle, x, w, rows=sample_rows(M, 24, li), what=f"{name} fwd M={M}")
    run_dgrad(puro, oracle, dy, w, rows=sample_rows(M, 24, li + 10), what=f"{name} dgrad M={M}")
    run_wgrad(puro, oracle, dy, x, rows=sample_rows(N, 16, li + 20), what=f"{name} wgrad M={M}")


@pytest.mark.parametrize("pow2", [False, True])
def test_outlier_fwd_bwd(puro, oracle, pow2):
    x, w, dy, _ = synth.outlier_inputs()
    M, K = x.shape
    N = w.shape[0]
    run_fwd(puro, oracle, x, w, rows=sample_rows(M, 32, 1), what="outlier fwd", pow2=pow2)
    run_dgrad(puro, oracle, dy, w, rows=sample_rows(M, 32, 2), what="outlier dgrad", pow2=pow2)
    run_wgrad(puro, oracle, dy, x, rows=sample_rows(N, 16, 3), what="outlier wgrad", pow2=pow2)


@pytest.mark.parametrize("li", range(4))
def test_layer_fwd_bwd_pow2(puro, oracle, li):
    name, K, N = synth.LINEARS[li]
    M = 8192
    x, w, dy = synth.linear_inputs(4, li, M, K, N)
    run_fwd(puro, oracle, x, w, rows=sample_rows(M, 24, li), what=f"{name} fwd M={M}", pow2=True)
    run_dgrad(puro, oracle, dy, w, rows=sample_rows(M, 24, li + 10), what=f"{name} dgrad M={M}",
              pow2=True)
    run_wgrad(puro, oracle, dy, x, rows=sample_rows(N, 16, li + 20), what=f"{name} wgrad M={M}",
              pow2=True)


def test_pow2_gemm_reads_only_scale_exponents(puro):
    """The _pow2 GEMMs take each scale as an 8-bit biased exponent: scales given as 1.5 * 2^e
    act as 2^e (documented behaviour for scales that did not come from the _pow2 quantisers)."""
    say("pow2 exponent-only scales")
    M, N, K = 256, 256, 256
    x = synth.randn_bf16((M, K), 1.0, 121).cuda()
    w = synth.randn_bf16((N, K), 0.02, 122).cuda()
    xq, sx = puro.puro_quant_act_1x128_pow2(x)
    wq, sw = puro.puro_quant_w_128x128_pow2(w)
    y1 = puro.puro_fp8_gemm_fwd_pow2(xq, sx, wq, sw)
    y2 = puro.puro_fp8_gemm_fwd_pow2(xq, sx * 1.5, wq, sw * 1.75)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


# Every element of one full-size output per big-tile kernel, for both scale rules: the 256x256
# forward (qkv at M = 4096: one round of 256 tiles), the 256x256 data gradient (down at
# M = 4096: 384 tiles), and every weight-gradient tile shape the model uses: 256x256
# (4096 x 4096), 192x256 (12288 x 2048), 256x192 (2048 x 6144), the 4-wave 128x128 (qkv,
# 4096 x 2048) and the split-reduction 128x128 (o, 2048 x 2048), over a 512-token reduction.
@pytest.mark.parametrize("p2", [False, True], ids=["amax448", "pow2"])
def test_big_tiles_full_output_fwd(puro, oracle, p2):
    name, K, N = synth.LINEARS[0]
    x, w, _ = synth.linear_inputs(1, 0, 4096, K, N)
    run_fwd(puro, oracle, x, w, what=f"{name} fwd M=4096 every element", pow2=p2)


@pytest.mark.parametrize("p2", [False, True], ids=["amax448", "pow2"])
def test_big_tiles_full_output_dgrad(puro, oracle, p2):
    name, K, N = synth.LINEARS[3]
    _, w, dy = synth.linear_inputs(1, 3, 4096, K, N)
    run_dgrad(puro, oracle, dy, w, what=f"{name} dgrad M=4096 every element", pow2=p2)


@pytest.mark.parametrize("p2", [False, True], ids=["amax448", "pow2"])
@pytest.mark.parametrize("N,K", [(4096, 4096), (12288, 2048), (2048, 6144), (4096, 2048),
                                 (2048, 2048)])
def test_big_tiles_full_output_wgrad(puro, oracle, N, K, p2):
    M = 512
    x = synth.randn_bf16((M, K), 1.0, 141 + K)
    dy = synth.randn_bf16((M, N), 1e-3, 142 + N)
    run_wgrad(puro, oracle, dy, x, what=f"wgrad {N}x{K} (M={M}) every element", pow2=p2)
