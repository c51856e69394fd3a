"""The composed linear-stack step against the oracle: a 2-layer stack of the Qwen3-1.7B-shaped
linears at M = 8192 tokens, built and launched exactly as the benchmark times it (fused
two-orientation quantisers, X's transposed copy made in the forward pass and consumed by the
weight gradient, intermediates shared across linears and layers), run once as a replay of the
captured step graph. Its device-drawn bf16 inputs are copied to the host and the oracle
recomputes from them:
  - every layer's weight codes and scales, and X's transposed codes and scales (bit-exact);
  - every layer's dW on sampled rows (acceptance tolerance);
  - the shared buffers that survive the step -- the last layer's Y of each output width, the
    first layer's dX of each input width, the first layer's gradient codes of each output
    width, and each linear slot's transposed gradient codes -- bit-exact or within tolerance.
A buffer routed to the wrong linear or layer shows up as a mismatch here even though it would
be bitwise identical across the step's launch orders. Three steps: the amax/448 step the
benchmark times by default, its power-of-two (`--pow2`) twin, and the unfused step
(`--unfused`: separate 1x128 and transposed quantisers instead of the two-orientation one)."""
import sys

import numpy as np
import pytest
import torch

from helpers import bf16_np, gemm_tolerance_violations

pytestmark = pytest.mark.gpu

M = 8192
LAYERS = 2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def sample_rows(total, n, seed):
    rng = np.random.default_rng(seed)
    pick = rng.choice(np.arange(1, total - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, total - 1], pick]))


def same(gpu: torch.Tensor, ref: np.ndarray, what: str):
    g = gpu.cpu().contiguous().numpy()
    assert g.shape == ref.shape, what
    bad = np.argwhere(g.view(np.uint8) != np.ascontiguousarray(ref).view(np.uint8))
    assert bad.size == 0, f"{what}: {len(bad)} byte mismatches, first {bad[:4].tolist()}"


def P(stack):
    """Scale rule of the stack under test (the _pow2 step for the pow2 parameter)."""
    return stack.test_pow2


def within(gpu: np.ndarray, ref: np.ndarray, what: str):
    nbad, worst = gemm_tolerance_violations(gpu, ref)
    assert nbad == 0, f"{what}: {nbad} out of tolerance (worst err/bound {worst:.3g})"
    say("  ", what, "worst err/bound", round(worst, 4))


@pytest.fixture(scope="module", params=[(True, False), (True, True), (False, False)],
                ids=["amax448", "pow2", "unfused"])
def stepped(request):
    import bench
    fused, pow2 = request.param
    say("stack parity: building", LAYERS, "layers at M =", M, "pow2" if pow2 else "",
        "" if fused else "unfused")
    main = torch.cuda.Stream()
    with torch.cuda.stream(main):
        stack = bench.Stack(LAYERS, M, fused=fused, pow2=pow2)
        stack.capture(overlap=False)
        stack.replay()
    torch.cuda.synchronize()
    say("stack parity: step replayed")
    stack.test_pow2 = pow2
    return stack


def test_per_layer_weights_and_transposed_x(stepped, oracle):
    for rec in stepped.linears:
        what = f"layer {rec['layer']} {rec['name']}"
        say("stack parity:", what, "weight and X^T codes")
        wq, sw = oracle.quant_w_128x128(bf16_np(rec["w"].cpu()), pow2=P(stepped))
        same(rec["wq"], wq, what + " wq")
        same(rec["sw"], sw, what + " sw")
        if "xtq" not in rec:
            continue  # unfused step: X's transposed copy is a shared buffer (checked below)
        xtq, sxt = oracle.quant_transpose(bf16_np(rec["x"].cpu()), pow2=P(stepped))
        same(rec["xtq"], xtq, what + " xtq")
        same(rec["sxt"], sxt, what + " sxt")


def test_per_layer_weight_gradients(stepped, oracle):
    for rec in stepped.linears:
        what = f"layer {rec['layer']} {rec['name']} dW"
        say("stack parity:", what)
        dytq, sdyt = oracle.quant_transpose(bf16_np(rec["dy"].cpu()), pow2=P(stepped))
        xtq, sxt = oracle.quant_transpose(bf16_np(rec["x"].cpu()), pow2=P(stepped))
        rows = sample_rows(rec["N"], 8, 31 * rec["layer"] + rec["li"])
        ref = oracle.gemm_wgrad(dytq, sdyt, xtq, sxt, rows=rows)
        got = rec["dw"][torch.as_tensor(rows).cuda()].cpu().numpy().astype(np.float64)
        within(got, ref, what)


def _last(stack, layer, name):
    return next(r for r in stack.linears if r["layer"] == layer and r["name"] == name)


def test_surviving_shared_buffers(stepped, oracle):
    sh = stepped.shared
    last, first = LAYERS - 1, 0
    rows = sample_rows(M, 16, 7)
    rsel = torch.as_tensor(rows).cuda()
    # forward: layer order qkv, o, gate_up, down; the last layer's last writer of each buffer
    for name, key_y in (("qkv", ("y", M, 4096)), ("gate_up", ("y", M, 12288)),
                        ("down", ("y", M, 2048))):
        rec = _last(stepped, last, name)
        xq, sx = oracle.quant_act_1x128(bf16_np(rec["x"].cpu()), pow2=P(stepped))
        wq, sw = oracle.quant_w_128x128(bf16_np(rec["w"].cpu()), pow2=P(stepped))
        say("stack parity: Y of layer", last, name)
        ref = oracle.gemm_fwd(xq, sx, wq, sw, rows=rows)
        within(sh[key_y][rsel].float().cpu().numpy().astype(np.float64), ref,
               f"Y layer {last} {name}")
        if name in ("gate_up", "down"):  # last writers of xq for K = 2048 and K = 6144
            same(sh[("xq", M, rec["K"])], xq, f"xq layer {last} {name}")
            same(sh[("sx", M, rec["K"])], sx, f"sx layer {last} {name}")
    # backward: layer order down, gate_up, o, qkv from the last layer to the first
    for name in ("qkv", "o", "gate_up", "down"):
        rec = _last(stepped, first, name)
        dy = bf16_np(rec["dy"].cpu())
        dytq, sdyt = oracle.quant_transpose(dy, pow2=P(stepped))
        same(sh[("dytq", rec["li"])], dytq, f"dytq slot {name} (layer {first})")
        same(sh[("sdyt", rec["li"])], sdyt, f"sdyt slot {name} (layer {first})")
        if name == "down":
            continue  # its dY codes are overwritten by o's (same width)
        dyq, sdy = oracle.quant_act_1x128(dy, pow2=P(stepped))
        same(sh[("dyq", M, rec["N"])], dyq, f"dyq layer {first} {name}")
        same(sh[("sdy", M, rec["N"])], sdy, f"sdy layer {first} {name}")
    for name in ("qkv", "down"):  # last writers of X's shared transposed copy (unfused step)
        rec = _last(stepped, first, name)
        if ("xtq", M, rec["K"]) in sh:
            xtq, sxt = oracle.quant_transpose(bf16_np(rec["x"].cpu()), pow2=P(stepped))
            same(sh[("xtq", M, rec["K"])], xtq, f"xtq layer {first} {name}")
            same(sh[("sxt", M, rec["K"])], sxt, f"sxt layer {first} {name}")
    for name in ("qkv", "down"):  # last writers of dX for K = 2048 and K = 6144
        rec = _last(stepped, first, name)
        dyq, sdy = oracle.quant_act_1x128(bf16_np(rec["dy"].cpu()), pow2=P(stepped))
        wq, sw = oracle.quant_w_128x128(bf16_np(rec["w"].cpu()), pow2=P(stepped))
        say("stack parity: dX of layer", first, name)
        ref = oracle.gemm_dgrad(dyq, sdy, wq, sw, rows=rows)
        within(sh[("dx", M, rec["K"])][rsel].float().cpu().numpy().astype(np.float64), ref,
               f"dX layer {first} {name}")
