"""Seeded synthetic inputs for the linear-layer GEMM path (no method arithmetic lives here).

Shapes follow a Qwen3-1.7B-shaped transformer with untied embeddings (the model named in the
PuRo-2B news post, jj-blog.pages.dev, driver-hack section, training-recipe paragraph: Qwen3-1.7B
configuration, sequence length 4096): hidden 2048, 16 query + 2x8 key/value heads of 128,
MLP width 6144 (gate and up fused), 28 layers. The pages train on web/code/math text; here every
tensor is seeded Gaussian noise of the stated std (bf16 by round-to-nearest-even from fp32).

Both the GPU path and the CPU oracle are fed from these generators; nothing here quantises,
scales or multiplies anything beyond drawing the inputs.
"""
from __future__ import annotations

import torch

HIDDEN = 2048
SEQ = 4096
N_LAYERS = 28
# (name, K = input features, N = output features) of the four linear GEMM groups of a layer.
LINEARS = (
    ("qkv", 2048, 4096),      # 16 q heads + 2 x 8 kv heads, head dim 128
    ("o", 2048, 2048),
    ("gate_up", 2048, 12288),  # fused gate and up projections, 2 x 6144
    ("down", 6144, 2048),
)
X_STD, W_STD, DY_STD = 1.0, 0.02, 1e-3
KIND_X, KIND_W, KIND_DY, KIND_PICK = 0, 1, 2, 3


def config_seed(config: int, linear: int, kind: int) -> int:
    """Seed of one tensor of a single-layer configuration."""
    return 1000 * config + 10 * linear + kind


def stack_seed(layer: int, linear: int, kind: int) -> int:
    """Seed of one tensor of the 28-layer stack configuration."""
    return 4_000_000 + 100 * layer + 10 * linear + kind


def randn_bf16(shape, std: float, seed: int, device="cpu") -> torch.Tensor:
    """N(0, std^2) samples as bf16. On the CPU the stream is torch's CPU Philox/MT generator;
    on a HIP device it is the device generator with the same seed (different numbers, same
    recipe) — used where only throughput is measured."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=gen, dtype=torch.float32, device=dev)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def tiny_forward_inputs():
    """256x256 X ~ N(0,1) and 256x256 W ~ N(0, 0.02^2), both drawn from seed 0 in that order."""
    gen = torch.Generator().manual_seed(0)
    x = torch.randn((256, 256), generator=gen, dtype=torch.float32).to(torch.bfloat16)
    w = (torch.randn((256, 256), generator=gen, dtype=torch.float32) * W_STD).to(torch.bfloat16)
    return x, w


def linear_inputs(config: int, linear: int, M: int, K: int, N: int, device="cpu"):
    """X [M, K], W [N, K], dY [M, N] for one linear of a single-layer configuration."""
    x = randn_bf16((M, K), X_STD, config_seed(config, linear, KIND_X), device)
    w = randn_bf16((N, K), W_STD, config_seed(config, linear, KIND_W), device)
    dy = randn_bf16((M, N), DY_STD, config_seed(config, linear, KIND_DY), device)
    return x, w, dy


def outlier_inputs(M: int = 16384, K: int = 6144, N: int = 2048, config: int = 3,
                   linear: int = 3):
    """Down-projection stress inputs: X ~ N(0,1) with floor(1%) of its input channels scaled
    x100, then floor(0.1%) of its 1x128 row tiles (along K) set to zero; W ~ N(0, 0.02^2) with one
    128x128 block scaled x50; dY ~ N(0, 1e-3^2). All picks are seeded draws without replacement."""
    x, w, dy = linear_inputs(config, linear, M, K, N)
    gen = torch.Generator().manual_seed(config_seed(config, linear, KIND_PICK))
    n_chan = K // 100
    chans = torch.randperm(K, generator=gen)[:n_chan]
    xf = x.float()
    xf[:, chans] *= 100.0
    n_tiles = (M * (K // 128)) // 1000
    tiles = torch.randperm(M * (K // 128), generator=gen)[:n_tiles]
    rows, tcols = tiles // (K // 128), tiles % (K // 128)
    xv = xf.view(M, K // 128, 128)
    xv[rows, tcols, :] = 0.0
    x = xf.to(torch.bfloat16)
    blk = int(torch.randint(0, (N // 128) * (K // 128), (1,), generator=gen))
    bi, bj = blk // (K // 128), blk % (K // 128)
    wf = w.float()
    wf[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128] *= 50.0
    w = wf.to(torch.bfloat16)
    picks = {"channels": chans, "zero_tiles": (rows, tcols), "w_block": (bi, bj)}
    return x, w, dy, picks
