"""The allocation-free projected step, puro_hyperball_step_noalloc (partial sums in the
library's own device scratch), called through the C ABI, against puro_hyperball_step with a
caller-provided workspace: the updated fp32 masters and their bf16 copies must be identical bit
for bit (same kernels, same reduction order), on two calls in a row, the second with a smaller
matrix, so the scratch left by the first call must not leak into the second."""
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_noalloc_matches_workspace_entry_point(puro):
    dev = torch.device("cuda:0")
    for shape, seed in (((6144, 2048), 11), ((384, 256), 12)):
        say("noalloc hyperball step", shape)
        g = torch.Generator().manual_seed(seed)
        w0 = (torch.randn(shape, generator=g) * 0.02).to(dev)
        u = torch.randn(shape, generator=g).to(dev)
        radius = puro.puro_frobenius_norm(w0.clone())
        wa = w0.clone()
        ba = puro.puro_hyperball_step(wa, u, 1e-3, radius)
        wb = w0.clone()
        bb = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        puro.puro_hyperball_step_noalloc(wb, u, 1e-3, radius, bb)
        torch.cuda.synchronize()
        assert torch.equal(wa.view(torch.int32), wb.view(torch.int32)), shape
        assert torch.equal(ba.view(torch.int16), bb.view(torch.int16)), shape
        assert not torch.equal(wb, w0)  # the step did move the matrix
