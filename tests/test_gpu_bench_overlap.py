"""The bench's two launch orders compute the same step: every dW, the last dX and Y, and the
quantised copies are bitwise identical after a serial step, an overlapped eager step and a
replay of the overlapped step captured as a graph (the kernels are deterministic, so any missing
dependency between the two streams would show as a difference)."""
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _snapshot(stack):
    outs = [dw.clone() for _, dw in stack.weights]
    outs += [t.clone() for t in stack.shared.values()]
    return outs


def _reset(stack):
    for _, dw in stack.weights:
        dw.fill_(-1.0)
    for t in stack.shared.values():
        t.zero_()


@pytest.mark.parametrize("fused", [True, False])
def test_overlapped_order_matches_serial(fused):
    import bench
    say("bench overlap vs serial, fused =", fused)
    main = torch.cuda.Stream()
    with torch.cuda.stream(main):
        stack = bench.Stack(2, 8192, fused=fused)
        stack.run()
        torch.cuda.synchronize()
        ref = _snapshot(stack)
        _reset(stack)
        stack.run(overlap=True)
        torch.cuda.synchronize()
        got = _snapshot(stack)
        for i, (a, b) in enumerate(zip(ref, got)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"eager output {i}"
        stack.capture(overlap=True)
        for rep in range(3):
            _reset(stack)
            torch.cuda.synchronize()
            stack.replay()
            torch.cuda.synchronize()
            got = _snapshot(stack)
            for i, (a, b) in enumerate(zip(ref, got)):
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), \
                    f"graph replay {rep}: output {i}"
