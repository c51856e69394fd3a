"""Pins of the oracle's optimizer step (the projected matrix update and AdamW) to things other
than itself: numpy's norm, torch.optim.AdamW run in float64 on the CPU (a library
implementation of the same textbook rule), hand-worked cases, and exact invariances."""
import numpy as np
import pytest
import torch


def _rand(shape, seed, std=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * std).astype(np.float32)


def test_frobenius_norm(oracle):
    assert oracle.frobenius_norm(np.array([3.0, 4.0], np.float32)) == 5.0
    assert oracle.frobenius_norm(np.zeros(8, np.float32)) == 0.0
    w = _rand((256, 384), 1, 0.02)
    ref = float(np.linalg.norm(w.astype(np.float64)))
    assert abs(oracle.frobenius_norm(w) - ref) <= 1e-13 * ref


def test_hyperball_hand_cases(oracle):
    # w = (3, 4), no update, radius 10 -> (6, 8)
    out = oracle.hyperball_update(np.array([3.0, 4.0], np.float32), np.zeros(2, np.float32),
                                  0.5, 10.0)
    assert np.array_equal(out, [6.0, 8.0])
    # w = (1, 0), u = (1, -1), lr = 1 -> v = (0, 1) -> radius 2 gives (0, 2)
    out = oracle.hyperball_update(np.array([1.0, 0.0], np.float32),
                                  np.array([1.0, -1.0], np.float32), 1.0, 2.0)
    assert np.array_equal(out, [0.0, 2.0])
    # zero matrix after the update stays zero
    out = oracle.hyperball_update(np.array([2.0, 2.0], np.float32),
                                  np.array([1.0, 1.0], np.float32), 2.0, 3.0)
    assert np.array_equal(out, [0.0, 0.0])


def test_hyperball_invariants(oracle):
    w = _rand((128, 256), 2, 0.02)
    u = _rand((128, 256), 3, 1.0)
    R, lr = 5.0, 0.01
    out = oracle.hyperball_update(w, u, lr, R)
    # lands on the sphere of radius R
    assert abs(np.linalg.norm(out) - R) <= 1e-13 * R
    # points along w - lr*u
    v = w.astype(np.float64) - lr * u.astype(np.float64)
    cos = float(np.sum(out * v) / (np.linalg.norm(out) * np.linalg.norm(v)))
    assert abs(cos - 1.0) <= 1e-13
    # scale invariance: (c w, c u) gives the same point for c a power of two (exact scaling)
    out2 = oracle.hyperball_update(w * np.float32(8.0), u * np.float32(8.0), lr, R)
    assert np.max(np.abs(out2 - out)) <= 1e-15 * R
    # a point already on the sphere with lr = 0 stays (up to binary64 rounding)
    on = (w.astype(np.float64) * (R / np.linalg.norm(w.astype(np.float64)))).astype(np.float32)
    out3 = oracle.hyperball_update(on, u, 0.0, float(np.linalg.norm(on.astype(np.float64))))
    assert np.max(np.abs(out3 - on)) <= 1e-15 * R


@pytest.mark.parametrize("wd,lr,b1,b2,eps", [(0.1, 1e-3, 0.9, 0.95, 1e-8),
                                              (0.0, 3e-4, 0.8, 0.999, 1e-6),
                                              (0.05, 1e-2, 0.9, 0.95, 1e-8)])
def test_adamw_matches_torch_float64(oracle, wd, lr, b1, b2, eps):
    shape = (64, 96)
    p0 = _rand(shape, 10, 0.02)
    grads = [_rand(shape, 11 + t, 1e-3) for t in range(4)]
    tp = torch.nn.Parameter(torch.tensor(p0, dtype=torch.float64))
    opt = torch.optim.AdamW([tp], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd)
    p, m, v = p0, np.zeros(shape, np.float32), np.zeros(shape, np.float32)
    for t, g in enumerate(grads, start=1):
        tp.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        po, mo, vo = oracle.adamw(p, g, m, v, lr, b1, b2, eps, wd, t)
        st = opt.state[tp]
        tp_np = tp.detach().numpy()
        # the oracle takes fp32 state in, so compare each step from the same fp32 inputs: carry
        # the torch state forward rounded to fp32 as the next inputs of both
        assert np.max(np.abs(po - tp_np)) <= 1e-12 * np.max(np.abs(tp_np))
        assert np.max(np.abs(mo - st["exp_avg"].numpy())) <= 1e-12 * np.max(np.abs(mo))
        assert np.max(np.abs(vo - st["exp_avg_sq"].numpy())) <= 1e-12 * np.max(np.abs(vo))
        p, m, v = (a.astype(np.float32) for a in (po, mo, vo))
        with torch.no_grad():
            tp.copy_(torch.tensor(p, dtype=torch.float64))
            st["exp_avg"].copy_(torch.tensor(m, dtype=torch.float64))
            st["exp_avg_sq"].copy_(torch.tensor(v, dtype=torch.float64))


def test_adamw_closed_forms(oracle):
    p = np.array([0.5, -0.25, 1.0, 0.0], np.float32)
    g = np.array([2.0, -4.0, 0.0, 1e-3], np.float32)
    z = np.zeros(4, np.float32)
    lr, eps = 0.01, 1e-8
    # first step, no decay: m_hat = g and v_hat = g^2, so p moves by lr * g / (|g| + eps)
    p64, g64 = p.astype(np.float64), g.astype(np.float64)
    po, mo, vo = oracle.adamw(p, g, z, z, lr, 0.9, 0.95, eps, 0.0, 1)
    assert np.allclose(po, p64 - lr * g64 / (np.abs(g64) + eps), rtol=0, atol=1e-15)
    assert np.allclose(mo, 0.1 * g64, rtol=1e-15, atol=0)
    # zero gradient and zero moments: only the decoupled decay acts
    po, _, _ = oracle.adamw(p, z, z, z, lr, 0.9, 0.95, eps, 0.1, 7)
    assert np.array_equal(po, p.astype(np.float64) * (1 - lr * 0.1))
    # a constant gradient from zero moments: the bias-corrected first moment equals g at every
    # step t, so the step is lr * g / (|g| + eps) every time (weight decay off)
    m, v, q = z, z, np.zeros(4, np.float32)
    for t in range(1, 6):
        qo, mo, vo = oracle.adamw(q, g, m, v, lr, 0.9, 0.95, eps, 0.0, t)
        step = qo - q.astype(np.float64)
        assert np.allclose(step, -lr * g64 / (np.abs(g64) + eps), rtol=1e-6, atol=1e-12)
        q, m, v = (a.astype(np.float32) for a in (qo, mo, vo))
