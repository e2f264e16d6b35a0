"""Pins of the AdamW / clipping oracle (readings R20, R21): closed forms for
constant and zero gradients, the library AdamW of PyTorch (a separate
implementation of the same textbook update) and PyTorch's global-norm
gradient clipping."""

import numpy as np
import pytest

from oracle import optim

torch = pytest.importorskip("torch")


def test_constant_gradient_moves_by_lr_per_step():
    """g constant: m_hat = g and v_hat = g^2 at every step, so with wd = 0
    each step moves p by lr * g / (|g| + eps)."""
    p, m, v = np.array([0.5, -2.0]), np.zeros(2), np.zeros(2)
    g = np.array([0.25, -3.0])
    lr, eps = 1e-2, 1e-8
    for t in range(1, 8):
        p, m, v = optim.adamw_step(p, m, v, g, t, lr, eps=eps)
        assert np.allclose(p, np.array([0.5, -2.0]) - t * lr * g / (np.abs(g) + eps), rtol=0, atol=1e-14)


def test_zero_gradient_is_pure_decay():
    p0 = np.array([1.0, -0.5, 3.0])
    p, m, v = p0.copy(), np.zeros(3), np.zeros(3)
    for t in range(1, 6):
        p, m, v = optim.adamw_step(p, m, v, np.zeros(3), t, lr=0.1, wd=0.01)
    assert np.allclose(p, p0 * (1 - 0.1 * 0.01) ** 5, rtol=1e-15, atol=0)


@pytest.mark.parametrize("wd", [0.0, 0.05])
def test_matches_torch_adamw(wd):
    rng = np.random.Generator(np.random.PCG64(3))
    p0 = rng.normal(0, 1, 300)
    grads = [rng.normal(0, 1, 300) for _ in range(6)]
    tp = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=1e-3, betas=(0.9, 0.95), eps=1e-6, weight_decay=wd)
    p, m, v = p0.copy(), np.zeros(300), np.zeros(300)
    for t, g in enumerate(grads, start=1):
        tp.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        p, m, v = optim.adamw_step(p, m, v, g, t, 1e-3, 0.9, 0.95, 1e-6, wd)
    assert np.allclose(p, tp.detach().numpy(), rtol=1e-13, atol=1e-15)


def test_clip_matches_torch_clip_grad_norm():
    rng = np.random.Generator(np.random.PCG64(4))
    gs = [rng.normal(0, 1, s) for s in (10, 33, 7)]
    for max_norm in (0.5, 100.0):
        ts = [torch.zeros(len(g), dtype=torch.float64, requires_grad=True) for g in gs]
        for t, g in zip(ts, gs):
            t.grad = torch.tensor(g, dtype=torch.float64)
        norm = torch.nn.utils.clip_grad_norm_(ts, max_norm)
        c, n = optim.clip_coefficient(gs, max_norm)
        assert np.isclose(n, float(norm), rtol=1e-14)
        for t, g in zip(ts, gs):
            assert np.allclose(t.grad.numpy(), g * c, rtol=1e-14, atol=0)
    c, _ = optim.clip_coefficient(gs, 0.0)
    assert c == 1.0
