"""AdamW update of the LoRA adapters with global-norm gradient clipping, in
fp64.  TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix: QLoRA trains the adapters with AdamW and paged optimizers
(QLoRA project page, technical architecture: optimizer AdamW and paged
optimizers); training stability comes from gradient clipping and learning
rate adjustment (project page, challenges and solutions); the large-model
example uses learning rate 1e-4 (project page, usage example).  Paged
optimizers keep optimizer state out of GPU memory to absorb memory spikes
(news write-up and Finnish article, third technique) -- where the state lives
does not change what is computed.

Readings:
  R20  AdamW is the decoupled-weight-decay Adam: with gradient g at step t
       (t = 1, 2, ...),
           m <- b1 m + (1 - b1) g,     v <- b2 v + (1 - b2) g^2,
           m_hat = m / (1 - b1^t),     v_hat = v / (1 - b2^t),
           p <- p - lr (m_hat / (sqrt(v_hat) + eps) + wd p).
       Master parameters, m and v are kept in fp32; the bf16 adapter used
       by the layer is the master rounded to nearest-even bf16.
  R21  Gradient clipping by the global L2 norm over all adapter gradients:
       with ||g|| the norm and c = max_norm / (||g|| + 1e-6), gradients are
       multiplied by c when c < 1 (no clipping when max_norm <= 0).
"""

from __future__ import annotations

import numpy as np


def clip_coefficient(grads, max_norm: float):
    """R21: (coefficient applied to the gradients, global norm), fp64."""
    g = np.concatenate([np.asarray(x, dtype=np.float64).ravel() for x in grads]) if len(grads) else np.zeros(0)
    norm = float(np.sqrt(np.sum(g * g)))
    if max_norm <= 0:
        return 1.0, norm
    c = max_norm / (norm + 1e-6)
    return (c if c < 1.0 else 1.0), norm


def adamw_step(p, m, v, g, t: int, lr: float, b1: float = 0.9, b2: float = 0.999, eps: float = 1e-8,
               wd: float = 0.0, grad_scale: float = 1.0):
    """R20 on fp64 copies: returns the new (p, m, v).  g is multiplied by
    grad_scale first (the clipping coefficient)."""
    p = np.asarray(p, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64) * grad_scale
    m = b1 * m + (1.0 - b1) * g
    v = b2 * v + (1.0 - b2) * g * g
    m_hat = m / (1.0 - b1 ** t)
    v_hat = v / (1.0 - b2 ** t)
    p = p - lr * (m_hat / (np.sqrt(v_hat) + eps) + wd * p)
    return p, m, v
