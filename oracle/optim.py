"""Learning-rate schedule, global-norm clip and AdamW.

Oracle code: test infrastructure only (see oracle/__init__.py).

PDS §4 optimisation paragraph: AdamW with betas (0.9, 0.95), eps 1e-8, weight
decay 0.1 on two-dimensional weights only, gradients clipped to global norm
1.0, learning rate rising linearly over 700 steps to 6e-4 and decaying by a
cosine to zero across all 18,865 steps.  GLM activity rows 10-12 (decoupled
weight decay, warmup + cosine, global L2-norm clipping) describe the same
three pieces.
"""
from __future__ import annotations

import math

import numpy as np

MAX_LR = 6e-4
WARMUP = 700
TOTAL_STEPS = 18865


def lr_at(t: float, max_lr: float = MAX_LR, warmup: int = WARMUP, total: int = TOTAL_STEPS) -> float:
    """Learning rate at 1-based optimizer step t: t/warmup * max_lr, then cosine to 0 at `total`."""
    if t <= warmup:
        return max_lr * t / warmup
    frac = (t - warmup) / (total - warmup)
    return 0.5 * max_lr * (1.0 + math.cos(math.pi * frac))


def global_norm(grads) -> float:
    """L2 norm over every gradient element, accumulated in float64."""
    s = 0.0
    for g in grads:
        g64 = np.asarray(g, dtype=np.float64)
        s += float(np.dot(g64.ravel(), g64.ravel()))
    return math.sqrt(s)


def clip_adamw(p, g, m, v, decay_mask, t, lr, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1,
               max_norm=1.0, dtype=np.float32):
    """One clip + AdamW step on flat arrays.  Returns (p, m, v, grad_norm); inputs are not modified.

    s = min(1, max_norm / ||g||); g <- s g; m <- b1 m + (1-b1) g; v <- b2 v + (1-b2) g^2;
    mhat = m / (1 - b1^t); vhat = v / (1 - b2^t);
    p <- p - lr * (mhat / (sqrt(vhat) + eps) + wd * p)  (wd only where decay_mask).
    Arithmetic runs in float64 and the stored state is rounded to `dtype`.
    """
    norm = global_norm([g])
    scale = min(1.0, max_norm / norm) if norm > 0 else 1.0
    g64 = np.asarray(g, dtype=np.float64) * scale
    m64 = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g64
    v64 = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g64 * g64
    mhat = m64 / (1.0 - beta1 ** t)
    vhat = v64 / (1.0 - beta2 ** t)
    p64 = np.asarray(p, dtype=np.float64)
    wd = np.where(decay_mask, weight_decay, 0.0)
    p64 = p64 - lr * (mhat / (np.sqrt(vhat) + eps) + wd * p64)
    return p64.astype(dtype), m64.astype(dtype), v64.astype(dtype), norm
