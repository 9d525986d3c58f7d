"""Single operations of the GPT-2 step, written as their plain definitions.

Oracle code: test infrastructure only (see oracle/__init__.py).  Arrays are
NumPy; the dtype of the inputs (float32 or float64) is the working precision.
"""
from __future__ import annotations

import numpy as np

LN_EPS = 1e-5
GELU_K = np.sqrt(2.0 / np.pi)
GELU_C = 0.044715


# --- LayerNorm (PDS text around Fig. 1: normalisation before attention and
# before the feed-forward part; statistics in 32-bit per the §4 precision
# paragraph).  Textbook LN: biased variance, eps added to the variance.

def layernorm_fwd(x, w, b, eps=LN_EPS):
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mean) * rstd
    return xhat * w + b, mean[..., 0], rstd[..., 0]


def layernorm_bwd(dy, x, w, mean, rstd):
    """Gradients of y = w * (x - mean) * rstd + b with respect to x, w, b."""
    xhat = (x - mean[..., None]) * rstd[..., None]
    dxhat = dy * w
    red = tuple(range(dy.ndim - 1))
    dw = (dy * xhat).sum(axis=red)
    db = dy.sum(axis=red)
    m1 = dxhat.mean(axis=-1, keepdims=True)
    m2 = (dxhat * xhat).mean(axis=-1, keepdims=True)
    dx = (dxhat - m1 - xhat * m2) * rstd[..., None]
    return dx, dw, db


# --- GELU, GPT-2's tanh form (Hendrycks & Gimpel): the MLP's non-linearity.

def gelu_fwd(u):
    a = GELU_K * (u + GELU_C * u ** 3)
    return 0.5 * u * (1.0 + np.tanh(a))


def gelu_grad(u):
    """d GELU(u) / du for the tanh form."""
    a = GELU_K * (u + GELU_C * u ** 3)
    t = np.tanh(a)
    da = GELU_K * (1.0 + 3.0 * GELU_C * u ** 2)
    return 0.5 * (1.0 + t) + 0.5 * u * (1.0 - t * t) * da


def gelu_bwd(u, dg):
    return dg * gelu_grad(u)


# --- Linear layer y = x W^T + b, W stored [out, in].

def linear_fwd(x, W, b=None):
    y = x @ W.T
    return y if b is None else y + b


def linear_bwd(dy, x, W, has_bias=True):
    """Returns dx, dW, db (db None without bias).  x, dy are [..., in] / [..., out]."""
    x2 = x.reshape(-1, x.shape[-1])
    dy2 = dy.reshape(-1, dy.shape[-1])
    dx = (dy2 @ W).reshape(x.shape)
    dW = dy2.T @ x2
    db = dy2.sum(axis=0) if has_bias else None
    return dx, dW, db


# --- Causal scaled dot-product attention (GLM activity 5: Q.K^T/sqrt(d),
# causal mask, softmax; activity 6: heads are parallel projections).  Each
# position attends to itself and all earlier positions.  The full T x T score
# matrix is materialised with an explicit -inf mask.

def causal_mask(T):
    return np.triu(np.ones((T, T), dtype=bool), k=1)


def attention_fwd(q, k, v):
    """q, k, v: [B, H, T, d].  Returns O [B, H, T, d], P [B, H, T, T], lse [B, H, T]."""
    d = q.shape[-1]
    T = q.shape[-2]
    s = (q @ np.swapaxes(k, -1, -2)) / np.sqrt(d).astype(q.dtype)
    s = np.where(causal_mask(T), -np.inf, s)
    mx = s.max(axis=-1, keepdims=True)
    e = np.exp(s - mx)
    den = e.sum(axis=-1, keepdims=True)
    p = e / den
    lse = (mx + np.log(den))[..., 0]
    return p @ v, p, lse


def attention_bwd(do, q, k, v, p):
    """Gradients of O = softmax(mask(q k^T / sqrt d)) v with respect to q, k, v."""
    d = q.shape[-1]
    scale = 1.0 / np.sqrt(d)
    dv = np.swapaxes(p, -1, -2) @ do
    dp = do @ np.swapaxes(v, -1, -2)
    ds = p * (dp - (dp * p).sum(axis=-1, keepdims=True))
    dq = (ds @ k) * scale
    dk = (np.swapaxes(ds, -1, -2) @ q) * scale
    return dq.astype(q.dtype), dk.astype(q.dtype), dv.astype(q.dtype)


# --- Masked softmax cross-entropy over the padded vocabulary (PDS text
# around Fig. 1: the softmax covers only the V real tokens, so the padding
# columns get no probability and no gradient).

# A target of IGNORE_TARGET marks a position whose loss is not taken (PDS,
# clinical-adaptation paragraph: the loss is taken on answers, not on
# questions): its row loss is 0 and its gradient row is 0.
IGNORE_TARGET = -100


def masked_xent_fwd(z, tgt, V):
    """z: [R, Vp] logits, tgt: [R] ids < V or IGNORE_TARGET.  Returns per-row loss [R]
    (0 on ignored rows) and probs [R, V]."""
    zr = z[:, :V]
    mx = zr.max(axis=1, keepdims=True)
    e = np.exp(zr - mx)
    den = e.sum(axis=1, keepdims=True)
    lse = mx[:, 0] + np.log(den[:, 0])
    keep = tgt != IGNORE_TARGET
    t = np.where(keep, tgt, 0)
    loss = np.where(keep, lse - zr[np.arange(z.shape[0]), t], 0.0)
    return loss, e / den


def masked_xent_bwd(probs, tgt, Vp, dloss):
    """d(dloss * sum_r loss_r)/dz: (p - onehot) * dloss on real columns, exactly 0 on padding
    and on the rows of ignored targets."""
    R, V = probs.shape
    keep = tgt != IGNORE_TARGET
    dz = np.zeros((R, Vp), dtype=probs.dtype)
    dz[:, :V] = probs
    dz[np.arange(R)[keep], tgt[keep]] -= 1.0
    dz[:, :V] *= dloss
    dz[~keep] = 0.0
    return dz


# --- Learned token and position lookup (GLM activity 4), tied token table.

def embedding_fwd(wte, wpe, tok):
    T = tok.shape[-1]
    return wte[tok] + wpe[:T]


def embedding_bwd(dx, tok, Vp, Tmax):
    """Scatter-add of dx rows into the token table; sum over the batch for positions."""
    C = dx.shape[-1]
    dwte = np.zeros((Vp, C), dtype=dx.dtype)
    np.add.at(dwte, tok.reshape(-1), dx.reshape(-1, C))
    dwpe = np.zeros((Tmax, C), dtype=dx.dtype)
    dwpe[:tok.shape[-1]] = dx.sum(axis=0)
    return dwte, dwpe
