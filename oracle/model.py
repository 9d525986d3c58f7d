"""GPT-2 style decoder-only model: parameters, seeded init, forward, backward.

Oracle code: test infrastructure only (see oracle/__init__.py).

Architecture (PDS text around Fig. 1): GPT-2's smallest configuration -- L
blocks, H heads, C channels, context Tmax, tied input/output embeddings; each
block normalises before attention and before the feed-forward part, with a
residual connection around both.  Vocabulary padded from V to Vp with the
softmax over the V real tokens only.  Init N(0, 0.02); projections that write
into the residual stream use 0.02 / sqrt(2L).

Flat parameter layout (the same order the HIP library documents): first the
decayed 2-D segment -- wte [Vp, C], wpe [Tmax, C], then per layer
c_attn.weight [3C, C], attn.c_proj.weight [C, C], c_fc.weight [4C, C],
mlp.c_proj.weight [C, 4C]; then the 1-D segment -- per layer ln_1.weight,
ln_1.bias, c_attn.bias [3C], attn.c_proj.bias, ln_2.weight, ln_2.bias,
c_fc.bias [4C], mlp.c_proj.bias; then ln_f.weight, ln_f.bias.  All weights are
[out, in] so a layer computes y = x W^T + b.  Q, K, V occupy rows [0, C),
[C, 2C), [2C, 3C) of c_attn and head h uses rows h*d .. h*d+d-1 of each.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import ops
from .rng import tensor_normal


@dataclass(frozen=True)
class Config:
    L: int
    H: int
    C: int
    V: int
    Vp: int
    Tmax: int

    @property
    def d(self):
        return self.C // self.H


CONFIGS = {
    # GPT-2 124M, vocab 50,257 padded to 50,304, context 1,024.
    "gpt2_124m": Config(L=12, H=12, C=768, V=50257, Vp=50304, Tmax=1024),
    # Tiny full-step model (2 layers, 4 heads, C=128, T=64).
    "tiny": Config(L=2, H=4, C=128, V=50257, Vp=50304, Tmax=64),
    # Wider/deeper scaling shape (16 layers, 24 heads, C=1536, vocab 8,449 -> 8,576).
    "wide": Config(L=16, H=24, C=1536, V=8449, Vp=8576, Tmax=1024),
    # Micro model for finite differences (oracle only).
    "micro": Config(L=2, H=2, C=16, V=61, Vp=64, Tmax=8),
}


def tensor_specs(cfg: Config):
    """[(name, shape, decayed)] in flat-layout order."""
    L, C = cfg.L, cfg.C
    specs = [("wte", (cfg.Vp, C), True), ("wpe", (cfg.Tmax, C), True)]
    for l in range(L):
        specs += [(f"h.{l}.attn.c_attn.weight", (3 * C, C), True),
                  (f"h.{l}.attn.c_proj.weight", (C, C), True),
                  (f"h.{l}.mlp.c_fc.weight", (4 * C, C), True),
                  (f"h.{l}.mlp.c_proj.weight", (C, 4 * C), True)]
    for l in range(L):
        specs += [(f"h.{l}.ln_1.weight", (C,), False),
                  (f"h.{l}.ln_1.bias", (C,), False),
                  (f"h.{l}.attn.c_attn.bias", (3 * C,), False),
                  (f"h.{l}.attn.c_proj.bias", (C,), False),
                  (f"h.{l}.ln_2.weight", (C,), False),
                  (f"h.{l}.ln_2.bias", (C,), False),
                  (f"h.{l}.mlp.c_fc.bias", (4 * C,), False),
                  (f"h.{l}.mlp.c_proj.bias", (C,), False)]
    specs += [("ln_f.weight", (C,), False), ("ln_f.bias", (C,), False)]
    return specs


def layout(cfg: Config):
    """{name: (offset, shape, decayed)} in the flat fp32 buffer."""
    out, off = {}, 0
    for name, shape, dec in tensor_specs(cfg):
        out[name] = (off, shape, dec)
        off += int(np.prod(shape))
    return out


def n_params(cfg: Config, padded: bool = True) -> int:
    n = sum(int(np.prod(s)) for _, s, _ in tensor_specs(cfg))
    return n if padded else n - (cfg.Vp - cfg.V) * cfg.C


def init_params(cfg: Config, seed: int = 1337):
    """Seeded init (PDS text around Fig. 1; seed from the §4 optimisation paragraph).

    2-D weights ~ N(0, 0.02), the two residual-writing projections per layer
    ~ N(0, 0.02/sqrt(2L)), wte padding rows 0, biases 0, LN gains 1.
    """
    p = {}
    resid_std = 0.02 / np.sqrt(2.0 * cfg.L)
    for tau, (name, shape, dec) in enumerate(tensor_specs(cfg)):
        n = int(np.prod(shape))
        if dec:
            std = resid_std if name.endswith("c_proj.weight") else 0.02
            a = tensor_normal(seed, tau, n, std).reshape(shape)
            if name == "wte":
                a[cfg.V:] = 0.0
        elif name.endswith("ln_1.weight") or name.endswith("ln_2.weight") or name == "ln_f.weight":
            a = np.ones(shape, dtype=np.float32)
        else:
            a = np.zeros(shape, dtype=np.float32)
        p[name] = a
    return p


def flatten(cfg: Config, tensors, dtype=np.float32):
    lay = layout(cfg)
    flat = np.zeros(n_params(cfg), dtype=dtype)
    for name, (off, shape, _) in lay.items():
        flat[off:off + int(np.prod(shape))] = np.asarray(tensors[name]).reshape(-1)
    return flat


def unflatten(cfg: Config, flat):
    return {name: flat[off:off + int(np.prod(shape))].reshape(shape)
            for name, (off, shape, _) in layout(cfg).items()}


def _split_heads(a, B, T, H, d):
    return a.reshape(B, T, H, d).transpose(0, 2, 1, 3)


def _merge_heads(a):
    B, H, T, d = a.shape
    return a.transpose(0, 2, 1, 3).reshape(B, T, H * d)


def forward(cfg: Config, P, tok, tgt=None, dtype=np.float64):
    """Forward pass.  Returns (mean loss or None, per-row loss [B,T] or None, cache).

    cache['logits'] holds z [B, T, Vp]; cache['resid'][l] the residual stream
    entering block l (and cache['resid'][L] the one leaving the last block).
    """
    P = {k: np.asarray(v, dtype=dtype) for k, v in P.items()}
    B, T = tok.shape
    C, H, d = cfg.C, cfg.H, cfg.d
    x = ops.embedding_fwd(P["wte"], P["wpe"], tok)
    cache = {"tok": tok, "tgt": tgt, "resid": [x], "layers": []}
    for l in range(cfg.L):
        pre = f"h.{l}."
        a, m1, r1 = ops.layernorm_fwd(x, P[pre + "ln_1.weight"], P[pre + "ln_1.bias"])
        qkv = ops.linear_fwd(a, P[pre + "attn.c_attn.weight"], P[pre + "attn.c_attn.bias"])
        q = _split_heads(qkv[..., :C], B, T, H, d)
        k = _split_heads(qkv[..., C:2 * C], B, T, H, d)
        v = _split_heads(qkv[..., 2 * C:], B, T, H, d)
        o, prob, lse = ops.attention_fwd(q, k, v)
        om = _merge_heads(o)
        x1 = x + ops.linear_fwd(om, P[pre + "attn.c_proj.weight"], P[pre + "attn.c_proj.bias"])
        a2, m2, r2 = ops.layernorm_fwd(x1, P[pre + "ln_2.weight"], P[pre + "ln_2.bias"])
        u = ops.linear_fwd(a2, P[pre + "mlp.c_fc.weight"], P[pre + "mlp.c_fc.bias"])
        g = ops.gelu_fwd(u)
        x2 = x1 + ops.linear_fwd(g, P[pre + "mlp.c_proj.weight"], P[pre + "mlp.c_proj.bias"])
        cache["layers"].append(dict(x=x, a=a, m1=m1, r1=r1, q=q, k=k, v=v, o=om, prob=prob, lse=lse,
                                    x1=x1, a2=a2, m2=m2, r2=r2, u=u, g=g))
        x = x2
        cache["resid"].append(x)
    yf, mf, rf = ops.layernorm_fwd(x, P["ln_f.weight"], P["ln_f.bias"])
    z = yf @ P["wte"].T
    cache.update(xf=x, yf=yf, mf=mf, rf=rf, logits=z)
    if tgt is None:
        return None, None, cache
    loss_rows, probs = ops.masked_xent_fwd(z.reshape(B * T, -1), tgt.reshape(-1), cfg.V)
    cache["probs"] = probs
    n_keep = int(np.count_nonzero(tgt != ops.IGNORE_TARGET))
    mean = float(loss_rows.sum() / n_keep) if n_keep else 0.0  # mean over the positions whose loss is taken
    return mean, loss_rows.reshape(B, T), cache


def backward(cfg: Config, P, cache, dloss, dtype=np.float64):
    """Exact gradients of dloss * sum_rows loss_row, as {name: array}."""
    P = {k: np.asarray(v, dtype=dtype) for k, v in P.items()}
    tok = cache["tok"]
    tgt = cache["tgt"]
    B, T = tok.shape
    C = cfg.C
    G = {}
    dz = ops.masked_xent_bwd(cache["probs"], tgt.reshape(-1), cfg.Vp, dloss)
    yf = cache["yf"].reshape(B * T, C)
    dyf = (dz @ P["wte"]).reshape(B, T, C)
    dwte_head = dz.T @ yf
    dx, G["ln_f.weight"], G["ln_f.bias"] = ops.layernorm_bwd(dyf, cache["xf"], P["ln_f.weight"],
                                                            cache["mf"], cache["rf"])
    for l in reversed(range(cfg.L)):
        pre = f"h.{l}."
        c = cache["layers"][l]
        # x2 = x1 + g W_fp^T + b_fp
        dg, G[pre + "mlp.c_proj.weight"], G[pre + "mlp.c_proj.bias"] = ops.linear_bwd(
            dx, c["g"], P[pre + "mlp.c_proj.weight"])
        du = ops.gelu_bwd(c["u"], dg)
        da2, G[pre + "mlp.c_fc.weight"], G[pre + "mlp.c_fc.bias"] = ops.linear_bwd(
            du, c["a2"], P[pre + "mlp.c_fc.weight"])
        dln2, G[pre + "ln_2.weight"], G[pre + "ln_2.bias"] = ops.layernorm_bwd(
            da2, c["x1"], P[pre + "ln_2.weight"], c["m2"], c["r2"])
        dx1 = dx + dln2
        # x1 = x + o W_p^T + b_p
        do, G[pre + "attn.c_proj.weight"], G[pre + "attn.c_proj.bias"] = ops.linear_bwd(
            dx1, c["o"], P[pre + "attn.c_proj.weight"])
        H, d = cfg.H, cfg.d
        dq, dk, dv = ops.attention_bwd(_split_heads(do, B, T, H, d), c["q"], c["k"], c["v"], c["prob"])
        dqkv = np.concatenate([_merge_heads(dq), _merge_heads(dk), _merge_heads(dv)], axis=-1)
        da, G[pre + "attn.c_attn.weight"], G[pre + "attn.c_attn.bias"] = ops.linear_bwd(
            dqkv, c["a"], P[pre + "attn.c_attn.weight"])
        dln1, G[pre + "ln_1.weight"], G[pre + "ln_1.bias"] = ops.layernorm_bwd(
            da, c["x"], P[pre + "ln_1.weight"], c["m1"], c["r1"])
        dx = dx1 + dln1
    dwte_emb, dwpe = ops.embedding_bwd(dx, tok, cfg.Vp, cfg.Tmax)
    G["wte"] = dwte_head + dwte_emb
    G["wpe"] = dwpe
    cache["dx0"] = dx
    return G


def loss_and_grads(cfg: Config, P, tok, tgt, dloss=None, dtype=np.float64):
    """Mean loss and gradients of dloss * sum of row losses (default dloss = 1 / the number of
    positions whose target is not ignored: the gradient of the mean)."""
    if dloss is None:
        dloss = 1.0 / max(1, int(np.count_nonzero(tgt != ops.IGNORE_TARGET)))
    loss, rows, cache = forward(cfg, P, tok, tgt, dtype=dtype)
    return loss, backward(cfg, P, cache, dloss, dtype=dtype), cache
