"""Kernel-level parity: each HIP kernel (through the C ABI) against the oracle's
op on the same seeded, bf16-rounded inputs.  Sizes span several tiles and a
ragged tail; the one-card micro-batch shapes (19,456 rows) are checked on
sampled rows or through properties."""
import math
import sys

import numpy as np
import pytest

from oracle import ops
import oracle
from transformer_lm_pretraining_amd import synth
from gpu_util import (bf16_round, to_dev_bf16, to_dev_f32, to_dev_i32, host, rel_l2, cosine, bf16_rne_bits,
                      assert_elementwise, abs_matmul, U32, BF16)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# ---------------------------------------------------------------- cross-entropy

@pytest.mark.parametrize("rows,V,Vp", [(300, 50257, 50304), (257, 8449, 8576), (64, 100, 128)])
def test_xent_parity(gpu_lib, rows, V, Vp):
    import torch
    from transformer_lm_pretraining_amd import lib
    say("xent", rows, V, Vp)
    z = bf16_round(synth.normal((rows, Vp), seed=11))
    z[:, V:] = 30.0  # planted garbage in the padding columns: a leak would dominate the softmax
    tgt = synth.targets(rows, V, seed=12)
    dloss = 1.0 / (rows * 3)
    zd = to_dev_bf16(z)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    loss = lib.xent(zd, to_dev_i32(tgt), V, dloss, True, flag)
    torch.cuda.synchronize()
    want, probs = ops.masked_xent_fwd(z, tgt, V)
    dz = ops.masked_xent_bwd(probs, tgt, Vp, dloss)
    np.testing.assert_allclose(host(loss), want, atol=1e-4, rtol=0)
    got = host(zd)
    assert np.all(got[:, V:] == 0.0)
    assert rel_l2(got, dz) <= 4e-3
    # element-wise: the bf16 rounding of each gradient (2^-8 relative, doubled) plus
    # 1e-6 dloss for the fp32 softmax near p = 1 (the target column's p - 1 cancels)
    assert_elementwise(got, dz, 2 * BF16 * np.abs(dz) + 1e-6 * dloss, "xent dz")
    assert int(flag.item()) == 0


def test_xent_full_rows_sampled_and_flag(gpu_lib):
    import torch
    from transformer_lm_pretraining_amd import lib
    rows, V, Vp = 19456, 50257, 50304
    say("xent full", rows)
    zd = torch.randn(rows, Vp, generator=torch.Generator(device="cuda").manual_seed(5), device="cuda").bfloat16()
    tgt = synth.targets(rows, V, seed=13)
    tgt[7] = V + 3  # out of range: flagged and clamped
    sample = np.r_[0:4, 9000:9004, rows - 4:rows]
    z_s = host(zd[torch.as_tensor(sample, device="cuda")])
    z_7 = host(zd[7:8])
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    loss = lib.xent(zd, to_dev_i32(tgt), V, 1.0 / rows, True, flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 1
    t_s = tgt[sample].copy()
    want, probs = ops.masked_xent_fwd(z_s, t_s, V)
    np.testing.assert_allclose(host(loss)[sample], want, atol=1e-4)
    dz = ops.masked_xent_bwd(probs, t_s, Vp, 1.0 / rows)
    got = host(zd[torch.as_tensor(sample, device="cuda")])
    assert rel_l2(got, dz) <= 4e-3
    assert_elementwise(got, dz, 2 * BF16 * np.abs(dz) + 1e-6 / rows, "xent dz sampled rows")
    assert np.all(got[:, V:] == 0)
    # the clamped row used target V-1
    w7, _ = ops.masked_xent_fwd(z_7, np.array([V - 1]), V)
    assert abs(host(loss)[7] - w7[0]) < 1e-4


def test_xent_ignored_targets(gpu_lib):
    """Targets equal to GPT2_IGNORE_TARGET: loss 0, an all-zero gradient row, no flag."""
    import torch
    from transformer_lm_pretraining_amd import lib
    rows, V, Vp = 301, 50257, 50304
    say("xent ignored", rows)
    z = bf16_round(synth.normal((rows, Vp), seed=15))
    tgt = synth.targets(rows, V, seed=16)
    tgt[::3] = lib.IGNORE_TARGET
    tgt[-1] = lib.IGNORE_TARGET
    keep = tgt != lib.IGNORE_TARGET
    zd = to_dev_bf16(z)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    loss = lib.xent(zd, to_dev_i32(tgt), V, 0.01, True, flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    want, probs = ops.masked_xent_fwd(z, tgt, V)
    got = host(loss)
    assert np.all(got[~keep] == 0)
    np.testing.assert_allclose(got[keep], want[keep], atol=2e-4)
    dz = host(zd)
    assert np.all(dz[~keep] == 0)
    dz_r = ops.masked_xent_bwd(probs, tgt, Vp, 0.01)[keep]
    assert rel_l2(dz[keep], dz_r) <= 4e-3
    assert_elementwise(dz[keep], dz_r, 2 * BF16 * np.abs(dz_r) + 1e-6 * 0.01, "xent dz kept rows")


# ---------------------------------------------------------------- LayerNorm

@pytest.mark.parametrize("rows,C", [(1003, 768), (130, 128), (67, 1536), (19456, 768)])
def test_layernorm_parity(gpu_lib, rows, C):
    import torch
    from transformer_lm_pretraining_amd import lib
    say("layernorm", rows, C)
    x = bf16_round(synth.normal((rows, C), seed=21))
    w = (1 + 0.1 * synth.normal((C,), seed=22)).astype(np.float32).astype(np.float64)
    b = (0.1 * synth.normal((C,), seed=23)).astype(np.float32).astype(np.float64)
    dy = bf16_round(synth.normal((rows, C), seed=24))
    dres0 = bf16_round(synth.normal((rows, C), seed=25))
    xd, wd, bd = to_dev_bf16(x), to_dev_f32(w), to_dev_f32(b)
    y, mean, rstd = lib.layernorm_fwd(xd, wd, bd)
    dres = to_dev_bf16(dres0)
    dw = to_dev_f32(np.full(C, 0.5))
    db = to_dev_f32(np.full(C, -0.25))
    lib.layernorm_bwd(xd, to_dev_bf16(dy), wd, mean, rstd, dres, 1, dw, db)
    torch.cuda.synchronize()
    yr, mr, rr = ops.layernorm_fwd(x, w, b)
    yg = host(y)
    assert np.all(np.abs(yg - yr) <= 2.0 ** -7 * np.abs(yr) + 1e-6)
    np.testing.assert_allclose(host(mean), mr, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(host(rstd), rr, rtol=1e-5)
    dx, dwr, dbr = ops.layernorm_bwd(dy, x, w, mr, rr)
    assert rel_l2(host(dres) - dres0, dx) <= 1e-2
    np.testing.assert_allclose(host(dw), dwr + 0.5, rtol=1e-4, atol=1e-3)
    np.testing.assert_allclose(host(db), dbr - 0.25, rtol=1e-4, atol=1e-3)
    # overwrite mode
    lib.layernorm_bwd(xd, to_dev_bf16(dy), wd, mean, rstd, dres, 0, dw, db)
    torch.cuda.synchronize()
    assert rel_l2(host(dres), dx) <= 1e-2


# ---------------------------------------------------------------- bias + GELU

@pytest.mark.parametrize("rows,N", [(1001, 3072), (64, 512), (19456, 3072)])
def test_bias_gelu_parity(gpu_lib, rows, N):
    import torch
    from transformer_lm_pretraining_amd import lib
    say("bias_gelu", rows, N)
    u = bf16_round(synth.normal((rows, N), seed=31))
    b = synth.normal((N,), std=0.02, seed=32).astype(np.float64)
    dout = bf16_round(synth.normal((rows, N), seed=33))
    pre, g = lib.bias_gelu_fwd(to_dev_bf16(u), to_dev_f32(b))
    db = to_dev_f32(np.zeros(N))
    dpre = lib.bias_gelu_bwd(pre, to_dev_bf16(dout), db)
    torch.cuda.synchronize()
    sample = slice(None) if rows <= 2048 else np.r_[0:16, rows // 2:rows // 2 + 16, rows - 16:rows]
    pre_r = (u + b)[sample]
    pg, gg = host(pre)[sample], host(g)[sample]
    assert np.all(np.abs(pg - pre_r) <= 2.0 ** -8 * np.abs(pre_r) + 1e-7)
    g_r = ops.gelu_fwd(pg)  # GELU of the stored pre-activation
    assert np.all(np.abs(gg - g_r) <= 2.0 ** -7 * np.abs(g_r) + 1e-6)
    dpre_r = ops.gelu_bwd(host(pre), dout)
    assert rel_l2(host(dpre), dpre_r) <= 1e-2
    # bias gradient = column sums of the stored dpre
    np.testing.assert_allclose(host(db), host(dpre).sum(0), rtol=1e-4, atol=1e-3)


def test_bias_grad_colsum(gpu_lib):
    import torch
    from transformer_lm_pretraining_amd import lib
    rows, N = 19456, 2304
    say("bias_grad", rows, N)
    dy = bf16_round(synth.normal((rows, N), seed=41))
    db = to_dev_f32(np.ones(N))
    lib.bias_grad(to_dev_bf16(dy), db)
    torch.cuda.synchronize()
    np.testing.assert_allclose(host(db), dy.sum(0) + 1, rtol=1e-4, atol=2e-3)


# ---------------------------------------------------------------- GEMM

# (1024, 50304, 768), (2000, 9000, 64) and (3000, 6000, 128) run more 256x256 tiles than there
# are CUs, with one-, two- and twelve-stage reductions and ragged last row / column tiles
@pytest.mark.parametrize("M,N,K", [(300, 200, 128), (256, 2304, 768), (1024, 50304, 768), (640, 768, 3072),
                                   (2000, 9000, 64), (3000, 6000, 128)])
def test_gemm_nt_parity(gpu_lib, M, N, K):
    import torch
    from transformer_lm_pretraining_amd import lib
    say("gemm_nt", M, N, K)
    A = bf16_round(synth.normal((M, K), seed=51))
    B = bf16_round(synth.normal((N, K), std=0.02, seed=52))
    bias = synth.normal((N,), std=0.1, seed=53).astype(np.float64)
    res = bf16_round(synth.normal((M, N), seed=54))
    out = lib.gemm_nt(to_dev_bf16(A), to_dev_bf16(B), to_dev_f32(bias), to_dev_bf16(res))
    plain = lib.gemm_nt(to_dev_bf16(A), to_dev_bf16(B))
    torch.cuda.synchronize()
    ref = A @ B.T
    assert rel_l2(host(plain), ref) <= 5e-3
    assert rel_l2(host(out), ref + bias + res) <= 5e-3
    # element-wise, over every tile including the ragged last row and column tiles:
    # bf16 rounding of the result (2^-8 relative) and fp32 summation over K terms
    # (at most K u |A||B|^T), both doubled; with bias and residual the product may be
    # rounded once more before the residual is added
    S = abs_matmul(A, B.T)
    assert_elementwise(host(plain), ref, 2 * BF16 * np.abs(ref) + 2 * K * U32 * S, "gemm_nt")
    full = ref + bias + res
    tol = 2 * BF16 * (np.abs(full) + np.abs(ref + bias)) + 2 * K * U32 * (S + np.abs(bias))
    assert_elementwise(host(out), full, tol, "gemm_nt + bias + residual")


# small-shape kernel; 256x256-tile kernel with a ragged last row tile; 384 tiles (more than CUs)
@pytest.mark.parametrize("M", [333, 4000, 8000])
def test_gemm_nt_gelu_parity(gpu_lib, M):
    import torch
    from transformer_lm_pretraining_amd import lib
    N, K = 3072, 768
    say("gemm_nt_gelu", M, N, K)
    A = bf16_round(synth.normal((M, K), seed=61))
    B = bf16_round(synth.normal((N, K), std=0.05, seed=62))
    bias = synth.normal((N,), std=0.1, seed=63).astype(np.float64)
    gprime, g = lib.gemm_nt_gelu(to_dev_bf16(A), to_dev_bf16(B), to_dev_f32(bias))
    torch.cuda.synchronize()
    ref = A @ B.T + bias
    assert rel_l2(host(g), ops.gelu_fwd(ref)) <= 5e-3
    # the stored derivative of the pre-activation, GELU'(pre), for the backward
    assert rel_l2(host(gprime), ops.gelu_grad(ref)) <= 5e-3
    assert np.max(np.abs(host(gprime) - ops.gelu_grad(ref))) <= 2e-2
    # element-wise: pre is rounded to bf16 (2^-8 |pre| + K u |A||B|^T + |bias|), which
    # moves GELU by at most 1.13x that (|GELU'| <= 1.13) and GELU' by at most 0.85x
    # (|GELU''| <= 0.8); then each output is rounded to bf16; all doubled
    dpre = BF16 * np.abs(ref) + K * U32 * (abs_matmul(A, B.T) + np.abs(bias))
    g_r, gp_r = ops.gelu_fwd(ref), ops.gelu_grad(ref)
    assert_elementwise(host(g), g_r, 2 * (BF16 * np.abs(g_r) + 1.13 * dpre) + 1e-6, "gemm_nt_gelu g")
    assert_elementwise(host(gprime), gp_r, 2 * (BF16 * np.abs(gp_r) + 0.85 * dpre) + 1e-5, "gemm_nt_gelu gprime")


# (2048, 712, 768): 9 tiles split over tokens; (512, 3000, 5120): 240 tiles in one pass.  In both the last
# output-row tile is ragged (200 and 184 of 256 rows), so the bias sums of its waves are partly out of range.
@pytest.mark.parametrize("M,N,K", [(256, 128, 128), (19456, 768, 768), (2048, 50304, 768), (4096, 768, 3072),
                                   (2048, 712, 768), (512, 3000, 5120)])
def test_gemm_tn_acc_parity(gpu_lib, M, N, K):
    import torch
    from transformer_lm_pretraining_amd import lib
    say("gemm_tn", M, N, K)
    dY = bf16_round(synth.normal((M, N), std=0.1, seed=71))
    X = bf16_round(synth.normal((M, K), seed=72))
    dW0 = synth.normal((N, K), std=0.3, seed=73).astype(np.float64)
    db0 = synth.normal((N,), std=0.3, seed=74).astype(np.float64)
    dW = to_dev_f32(dW0)
    db = to_dev_f32(db0)
    lib.gemm_tn_acc(to_dev_bf16(dY), to_dev_bf16(X), dW, db)
    torch.cuda.synchronize()
    ref = dY.T @ X
    got = host(dW) - dW0.astype(np.float32)
    assert rel_l2(got, ref) <= 1e-4
    # element-wise: fp32 summation over the M tokens in any order (at most M u |dY|^T|X|,
    # doubled) and the rounding of the accumulated fp32 value
    tol = 2 * M * U32 * abs_matmul(dY.T, X) + 2 * U32 * (np.abs(dW0) + np.abs(ref))
    assert_elementwise(got, ref, tol, "gemm_tn_acc")
    np.testing.assert_allclose(host(db) - db0.astype(np.float32), dY.sum(0), rtol=1e-4, atol=1e-3)
    # without the bias pointer the weight gradient alone accumulates
    dW2 = to_dev_f32(np.zeros((N, K)))
    lib.gemm_tn_acc(to_dev_bf16(dY), to_dev_bf16(X), dW2)
    torch.cuda.synchronize()
    assert rel_l2(host(dW2), ref) <= 1e-4


@pytest.mark.parametrize("M", [515, 4000, 6900])  # 6900: 324 tiles (more than CUs), ragged last row tile
def test_gemm_nt_dgelu_parity(gpu_lib, M):
    import torch
    from transformer_lm_pretraining_amd import lib
    N, K = 3072, 768
    say("gemm_nt_dgelu", M, N, K)
    A = bf16_round(synth.normal((M, K), seed=65))
    B = bf16_round(synth.normal((N, K), std=0.05, seed=66))
    pre = bf16_round(synth.normal((M, N), seed=67))
    gprime = bf16_round(ops.gelu_grad(pre))  # what the forward stores for this pre-activation
    out = lib.gemm_nt_dgelu(to_dev_bf16(A), to_dev_bf16(B), to_dev_bf16(gprime))
    torch.cuda.synchronize()
    AB = A @ B.T
    ref = ops.gelu_bwd(pre, AB)
    assert rel_l2(host(out), ref) <= 5e-3
    # element-wise: the stored GELU' is bf16 (2^-8 relative), the product's fp32 sum
    # (K u |A||B|^T |GELU'|) and the output rounding (2^-8), all doubled
    tol = 2 * (2 * BF16 * np.abs(ref) + K * U32 * abs_matmul(A, B.T) * np.abs(gprime))
    assert_elementwise(host(out), ref, tol, "gemm_nt_dgelu")


# ---------------------------------------------------------------- attention

def _split(qkv, B, T, H, C):
    d = C // H
    q = qkv[:, :C].reshape(B, T, H, d).transpose(0, 2, 1, 3)
    k = qkv[:, C:2 * C].reshape(B, T, H, d).transpose(0, 2, 1, 3)
    v = qkv[:, 2 * C:].reshape(B, T, H, d).transpose(0, 2, 1, 3)
    return q, k, v


def _merge(a):
    B, H, T, d = a.shape
    return a.transpose(0, 2, 1, 3).reshape(B * T, H * d)


def attention_bounds(q, k, v, p, o, do, dq, dk, dv):
    """Element-wise error bounds for O, dQ, dK, dV (head layout [..., T, d]), from the
    oracle's values.  The kernels round P to bf16 before P.V and again when they recompute
    it in the backward (2^-8 relative), round dS = P (dP - D) to bf16 (2^-8 more) and
    round every output to bf16; fp32 sums over at most T terms add T u of the same scales.
    |dS| is bounded by P (|dP| + |D|), which holds where dP - D cancels.  All doubled."""
    T, d = q.shape[-2], q.shape[-1]
    sc = 1.0 / math.sqrt(d)
    tr = lambda a: np.swapaxes(a, -1, -2)
    dP = do @ tr(v)
    D = (do * o).sum(-1, keepdims=True)
    sum_err = d * U32 * (np.abs(do) @ tr(np.abs(v)) + (np.abs(do) * np.abs(o)).sum(-1, keepdims=True))
    W = p * (np.abs(dP) + np.abs(D) + sum_err)
    tol_o = 2 * ((BF16 + T * U32) * (p @ np.abs(v)) + BF16 * np.abs(o))
    tol_dv = 2 * ((BF16 + T * U32) * (tr(p) @ np.abs(do)) + BF16 * np.abs(dv))
    tol_dq = 2 * ((2 * BF16 + T * U32) * sc * (W @ np.abs(k)) + BF16 * np.abs(dq))
    tol_dk = 2 * ((2 * BF16 + T * U32) * sc * (tr(W) @ np.abs(q)) + BF16 * np.abs(dk))
    return tol_o, tol_dq, tol_dk, tol_dv


@pytest.mark.parametrize("B,T,H,C", [(2, 256, 4, 256), (3, 192, 4, 128), (1, 64, 2, 128), (1, 1024, 12, 768)])
def test_attention_parity(gpu_lib, B, T, H, C):
    import torch
    from transformer_lm_pretraining_amd import lib
    say("attention", B, T, H, C)
    qkv = bf16_round(synth.normal((B * T, 3 * C), seed=81))
    dout = bf16_round(synth.normal((B * T, C), seed=82))
    qd = to_dev_bf16(qkv)
    out, lse = lib.attention_fwd(qd, B, T, H, C)
    dqkv = lib.attention_bwd(qd, out, to_dev_bf16(dout), lse, B, T, H, C)
    torch.cuda.synchronize()
    q, k, v = _split(qkv, B, T, H, C)
    o, p, lse_r = ops.attention_fwd(q, k, v)
    assert rel_l2(host(out), _merge(o)) <= 1e-2
    np.testing.assert_allclose(host(lse), lse_r, atol=2e-3)
    do = _split(np.concatenate([dout] * 3, 1), B, T, H, C)[0]
    dq, dk, dv = ops.attention_bwd(do, q, k, v, p)
    tols = attention_bounds(q, k, v, p, o, do, dq, dk, dv)
    assert_elementwise(host(out), _merge(o), _merge(tols[0]), "attention O")
    g = host(dqkv)
    for part, ref, tol in zip(range(3), (dq, dk, dv), tols[1:]):
        got = g[:, part * C:(part + 1) * C]
        assert rel_l2(got, _merge(ref)) <= 2e-2, part
        assert cosine(got, _merge(ref)) >= 0.999, part
        assert_elementwise(got, _merge(ref), _merge(tol), f"attention d{'qkv'[part]}")


@pytest.mark.parametrize("slope", [0.1, -0.1])
def test_attention_drifting_scores(gpu_lib, slope):
    """Scores that rise (or fall) by ~6 nats per 64-key block: the forward's
    running reference max has to move on later blocks, not only the first."""
    import torch
    from transformer_lm_pretraining_amd import lib
    B, T, H, C = 1, 512, 2, 128
    d = C // H
    say("attention drifting", slope)
    qkv = synth.normal((B * T, 3 * C), std=0.3, seed=83)
    pos = np.arange(T, dtype=np.float64)[:, None]
    for h in range(H):
        qkv[:, h * d:(h + 1) * d] += 1.0                                # q ~ all-ones direction
        qkv[:, C + h * d:C + (h + 1) * d] += slope * 8.0 * pos / d      # q.k/sqrt(d) ~ slope * key index
    qkv = bf16_round(qkv)
    out, lse = lib.attention_fwd(to_dev_bf16(qkv), B, T, H, C)
    torch.cuda.synchronize()
    q, k, v = _split(qkv, B, T, H, C)
    o, p, lse_r = ops.attention_fwd(q, k, v)
    assert rel_l2(host(out), _merge(o)) <= 1e-2
    tol_o = 2 * ((BF16 + T * U32) * (p @ np.abs(v)) + BF16 * np.abs(o))
    assert_elementwise(host(out), _merge(o), _merge(tol_o), "attention O, drifting scores")
    np.testing.assert_allclose(host(lse), lse_r, atol=2e-3 * max(1.0, np.abs(lse_r).max() / 8))


def test_attention_full_size_sampled_heads(gpu_lib):
    import torch
    from transformer_lm_pretraining_amd import lib
    B, T, H, C = 19, 1024, 12, 768
    say("attention full", B, T, H, C)
    qkv = bf16_round(synth.normal((B * T, 3 * C), seed=91))
    dout = bf16_round(synth.normal((B * T, C), seed=92))
    qd = to_dev_bf16(qkv)
    out, lse = lib.attention_fwd(qd, B, T, H, C)
    dqkv = lib.attention_bwd(qd, out, to_dev_bf16(dout), lse, B, T, H, C)
    torch.cuda.synchronize()
    og, dg = host(out), host(dqkv)
    d = C // H
    for b, h in ((0, 0), (18, 11), (7, 5)):
        rows = slice(b * T, (b + 1) * T)
        cols = slice(h * d, (h + 1) * d)
        q = qkv[rows, cols][None, None]
        k = qkv[rows, C + h * d:C + (h + 1) * d][None, None]
        v = qkv[rows, 2 * C + h * d:2 * C + (h + 1) * d][None, None]
        o, p, lse_r = ops.attention_fwd(q, k, v)
        assert rel_l2(og[rows, cols], o[0, 0]) <= 1e-2
        np.testing.assert_allclose(host(lse)[b, h], lse_r[0, 0], atol=2e-3)
        do = dout[rows, cols][None, None]
        dq, dk, dv = ops.attention_bwd(do, q, k, v, p)
        tols = attention_bounds(q, k, v, p, o, do, dq, dk, dv)
        assert_elementwise(og[rows, cols], o[0, 0], tols[0][0, 0], f"attention O head ({b},{h})")
        for off, ref, tol in ((0, dq, tols[1]), (C, dk, tols[2]), (2 * C, dv, tols[3])):
            got = dg[rows, off + h * d:off + (h + 1) * d]
            assert rel_l2(got, ref[0, 0]) <= 2e-2
            assert cosine(got, ref[0, 0]) >= 0.999
            assert_elementwise(got, ref[0, 0], tol[0, 0], f"attention grad head ({b},{h}) part {off // C}")


# ---------------------------------------------------------------- embedding

def test_embedding_parity(gpu_lib):
    import torch
    from transformer_lm_pretraining_amd import lib
    B, T, C, V, Vp = 4, 256, 768, 50257, 50304
    say("embedding", B, T, C)
    tok, _ = synth.micro_batches(1, B, T, V, seed=3)[0]
    wte = bf16_round(synth.normal((Vp, C), std=0.02, seed=101))
    wpe = bf16_round(synth.normal((T, C), std=0.02, seed=102))
    x = lib.embedding_fwd(to_dev_i32(tok), to_dev_bf16(wte), to_dev_bf16(wpe), V)
    dx = bf16_round(synth.normal((B * T, C), seed=103))
    dwte = to_dev_f32(np.zeros((Vp, C)))
    dwpe = to_dev_f32(np.zeros((T, C)))
    lib.embedding_bwd(to_dev_i32(tok), to_dev_bf16(dx), dwte, dwpe, V)
    torch.cuda.synchronize()
    ref = ops.embedding_fwd(wte, wpe, tok).reshape(B * T, C)
    assert np.all(np.abs(host(x) - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-9)
    rw, rp = ops.embedding_bwd(dx.reshape(B, T, C), tok, Vp, T)
    np.testing.assert_allclose(host(dwte), rw, rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(host(dwpe), rp, rtol=1e-5, atol=1e-5)
    assert np.all(host(dwte)[V:] == 0)


def test_embedding_bwd_hot_tokens_and_invalid_ids(gpu_lib):
    """Token-table scatter at the full batch (Zipf ids: token 0 covers ~14% of rows), plus
    a batch where one id fills 300 rows (runs crossing many sorting windows) and ids
    outside [0, V) that must be skipped, and a batch of 71,680 rows (two sort chunks).
    A second call gives the same bits (the rows of a token are summed in a fixed order)."""
    import torch
    from transformer_lm_pretraining_amd import lib
    V, Vp = 50257, 50304
    for case in ("zipf_full", "hot_invalid", "over_65535_rows"):
        C = 128 if case == "over_65535_rows" else 768
        if case == "zipf_full":
            B, T = 19, 1024
            tok, _ = synth.micro_batches(1, B, T, V, seed=11)[0]
        elif case == "over_65535_rows":  # the sort works on chunks of at most 65,535 rows
            B, T = 70, 1024
            tok, _ = synth.micro_batches(1, B, T, V, seed=14)[0]
        else:
            B, T = 2, 512
            tok = np.ascontiguousarray(synth.micro_batches(1, B, T, V, seed=12)[0][0])
            flat = tok.reshape(-1)
            assert np.shares_memory(flat, tok)
            flat[np.arange(5, 1024, 3)[:300]] = 7
            flat[[0, 100, 777]] = [-1, V + 3, V]
        say("embedding_bwd", case, B, T)
        dx = bf16_round(synth.normal((B * T, C), seed=13))
        dwte = to_dev_f32(np.zeros((Vp, C)))
        dwpe = to_dev_f32(np.zeros((T, C)))
        lib.embedding_bwd(to_dev_i32(tok), to_dev_bf16(dx), dwte, dwpe, V)
        torch.cuda.synchronize()
        valid = (tok.reshape(-1) >= 0) & (tok.reshape(-1) < V)
        tok_ref = np.where(valid, tok.reshape(-1), 0).reshape(B, T)
        dx_ref = np.where(valid[:, None], dx, 0.0).astype(np.float32)
        rw, rp = ops.embedding_bwd(dx_ref.reshape(B, T, C), tok_ref, Vp, T)
        _, rp = ops.embedding_bwd(dx.reshape(B, T, C), tok_ref, Vp, T)  # positions take every row
        np.testing.assert_allclose(host(dwte), rw, rtol=1e-5, atol=1e-4)
        np.testing.assert_allclose(host(dwpe), rp, rtol=1e-5, atol=1e-5)
        assert np.all(host(dwte)[V:] == 0)
        again = to_dev_f32(np.zeros((Vp, C)))
        lib.embedding_bwd(to_dev_i32(tok), to_dev_bf16(dx), again, to_dev_f32(np.zeros((T, C))), V)
        torch.cuda.synchronize()
        assert torch.equal(dwte, again)


# ---------------------------------------------------------------- clip + AdamW

@pytest.mark.parametrize("gscale", [1e-4, 1.0])
def test_clip_adamw_parity(gpu_lib, gscale):
    import torch
    from transformer_lm_pretraining_amd import lib
    n, n_decay = 1 << 20, 700 * 1024
    say("adamw", n, gscale)
    p = synth.normal((n,), std=0.02, seed=111)
    g = synth.normal((n,), std=gscale, seed=112)
    m = synth.normal((n,), std=1e-3, seed=113)
    v = np.abs(synth.normal((n,), std=1e-4, seed=114))
    mask = np.arange(n) < n_decay
    t, lr = 5, 3e-4
    pd, gd, md, vd = (to_dev_f32(a) for a in (p, g, m, v))
    shadow = torch.empty(n_decay, dtype=torch.bfloat16, device="cuda")
    norm = lib.clip_adamw(pd, gd, md, vd, shadow, n_decay, lr, t)
    torch.cuda.synchronize()
    pr, mr, vr, nr = oracle.clip_adamw(p, g, m, v, mask, t, lr)
    assert abs(float(norm.item()) - nr) <= 1e-6 * nr
    # 1e-6 relative to the magnitudes that enter each update (the stored value can
    # cancel to ~0, where a relative bound on the result alone is meaningless)
    s = min(1.0, 1.0 / nr)
    gs = np.abs(g.astype(np.float64)) * s
    m_scale = 0.9 * np.abs(m) + 0.1 * gs
    v_scale = 0.95 * v + 0.05 * gs * gs
    mhat = m_scale / (1 - 0.9 ** t)
    vhat = v_scale / (1 - 0.95 ** t)
    p_scale = np.abs(p) + lr * (mhat / (np.sqrt(np.abs(vr) / (1 - 0.95 ** t)) + 1e-8) + 0.1 * np.abs(p))
    for got, ref, scale in ((pd, pr, p_scale), (md, mr, m_scale), (vd, vr, v_scale)):
        gh = got.cpu().numpy()
        err = np.abs(gh.astype(np.float64) - ref.astype(np.float64))
        bound = 1e-6 * np.maximum(np.abs(ref.astype(np.float64)), scale) + 1e-30
        assert np.all(err <= bound), float((err / bound).max())
    assert np.all(gd.cpu().numpy() == 0)
    sh = shadow.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(sh, bf16_rne_bits(pd.cpu().numpy()[:n_decay]))


# ---------------------------------------------------------------- empty inputs

def test_zero_rows_are_no_ops(gpu_lib):
    """rows = 0 through the C ABI: status OK, no output element written and no
    gradient accumulated (the buffers are real; only the row count is zero)."""
    import torch
    from transformer_lm_pretraining_amd import lib
    say("zero rows")
    L, st = lib.load(), lib._stream()
    P = lib._ptr
    C, N, Vp = 256, 256, 128
    x = torch.full((4, C), 1.5, dtype=torch.bfloat16, device="cuda")
    y = torch.full((4, C), -7.0, dtype=torch.bfloat16, device="cuda")
    w = torch.ones(C, dtype=torch.float32, device="cuda")
    stats = torch.full((2, 4), 3.0, dtype=torch.float32, device="cuda")
    acc = torch.full((2, N), 0.25, dtype=torch.float32, device="cuda")
    z = torch.full((4, Vp), 2.0, dtype=torch.bfloat16, device="cuda")
    tgt = torch.zeros(4, dtype=torch.int32, device="cuda")
    loss = torch.full((4,), 9.0, dtype=torch.float32, device="cuda")
    s = lib._scratch(1 << 16)
    before = [t.clone() for t in (x, y, stats, acc, z, loss)]
    assert L.gpt2k_xent(P(z), P(tgt), P(loss), 0, 100, Vp, 1.0, 1, None, st) == 0
    assert L.gpt2k_layernorm_fwd(P(x), P(w), P(w), P(y), P(stats[0]), P(stats[1]), 0, C, st) == 0
    assert L.gpt2k_layernorm_bwd(P(x), P(x), P(w), P(stats[0]), P(stats[1]), P(y), 1, P(acc[0]), P(acc[1]), P(s),
                                 s.numel(), 0, C, st) == 0
    assert L.gpt2k_bias_gelu_fwd(P(x), P(w), P(y), P(y), 0, N, st) == 0
    assert L.gpt2k_bias_gelu_bwd(P(x), P(x), P(y), P(acc[0]), P(s), s.numel(), 0, N, st) == 0
    assert L.gpt2k_bias_grad(P(x), P(acc[1]), P(s), s.numel(), 0, N, st) == 0
    torch.cuda.synchronize()
    for a, b in zip(before, (x, y, stats, acc, z, loss)):
        assert torch.equal(a, b)
