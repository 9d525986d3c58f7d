"""Kernel timing through the C ABI (gpt2_prof_enable / gpt2_prof_read), which the
bench's roofline is built on: every launch of a class is counted once, its
algorithmic work is the sum of 2*M*N*K over the products it ran (from the shapes
of the step's products, computed here independently), and the durations the
launches record at each kernel's start and end are positive and fit inside the
step's wall time."""
import time

import numpy as np
import pytest

import oracle
from oracle.model import CONFIGS, init_params
from transformer_lm_pretraining_amd import synth
from gpu_util import to_dev_i32

pytestmark = pytest.mark.gpu


def _one_pass(model, td, gd, dloss):
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    model.forward(td, gd, dloss=dloss)
    model.backward()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def test_kernel_timing_counts_work_and_durations(gpu_lib):
    from transformer_lm_pretraining_amd import lib
    cfg = CONFIGS["tiny"]
    L, H, C, Vp = cfg.L, cfg.H, cfg.C, cfg.Vp
    B, T = 4, 64
    BT, D = B * T, cfg.C // cfg.H
    print("prof: tiny model, one forward + backward with every class timed", flush=True)
    model = lib.GPT2(lib.make_config(L, H, C, cfg.V, Vp, cfg.Tmax, B, T), init=oracle.flatten(cfg, init_params(cfg, 1337)))
    tok, tgt = synth.micro_batches(1, B, T, cfg.V, seed=53)[0]
    td, gd = to_dev_i32(tok), to_dev_i32(tgt)
    dloss = 1.0 / BT
    _one_pass(model, td, gd, dloss)  # warm
    names = {v: k for k, v in lib.kernel_class_names().items()}
    model.prof_enable(-1)
    wall_ms = _one_pass(model, td, gd, dloss) * 1e3
    got = {n: model.prof_read(names[n]) for n in names}
    model.prof_enable(0)

    # launches per class, from the structure of one forward (with targets) and backward
    expect_n = {"embedding_fwd": 1, "layernorm_fwd": 2 * L + 1, "layernorm_bwd": 2 * L + 1, "attn_fwd": L,
                "attn_dq": L, "attn_dkdv": L, "xent": 1, "mean": 1,
                "gemm_nt": 2 * (3 * L + 1), "gemm_nt_gelu": L, "gemm_nt_dgelu": L}
    for n, k in expect_n.items():
        assert got[n][1] == k, (n, got[n])
    # algorithmic work: sum of 2 M N K over the class's products
    nt = 2 * BT * (16 * L * C * C + 2 * Vp * C)  # QKV, projection, FC-proj and lm_head, forward and input gradient
    assert got["gemm_nt"][2] == pytest.approx(nt, rel=1e-12)
    assert got["gemm_nt_gelu"][2] == pytest.approx(2 * BT * 4 * C * C * L, rel=1e-12)
    assert got["gemm_nt_dgelu"][2] == pytest.approx(2 * BT * 4 * C * C * L, rel=1e-12)
    tn = got["gemm_tn_acc"][2] + got["gemm_tn_splitk"][2]
    assert tn == pytest.approx(2 * BT * (12 * L * C * C + Vp * C), rel=1e-12)
    pairs = B * H * T * (T + 1) / 2  # causal (query, key) pairs of one layer
    assert got["attn_fwd"][2] == pytest.approx(L * pairs * 2 * D * 2, rel=1e-12)  # S = Q K^T and O = P V
    # durations: every recorded class took time, and all of them fit in the pass
    total = 0.0
    for n, (ms, cnt, _) in got.items():
        if cnt:
            assert np.isfinite(ms) and ms > 0.0, (n, ms)
            total += ms
    assert total <= wall_ms, (total, wall_ms)

    # a single class: the same launches and work, nothing else recorded
    model.prof_enable(names["gemm_nt"])
    _one_pass(model, td, gd, dloss)
    only = model.prof_read(-1)
    model.prof_enable(0)
    assert only[1] == got["gemm_nt"][1] and only[2] == pytest.approx(nt, rel=1e-12)
