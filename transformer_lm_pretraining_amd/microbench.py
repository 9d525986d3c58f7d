"""Kernel microbench at one card's micro-batch shape: the memory-bound kernels of the
step on their own, through the kernel-level C ABI (include/gpt2mi_kernels.h).

  - fused masked softmax cross-entropy forward + backward, in place, on 19,456 x 50,304
    bf16 logits ~ N(0, 1) (the softmax over the 50,257 real columns; Pretraining and
    adapting a language model on a dependency-free stack, vocabulary padding paragraph);
  - LayerNorm forward and backward (accumulating the residual-stream gradient) on
    19,456 x 768, fp32 statistics (same page, precision paragraph);
  - bias + GELU forward and backward on 19,456 x 3,072 (the stand-alone kernels; the
    training step fuses both into its GEMM epilogues).

Each launch is bracketed by HIP events on its stream; a kernel's figure is the median of
20 launches after 5 warmups.  Inputs rotate over copies totalling at least 1 GiB, so the
256 MB last-level cache cannot hold them between launches.  Bytes are the algorithmic
ones (each operand read once, each result written once), and the rate is compared with
the 8 TB/s HBM3E peak.

    python -m transformer_lm_pretraining_amd.microbench [--rows 19456]
"""
from __future__ import annotations

import argparse
import json
import math

from . import lib, synth

PEAK_HBM = 8.0e12
ROTATE_BYTES = 1 << 30


def _time(fn, n_sets, warmup=5, reps=20):
    """Median ms of fn(i) over reps launches (set i % n_sets), each bracketed by events."""
    import torch
    for i in range(warmup):
        fn(i % n_sets)
    ts = []
    for i in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn((warmup + i) % n_sets)
        e1.record()
        ts.append((e0, e1))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ts)
    return ms[len(ms) // 2]


def _sets(bytes_per_set):
    return max(1, math.ceil(ROTATE_BYTES / bytes_per_set))


def run(rows=19456, C=768, N=3072, V=50257, Vp=50304, seed=1337):
    import torch
    L = lib.load()
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    bf = torch.bfloat16
    s = lib._stream()

    def randn(*shape, std=1.0, dtype=bf):
        return (torch.randn(*shape, generator=gen, device=dev) * std).to(dtype)

    out = []

    def report(name, nbytes, ms, sets):
        rate = nbytes / (ms * 1e-3)
        rec = {"kernel": name, "rows": rows, "bytes": int(nbytes), "median_us": round(ms * 1e3, 2),
               "TB_per_s": round(rate / 1e12, 3), "frac_of_8TBps": round(rate / PEAK_HBM, 3), "input_sets": sets}
        out.append(rec)
        print(json.dumps(rec), flush=True)

    # cross-entropy: one logits buffer is already far larger than the cache
    T = 1024 if rows % 1024 == 0 else rows
    _, tgt = synth.micro_batches(1, rows // T, T, V, seed=seed)[0]
    tgt_d = torch.from_numpy(tgt.reshape(-1)).to(dev)
    logits = randn(rows, Vp)
    loss = torch.empty(rows, dtype=torch.float32, device=dev)
    dloss = 1.0 / rows

    def ce(_):
        lib.check(L.gpt2k_xent(lib._ptr(logits), lib._ptr(tgt_d), lib._ptr(loss), rows, V, Vp, dloss, 1, None, s),
                  "gpt2k_xent")
    report("xent fwd+bwd (in place)", 2 * 2 * rows * Vp + 4 * rows + 4 * rows, _time(ce, 1), 1)
    del logits

    # LayerNorm forward
    per = 2 * 2 * rows * C + 8 * rows
    n = _sets(per)
    w = (1.0 + 0.1 * torch.randn(C, generator=gen, device=dev)).float()
    b = (0.1 * torch.randn(C, generator=gen, device=dev)).float()
    xs = [randn(rows, C) for _ in range(n)]
    ys = [torch.empty(rows, C, dtype=bf, device=dev) for _ in range(n)]
    means = [torch.empty(rows, dtype=torch.float32, device=dev) for _ in range(n)]
    rstds = [torch.empty(rows, dtype=torch.float32, device=dev) for _ in range(n)]

    def lnf(i):
        lib.check(L.gpt2k_layernorm_fwd(lib._ptr(xs[i]), lib._ptr(w), lib._ptr(b), lib._ptr(ys[i]),
                                        lib._ptr(means[i]), lib._ptr(rstds[i]), rows, C, s), "gpt2k_layernorm_fwd")
    report("layernorm fwd", per, _time(lnf, n), n)

    # LayerNorm backward: x, dy, dres in; dres out; statistics in
    per_b = 4 * 2 * rows * C + 8 * rows
    nb = max(1, min(n, _sets(per_b)))
    dys = [randn(rows, C) for _ in range(nb)]
    dres = [randn(rows, C) for _ in range(nb)]
    dw = torch.zeros(C, dtype=torch.float32, device=dev)
    db = torch.zeros(C, dtype=torch.float32, device=dev)
    sb = lib.scratch_bytes(1, rows, C)
    scr = torch.empty(max(256, sb), dtype=torch.uint8, device=dev)

    def lnb(i):
        lib.check(L.gpt2k_layernorm_bwd(lib._ptr(xs[i]), lib._ptr(dys[i]), lib._ptr(w), lib._ptr(means[i]),
                                        lib._ptr(rstds[i]), lib._ptr(dres[i]), 1, lib._ptr(dw), lib._ptr(db),
                                        lib._ptr(scr), scr.numel(), rows, C, s), "gpt2k_layernorm_bwd")
    report("layernorm bwd (accumulating)", per_b, _time(lnb, nb), nb)  # statistics from the forward runs above
    del xs, ys, dys, dres

    # bias + GELU forward and backward
    per_g = 3 * 2 * rows * N
    ng = _sets(per_g)
    bias = (0.02 * torch.randn(N, generator=gen, device=dev)).float()
    us = [randn(rows, N) for _ in range(ng)]
    pres = [torch.empty(rows, N, dtype=bf, device=dev) for _ in range(ng)]
    gs = [torch.empty(rows, N, dtype=bf, device=dev) for _ in range(ng)]

    def gf(i):
        lib.check(L.gpt2k_bias_gelu_fwd(lib._ptr(us[i]), lib._ptr(bias), lib._ptr(pres[i]), lib._ptr(gs[i]),
                                        rows, N, s), "gpt2k_bias_gelu_fwd")
    report("bias+gelu fwd", per_g, _time(gf, ng), ng)
    dbg = torch.zeros(N, dtype=torch.float32, device=dev)
    sg = lib.scratch_bytes(2, rows, N)
    scr2 = torch.empty(max(256, sg), dtype=torch.uint8, device=dev)
    dgs = [randn(rows, N) for _ in range(ng)]

    def gb(i):  # dpre into gs[i] (the forward's g, no longer needed)
        lib.check(L.gpt2k_bias_gelu_bwd(lib._ptr(pres[i]), lib._ptr(dgs[i]), lib._ptr(gs[i]), lib._ptr(dbg),
                                        lib._ptr(scr2), scr2.numel(), rows, N, s), "gpt2k_bias_gelu_bwd")
    report("bias+gelu bwd", per_g, _time(gb, ng), ng)
    torch.cuda.synchronize()
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--rows", type=int, default=19456)
    a = ap.parse_args(argv)
    import torch
    torch.cuda.set_device(0)
    run(rows=a.rows)


if __name__ == "__main__":
    main()
