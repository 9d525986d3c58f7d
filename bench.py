#!/usr/bin/env python3
"""Training-throughput benchmark: GPT-2 124M on one MI355X, one card's share of
the pretraining recipe (Pretraining and adapting a language model on a
dependency-free stack, §4.4: 19 sequences x 1,024 tokens x 9 accumulation
micro-steps per optimizer step; §4 optimisation: clip 1.0 + AdamW).

A step = 9 x (gpt2_forward + gpt2_backward) + gpt2_clip_adamw at the
warmup-step-350 learning rate, all on device-resident synthetic Zipf/EOT
tokens.  Prints one JSON line (rank 0): tokens/s, MFU against the bf16 dense
MFMA peak, the roofline of the dominant kernel (HIP events recorded at each of
its launches' start and end, on steps run right after the timed region) and the
CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15     # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12      # MI355X HBM3E, B/s
METRIC = "GPT-2 124M train tokens/s on 1 MI355X (19x1024x9 accum); MFU vs bf16 peak"

# HBM traffic per launch from two rocprofv3 counter runs (FETCH_SIZE, then WRITE_SIZE,
# KiB per dispatch averaged over the gpt2_124m workload), each scaled by what the same
# counter reads for a plain 1 GiB copy (read x2.000, write x1.000).  Valid only for the
# kernel sources the counters were taken on: a changed source reports null.
TRAFFIC_COUNTERS = {
    ("gpt2_124m", "gemm_nt"): {
        "sources": {"k_gemm.hip": "b8344409dd37bdfedee803c7278cbaba12df931c50d43d6d5f0bb6aa3237cf0e",
                    "common.h": "cf6fa5b5bb317912ce3a6971f3641f290fff999d25ba220d2eb2b451f72c2ecd"},
        "fetch_kib": 96527.00, "fetch_scale": 1.99994, "write_kib": 64086.49, "write_scale": 1.0,
    },
}


def counted_traffic(workload, kernel):
    """Bytes per launch from the counter runs, or None when none were taken for this
    kernel and workload or its sources changed since."""
    import hashlib
    rec = TRAFFIC_COUNTERS.get((workload, kernel))
    if rec is None:
        return None
    csrc = os.path.join(ROOT, "transformer_lm_pretraining_amd", "csrc")
    for name, digest in rec["sources"].items():
        with open(os.path.join(csrc, name), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != digest:
                return None
    return round((rec["fetch_kib"] * rec["fetch_scale"] + rec["write_kib"] * rec["write_scale"]) * 1024)

WORKLOADS = {
    # name: (L, H, C, V, Vp, Tmax, B, T, n_micro)
    "gpt2_124m": (12, 12, 768, 50257, 50304, 1024, 19, 1024, 9),
    "wide_16l_1536": (16, 24, 1536, 8449, 8576, 1024, 8, 1024, 8),
}


def flop_per_token(L, H, C, V, T):
    """Algorithmic training FLOP per token: 3 x forward (linear 24 C^2 L, causal attention
    2 C (T+1) L, lm_head over the real vocabulary 2 C V)."""
    return 3 * (24 * C * C * L + 2 * C * (T + 1) * L + 2 * C * V)


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(L, H, C, V, Vp, Tmax, T_sample, B_sample=3, n_adam=1 << 24, tokens_per_step=175104):
    """The oracle (NumPy fp32) on the host cores: B_sample whole sequences of T_sample tokens
    (the workload's sequence length, so attention's quadratic term is at full size)
    forward+backward through the full model, plus clip+AdamW on n_adam parameters,
    scaled to the whole parameter count and amortised over the step's tokens."""
    import numpy as np
    import oracle
    from oracle.model import Config, tensor_specs
    from transformer_lm_pretraining_amd import synth
    cfg = Config(L=L, H=H, C=C, V=V, Vp=Vp, Tmax=Tmax)
    P = {}
    for i, (name, shape, dec) in enumerate(tensor_specs(cfg)):
        P[name] = synth.normal(shape, std=0.02, seed=1000 + i) if dec else np.ones(shape, np.float32)
    tok, tgt = synth.micro_batches(1, B_sample, T_sample, V, seed=5)[0]
    t0 = time.perf_counter()
    oracle.loss_and_grads(cfg, P, tok, tgt, dtype=np.float32)
    t_fb = time.perf_counter() - t0
    p = synth.normal((n_adam,), std=0.02, seed=7)
    g = synth.normal((n_adam,), std=1e-3, seed=8)
    z = np.zeros(n_adam, np.float32)
    t0 = time.perf_counter()
    oracle.clip_adamw(p, g, z, z, np.ones(n_adam, bool), 350, oracle.lr_at(350))
    t_adam = time.perf_counter() - t0
    n_params = oracle.n_params(cfg)
    t_tok = t_fb / (B_sample * T_sample) + t_adam * (n_params / n_adam) / tokens_per_step
    cores = len(os.sched_getaffinity(0))
    return {"value": round(1.0 / t_tok, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": (f"full model, {B_sample} sequences x {T_sample} tokens forward+backward in fp32 ({t_fb:.1f} s) "
                       f"+ clip/AdamW on {n_adam} params ({t_adam:.2f} s) scaled to {n_params} params "
                       f"and amortised over {tokens_per_step} tokens/step")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gpt2_124m", choices=sorted(WORKLOADS))
    ap.add_argument("--lanes", type=int, default=2,
                    help="micro-steps in flight at once, each lane on its own stream (1 = all on one stream)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-roofline", action="store_true", help="skip the per-kernel event timing")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (HBM counter calibration)")
    args = ap.parse_args()

    if args.calibrate_copy:
        import torch
        torch.cuda.set_device(0)
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 2, "copy_bytes_written": dst.numel() * 2,
                          "launches": 5}), flush=True)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the training step runs on one GPU only; --gpus > 1 (or WORLD_SIZE > 1) is not "
              "supported.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from transformer_lm_pretraining_amd import lib, synth
    from transformer_lm_pretraining_amd.train import lr_at

    L, H, C, V, Vp, Tmax, B, T, n_micro = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    cfg = lib.make_config(L, H, C, V, Vp, Tmax, B, T)
    model = lib.GPT2(cfg, seed=1337)
    nl = max(1, min(args.lanes, n_micro, 1 + lib.MAX_LANES))
    lanes = [model] + [model.add_lane() for _ in range(nl - 1)]
    main_stream = torch.cuda.current_stream()
    streams = [torch.cuda.Stream() for _ in range(nl)] if nl > 1 else [main_stream]
    n_steps = args.warmup + 1 + args.steps + 5  # warmup, breakdown, timed and roofline steps
    toks = synth.token_stream(n_steps * n_micro * B * T + 1, V)
    data = torch.from_numpy(toks).cuda()  # device-resident before timing
    BT = B * T
    tokens_per_step = BT * n_micro
    dloss = 1.0 / tokens_per_step
    losses = torch.zeros(n_micro, dtype=torch.float32, device="cuda")
    t_adam = 350

    def step(i, serial=False):
        """Micro-step k runs on lane k % nl, each lane on its own stream; lane 1 starts once
        lane 0's first forward is done, so a forward of one lane meets a backward of the other.
        serial: every micro-step on the main stream (the same lanes, so the same arithmetic)."""
        st = [main_stream] * nl if serial else streams
        for x in st:
            x.wait_stream(main_stream)  # the last update is done
        first_fwd = torch.cuda.Event()
        for k in range(n_micro):
            base = (i * n_micro + k) * BT
            tok = data[base:base + BT].view(B, T)
            tgt = data[base + 1:base + 1 + BT].view(B, T)
            j = k % nl
            with torch.cuda.stream(st[j]):
                if k == 1 and nl > 1:
                    st[1].wait_event(first_fwd)
                lanes[j].forward(tok, tgt, dloss=dloss, loss_out=losses[k:k + 1])
                if k == 0 and nl > 1:
                    first_fwd.record(st[0])
                lanes[j].backward()
        for x in st:
            main_stream.wait_stream(x)
        model.clip_adamw(lr_at(t_adam), t_adam)

    say(f"bench: {args.workload} B={B} T={T} x{n_micro} micro-steps; warmup {args.warmup}, timed {args.steps}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    say(f"warmup done, loss {float(losses.mean()):.4f}")

    names = lib.kernel_class_names()
    breakdown, dominant = {}, None
    def prof_enable(k):
        for ln in lanes:
            ln.prof_enable(k)

    def prof_read(k):
        tot = [0.0, 0, 0.0]
        for ln in lanes:
            for q, x in enumerate(ln.prof_read(k)):
                tot[q] += x
        return tot

    if not args.no_roofline:
        # per-kernel breakdown: one step with every launch timed, its micro-steps one after another
        prof_enable(-1)
        step(args.warmup, serial=True)
        for k, n in names.items():
            ms, cnt, work = prof_read(k)
            if cnt:
                breakdown[n] = {"ms_per_step": round(ms, 3), "launches": cnt}
        prof_enable(0)
        dominant = max(breakdown, key=lambda n: breakdown[n]["ms_per_step"])
        dom_id = [k for k, n in names.items() if n == dominant][0]
        tot = sum(v["ms_per_step"] for v in breakdown.values())
        say("per-kernel ms/step (event-timed): " + ", ".join(
            f"{n} {v['ms_per_step']:.2f}" for n, v in sorted(breakdown.items(), key=lambda x: -x[1]["ms_per_step"])))
        say(f"sum {tot:.1f} ms; dominant kernel: {dominant}")

    first = args.warmup + 1
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(args.steps):
        step(first + i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    per_step = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    last_loss = float(losses.mean())
    if not math.isfinite(last_loss):
        say(f"loss is not finite: {last_loss}")
        sys.exit(1)

    roof = None
    if dominant is not None:
        # The dominant class timed launch by launch on its stream.  With lanes the timed
        # region overlaps kernels of different lanes, so a launch's duration there is not
        # the kernel's own; this region runs the next steps of the same workload with the
        # micro-steps one after another, every launch of the class bracketed by events.
        n_roof = max(1, min(args.steps, 5))
        prof_enable(dom_id)
        torch.cuda.synchronize()
        r0 = time.perf_counter()
        for i in range(n_roof):
            step(first + args.steps + i, serial=True)
        torch.cuda.synchronize()
        roof_wall = time.perf_counter() - r0
        traffic = counted_traffic(args.workload, dominant)
        ms, cnt, work = prof_read(dom_id)
        prof_enable(0)
        avg_ms = ms / cnt
        if dominant in lib.MFMA_CLASSES:
            achieved = work / (ms * 1e-3) / 1e12
            roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                    "frac": round(achieved / (PEAK_BF16 / 1e12), 4), "traffic": traffic,
                    "traffic_unit": "bytes per launch"}
        else:
            achieved = work / (ms * 1e-3) / 1e9
            roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                    "frac": round(achieved / (PEAK_HBM / 1e9), 4), "traffic": traffic,
                    "traffic_unit": "bytes per launch"}
        roof.update({"kernel": dominant, "launches": cnt, "avg_launch_ms": round(avg_ms, 4),
                     "work_per_launch": work / cnt,
                     "timing": f"HIP events recorded by each launch of the class at the kernel's start and end, {n_roof} steps right "
                               "after the throughput region with the micro-steps in sequence",
                     "serial_ms_per_step": round(roof_wall * 1e3 / n_roof, 3)})

    tps = tokens_per_step * args.steps / wall
    fpt = flop_per_token(L, H, C, V, T)
    med15 = float(np.median(per_step[-15:]))
    out = {
        "metric": METRIC if args.workload == "gpt2_124m" else f"{args.workload} train tokens/s on 1 MI355X",
        "value": round(tps, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: L={L} H={H} C={C} V={V} (padded {Vp}), {B} seq x {T} tok x "
                               f"{n_micro} accumulation micro-steps, clip 1.0 + AdamW at step {t_adam}",
                   "global_batch": tokens_per_step, "seq_len": T, "micro_batch": B, "accum": n_micro,
                   "parallelism": "single-gpu", "lanes": nl},
        "mfu": round(tps * fpt / PEAK_BF16, 4),
        "flop_per_token": fpt,
        "median_last15_ms": round(med15, 3),
        "loss": round(last_loss, 4),
        "roofline": roof,
        "kernels_ms_per_step": {k: v["ms_per_step"] for k, v in breakdown.items()},
        "context": "pages' figure 43,374 tok/s (one card of unnamed hardware, whole loop incl. data and eval); "
                   "context only",
    }
    if not args.no_cpu_baseline:
        say("timing the CPU oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(L, H, C, V, Vp, Tmax, T_sample=T, tokens_per_step=tokens_per_step)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
