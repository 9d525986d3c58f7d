"""Text summaries of rocprofv3 output for the training step's kernels.

    python -m transformer_lm_pretraining_amd.profile_summary stats KERNEL_STATS.csv
    python -m transformer_lm_pretraining_amd.profile_summary counters --a A.csv --b B.csv \
        --fetch FETCH.csv --write WRITE.csv --copy-fetch CF.csv --copy-write CW.csv
    python -m transformer_lm_pretraining_amd.profile_summary block KERNEL_TRACE.csv --layers 12
    python -m transformer_lm_pretraining_amd.profile_summary grid KERNEL_TRACE.csv
    python -m transformer_lm_pretraining_amd.profile_summary timeline KERNEL_TRACE.csv --first 2 --last 3
    python -m transformer_lm_pretraining_amd.profile_summary ntclass [KERNEL_TRACE.csv] [--fetch F.csv --write W.csv
        --copy-fetch CF.csv --copy-write CW.csv] [model sizes]
    python -m transformer_lm_pretraining_amd.profile_summary hbm KERNEL_TRACE.csv [--fetch F.csv --write W.csv
        --copy-fetch CF.csv --copy-write CW.csv] [model sizes]

stats: per-kernel calls, average and total duration from a --kernel-trace --stats run.
counters: per kernel (and grid size) from --pmc runs: MFMA-busy fraction of the SIMD
  cycles (SQ_VALU_MFMA_BUSY_CYCLES over 1,024 SIMDs x GRBM_GUI_ACTIVE per XCD; the GRBM
  counters are summed over the 8 XCDs), instructions per wave, and HBM bytes per
  dispatch (FETCH_SIZE and WRITE_SIZE in KiB, each scaled by what the counter reads for
  a plain copy of known size).
block: time of one transformer block's kernels per micro-step, taken from the dispatch
  sequence of a step trace (the block kernels between the embedding and the final
  LayerNorm in the forward, and between the final LayerNorm's backward and the grouped
  weight-gradient launch in the backward), plus 1/L of the weight-gradient launches.
grid: calls, average and total duration per kernel and grid size, from the kernel trace.
ntclass: the dominant kernel class (NT GEMMs with a bf16 output: gemm_nt_w8_kernel<0> and <5>) per
  micro-step: its launches by grid size, time, the FLOP of its 6L + 2 products (sum of 2MNK from the model
  sizes) and the fraction of the 2.5 PF bf16 peak; with counter files (--fetch, --write, --copy-fetch,
  --copy-write; the trace may be omitted) its HBM bytes per launch against the algorithmic bytes.
timeline: for a range of optimizer steps of a step trace (a step ends at its AdamW launch): the step
  time, the share of it during which the GPU ran at least one kernel and at least two at once, and per
  kernel the calls, average duration, summed duration and active time (the union of its launches'
  intervals; launches of different lanes may overlap).
hbm: the memory-bound kernels' average duration, algorithmic bytes (from the model sizes), achieved TB/s
  against 8 TB/s, and with counter files the HBM bytes they moved (FETCH_SIZE and WRITE_SIZE scaled by a
  plain copy's readings).
Model sizes: --layers L --c C --bt B*T --t T --vp padded vocabulary (defaults: GPT-2 124M at 19 x 1024).
"""
from __future__ import annotations

import argparse
import collections
import csv
import re
import sys

N_SIMD = 1024   # 256 CUs x 4 SIMDs
N_XCD = 8


def short(name: str) -> str:
    n = re.sub(r"\(anonymous namespace\)::", "", name)
    n = re.sub(r"^void ", "", n)
    if "at::native" in n:
        return "torch:" + n.split("<")[0].split("::")[-1]
    return n.split("(")[0].strip()


def cmd_stats(path: str, top: int) -> None:
    rows = list(csv.DictReader(open(path)))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    print("%-52s %7s %10s %10s %6s" % ("kernel", "calls", "avg_us", "total_ms", "pct"))
    for r in rows[:top]:
        print("%-52s %7d %10.2f %10.2f %6.1f" % (short(r["Name"])[:52], int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                                              float(r["TotalDurationNs"]) / 1e6,
                                              100.0 * float(r["TotalDurationNs"]) / total))


def per_dispatch(path: str):
    """{(kernel, grid): {counter: mean over dispatches of the per-dispatch sum}}"""
    acc = collections.defaultdict(lambda: collections.defaultdict(float))
    seen = set()
    for r in csv.DictReader(open(path)):
        key = (short(r["Kernel_Name"]), int(r["Grid_Size"]))
        acc[key][r["Counter_Name"]] += float(r["Counter_Value"])
        seen.add((key, r["Dispatch_Id"]))
    count = collections.Counter(k for k, _ in seen)
    return {k: {c: v / count[k] for c, v in d.items()} | {"_n": count[k]} for k, d in acc.items()}


def copy_kib(path: str, counter: str) -> float:
    vals = [v[counter] for k, v in per_dispatch(path).items() if "copy" in k[0].lower()]
    return sum(vals) / len(vals)


def cmd_counters(a, b, fetch, write, cfetch, cwrite, top: int) -> None:
    A, B = per_dispatch(a), per_dispatch(b) if b else {}
    F, W = per_dispatch(fetch), per_dispatch(write)
    fs = (1 << 20) / copy_kib(cfetch, "FETCH_SIZE")   # a 1 GiB copy reads 1,048,576 KiB
    ws = (1 << 20) / copy_kib(cwrite, "WRITE_SIZE")
    print("copy calibration: FETCH_SIZE x %.5f, WRITE_SIZE x %.5f" % (fs, ws))
    keys = sorted(A, key=lambda k: -A[k]["GRBM_GUI_ACTIVE"] * A[k]["_n"])[:top]
    print("%-44s %8s %5s %6s %8s %8s %7s %6s %6s %6s" % ("kernel", "grid", "n", "mfma", "read_MB", "write_MB", "valu/w",
                                                         "mfma/w", "lds/w", "tr/w"))
    for k in keys:
        a_, b_ = A[k], B.get(k, {})
        cyc = a_["GRBM_GUI_ACTIVE"] / N_XCD
        mfma = a_.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (cyc * N_SIMD) if cyc else 0.0
        rd = F.get(k, {}).get("FETCH_SIZE", float("nan")) * 1024 * fs / 1e6
        wr = W.get(k, {}).get("WRITE_SIZE", float("nan")) * 1024 * ws / 1e6
        waves = b_.get("SQ_WAVES", float("nan"))
        per = lambda c: b_.get(c, float("nan")) / waves
        print("%-44s %8d %5d %6.3f %8.1f %8.1f %7.0f %6.0f %6.0f %6.0f" % (
            k[0][:44], k[1], a_["_n"], mfma, rd, wr, per("SQ_INSTS_VALU"), per("SQ_INSTS_MFMA"), per("SQ_INSTS_LDS"),
            per("SQ_INSTS_VALU_TRANS_F32")))


FWD_BLOCK = ["ln_fwd", "gemm_nt", "attn_fwd", "gemm_nt", "ln_fwd", "gemm_nt", "gemm_nt"]


def cmd_block(path: str, layers: int, first=None, last=None) -> None:
    """Per-block time of a one-lane step trace (or of optimizer steps first..last of it)."""
    rows = rows_in_steps(path, first, last)
    seq = [(short(r["Kernel_Name"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3) for r in rows]
    # micro-steps: each forward starts with the embedding kernel
    starts = [i for i, (n, _) in enumerate(seq) if n.startswith("embedding_fwd")]
    whole = starts[1:-1] if first is None else starts  # a step range holds whole micro-steps
    blocks, dw = [], []
    for s in whole:  # without a range the first one is skipped (warm caches)
        fwd = seq[s + 1: s + 1 + 7 * layers]
        assert all(n.startswith(p) for (n, _), p in zip(fwd, FWD_BLOCK * layers)), [n for n, _ in fwd[:7]]
        i = s + 1 + 7 * layers
        while not seq[i][0].startswith("ln_bwd"):  # ln_f forward, lm_head, loss, lm_head backward
            i += 1
        i += 1  # past ln_f's backward
        j = i
        while not seq[j][0].startswith("gemm_tn"):
            j += 1
        bwd = seq[i:j]
        k = j
        while seq[k][0].startswith(("gemm_tn", "splitk")):
            k += 1
        # the grouped weight-gradient launch and its tail cover every block; the lm_head's
        # weight gradient ran before the blocks' backward
        blocks.append((sum(t for _, t in fwd) + sum(t for _, t in bwd)) / layers)
        dw.append(sum(t for _, t in seq[j:k]) / layers)
    n = len(blocks)
    print("micro-steps %d; per block: forward+input-gradient kernels %.1f us, share of the weight-gradient "
          "launches %.1f us, total %.1f us" % (n, sum(blocks) / n, sum(dw) / n, (sum(blocks) + sum(dw)) / n))


def trace_rows(path: str):
    return sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))


def rows_in_steps(path: str, first=None, last=None):
    """The trace's dispatches, or those of optimizer steps first..last (0-based, inclusive)."""
    rows = trace_rows(path)
    if first is None:
        return rows
    win = step_windows(rows)
    t0, t1 = win[first][0], win[last][1]
    return [r for r in rows if int(r["Start_Timestamp"]) >= t0 and int(r["End_Timestamp"]) <= t1]


def by_grid(path: str, first=None, last=None):
    """{(kernel, grid): [durations in us]} over the trace (or steps first..last of it)"""
    d = collections.defaultdict(list)
    for r in rows_in_steps(path, first, last):
        d[(short(r["Kernel_Name"]), int(r["Grid_Size_X"]))].append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return d


def cmd_grid(path: str, top: int) -> None:
    d = by_grid(path)
    print("%-44s %10s %6s %10s %10s" % ("kernel", "grid", "calls", "avg_us", "total_ms"))
    for k in sorted(d, key=lambda k: -sum(d[k]))[:top]:
        v = d[k]
        print("%-44s %10d %6d %10.2f %10.2f" % (k[0][:44], k[1], len(v), sum(v) / len(v), sum(v) / 1e3))


def step_windows(rows):
    """[(start_ns, end_ns)] of the optimizer steps in a trace: a step ends with its AdamW launch
    and starts where the previous one ended (the first at the first dispatch)."""
    ends = [int(r["End_Timestamp"]) for r in rows if short(r["Kernel_Name"]).startswith("adamw_kernel")]
    starts = [int(rows[0]["Start_Timestamp"])] + ends[:-1]
    return list(zip(starts, ends))


def cmd_timeline(path: str, first: int, last: int, top: int) -> None:
    """Steps first..last (0-based, in dispatch order) of a step trace: wall time, the time the
    GPU ran at least one kernel and at least two at once, and per kernel the calls, average
    duration and the time at least one of its launches ran (the union of their intervals)."""
    rows = trace_rows(path)
    win = step_windows(rows)
    t0, t1 = win[first][0], win[last][1]
    sel = [r for r in rows if int(r["Start_Timestamp"]) >= t0 and int(r["End_Timestamp"]) <= t1]
    ev = []
    for r in sel:
        ev.append((int(r["Start_Timestamp"]), 1))
        ev.append((int(r["End_Timestamp"]), -1))
    ev.sort()
    busy = two = 0
    level, prev = 0, t0
    for t, d in ev:
        if level >= 1:
            busy += t - prev
        if level >= 2:
            two += t - prev
        level += d
        prev = t

    def union(iv):
        iv.sort()
        tot, lo, hi = 0, None, None
        for a, b in iv:
            if hi is None or a > hi:
                if hi is not None:
                    tot += hi - lo
                lo, hi = a, b
            else:
                hi = max(hi, b)
        return tot + (hi - lo if hi is not None else 0)

    per = collections.defaultdict(list)
    for r in sel:
        per[short(r["Kernel_Name"])].append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    n = last - first + 1
    wall = t1 - t0
    print("steps %d..%d (%d): %.3f ms per step; GPU running >= 1 kernel %.1f%% of the time, >= 2 kernels %.1f%%"
          % (first, last, n, wall / n / 1e6, 100.0 * busy / wall, 100.0 * two / wall))
    print("%-44s %7s %10s %14s %14s" % ("kernel", "calls", "avg_us", "sum_ms/step", "active_ms/step"))
    for k in sorted(per, key=lambda k: -sum(b - a for a, b in per[k]))[:top]:
        iv = per[k]
        tot = sum(b - a for a, b in iv)
        print("%-44s %7d %10.2f %14.2f %14.2f" % (k[:44], len(iv), tot / len(iv) / 1e3, tot / n / 1e6,
                                                  union(list(iv)) / n / 1e6))


NT_CLASS = ("gemm_nt_w8_kernel<0,", "gemm_nt_w8_kernel<5,")
PEAK_BF16 = 2.5e15


def nt_products(L: int, C: int, BT: int, Vp: int):
    """(name, M, N, K) of the class's products in one micro-step"""
    per_layer = [("QKV", BT, 3 * C, C), ("attention projection + residual", BT, C, C),
                 ("FC-proj + residual", BT, C, 4 * C), ("FC input gradient", BT, C, 4 * C),
                 ("attention-projection input gradient", BT, C, C), ("QKV input gradient", BT, C, 3 * C)]
    return per_layer * L + [("lm_head forward", BT, Vp, C), ("lm_head input gradient", BT, C, Vp)]


def nt_traffic(fetch, write, cfetch, cwrite, L, C, BT, Vp) -> None:
    """HBM bytes per launch of the class from counter runs, against its algorithmic bytes"""
    F, W = per_dispatch(fetch), per_dispatch(write)
    fs = (1 << 20) / copy_kib(cfetch, "FETCH_SIZE")
    ws = (1 << 20) / copy_kib(cwrite, "WRITE_SIZE")
    cls = [k for k in F if k[0].startswith(NT_CLASS)]
    n = sum(F[k]["_n"] for k in cls)
    fk = sum(F[k]["FETCH_SIZE"] * F[k]["_n"] for k in cls) / n
    wk = sum(W[k]["WRITE_SIZE"] * W[k]["_n"] for k in cls) / n
    rd, wr = fk * 1024 * fs / 1e6, wk * 1024 * ws / 1e6
    res = ("attention projection + residual", "FC-proj + residual")
    prods = nt_products(L, C, BT, Vp)
    # A + B + output (+ residual input), bf16
    alg = sum(2 * (m * k + n_ * k + m * n_) + (2 * m * n_ if nm in res else 0) for nm, m, n_, k in prods) / len(prods) / 1e6
    print("copy calibration: FETCH_SIZE x %.5f, WRITE_SIZE x %.5f" % (fs, ws))
    print("counter traffic over %d dispatches: FETCH_SIZE avg %.2f KiB -> %.1f MB read, WRITE_SIZE avg %.2f KiB -> "
          "%.1f MB written per launch" % (n, fk, rd, wk, wr))
    print("traffic %.1f MB per launch; algorithmic %.1f MB per launch (A + B + output [+ residual], bf16, averaged "
          "over the %d products); ratio %.2f" % (rd + wr, alg, len(prods), (rd + wr) / alg))
    print("by grid (MB read / written per launch):")
    for k in sorted(cls, key=lambda k: k[1]):
        print("  %-44s %10d %9.1f / %8.1f" % (k[0][:44], k[1], F[k]["FETCH_SIZE"] * 1024 * fs / 1e6,
                                             W[k]["WRITE_SIZE"] * 1024 * ws / 1e6))


def cmd_ntclass(path: str, L: int, C: int, BT: int, Vp: int, first=None, last=None) -> None:
    d = by_grid(path, first, last)
    if first is not None:
        print("optimizer steps %d..%d of the trace" % (first, last))
    micro = sum(len(v) for k, v in d.items() if k[0].startswith("xent_kernel"))
    cls = {k: v for k, v in d.items() if k[0].startswith(NT_CLASS)}
    prods = nt_products(L, C, BT, Vp)
    flop = sum(2.0 * m * n * k for _, m, n, k in prods)
    print("micro-steps in the trace: %d; class launches per micro-step: %d" % (micro, len(prods)))
    print("%-44s %10s %6s %10s %12s" % ("kernel", "grid", "calls", "avg_us", "per_micro_us"))
    tot = 0.0
    for k in sorted(cls, key=lambda k: -sum(cls[k])):
        v = cls[k]
        tot += sum(v)
        print("%-44s %10d %6d %10.2f %12.1f" % (k[0][:44], k[1], len(v), sum(v) / len(v), sum(v) / micro))
    t_micro = tot / micro
    print("time per micro-step %.1f us over %d launches = %.2f us per launch" % (t_micro, len(prods), t_micro / len(prods)))
    print("work per micro-step %.1f GFLOP (%.2f GFLOP per launch) -> %.1f TFLOP/s = %.3f of 2.5 PF" % (
        flop / 1e9, flop / len(prods) / 1e9, flop / (t_micro * 1e-6) / 1e12, flop / (t_micro * 1e-6) / PEAK_BF16))


def mem_kernels(L: int, C: int, BT: int, T: int, Vp: int, G: int = 1):
    """(kernel prefix, label, algorithmic bytes per launch); G gradient accumulators (one per lane)
    are read by the norm and read and zeroed by the update"""
    n_decay = Vp * C + T * C + L * 12 * C * C
    n_params = n_decay + L * 13 * C + 2 * C
    return [("xent_kernel", "CE: logits read, dz written in place", 4 * BT * Vp),
            ("ln_fwd16_kernel", "LayerNorm fwd: R x, W y, W mean/rstd", 4 * BT * C + 8 * BT),
            ("ln_bwd_kernel", "LayerNorm bwd: R x, dy, dres, mean/rstd, W dx", 8 * BT * C + 8 * BT),
            ("adamw_kernel", "AdamW: R p,g,m,v; W p,m,v; zero g; W shadow", (24 + 8 * G) * n_params + 2 * n_decay),
            ("sumsq_kernel", "global norm: R grads", 4 * G * n_params),
            ("transpose_batch_kernel", "transposed bf16 weight copies, R + W", 4 * (Vp * C + 12 * L * C * C)),
            ("embedding_fwd_kernel", "embedding fwd: R wte rows, wpe rows, W x0", 4 * BT * C + 2 * T * C)]


def cmd_hbm(path, fetch, write, cfetch, cwrite, L, C, BT, T, Vp, first=None, last=None, G=1) -> None:
    d = by_grid(path, first, last)
    F = per_dispatch(fetch) if fetch else {}
    W = per_dispatch(write) if write else {}
    fs = (1 << 20) / copy_kib(cfetch, "FETCH_SIZE") if cfetch else None
    ws = (1 << 20) / copy_kib(cwrite, "WRITE_SIZE") if cwrite else None
    if fs and ws:
        print("copy calibration: FETCH_SIZE x %.5f, WRITE_SIZE x %.5f" % (fs, ws))
    print("%-18s %-46s %9s %9s %6s %6s %10s" % ("kernel", "algorithmic bytes", "MB", "avg_us", "TB/s", "of 8", "counter MB"))
    for pre, label, nbytes in mem_kernels(L, C, BT, T, Vp, G):
        ks = [k for k in d if k[0].startswith(pre)]
        if not ks:
            continue
        v = [x for k in ks for x in d[k]]
        us = sum(v) / len(v)
        cnt = ""
        fk = [k for k in F if k[0].startswith(pre)]
        wk = [k for k in W if k[0].startswith(pre)]
        if fs and ws and fk and wk:
            cnt = "%.1f" % ((F[fk[0]]["FETCH_SIZE"] * fs + W[wk[0]]["WRITE_SIZE"] * ws) * 1024 / 1e6)
        print("%-18s %-46s %9.1f %9.2f %6.2f %6.3f %10s" % (pre.replace("_kernel", ""), label[:46], nbytes / 1e6, us,
                                                          nbytes / (us * 1e-6) / 1e12, nbytes / (us * 1e-6) / 8e12, cnt))


def model_args(p) -> None:
    p.add_argument("--layers", type=int, default=12)
    p.add_argument("--c", type=int, default=768)
    p.add_argument("--bt", type=int, default=19456)
    p.add_argument("--t", type=int, default=1024)
    p.add_argument("--vp", type=int, default=50304)
    p.add_argument("--grads", type=int, default=1, help="gradient accumulators (lanes) the update reads")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("path")
    s.add_argument("--top", type=int, default=30)
    c = sub.add_parser("counters")
    for k in ("a", "b", "fetch", "write", "copy_fetch", "copy_write"):
        c.add_argument("--" + k.replace("_", "-"), required=k != "b")
    c.add_argument("--top", type=int, default=30)
    bl = sub.add_parser("block")
    bl.add_argument("path")
    bl.add_argument("--layers", type=int, default=12)
    bl.add_argument("--first", type=int, help="first optimizer step of the trace to count (0-based)")
    bl.add_argument("--last", type=int, help="last optimizer step to count (inclusive)")
    tl = sub.add_parser("timeline")
    tl.add_argument("trace")
    tl.add_argument("--first", type=int, required=True, help="first optimizer step (0-based)")
    tl.add_argument("--last", type=int, required=True, help="last optimizer step (0-based, inclusive)")
    tl.add_argument("--top", type=int, default=30)
    g = sub.add_parser("grid")
    g.add_argument("path")
    g.add_argument("--top", type=int, default=40)
    n = sub.add_parser("ntclass")
    n.add_argument("path", nargs="?")
    n.add_argument("--first", type=int, help="first optimizer step of the trace to count (0-based)")
    n.add_argument("--last", type=int, help="last optimizer step to count (inclusive)")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        n.add_argument("--" + k.replace("_", "-"))
    model_args(n)
    h = sub.add_parser("hbm")
    h.add_argument("path")
    h.add_argument("--first", type=int, help="first optimizer step of the trace to count (0-based)")
    h.add_argument("--last", type=int, help="last optimizer step to count (inclusive)")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        h.add_argument("--" + k.replace("_", "-"))
    model_args(h)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        cmd_stats(a.path, a.top)
    elif a.cmd == "counters":
        cmd_counters(a.a, a.b, a.fetch, a.write, a.copy_fetch, a.copy_write, a.top)
    elif a.cmd == "block":
        cmd_block(a.path, a.layers, a.first, a.last)
    elif a.cmd == "grid":
        cmd_grid(a.path, a.top)
    elif a.cmd == "timeline":
        cmd_timeline(a.trace, a.first, a.last, a.top)
    elif a.cmd == "ntclass":
        if a.path:
            cmd_ntclass(a.path, a.layers, a.c, a.bt, a.vp, a.first, a.last)
        if a.fetch:
            nt_traffic(a.fetch, a.write, a.copy_fetch, a.copy_write, a.layers, a.c, a.bt, a.vp)
    else:
        cmd_hbm(a.path, a.fetch, a.write, a.copy_fetch, a.copy_write, a.layers, a.c, a.bt, a.t, a.vp, a.first,
                a.last, a.grads)


if __name__ == "__main__":
    sys.exit(main())
