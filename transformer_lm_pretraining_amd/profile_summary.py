"""Text summaries of rocprofv3 output for the training step's kernels.

    python -m transformer_lm_pretraining_amd.profile_summary stats KERNEL_STATS.csv
    python -m transformer_lm_pretraining_amd.profile_summary counters --a A.csv --b B.csv \
        --fetch FETCH.csv --write WRITE.csv --copy-fetch CF.csv --copy-write CW.csv
    python -m transformer_lm_pretraining_amd.profile_summary block KERNEL_TRACE.csv --layers 12

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


def cmd_block(path: str, layers: int) -> None:
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))
    seq = [(short(r["Kernel_Name"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3) for r in rows]
    # micro-steps: each forward starts with the embedding kernel
    starts = [i for i, (n, _) in enumerate(seq) if n.startswith("embedding_fwd")]
    blocks, dw = [], []
    for s in starts[1:-1]:  # whole micro-steps only, the first one skipped (warm caches)
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
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        cmd_stats(a.path, a.top)
    elif a.cmd == "counters":
        cmd_counters(a.a, a.b, a.fetch, a.write, a.copy_fetch, a.copy_write, a.top)
    else:
        cmd_block(a.path, a.layers)


if __name__ == "__main__":
    sys.exit(main())
