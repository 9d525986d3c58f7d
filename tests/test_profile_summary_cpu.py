"""Host-side checks of the rocprofv3 summary tool on a synthetic kernel trace whose
answers are known by construction: step windows end at the AdamW launches, the
timeline's busy and overlap shares, per-kernel active time as the union of launch
intervals, and step-range selection of the dominant-class figures."""
import csv

from transformer_lm_pretraining_amd import profile_summary as ps

FIELDS = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X"]


def write_trace(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for name, a, b, grid in rows:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": a, "End_Timestamp": b, "Grid_Size_X": grid})


GEMM = "void (anonymous namespace)::gemm_nt_w8_kernel<0, 2, 64>((anonymous namespace)::GemmParams)"
LN = "void (anonymous namespace)::ln_fwd16_kernel<3>(x)"
ADAM = "void (anonymous namespace)::adamw_kernel<1>(x)"
XENT = "void (anonymous namespace)::xent_kernel<13>(x)"


MS = 1_000_000  # trace timestamps are in ns; the synthetic times below are in ms


def trace_rows():
    # step 0 (serial): gemm 0-100, ln 100-110, xent 110-150, adamw 150-160
    # step 1 (two lanes): gemm 200-300 and gemm 250-330 overlap, ln 330-340, xent 340-400, adamw 400-420
    ms = [(GEMM, 0, 100, 116736), (LN, 100, 110, 196608), (XENT, 110, 150, 9961472), (ADAM, 150, 160, 1024),
          (GEMM, 200, 300, 116736), (GEMM, 250, 330, 116736), (LN, 330, 340, 196608),
          (XENT, 340, 400, 9961472), (ADAM, 400, 420, 1024)]
    return [(n, a * MS, b * MS, g) for n, a, b, g in ms]


def test_step_windows_and_range_selection(tmp_path):
    p = tmp_path / "trace.csv"
    write_trace(p, trace_rows())
    rows = ps.trace_rows(str(p))
    assert ps.step_windows(rows) == [(0, 160 * MS), (160 * MS, 420 * MS)]
    names = [ps.short(r["Kernel_Name"]) for r in ps.rows_in_steps(str(p), 1, 1)]
    assert names.count("gemm_nt_w8_kernel<0, 2, 64>") == 2 and len(names) == 5
    d = ps.by_grid(str(p), 0, 0)
    assert d[("gemm_nt_w8_kernel<0, 2, 64>", 116736)] == [100_000.0]  # us


def test_timeline_busy_overlap_and_active_time(tmp_path, capsys):
    p = tmp_path / "trace.csv"
    write_trace(p, trace_rows())
    ps.cmd_timeline(str(p), 1, 1, 10)
    out = capsys.readouterr().out
    # step 1 spans 160..420 ms (260); kernels run 200..420 (220 busy), two at once 250..300 (50)
    assert "steps 1..1 (1): 260.000 ms per step; GPU running >= 1 kernel 84.6% of the time, >= 2 kernels 19.2%" in out
    gemm = [l for l in out.splitlines() if l.startswith("gemm_nt_w8_kernel")][0].split()
    # two launches of 100 and 80 ms: average 90,000 us, summed 180 ms, active (union 200..330) 130 ms
    assert gemm[-4:] == ["2", "90000.00", "180.00", "130.00"]
    ps.cmd_timeline(str(p), 0, 0, 10)
    assert ">= 2 kernels 0.0%" in capsys.readouterr().out


def test_hbm_table_step_range_and_accumulators(tmp_path, capsys):
    # step 1 of the synthetic trace: one LayerNorm forward of 10 ms (10,000 us)
    p = tmp_path / "trace.csv"
    write_trace(p, trace_rows())
    ps.cmd_hbm(str(p), None, None, None, None, 12, 768, 19456, 1024, 50304, first=1, last=1)
    ln = [l for l in capsys.readouterr().out.splitlines() if l.startswith("ln_fwd16")][0].split()
    assert ln[-3:] == ["10000.00", "0.01", "0.001"]  # 59.9 MB in 10 ms
    # algorithmic bytes of the update and the norm grow by 8 and 4 B per parameter with each accumulator
    one = {k: b for k, _, b in ps.mem_kernels(12, 768, 19456, 1024, 50304, 1)}
    two = {k: b for k, _, b in ps.mem_kernels(12, 768, 19456, 1024, 50304, 2)}
    n_params = 124_475_904
    assert two["adamw_kernel"] - one["adamw_kernel"] == 8 * n_params
    assert two["sumsq_kernel"] == 2 * one["sumsq_kernel"] == 8 * n_params
