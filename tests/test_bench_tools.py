"""Host logic of bench.py's rocprofv3 counter summary (no GPU): grouping by
kernel and grid, per-dispatch means, and the derived ratios."""

import csv

import bench

NAME = ("void fp8blk::(anonymous namespace)::gemm_kernel<fp8blk::(anonymous namespace)::Tile<256, 256, 2, 4, 2, "
        "false, 0> >(unsigned char const*, float const*, unsigned char const*, float const*, long, long, long, "
        "unsigned short*, long, long)")


def _write(path, rows):
    cols = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
            "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(cols, r)))


def test_short_kernel_name_keeps_template_arguments():
    assert bench.short_kernel_name(NAME) == "gemm_kernel<Tile<256, 256, 2, 4, 2, false, 0> >"
    assert bench.short_kernel_name("void splitk_reduce_kernel(float const*)") == "splitk_reduce_kernel"


def test_derived_ratios(tmp_path):
    cycles, ns = 1000.0, 1000.0  # 1 GHz
    rows = []
    for d in (1, 2):
        for c, v in (("GRBM_GUI_ACTIVE", 8 * cycles),                       # counted once per XCD
                     ("SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * cycles * 256 * 4),  # half of every SIMD's cycles
                     ("SQ_INSTS_VALU_MFMA_MOPS_F8", 1e6 * d),               # 512 FLOPs per MOP
                     ("TCC_HIT_sum", 3.0), ("TCC_MISS_sum", 1.0)):
            rows.append((d, 256 * 64, NAME, c, v, 0, ns))
    p = tmp_path / "c.csv"
    _write(p, rows)
    out = bench.summarize_counters([str(p)])
    line = [ln for ln in out.splitlines() if "gemm_kernel" in ln][0]
    cells = [c.strip() for c in line.strip("|").split("|")]
    assert cells[1] == "256" and cells[2] == "2" and cells[3] == "1.0"   # workgroups, dispatches, us
    assert "clock 1.00 GHz" in cells[4]
    assert "MFMA busy 50.0%" in cells[4]
    assert "FP8 MFMA 0.768 GFLOP = 768 TFLOP/s" in cells[4]              # mean of 1e6 and 2e6 MOPs
    assert "L2 hit 75.0%" in cells[4]


def test_groups_by_grid_and_sorts_by_time(tmp_path):
    rows = [(1, 64 * 10, NAME, "SQ_WAVES", 1.0, 0, 100.0),
            (2, 64 * 20, NAME, "SQ_WAVES", 2.0, 0, 5000.0),
            (3, 64 * 20, NAME, "SQ_WAVES", 4.0, 0, 7000.0)]
    p = tmp_path / "c.csv"
    _write(p, rows)
    lines = [ln for ln in bench.summarize_counters([str(p)]).splitlines() if "gemm_kernel" in ln]
    assert len(lines) == 2
    first = [c.strip() for c in lines[0].strip("|").split("|")]
    assert first[1] == "20" and first[2] == "2" and first[3] == "6.0" and "SQ_WAVES 3" in first[5]


def test_step_trace_groups_gemm_launches_by_layer(tmp_path):
    # one warm-up and two timed steps of the two MoE layers; the second layer's
    # launch is split over two GEMM-family dispatches, and a fused producer
    # (whose name also holds "quant_act_kernel") and a side-section GEMM follow
    qw = "fp8blk::(anonymous namespace)::quant_weight_kernel(long)"
    qa = "fp8blk::(anonymous namespace)::quant_act_kernel(long)"
    gm = "void fp8blk::(anonymous namespace)::grouped_gemm_persistent_kernel<Tile>(long)"
    red = "fp8blk::(anonymous namespace)::splitk_reduce_kernel(long)"
    silu = "fp8blk::(anonymous namespace)::silu_mul_quant_act_kernel(long)"
    seq = []
    for step in range(3):
        seq += [(qw, 5), (qw, 5), (qa, 3), (gm, 100 + step), (qa, 3), (gm, 40), (red, 10 + step)]
    seq += [(silu, 7), (gm, 999)]
    path = tmp_path / "kt_kernel_trace.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 1000
        rows = []
        for name, us in seq:
            rows.append({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + us * 1000})
            t += us * 1000 + 500
        for r in reversed(rows):  # the summary orders by start time, not by row
            w.writerow(r)
    out = bench.summarize_step_trace(str(path), "moe", 1, 2)
    # timed steps 1 and 2: gate_up (101 + 102) / 2, down (40 + 11 + 40 + 12) / 2
    assert "moe_gate_up 101.5, moe_down 51.5 us" in out
    assert "mean per launch 76.5 us" in out


def test_more_than_one_gpu_is_refused():
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for extra, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py")] + extra, capture_output=True, text=True,
                           env=dict(os.environ, **env), timeout=120)
        assert r.returncode == 2
        assert "exactly one GPU" in r.stderr and r.stdout == ""
