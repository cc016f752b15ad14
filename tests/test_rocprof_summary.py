"""Host logic of the rocprofv3 CSV summarizer (synthetic CSV files, no GPU)."""
import csv
import json

import rocprof_summary as RS

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(path, rows):
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(FIELDS, r)))


def test_counters_sum_rows_of_a_dispatch_then_average(tmp_path, capsys):
    k = "void (anonymous namespace)::gemm_tile_kernel<4, false>(GemmArgs)"
    _write(tmp_path / "a" / "run_counter_collection.csv", [
        (1, k, "SQ_INSTS_MFMA", 10), (1, k, "SQ_INSTS_MFMA", 30),   # two rows of dispatch 1
        (2, k, "SQ_INSTS_MFMA", 20),
        (3, "quant_act_kernel<1>(Args)", "SQ_INSTS_MFMA", 0),
    ])
    RS.main(["counters", str(tmp_path / "a"), "--kernel", "gemm_tile_kernel", "--cmd", "c", "--title", "t"])
    out = capsys.readouterr().out
    line = [l for l in out.splitlines() if l.startswith("SQ_INSTS_MFMA")][0]
    assert float(line.split()[1]) == 30.0 and "(2 dispatches)" in line


def test_traffic_scales_by_the_copy_calibration(tmp_path, capsys):
    k = "gemm_tile_kernel<4, false>(GemmArgs)"
    cp = "__amd_rocclr_copyBuffer"
    _write(tmp_path / "f" / "run_counter_collection.csv", [
        (1, cp, "FETCH_SIZE", 512.0), (2, cp, "FETCH_SIZE", 4.0), (3, k, "FETCH_SIZE", 100.0)])
    _write(tmp_path / "w" / "run_counter_collection.csv", [
        (1, cp, "WRITE_SIZE", 1024.0), (3, k, "WRITE_SIZE", 10.0)])
    RS.main(["traffic", "--fetch", str(tmp_path / "f"), "--write", str(tmp_path / "w"), "--kernel", "gemm_tile",
             "--copy-bytes", str(1024 * 1024), "--cmd-fetch", "a", "--cmd-write", "b"])
    d = json.loads(capsys.readouterr().out)
    # the copy read 1 MiB but FETCH_SIZE saw 512 KiB: factor 2; WRITE_SIZE saw all of it
    assert d["fetch_scale"] == 2.0 and d["write_scale"] == 1.0
    assert d["hbm_bytes_per_launch"] == 100 * 1024 * 2 + 10 * 1024


def test_gaps_split_at_spin_kernels_and_pair_neighbours(tmp_path, capsys):
    d = tmp_path / "t"
    d.mkdir()
    cols = ["Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    rows = [("warmup_kernel(A)", 0, 10),
            ("at::cuda::spin_kernel(long)", 20, 1000)]
    t = 1000
    for i in range(10):                       # phase "raw": back to back
        rows.append(("void (anonymous namespace)::quant_act_kernel<1>(A)", t, t + 3000)); t += 3000
        rows.append(("void (anonymous namespace)::gemm_tile_kernel<4, false>(G)", t, t + 9000)); t += 9000
    rows.append(("at::cuda::spin_kernel(long)", t, t + 500)); t += 500
    for i in range(10):                       # phase "graph": 8 us before each step
        t += 8000
        rows.append(("void (anonymous namespace)::quant_act_kernel<1>(A)", t, t + 3000)); t += 3000
        rows.append(("void (anonymous namespace)::gemm_tile_kernel<4, false>(G)", t, t + 9000)); t += 9000
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        w.writerows(rows)
    RS.main(["gaps", str(d), "--cmd", "c", "--labels", "raw,graph"])
    out = capsys.readouterr().out
    raw, graph = out.split("## graph")
    assert "## raw: 20 dispatches" in raw and "warmup" not in out
    assert "gap gemm_tile_kernel<4, false> -> quant_act_kernel<1>: n=9 p50 0.00" in raw
    assert "gap gemm_tile_kernel<4, false> -> quant_act_kernel<1>: n=9 p50 8.00 p90 8.00" in graph
    assert "gap quant_act_kernel<1> -> gemm_tile_kernel<4, false>: n=10 p50 0.00" in graph
    assert "duration p50     9.00" in graph
