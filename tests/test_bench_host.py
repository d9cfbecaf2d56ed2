"""Host-side logic of bench.py that runs without a GPU: the refusal of
several GPUs and the kernel-trace table of the profile summaries."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def _trace(tmp_path, rows):
    d = tmp_path / "prof" / "host"
    d.mkdir(parents=True)
    keys = ["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Workgroup_Size_X",
            "Workgroup_Size_Y", "Workgroup_Size_Z", "Start_Timestamp", "End_Timestamp"]
    with open(d / "run_kernel_trace.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=keys)
        w.writeheader()
        for name, grid, wg, t0, t1 in rows:
            w.writerow({"Kernel_Name": name, "Grid_Size_X": grid[0], "Grid_Size_Y": grid[1],
                        "Grid_Size_Z": grid[2], "Workgroup_Size_X": wg, "Workgroup_Size_Y": 1,
                        "Workgroup_Size_Z": 1, "Start_Timestamp": t0, "End_Timestamp": t1})
    return str(tmp_path / "prof")


def test_trace_table_groups_by_kernel_and_grid(tmp_path, capsys):
    gu = "void qmoe::ffn_decode_kernel<0, 2, true>(qmoe::FfnParams)"
    dn = "void qmoe::ffn_decode_kernel<1, 4, true>(qmoe::FfnParams)"
    rows = [(gu, (256 * 100, 1, 1), 256, 0, 300_000),       # 100 blocks, 300 us
            (gu, (256 * 100, 1, 1), 256, 0, 310_000),       # same launch size, 310 us
            (gu, (256 * 8, 1, 1), 256, 0, 12_000),          # another launch size
            (dn, (256 * 4, 2, 1), 256, 1_000, 6_000),       # 4 x 2 blocks
            ("void qmoe::route_decode_kernel<4>(qmoe::RouteDecodeParams)", (1024 * 14, 16, 1),
             1024, 0, 21_000),
            ("__amd_rocclr_copyBuffer", (64, 1, 1), 64, 0, 1_000)]   # not a library kernel
    bench.summarize_trace(_trace(tmp_path, rows))
    out = capsys.readouterr().out.splitlines()
    body = [line for line in out if line.startswith("| ") and "---" not in line][1:]
    table = {(c[1].strip(), int(c[2])): c for c in (line.split("|") for line in body)}
    assert set(table) == {("ffn_gate_up ffn_decode_kernel<0, 2, true>", 100),
                          ("ffn_gate_up ffn_decode_kernel<0, 2, true>", 8),
                          ("ffn_down ffn_decode_kernel<1, 4, true>", 8),
                          ("route_decode_kernel<4>", 224)}
    big = table[("ffn_gate_up ffn_decode_kernel<0, 2, true>", 100)]
    assert int(big[3]) == 2
    assert float(big[4]) == pytest.approx(305.0)
    assert (float(big[5]), float(big[6])) == (300.0, 310.0)
    assert float(table[("ffn_down ffn_decode_kernel<1, 4, true>", 8)][4]) == pytest.approx(5.0)
    # the largest total time comes first
    assert body[0].split("|")[1].strip().startswith("ffn_gate_up") and int(body[0].split("|")[2]) == 100
    assert "ffn_gate_up: 3 launches, average 207.333 us" in out
    assert "ffn_down: 1 launches, average 5.000 us" in out


def test_prefill_counter_summary(tmp_path, capsys):
    """Counters averaged per dispatch per prefill kernel; FETCH_SIZE scaled by
    the 256 MiB calibration copy; MFMA busy fraction from the two counters."""
    d = tmp_path / "pmc"
    d.mkdir()
    pk = "void qmoe::prefill_kernel<1, 1, 8, false>(qmoe::PrefillParams, int)"
    cp = "__amd_rocclr_copyBuffer"
    rows = [(cp, 1, "FETCH_SIZE", 131072.0),                  # 256 MiB read -> 128 Ki
            (pk, 2, "FETCH_SIZE", 1000.0), (pk, 3, "FETCH_SIZE", 3000.0),
            (pk, 2, "SQ_VALU_MFMA_BUSY_CYCLES", 1024.0 * 0.5), (pk, 2, "GRBM_GUI_ACTIVE", 1.0),
            (pk, 3, "SQ_VALU_MFMA_BUSY_CYCLES", 1024.0 * 0.5), (pk, 3, "GRBM_GUI_ACTIVE", 1.0)]
    with open(d / "x_counter_collection.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                           "Counter_Value"])
        w.writeheader()
        for name, disp, c, v in rows:
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": c,
                        "Counter_Value": v})
    bench.summarize_prefill_pmc([str(d)])
    out = capsys.readouterr().out
    line = [l for l in out.splitlines() if l.startswith("| prefill_kernel")][0]
    assert "| 2 |" in line and "2000" in line
    # 2000 KiB per launch x 2 (the copy read 256 MiB as 128 Ki units) = 4096000 B
    assert "FETCH_SIZE 4.1 MB per launch" in out
    assert "MFMA busy 0.5000" in out
