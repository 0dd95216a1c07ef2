"""CPU tier: bench.py's host logic (no GPU): the one-GPU guard, the
summaries that turn rocprofv3 CSVs into the committed profiles, and the
staleness check of the recorded HBM traffic."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write_csv(path, fields, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_more_than_one_gpu_exits():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_summarize_trace_splits_runs(tmp_path, capsys):
    """Runs of one (kernel, grid) end when more than 12 other dispatches pass."""
    rows, i = [], 0

    def add(name, grid, us, n):
        nonlocal i
        for _ in range(n):
            i += 1
            rows.append({"Dispatch_Id": i, "Kernel_Name": f"void bd::(anonymous namespace)::{name}(int)",
                         "Grid_Size_X": grid, "Grid_Size_Y": 1, "Workgroup_Size_X": 256,
                         "Start_Timestamp": 1000 * i, "End_Timestamp": 1000 * i + int(us * 1000)})

    add("kern_a", 1024, 5.0, 3)
    add("kern_b", 2048, 7.0, 13)
    add("kern_a", 1024, 9.0, 2)
    path = tmp_path / "trace.csv"
    _write_csv(path, list(rows[0]), rows)
    bench.summarize_trace(str(path))
    lines = [ln.split() for ln in capsys.readouterr().out.splitlines()[1:]]
    got = [(ln[0], int(ln[1]), int(ln[4]), float(ln[5])) for ln in lines]
    assert got == [("bd::kern_a", 1024, 3, 5.0), ("bd::kern_b", 2048, 13, 7.0), ("bd::kern_a", 1024, 2, 9.0)]


def test_summarize_kernels_totals_per_call(tmp_path, capsys):
    """Per-kernel totals over the kernels matching a pattern, divided by the
    number of anchor dispatches (one per entry-point call); template
    arguments stay in the name, other kernels are ignored."""
    rows, i = [], 0

    def add(name, us, n):
        nonlocal i
        for _ in range(n):
            i += 1
            rows.append({"Dispatch_Id": i, "Kernel_Name": f"void bd::(anonymous namespace)::{name}(int, float*)",
                         "Grid_Size_X": 256, "Grid_Size_Y": 1, "Workgroup_Size_X": 256,
                         "Start_Timestamp": 1000 * i, "End_Timestamp": 1000 * i + int(us * 1000)})

    for _ in range(2):
        add("ms_pass<true>", 10.0, 2)
        add("ms_solve", 30.0, 1)
        add("gemv_stream<1>", 99.0, 1)
    path = tmp_path / "trace.csv"
    _write_csv(path, list(rows[0]), rows)
    bench.summarize_kernels(str(path), "ms_", "ms_solve")
    out = capsys.readouterr().out.splitlines()
    assert out[0].startswith("2 calls")
    body = {ln.split()[0]: ln.split() for ln in out[2:]}
    assert set(body) == {"ms_solve", "ms_pass<true>", "total"}
    assert int(body["ms_pass<true>"][1]) == 4 and float(body["ms_pass<true>"][5]) == 20.0
    assert float(body["ms_solve"][5]) == 30.0 and float(body["total"][1]) == 50.0


def test_summarize_counters_scales_and_picks_the_step_grid(tmp_path):
    """A copy of 256 MiB that FETCH_SIZE reads as half its bytes gives the
    factor 2; each entry's bytes are the median of its dispatches on the
    grid seen most often (a stray grid of the same kernel is ignored)."""
    copy_mb = 256
    fetch_rows, write_rows = [], []

    def add(name, grid, fetch_b, write_b, n=3):
        for _ in range(n):
            base = {"Kernel_Name": f"void bd::(anonymous namespace)::{name}(int)", "Grid_Size": grid}
            fetch_rows.append({**base, "Counter_Name": "FETCH_SIZE", "Counter_Value": fetch_b / 2 / 1024})
            write_rows.append({**base, "Counter_Name": "WRITE_SIZE", "Counter_Value": write_b / 1024})

    add("__amd_rocclr_copyBuffer", 4096, 4 * (copy_mb << 20), 4 * (copy_mb << 20), n=1)  # not the probe
    algo = bench.DecodeStep.algorithmic_bytes()
    names = {"compress_row": ["compress_rows<true, false>"],
             "compress_matrix": ["compress_rows<true, true>", "alpha_matrix_finish"],
             "reconstruct": ["reconstruct_rows<false>"],
             "linear_m1_row": ["gemv_stream<1, 1, 8, false, true, false>"],
             "linear_m1_matrix": ["gemv_stream<1, 1, 8, true, true, false>"],
             "linear_m4_row": ["gemv_stream<4, 1, 4, false, true, true>"],
             "linear_m4_matrix": ["gemv_stream<4, 1, 4, true, true, true>"],
             "linear_m16_row": ["gemv_rows<8, 8, 1, 1, false, false>"],
             "linear_m16_matrix": ["gemv_rows<8, 8, 1, 1, false, true>"]}
    assert set(names) == set(bench.STEP_KERNELS)
    for entry, kernels in names.items():
        for k in kernels:
            add(k, 1048576, algo[entry] // len(kernels), 4096)
    add("compress_rows<true, false>", 64, 10 ** 9, 10 ** 9, n=2)   # another call of the kernel
    add("__amd_rocclr_copyBuffer", 4096, copy_mb << 20, copy_mb << 20, n=1)  # the probe, issued last
    fields = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    _write_csv(tmp_path / "f.csv", fields, fetch_rows)
    _write_csv(tmp_path / "w.csv", fields, write_rows)
    bench.summarize_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), copy_mb, "cmd", out_dir=str(tmp_path))
    rec = json.load(open(tmp_path / "traffic.json"))
    assert rec["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert rec["calibration"]["write_factor"] == pytest.approx(1.0)
    assert rec["kernels"]["compress_row"]["fetch_bytes"] == algo["compress_row"]
    e = rec["kernels"]["reconstruct"]
    assert e["fetch_bytes"] == algo["reconstruct"] and e["write_bytes"] == 4096
    assert e["ratio"] == pytest.approx((algo["reconstruct"] + 4096) / algo["reconstruct"], abs=1e-4)
    cm = rec["kernels"]["compress_matrix"]
    assert cm["fetch_bytes"] == 2 * (algo["compress_matrix"] // 2) and cm["write_bytes"] == 2 * 4096
    assert cm["source_sha"] == bench.source_sha("compress.hip")


def test_summarize_mfma_busy_and_clock(tmp_path, capsys):
    """busy = MFMA busy cycles over (GRBM_GUI_ACTIVE / 8) x 1024 SIMDs; clock =
    (GRBM_GUI_ACTIVE / 8) over the dispatch's duration; rate = MFMA
    instructions x 32768 flop (bf16 32x32x16) over the duration."""
    us, ghz, busy = 100.0, 1.8, 0.5
    xcd_cycles = ghz * 1e3 * us
    n_mfma = 2880000
    vals = {"GRBM_GUI_ACTIVE": 8 * xcd_cycles, "SQ_VALU_MFMA_BUSY_CYCLES": busy * xcd_cycles * 1024,
            "SQ_INSTS_MFMA": n_mfma, "SQ_INSTS_VALU": 4 * n_mfma, "SQ_INSTS_LDS": 1.5 * n_mfma,
            "SQ_LDS_BANK_CONFLICT": 0,
            "SQ_BUSY_CYCLES": 1, "SQ_WAVE_CYCLES": 1, "SQ_ACTIVE_INST_VALU": 1}
    assert set(vals) == set(bench.MFMA_COUNTERS)
    rows = []
    for d in (1, 2):
        for n, v in vals.items():
            rows.append({"Dispatch_Id": d, "Kernel_Name": "void bd::(anonymous namespace)::gemm_tiles_w8<false, false, false, 256>(int)",
                         "Grid_Size": 131072, "Counter_Name": n, "Counter_Value": v,
                         "Start_Timestamp": 10 ** 6 * d, "End_Timestamp": 10 ** 6 * d + int(us * 1000)})
    _write_csv(tmp_path / "c.csv", list(rows[0]), rows)
    bench.summarize_mfma(str(tmp_path / "c.csv"))
    line = capsys.readouterr().out.splitlines()[1].split()
    # kernel name has spaces: count from the end
    n, avg_us, mf, b, clk, tf, valu, lds, cf = line[-9:]
    assert int(n) == 2 and float(avg_us) == pytest.approx(us)
    assert float(b) == pytest.approx(100 * busy) and float(clk) == pytest.approx(ghz)
    assert float(mf) == n_mfma and float(tf) == pytest.approx(n_mfma * 32768 / us / 1e6, abs=1)
    assert float(valu) == pytest.approx(4.0) and float(lds) == pytest.approx(1.5)


def test_traffic_is_dropped_when_the_kernel_source_changed(monkeypatch):
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    entry = "compress_row"
    assert entry in rec["kernels"]
    monkeypatch.setattr(bench, "source_sha", lambda src: rec["kernels"][entry]["source_sha"])
    assert bench.traffic_for(entry) == rec["kernels"][entry]["bytes_per_launch"]
    monkeypatch.setattr(bench, "source_sha", lambda src: "0" * 16)
    assert bench.traffic_for(entry) is None


def test_summarize_gemm_counters(tmp_path):
    """A prefill shape's fused call (GEMM + split reduce) and unfused call
    (reconstruct + vendor GEMM), and the grouped GEMM, from synthetic counter
    CSVs: medians per kernel, scaled by the copy calibration, summed per call,
    recorded under "gemm" without touching the decode entries."""
    import bench

    copy_mb = 256
    fetch_rows, write_rows = [], []

    def add(name, fetch_b, write_b, n=3):
        for _ in range(n):
            base = {"Kernel_Name": f"void bd::(anonymous namespace)::{name}(int)", "Grid_Size": 64}
            fetch_rows.append({**base, "Counter_Name": "FETCH_SIZE", "Counter_Value": fetch_b / 2 / 1024})
            write_rows.append({**base, "Counter_Name": "WRITE_SIZE", "Counter_Value": write_b / 1024})

    add("__amd_rocclr_copyBuffer", 3 * (copy_mb << 20), 3 * (copy_mb << 20), n=1)  # a weight copy, not the probe
    add("gemm_tiles_w8<false, false, true, 128>", 1000 * 1024, 8 * 1024 ** 2)
    add("splitk_reduce<128>", 8 * 1024 ** 2, 4 * 1024 ** 2)
    add("reconstruct_rows<false>", 17 * 1024 ** 2, 16 * 1024 ** 2)
    add("__amd_rocclr_copyBuffer", copy_mb << 20, copy_mb << 20, n=1)
    fields = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    _write_csv(tmp_path / "f.csv", fields, fetch_rows)
    _write_csv(tmp_path / "w.csv", fields, write_rows)
    (tmp_path / "traffic.json").write_text(json.dumps({"kernels": {"linear_m1_row": {"bytes_per_launch": 7}}}))
    bench.summarize_gemm_counters("prefill_k/v", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), copy_mb, "cmd",
                                  out_dir=str(tmp_path))
    rec = json.load(open(tmp_path / "traffic.json"))
    assert rec["kernels"]["linear_m1_row"]["bytes_per_launch"] == 7
    e = rec["gemm"]["prefill_k/v"]
    assert e["fused"]["fetch_bytes"] == 1000 * 1024 + 8 * 1024 ** 2
    assert e["fused"]["write_bytes"] == 12 * 1024 ** 2
    assert e["unfused"]["fetch_bytes"] == 17 * 1024 ** 2 and e["unfused"]["write_bytes"] == 16 * 1024 ** 2
    assert e["bytes_per_launch"] == e["fused"]["bytes_per_launch"] == 1000 * 1024 + 20 * 1024 ** 2
    assert e["algorithmic"]["weights_fused"] == 1024 * 8192 * 2 + 1024 * 1024 + 4 * 1024
    assert e["source_sha"] == bench.source_sha("gemm.hip")


def test_summarize_stack_assigns_linears_by_order(tmp_path, capsys):
    """The m = 1 launches of the stack's decode pass are the linears in the
    stack's order (q, k, v, o, gate, up, down per layer): dispatch i is
    linear i mod 7, and the pass rate is the algorithmic bytes over the
    summed kernel time; a launch count that is not whole passes is refused."""
    from tenant_fine_tune_amd.stack import LAYER_SHAPES

    rows, i = [], 0

    def add(name, us):
        nonlocal i
        i += 1
        rows.append({"Dispatch_Id": i, "Kernel_Name": f"void bd::(anonymous namespace)::{name}(int)",
                     "Grid_Size_X": 4096, "Grid_Size_Y": 1, "Workgroup_Size_X": 256,
                     "Start_Timestamp": 10 ** 6 * i, "End_Timestamp": 10 ** 6 * i + int(us * 1000)})

    n_layers, passes = 2, 3
    for _ in range(passes):
        for _ in range(n_layers):
            for j, _ in enumerate(LAYER_SHAPES):
                add("gemv_stream<1, 1, 8, false, true, false>", 10.0 * (j + 1))
        add("gemm_tiles_w8<false, false, false, 256>", 100.0)
    path = tmp_path / "trace.csv"
    _write_csv(path, list(rows[0]), rows)
    bench.summarize_stack(str(path), n_layers)
    out = capsys.readouterr().out.splitlines()
    assert out[0] == f"decode m = 1: {passes} passes x {n_layers * len(LAYER_SHAPES)} linears"
    per = {ln.split()[0]: ln.split() for ln in out[2:2 + len(LAYER_SHAPES)]}
    tot_b = 0
    for j, (name, d_out, d_in) in enumerate(LAYER_SHAPES):
        b = d_out * d_in * 2 + d_out * d_in // 8 + 4 * d_out + 2 * d_in + 2 * d_out
        tot_b += b
        assert int(per[name][-5]) == passes * n_layers and float(per[name][-4]) == 10.0 * (j + 1)
        assert int(per[name][-2]) == b
    pass_us = n_layers * sum(10.0 * (j + 1) for j in range(len(LAYER_SHAPES)))
    assert f"{tot_b * n_layers / pass_us / 1e3:.1f} GB/s" in out[2 + len(LAYER_SHAPES)]
    with pytest.raises(SystemExit):
        bench.summarize_stack(str(path), n_layers + 2)


def test_summarize_wave_states(tmp_path, capsys):
    """Wave-state counters over SQ_WAVE_CYCLES, MFMA busy over the SIMD cycles
    (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs), LDS FIFO-full over busy cycles."""
    name = "void bd::(anonymous namespace)::gemm_tiles_w8<false, false, false, 256>(int)"
    fields = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    a = [{"Kernel_Name": name, "Grid_Size": 131072, "Counter_Name": c, "Counter_Value": v}
         for c, v in (("SQ_WAVE_CYCLES", 1000), ("SQ_WAIT_ANY", 250), ("SQ_WAIT_INST_ANY", 400),
                      ("SQ_WAIT_INST_LDS", 70), ("SQ_ACTIVE_INST_ANY", 330), ("SQ_ACTIVE_INST_VALU", 190),
                      ("SQ_ACTIVE_INST_LDS", 75), ("SQ_ACTIVE_INST_VMEM", 40))]
    b = [{"Kernel_Name": name, "Grid_Size": 131072, "Counter_Name": c, "Counter_Value": v}
         for c, v in (("SQ_BUSY_CYCLES", 200), ("SQ_VALU_MFMA_BUSY_CYCLES", 6144),
                      ("SQ_LDS_DATA_FIFO_FULL", 40), ("SQ_LDS_CMD_FIFO_FULL", 30), ("GRBM_GUI_ACTIVE", 80))]
    _write_csv(tmp_path / "a.csv", fields, a)
    _write_csv(tmp_path / "b.csv", fields, b)
    bench.summarize_wave_states(str(tmp_path / "a.csv"), str(tmp_path / "b.csv"))
    row = capsys.readouterr().out.splitlines()[1].split()
    assert row[-9:] == ["0.250", "0.400", "0.070", "0.330", "0.190", "0.075", "0.040", "0.600", "0.350"]
