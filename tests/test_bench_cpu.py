"""Host-side helpers of bench.py: the counter summaries that feed
`roofline.traffic` and the per-configuration counter means, run on small
synthetic rocprofv3-style CSV files, and the single-GPU guard."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

GEMM_A = "void convrot::(anonymous namespace)::gemm_dma_kernel<(convrot::GemmMode)1, 4, 2, 2, 2, 3, 256, false>(x)"
GEMM_B = "void convrot::(anonymous namespace)::gemm_dma_kernel<(convrot::GemmMode)1, 2, 2, 1, 1, 4, 256, false>(x)"
PRO = "void convrot::(anonymous namespace)::prologue_persistent_kernel<0, false>(y)"
COPY = "void at::native::elementwise_kernel<128, 4>(z)"


def _write(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (k, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v})


def test_summarize_pmc_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    kib = 1024.0
    # the copy reads and writes COPY_BYTES; FETCH_SIZE shows half of its reads
    fetch = [(COPY, bench.COPY_BYTES / kib / 2), (GEMM_A, 100.0), (GEMM_B, 300.0), (PRO, 10.0)]
    write = [(COPY, bench.COPY_BYTES / kib), (GEMM_A, 50.0), (GEMM_B, 70.0), (PRO, 4.0)]
    _write(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _write(tmp_path / "w.csv", "WRITE_SIZE", write)
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(out))
    bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    rec = json.loads(out.read_text())
    assert rec["launches"] == 2
    assert rec["copy_calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert rec["copy_calibration"]["write_factor"] == pytest.approx(1.0)
    # per launch: (100 + 300) / 2 KiB read x 2 + (50 + 70) / 2 KiB written x 1
    assert rec["hbm_bytes_per_launch"] == round((200.0 * 2 + 60.0) * 1024)
    assert rec["prologue"]["hbm_bytes_per_launch"] == round((10.0 * 2 + 4.0) * 1024)
    assert rec["source_sha256_16"] == bench.source_hash(bench.GEMM_SRC)


def test_summarize_pmc_splits_the_hbm_scale_prologue(tmp_path, monkeypatch):
    # --profile-kernels order: the sweep (prologue + GEMM), the calibration
    # copy (bitwise not), then one prologue call at HBM scale
    kib = 1024.0
    copy = "void at::native::vectorized_elementwise_kernel<4, at::native::bitwise_not_kernel_cuda(x)>(z)"
    fetch = [(PRO, 10.0), (GEMM_A, 100.0), (PRO, 12.0), (GEMM_A, 300.0), (copy, bench.COPY_BYTES / kib / 2),
             (PRO, 5000.0)]
    write = [(PRO, 4.0), (GEMM_A, 50.0), (PRO, 6.0), (GEMM_A, 70.0), (copy, bench.COPY_BYTES / kib), (PRO, 900.0)]
    _write(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _write(tmp_path / "w.csv", "WRITE_SIZE", write)
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(out))
    bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    rec = json.loads(out.read_text())
    assert rec["launches"] == 2
    assert rec["prologue"]["launches"] == 2
    assert rec["prologue"]["hbm_bytes_per_launch"] == round((11.0 * 2 + 5.0) * 1024)
    h = rec["prologue_hbm_scale"]
    M, K = bench.HBM_SCALE_MK
    assert h["launches"] == 1 and (h["M"], h["K"]) == (M, K)
    assert h["hbm_bytes_per_launch"] == round((5000.0 * 2 + 900.0) * 1024)
    assert h["algorithmic_bytes_per_launch"] == 3 * M * K + 4 * M


BAND = "void convrot::(anonymous namespace)::band_kernel<32>(convrot::GemmArgs, __half const*, long, long)"


def test_summarize_pmc_reports_the_one_launch_layer(tmp_path, monkeypatch):
    # the K = 256 layers run as one launch after the staged sweep; their
    # traffic is its own record, not part of the GEMM's average
    kib = 1024.0
    copy = "void at::native::vectorized_elementwise_kernel<4, at::native::bitwise_not_kernel_cuda(x)>(z)"
    fetch = [(PRO, 10.0), (GEMM_A, 100.0), (BAND, 3000.0), (BAND, 3100.0), (copy, bench.COPY_BYTES / kib / 2)]
    write = [(PRO, 4.0), (GEMM_A, 50.0), (BAND, 12000.0), (BAND, 12000.0), (copy, bench.COPY_BYTES / kib)]
    _write(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _write(tmp_path / "w.csv", "WRITE_SIZE", write)
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(out))
    bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    rec = json.loads(out.read_text())
    assert rec["launches"] == 1 and rec["hbm_bytes_per_launch"] == round((100.0 * 2 + 50.0) * 1024)
    b = rec["band"]
    assert b["launches"] == 2 and b["K"] == 256
    assert b["hbm_bytes_per_launch"] == round((3050.0 * 2 + 12000.0) * 1024)
    M, N = b["M"], b["N"]
    assert b["algorithmic_bytes_per_launch"] == 2 * M * 256 + N * 256 + 4 * N + 2 * M * N


def test_counter_means_reports_the_one_launch_layer(tmp_path, capsys):
    _write(tmp_path / "a.csv", "SQ_INSTS_VALU", [(GEMM_A, 10.0), (BAND, 500.0), (BAND, 700.0)])
    bench.counter_means([str(tmp_path / "a.csv")])
    out = json.loads(capsys.readouterr().out)
    assert out["band"]["SQ_INSTS_VALU"] == 600.0 and out["band"]["dispatches"] == 2


def test_summarize_pmc_rejects_mismatched_runs(tmp_path, monkeypatch):
    _write(tmp_path / "f.csv", "FETCH_SIZE", [(COPY, 1.0), (GEMM_A, 1.0), (GEMM_A, 2.0)])
    _write(tmp_path / "w.csv", "WRITE_SIZE", [(COPY, 1.0), (GEMM_A, 1.0)])
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(tmp_path / "t.json"))
    with pytest.raises(SystemExit):
        bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    assert not (tmp_path / "t.json").exists()


def test_counter_means_per_configuration(tmp_path, capsys):
    _write(tmp_path / "a.csv", "SQ_INSTS_MFMA", [(GEMM_A, 10.0), (GEMM_A, 30.0), (GEMM_B, 4.0), (PRO, 0.0),
                                                 (COPY, 99.0)])
    _write(tmp_path / "b.csv", "SQ_WAVES", [(GEMM_A, 8.0), (GEMM_A, 8.0), (GEMM_B, 4.0), (PRO, 16.0)])
    bench.counter_means([str(tmp_path / "a.csv"), str(tmp_path / "b.csv")])
    out = json.loads(capsys.readouterr().out)
    a = out["gemm<(convrot::GemmMode)1, 4, 2, 2, 2, 3, 256, false>"]
    b = out["gemm<(convrot::GemmMode)1, 2, 2, 1, 1, 4, 256, false>"]
    assert a["SQ_INSTS_MFMA"] == 20.0 and a["SQ_WAVES"] == 8.0 and a["dispatches"] == 2
    assert b["SQ_INSTS_MFMA"] == 4.0 and b["dispatches"] == 1
    assert out["prologue"]["SQ_WAVES"] == 16.0
    # the three GEMM dispatches are the first layers of the sweep (2048 x 2048)
    shape = out["gemm 2048x2048"]
    assert shape["dispatches"] == 3 and shape["SQ_INSTS_MFMA"] == round(44.0 / 3, 1)
    assert len(out) == 4      # the copy kernel is not reported


def test_gemm_dispatches_map_to_the_sweep_layers():
    # the i-th GEMM dispatch of a profiling run is layer i mod 448 of the
    # sweep's order: 168 x (2048, 2048), 84 x (256, 2048), 84 x (6144, 256), ...
    import workload as wl
    layers = sum(n for (_, _, n) in wl.LAYER_SHAPES)
    ids = [10 + 3 * i for i in range(2 * layers)]          # two steps, ids with gaps
    keys = bench._gemm_shape_keys(reversed(ids))
    assert keys[ids[0]] == "2048x2048" and keys[ids[167]] == "2048x2048"
    assert keys[ids[168]] == "256x2048" and keys[ids[251]] == "256x2048"
    assert keys[ids[252]] == "6144x256" and keys[ids[layers - 1]] == "2048x8192"
    assert keys[ids[layers]] == "2048x2048"                # second step starts over
    counts = {}
    for k in keys.values():
        counts[k] = counts.get(k, 0) + 1
    assert counts == {f"{n}x{k}": 2 * c for (n, k, c) in wl.LAYER_SHAPES}


def test_counter_means_keeps_the_hbm_scale_prologue_apart(tmp_path, capsys):
    copy = "void at::native::vectorized_elementwise_kernel<4, at::native::bitwise_not_kernel_cuda(x)>(z)"
    _write(tmp_path / "a.csv", "SQ_WAVES", [(PRO, 16.0), (GEMM_A, 8.0), (PRO, 16.0), (copy, 1.0), (PRO, 512.0)])
    bench.counter_means([str(tmp_path / "a.csv")])
    out = json.loads(capsys.readouterr().out)
    assert out["prologue"]["SQ_WAVES"] == 16.0 and out["prologue"]["dispatches"] == 2
    assert out["prologue_hbm_scale"]["SQ_WAVES"] == 512.0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "single-GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_host_cpu_description():
    h = bench.host_cpu()
    assert h["logical_cpus"] >= 1 and h["cpus_usable_by_this_process"] >= 1
    if h["physical_cores"]:
        assert 1 <= h["physical_cores"] <= h["logical_cpus"]
        assert h["smt_per_core"] >= 1


def test_summarize_trace_finds_the_gemm_only_replays(tmp_path, monkeypatch):
    # two replays of 448 GEMM launches (1 us kernels, 2 us apart), one other
    # run of 3 GEMMs interleaved with another kernel that must be ignored
    rows, did, t = [], 0, 0
    def add(name, dur, gap):
        nonlocal did, t
        rows.append({"Dispatch_Id": did, "Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur})
        did += 1
        t += gap
    for _ in range(2):
        for _ in range(448):
            add(GEMM_A, 1000, 2000)
        add(COPY, 500, 1000)
    for _ in range(3):
        add(GEMM_A, 5000, 6000)
        add(PRO, 500, 1000)
    path = tmp_path / "trace.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(rows)
    out = tmp_path / "trace.json"
    monkeypatch.setattr(bench, "TRACE_JSON", str(out))
    bench.summarize_trace(str(path))
    rec = json.loads(out.read_text())
    assert rec["replays"] == 2 and rec["mean_kernel_us"] == 1.0
    # replays launched back to back form one run of 2 x 448: split, not dropped
    rows2 = [dict(r) for r in rows if r["Kernel_Name"] == GEMM_A][:896]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(rows2)
    bench.summarize_trace(str(path))
    assert json.loads(out.read_text())["replays"] == 2
    # span: 447 gaps of 2 us plus the last 1 us kernel, over 448 launches
    assert abs(rec["mean_span_per_launch_us"] - (447 * 2.0 + 1.0) / 448) < 1e-3
