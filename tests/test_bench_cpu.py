"""bench.py's host-side logic: the one-GPU guard and the conversion of
rocprofv3 counter runs into per-launch HBM bytes (no GPU needed)."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
          "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
          "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def write_run(root, name, counter, rows):
    d = root / name
    d.mkdir()
    with open(d / f"{name}_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (kernel, value) in enumerate(rows):
            row = {k: 0 for k in FIELDS}
            row.update(Dispatch_Id=i + 1, Kernel_Name=kernel, Counter_Name=counter, Counter_Value=value)
            w.writerow(row)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_write_traffic_scales_counters_by_the_copy_probe(tmp_path, monkeypatch):
    # Copy probe: 1 GiB read reports 2^19 KiB of FETCH_SIZE (factor 2), 1 GiB
    # written reports 2^20 KiB of WRITE_SIZE (factor 1).
    copy = "__amd_rocclr_copyBuffer"
    write_run(tmp_path, "copy_fetch", "FETCH_SIZE", [("fill", 7.0), (copy, 524288.0)])
    write_run(tmp_path, "copy_write", "WRITE_SIZE", [(copy, 1048576.0)])
    gu, dn = "void moe::k_gate_up<16, 4>(x)", "void moe::k_down<16>(y)"
    tg, td = "void moe::k_expert_tiled<0>(z)", "void moe::k_expert_tiled<1>(z)"
    write_run(tmp_path, "dec_fetch", "FETCH_SIZE", [(gu, 100.0), (gu, 300.0), (dn, 50.0), ("other", 1e9)])
    write_run(tmp_path, "dec_write", "WRITE_SIZE", [(gu, 10.0), (gu, 30.0), (dn, 5.0)])
    write_run(tmp_path, "pre_fetch", "FETCH_SIZE", [(tg, 1000.0), (td, 400.0)])
    write_run(tmp_path, "pre_write", "WRITE_SIZE", [(tg, 100.0), (td, 40.0)])
    out = tmp_path / "profiles"
    out.mkdir()
    monkeypatch.setattr(bench, "PROFILES", str(out))
    bench.write_traffic(str(tmp_path))
    rec = json.load(open(out / "traffic_gate_up_decode.json"))
    assert rec["dispatches"] == 2
    assert rec["fetch_factor"] == pytest.approx(2.0) and rec["write_factor"] == pytest.approx(1.0)
    # mean FETCH 200 KiB x 2 + mean WRITE 20 KiB x 1
    assert rec["hbm_bytes_per_launch"] == pytest.approx((200 * 2 + 20) * 1024)
    assert rec["source_hash"] == bench.kernel_source_hash()
    rec = json.load(open(out / "traffic_down_prefill.json"))
    assert rec["hbm_bytes_per_launch"] == pytest.approx((400 * 2 + 40) * 1024)
    # The figures are used only while the kernel sources are unchanged.
    assert bench.load_traffic("decode", "gate_up") == pytest.approx(420 * 1024)
    rec = json.load(open(out / "traffic_gate_up_decode.json"))
    rec["source_hash"] = "0" * 16
    json.dump(rec, open(out / "traffic_gate_up_decode.json", "w"))
    assert bench.load_traffic("decode", "gate_up") is None


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    csrc = tmp_path / "sparse_moe_transformer_ffn_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in bench.EXPERT_SOURCES:
        (csrc / name).write_text("int a = 1;  // one\n\n// note\nint b = 2;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    (csrc / bench.EXPERT_SOURCES[0]).write_text("int a = 1;  // changed prose\n// more\nint b = 2;\n")
    assert bench.kernel_source_hash() == h0
    (csrc / bench.EXPERT_SOURCES[0]).write_text("int a = 3;\nint b = 2;\n")
    assert bench.kernel_source_hash() != h0
