"""Host-side checks of bench.py that need no GPU: the one-GPU refusal and the
kernel-source hash that keys the recorded HBM traffic."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_code_text_ignores_comments_and_blank_lines():
    a = "int x = 1;  // a note\n\n/* block\n comment */\nint y = 2;\n"
    b = "int x = 1;\n// another note\nint y = 2;   \n"
    assert bench.code_text(a) == bench.code_text(b) == "int x = 1;\nint y = 2;"
    assert bench.code_text("int x = 1;\n") != bench.code_text("int x = 2;\n")


def test_kernel_source_hash_follows_code_not_comments():
    files = {}
    for name in bench.KERNEL_SOURCES:
        path = os.path.join(ROOT, "tiled_online_softmax_05_amd", "csrc", name)
        with open(path) as f:
            files[path] = f.read()
    h0 = bench.kernel_source_hash(lambda p: files[p])
    assert h0 == bench.kernel_source_hash()
    first = next(iter(files))
    commented = dict(files)
    commented[first] = "// an added comment line\n" + files[first]
    assert bench.kernel_source_hash(lambda p: commented[p]) == h0
    changed = dict(files)
    changed[first] = files[first] + "\nstatic int added_symbol;\n"
    assert bench.kernel_source_hash(lambda p: changed[p]) != h0



def test_counter_records_are_read_back(tmp_path, monkeypatch):
    """--record-counters turns rocprofv3 counter CSVs into the two records;
    bench.py reports them while the kernel source hash matches and null
    otherwise."""
    import csv as _csv
    header = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
              "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
              "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
              "Counter_Value", "Start_Timestamp", "End_Timestamp"]

    def write(sub, kernel, counters, n):
        d = tmp_path / sub
        d.mkdir()
        with open(d / "run_counter_collection.csv", "w", newline="") as f:
            w = _csv.writer(f)
            w.writerow(header)
            for i in range(1, n + 1):
                for name, value in counters.items():
                    w.writerow([i, i, "Agent 1", 1, 1, 1, 1, 1, kernel, 256, 0, 0, 0, 0, 0,
                                name, value, 0, 1])
    kern = "x_attn_fwd_bf16_kernel_y"
    write("pmc_fetch", kern, {"FETCH_SIZE": 1000.0}, 25)
    write("pmc_write", kern, {"WRITE_SIZE": 500.0}, 25)
    write("pmc_copy_fetch", "copy_kernel", {"FETCH_SIZE": 524288.0}, 3)
    write("pmc_copy_write", "copy_kernel", {"WRITE_SIZE": 1048576.0}, 3)
    write("pmc_mfma", kern, {"SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 600.0, "GRBM_GUI_ACTIVE": 8 * 1000.0}, 25)
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    monkeypatch.setattr(bench, "MFMA_FILE", str(tmp_path / "mfma.json"))
    bench.record_counters(str(tmp_path), bench.COUNTER_COMMANDS)
    assert bench.measured_traffic("prefill_h32_s4096_d128") == 2 * 1000 * 1024 + 500 * 1024
    assert bench.measured_mfma_busy("prefill_h32_s4096_d128") == 0.6
    monkeypatch.setattr(bench, "kernel_source_hash", lambda read=None: "0000000000000000")
    assert bench.measured_traffic("prefill_h32_s4096_d128") is None
    assert bench.measured_mfma_busy("prefill_h32_s4096_d128") is None
