"""bench.py host logic on the CPU: the one-GPU contract and the traffic summary built from counter CSVs."""
import csv
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def _write_counters(directory, counter, rows):
    os.makedirs(directory, exist_ok=True)
    with open(os.path.join(directory, "t_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_summary_scales_by_the_copy(tmp_path):
    row = "a3_fp8_gate_up_m2048"
    nbytes, _ = bench.kernel_work(row)
    launches = 1
    copy_kib = bench.TRAFFIC_COPY_BYTES / 1024
    neg = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel>"
    # an earlier copy-like kernel from set-up, then the two markers around 2 passes of the row; the fetch
    # counter reads half of the copy's bytes, the write counter all of them
    fetch = [(neg, 7.0)] + [(neg, copy_kib / 2)] + [("qr::gemv_kernel", 100.0)] * (2 * launches) + [(neg, copy_kib / 2)]
    write = [(neg, 7.0)] + [(neg, copy_kib)] + [("qr::gemv_kernel", 10.0)] * (2 * launches) + [(neg, copy_kib)]
    _write_counters(str(tmp_path / "f"), "FETCH_SIZE", fetch)
    _write_counters(str(tmp_path / "w"), "WRITE_SIZE", write)
    md = bench.traffic_summary(str(tmp_path / "f"), str(tmp_path / "w"), row, 2, "cmd")
    fields = dict(line.split(": ", 1) for line in md.splitlines() if line.startswith("traffic_"))
    assert fields["traffic_row"] == row
    assert int(fields["traffic_bytes_per_launch"]) == (100 * 2 + 10) * 1024
    assert fields["traffic_sources_sha256"] == bench.sources_digest(row)
    assert "| algorithmic (what the method must move) | %d |" % nbytes in md
    assert nbytes == 37888 * 3584 + 4 * 37888 + 2048 * 3584 + 4 * 2048 + 2 * 2048 * 37888
    # a call that runs two kernels (a split-K reduction after the linear): both count toward that call
    fetch2 = fetch[:-1] + [("qr::splitk_reduce_kernel", 50.0)] * (2 * launches) + fetch[-1:]
    write2 = write[:-1] + [("qr::splitk_reduce_kernel", 4.0)] * (2 * launches) + write[-1:]
    _write_counters(str(tmp_path / "f2"), "FETCH_SIZE", fetch2)
    _write_counters(str(tmp_path / "w2"), "WRITE_SIZE", write2)
    md2 = bench.traffic_summary(str(tmp_path / "f2"), str(tmp_path / "w2"), row, 2, "cmd")
    fields2 = dict(line.split(": ", 1) for line in md2.splitlines() if line.startswith("traffic_"))
    assert int(fields2["traffic_bytes_per_launch"]) == (100 * 2 + 50 * 2 + 10 + 4) * 1024


def test_traffic_is_only_reported_for_the_current_sources(tmp_path, monkeypatch):
    """The figure is valid while the sources of the row's kernels (and the shared headers and ABI) are
    unchanged; a change elsewhere in the library leaves it valid."""
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    csrc = tmp_path / "quantized_rollout_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in bench.SHARED_SOURCES + sum(bench.ROW_SOURCES.values(), []) + ["qr_moe.hip"]:
        (csrc / name).write_text("v1 " + name)
    digest = bench.sources_digest("a3_fp8_gate_up_m2048")
    (tmp_path / "profiles" / "traffic_x.md").write_text(
        "traffic_row: a3_fp8_gate_up_m2048\ntraffic_bytes_per_launch: 123\ntraffic_sources_sha256: %s\n" % digest)
    assert bench.read_traffic("a3_fp8_gate_up_m2048") == 123
    assert bench.read_traffic("a3_fp8_gate_up_m512") is None
    (csrc / "qr_moe.hip").write_text("v2")  # not a source of the row's kernels
    assert bench.read_traffic("a3_fp8_gate_up_m2048") == 123
    (csrc / "qr_linear.hip").write_text("v2")
    assert bench.read_traffic("a3_fp8_gate_up_m2048") is None
    (csrc / "qr_linear.hip").write_text("v1 qr_linear.hip")
    assert bench.read_traffic("a3_fp8_gate_up_m2048") == 123
    (csrc / "qr_device.hpp").write_text("v2")
    assert bench.read_traffic("a3_fp8_gate_up_m2048") is None


def test_step_work_and_roofline_bounds():
    """The step's operations (2 M N K over every linear, layer and batch) and the binding roofline per batch."""
    nb, no = bench.Dense7B.step_work()
    lins = [(4608, 3584), (3584, 3584), (37888, 3584), (3584, 18944)]
    ms = (1, 16, 128, 512, 2048)
    assert no == bench.LAYERS * sum(2 * m * n * k for m in ms for n, k in lins)
    assert nb == bench.LAYERS * sum(n * k + 4 * n + 2 * m * k + 2 * m * n for m in ms for n, k in lins)
    assert [bench.bound_of(m) for m in ms] == ["hbm", "hbm", "hbm", "mfma", "mfma"]
    assert abs(bench.frac_of(2048, 0, 5e12, 1.0) - 1.0) < 1e-12        # 5 TFLOP in 1 ms = 5 PFLOP/s
    assert abs(bench.frac_of(16, 8e9, 0, 1.0) - 1.0) < 1e-12           # 8 GB in 1 ms = 8 TB/s
