"""Host logic of bench.py, no GPU needed: the one-GPU guard, the rocprofv3
summary arithmetic (per-kernel durations, counter calibration by the probe
and the dequantisation of known size, the dominant kernel's traffic), and
the rule that stored traffic is reported only for the kernel sources it was
measured on.  The csv files are written here in rocprofv3's column layout."""
import csv
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DOM = "void qmv::" + bench.DOMINANT + "(qmv::RowsParams)"
PROBE = "qmv::(anonymous namespace)::probe_read(unsigned char const*, unsigned long, unsigned int*)"
DEQ = "void qmv::(anonymous namespace)::dequant_q4_k(unsigned char const*, long, float*)"


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_summarize_trace_durations(tmp_path):
    # dominant kernel: 10 us and 11 us; the probe: 600 us
    rows = [(DOM, 1000, 11000), (DOM, 20000, 31000), (PROBE, 0, 600000)]
    write_csv(str(tmp_path / "t" / "run_kernel_trace.csv"),
              ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    r = run_bench("--summarize", str(tmp_path / "t"))
    assert r.returncode == 0, r.stderr
    assert f"dominant kernel {bench.DOMINANT}: 2 dispatches, mean 10.500 us" in r.stdout
    probe_line = [ln for ln in r.stdout.splitlines() if ln.strip().startswith("probe_read")][0]
    assert probe_line.split()[1:4] == ["1", "600.00", "600.00"]


def test_summarize_counter_calibration(tmp_path):
    # the probe reads 4 GiB per dispatch: 2^21 FETCH_SIZE units means 2048 B
    # per unit; the 4096 x 4096 f32 dequantisation writes 64 MiB: 65536
    # WRITE_SIZE units means 1024 B per unit
    fetch = [(PROBE, "FETCH_SIZE", 2097152.0), (PROBE, "FETCH_SIZE", 2097152.0),
             (DOM, "FETCH_SIZE", 20000.0), (DOM, "FETCH_SIZE", 19000.0)]
    write = [(DEQ, "WRITE_SIZE", 65536.0), (DOM, "WRITE_SIZE", 68.0), (DOM, "WRITE_SIZE", 68.0)]
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    write_csv(str(tmp_path / "fetch" / "run_counter_collection.csv"), hdr, fetch)
    write_csv(str(tmp_path / "write" / "run_counter_collection.csv"), hdr, write)
    r = run_bench("--summarize", str(tmp_path / "fetch"), str(tmp_path / "write"))
    assert r.returncode == 0, r.stderr
    kv = dict(ln.split(":", 1) for ln in r.stdout.splitlines() if ln.endswith(tuple("0123456789abcdef"))
              and ":" in ln and not ln.startswith(" "))
    assert int(kv["fetch_bytes_per_launch"]) == 19500 * 2048
    assert int(kv["write_bytes_per_launch"]) == 68 * 1024
    assert int(kv["traffic_bytes_per_launch"]) == 19500 * 2048 + 68 * 1024
    assert kv["source_sha256"].strip() == bench.kernel_source_hash()


def test_stored_traffic_needs_matching_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.stored_traffic() is None                      # no summary
    f.write_text(f"traffic_bytes_per_launch: 123\nsource_sha256: {'0' * 64}\n")
    assert bench.stored_traffic() is None                      # other kernel sources
    f.write_text(f"traffic_bytes_per_launch: 123\nsource_sha256: {bench.kernel_source_hash()}\n")
    assert bench.stored_traffic() == 123.0
