"""Host checks of bench.py's bookkeeping (no GPU): the refusal of more than one GPU, the
HBM-traffic and clock summaries it writes from rocprofv3 counter CSVs, and the rule that a
summary counts only while the kernel's sources are unchanged."""

import csv
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(tmp_path, monkeypatch):
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    monkeypatch.setattr(mod, "TRAFFIC_FILE", str(tmp_path / "traffic.txt"))
    monkeypatch.setattr(mod, "CLOCK_FILE", str(tmp_path / "clock.txt"))
    return mod


def _counter_csv(path, counter, rows):
    """rows: (dispatch id, kernel name, value)."""
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for did, name, val in rows:
            w.writerow([did, name, counter, val])


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_summary_round_trip(tmp_path, monkeypatch):
    b = _bench(tmp_path, monkeypatch)
    attn = "void mi355::attn_fwd_bf16_kernel<128, true>(Params)"
    soft = "void mi355::softmax_rows_reg<1, 16, true>(float const*)"
    copy = "__amd_rocclr_copyBuffer"
    # a 1 GiB copy reads 2^20 KiB on the fetch counter at scale 1 and 2^19 at scale 2;
    # small copies (host transfers) must not calibrate
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [
        (1, copy, 4.0), (2, attn, 300000.0), (3, attn, 280000.0), (4, attn, 290000.0),
        (5, soft, 524288.0), (6, copy, 524288.0), (7, copy, 524288.0)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [
        (1, copy, 2.0), (2, attn, 131072.0), (3, attn, 131072.0), (4, attn, 131072.0),
        (5, soft, 1048576.0), (6, copy, 1048576.0), (7, copy, 1048576.0)])
    b.write_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 1024)
    t = b.read_traffic()
    assert set(t) == {"attn_fwd_bf16", "softmax_rows"}
    # median fetch 290000 KiB x 2 (calibration), write 131072 KiB x 1
    assert t["attn_fwd_bf16"] == pytest.approx(290000.0 * 1024 * 2 + 131072.0 * 1024)
    assert t["softmax_rows"] == pytest.approx(2 * (1 << 30))


def test_clock_summary_round_trip(tmp_path, monkeypatch):
    b = _bench(tmp_path, monkeypatch)
    attn = "void mi355::attn_fwd_bf16_kernel<128, true>(Params)"
    rows, trace = [], []
    for i in range(8):
        dur_ns = 1_000_000  # 1 ms
        ghz = 1.5 if i < 2 else 1.7  # the first quarter (cold) is dropped
        rows.append((i, attn, 8 * ghz * 1e9 * dur_ns * 1e-9))
        trace.append({"Dispatch_Id": i, "Start_Timestamp": 10 * dur_ns * i, "End_Timestamp": 10 * dur_ns * i + dur_ns})
    _counter_csv(tmp_path / "c.csv", "GRBM_GUI_ACTIVE", rows)
    with open(tmp_path / "t.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(trace)
    b.write_clock(str(tmp_path / "c.csv"), str(tmp_path / "t.csv"))
    clk = b.read_clock()
    assert float(clk["ghz_median"]) == pytest.approx(1.7, rel=1e-4)
    assert int(clk["dispatches"]) == 6


def test_summaries_expire_when_sources_change(tmp_path, monkeypatch):
    b = _bench(tmp_path, monkeypatch)
    line = f"kernel attn_fwd_bf16 sources_sha256_16 {b.sources_sha('attn_fwd_bf16')} fetch_bytes 10 write_bytes 5\n"
    (tmp_path / "traffic.txt").write_text(line)
    assert b.read_traffic() == {"attn_fwd_bf16": 15.0}
    (tmp_path / "traffic.txt").write_text(line.replace(b.sources_sha("attn_fwd_bf16"), "0" * 16))
    assert b.read_traffic() == {}
