"""bench.py's host-side helpers (no GPU): the kernel-name decoder and the
summaries that turn rocprofv3 counter and trace runs into profiles/ tables."""
import csv
import importlib.util
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_kernel_names(bench):
    k = bench._kernel_name
    assert k("_ZN2pa11decode_mfmaIDF16_Li128ELi16ELi1ELi2ELi2ELb0ELb1EEEvNS_9SplitArgsIT_EEPKiS5_") == \
        "pa::decode_mfma<_Float16, 128, 16, 1, 2, 2, false, true>"
    assert k("_ZN2pa13combine_splitINS_6bf16_tELi128ELi1ELi1ELi8EEEvNS_16SplitCombineArgsIT_EE") == \
        "pa::combine_split<pa::bf16_t, 128, 1, 1, 8>"
    assert k("_ZN2pa11decode_valuIfLi64ELi16ELi4ELb0EEEvNS_10DecodeArgsIT_EE") == \
        "pa::decode_valu<float, 64, 16, 4, false>"
    # names the trace already demangled, or of other libraries, are left alone
    assert k("void pa::combine_split<pa::bf16_t, 128, 4>(x)") == "void pa::combine_split<pa::bf16_t, 128, 4>(x)"
    assert k("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"
    # an argument form it does not know: the mangled name is kept
    assert k("_ZN2pa3fooIdEEvv") == "_ZN2pa3fooIdEEvv"


FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "pmc_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(FIELDS, r)))


def test_summarize_traffic(bench, tmp_path, monkeypatch, capsys):
    d = tmp_path / "prof"
    kib = 256 * 1024  # a 256 MiB copy
    # the copy reads as half its bytes in FETCH_SIZE (64-byte units of 128-byte moves)
    _write_counters(str(d / "cal_fetch"), [(1, "copy", "FETCH_SIZE", kib / 2), (2, "setup", "FETCH_SIZE", 4),
                                          (3, "copy", "FETCH_SIZE", kib / 2)])
    _write_counters(str(d / "cal_write"), [(1, "copy", "WRITE_SIZE", kib)])
    # two dispatches of pass 1 (one counter split over two rows of a dispatch) and a combine
    _write_counters(str(d / "fetch_w"), [(10, "pa::decode_mfma<...>", "FETCH_SIZE", 300.0),
                                         (10, "pa::decode_mfma<...>", "FETCH_SIZE", 200.0),
                                         (11, "pa::decode_mfma<...>", "FETCH_SIZE", 500.0),
                                         (12, "pa::combine_split<...>", "FETCH_SIZE", 8.0)])
    _write_counters(str(d / "write_w"), [(10, "pa::decode_mfma<...>", "WRITE_SIZE", 10.0),
                                         (12, "pa::combine_split<...>", "WRITE_SIZE", 1.0)])
    with open(d / "fetch_w.out", "w") as f:
        f.write("log line\n" + json.dumps({"configs": {"w": {"kv_bytes_per_step": 1000 * 1024}}}) + "\n")
    out_json = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out_json))
    bench.summarize_traffic(str(d))
    data = json.loads(out_json.read_text())
    assert data["copy_scale"]["FETCH_SIZE"] == pytest.approx(2.0)
    assert data["copy_scale"]["WRITE_SIZE"] == pytest.approx(1.0)
    e = data["w"]
    assert e["pass 1"]["fetch_kib_raw"] == pytest.approx(500.0)  # per dispatch
    assert e["pass 1"]["read_bytes"] == pytest.approx(500.0 * 1024 * 2)
    assert e["pass 1"]["write_bytes"] == pytest.approx(10.0 * 1024)
    assert e["combine"]["read_bytes"] == pytest.approx(8.0 * 1024 * 2)
    assert e["hbm_bytes_per_launch"] == pytest.approx(500.0 * 1024 * 2 + 10.0 * 1024)
    assert e["kernel_source_sha"] == bench.kernel_source_hash()
    table = capsys.readouterr().out
    assert "| w | pass 1 | 2 | 500.0 |" in table and "| 1.000 |" in table


def test_summarize_trace(bench, tmp_path, capsys):
    d = tmp_path / "kt"
    d.mkdir()
    with open(d / "kt_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow(["_ZN2pa11decode_mfmaIDF16_Li128ELi16ELi1ELi2ELi2ELb0ELb1EEEvNS_9SplitArgsIT_EEPKiS5_",
                    220, 1e7, 45880.0, 84.9, 44230.0, 60150.0, 1.0])
    bench.summarize_trace(str(d))
    out = capsys.readouterr().out.splitlines()
    assert out[0].startswith("| kernel | calls | avg us")
    assert out[2] == "| pa::decode_mfma<_Float16, 128, 16, 1, 2, 2, false, true> | 220 | 45.88 | 44.23 | 60.15 | 84.9% |"
