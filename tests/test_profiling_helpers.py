"""The arithmetic of the rocprofv3 summary helpers on small synthetic CSV
files (no GPU): per-dispatch counter means, the copy-calibrated HBM bytes of
the traffic report, its digest guard, and the kernel-trace table."""
import csv

import pytest

from geometric_context_attention_amd import profiling as P


def _pmc_csv(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, c, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})
    return str(path)


def test_pmc_means_per_dispatch(tmp_path):
    path = _pmc_csv(tmp_path / "p.csv", [("gca::k_attn_bf16<8>", "FETCH_SIZE", 100.0),
                                         ("gca::k_attn_bf16<8>", "FETCH_SIZE", 300.0),
                                         ("gca::k_merge_evict", "FETCH_SIZE", 7.0)])
    s = P.summarize_pmc(path, "k_attn_bf16")
    assert s["FETCH_SIZE"]["total"] == 400.0
    assert s["FETCH_SIZE"]["dispatches"] == 2
    assert s["FETCH_SIZE"]["per_dispatch"] == 200.0
    assert P.pmc_per_dispatch(path, "k_merge_evict", "FETCH_SIZE") == 7.0
    with pytest.raises(KeyError):
        P.pmc_per_dispatch(path, "k_attn_bf16", "WRITE_SIZE")


def test_traffic_report_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    # the copy kernels read 4096 B and wrote 8192 B; FETCH_SIZE saw half of
    # the bytes (2 KiB), WRITE_SIZE all of them (8 KiB): scales x2 and x1
    fetch = _pmc_csv(tmp_path / "f.csv", [("k_attn_bf16", "FETCH_SIZE", 10.0), ("k_attn_bf16", "FETCH_SIZE", 30.0)])
    write = _pmc_csv(tmp_path / "w.csv", [("k_attn_bf16", "WRITE_SIZE", 5.0)])
    cal_f = _pmc_csv(tmp_path / "cf.csv", [("elementwise_kernel", "FETCH_SIZE", 1.0),
                                           ("elementwise_kernel", "FETCH_SIZE", 1.0)])
    cal_w = _pmc_csv(tmp_path / "cw.csv", [("elementwise_kernel", "WRITE_SIZE", 8.0)])
    text = P.traffic_report(fetch, write, cal_f, cal_w, "k_attn_bf16", kv_bytes=40960.0, cal_read=4096.0,
                            cal_written=8192.0, workload="synthetic", commands=["rocprofv3 ..."])
    fields = dict(ln.split(": ", 1) for ln in text.splitlines() if ": " in ln and not ln.startswith("#"))
    assert float(fields["fetch_bytes_per_launch"]) == pytest.approx(20 * 1024 * 2)
    assert float(fields["write_bytes_per_launch"]) == pytest.approx(5 * 1024)
    assert float(fields["hbm_bytes_per_launch"]) == pytest.approx(40 * 1024 + 5 * 1024)
    assert fields["kernel_source_sha256"] == P.kernel_source_digest()
    out = tmp_path / "traffic.txt"
    out.write_text(text)
    assert P.read_traffic(str(out)) == pytest.approx(45 * 1024)
    # a summary taken on another kernel source is not reported
    out.write_text(text.replace(P.kernel_source_digest(), "0" * 64))
    assert P.read_traffic(str(out)) is None
    assert P.read_traffic(str(tmp_path / "missing.txt")) is None


def test_trace_report_table(tmp_path):
    path = tmp_path / "kt_kernel_stats.csv"
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs",
                                           "Percentage"])
        w.writeheader()
        w.writerow({"Name": "gca::k_attn_bf16(gca::AttnArgs)", "Calls": 4, "TotalDurationNs": 600000,
                    "AverageNs": 150000, "MinNs": 100000, "MaxNs": 200000, "Percentage": 95.0})
    text = P.trace_report(str(path), "title", "synthetic", ["rocprofv3 --kernel-trace --stats ..."],
                          bench_line='{"value": 1}')
    assert "gca::k_attn_bf16(gca::AttnArgs) | 4 | 0.60 | 150.00 | 100.00 | 200.00 | 95.00" in text
    assert f"# kernel_source_sha256: {P.kernel_source_digest()}" in text
    assert "rocprofv3" in text and '{"value": 1}' in text
