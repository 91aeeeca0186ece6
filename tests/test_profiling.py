"""The profiler report (CPU): counter scaling and the stored-traffic lookup,
on hand-made rocprofv3 CSV files."""
import csv
import json
import os

from tiered_kv_cache_hs_amd import inputs as I
from tiered_kv_cache_hs_amd import profiling as P


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def test_report_scales_counters_by_the_copy_reading(tmp_path):
    out = str(tmp_path)
    # the 256 MiB copy reads as 128 MiB of FETCH_SIZE and 256 MiB of WRITE_SIZE
    _write(f"{out}/pmc_copy_FETCH_SIZE/h/run_counter_collection.csv", ["Kernel_Name", "Counter_Value"],
           [["__amd_rocclr_copyBuffer", 131072.0]])
    _write(f"{out}/pmc_copy_WRITE_SIZE/h/run_counter_collection.csv", ["Kernel_Name", "Counter_Value"],
           [["__amd_rocclr_copyBuffer", 262144.0]])
    for c, vals in (("FETCH_SIZE", [100.0, 300.0, 200.0]), ("WRITE_SIZE", [10.0, 10.0, 40.0])):
        _write(f"{out}/pmc_wl1_{c}/h/run_counter_collection.csv", ["Kernel_Name", "Counter_Value"],
               [["hs_k_attn_mha<float, 64, 1, true>(...)", v] for v in vals])
    kname = "void hs::(anonymous namespace)::hs_k_attn_mha<float, 64, 1, true>(hs::UnitDesc const*)"
    _write(f"{out}/trace_wl1/h/bench_kernel_stats.csv",
           ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"],
           [[kname, 64, 11000, 10000, 12000, 50.0]])
    _write(f"{out}/trace_wl1/h/bench_kernel_trace.csv",
           ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "VGPR_Count"],
           [[kname, 1000 * i, 1000 * i + 5000 + (9000 if i % 32 == 0 else 0), 96]
            for i in range(64)])
    P.report([1], out)
    doc = json.load(open(f"{out}/report/pmc_traffic.json"))
    assert doc["scale"]["FETCH_SIZE"] == 2.0 and doc["scale"]["WRITE_SIZE"] == 1.0
    (e,) = doc["entries"]
    assert e["kernel"] == "hs_k_attn_mha" and e["workload"] == I.workload(1).name
    assert e["traffic_bytes"] == int((200.0 * 2.0 + 10.0) * 1024)
    assert e["sources_sha1"] == P.kernel_sources_sha1("hs_k_attn_mha")
    md = open(f"{out}/report/hs_kernels_{I.workload(1).name}.md").read()
    assert "| hs_k_attn_mha<float, 64, 1, true> | 62 | 5.00 | 5.00 |" in md  # cold steps dropped
    assert "| hs_k_attn_mha<float, 64, 1, true> | 64 | 11.00 | 10.00 | 12.00 | 50.00 |" in md
    assert "| hs_k_attn_mha<float, 64, 1, true> | 96 |" in md


def test_stored_traffic_only_while_sources_match(tmp_path, monkeypatch):
    f = tmp_path / "pmc.json"
    good = P.kernel_sources_sha1("hs_k_resolve")
    f.write_text(json.dumps({"entries": [
        {"workload": "w", "kernel": "hs_k_resolve", "sources_sha1": good, "traffic_bytes": 123},
        {"workload": "w", "kernel": "hs_k_gather", "sources_sha1": "0" * 40, "traffic_bytes": 9}]}))
    monkeypatch.setattr(P, "PMC_FILE", str(f))
    assert P.stored_traffic("w", "hs_k_resolve") == 123
    assert P.stored_traffic("w", "hs_k_gather") is None
    assert P.stored_traffic("other", "hs_k_resolve") is None


def test_bench_report_takes_the_launches_the_benchmark_times(tmp_path):
    """The measured-benchmark summary averages, per kernel, the dispatches of
    the benchmark's last (eager, dispatch-timed) pass: the last K of 5 (W + K);
    and recomputes the roofline fraction from those durations."""
    out = str(tmp_path)
    W, K = 2, 4
    kname = "void hs::(anonymous namespace)::hs_k_resolve<1024, 4, 2, true>(hs::UnitDesc const*)"
    # five passes of W + K steps; durations 10 us in the first four passes,
    # 20 us in the eager pass's warm-up steps and 30 us in its K timed ones
    durs = [10.0] * (4 * (W + K)) + [20.0] * W + [30.0] * K
    _write(f"{out}/trace_bench/h/bench_kernel_trace.csv",
           ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
           [[kname, 100000 * i, 100000 * i + int(d * 1000)] for i, d in enumerate(durs)])
    line = {"metric": "m", "value": 1.0, "warmup": W, "steps": K,
            "config": {"workload": I.workload(3).name, "path": "p"},
            "kernels_us": {"resolve": 33.0},
            "roofline": {"kernel": "hs_k_resolve", "bytes_per_launch": 1_500_000, "peak": 63.0,
                         "unit": "GB/s", "frac": 0.7, "avg_us": 33.0}}
    os.makedirs(out, exist_ok=True)
    with open(f"{out}/trace_bench.log", "w") as fh:
        fh.write("noise\n" + json.dumps(line) + "\n")
    md = open(P.bench_report(out)).read()
    assert "| hs_k_resolve<1024, 4, 2, true> | 30 | 30.00 | 30.00 | 33.00 | 10.00 |" in md
    # 1.5 MB / 30 us = 50 GB/s = 0.7937 of 63
    assert "= 50.00 GB/s, frac 0.7937" in md
