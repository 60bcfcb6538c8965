"""Host logic of the benchmark: the refusal of more than one GPU, and the
summaries of rocprofv3 kernel traces and counter runs that the committed
profiles (and the bench line's `traffic`) are made with, on small synthetic
inputs whose statistics are known."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

pytestmark = pytest.mark.filterwarnings("ignore")

FIELDS = ["Kind", "Agent_Id", "Queue_Id", "Kernel_Name", "Correlation_Id", "Start_Timestamp",
          "End_Timestamp"]
CASES = {"q4_0_gemv_case_a": {"bytes": 8_000_000, "ms": 0.0051},
         "q8_0_gemm_case_b": {"flops": 2_500_000_000, "ms": 0.0102}}
KERNELS = {"q4_0_gemv_case_a": "void lqmm::(anonymous namespace)::kern_a<1, 2>(int const*, int)",
           "q8_0_gemm_case_b": "void lqmm::(anonymous namespace)::kern_b<8>(int const*, int)"}


def _trace(tmp_path, per=10):
    """A kernel trace: three settle launches of each kernel, the begin marker,
    `per` timed launches of each case (case a: 1..per us, case b: 10 us
    apart from its fifth launch, 30 us), the end marker, one context launch."""
    rows, t = [], 1_000_000

    def add(name, dur_us):
        nonlocal t
        rows.append({"Kind": "KERNEL_DISPATCH", "Agent_Id": 1, "Queue_Id": 1, "Kernel_Name": name,
                     "Correlation_Id": len(rows), "Start_Timestamp": t,
                     "End_Timestamp": t + int(dur_us * 1000)})
        t += int(dur_us * 1000) + 500
    for _ in range(3):
        add(KERNELS["q4_0_gemv_case_a"], 4.0)
        add(KERNELS["q8_0_gemm_case_b"], 8.0)
    add("(anonymous namespace)::timed_region_begin_marker()", 1.0)
    for i in range(per):
        add(KERNELS["q4_0_gemv_case_a"], float(i + 1))
    for i in range(per):
        add(KERNELS["q8_0_gemm_case_b"], 30.0 if i == 4 else 10.0)
    add("(anonymous namespace)::timed_region_end_marker()", 1.0)
    add("Cijk_Ailk_Bljk_HHS_BH_MT128x128x64_MI16x16x1_SN", 50.0)
    d = tmp_path / "trace" / "host"
    d.mkdir(parents=True)
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        w.writerows(rows)
    line = {"metric": "m", "steps": per, "warmup": 2, "cases": CASES,
            "config": {"workload": "synthetic trace"},
            "roofline": {"case": "q4_0_gemv_case_a", "frac": 0.5}}
    log = tmp_path / "bench.log"
    log.write_text("[bench] noise\n" + json.dumps(line) + "\n")
    return str(tmp_path / "trace"), str(log)


def test_summarize_trace_statistics(tmp_path):
    trace, log = _trace(tmp_path)
    out = tmp_path / "trace.md"
    bench.summarize_trace(trace, log, str(out), "CMD")
    text = out.read_text()
    rows = {l.split("|")[1].strip(): [c.strip() for c in l.split("|")[1:-1]]
            for l in text.splitlines() if l.startswith("| q")}
    a, b = rows["q4_0_gemv_case_a"], rows["q8_0_gemm_case_b"]
    # case a: durations 1..10 us: mean 5.5, median 5.5, p10 1.9, p90 9.1 (linear interpolation)
    assert a[1] == "`kern_a<1, 2>`" and a[2] == "10"
    assert [float(v) for v in a[3:7]] == [5.5, 5.5, 1.9, 9.1]
    assert a[7] == "5.10"                                # the bench line's event time
    assert a[8] == f"{8e6 / 5.5e-6 / 1e9:.0f} GB/s"
    assert float(a[9]) == pytest.approx(8e6 / 5.5e-6 / 1e9 / bench.HBM_PEAK_GBS, abs=6e-4)
    # case b: nine launches of 10 us and one of 30 us; flops against the f16 peak
    assert [float(v) for v in b[3:5]] == [12.0, 10.0]
    assert b[8] == f"{2.5e9 / 12e-6 / 1e12:.1f} TFLOP/s"
    # launches outside the markers are listed apart, vendor kernels by tile name
    assert "| `kern_a<1, 2>` | 3 | 4.00 | 4.00 |" in text
    assert "vendor GEMM Ailk MT128x128x64_MI16x16x1" in text
    assert "CMD" in text


def test_summarize_series_blocks(tmp_path):
    trace, log = _trace(tmp_path, per=20)
    out = tmp_path / "series.md"
    bench.summarize_series(trace, log, str(out), "CMD")
    text = out.read_text()
    # case a: 1..20 us, blocks of ten: means 5.5 and 15.5; settle launches 3 at 4 us
    assert "- q4_0_gemv_case_a: 5.5, 15.5" in text
    assert "| q4_0_gemv_case_a | `kern_a<1, 2>` | 1.00 | 10.50 | 20.00 | 3, 4.00 |" in text
    # case b: one 30 us launch in the first block
    assert "- q8_0_gemm_case_b: 12.0, 10.0" in text


def test_trace_must_split_over_cases(tmp_path):
    trace, log = _trace(tmp_path)
    line = json.loads(open(log).read().splitlines()[-1])
    line["cases"]["third_case"] = {"bytes": 1, "ms": 0.001}
    with open(log, "w") as f:
        f.write(json.dumps(line) + "\n")
    with pytest.raises(SystemExit):
        bench.summarize_trace(trace, log, str(tmp_path / "x.md"), "CMD")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout + r.stderr


def _pmc(d, rows):
    d.mkdir(parents=True)
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        w.writerows(rows)


def test_summarize_traffic_scaling(tmp_path, monkeypatch):
    """FETCH_SIZE and WRITE_SIZE per dispatch (KiB), each scaled by what it
    reads for the calibration copy of 256 MiB: here FETCH_SIZE counts half
    the bytes (scale 2) and WRITE_SIZE all of them (scale 1)."""
    kern = "void lqmm::(anonymous namespace)::kern_a<1, 2>(int const*, int)"
    neg = "void at::native::vectorized_elementwise_kernel<4, neg_kernel_cuda>(int)"
    pmc = tmp_path / "pmc"
    fetch, write = [], []
    for i, (fv, wv) in enumerate([(1000.0, 10.0), (1002.0, 10.0), (998.0, 10.0)]):
        # a counter is summed over the rows of one dispatch (one per XCD here: two halves)
        fetch += [dict(Dispatch_Id=i, Kernel_Name=kern, Counter_Name="FETCH_SIZE",
                       Counter_Value=fv / 2)] * 2
        write += [dict(Dispatch_Id=i, Kernel_Name=kern, Counter_Name="WRITE_SIZE",
                       Counter_Value=wv)]
    fetch.append(dict(Dispatch_Id=9, Kernel_Name=neg, Counter_Name="FETCH_SIZE",
                      Counter_Value=256 * 1024 / 2))
    write.append(dict(Dispatch_Id=9, Kernel_Name=neg, Counter_Name="WRITE_SIZE",
                      Counter_Value=256 * 1024))
    _pmc(pmc / "case_a.fetch" / "host", fetch)
    _pmc(pmc / "case_a.write" / "host", write)
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    bench.summarize_traffic(str(pmc), 256, "CMD")
    t = json.loads(out.read_text())
    c = t["cases"]["case_a"]
    assert c["fetch_scale"] == 2.0 and c["write_scale"] == 1.0
    assert c["dispatches"] == {"fetch": 3, "write": 3}
    assert c["fetch_kib_per_dispatch"] == 1000.0 and c["write_kib_per_dispatch"] == 10.0
    assert c["hbm_bytes_per_launch"] == (1000 * 2 + 10) * 1024
    assert t["kernel_source_sha256"] == bench.kernel_source_sha256()
    assert t["command"] == "CMD"
