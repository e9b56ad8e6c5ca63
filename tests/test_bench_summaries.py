"""Host-side checks of bench.py's profile summaries (no GPU): the kernel-trace
summary reads rocprofv3's kernel_stats.csv and, given the profiled run's stdout,
sets the run's own event time of the GEMM call beside the sum of the averages of
the two kernels that call launches."""
import importlib.util
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _stats_dir(tmp_path):
    d = tmp_path / "trace" / "host"
    d.mkdir(parents=True)
    (d / "bench_kernel_stats.csv").write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        '"void qk::v4::gemm_fast_kernel<1, true>(qk::v4::GemmGroup)",17,1,1500000,80.0,1400000,1600000,0\n'
        '"void qk::v4::lora_xa_kernel<1, true>(qk::v4::XaGroup)",17,1,100000,5.0,90000,110000,0\n'
        '"qk::dq_quantize_group(qk::DqGroup)",17,1,8000,0.4,7000,9000,0\n')
    return tmp_path / "trace"


def test_trace_summary_with_the_runs_own_event_time(tmp_path):
    bench = _bench()
    log = tmp_path / "run.log"
    line = {"metric": "m", "roofline": {"us_per_launch": 1632.0, "kernel": "the GEMM call",
                                        "achieved": 1000.0, "unit": "TFLOP/s"}}
    log.write_text("progress line\n" + json.dumps(line) + "\n")
    out = tmp_path / "stats.md"
    assert bench.summarize_trace(str(_stats_dir(tmp_path)), str(out), "cmd", str(log)) == 0
    text = out.read_text()
    assert "| 17 | 1500.00 | 1400.00 | 1600.00 | 80.00% |" in text
    assert "1632.00 us per grouped GEMM call" in text
    # 1500 + 100 = 1600 us in the trace; the events read 2.0% more
    assert "1500.00 + 100.00): 1600.00 us (+2.0% for the events)" in text


def test_trace_summary_without_a_bench_line_fails(tmp_path):
    bench = _bench()
    log = tmp_path / "run.log"
    log.write_text("no json here\n")
    assert bench.summarize_trace(str(_stats_dir(tmp_path)), str(tmp_path / "s.md"), "cmd", str(log)) == 1
    assert bench.summarize_trace(str(tmp_path / "missing"), str(tmp_path / "s.md"), "cmd") == 1
