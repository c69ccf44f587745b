"""Host-side checks of bench.py: the multi-GPU refusal, the workload's op
count, and the rule that HBM byte counters are reported only for the kernel
source they were taken on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_step_ops_of_the_dit_block():
    # QKV, out, MLP-up, MLP-down of the 1024px block at 8192 tokens
    shapes = [(8192, 3072, 9216), (8192, 3072, 3072), (8192, 3072, 12288), (8192, 12288, 3072)]
    assert [(s.M, s.K, s.N) for s in bench.WORKLOAD.linears] == shapes
    assert bench.WORKLOAD.ops == sum(2 * m * k * n for m, k, n in shapes) == 1855425871872


def test_comparators_run_before_the_timed_steps():
    src = open(os.path.join(ROOT, "bench.py")).read()
    main = src[src.index("def main():"):]
    timed = main.index('log(f"timing {args.steps} steps")')
    for phase in ('log("other workloads")', 'log("bf16 comparator")', 'log("fp8 variant")',
                  'log("dequantize-to-bf16 comparator")', "cold_timings("):
        assert main.index(phase) < timed, phase


def test_defaults_time_a_steady_state():
    sys_argv = sys.argv
    try:
        sys.argv = ["bench.py"]
        args = bench.parse()
    finally:
        sys.argv = sys_argv
    assert args.gpus == 1 and args.warmup >= 50 and args.steps >= 100


def test_traffic_reported_only_for_its_source(tmp_path, monkeypatch):
    rec = json.load(open(bench.PROFILE_TRAFFIC))
    assert set(rec) >= {"gemm_source_sha256", "fetch", "write", "bytes_per_step"}
    assert rec["bytes_per_step"] == rec["fetch"]["bytes_per_step"] + rec["write"]["bytes_per_step"]
    assert len(rec["fetch"]["per_launch_bytes"]) == len(rec["write"]["per_launch_bytes"]) == 4
    # the same record against a source whose hash it names, and against another one
    src = tmp_path / "gemm.hip"
    src.write_bytes(open(bench.GEMM_SOURCE, "rb").read())
    monkeypatch.setattr(bench, "GEMM_SOURCE", str(src))
    prof = tmp_path / "traffic.json"
    import hashlib
    rec["gemm_source_sha256"] = hashlib.sha256(src.read_bytes()).hexdigest()
    prof.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", str(prof))
    assert bench.gemm_traffic() == rec["bytes_per_step"]
    src.write_bytes(src.read_bytes() + b"\n// changed\n")
    assert bench.gemm_traffic() is None


@pytest.mark.parametrize("line", ["processor : 0\nmodel name\t: Some CPU @ 2.0GHz\n"])
def test_cpu_model_parsing(tmp_path, monkeypatch, line):
    f = tmp_path / "cpuinfo"
    f.write_text(line)
    real_open = open

    def fake_open(path, *a, **k):
        return real_open(f if path == "/proc/cpuinfo" else path, *a, **k)

    monkeypatch.setattr("builtins.open", fake_open)
    assert bench.cpu_model() == "Some CPU @ 2.0GHz"


def test_loaded_clock_samples_keep_only_readings_under_load():
    samples = [(0.5, 2405.0, 290.0),    # before the load started
               (1.2, 1750.0, 1210.0), (1.9, 1690.0, 1390.0),
               (2.4, 2400.0, 310.0),    # queue momentarily empty
               (3.5, 1800.0, 1100.0)]   # after the load ended
    assert bench.loaded_samples(samples, 1.0, 3.0, 1400.0) == [(1750.0, 1210.0), (1690.0, 1390.0)]
    assert bench.loaded_samples(samples, 1.0, 3.0, None) == [(1750.0, 1210.0), (1690.0, 1390.0),
                                                              (2400.0, 310.0)]


def test_fraction_at_the_loaded_clock():
    """The peak scales with the clock: at half the nominal clock the same
    achieved rate is twice the fraction; no clock reading, no figure."""
    import bench
    full = bench.at_clock(2500.0, 2400)
    half = bench.at_clock(2500.0, 1200)
    assert full["peak"] == 5000.0 and full["frac"] == 0.5
    assert half["peak"] == 2500.0 and half["frac"] == 1.0
    assert bench.at_clock(2500.0, None) is None and bench.at_clock(2500.0, 0) is None
