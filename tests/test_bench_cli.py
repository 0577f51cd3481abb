"""Command-line contract of bench.py that holds without a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line for a run that did not happen


def test_help_lists_the_timing_flags():
    r = run_bench("--help")
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--warm-seconds", "--workload", "--gpus"):
        assert flag in r.stdout


def test_fused_step_refused_where_it_does_not_apply():
    # refused before any GPU work: FP8 rows, the staged path, and workloads
    # whose step appends a multi-row tail
    for extra in (["--format", "fp8"], ["--path", "staged"], ["--workload", "ragged"],
                  ["--workload", "million"], ["--op", "mtp"]):
        r = run_bench("--step", "fused", *extra)
        assert r.returncode != 0, extra
        assert "--step fused needs" in r.stderr, extra
        assert r.stdout.strip() == ""


def test_traffic_record_format():
    # the stored HBM counter figures are keyed by the decode kernel's source
    # hash (bench.py reports them only for the kernel they were taken on), and
    # each total is the sum of its fetched and written bytes
    rec = os.path.join(ROOT, "profiles", "decode_traffic.txt")
    rows = [l.split() for l in open(rec) if l.strip() and not l.startswith("#")]
    assert rows, "no traffic record"
    for row in rows:
        assert len(row) == 5 and len(row[1]) == 16
        assert int(row[2]) == int(row[3]) + int(row[4])
