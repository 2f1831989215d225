"""Host-side logic of bench.py (no GPU): the one-GPU guard and the lookup of
HBM traffic in the committed rocprofv3 counter summaries."""

import glob
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=300)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def _traffic_lines():
    for path in glob.glob(os.path.join(ROOT, "profiles", "*_rocprof.txt")):
        for line in open(path):
            if line.startswith("traffic_bytes "):
                sym = line[len("traffic_bytes "):line.index(" grid=")]
                fields = line.split()
                yield path, sym, int(fields[-2]), fields[-1].split("=", 1)[1]


def test_counter_traffic_reads_the_dominant_kernel():
    # the dense workload's dominant kernel is the wgrad GEMM; its summary line
    # must be found and returned as bytes per launch
    # (None once the kernel's sources differ from those the counters were taken on)
    sym = bench.KERNEL_SYMBOL["gemm_wgrad"]
    want = [(b, h) for p, s, b, h in _traffic_lines()
            if os.path.basename(p) == "dense_8192x4096x4096_rocprof.txt" and s == sym]
    assert len(want) == 1
    got = bench.counter_traffic("dense_8192x4096x4096", "gemm_wgrad")
    if want[0][1] != bench.kernel_source_hash(sym):
        assert got is None
        return
    assert got == want[0][0]
    # above the algorithmic bytes (two 32 MiB operands and a 32 MiB output)
    # and below what no cache reuse at all would move
    assert 96 << 20 < got < 1 << 30


def test_counter_traffic_without_a_summary_is_none():
    assert bench.counter_traffic("linear_fwd_256x512x256", "gemm_fwd") is None
    assert bench.counter_traffic("dense_8192x4096x4096", "no_such_kernel") is None
    assert bench.kernel_source_hash("no_such_kernel<0>") is None


def test_source_hash_ignores_comments_but_not_code():
    code = 'int a = 1; // note\n/* block\n  note */ const char* s = "x // kept"; char q = \'"\'; a /= 2;\n'
    assert bench._code_only(code) == 'int a = 1; const char* s = "x // kept"; char q = \'"\'; a /= 2;'
    # a comment edit and a whitespace change leave the code unchanged; a code edit does not
    assert bench._code_only(code.replace("note", "other words")) == bench._code_only(code)
    assert bench._code_only(code.replace("a = 1;", "a  =\n 1;")) == bench._code_only(code)
    assert bench._code_only(code.replace("a /= 2", "a /= 3")) != bench._code_only(code)


def test_clock_samples_count_each_table_update_once():
    # the driver's metrics table changes about once a second; repeated reads of
    # one update, and the update current before the work started, are not samples
    c = bench.ClockSampler.__new__(bench.ClockSampler)
    c.ts0, c.error, c.extra_steps = 100, None, 0
    c.samples = [(100, 250.0, 1900.0), (100, 250.0, 1900.0), (200, 2000.0, 2000.0), (200, 2000.0, 2000.0),
                 (300, 1900.0, 2000.0)]
    assert c.fresh() == [(2000.0, 2000.0), (1900.0, 2000.0)]
    summ = c.summary(extra_steps=3)
    assert summ["samples"] == 2 and summ["sclk_mhz"] == 1950 and summ["sclk_min_mhz"] == 1900
    assert "3 further untimed steps" in summ["source"]
    c.samples = [(100, 250.0, 1900.0)]
    summ = c.summary()
    assert summ["sclk_mhz"] is None and summ["samples"] == 0 and "not updated" in summ["error"]
