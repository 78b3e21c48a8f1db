"""Host-side tests of the measurement plumbing (no GPU needed).

* bench.py refuses more than one GPU before touching torch or the device;
* the HBM-traffic record is reported only while it matches the current Pass 1
  source, and the counter-to-bytes calibration computes what it states;
* the CPU oracle baseline runs on a bounded sample and reports its size.
"""

import argparse
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402
from exact_softmax_attention_fbob_amd import profiling  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _write_counters(path, rows):
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=fields)
        wr.writeheader()
        for r in rows:
            wr.writerow(dict(zip(fields, r)))


def test_traffic_record_calibration_and_digest(tmp_path, monkeypatch):
    # counters in KiB as rocprofv3 reports them; the copy of 2 MiB reads 1024 KiB
    # on FETCH_SIZE (factor 2) and writes 2048 KiB (factor 1)
    _write_counters(tmp_path / "f.csv", [(1, "void fbob::pass1_kernel<...>", "FETCH_SIZE", 100.0),
                                         (2, "void fbob::pass1_kernel<...>", "FETCH_SIZE", 300.0),
                                         (3, "other_kernel", "FETCH_SIZE", 9e9)])
    _write_counters(tmp_path / "w.csv", [(1, "void fbob::pass1_kernel<...>", "WRITE_SIZE", 50.0),
                                         (2, "void fbob::pass1_kernel<...>", "WRITE_SIZE", 50.0)])
    _write_counters(tmp_path / "cf.csv", [(7, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 1024.0)])
    _write_counters(tmp_path / "cw.csv", [(7, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 2048.0)])
    out = tmp_path / "rec.json"
    a = argparse.Namespace(fetch=str(tmp_path / "f.csv"), write=str(tmp_path / "w.csv"),
                           copy_fetch=str(tmp_path / "cf.csv"), copy_write=str(tmp_path / "cw.csv"),
                           copy_mib=2, kernel="pass1_kernel", copy_kernel="copyBuffer",
                           workload="h12_n16384_d64_bf16_u01", out=str(out))
    profiling.record(a)
    rec = json.loads(out.read_text())
    assert rec["copy_calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert rec["copy_calibration"]["write_scale"] == pytest.approx(1.0)
    assert rec["read_bytes_per_launch"] == pytest.approx(200.0 * 1024 * 2.0)  # mean of 100, 300
    assert rec["write_bytes_per_launch"] == pytest.approx(50.0 * 1024)
    # bench reports the record only while the digest and the workload match
    monkeypatch.setitem(bench.TRAFFIC_FILES, "pass1_kernel", str(out))
    assert bench.measured_traffic("h12_n16384_d64_bf16_u01") == pytest.approx(
        rec["bytes_per_launch"])
    assert bench.measured_traffic("gpt2_heads_h12_n4096_d64_bf16") is None
    rec["kernel_source_digest"] = "0" * 16
    out.write_text(json.dumps(rec))
    assert bench.measured_traffic("h12_n16384_d64_bf16_u01") is None


def test_source_digest_ignores_comments_only():
    """The counter records are keyed to the code: comments, blank lines and trailing
    spaces do not change the digest, any code change does."""
    a = "int f(int x) {  // doubled\n  return 2 * x; /* why */\n}\n"
    b = "/* header */\nint f(int x) {\n\n  return 2 * x;   \n}\n"
    c = "int f(int x) {\n  return 3 * x;\n}\n"
    assert bench._code_only(a) == bench._code_only(b) == profiling._code_only(a)
    assert bench._code_only(a) != bench._code_only(c)


def test_bench_and_profiling_digest_agree():
    """bench.py and the recorder hash the same Pass 1 and Pass 2 sources."""
    for k in ("pass1_kernel", "pass2_kernel"):
        assert bench.kernel_source_digest(k) == profiling.source_digest(k)


def test_clock_sampler_without_a_gpu():
    """Off a GPU (or without clock access) the sampler reports no clock instead of
    failing, and the bench line then carries nulls for the clock-scaled fractions."""
    with bench.ClockSampler(0, period=0.01) as c:
        pass
    r = c.result()
    assert set(r) == {"samples", "xcd_mean", "average"}
    assert r["xcd_mean"] is None or r["xcd_mean"] > 0


def test_cpu_baseline_on_a_tiny_workload():
    w = workloads.small("tiny_h2_n96_d64_bf16", B=1, H=2, N=96, d=64, dtype="bf16", seed=5)
    r = bench.cpu_baseline(w, budget_s=0.5)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert r["value"] > 0 and r["cores"] >= 1
    assert r["sample"].startswith("192 rows in 2 of 2 heads"), r["sample"]
    # a GQA workload maps query heads to their key/value heads and a causal one counts
    # only the unmasked pairs
    g = workloads.small("tiny_gqa", B=1, H=4, N=64, d=64, dtype="bf16", seed=6, causal=True,
                        extra={"Hkv": 2})
    r = bench.cpu_baseline(g, budget_s=30.0, max_heads=3)
    assert r["sample"].startswith("192 rows in 3 of 4 heads"), r["sample"]
    assert r["extrapolated_full_bob_s"] > 0


@pytest.mark.parametrize("mode", [["--fill-sweep"], ["--causal-ab"], ["--causal-split"], ["--n-sweep"],
                                  ["--row-sums"], ["--split-audit"],
                                  ["--max-n"],
                                  ["--workspace", "--workload", "gpt2_heads_h12_n4096_d64_bf16"]])
def test_measurement_modes_parse_and_need_a_gpu(mode):
    """Each measurement mode parses its arguments and, without a visible GPU, stops with
    exit status 3 and a message instead of falling back to anything on the CPU."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *mode],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 3, r.stderr
    assert "no GPU visible" in r.stderr


def test_sync_debug_flag_is_read_at_import():
    """FBOB_SYNC_DEBUG is read by the binding once, at import (no GPU needed)."""
    code = "import exact_softmax_attention_fbob_amd as fb; print(fb._SYNC_DEBUG)"
    for val, want in (("1", "True"), ("0", "False"), ("", "False")):
        env = dict(os.environ, FBOB_SYNC_DEBUG=val)
        r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                           timeout=300, cwd=ROOT, env=env)
        assert r.returncode == 0, r.stderr
        assert r.stdout.strip() == want, (val, r.stdout)
