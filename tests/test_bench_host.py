"""Host-side checks of bench.py (no GPU): the one-GPU refusal, the trace
summary, the HBM-traffic lookup with its source digests, and the profiler
detection that keeps the clock query from starting a child process under
rocprofv3."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr + r.stdout


def test_summarize_trace_groups_by_kernel_and_grid(tmp_path, capsys):
    rows = [("void ox::patch::conv3x3_reduce<1, 4, 1, 2>(ox::ConvArgs)", 131072, 1000, 8000),
            ("void ox::patch::conv3x3_reduce<1, 4, 1, 2>(ox::ConvArgs)", 131072, 9000, 16000),
            ("void ox::patch::conv3x3_reduce<1, 4, 1, 2>(ox::ConvArgs)", 131072, 17000, 26000),
            ("void ox::pw::conv1x1_reduce<2, 2, 1, 2>(ox::ConvArgs)", 102400, 30000, 37000),
            ("void at::native::copy_kernel(int)", 4096, 40000, 41000)]
    p = tmp_path / "k_kernel_trace.csv"
    with open(p, "w") as f:
        f.write("Kernel_Name,Grid_Size,Start_Timestamp,End_Timestamp\n")
        for name, grid, t0, t1 in rows:
            f.write('"%s",%d,%d,%d\n' % (name, grid, t0, t1))
    bench.summarize_trace(str(p))
    out = capsys.readouterr().out.splitlines()
    body = [l for l in out if l.startswith("| `")]
    assert len(body) == 2                      # torch's kernel left out
    # three dispatches of 7, 7 and 9 us: median 7, min 7, mean 7.67
    assert body[0] == "| `void ox::patch::conv3x3_reduce<1, 4, 1, 2>` | 131072 | 3 | 7.00 | 7.00 | 7.67 |"
    assert body[1].startswith("| `void ox::pw::conv1x1_reduce<2, 2, 1, 2>` | 102400 | 1 | 7.00 |")


def test_measured_traffic_follows_the_sources(tmp_path, monkeypatch):
    # a summary entry is used only while the digest of the kernel's sources
    # matches the one recorded with the counters
    src = tmp_path / "k.hip"
    src.write_text("kernel source\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    digest = bench._sources_digest(["k.hip"])
    (tmp_path / "profiles" / "hbm_traffic_wl_bf16.txt").write_text(
        "# comment\nkernel=fam/bf16|k.hip|%s|123456\n" % digest)
    assert bench.measured_traffic("fam/bf16", "wl", "bf16") == (123456.0, "profiles/hbm_traffic_wl_bf16.txt")
    assert bench.measured_traffic("other/bf16", "wl", "bf16") is None
    assert bench.measured_traffic("fam/bf16", "wl", "f32") is None      # no summary for this dtype
    src.write_text("kernel source, changed\n")
    assert bench.measured_traffic("fam/bf16", "wl", "bf16") is None


@pytest.mark.parametrize("env,expect", [
    ({}, False),
    ({"LD_PRELOAD": "/opt/rocm/lib/rocprofiler-sdk/librocprofiler-sdk-tool.so"}, True),
    ({"ROCPROF_OUTPUT_PATH": "/tmp/x"}, True),
    ({"LD_PRELOAD": "/usr/lib/libother.so"}, False),
])
def test_profiler_detection(monkeypatch, env, expect):
    for k in list(os.environ):
        if k.startswith("ROCPROF") or k == "LD_PRELOAD":
            monkeypatch.delenv(k, raising=False)
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    assert bench.under_profiler() is expect
    if expect:
        assert bench.gpu_clocks() is None       # no child process under a profiler
