"""Host-side logic of bench.py, without a GPU: the one-GPU refusal, the step's algorithmic byte
count, and the guard that reports a profile's traffic figure only for the sources it measured."""
import os
import shutil
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_bench(args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, env=env)


def test_more_than_one_gpu_is_refused():
    r = _run_bench(["--gpus", "2"])
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
    r = _run_bench([], env=dict(os.environ, WORLD_SIZE="4"))  # as under a multi-rank launcher
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_step_bytes():
    H = 5120
    post_row = 2 * (4 * H + H + 4 * H) + 4 * (4 + 16)  # R, x in; R' out; post, comb
    pre_row = 2 * (4 * H + H) + 4 * (4 + 4 + 16)       # R' in; y out; pre, post, comb out
    assert (bench.POST_BYTES_ROW, bench.PRE_BYTES_ROW) == (post_row, pre_row) == (92240, 51296)
    assert bench.STEP_BYTES == 4096 * (post_row + pre_row) + 24 * 4 * H * 4 + 2 * H
    assert bench.ROOFLINE_KERNEL["fused"][1] == 4096 * post_row + 24 * 4 * H * 4


def test_traffic_record_follows_the_source_hash(tmp_path, monkeypatch):
    csrc = tmp_path / "hyper_connection_residual_hc_amd" / "csrc"
    csrc.mkdir(parents=True)
    files = ["hc_pipe.hip", "hc_device.h", "hc_launch.h"]
    for f in files:
        shutil.copy(os.path.join(ROOT, "hyper_connection_residual_hc_amd", "csrc", f), csrc / f)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h = bench.kernel_source_hash(files)
    assert len(h) == 16 and h == bench.kernel_source_hash(files)
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "k.md").write_text(
        "text\ntraffic-record: kernel=stats_kernel<10,true> M=4096 source=%s bytes=123456789\n" % h)
    name = "stats_kernel<10,true> (hc_post_stats)"
    assert bench.recorded_traffic(name, files) == 123456789
    assert bench.recorded_traffic(name, files, 16384) is None  # another row count
    assert bench.recorded_traffic("post_kernel (hc_post)", files) is None  # another kernel
    with open(csrc / "hc_pipe.hip", "a") as fh:  # the kernel's source changes
        fh.write("\n")
    assert bench.recorded_traffic(name, files) is None


def test_trace_regions_split_the_step_and_back_to_back_launches(tmp_path):
    """The last K dispatches of a kernel are the back-to-back region, the K before them the
    timed step region; other kernels and the setup / warm-up dispatches do not count."""
    K, W = 4, 2
    lines = ["Kind,Kernel_Name,Start_Timestamp,End_Timestamp"]
    t = 0
    def add(name, us):
        nonlocal t
        lines.append('KERNEL_DISPATCH,"%s",%d,%d' % (name, t, t + int(us * 1000)))
        t += int(us * 1000) + 500
    stats = "void hc::stats_kernel<10, true>(hc::PipeArgs)"
    fin = "void hc::pre_finish_kernel<10, false>(float const*, int)"
    add("void hc::stats_kernel<10, false>(hc::PipeArgs)", 40.0)  # setup pre
    add(fin, 30.0)
    for i in range(W + K):  # warm-up and timed steps
        add(stats, 70.0 if i >= W else 90.0)
        add(fin, 33.0)
    for i in range(K):
        add(stats, 80.0 + i)  # back to back
    for i in range(K):
        add(fin, 36.0)
    path = tmp_path / "run_kernel_trace.csv"
    path.write_text("\n".join(lines) + "\n")
    rec = bench.trace_regions(str(path), K, ["stats_kernel<10,true>", "pre_finish_kernel<10,"])
    assert rec[0]["dispatches"] == W + 2 * K
    assert rec[0]["step_region_avg_us"] == pytest.approx(70.0)
    assert rec[0]["back_to_back_avg_us"] == pytest.approx(81.5)
    assert rec[1]["dispatches"] == 1 + W + 2 * K
    assert rec[1]["step_region_avg_us"] == pytest.approx(33.0)
    assert rec[1]["back_to_back_avg_us"] == pytest.approx(36.0)
