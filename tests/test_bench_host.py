"""Host-side logic of bench.py, without a GPU: the one-GPU refusal, the step's algorithmic byte
count, and the guard that reports a profile's traffic figure only for the sources it measured."""
import os
import shutil
import subprocess
import sys

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
        "text\ntraffic-record: kernel=pipe_kernel<true> M=4096 source=%s bytes=123456789\n" % h)
    name = "pipe_kernel<true> (hc_post_stats)"
    assert bench.recorded_traffic(name, files) == 123456789
    assert bench.recorded_traffic("post_kernel (hc_post)", files) is None  # another kernel
    with open(csrc / "hc_pipe.hip", "a") as fh:  # the kernel's source changes
        fh.write("\n")
    assert bench.recorded_traffic(name, files) is None
