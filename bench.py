"""Throughput of the mHC post + pre hot path on one MI355X.

One step = hc_post of the attention site followed by hc_pre of the FFN site on the same
M = 4096 rows (H = 5120, 4 streams): the decoder layer's back-to-back sequence
(deepseek_v4.py, DeepseekV4DecoderLayer.forward: hc_post(attn) then hc_pre(ffn)), i.e. one
pre and one post over one batch. The post's coefficients come from an attention-site pre run
at setup. Inputs are seeded synthetic tensors with the distributions of the one-GPU test page;
several independent input sets rotate so that no step finds its inputs in the 256 MB
Infinity Cache.

The default path runs the step as the fused post -> pre (hc_post_pre: one kernel writes R' and
the FFN site's mix-stat partials in one pass, a second one finishes the pre); --path unfused
runs hc_post then hc_pre. The metric's timed region has no events inside the steps.

Prints one JSON line: rows/s of the whole step, the HBM roofline of the dominant kernel and the
CPU oracle's rows/s on a bounded sample of the same workload. The dominant kernel (the fused
path's hc_post_stats, i.e. stats_kernel<10, true>; or hc_post) is timed in a region of its own:
K back-to-back launches on the rotating input sets between one pair of HIP events recorded on
the stream it runs on, divided by K. The roofline's "traffic" is the HBM byte count that
rocprofv3's FETCH_SIZE / WRITE_SIZE counters gave for that kernel; it is read from the summary
under profiles/ and reported only while the kernel's source files still hash to what that
summary records (null otherwise). "traffic_gbps" is that byte count over the same
back-to-back duration.

--workload config3 / config4 time the other two chained workloads instead (one JSON line
each, no CPU baseline): the M = 1500 chain pre(attn) -> post -> pre(ffn), and the M = 16384
prefill chunk post -> pre(ffn) -> row-local MXFP8 of y (prefill_sp.py, module docstring
stage 2), run as hc_post_pre_mxfp8.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

M_BENCH = 4096
H = 5120
HC = 4
PEAK_HBM_GBS = 8000.0
# algorithmic bytes per row (what the method must move at least once)
POST_BYTES_ROW = 2 * (HC * H + H + HC * H) + 4 * (HC + HC * HC)  # R + x in, R' out, post + comb
PRE_BYTES_ROW = 2 * (HC * H + H) + 4 * (HC + HC + HC * HC)  # R in, y out, pre/post/comb out
FN_BYTES = 24 * 4 * H * 4  # fn once per call (fp32 layout; the packed bf16 parts are 1.67x)
PRE_BYTES_CALL = FN_BYTES + 2 * H  # fn and the norm weight, once per call
STEP_BYTES = M_BENCH * (POST_BYTES_ROW + PRE_BYTES_ROW) + PRE_BYTES_CALL
# the dominant kernel of each path and the algorithmic bytes one launch moves
ROOFLINE_KERNEL = {
    "fused": ("stats_kernel<10,true> (hc_post_stats)", M_BENCH * POST_BYTES_ROW + FN_BYTES,
              ["hc_pipe.hip", "hc_device.h", "hc_launch.h"]),
    "unfused": ("post_kernel (hc_post)", M_BENCH * POST_BYTES_ROW,
                ["hc_post.hip", "hc_device.h", "hc_launch.h"]),
}


def kernel_source_hash(files) -> str:
    csrc = os.path.join(ROOT, "hyper_connection_residual_hc_amd", "csrc")
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel: str, files, M: int = M_BENCH):
    """HBM bytes per launch of `kernel` on M rows from a profiles/ summary line
    `traffic-record: kernel=<name> M=<M> source=<hash> bytes=<n>`, if its hash is current."""
    want = kernel_source_hash(files)
    pat = re.compile(r"traffic-record: kernel=(\S+) M=(\d+) source=(\w+) bytes=(\d+)")
    name = kernel.split()[0]
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as fh:
            for m in pat.finditer(fh.read()):
                if m.group(1) == name and int(m.group(2)) == M and m.group(3) == want:
                    return int(m.group(4))
    return None


def trace_regions(csv_path: str, steps: int, kernels) -> list:
    """Per-region average durations from a rocprofv3 kernel trace (`*_kernel_trace.csv`) of a
    bench run with --steps `steps`. For each kernel name in `kernels` (matched with spaces
    removed, e.g. "stats_kernel<10,true>"), its dispatches in start order end with the K
    back-to-back launches timed for the roofline (K = steps), preceded by the K launches of the
    timed step region; both averages are returned with the average over all its dispatches."""
    import csv
    out = []
    with open(csv_path, newline="") as fh:
        rows = list(csv.DictReader(fh))
    for name in kernels:
        d = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows
                   if name in r["Kernel_Name"].replace(" ", ""))
        us = [(e - b) / 1000.0 for b, e in d]
        rec = {"kernel": name, "dispatches": len(us),
               "all_avg_us": sum(us) / len(us) if us else None}
        if len(us) >= 2 * steps:
            rec["step_region_avg_us"] = sum(us[-2 * steps:-steps]) / steps
            rec["back_to_back_avg_us"] = sum(us[-steps:]) / steps
        out.append(rec)
    return out


def cpu_baseline(rows: int, target_s: float):
    """The oracle (as it stands) on `rows`-row samples of the same workload, repeated until
    about target_s seconds of CPU work; returns rows/s and the BLAS thread count."""
    import numpy as np

    from hyper_connection_residual_hc_amd import inputs
    from oracle import hc_oracle as o
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    fn_a, sc_a, ba_a = inputs.hc_params(inputs.SEED_ATTN)
    fn_f, sc_f, ba_f = inputs.hc_params(inputs.SEED_FFN)
    w_f = inputs.bits(inputs.norm_weight(inputs.SEED_NORM_FFN))
    R = inputs.bits(inputs.residual(rows, M_BENCH))
    x = inputs.bits(inputs.sublayer_out(rows, M_BENCH + 1))
    pre_a = o.hc_pre(R, fn_a.numpy(), sc_a.numpy(), ba_a.numpy(),
                     inputs.bits(inputs.norm_weight(inputs.SEED_NORM_ATTN)))
    post32 = pre_a["post"].astype(np.float32)
    comb32 = pre_a["comb"].astype(np.float32)
    done, t0 = 0, time.perf_counter()
    while True:
        _, R1 = o.hc_post(x, R, post32, comb32)
        o.hc_pre(R1, fn_f.numpy(), sc_f.numpy(), ba_f.numpy(), w_f)
        done += rows
        el = time.perf_counter() - t0
        if el >= target_s:
            break
    return done / el, threads, el, done


def ops_table(args, sets, fnp, sc, ba, w, torch, ops, inputs, d) -> int:
    """Every entry point alone on the bench's rotating M=4096 input sets: one JSON line each
    with the wall-clock time per call and the algorithmic bytes it moves."""
    M = M_BENCH
    dev = sets[0][0].device
    fh, sh, bh = map(d, inputs.hc_head_params(inputs.SEED_HEAD))
    fnp_h = ops.head_fn_pack(fh)
    extra = []
    for R, x, post, comb, o in sets:
        mixes = torch.empty(M, 24, device=dev)
        ops.pre_stats(R, fnp, mixes=mixes, want_sumsq=False, workspace=o["ws"])
        pre = torch.empty(M, HC, device=dev)
        y = torch.empty(M, H, dtype=torch.bfloat16, device=dev)
        ops.combine_norm(R, post, w, out=y)
        extra.append(dict(mixes=mixes, pre=pre, y=y,
                          q=torch.empty(M, H, dtype=torch.uint8, device=dev),
                          s=torch.empty(M, H // 32, dtype=torch.uint8, device=dev),
                          sw=torch.empty(M * H // 32, dtype=torch.uint8, device=dev)))
    torch.cuda.synchronize()
    coef_o = 4 * (HC + HC + HC * HC)  # pre, post, comb written
    table = {
        "hc_post": (lambda k, s, e: ops.post(s[1], s[0], s[2], s[3], out=s[4]["R1"]),
                    M * POST_BYTES_ROW),
        "hc_pre_stats": (lambda k, s, e: ops.pre_stats(s[0], fnp, mixes=e["mixes"], want_sumsq=False,
                                                       workspace=s[4]["ws"]),
                         M * (2 * HC * H + 4 * 24) + FN_BYTES),
        "hc_sinkhorn": (lambda k, s, e: ops.sinkhorn(e["mixes"], sc, ba,
                                                     out=(e["pre"], s[4]["post"], s[4]["comb"])),
                        M * (4 * 24 + coef_o)),
        "hc_combine_norm": (lambda k, s, e: ops.combine_norm(s[0], s[2], w, out=s[4]["y"]),
                            M * (2 * HC * H + 4 * HC + 2 * H) + 2 * H),
        "hc_pre": (lambda k, s, e: ops.pre(s[0], fnp, sc, ba, w,
                                           out=(s[4]["y"], s[4]["post"], s[4]["comb"], None),
                                           workspace=s[4]["ws"]),
                   M * PRE_BYTES_ROW + PRE_BYTES_CALL),
        "hc_post_pre": (lambda k, s, e: ops.post_pre(s[1], s[0], s[2], s[3], fnp, sc, ba, w,
                                                     out=(s[4]["R1"], s[4]["y"], s[4]["post"],
                                                          s[4]["comb"], None),
                                                     workspace=s[4]["ws"]),
                        M * (POST_BYTES_ROW + 2 * H + 4 * (HC + HC * HC)) + PRE_BYTES_CALL),
        "hc_pre_mxfp8 (no bf16 y)": (lambda k, s, e: ops.pre_mxfp8(
            s[0], fnp, sc, ba, w, out=(None, e["q"], e["s"], s[4]["post"], s[4]["comb"], None),
            workspace=s[4]["ws"]), M * (2 * HC * H + H + H // 32 + 4 * (HC + HC * HC)) + PRE_BYTES_CALL),
        "mxfp8_quant_rows": (lambda k, s, e: ops.mxfp8_quant_rows(e["y"], q=e["q"], scales=e["s"]),
                             M * (2 * H + H + H // 32)),
        "mxfp8_swizzle_128x4": (lambda k, s, e: ops.mxfp8_swizzle_128x4(e["s"], out=e["sw"]),
                                M * 2 * (H // 32)),
        "hc_head": (lambda k, s, e: ops.head(s[0], fnp_h, sh, bh, out=e["y"], workspace=s[4]["ws"]),
                    M * (2 * HC * H + 2 * H) + 4 * HC * 4 * H),
    }
    for name, (fn_, nbytes) in table.items():
        for k in range(args.warmup):
            fn_(k, sets[k % len(sets)], extra[k % len(sets)])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            fn_(k, sets[k % len(sets)], extra[k % len(sets)])
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) * 1e6 / args.steps
        print(json.dumps({"op": name, "M": M, "H": H, "us_per_call_wall": us,
                          "algorithmic_bytes": nbytes,
                          "algorithmic_gbps_wall": nbytes / (us * 1e-6) / 1e9}), flush=True)
    return 0


def small_table(args, torch, ops, inputs, d) -> int:
    """Small batches (decode and verify steps run hc pre / post on a few rows, short prefill
    chunks on a few hundred): GPU time per call of hc_pre, hc_post_pre, hc_post and hc_head at
    M = 1 .. 1024, measured as a HIP graph of back-to-back calls replayed (so the host's launch
    cost is not in it), one JSON line per (entry point, M)."""
    dev = torch.device("cuda:0")
    fn_a, sc_a, ba_a = map(d, inputs.hc_params(inputs.SEED_ATTN))
    fn_f, sc_f, ba_f = map(d, inputs.hc_params(inputs.SEED_FFN))
    w_a = d(inputs.norm_weight(inputs.SEED_NORM_ATTN))
    w_f = d(inputs.norm_weight(inputs.SEED_NORM_FFN))
    fnp_a, fnp_f = ops.fn_pack(fn_a), ops.fn_pack(fn_f)
    fh, sh, bh = map(d, inputs.hc_head_params(inputs.SEED_HEAD))
    fnp_h = ops.head_fn_pack(fh)
    calls = 50

    def graph_us(fn_):
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            for _ in range(3):
                fn_()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for _ in range(calls):
                fn_()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(1, args.steps // 20)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * calls)

    for M in (1, 2, 4, 8, 16, 64, 256, 1024):
        R = d(inputs.residual(M, M))
        x = d(inputs.sublayer_out(M, M + 1))
        _, post, comb, _ = ops.pre(R, fnp_a, sc_a, ba_a, w_a)
        R1 = torch.empty_like(R)
        y = torch.empty(M, H, dtype=torch.bfloat16, device=dev)
        po, co = torch.empty(M, HC, device=dev), torch.empty(M, HC, HC, device=dev)
        ws = torch.empty(max(ops.pre_workspace_bytes(M, H), ops.post_pre_workspace_bytes(M, H)),
                         dtype=torch.uint8, device=dev)
        table = {
            "hc_pre": lambda: ops.pre(R, fnp_f, sc_f, ba_f, w_f, out=(y, po, co, None),
                                      workspace=ws),
            "hc_post_pre": lambda: ops.post_pre(x, R, post, comb, fnp_f, sc_f, ba_f, w_f,
                                                out=(R1, y, po, co, None), workspace=ws),
            "hc_post": lambda: ops.post(x, R, post, comb, out=R1),
            "hc_head": lambda: ops.head(R, fnp_h, sh, bh, out=y, workspace=ws),
        }
        for name, fn_ in table.items():
            print(json.dumps({"op": name, "M": M, "H": H, "us_per_call_graph": graph_us(fn_)}),
                  flush=True)
    return 0


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def back_to_back_ms(torch, fn_, k: int) -> float:
    """Average time per launch of fn_(i), i = 0 .. k-1, enqueued back to back on torch's
    current stream between one pair of HIP events recorded on that stream."""
    e0, e1 = _events(torch)
    torch.cuda.synchronize()
    e0.record()
    for i in range(k):
        fn_(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / k


def copy_ceiling_gbs(torch, dev) -> float:
    """A plain 1 GiB device copy (read + write bytes / time): the practical HBM ceiling."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ms = back_to_back_ms(torch, lambda i: dst.copy_(src), 10)
    del src, dst
    return 2 * (1 << 30) / (ms * 1e-3) / 1e9


# chained workloads other than the metric step, timed with --workload
CHAIN_WORKLOADS = {
    # M, rows per op of the chain (survey accounting: each op's algorithmic bytes), sets
    "config3": dict(M=1500, sets=6,
                    desc="mHC chain pre(attn) -> post -> pre(ffn), M=1500 rows, H=5120, "
                         "4 streams: hc_pre then hc_post_pre",
                    row_bytes=PRE_BYTES_ROW + POST_BYTES_ROW + PRE_BYTES_ROW,
                    call_bytes=2 * PRE_BYTES_CALL),
    "config4": dict(M=16384, sets=2,
                    desc="mHC prefill chunk post -> pre(ffn) -> row-local MXFP8 of y, M=16384 "
                         "rows, H=5120, 4 streams: hc_post_pre_mxfp8 (R', y bf16, y e4m3 + "
                         "ue8m0 scales per 32 columns)",
                    row_bytes=POST_BYTES_ROW + PRE_BYTES_ROW + (2 * H + H + H // 32),
                    call_bytes=PRE_BYTES_CALL),
}


def chain_workload(args, torch, ops, inputs, d) -> int:
    wl = CHAIN_WORKLOADS[args.workload]
    M = wl["M"]
    dev = torch.device("cuda:0")
    fn_a, sc_a, ba_a = map(d, inputs.hc_params(inputs.SEED_ATTN))
    fn_f, sc_f, ba_f = map(d, inputs.hc_params(inputs.SEED_FFN))
    w_a = d(inputs.norm_weight(inputs.SEED_NORM_ATTN))
    w_f = d(inputs.norm_weight(inputs.SEED_NORM_FFN))
    fnp_a, fnp_f = ops.fn_pack(fn_a), ops.fn_pack(fn_f)
    sets = []
    for k in range(wl["sets"]):
        R = d(inputs.residual(M, M + 1000 * k))
        x = d(inputs.sublayer_out(M, M + 1 + 1000 * k))
        o = dict(R1=torch.empty_like(R), y=torch.empty(M, H, dtype=torch.bfloat16, device=dev),
                 y1=torch.empty(M, H, dtype=torch.bfloat16, device=dev),
                 post=torch.empty(M, HC, device=dev), comb=torch.empty(M, HC, HC, device=dev),
                 post1=torch.empty(M, HC, device=dev), comb1=torch.empty(M, HC, HC, device=dev),
                 q=torch.empty(M, H, dtype=torch.uint8, device=dev),
                 s=torch.empty(M, H // 32, dtype=torch.uint8, device=dev),
                 ws=torch.empty(ops.post_pre_workspace_bytes(M, H), dtype=torch.uint8, device=dev))
        # config 4's post takes the attention site's coefficients from a setup pre
        ops.pre(R, fnp_a, sc_a, ba_a, w_a, out=(o["y1"], o["post1"], o["comb1"], None),
                workspace=o["ws"])
        sets.append((R, x, o))
    torch.cuda.synchronize()

    def step(k):
        R, x, o = sets[k % len(sets)]
        if args.workload == "config3":
            ops.pre(R, fnp_a, sc_a, ba_a, w_a, out=(o["y1"], o["post1"], o["comb1"], None),
                    workspace=o["ws"])
            ops.post_pre(x, R, o["post1"], o["comb1"], fnp_f, sc_f, ba_f, w_f,
                         out=(o["R1"], o["y"], o["post"], o["comb"], None), workspace=o["ws"])
        else:
            ops.post_pre_mxfp8(x, R, o["post1"], o["comb1"], fnp_f, sc_f, ba_f, w_f,
                               R_out=o["R1"],
                               out=(o["y"], o["q"], o["s"], o["post"], o["comb"], None),
                               workspace=o["ws"])

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    nbytes = M * wl["row_bytes"] + wl["call_bytes"]

    # the dominant kernel (stats_kernel<10, true>, the fused post + mix stats) back to back
    def post_stats(k):
        R, x, o = sets[k % len(sets)]
        ops.post_stats(x, R, o["post1"], o["comb1"], fnp_f, out=o["R1"], workspace=o["ws"])
    kms = back_to_back_ms(torch, post_stats, args.steps)
    kname, _, kfiles = ROOFLINE_KERNEL["fused"]
    kbytes = M * POST_BYTES_ROW + FN_BYTES
    gbs = nbytes / (ms * 1e-3) / 1e9
    traffic = recorded_traffic(kname, kfiles, M)
    print(json.dumps({
        "workload": args.workload, "M": M, "H": H, "steps": args.steps, "warmup": args.warmup,
        "desc": wl["desc"], "ms_per_step": ms, "rows_per_s": M / (ms * 1e-3),
        "algorithmic_bytes_step": nbytes, "algorithmic_gbps_step": gbs,
        "algorithmic_frac_step": gbs / PEAK_HBM_GBS,
        "ideal_us_at_peak": nbytes / (PEAK_HBM_GBS * 1e9) * 1e6,
        "roofline": {"kernel": kname, "bound": "hbm",
                     "ms": kms, "achieved": kbytes / (kms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": kbytes / (kms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "algorithmic_bytes": kbytes,
                     "traffic": traffic,
                     "traffic_gbps": traffic / (kms * 1e-3) / 1e9 if traffic else None,
                     "source": kernel_source_hash(kfiles)},
        "input_sets": len(sets),
    }), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=3, help="rotating independent input sets")
    ap.add_argument("--cpu-rows", type=int, default=256)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ops", action="store_true",
                    help="instead of the step: time every entry point alone at M=4096 and print "
                         "one JSON line per entry point (wall clock per call; run it under "
                         "rocprofv3 --kernel-trace for kernel durations)")
    ap.add_argument("--small", action="store_true",
                    help="instead of the step: GPU time per call of small batches "
                         "(M = 1 .. 1024) from HIP graph replays, one JSON line each")
    ap.add_argument("--workload", choices=["step", "config3", "config4"], default="step",
                    help="step: the metric (post + pre at M=4096); config3 / config4: the "
                         "M=1500 pre -> post -> pre chain or the M=16384 post -> pre -> MXFP8 "
                         "prefill chunk")
    ap.add_argument("--path", choices=["fused", "unfused"], default="fused",
                    help="fused: hc_post_pre (post with the next pre's mix stats in one pass, "
                         "then the pre finish); unfused: hc_post then hc_pre")
    ap.add_argument("--trace-regions", metavar="CSV",
                    help="no GPU work: read a rocprofv3 kernel trace of a bench run made with the "
                         "same --steps / --path / --workload and print, per kernel of the step, "
                         "its average duration in the timed step region and in the back-to-back "
                         "region the roofline is taken from")
    args = ap.parse_args()
    if args.trace_regions:
        if args.workload != "step":  # the chains time only their dominant kernel back to back
            names = ["stats_kernel<10,true>"]
        elif args.path == "fused":
            names = ["stats_kernel<10,true>", "pre_finish_kernel<10,"]
        else:
            names = ["post_kernel", "stats_kernel<10,false>", "pre_finish_kernel<10,"]
        for rec in trace_regions(args.trace_regions, args.steps, names):
            print(json.dumps(rec))
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the mHC path is row-local and the library has no "
              "multi-GPU leg (rows would shard across GPUs with no exchange inside the path).",
              file=sys.stderr)
        return 2

    import torch

    from hyper_connection_residual_hc_amd import _lib, inputs, ops

    if not os.path.exists(_lib.LIB_PATH):
        from hyper_connection_residual_hc_amd import build
        build.build()
    dev = torch.device("cuda:0")
    d = lambda t: t.to(dev).contiguous()  # noqa: E731
    if args.small:
        return small_table(args, torch, ops, inputs, d)
    if args.workload != "step":
        return chain_workload(args, torch, ops, inputs, d)

    fn_a, sc_a, ba_a = map(d, inputs.hc_params(inputs.SEED_ATTN))
    fn_f, sc_f, ba_f = map(d, inputs.hc_params(inputs.SEED_FFN))
    w_a = d(inputs.norm_weight(inputs.SEED_NORM_ATTN))
    w_f = d(inputs.norm_weight(inputs.SEED_NORM_FFN))
    fnp_a, fnp_f = ops.fn_pack(fn_a), ops.fn_pack(fn_f)

    M = M_BENCH
    sets = []
    for k in range(args.sets):
        R = d(inputs.residual(M, M + 1000 * k))
        x = d(inputs.sublayer_out(M, M + 1 + 1000 * k))
        _, post, comb, _ = ops.pre(R, fnp_a, sc_a, ba_a, w_a)  # setup: attention-site pre
        outs = dict(R1=torch.empty_like(R), y=torch.empty(M, H, dtype=torch.bfloat16, device=dev),
                    post=torch.empty(M, HC, device=dev), comb=torch.empty(M, HC, HC, device=dev),
                    ws=torch.empty(ops.pre_workspace_bytes(M, H), dtype=torch.uint8, device=dev))
        sets.append((R, x, post, comb, outs))
    torch.cuda.synchronize()
    if args.ops:
        return ops_table(args, sets, fnp_f, sc_f, ba_f, w_f, torch, ops, inputs, d)

    def step(k):
        """One step as the product runs it: no events inside."""
        R, x, post, comb, o = sets[k % len(sets)]
        if args.path == "fused":
            ops.post_pre(x, R, post, comb, fnp_f, sc_f, ba_f, w_f,
                         out=(o["R1"], o["y"], o["post"], o["comb"], None), workspace=o["ws"])
        else:
            ops.post(x, R, post, comb, out=o["R1"])
            ops.pre(o["R1"], fnp_f, sc_f, ba_f, w_f, out=(o["y"], o["post"], o["comb"], None),
                    workspace=o["ws"])

    def first_kernel(k):
        """The dominant kernel alone: hc_post_stats (stats_kernel<10, true>) or hc_post."""
        R, x, post, comb, o = sets[k % len(sets)]
        if args.path == "fused":
            ops.post_stats(x, R, post, comb, fnp_f, out=o["R1"], workspace=o["ws"])
        else:
            ops.post(x, R, post, comb, out=o["R1"])

    def second_part(k):
        """The rest of the step alone, on the R' the first kernel left in the same set."""
        R, x, post, comb, o = sets[k % len(sets)]
        if args.path == "fused":
            ops.pre_finish(o["R1"], o["ws"], sc_f, ba_f, w_f,
                           out=(o["y"], o["post"], o["comb"], None))
        else:
            ops.pre(o["R1"], fnp_f, sc_f, ba_f, w_f, out=(o["y"], o["post"], o["comb"], None),
                    workspace=o["ws"])

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    # the metric's timed region: exactly K steps, synchronised on both sides
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps

    # the dominant kernel's region: K launches back to back between one event pair; then the
    # second part of the step the same way (each set's R' and workspace are from its step)
    first_ms = back_to_back_ms(torch, first_kernel, args.steps)
    second_ms = back_to_back_ms(torch, second_part, args.steps)
    copy_gbs = copy_ceiling_gbs(torch, dev)

    kname, kbytes, kfiles = ROOFLINE_KERNEL[args.path]
    k_gbs = kbytes / (first_ms * 1e-3) / 1e9
    if args.path == "fused":
        kernels_ms = {"hc_post_stats (stats_kernel<10,true>)": first_ms,
                      "hc_pre_finish (pre_finish_kernel)": second_ms}
    else:
        kernels_ms = {"hc_post (post_kernel)": first_ms,
                      "hc_pre (stats_kernel<10,false> + pre_finish_kernel)": second_ms}
    rows_s = M / (ms_step * 1e-3)
    step_gbs = STEP_BYTES / (ms_step * 1e-3) / 1e9
    traffic = recorded_traffic(kname, kfiles)
    result = {
        "metric": "mHC pre+post rows/s and achieved HBM GB/s at M=4096, H=5120 (1 MI355X)",
        "value": rows_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded, distributions of the one-GPU test page)",
        "config": {
            "workload": "mHC hc_post (attention site) then hc_pre (FFN site), M=4096 rows, "
                        "H=5120, 4 streams, 20 Sinkhorn rounds, fused combine+RMSNorm",
            "M": M, "H": H, "hc": HC, "io_dtype": "bf16", "input_sets": args.sets,
            "parallelism": "none (1 GPU)",
        },
        # the step's algorithmic bytes (each op's own inputs and outputs, R' counted as written
        # by the post and read by the pre) over its wall-clock time; part of the R' read may be
        # served by the Infinity Cache, so this is not an HBM-only figure
        "algorithmic_gbps_step": step_gbs,
        "algorithmic_frac_step": step_gbs / PEAK_HBM_GBS,
        "algorithmic_bytes_step": STEP_BYTES,
        "copy_ceiling_gbps": copy_gbs,
        "path": args.path,
        "kernels_ms_back_to_back": kernels_ms,
        "roofline": {
            "kernel": kname,
            "bound": "hbm",
            "achieved": k_gbs,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": k_gbs / PEAK_HBM_GBS,
            "algorithmic_bytes": kbytes,
            "traffic": traffic,
            # the counted HBM bytes over the same back-to-back duration (null with traffic)
            "traffic_gbps": traffic / (first_ms * 1e-3) / 1e9 if traffic else None,
            "source": kernel_source_hash(kfiles),
        },
    }
    if not args.no_cpu_baseline:
        v, cores, el, done = cpu_baseline(args.cpu_rows, args.cpu_seconds)
        result["cpu_baseline"] = {
            "value": v, "unit": "rows/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} rows ({args.cpu_rows}-row batches of the same post+pre workload, "
                      f"{el:.1f} s, numpy float64)",
        }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
