#!/usr/bin/env python3
"""Benchmark of the log-sum-exp engine on one MI355X.

One step = one log_softmax_rows call over the 4096 x 393216 fp32 workload
(N(0,1), seed 4) with the input already resident in HBM.  W untimed warm-up
steps, then exactly K timed steps bracketed by torch.cuda.synchronize();
rank 0 prints ONE JSON line.

  value      algorithmic bytes (read x once + write y once = 8 B/element)
             divided by the wall time per step, in GB/s (1e9 B/s)
  roofline   the same algorithmic bytes over the average duration of one
             launch measured with HIP events on the launch stream, against
             MI355X's 8 TB/s HBM peak; `traffic` is the HBM bytes per launch
             read from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
             summary (null when the kernel sources changed since)
  cpu_baseline  the fp64 C oracle on a bounded sample of the same rows
  secondary  the other hot-path cases, each timed the same way: logsumexp
             over dim 0 of (32, 2048, 4096), the conv chain on
             (128, 8, 128, 128), and the two small cases

Flags: --gpus N (only 1 is supported: this build runs on one GPU),
--steps K, --warmup W, --no-cpu-baseline, --no-secondary,
--only {rows_large,axis0_large,axis0_walk,conv_chain,softmax_large,axis_chain_layout,copy,
        copy_tile,copy_stream,copy_tile_1_per_cu,rows_odd_cols,rows_offset_view,
        chain_600x520_recompute,chain_600x520_staged,rows_large_reread,short_rows_128,
        short_rows_99,few_outputs,channel_blocks,one_long_row}
to run just that kernel
(for profiler runs; prints timing only).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix, published
METRIC = "GB/s and % of HBM roofline for log_softmax 4096x393216 fp32 on 1 MI355X"
ROWS, COLS = 4096, 393216
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "log_softmax_rows_4096x393216_traffic.md")
PROFILE_STATS = os.path.join(ROOT, "profiles", "log_softmax_rows_4096x393216_kernel_stats.md")
BENCH_COPY_LIB = os.path.join(ROOT, "libbench_copy.so")
KERNEL_SOURCES = ["log_softmax_reductions_amd/csrc/lse_rows.hip",
                  "log_softmax_reductions_amd/csrc/lse_device.hpp",
                  "log_softmax_reductions_amd/csrc/lse_internal.hpp"]


def kernel_source_hash(files=KERNEL_SOURCES) -> str:
    """sha256 (16 hex digits) of the kernel sources with comments and blank
    space removed, so that only a change to the code retires a recorded
    counter summary."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)   # block comments
        text = re.sub(r"//[^\n]*", " ", text)                 # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_from_profile():
    """HBM bytes per launch from the committed counter summary, or None if the
    summary is missing or was taken on different kernel sources."""
    try:
        text = open(PROFILE_TRAFFIC).read()
    except OSError:
        return None
    m_hash = re.search(r"kernel source hash:\s*`?([0-9a-f]{16})", text)
    m_bytes = re.search(r"HBM bytes per launch \(scaled\):\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def profiled_kernel():
    """(name, avg ns) of the dominant kernel in the committed rocprofv3 summary
    of the workload (its first table row), or (None, None)."""
    try:
        text = open(PROFILE_STATS).read()
    except OSError:
        return None, None
    m = re.search(r"^\| `(?:void )?([^`]+)` \| \d+ \| (\d+) \|", text, flags=re.M)
    return (m.group(1), int(m.group(2))) if m else (None, None)


def timed_launches(fn, steps, warmup):
    """Run fn warmup times, then `steps` times with a HIP event pair around each
    launch on the current stream.  Returns (wall_ms_per_step, event_ms_list)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return wall, [a.elapsed_time(b) for a, b in evs]


def cpu_baseline(x_dev, target_s=10.0):
    """The fp64 oracle (as it stands) on whole rows of the workload, timed on
    the host's cores: blocks of 64 rows in order, starting over at row 0 when
    the workload is done, until about target_s of timed wall time (host copies
    of the rows are made once and are not timed)."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    oracle.load()
    block, host = 64, {}
    rows_done, secs, r = 0, 0.0, 0
    while secs < target_s and rows_done < 64 * ROWS:
        if r not in host:
            host[r] = x_dev[r:r + block].cpu().numpy()
        t0 = time.perf_counter()
        oracle.log_softmax_rows(host[r], want_y=True, nthreads=threads)
        secs += time.perf_counter() - t0
        rows_done += host[r].shape[0]
        r = (r + block) % ROWS
    del host
    nbytes = rows_done * COLS * 8
    # the same oracle on one core, over 16 rows
    xs = x_dev[:16].cpu().numpy()
    t0 = time.perf_counter()
    oracle.log_softmax_rows(xs, want_y=True, nthreads=1)
    one = 16 * COLS * 8 / (time.perf_counter() - t0) / 1e9
    return {"value": round(nbytes / secs / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{rows_done} rows ({rows_done / ROWS:.2f} passes over the {ROWS} rows "
                      f"x {COLS} cols of the same workload), fp64 log_softmax incl. the y "
                      f"write, {secs:.1f} s wall",
            "value_1core": round(one, 4), "cpu_model": cpu_model(),
            "per_config": oracle_per_config(x_dev, threads)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_per_config(x_rows, threads):
    """The same oracle on a bounded sample of each other configuration (about
    a second each), in the unit of that configuration's GPU figure."""
    import oracle
    from log_softmax_reductions_amd import inputs

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    res = {}
    x = inputs.make("axis0_large", "cuda")[:, :512].contiguous().cpu().numpy()   # (32, 512, 4096)
    sec = timed(lambda: oracle.lse_axis0(x.reshape(32, -1), nthreads=threads))
    res["axis0_large"] = {"value": round((x.size + x.size // 32) * 4 / sec / 1e9, 3),
                          "unit": "GB/s", "sample": "512 of 2048 rows of B, all 32 planes"}
    x = x_rows[:64].cpu().numpy()
    sec = timed(lambda: oracle.softmax_rows(x, nthreads=threads))
    res["softmax_large"] = {"value": round(x.size * 8 / sec / 1e9, 3), "unit": "GB/s",
                            "sample": "64 of 4096 rows"}
    x = inputs.normal((16, 64, 126 * 126), seed=12, device="cuda").cpu().numpy()
    sec = timed(lambda: oracle.log_softmax_axis(x, nthreads=threads))
    res["log_softmax_axis_chain_layout"] = {"value": round(x.size * 8 / sec / 1e9, 3),
                                            "unit": "GB/s", "sample": "16 of 128 outer slices"}
    xc, w, b, g, be = (t[:2] if i == 0 else t for i, t in
                       enumerate(inputs.make("conv_chain", "cuda")))
    cpu = [t.cpu().numpy() for t in (xc, w, b, g, be)]
    sec = timed(lambda: oracle.fused_chain(*cpu, 16, 1e-5, nthreads=threads))
    res["conv_chain"] = {"value": round(2 * 2 * 64 * 72 * 126 * 126 / sec / 1e12, 4),
                         "unit": "conv TFLOP/s", "sample": "2 of 128 samples"}
    return res


def bench_rows_large(steps, warmup):
    import torch
    import log_softmax_reductions_amd as L
    from log_softmax_reductions_amd import inputs
    x = inputs.make("rows_large", "cuda")
    y = torch.empty_like(x)
    ws = torch.empty(L.log_softmax_rows_workspace_bytes(ROWS, COLS), dtype=torch.uint8,
                     device="cuda")
    wall, ev = timed_launches(lambda: L.log_softmax_rows(x, y, ws), steps, warmup)
    return x, y, wall, ev


def copy_ceiling(x, y, steps=5, warmup=2):
    """GB/s of device copies of the same bytes (read x, write y): an achievable
    denominator beside the 8 TB/s peak.  Our own HIP copies (bench_copy.hip:
    "tile" = the log_softmax kernel's access pattern without the arithmetic,
    "tile_2_per_cu" / "tile_1_per_cu" = the same capped at 2 / 1 workgroups
    per CU by unused LDS (fewer requests in flight), "stream" = grid-stride
    non-temporal, "plain" = one float4 per work-item) and torch's copy_ (the
    runtime's blit kernel); the ceiling is the fastest of ours."""
    import ctypes
    import torch
    lib = ctypes.CDLL(BENCH_COPY_LIB)
    lib.bench_copy.restype = ctypes.c_int
    lib.bench_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                               ctypes.c_void_p]
    lib.bench_copy_capped.restype = ctypes.c_int
    lib.bench_copy_capped.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_int, ctypes.c_void_p]
    n = x.numel()
    out = {}
    for v, name in enumerate(("tile", "stream", "plain")):
        def run(v=v):
            st = torch.cuda.current_stream().cuda_stream
            assert lib.bench_copy(x.data_ptr(), y.data_ptr(), n, v, st) == 0
        _, ev = timed_launches(run, steps, warmup)
        out[name] = round(2 * n * 4 / (sum(ev) / len(ev) * 1e-3) / 1e9, 1)
    for lds, name in ((54 * 1024, "tile_2_per_cu"), (81 * 1024, "tile_1_per_cu")):
        def run_capped(lds=lds):
            st = torch.cuda.current_stream().cuda_stream
            assert lib.bench_copy_capped(x.data_ptr(), y.data_ptr(), n, lds, st) == 0
        _, ev = timed_launches(run_capped, steps, warmup)
        out[name] = round(2 * n * 4 / (sum(ev) / len(ev) * 1e-3) / 1e9, 1)
    _, ev = timed_launches(lambda: y.copy_(x), steps, warmup)
    out["torch_copy_"] = round(2 * n * 4 / (sum(ev) / len(ev) * 1e-3) / 1e9, 1)
    return max(v for k, v in out.items() if k != "torch_copy_"), out


SHORT_ROWS = 1 << 20
FEW_OUT_SHAPE = (1 << 20, 64)   # 64 outputs over 2^20 planes
CHANNEL_SHAPE = (1024, 2048, 49)  # channel reduction over 7 x 7 maps (contiguous blocks)
LONG_ROW = 100_000_000


def bench_secondary(steps=10, warmup=3):
    import torch
    import log_softmax_reductions_amd as L
    from log_softmax_reductions_amd import inputs
    out = {}
    # logsumexp over dim 0 of (32, 2048, 4096): 1 GiB read + 32 MiB written
    x = inputs.make("axis0_large", "cuda")
    o = torch.empty(x.shape[1:], device="cuda")
    wall, ev = timed_launches(lambda: L.lse_reduce_axis0(x, o), steps, warmup)
    nbytes = x.numel() * 4 + o.numel() * 4
    avg = sum(ev) / len(ev)
    out["axis0_large"] = {"workload": "logsumexp dim=0 (32,2048,4096) fp32 N(0,4)",
                          "ms": round(avg, 4), "GB/s": round(nbytes / avg / 1e6, 1),
                          "hbm_frac": round(nbytes / avg / 1e6 / HBM_PEAK_GBS, 4)}
    del x, o
    # many planes: logsumexp over dim 0 of (64, 4194304) takes the plane walk
    x = inputs.normal((64, 4194304), seed=13, sigma=2.0, device="cuda")
    o = torch.empty((4194304,), device="cuda")
    wall, ev = timed_launches(lambda: L.lse_reduce_axis0(x, o), steps, warmup)
    nbytes = x.numel() * 4 + o.numel() * 4
    avg = sum(ev) / len(ev)
    out["axis0_walk"] = {"workload": "logsumexp dim=0 (64,4194304) fp32 N(0,4)",
                         "ms": round(avg, 4), "GB/s": round(nbytes / avg / 1e6, 1),
                         "hbm_frac": round(nbytes / avg / 1e6 / HBM_PEAK_GBS, 4)}
    del x, o
    # conv chain (128, 8, 128, 128) -> (128, 1, 126, 126)
    x, w, b, g, be = inputs.make("conv_chain", "cuda")
    o = torch.empty((128, 1, 126, 126), device="cuda")
    ws = torch.empty(L.fused_conv_gn_act_lse_workspace_bytes(128, 8, 128, 128, 64, 3, 16),
                     dtype=torch.uint8, device="cuda")
    # A 0.2 ms kernel needs ~100 calls before the GPU's clocks have ramped up
    # (timed from a cold start its first few dozen calls read 5-10 % slower).
    chain_warmup = max(warmup, 100)
    wall, ev = timed_launches(lambda: L.fused_conv_gn_act_lse(x, w, b, g, be, 16, 1e-5, o, ws),
                              steps, chain_warmup)
    avg = sum(ev) / len(ev)
    flop = 2 * 128 * 64 * 8 * 9 * 126 * 126   # one direct conv, counted once
    # Winograd F(2x2, 3x3): 16 positions x 64 x 8 multiply-adds per 2x2 block;
    # 63 tile rows x 64 blocks per sample (the last block column is padding).
    mfma_flop = 2 * 16 * 64 * 8 * 63 * 64 * 128
    # the same chain on samples too large for the fused launch (8 x 600 x 520:
    # 748 tile pairs per sample): statistics launch + apply launch, the apply
    # recomputing the conv (the default) or reading it back from a staging
    # area sized for the Infinity Cache
    xl, wl, bl, gl, bel = inputs.conv_chain_inputs(N=8, H=600, W=520, seed=5, device="cuda")
    ol = torch.empty((8, 1, 598, 518), device="cuda")
    two = {}
    for path, name in ((2, "recompute"), (3, "staged")):
        L.lse_testing_set_chain_path(path)
        wsl = torch.empty(L.fused_conv_gn_act_lse_workspace_bytes(8, 8, 600, 520, 64, 3, 16),
                          dtype=torch.uint8, device="cuda")
        _, evl = timed_launches(
            lambda: L.fused_conv_gn_act_lse(xl, wl, bl, gl, bel, 16, 1e-5, ol, wsl), steps,
            max(warmup, 20))
        L.lse_testing_set_chain_path(0)
        two[name + "_ms"] = round(sum(evl) / len(evl), 4)
        del wsl
    out["conv_chain_8x600x520_two_launch"] = {
        "workload": "the chain on x (8,8,600,520): statistics + apply launches", **two}
    del xl, wl, bl, gl, bel, ol
    out["conv_chain"] = {"workload": "conv3x3 8->64, GN16, tanh, hardswish, +res, LSE dim=1, "
                                     "x (128,8,128,128)",
                         "ms": round(avg, 4), "warmup_calls": chain_warmup,
                         "conv_TFLOP/s": round(flop / avg / 1e9, 2),
                         "direct_conv_equiv_frac_of_fp32_mfma_peak":
                             round(flop / avg / 1e9 / FP32_MFMA_PEAK_TFLOPS, 4),
                         "executed_mfma_TFLOP/s": round(mfma_flop / avg / 1e9, 2),
                         "executed_mfma_frac_of_fp32_peak":
                             round(mfma_flop / avg / 1e9 / FP32_MFMA_PEAK_TFLOPS, 4),
                         "note": "one fused kernel: conv_TFLOP/s counts the direct conv's "
                                 "18.73 GFLOP; the kernel computes it as Winograd F(2x2,3x3) "
                                 "on fp32 MFMA (8.46 GFLOP executed); each sample's GroupNorm "
                                 "statistics are merged across workgroups"}
    del x, w, b, g, be, o, ws
    # widened rows: softmax on the same 4096 x 393216 workload, and the
    # middle-axis reductions on the chain's (N, C, H*W) = (128, 64, 15876) layout
    x = inputs.make("rows_large", "cuda")
    y = torch.empty_like(x)
    ws = torch.empty(L.log_softmax_rows_workspace_bytes(ROWS, COLS), dtype=torch.uint8,
                     device="cuda")
    wall, ev = timed_launches(lambda: L.softmax_rows(x, y, ws), steps, warmup)
    avg = sum(ev) / len(ev)
    out["softmax_large"] = {"workload": "softmax dim=1 (4096,393216) fp32 N(0,1)",
                            "ms": round(avg, 4), "GB/s": round(8 * x.numel() / avg / 1e6, 1),
                            "hbm_frac": round(8 * x.numel() / avg / 1e6 / HBM_PEAK_GBS, 4)}
    del x, y, ws
    x = inputs.normal((128, 64, 126 * 126), seed=12, device="cuda")
    o = torch.empty((128, 126 * 126), device="cuda")
    wall, ev = timed_launches(lambda: L.lse_reduce_axis(x, 1, o), steps, warmup)
    avg = sum(ev) / len(ev)
    nb = 4 * (x.numel() + o.numel())
    out["lse_axis_chain_layout"] = {"workload": "logsumexp dim=1 of (128,64,15876) fp32 N(0,1)",
                                    "ms": round(avg, 4), "GB/s": round(nb / avg / 1e6, 1),
                                    "hbm_frac": round(nb / avg / 1e6 / HBM_PEAK_GBS, 4)}
    y = torch.empty_like(x)
    wall, ev = timed_launches(lambda: L.log_softmax_axis(x, 1, y), steps, warmup)
    avg = sum(ev) / len(ev)
    nb = 8 * x.numel()
    out["log_softmax_axis_chain_layout"] = {
        "workload": "log_softmax dim=1 of (128,64,15876) fp32 N(0,1)",
        "ms": round(avg, 4), "GB/s": round(nb / avg / 1e6, 1),
        "hbm_frac": round(nb / avg / 1e6 / HBM_PEAK_GBS, 4)}
    del x, o, y
    # rows that the 16-byte path does not cover as a whole: an odd row length
    # (every row starts at a different alignment) and the workload viewed one
    # float past a 16-byte boundary (x misaligned, y aligned)
    for key, cols, off in (("rows_odd_cols", COLS - 1, 0), ("rows_offset_view", COLS, 1)):
        buf = inputs.normal((ROWS * cols + off,), seed=41, device="cuda")
        x = buf[off:].view(ROWS, cols)
        y = torch.empty((ROWS, cols), device="cuda")
        ws = torch.empty(L.log_softmax_rows_workspace_bytes(ROWS, cols), dtype=torch.uint8,
                         device="cuda")
        wall, ev = timed_launches(lambda: L.log_softmax_rows(x, y, ws), steps, warmup)
        avg = sum(ev) / len(ev)
        nb = 8 * x.numel()
        out[key] = {"workload": f"log_softmax dim=1 ({ROWS},{cols}) fp32 N(0,1), x at byte "
                                f"offset {4 * off} from a 256-byte boundary",
                    "ms": round(avg, 4), "GB/s": round(nb / avg / 1e6, 1),
                    "hbm_frac": round(nb / avg / 1e6 / HBM_PEAK_GBS, 4)}
        del buf, x, y, ws
    # the split rows re-reading each chunk for the write (through the caches)
    # instead of keeping it in registers: the comparison design
    x = inputs.make("rows_large", "cuda")
    y = torch.empty_like(x)
    ws = torch.empty(L.log_softmax_rows_workspace_bytes(ROWS, COLS), dtype=torch.uint8,
                     device="cuda")
    L.lse_testing_set_rows_reread(True)
    wall, ev = timed_launches(lambda: L.log_softmax_rows(x, y, ws), steps, warmup)
    L.lse_testing_set_rows_reread(False)
    avg = sum(ev) / len(ev)
    out["rows_large_reread"] = {
        "workload": "log_softmax (4096,393216) fp32, chunks re-read for the write (comparison)",
        "ms": round(avg, 4), "GB/s": round(8 * x.numel() / avg / 1e6, 1),
        "hbm_frac": round(8 * x.numel() / avg / 1e6 / HBM_PEAK_GBS, 4)}
    del x, y, ws
    # the allocation-free entry point on the workload (static device scratch)
    x = inputs.make("rows_large", "cuda")
    y = torch.empty_like(x)
    wall, ev = timed_launches(lambda: L.log_softmax_rows_noalloc(x, y), steps, warmup)
    avg = sum(ev) / len(ev)
    out["rows_large_noalloc"] = {"workload": "log_softmax_rows_noalloc (4096,393216) fp32 N(0,1)",
                                 "ms": round(avg, 4), "GB/s": round(8 * x.numel() / avg / 1e6, 1),
                                 "hbm_frac": round(8 * x.numel() / avg / 1e6 / HBM_PEAK_GBS, 4)}
    del x, y
    # short rows over the last dim (a segment of lanes per row, several rows per
    # wave): 128 columns (16-byte rows) and 99 columns (odd length: 4-byte loads)
    for cols in (128, 99):
        x = inputs.normal((SHORT_ROWS, cols), seed=17 + cols, sigma=2.0, device="cuda")
        o = torch.empty((SHORT_ROWS,), device="cuda")
        y = torch.empty_like(x)
        _, ev = timed_launches(lambda: L.lse_reduce_axis(x, 1, o), steps, warmup)
        lse_ms = sum(ev) / len(ev)
        _, ev = timed_launches(lambda: L.log_softmax_axis(x, 1, y), steps, warmup)
        lsm_ms = sum(ev) / len(ev)
        nb_lse, nb_lsm = 4 * (x.numel() + o.numel()), 8 * x.numel()
        out[f"short_rows_{cols}"] = {
            "workload": f"logsumexp and log_softmax dim=1 of ({SHORT_ROWS},{cols}) fp32 N(0,4)",
            "lse_ms": round(lse_ms, 4), "lse_GB/s": round(nb_lse / lse_ms / 1e6, 1),
            "lse_hbm_frac": round(nb_lse / lse_ms / 1e6 / HBM_PEAK_GBS, 4),
            "log_softmax_ms": round(lsm_ms, 4),
            "log_softmax_GB/s": round(nb_lsm / lsm_ms / 1e6, 1),
            "log_softmax_hbm_frac": round(nb_lsm / lsm_ms / 1e6 / HBM_PEAK_GBS, 4)}
        del x, o, y
    # few outputs over many planes (the column split, workspace from the
    # binding) and one very long row (split logsumexp / three-launch log_softmax)
    x = inputs.normal(FEW_OUT_SHAPE, seed=19, sigma=2.0, device="cuda")
    o = torch.empty(FEW_OUT_SHAPE[1:], device="cuda")
    y = torch.empty_like(x)
    _, ev = timed_launches(lambda: L.lse_reduce_axis0(x, o), steps, warmup)
    lse_ms = sum(ev) / len(ev)
    _, ev = timed_launches(lambda: L.log_softmax_axis(x, 0, y), steps, warmup)
    lsm_ms = sum(ev) / len(ev)
    nb_lse, nb_lsm = 4 * (x.numel() + o.numel()), 8 * x.numel()
    out["few_outputs"] = {
        "workload": f"logsumexp and log_softmax dim=0 of {FEW_OUT_SHAPE} fp32 N(0,4)",
        "lse_ms": round(lse_ms, 4), "lse_GB/s": round(nb_lse / lse_ms / 1e6, 1),
        "lse_hbm_frac": round(nb_lse / lse_ms / 1e6 / HBM_PEAK_GBS, 4),
        "log_softmax_ms": round(lsm_ms, 4), "log_softmax_GB/s": round(nb_lsm / lsm_ms / 1e6, 1),
        "log_softmax_hbm_frac": round(nb_lsm / lsm_ms / 1e6 / HBM_PEAK_GBS, 4),
        "note": "log_softmax reads x twice here (pairs, merge, write launches)"}
    del x, o, y
    # a channel reduction over small feature maps: contiguous (2048, 49) blocks
    # read as flat sweeps
    x = inputs.normal(CHANNEL_SHAPE, seed=29, sigma=2.0, device="cuda")
    o = torch.empty((CHANNEL_SHAPE[0], CHANNEL_SHAPE[2]), device="cuda")
    y = torch.empty_like(x)
    _, ev = timed_launches(lambda: L.lse_reduce_axis(x, 1, o), steps, warmup)
    lse_ms = sum(ev) / len(ev)
    _, ev = timed_launches(lambda: L.log_softmax_axis(x, 1, y), steps, warmup)
    lsm_ms = sum(ev) / len(ev)
    nb_lse, nb_lsm = 4 * (x.numel() + o.numel()), 8 * x.numel()
    out["channel_blocks"] = {
        "workload": f"logsumexp and log_softmax dim=1 of {CHANNEL_SHAPE} fp32 N(0,4)",
        "lse_ms": round(lse_ms, 4), "lse_GB/s": round(nb_lse / lse_ms / 1e6, 1),
        "lse_hbm_frac": round(nb_lse / lse_ms / 1e6 / HBM_PEAK_GBS, 4),
        "log_softmax_ms": round(lsm_ms, 4), "log_softmax_GB/s": round(nb_lsm / lsm_ms / 1e6, 1),
        "log_softmax_hbm_frac": round(nb_lsm / lsm_ms / 1e6 / HBM_PEAK_GBS, 4),
        "note": "log_softmax: 4 chunks per block held in registers, pairs exchanged through the workspace"}
    del x, o, y
    x = inputs.normal((1, LONG_ROW), seed=23, device="cuda")
    o = torch.empty((1,), device="cuda")
    y = torch.empty_like(x)
    _, ev = timed_launches(lambda: L.lse_reduce_axis(x, 1, o), steps, warmup)
    lse_ms = sum(ev) / len(ev)
    _, ev = timed_launches(lambda: L.log_softmax_rows(x, y), steps, warmup)
    lsm_ms = sum(ev) / len(ev)
    out["one_long_row"] = {
        "workload": f"logsumexp and log_softmax of one row of {LONG_ROW} fp32 N(0,1)",
        "lse_ms": round(lse_ms, 4), "lse_GB/s": round(4 * LONG_ROW / lse_ms / 1e6, 1),
        "log_softmax_ms": round(lsm_ms, 4),
        "log_softmax_GB/s": round(8 * LONG_ROW / lsm_ms / 1e6, 1),
        "log_softmax_hbm_frac": round(8 * LONG_ROW / lsm_ms / 1e6 / HBM_PEAK_GBS, 4),
        "note": "log_softmax reads x twice here (more chunks than can wait for each other)"}
    del x, o, y
    # small cases: hot latency per call, eagerly from Python (host launch
    # included) and as back-to-back calls replayed from a HIP graph
    x = inputs.make("rows_small", "cuda")
    y = torch.empty_like(x)
    wall, ev = timed_launches(lambda: L.log_softmax_rows(x, y), 50, 10)
    out["rows_small"] = {"workload": "log_softmax dim=1 (128,4096) with -inf/x50 entries",
                         "us": round(1e3 * sum(ev) / len(ev), 2),
                         "us_graph": graph_us_per_call(lambda: L.log_softmax_rows(x, y))}
    x = inputs.make("axis0_small", "cuda")
    o = torch.empty((10, 32), device="cuda")
    wall, ev = timed_launches(lambda: L.lse_reduce_axis0(x, o), 50, 10)
    out["axis0_small"] = {"workload": "logsumexp dim=0 (4,10,32)",
                          "us": round(1e3 * sum(ev) / len(ev), 2),
                          "us_graph": graph_us_per_call(lambda: L.lse_reduce_axis0(x, o))}
    return out


def graph_us_per_call(fn, calls=100, replays=10):
    """Per-call GPU time of `calls` back-to-back calls captured in one HIP graph."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return round(1e3 * a.elapsed_time(b) / (calls * replays), 2)


def run_only(which, steps, warmup):
    """Run one kernel alone (profiler runs) and print its event timing."""
    import torch
    import log_softmax_reductions_amd as L
    from log_softmax_reductions_amd import inputs
    if which == "rows_large":
        _, _, wall, ev = bench_rows_large(steps, warmup)
    elif which == "axis0_large":
        x = inputs.make("axis0_large", "cuda")
        o = torch.empty(x.shape[1:], device="cuda")
        wall, ev = timed_launches(lambda: L.lse_reduce_axis0(x, o), steps, warmup)
    elif which == "axis0_walk":
        x = inputs.normal((64, 4194304), seed=13, sigma=2.0, device="cuda")
        o = torch.empty((4194304,), device="cuda")
        wall, ev = timed_launches(lambda: L.lse_reduce_axis0(x, o), steps, warmup)
    elif which == "conv_chain":
        x, w, b, g, be = inputs.make("conv_chain", "cuda")
        o = torch.empty((128, 1, 126, 126), device="cuda")
        wall, ev = timed_launches(lambda: L.fused_conv_gn_act_lse(x, w, b, g, be, 16, 1e-5, o),
                                  steps, warmup)
    elif which in ("short_rows_128", "short_rows_99"):
        # logsumexp then log_softmax over the last dim of (2^20, cols)
        cols = int(which.rsplit("_", 1)[1])
        x = inputs.normal((SHORT_ROWS, cols), seed=17 + cols, sigma=2.0, device="cuda")
        o = torch.empty((SHORT_ROWS,), device="cuda")
        y = torch.empty_like(x)
        timed_launches(lambda: L.lse_reduce_axis(x, 1, o), steps, warmup)
        wall, ev = timed_launches(lambda: L.log_softmax_axis(x, 1, y), steps, warmup)
    elif which == "few_outputs":
        # logsumexp then log_softmax over dim 0 of (2^20, 64)
        x = inputs.normal(FEW_OUT_SHAPE, seed=19, sigma=2.0, device="cuda")
        o = torch.empty(FEW_OUT_SHAPE[1:], device="cuda")
        y = torch.empty_like(x)
        timed_launches(lambda: L.lse_reduce_axis0(x, o), steps, warmup)
        wall, ev = timed_launches(lambda: L.log_softmax_axis(x, 0, y), steps, warmup)
    elif which == "channel_blocks":
        # logsumexp then log_softmax over dim 1 of (1024, 2048, 49)
        x = inputs.normal(CHANNEL_SHAPE, seed=29, sigma=2.0, device="cuda")
        o = torch.empty((CHANNEL_SHAPE[0], CHANNEL_SHAPE[2]), device="cuda")
        y = torch.empty_like(x)
        timed_launches(lambda: L.lse_reduce_axis(x, 1, o), steps, warmup)
        wall, ev = timed_launches(lambda: L.log_softmax_axis(x, 1, y), steps, warmup)
    elif which == "one_long_row":
        x = inputs.normal((1, LONG_ROW), seed=23, device="cuda")
        o = torch.empty((1,), device="cuda")
        y = torch.empty_like(x)
        timed_launches(lambda: L.lse_reduce_axis(x, 1, o), steps, warmup)
        wall, ev = timed_launches(lambda: L.log_softmax_rows(x, y), steps, warmup)
    elif which in ("chain_600x520_recompute", "chain_600x520_staged"):
        # the two-launch chain on samples too large for one fused launch
        x, w, b, g, be = inputs.conv_chain_inputs(N=8, H=600, W=520, seed=5, device="cuda")
        o = torch.empty((8, 1, 598, 518), device="cuda")
        L.lse_testing_set_chain_path(2 if which.endswith("recompute") else 3)
        ws = torch.empty(L.fused_conv_gn_act_lse_workspace_bytes(8, 8, 600, 520, 64, 3, 16),
                         dtype=torch.uint8, device="cuda")
        wall, ev = timed_launches(lambda: L.fused_conv_gn_act_lse(x, w, b, g, be, 16, 1e-5, o, ws),
                                  steps, warmup)
        L.lse_testing_set_chain_path(0)
    elif which == "rows_large_reread":
        L.lse_testing_set_rows_reread(True)
        _, _, wall, ev = bench_rows_large(steps, warmup)
        L.lse_testing_set_rows_reread(False)
    elif which == "softmax_large":
        x = inputs.make("rows_large", "cuda")
        y = torch.empty_like(x)
        ws = torch.empty(L.log_softmax_rows_workspace_bytes(ROWS, COLS), dtype=torch.uint8,
                         device="cuda")
        wall, ev = timed_launches(lambda: L.softmax_rows(x, y, ws), steps, warmup)
    elif which == "axis_chain_layout":
        x = inputs.normal((128, 64, 126 * 126), seed=12, device="cuda")
        o = torch.empty((128, 126 * 126), device="cuda")
        y = torch.empty_like(x)
        wall, ev = timed_launches(lambda: (L.lse_reduce_axis(x, 1, o),
                                           L.log_softmax_axis(x, 1, y)), steps, warmup)
    elif which == "copy":
        # plain device copy of 1 GiB: calibrates the HBM byte counters
        a = torch.empty(1 << 28, device="cuda")
        c = torch.empty_like(a)
        wall, ev = timed_launches(lambda: c.copy_(a), steps, warmup)
    elif which in ("copy_tile", "copy_stream", "copy_tile_1_per_cu"):
        # our copy kernels on the workload's bytes (the copy ceiling)
        import ctypes
        lib = ctypes.CDLL(BENCH_COPY_LIB)
        lib.bench_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                   ctypes.c_int, ctypes.c_void_p]
        lib.bench_copy_capped.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                          ctypes.c_int, ctypes.c_void_p]
        a = inputs.make("rows_large", "cuda")
        c = torch.empty_like(a)
        st = torch.cuda.current_stream().cuda_stream
        if which == "copy_tile_1_per_cu":
            run = lambda: lib.bench_copy_capped(a.data_ptr(), c.data_ptr(), a.numel(), 81 * 1024, st)
        else:
            v = 0 if which == "copy_tile" else 1
            run = lambda: lib.bench_copy(a.data_ptr(), c.data_ptr(), a.numel(), v, st)
        wall, ev = timed_launches(run, steps, warmup)
    elif which in ("rows_odd_cols", "rows_offset_view"):
        cols, off = (COLS - 1, 0) if which == "rows_odd_cols" else (COLS, 1)
        buf = inputs.normal((ROWS * cols + off,), seed=41, device="cuda")
        x = buf[off:].view(ROWS, cols)
        y = torch.empty((ROWS, cols), device="cuda")
        wall, ev = timed_launches(lambda: L.log_softmax_rows(x, y), steps, warmup)
    else:
        raise SystemExit(f"unknown --only {which}")
    print(json.dumps({"only": which, "steps": steps, "wall_ms": round(wall, 4),
                      "event_ms_avg": round(sum(ev) / len(ev), 4),
                      "event_ms_min": round(min(ev), 4),
                      "event_ms_median": round(statistics.median(ev), 4)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--only", default=None)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.only:
        run_only(args.only, args.steps, args.warmup)
        return

    x, y, wall_ms, ev = bench_rows_large(args.steps, args.warmup)
    alg_bytes = 2 * 4 * ROWS * COLS
    value = alg_bytes / (wall_ms * 1e-3) / 1e9
    ev_avg = sum(ev) / len(ev)
    achieved = alg_bytes / (ev_avg * 1e-3) / 1e9
    kname, kns = profiled_kernel()
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "log_softmax dim=1, x (4096, 393216) fp32 i.i.d. N(0,1), seed 4",
                   "rows": ROWS, "cols": COLS, "elements_per_s": round(ROWS * COLS /
                                                                       (wall_ms * 1e-3), 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile(),
                     "kernel": kname, "kernel_avg_ns_rocprof": kns,
                     "event_ms_avg": round(ev_avg, 4), "event_ms_min": round(min(ev), 4),
                     "event_ms_median": round(statistics.median(ev), 4)},
    }
    copy_gbs, copies = copy_ceiling(x, y)
    line["roofline"]["copy_ceiling_GBs"] = copy_gbs
    line["roofline"]["copies_GBs"] = copies
    line["roofline"]["frac_of_copy"] = round(achieved / copy_gbs, 4)
    if not args.no_secondary:
        line["secondary"] = bench_secondary()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
