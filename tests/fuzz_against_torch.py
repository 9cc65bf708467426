"""Randomized sweep of the axis and row entry points against float64 torch on
the GPU (a supplementary check, not a parity test: parity is against the fp64
oracle in the test_gpu_* files).  Shapes, views (offsets, padded planes and
runs, row pitches), scales and special values are drawn at random; every call
goes through the Python binding (workspace entry points) and the axis calls
also through the entry points without a workspace; the fused conv chain is
checked against conv2d, group_norm, tanh and hardswish in float64 torch.

torch's log_softmax and softmax give NaN for every entry of a row or column
holding +inf; the oracle and the kernels give -inf (log_softmax) or 0
(softmax) for its finite entries and NaN for the +inf entry itself, so those
two outputs are not compared when +inf was planted.

    python tests/fuzz_against_torch.py [seed] [seconds]
"""
import math
import os
import sys
import time

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import log_softmax_reductions_amd as L  # noqa: E402
from log_softmax_reductions_amd import _lib  # noqa: E402
lib = _lib.load()
DEV = "cuda"
rng = np.random.default_rng(int(sys.argv[1]) if len(sys.argv) > 1 else 7)
budget_s = float(sys.argv[2]) if len(sys.argv) > 2 else 240
st = torch.cuda.current_stream().cuda_stream
def bad(got, ref, atol=1e-5, rtol=2e-6):
    got = got.double(); ref = ref.double()
    fin = torch.isfinite(ref)
    err = ((got - ref).abs() > atol + rtol * ref.abs()) & fin
    cls = (~fin) & ~((got == ref) | (torch.isnan(got) & torch.isnan(ref)))
    return int(err.sum() + cls.sum())
def logu(lo, hi): return int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))
t0 = time.time(); n_cases = 0; fails = []
while time.time() - t0 < budget_s:
    kind = rng.choice(["axis", "axis", "rows", "chain"])
    sigma = float(rng.choice([0.5, 2.0, 8.0]))
    if kind == "axis":
        inner = logu(1, 5000); R = logu(1, 200000)
        while inner * R > 6_000_000: R = max(1, R // 2)
        outer = logu(1, max(1, min(4000, 12_000_000 // (inner * R))))
        pad_in = int(rng.choice([0, 0, 0, 1, 3, 4])); pad_pl = int(rng.choice([0, 0, 1, 5])); off = int(rng.choice([0, 0, 1, 2, 3]))
        shape_big = (outer, R + pad_pl, inner + pad_in)
        nbig = outer * (R + pad_pl) * (inner + pad_in)
        buf = torch.randn(nbig + off, device=DEV) * sigma
        x = buf[off:].view(shape_big)[:, :R, :inner]
        pinf = False
        if rng.random() < 0.2 and x.numel():
            idx = tuple(int(rng.integers(0, s)) for s in x.shape)
            v = float(rng.choice([np.inf, -np.inf, np.nan])); x[idx] = v; pinf = v == np.inf
        ref_l = torch.logsumexp(x.double(), 1)
        ref_y = torch.log_softmax(x.double(), 1)
        got_l = L.lse_reduce_axis(x, 1); got_y = L.log_softmax_axis(x, 1)
        torch.cuda.synchronize()
        nb = bad(got_l, ref_l) + (0 if pinf else bad(got_y, ref_y))
        # no-workspace entry points on a contiguous copy
        xd = x.contiguous(); o2 = torch.empty((outer, inner), device=DEV); y2 = torch.empty_like(xd)
        _lib.check(lib.lse_reduce_axis(xd.data_ptr(), o2.data_ptr(), outer, R, inner, st), "lse")
        _lib.check(lib.log_softmax_axis(xd.data_ptr(), y2.data_ptr(), outer, R, inner, st), "lsm")
        torch.cuda.synchronize()
        nb += bad(o2, ref_l) + (0 if pinf else bad(y2, ref_y))
        tag = f"axis {outer}x{R}x{inner} pad {pad_pl},{pad_in} off {off} sigma {sigma}"
        del buf, x, xd, o2, y2, got_l, got_y, ref_l, ref_y
    elif kind == "chain":
        # conv 3x3 (8 -> 64) -> GroupNorm -> tanh -> hardswish -> + conv -> logsumexp over
        # channels, against the same steps in float64 torch; 5e-4 relative, as the chain's tests
        N = int(rng.integers(1, 5)); H = logu(3, 200); W = logu(3, 200)
        groups = int(rng.choice([1, 2, 4, 8, 16]))
        x = torch.randn(N, 8, H, W, device=DEV) * sigma
        w = (torch.rand(64, 8, 3, 3, device=DEV) * 2 - 1) / math.sqrt(72)
        b = (torch.rand(64, device=DEV) * 2 - 1) / math.sqrt(72)
        g = 1 + (torch.rand(64, device=DEV) - 0.5) if rng.random() < 0.5 else torch.ones(64, device=DEV)
        be = (torch.rand(64, device=DEV) - 0.5) if rng.random() < 0.5 else torch.zeros(64, device=DEV)
        got = L.fused_conv_gn_act_lse(x, w, b, g, be, groups, 1e-5)
        c = torch.nn.functional.conv2d(x.double(), w.double(), b.double())
        gn = torch.nn.functional.group_norm(c, groups, g.double(), be.double(), 1e-5)
        u = c + torch.nn.functional.hardswish(torch.tanh(gn))
        ref = torch.logsumexp(u, 1, keepdim=True)
        torch.cuda.synchronize()
        nb = bad(got, ref, atol=0.0, rtol=5e-4)
        tag = f"chain N={N} H={H} W={W} groups={groups} sigma {sigma}"
        del x, w, b, g, be, got, c, gn, u, ref
    else:
        cols = logu(1, 3_000_000); rows = logu(1, max(1, min(5000, 20_000_000 // cols)))
        pitch = cols + int(rng.choice([0, 0, 1, 4, 33])); off = int(rng.choice([0, 0, 1, 3]))
        buf = torch.randn(rows * pitch + off, device=DEV) * sigma
        x = buf[off:off + rows * pitch].view(rows, pitch)[:, :cols]
        pinf = False
        if rng.random() < 0.2:
            v = float(rng.choice([np.inf, -np.inf, np.nan]))
            x[int(rng.integers(0, rows)), int(rng.integers(0, cols))] = v; pinf = v == np.inf
        ref_y = torch.log_softmax(x.double(), 1); ref_s = torch.softmax(x.double(), 1); ref_l = torch.logsumexp(x.double(), 1)
        y = L.log_softmax_rows(x); s = L.softmax_rows(x); l = L.lse_reduce_axis(x, 1)
        torch.cuda.synchronize()
        nb = bad(l, ref_l) + (0 if pinf else bad(y, ref_y) + bad(s, ref_s, atol=1e-37, rtol=1e-5))
        tag = f"rows {rows}x{cols} pitch {pitch} off {off} sigma {sigma}"
        del buf, x, y, s, l, ref_y, ref_s, ref_l
    n_cases += 1
    if nb:
        fails.append(tag); print("FAIL", tag, nb, flush=True)
    if n_cases % 50 == 0:
        print(f"{n_cases} cases, {len(fails)} failures, {time.time() - t0:.0f} s", flush=True)
        torch.cuda.empty_cache()
print(f"done: {n_cases} cases, {len(fails)} failures", flush=True)
