"""GPU parity of lse_reduce_axis and log_softmax_axis (middle axis of an
(outer, R, inner) array) through the C ABI against the fp64 oracle."""
import numpy as np
import pytest
import torch

import log_softmax_reductions_amd as L
from log_softmax_reductions_amd import inputs
from tests.parity import compare

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("outer,R,inner", [(1, 4, 320), (3, 5, 7), (2, 64, 36), (4, 1, 9),
                                           (5, 33, 1), (7, 32, 1000), (2, 70, 65), (128, 64, 100),
                                           (3, 17, 4097), (1, 100, 8),
                                           # plane-split paths: ragged last slice, resident
                                           # up to 16 slices of 16 planes, streamed beyond
                                           (1, 33, 256), (1, 40, 4), (2, 200, 128),
                                           (8, 128, 4096), (1, 257, 64), (3, 1024, 32),
                                           (1, 2048, 8192)])
def test_lse_and_log_softmax_axis(orc, outer, R, inner):
    x = inputs.normal((outer, R, inner), seed=outer * 7919 + R * 31 + inner, sigma=3.0,
                      device=DEV)
    out = L.lse_reduce_axis(x, 1)
    y = L.log_softmax_axis(x, 1)
    torch.cuda.synchronize()
    xc = x.cpu().numpy()
    compare(out.cpu().numpy(), orc.lse_axis(xc), what=f"lse_axis {outer}x{R}x{inner}")
    compare(y.cpu().numpy(), orc.log_softmax_axis(xc), what=f"lsm_axis {outer}x{R}x{inner}")


def test_axis_dims_of_a_4d_tensor(orc):
    """The binding's dim argument: reducing each dim of an (N, C, H, W) tensor."""
    x = inputs.normal((3, 6, 5, 8), seed=11, device=DEV)
    xc = x.cpu().numpy()
    for d in range(4):
        got = L.lse_reduce_axis(x, d).cpu().numpy()
        outer = int(np.prod(xc.shape[:d])) if d else 1
        ref = orc.lse_axis(xc.reshape(outer, xc.shape[d], -1)).reshape(got.shape)
        compare(got, ref, what=f"dim {d}")


def test_axis_misaligned_and_special(orc):
    buf = inputs.normal((2 * 9 * 33 + 1,), seed=5, device=DEV)
    x = buf[1:].view(2, 9, 33).clone()
    x[0, :, 0] = -float("inf")
    x[1, 3, 5] = float("inf")
    x[1, 4, 6] = float("nan")
    xm = torch.empty(x.numel() + 1, device=DEV)[1:].view_as(x)   # misaligned copy
    xm.copy_(x)
    for t in (x, xm):
        compare(L.lse_reduce_axis(t, 1).cpu().numpy(), orc.lse_axis(x.cpu().numpy()),
                what="lse special")
        compare(L.log_softmax_axis(t, 1).cpu().numpy(), orc.log_softmax_axis(x.cpu().numpy()),
                what="lsm special")


def test_chain_layout_channel_lse(orc):
    """The chain's channel reduction layout: (128, 64, 126*126), sampled outer
    slices against the oracle, every output against torch-free properties."""
    x = inputs.normal((128, 64, 126 * 126), seed=12, device=DEV)
    out = L.lse_reduce_axis(x, 1)
    y = L.log_softmax_axis(x, 1)
    torch.cuda.synchronize()
    for o in (0, 77, 127):
        xs = x[o:o + 1].cpu().numpy()
        compare(out[o:o + 1].cpu().numpy(), orc.lse_axis(xs), what=f"chain layout lse {o}")
        compare(y[o:o + 1].cpu().numpy(), orc.log_softmax_axis(xs), what=f"chain layout lsm {o}")
    assert (torch.logsumexp(y.double(), dim=1).abs() < 1e-5).all()


@pytest.mark.parametrize("R", [40, 96, 300])
def test_axis_split_special_values(orc, R):
    """Non-finite values confined to one wave's slice of planes: a slice that
    counts nothing (all -inf) must drop out of the merge, a +inf in one slice
    must win over finite slices, NaN must poison only its own output."""
    x = inputs.normal((2, R, 64), seed=R, sigma=4.0, device=DEV)
    x[0, :, 0] = -float("inf")                 # every plane: LSE -inf, log_softmax NaN
    x[0, : R // 4, 1] = -float("inf")          # the first slice(s) empty
    x[0, R // 2:, 2] = -float("inf")           # the last slices empty
    x[1, R - 1, 3] = float("inf")              # +inf in the last slice only
    x[1, 0, 4] = float("inf")
    x[1, R // 2, 4] = float("inf")             # two +inf in different slices
    x[1, R // 3, 5] = float("nan")
    x[0, :, 6] = 80.0                          # equal values: v + log R
    x[0, 1, 7] = -80.0
    xc = x.cpu().numpy()
    compare(L.lse_reduce_axis(x, 1).cpu().numpy(), orc.lse_axis(xc), what=f"split lse R={R}")
    compare(L.log_softmax_axis(x, 1).cpu().numpy(), orc.log_softmax_axis(xc),
            what=f"split lsm R={R}")
    xm = torch.empty(x.numel() + 1, device=DEV)[1:].view_as(x)   # misaligned: scalar path
    xm.copy_(x)
    compare(L.log_softmax_axis(xm, 1).cpu().numpy(), orc.log_softmax_axis(xc),
            what=f"misaligned lsm R={R}")


@pytest.mark.parametrize("outer,R,inner,offset", [
    (1, 9, 4 * 64 * 29 + 4, 0),    # misaligned planes: 30 = 8 x 3 + 6 one-wave workgroups
    (1, 20, 4 * 64 * 5 + 4, 0),    # 6 workgroups, fewer than 8: plain order
    (3, 40, 4 * 64 * 16 + 12, 0),  # plane split (R >= 33), misaligned planes
    (2, 9, 4 * 64 * 19, 4),        # aligned stride, x 16 B past a cache line: 38 workgroups
])
def test_xcd_order_covers_every_output_once(orc, outer, R, inner, offset):
    """Misaligned planes or base: workgroups take their output runs in the
    XCD-grouped order, whose last grid % 8 workgroups keep their own index;
    every output must still be written exactly once."""
    buf = inputs.normal((outer * R * inner + offset,), seed=inner + offset, sigma=3.0, device=DEV)
    x = buf[offset:].view(outer, R, inner)
    out = torch.full((outer, inner), float("nan"), device=DEV)
    y = torch.full((outer, R, inner), float("nan"), device=DEV)
    L.lse_reduce_axis(x, 1, out)
    L.log_softmax_axis(x, 1, y)
    torch.cuda.synchronize()
    xc = x.cpu().numpy()
    compare(out.cpu().numpy(), orc.lse_axis(xc), what=f"lse_axis {outer}x{R}x{inner}+{offset}")
    compare(y.cpu().numpy(), orc.log_softmax_axis(xc),
            what=f"lsm_axis {outer}x{R}x{inner}+{offset}")


@pytest.mark.parametrize("rows,cols,pad", [(3, 1024, 0), (5, 5000, 0), (2, 16384, 0),
                                           (3, 16388, 0), (2, 100000, 0), (1, 393216, 0),
                                           (4, 1027, 0), (6, 3000, 5), (3, 40000, 4),
                                           # streamed rows with scalar loads
                                           (2, 20001, 0), (2, 30000, 3)])
def test_last_axis_as_rows(orc, rows, cols, pad):
    """Reducing a contiguous last axis of 1024 values or more runs one
    workgroup per row (register tile up to 16384 columns, streamed beyond);
    rows may be `pad` floats apart (a column slice)."""
    big = inputs.normal((rows, cols + pad), seed=rows * 131 + cols, sigma=3.0, device=DEV)
    x = big[:, :cols]
    xc = x.contiguous().cpu().numpy().reshape(rows, cols, 1)
    out = L.lse_reduce_axis(x, 1)
    y = L.log_softmax_axis(x, 1)
    torch.cuda.synchronize()
    compare(out.cpu().numpy(), orc.lse_axis(xc).reshape(rows), what=f"lse last axis {rows}x{cols}")
    compare(y.cpu().numpy(), orc.log_softmax_axis(xc).reshape(rows, cols),
            what=f"lsm last axis {rows}x{cols}")
    # the same values through the row entry point: log_softmax identical bit for bit
    # on the register-tile path
    if cols <= 16384:
        assert torch.equal(L.log_softmax_rows(x), y)


def test_last_axis_special_values(orc):
    x = inputs.normal((6, 20000), seed=77, sigma=2.0, device=DEV)
    x[0, :] = -float("inf")
    x[1, 123] = float("inf")
    x[2, 4567] = float("nan")
    x[3, :] = -float("inf"); x[3, 19999] = 1.5
    x[4, 5] = float("inf"); x[4, 6] = float("nan")
    for xv in (x, x[:, :5000]):          # streamed rows, register-tile rows
        xc = xv.contiguous().cpu().numpy()
        out = L.lse_reduce_axis(xv, 1)
        y = L.log_softmax_axis(xv, 1)
        torch.cuda.synchronize()
        r = xc.shape
        compare(out.cpu().numpy(), orc.lse_axis(xc.reshape(*r, 1)).reshape(r[0]),
                what=f"lse last axis special {r}")
        compare(y.cpu().numpy(), orc.log_softmax_axis(xc.reshape(*r, 1)).reshape(r),
                what=f"lsm last axis special {r}")


@pytest.mark.parametrize("outer,R,inner", [(1, 2, (1 << 29) + 1000), (3, 3, 200_000_000)])
def test_axis_more_outputs_than_one_launch(orc, outer, R, inner):
    """More than 2^29 outputs run as several launches (over the inner run,
    or over outer blocks): sampled columns on both sides of each split
    against the oracle (logsumexp and log_softmax), and every column by
    property on a window across a split."""
    x = inputs.normal((outer, R, inner), seed=inner % 1009, device=DEV)
    out = L.lse_reduce_axis(x, 1)
    torch.cuda.synchronize()
    cols = [0, 1, (1 << 29) - 1, (1 << 29), inner - 1] if outer == 1 else [0, 5, inner - 1]
    cols = [c for c in cols if c < inner]
    xs = x[:, :, cols].cpu().numpy()
    compare(out[:, cols].cpu().numpy(), orc.lse_axis(xs), what="lse split")
    w = slice(max(0, min(inner, 1 << 29) - 100_000), min(inner, (1 << 29) + 100_000))
    ref = torch.logsumexp(x[:, :, w].double(), dim=1)
    assert (out[:, w].double() - ref).abs().max().item() < 1e-5 + 2e-6 * ref.abs().max().item()
    del out
    y = L.log_softmax_axis(x, 1)
    torch.cuda.synchronize()
    compare(y[:, :, cols].cpu().numpy(), orc.log_softmax_axis(xs), what="lsm split")
    assert torch.logsumexp(y[:, :, w].double(), dim=1).abs().max().item() < 1e-5


@pytest.mark.parametrize("outer,R,inner", [(2, 4, 1 << 28), (2, 20, 1 << 26)])
def test_axis_lane_offsets_beyond_32_bits(orc, outer, R, inner):
    """x and y larger than 4 GiB per launch (8 and 10.7 GB): the register-block
    kernels take 64-bit lane offsets instead of one 32-bit offset from a scalar
    plane pointer.  Sampled columns of both outer slices against the oracle,
    and a window at the far end of x by property."""
    x = inputs.normal((outer, R, inner), seed=29 + R, device=DEV)
    cols = [0, 3, 4, inner // 2 + 1, inner - 5, inner - 1]
    xs = x[:, :, cols].cpu().numpy()
    out = L.lse_reduce_axis(x, 1)
    torch.cuda.synchronize()
    compare(out[:, cols].cpu().numpy(), orc.lse_axis(xs), what="lse 64-bit offsets")
    w = slice(inner - 100_000, inner)
    ref = torch.logsumexp(x[:, :, w].double(), dim=1)
    assert (out[:, w].double() - ref).abs().max().item() < 1e-5 + 2e-6 * ref.abs().max().item()
    del out
    y = L.log_softmax_axis(x, 1)
    torch.cuda.synchronize()
    compare(y[:, :, cols].cpu().numpy(), orc.log_softmax_axis(xs), what="lsm 64-bit offsets")
    assert torch.logsumexp(y[:, :, w].double(), dim=1).abs().max().item() < 1e-5


@pytest.mark.parametrize("outer,R,inner,off", [(1, 3, 5, 1), (2, 8, 4, 1), (3, 16, 37, 2),
                                               (1, 20, 4099, 3), (2, 32, 1027, 1), (1, 32, 4096, 1),
                                               (2, 40, 258, 0), (1, 70, 513, 2), (4, 5, 7, 0),
                                               (1, 1, 9, 1), (3, 2, 3, 1), (1, 150, 66, 3)])
def test_axis_ragged_and_offset_runs(orc, outer, R, inner, off):
    """Layouts off the 16-byte grid (x and the output at a 4-byte phase, inner
    not a multiple of 4): 16-byte accesses at 4-byte alignment, the last lane
    of each run re-reading the run's last 4 columns and writing only its own.
    Every output against the oracle; the floats around the output untouched."""
    n = outer * R * inner
    buf = inputs.normal((n + 8,), seed=outer * 131 + R * 17 + inner + off, sigma=3.0, device=DEV)
    x = buf[off:off + n].view(outer, R, inner)
    xc = x.cpu().numpy()
    big = torch.full((outer * R * inner + 16,), 7.0, device=DEV)
    out = big[off:off + outer * inner].view(outer, inner)
    L.lse_reduce_axis(x, 1, out)
    torch.cuda.synchronize()
    compare(out.cpu().numpy(), orc.lse_axis(xc), what=f"lse ragged {outer}x{R}x{inner}+{off}")
    assert torch.all(big[:off] == 7.0) and torch.all(big[off + outer * inner:] == 7.0)
    big.fill_(7.0)
    y = big[off:off + n].view(outer, R, inner)
    L.log_softmax_axis(x, 1, y)
    torch.cuda.synchronize()
    compare(y.cpu().numpy(), orc.log_softmax_axis(xc), what=f"lsm ragged {outer}x{R}x{inner}+{off}")
    assert torch.all(big[:off] == 7.0) and torch.all(big[off + n:] == 7.0)


@pytest.mark.parametrize("outer,R,inner", [(1000, 1, 4), (1000, 2, 2), (777, 2, 4), (1001, 3, 4),
                                           (500, 6, 2), (300, 16, 4), (300, 100, 4), (257, 256, 4),
                                           (100, 512, 2), (60, 255, 4), (50, 511, 2),
                                           (300, 100, 8), (1000, 3, 8), (200, 64, 16),
                                           (100, 16, 64), (64, 1, 256), (50, 4, 256),
                                           (70, 33, 16),
                                           # wave-wide segments of up to 64 values per lane
                                           (40, 1000, 2), (30, 300, 8), (20, 1024, 4),
                                           (10, 17, 256)])
@pytest.mark.parametrize("layout", ["packed", "offset", "pitched"])
def test_axis_short_interleaved_blocks(orc, outer, R, inner, layout):
    """Blocks of R planes x 2, 4, ... 256 outputs, contiguous and at most 4096
    values: segments of lanes per block, each lane folding its 4-value vectors
    into the outputs they interleave (16-byte loads, at a 4-byte offset too;
    blocks at a padded pitch; special values in one block; outputs between
    guard values)."""
    pad = 4 if layout == "pitched" else 0
    off = 1 if layout == "offset" else 0
    blk = R * inner + pad
    buf = inputs.normal((outer * blk + off,), seed=outer + R * 7 + inner, sigma=3.0, device=DEV)
    x = buf[off:].view(outer, blk)[:, :R * inner].view(outer, R, inner)
    xs = x[min(5, outer - 1)]
    xs[:, 0] = -float("inf")                        # an all -inf output
    if R > 1:
        xs[R // 2, 1] = float("inf")
    xc = x.contiguous().cpu().numpy()
    obuf = torch.full((outer, inner + 3), 7.0, device=DEV)
    out = L.lse_reduce_axis(x, 1, out=obuf[:, :inner])
    ybuf = torch.full((outer * blk + off,), 7.0, device=DEV)
    yv = ybuf[off:].view(outer, blk)[:, :R * inner].view(outer, R, inner)
    y = L.log_softmax_axis(x, 1, y=yv)
    torch.cuda.synchronize()
    what = f"interleaved {layout} {outer}x{R}x{inner}"
    compare(out.cpu().numpy(), orc.lse_axis(xc), what="lse " + what)
    compare(y.cpu().numpy(), orc.log_softmax_axis(xc), what="lsm " + what)
    assert (obuf[:, inner:] == 7.0).all()
    if pad:
        assert (ybuf[off:].view(outer, blk)[:, R * inner:] == 7.0).all()


@pytest.mark.parametrize("outer,R,inner", [(1000, 16, 3), (300, 100, 5), (100, 50, 12),
                                           (77, 257, 6), (50, 300, 9), (1000, 1, 7), (200, 3, 11),
                                           (64, 200, 15), (500, 64, 3)])
@pytest.mark.parametrize("layout", ["packed", "offset", "pitched"])
def test_axis_blocks_with_odd_outputs(orc, outer, R, inner, layout):
    """Blocks of R planes x 3..15 outputs (not a power of two), which the
    axis kernels (or the column split) take: x at a 4-byte offset and blocks
    at a padded pitch too; special values in one block; guard values around
    the outputs."""
    pad = 3 if layout == "pitched" else 0
    off = 1 if layout == "offset" else 0
    blk = R * inner + pad
    buf = inputs.normal((outer * blk + off,), seed=outer + R * 5 + inner, sigma=3.0, device=DEV)
    x = buf[off:].view(outer, blk)[:, :R * inner].view(outer, R, inner)
    xs = x[min(3, outer - 1)]
    xs[:, 0] = -float("inf")
    xs[R // 2, inner - 1] = float("nan")
    if R > 1:
        xs[R - 1, 1] = float("inf")
    xc = x.contiguous().cpu().numpy()
    obuf = torch.full((outer, inner + 2), 7.0, device=DEV)
    out = L.lse_reduce_axis(x, 1, out=obuf[:, :inner])
    ybuf = torch.full((outer * blk + off,), 7.0, device=DEV)
    yv = ybuf[off:].view(outer, blk)[:, :R * inner].view(outer, R, inner)
    y = L.log_softmax_axis(x, 1, y=yv)
    torch.cuda.synchronize()
    what = f"odd outputs {layout} {outer}x{R}x{inner}"
    compare(out.cpu().numpy(), orc.lse_axis(xc), what="lse " + what)
    compare(y.cpu().numpy(), orc.log_softmax_axis(xc), what="lsm " + what)
    assert (obuf[:, inner:] == 7.0).all()
    if pad:
        assert (ybuf[off:].view(outer, blk)[:, R * inner:] == 7.0).all()
