"""GPU parity of the axis reductions with few outputs over many planes (the
column split with a workspace, and one workgroup per tile without one), and of
long last-axis rows with a workspace (split logsumexp rows, log_softmax rows of
more chunks than can wait for each other), against the fp64 oracle."""

import numpy as np
import pytest
import torch

import log_softmax_reductions_amd as L
from log_softmax_reductions_amd import _lib, inputs
from tests.parity import compare

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _raw_axis(x, R, inner, lsm):
    """The entry points without a workspace on a contiguous (outer, R, inner) x."""
    lib = _lib.load()
    outer = x.numel() // (R * inner)
    out = torch.empty((outer, R, inner) if lsm else (outer, inner), device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    fn = lib.log_softmax_axis if lsm else lib.lse_reduce_axis
    _lib.check(fn(x.data_ptr(), out.data_ptr(), outer, R, inner, st), "raw axis")
    return out


# (outer, R, inner): 1 to 64 lanes per plane, 16-byte and scalar lanes, ragged
# tiles and chunks, several outer blocks, the plane-count threshold
COLS_SHAPES = [(1, 200000, 4), (1, 100003, 7), (1, 50000, 16), (2, 30011, 33), (1, 20000, 100),
               (1, 10000, 256), (1, 3001, 1000), (3, 2000, 4096), (1, 60000, 2), (4, 9000, 3),
               (1, 64, 64), (1, 63, 64), (5, 777, 40), (1, 131072, 1),
               # many outer blocks of narrow runs
               (300, 500, 16), (120, 300, 64), (2000, 100, 4), (64, 1000, 100)]


@pytest.mark.parametrize("outer,R,inner", COLS_SHAPES)
def test_cols_vs_oracle(orc, outer, R, inner):
    x = inputs.normal((outer, R, inner), seed=outer * 31 + R + inner, sigma=3.0, device=DEV)
    xc = x.cpu().numpy()
    ref_l, ref_y = orc.lse_axis(xc), orc.log_softmax_axis(xc)
    out = L.lse_reduce_axis(x, 1)          # with a workspace when the sizes call for one
    y = L.log_softmax_axis(x, 1)
    torch.cuda.synchronize()
    what = f"{outer}x{R}x{inner}"
    compare(out.cpu().numpy(), ref_l, what="cols lse ws " + what)
    compare(y.cpu().numpy(), ref_y, what="cols lsm ws " + what)
    # the entry points without a workspace (one workgroup per tile, or the
    # plane-split kernels)
    out0 = _raw_axis(x, R, inner, False)
    y0 = _raw_axis(x, R, inner, True)
    torch.cuda.synchronize()
    compare(out0.cpu().numpy(), ref_l, what="cols lse no ws " + what)
    compare(y0.cpu().numpy(), ref_y, what="cols lsm no ws " + what)
    if outer == 1:
        a0 = L.lse_reduce_axis0(x[0])
        torch.cuda.synchronize()
        compare(a0.cpu().numpy(), ref_l.reshape(-1), what="axis0 ws " + what)


def test_cols_special_values(orc):
    """Columns of 100000 planes: all -inf, one +inf, a NaN in the last plane,
    one finite value among -inf, -inf over the first chunks only (empty chunk
    pairs), a huge value, a large common offset, equal values."""
    R = 100000
    x = inputs.normal((R, 8), seed=3, device=DEV)
    x[:, 0] = -float("inf")
    x[5000, 1] = float("inf")
    x[R - 1, 2] = float("nan")
    x[:, 3] = -float("inf"); x[77777, 3] = 1.5
    x[:60000, 4] = -float("inf")
    x[10, 5] = 1e30
    x[:, 6] += 1000.0
    x[:, 7] = 3.0
    xc = x.cpu().numpy().reshape(1, R, 8)
    ref_l, ref_y = orc.lse_axis(xc), orc.log_softmax_axis(xc)
    for ws in (True, False):
        if ws:
            out, y = L.lse_reduce_axis(x, 0), L.log_softmax_axis(x, 0)
        else:
            out, y = _raw_axis(x, R, 8, False), _raw_axis(x, R, 8, True)
        torch.cuda.synchronize()
        compare(out.cpu().numpy(), ref_l, what=f"cols special lse ws={ws}")
        compare(y.cpu().numpy(), ref_y, what=f"cols special lsm ws={ws}")
        o = out.cpu().numpy().reshape(-1)
        assert o[0] == -np.inf and o[1] == np.inf and np.isnan(o[2])


@pytest.mark.parametrize("layout", ["inner_slice", "offset", "out_strided", "plane_pitch"])
def test_cols_strided_views(orc, layout):
    """Views: an inner slice (pitch > inner), x at a 4-byte offset, outputs
    with padded outer and plane pitches (two outer blocks), planes 2 floats
    apart with inner = 1 (scalar lanes)."""
    R, inner, outer = 50000, 24, 1
    if layout == "inner_slice":
        x = inputs.normal((R, 40), seed=7, device=DEV)[:, 5:5 + inner]
    elif layout == "offset":
        x = inputs.normal((R * inner + 1,), seed=8, device=DEV)[1:].view(R, inner)
    elif layout == "out_strided":
        outer = 2
        x = inputs.normal((outer, R, inner), seed=9, device=DEV)
    else:
        inner = 1
        x = inputs.normal((R, 2), seed=10, device=DEV)[:, :1]
    xc = x.contiguous().cpu().numpy().reshape(outer, R, inner)
    ref_l, ref_y = orc.lse_axis(xc), orc.log_softmax_axis(xc)
    if layout == "out_strided":
        obuf = torch.full((outer, inner + 5), 7.0, device=DEV)
        out = L.lse_reduce_axis(x, 1, out=obuf[:, :inner])
        ybuf = torch.full((outer, R, inner + 3), 7.0, device=DEV)
        y = L.log_softmax_axis(x, 1, y=ybuf[:, :, :inner])
    else:
        out = L.lse_reduce_axis(x, 0)
        y = L.log_softmax_axis(x, 0)
    torch.cuda.synchronize()
    compare(out.cpu().numpy(), ref_l, what=f"cols view lse {layout}")
    compare(y.cpu().numpy(), ref_y, what=f"cols view lsm {layout}")
    if layout == "out_strided":
        assert (obuf[:, inner:] == 7.0).all()
        assert (ybuf[:, :, inner:] == 7.0).all()


def test_cols_workspace_reuse_and_determinism(orc):
    """A caller's workspace full of garbage, reused: bit-identical results on
    every call (the merges run in a fixed order)."""
    R, inner = 300000, 12
    x = inputs.normal((R, inner), seed=12, sigma=2.0, device=DEV)
    need = max(L.lse_axis_workspace_bytes(1, R, inner), L.lse_axis_workspace_bytes(1, R, inner, True))
    assert need > 0
    ws = torch.full((need,), 255, dtype=torch.uint8, device=DEV)
    a = L.lse_reduce_axis(x, 0, ws=ws).clone()
    ya = L.log_softmax_axis(x, 0, ws=ws).clone()
    ws.fill_(0x7f)
    b = L.lse_reduce_axis(x, 0, ws=ws)
    yb = L.log_softmax_axis(x, 0, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(ya, yb)
    compare(a.cpu().numpy(), orc.lse_axis(x.cpu().numpy().reshape(1, R, inner)).reshape(inner),
            what="cols ws reuse")


@pytest.mark.parametrize("rows,cols,off", [(2, 4194305, 0), (1, 5000000, 0), (1, 4500001, 1),
                                           (3, 4194304, 0), (2, 2097153, 0), (1, 3000001, 1)])
@pytest.mark.parametrize("softmax", [False, True])
def test_rows_many_chunks(orc, rows, cols, off, softmax):
    """Rows of more than 128 chunks (4M columns) take three launches (tile
    pairs, merge per row, write); exactly 128 chunks, and 65-92, still wait
    for each other.  Odd lengths and a 4-byte offset take the scalar write."""
    buf = inputs.normal((rows * cols + off,), seed=cols + off, sigma=2.0, device=DEV)
    x = buf[off:].view(rows, cols)
    xc = x.cpu().numpy()
    y = L.softmax_rows(x) if softmax else L.log_softmax_rows(x)
    torch.cuda.synchronize()
    if softmax:
        compare(y.cpu().numpy(), orc.softmax_rows(xc), what=f"softmax many chunks {rows}x{cols}",
                rtol=1e-5, atol=1e-37)
    else:
        ref, _ = orc.log_softmax_rows(xc)
        compare(y.cpu().numpy(), ref, what=f"lsm many chunks {rows}x{cols}")
        # the same rows through the axis call (workspace from the binding)
        ya = L.log_softmax_axis(x, 1)
        torch.cuda.synchronize()
        compare(ya.cpu().numpy(), ref, what=f"lsm axis many chunks {rows}x{cols}")


def test_rows_many_chunks_special(orc):
    """Three-launch rows: all -inf, +inf, NaN in the last tile, one finite value."""
    cols = 4400000
    x = inputs.normal((4, cols), seed=21, device=DEV)
    x[0, :] = -float("inf")
    x[1, 1234567] = float("inf")
    x[2, cols - 1] = float("nan")
    x[3, :] = -float("inf"); x[3, 2000000] = 0.5
    xc = x.cpu().numpy()
    ref, _ = orc.log_softmax_rows(xc)
    y = L.log_softmax_rows(x)
    torch.cuda.synchronize()
    yc = y.cpu().numpy()
    compare(yc, ref, what="many chunks special")
    assert np.isnan(yc[0]).all() and np.isnan(yc[2]).all() and yc[3, 2000000] == 0.0


@pytest.mark.parametrize("rows,cols", [(1, 5000001), (8, 1000000), (3, 16385)])
def test_lse_last_axis_split_rows(orc, rows, cols):
    """Long last-axis logsumexp rows with a workspace: tile pairs then a merge
    per row (few rows)."""
    x = inputs.normal((rows, cols), seed=rows + cols, sigma=3.0, device=DEV)
    assert L.lse_axis_workspace_bytes(rows, cols, 1) > 0
    out = L.lse_reduce_axis(x, 1)
    torch.cuda.synchronize()
    compare(out.cpu().numpy(), orc.lse_axis(x.cpu().numpy().reshape(rows, cols, 1)).reshape(rows),
            what=f"lse split rows {rows}x{cols}")


@pytest.mark.parametrize("outer,R,inner,lsm", [(1, 1048576, 64, False), (16, 65536, 64, False),
                                               (1, 300000, 49, True), (1, 100000, 1000, False)])
def test_long_streams_within_tolerance(orc, outer, R, inner, lsm):
    """The entry points without a workspace fold hundreds of thousands of
    planes per lane into one running sum: small terms must not be rounded
    away against it (the plain running sum ran 1.9 x over the tolerance on
    (1, 1048576, 64))."""
    x = inputs.normal((outer, R, inner), seed=R + inner, sigma=3.0, device=DEV)
    got = _raw_axis(x, R, inner, lsm)
    torch.cuda.synchronize()
    xc = x.cpu().numpy()
    ref = orc.log_softmax_axis(xc) if lsm else orc.lse_axis(xc)
    compare(got.cpu().numpy(), ref, what=f"long stream {outer}x{R}x{inner} lsm={lsm}")
