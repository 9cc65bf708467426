"""GPU parity of the middle-axis reductions over contiguous (R, inner) blocks
with a short inner run (read as flat sweeps whose width is a multiple of both
4 and inner), against the fp64 oracle: chunked blocks (pair launch, then a
merge or an apply launch), whole blocks per workgroup, the entry points
without a workspace, views at other 4-byte phases and with padded block
pitches, special values and run-to-run bit equality."""

import numpy as np
import pytest
import torch

import log_softmax_reductions_amd as L
from log_softmax_reductions_amd import _lib, inputs
from tests.parity import compare

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _raw(x, outer, R, inner, lsm):
    """The entry points without a workspace on a contiguous (outer, R, inner) x."""
    lib = _lib.load()
    out = torch.empty((outer, R, inner) if lsm else (outer, inner), device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    fn = lib.log_softmax_axis if lsm else lib.lse_reduce_axis
    _lib.check(fn(x.data_ptr(), out.data_ptr(), outer, R, inner, st), "axis without workspace")
    return out


# (outer, R, inner): every inner run width class (merge widths of 1 to 64
# lanes per column), ragged last chunks and sweeps, chunked (few blocks) and
# whole-block (many blocks) plans
BLOCK_SHAPES = [(40, 4000, 49), (33, 5001, 5), (64, 2000, 3), (48, 3001, 13), (32, 777, 25),
                (100, 900, 63), (36, 1000, 127), (40, 400, 100), (50, 2500, 6), (1100, 100, 49),
                (1500, 41, 50), (1024, 199, 7), (1200, 30, 86), (3000, 1000, 5), (700, 500, 2),
                # logsumexp over large blocks of wider runs (one partial per lane and column)
                (40, 600, 196), (36, 520, 255), (33, 300, 256),
                # few long blocks: hundreds of chunks per block, merged by a wave per column
                (1, 300000, 49), (3, 100003, 7), (2, 200000, 6), (1, 150001, 100),
                # log_softmax over few long blocks of aligned runs (pairs, a wave per
                # column merging up to 1024 chunks per round of loads, then the apply)
                (1, 300000, 64), (3, 100001, 16), (2, 600000, 8), (5, 40000, 128)]


@pytest.mark.parametrize("outer,R,inner", BLOCK_SHAPES)
def test_blocks_vs_oracle(orc, outer, R, inner):
    x = inputs.normal((outer, R, inner), seed=outer * 7 + R + inner, sigma=3.0, device=DEV)
    xc = x.cpu().numpy()
    ref_l, ref_y = orc.lse_axis(xc), orc.log_softmax_axis(xc)
    what = f"{outer}x{R}x{inner}"
    out = L.lse_reduce_axis(x, 1)
    y = L.log_softmax_axis(x, 1)
    torch.cuda.synchronize()
    compare(out.cpu().numpy(), ref_l, what="blocks lse ws " + what)
    compare(y.cpu().numpy(), ref_y, what="blocks lsm ws " + what)
    out0 = _raw(x, outer, R, inner, False)
    y0 = _raw(x, outer, R, inner, True)
    torch.cuda.synchronize()
    compare(out0.cpu().numpy(), ref_l, what="blocks lse no ws " + what)
    compare(y0.cpu().numpy(), ref_y, what="blocks lsm no ws " + what)


@pytest.mark.parametrize("layout", ["offset1", "offset3", "block_pitch", "out_pitch", "aligned16"])
@pytest.mark.parametrize("outer,R,inner", [(40, 3000, 49), (1100, 60, 49), (600, 128, 16)])
def test_blocks_views(orc, layout, outer, R, inner):
    """x at a 4- or 12-byte offset, blocks with padding between them (x and
    y), outputs with a padded outer pitch; (600, 128, 16) on the 16-byte grid
    takes the blocks only without a workspace.  Padding must stay untouched."""
    n = R * inner
    if layout.startswith("offset"):
        k = int(layout[-1])
        x = inputs.normal((outer * n + k,), seed=k + inner, sigma=2.0, device=DEV)[k:].view(outer, R, inner)
    elif layout == "block_pitch":
        x = inputs.normal((outer, n + 9), seed=5, sigma=2.0, device=DEV)[:, :n].unflatten(1, (R, inner))
    else:
        x = inputs.normal((outer, R, inner), seed=6, sigma=2.0, device=DEV)
    xc = x.contiguous().cpu().numpy()
    ref_l, ref_y = orc.lse_axis(xc), orc.log_softmax_axis(xc)
    what = f"{layout} {outer}x{R}x{inner}"
    if layout in ("block_pitch", "out_pitch"):
        obuf = torch.full((outer, inner + 3), 7.0, device=DEV)
        ybuf = torch.full((outer, n + 5), 7.0, device=DEV)
        out = L.lse_reduce_axis(x, 1, out=obuf[:, :inner])
        y = L.log_softmax_axis(x, 1, y=ybuf[:, :n].unflatten(1, (R, inner)))
    else:
        out = L.lse_reduce_axis(x, 1)
        y = L.log_softmax_axis(x, 1)
    torch.cuda.synchronize()
    compare(out.cpu().numpy(), ref_l, what="blocks view lse " + what)
    compare(y.cpu().numpy(), ref_y, what="blocks view lsm " + what)
    if layout in ("block_pitch", "out_pitch"):
        assert (obuf[:, inner:] == 7.0).all() and (ybuf[:, n:] == 7.0).all()
    if outer >= 512:  # the entry points without a workspace take whole blocks
        xd = x.contiguous()
        compare(_raw(xd, outer, R, inner, False).cpu().numpy(), ref_l, what="blocks view lse no ws " + what)
        compare(_raw(xd, outer, R, inner, True).cpu().numpy(), ref_y, what="blocks view lsm no ws " + what)


@pytest.mark.parametrize("outer,R", [(40, 3000), (1100, 60)])
def test_blocks_special_values(orc, outer, R):
    """Columns all -inf, one +inf, a NaN in the last plane, one finite value
    among -inf, -inf over the first half (empty early chunks), a huge value,
    a large common offset, equal values."""
    inner = 49
    x = inputs.normal((outer, R, inner), seed=11, device=DEV)
    x[:, :, 0] = -float("inf")
    x[:, R // 3, 1] = float("inf")
    x[:, R - 1, 2] = float("nan")
    x[:, :, 3] = -float("inf"); x[:, R // 2 + 1, 3] = 1.5
    x[:, : R // 2, 4] = -float("inf")
    x[:, 10, 5] = 1e30
    x[:, :, 6] += 1000.0
    x[:, :, 7] = 3.0
    xc = x.cpu().numpy()
    ref_l, ref_y = orc.lse_axis(xc), orc.log_softmax_axis(xc)
    for ws in (True, False):
        if ws:
            out, y = L.lse_reduce_axis(x, 1), L.log_softmax_axis(x, 1)
        else:
            out, y = _raw(x, outer, R, inner, False), _raw(x, outer, R, inner, True)
        torch.cuda.synchronize()
        compare(out.cpu().numpy(), ref_l, what=f"blocks special lse ws={ws}")
        compare(y.cpu().numpy(), ref_y, what=f"blocks special lsm ws={ws}")
        o = out.cpu().numpy()
        assert (o[:, 0] == -np.inf).all() and (o[:, 1] == np.inf).all() and np.isnan(o[:, 2]).all()


def test_blocks_bit_identical_reruns():
    """Chunk pairs merge in a fixed order: repeated calls are bit-identical."""
    x = inputs.normal((40, 4000, 63), seed=13, sigma=2.0, device=DEV)
    a, ya = L.lse_reduce_axis(x, 1).clone(), L.log_softmax_axis(x, 1).clone()
    for _ in range(3):
        b, yb = L.lse_reduce_axis(x, 1), L.log_softmax_axis(x, 1)
        torch.cuda.synchronize()
        assert torch.equal(a, b) and torch.equal(ya, yb)


@pytest.mark.parametrize("outer,R,inner", [(1100, 1000, 49), (1100, 8001, 5), (700, 701, 127),
                                           (50, 4000, 49), (32, 30000, 5), (20, 50000, 10),
                                           (256, 2048, 49), (100, 6000, 63)])
def test_blocks_resident_helping_bit_identical(orc, outer, R, inner):
    """log_softmax over blocks split into chunks that wait for each other (grids
    of 160 to 2200 workgroups; ragged last chunks): at a poll limit of 0 no owner
    publishes, so every chunk's pairs come from the helping path (re-read from
    x); the result must equal the default run bit for bit, and the oracle."""
    x = inputs.normal((outer, R, inner), seed=outer + R + inner, sigma=3.0, device=DEV)
    y = L.log_softmax_axis(x, 1).clone()
    try:
        L.lse_testing_set_spin_limit(0)
        yh = L.log_softmax_axis(x, 1)
        torch.cuda.synchronize()
    finally:
        L.lse_testing_set_spin_limit(1 << 24)
    assert torch.equal(y, yh)
    compare(yh.cpu().numpy(), orc.log_softmax_axis(x.cpu().numpy()), what=f"helped {outer}x{R}x{inner}")
