"""Seeded random shapes chosen to cross the dispatch thresholds of the axis and
row reductions: short segments and interleaved short blocks, the column split
(few outputs over many planes) with and without a workspace, the axis kernels,
split logsumexp rows and rows of more chunks than can wait for each other.
Every result is checked against the fp64 oracle, including a special value
(+-inf, NaN) in a quarter of the axis cases.  The draws come from one fixed
numpy seed and appear in the test ids; sizes stay small enough for the oracle."""
import numpy as np
import pytest
import torch

import log_softmax_reductions_amd as L
from log_softmax_reductions_amd import _lib, inputs
from tests.parity import compare

pytestmark = pytest.mark.gpu
DEV = "cuda"
_rng = np.random.default_rng(20261203)
_MAX_ELEMS = 1_500_000

AXIS_CASES = []
for i in range(40):
    inner = int(_rng.choice([1, 2, 3, 4, 5, 7, 8, 12, 16, 33, 49, 64, 100, 128, 256, 257,
                             1000, 4096]))
    R = int(_rng.choice([1, 2, 3, 4, 7, 16, 31, 32, 33, 64, 65, 100, 256, 257, 600, 1024,
                         3000, 20000, 70000]))
    while R * inner > _MAX_ELEMS and R > 1:
        R //= 2
    top = max(1, min(_MAX_ELEMS // (R * inner), 2000))
    outer = int(round(float(np.exp(_rng.uniform(0.0, np.log(top))))))   # log-uniform
    layout = ["packed", "offset", "strided"][i % 3]
    special = float(_rng.choice([np.inf, -np.inf, np.nan])) if i % 4 == 0 else 0.0
    AXIS_CASES.append((outer, R, inner, layout, special))


def _axis_view(outer, R, inner, layout, seed):
    if layout == "packed":
        return inputs.normal((outer, R, inner), seed=seed, sigma=3.0, device=DEV)
    if layout == "offset":
        n = outer * R * inner
        return inputs.normal((n + 1,), seed=seed, sigma=3.0, device=DEV)[1:].view(outer, R, inner)
    # inner run 3 floats short of its pitch, one spare plane per outer block
    return inputs.normal((outer, R + 1, inner + 3), seed=seed, sigma=3.0,
                         device=DEV)[:, :R, :inner]


def _raw_axis(x, outer, R, inner, lsm):
    """The entry points without a workspace, on a contiguous x."""
    lib = _lib.load()
    out = torch.empty((outer, R, inner) if lsm else (outer, inner), device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    fn = lib.log_softmax_axis if lsm else lib.lse_reduce_axis
    _lib.check(fn(x.data_ptr(), out.data_ptr(), outer, R, inner, st), "axis without workspace")
    return out


@pytest.mark.parametrize("outer,R,inner,layout,special", AXIS_CASES)
def test_random_axis_paths(orc, outer, R, inner, layout, special):
    seed = outer * 100003 + R * 101 + inner
    x = _axis_view(outer, R, inner, layout, seed)
    if special != 0.0:
        g = np.random.default_rng(seed)
        x[int(g.integers(0, outer)), int(g.integers(0, R)), int(g.integers(0, inner))] = special
    xc = x.contiguous().cpu().numpy()
    ref_l, ref_y = orc.lse_axis(xc), orc.log_softmax_axis(xc)
    tag = f"({outer},{R},{inner}) {layout} special {special}"
    out = L.lse_reduce_axis(x, 1)            # with a workspace when the sizes call for one
    y = L.log_softmax_axis(x, 1)
    torch.cuda.synchronize()
    compare(out.cpu().numpy(), ref_l, what="lse ws " + tag)
    compare(y.cpu().numpy(), ref_y, what="lsm ws " + tag)
    xd = x.contiguous()
    out0 = _raw_axis(xd, outer, R, inner, False)
    y0 = _raw_axis(xd, outer, R, inner, True)
    torch.cuda.synchronize()
    compare(out0.cpu().numpy(), ref_l, what="lse no ws " + tag)
    compare(y0.cpu().numpy(), ref_y, what="lsm no ws " + tag)


ROW_CASES = []
for i in range(24):
    cols = int(_rng.choice([1, 2, 3, 5, 17, 64, 99, 255, 256, 1000, 1025, 2048, 2049, 4097,
                            16383, 16384, 32769, 100003, 2100000]))
    rows = int(_rng.integers(1, max(2, min(3000, 3_000_000 // cols)) + 1))
    ROW_CASES.append((rows, cols, i % 2))


@pytest.mark.parametrize("rows,cols,off", ROW_CASES)
def test_random_row_paths(orc, rows, cols, off):
    """Rows through log_softmax, softmax and the last-axis logsumexp, x packed
    or at a 4-byte offset."""
    buf = inputs.normal((rows * cols + off,), seed=rows * 7 + cols, sigma=2.0, device=DEV)
    x = buf[off:].view(rows, cols)
    xc = x.cpu().numpy()
    tag = f"({rows},{cols}) +{off}"
    ref, ref_lse = orc.log_softmax_rows(xc)
    y = L.log_softmax_rows(x)
    s = L.softmax_rows(x)
    out = L.lse_reduce_axis(x, 1)
    torch.cuda.synchronize()
    compare(y.cpu().numpy(), ref, what="rows log_softmax " + tag)
    compare(s.cpu().numpy(), orc.softmax_rows(xc), rtol=1e-5, atol=1e-37,
            what="rows softmax " + tag)
    compare(out.cpu().numpy(), ref_lse, what="rows logsumexp " + tag)
