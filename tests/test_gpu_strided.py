"""GPU parity of the strided entry points (views into larger buffers) through
the C ABI against the fp64 oracle run on the same values made contiguous, and
checks that nothing outside the output view is written."""
import numpy as np
import pytest
import torch

import log_softmax_reductions_amd as L
from log_softmax_reductions_amd import inputs
from tests.parity import compare

pytestmark = pytest.mark.gpu
DEV = "cuda"
SENTINEL = 12345.0


def _padded_out(shape, pad_last, dev=DEV):
    """A view of `shape` into a buffer whose last dim is pad_last longer, the
    padding filled with a sentinel."""
    big = torch.full(tuple(shape[:-1]) + (shape[-1] + pad_last,), SENTINEL, device=dev)
    return big, big[..., :shape[-1]]


def _untouched(big, view):
    mask = torch.ones_like(big, dtype=torch.bool)
    mask[..., :view.shape[-1]] = False
    return bool((big[mask] == SENTINEL).all())


@pytest.mark.parametrize("rows,cols,padx,pady", [(64, 4096, 4, 8), (37, 1000, 3, 1),
                                                   (8, 100000, 4, 12), (5, 393216, 1, 4),
                                                   (16, 50000, 0, 4), (4, 65536, 4, 4)])
def test_rows_with_pitch(orc, rows, cols, padx, pady):
    """log_softmax_rows / softmax_rows on column slices of wider matrices:
    vector and scalar pitches, single-workgroup and split rows."""
    xbig = inputs.normal((rows, cols + padx), seed=rows + cols, sigma=3.0, device=DEV)
    x = xbig[:, :cols]
    xc = x.contiguous().cpu().numpy()
    ybig, y = _padded_out((rows, cols), pady)
    L.log_softmax_rows(x, y)
    torch.cuda.synchronize()
    ref, _ = orc.log_softmax_rows(xc, want_y=True)
    compare(y.cpu().numpy(), ref, what=f"strided log_softmax {rows}x{cols}")
    assert _untouched(ybig, y)
    sbig, s = _padded_out((rows, cols), pady)
    L.softmax_rows(x, s)
    torch.cuda.synchronize()
    compare(s.cpu().numpy(), orc.softmax_rows(xc), atol=1e-37, rtol=1e-5,
            what=f"strided softmax {rows}x{cols}")
    assert _untouched(sbig, s)
    # the contiguous call on the same values gives bit-identical results
    if padx % 4 == 0 and pady % 4 == 0:
        assert torch.equal(L.log_softmax_rows(x.contiguous()), y)


@pytest.mark.parametrize("shape,dim,sl", [
    ((4, 70, 300), 1, (slice(None), slice(3, 67), slice(None))),        # slice of planes
    ((4, 64, 300), 1, (slice(None), slice(None), slice(0, 256))),       # slice of the inner run
    ((6, 40, 33), 1, (slice(None), slice(None), slice(1, 30))),         # unaligned inner slice
    ((2, 300, 64), 1, (slice(None), slice(0, 290, 1), slice(None))),    # streamed split
    ((1, 2048, 8200), 1, (slice(None), slice(None), slice(0, 8192))),   # few outputs, long R
    ((3, 20, 5, 8), 1, (slice(None), slice(None), 2, slice(None))),     # a selected dim
    ((64, 48), 0, (slice(0, 40), slice(None))),                         # leading axis
])
def test_axis_views(orc, shape, dim, sl):
    big = inputs.normal(shape, seed=sum(shape), sigma=3.0, device=DEV)
    x = big[sl]
    assert not x.is_contiguous() or x.dim() == 2
    xc = x.contiguous()
    d = dim % x.dim()
    outer = int(np.prod(x.shape[:d])) if d else 1
    R = x.shape[d]
    xn = xc.cpu().numpy().reshape(outer, R, -1)
    got = L.lse_reduce_axis(x, d)
    torch.cuda.synchronize()
    compare(got.cpu().numpy().reshape(outer, -1), orc.lse_axis(xn), what=f"strided lse {shape}")
    y = L.log_softmax_axis(x, d)
    torch.cuda.synchronize()
    compare(y.cpu().numpy().reshape(outer, R, -1), orc.log_softmax_axis(xn),
            what=f"strided lsm {shape}")
    # a strided output: y written into a padded buffer, padding untouched
    ybig, yv = _padded_out(tuple(x.shape), 4)
    L.log_softmax_axis(x, d, yv)
    torch.cuda.synchronize()
    assert _untouched(ybig, yv)
    compare(yv.contiguous().cpu().numpy().reshape(outer, R, -1), orc.log_softmax_axis(xn),
            what=f"strided lsm, strided y {shape}")


def test_axis_strided_output_of_logsumexp(orc):
    """lse_reduce_axis into a column slice of a wider output matrix."""
    x = inputs.normal((8, 64, 1000), seed=21, device=DEV)
    obig, ov = _padded_out((8, 1000), 24)
    L.lse_reduce_axis(x, 1, ov)
    torch.cuda.synchronize()
    assert _untouched(obig, ov)
    compare(ov.cpu().numpy(), orc.lse_axis(x.cpu().numpy()), what="lse into a padded output")


def test_chain_layout_channel_slice(orc):
    """The chain's channel reduction on a view: 60 of 64 channels of
    (128, 64, 15876), sampled outer slices."""
    big = inputs.normal((128, 64, 126 * 126), seed=12, device=DEV)
    x = big[:, 2:62]
    out = L.lse_reduce_axis(x, 1)
    y = L.log_softmax_axis(x, 1)
    torch.cuda.synchronize()
    for o in (0, 64, 127):
        xs = x[o:o + 1].contiguous().cpu().numpy()
        compare(out[o:o + 1].cpu().numpy(), orc.lse_axis(xs), what=f"channel slice lse {o}")
        compare(y[o:o + 1].cpu().numpy(), orc.log_softmax_axis(xs), what=f"channel slice lsm {o}")


def test_unsupported_layouts_raise():
    x = inputs.normal((4, 6, 5, 8), seed=3, device=DEV)
    with pytest.raises(ValueError):
        L.lse_reduce_axis(x[..., :6], 1)          # inner dims do not form one run
    with pytest.raises(ValueError):
        L.log_softmax_rows(x[:, 0, 0, :].t())     # rows not contiguous
    with pytest.raises(L.LseError, match="LSE_ERR_SHAPE"):
        # a y view whose planes would collide: stride 0 over R (an expanded view)
        L.log_softmax_axis(x[:, :, 0, :], 1, torch.empty(4, 1, 8, device=DEV).expand(4, 6, 8))
