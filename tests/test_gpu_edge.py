"""Empty and degenerate inputs through every entry point on the GPU: empty
tensors are no-ops that return empty results, and the sizes whose result the
definition fixes exactly are checked bit for bit (one value reduced gives
itself; one column gives log_softmax 0 and softmax 1; -inf stays -inf).  The
invariants of the definition are checked on the GPU results too: R equal
values give v + log R, a shift moves the LSE by the shift, and the order of
the reduced values does not matter."""
import numpy as np
import pytest
import torch

import log_softmax_reductions_amd as L
from log_softmax_reductions_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_empty_inputs():
    e = torch.empty(0, 7, device=DEV)
    assert L.log_softmax_rows(e).shape == (0, 7)
    assert L.softmax_rows(e).shape == (0, 7)
    assert L.lse_reduce_axis0(torch.empty(3, 0, device=DEV)).shape == (0,)
    assert L.lse_reduce_axis(torch.empty(0, 5, 9, device=DEV), 1).shape == (0, 9)
    assert L.log_softmax_axis(torch.empty(2, 5, 0, device=DEV), 1).shape == (2, 5, 0)
    p = L.lse_rows_partial(e, 4)
    assert p.shape == (0, 2, 2)
    assert L.lse_rows_merge(p).shape == (0,)
    x, w, b, g, be = inputs.conv_chain_inputs(N=1, H=6, W=6, seed=1, device=DEV)
    out = L.fused_conv_gn_act_lse(x[:0], w, b, g, be, 16, 1e-5)
    assert out.shape == (0, 1, 4, 4)
    torch.cuda.synchronize()


def test_single_value_reductions_are_exact():
    x = inputs.normal((1, 4097), seed=7, sigma=30.0, device=DEV)
    x[0, 5] = -float("inf")
    # one plane: LSE of one value is that value, m + log(1) with log(1) = 0
    assert torch.equal(L.lse_reduce_axis0(x), x[0])
    assert torch.equal(L.lse_reduce_axis(x.view(1, 1, 4097), 1), x.view(1, 4097))
    # one column: log_softmax is x - x = 0 (NaN for -inf), softmax is 1
    col = x.view(4097, 1)
    y = L.log_softmax_rows(col)
    s = L.softmax_rows(col)
    torch.cuda.synchronize()
    fin = torch.isfinite(col)
    assert torch.equal(y[fin], torch.zeros_like(y[fin]))
    assert torch.isnan(y[~fin]).all()
    assert torch.equal(s[fin], torch.ones_like(s[fin]))
    assert torch.isnan(s[~fin]).all()
    # log_softmax over an axis of length 1: 0 everywhere finite
    z = L.log_softmax_axis(x.view(1, 1, 4097), 1)
    assert torch.equal(z.view(-1)[fin.view(-1)], torch.zeros(int(fin.sum()), device=DEV))


def test_constant_rows_are_log_of_length():
    """A row of equal values v: LSE = v + log(n) and log_softmax = -log(n)."""
    for cols in (3, 4096, 100000):
        x = torch.full((2, cols), 2.5, device=DEV)
        y = L.log_softmax_rows(x)
        torch.cuda.synchronize()
        ref = -torch.log(torch.tensor(float(cols), dtype=torch.float64)).item()
        assert (y.double() - ref).abs().max().item() <= 1e-5 + 2e-6 * abs(ref)


def test_side_stream_with_internal_workspace(orc):
    """A split row computed on a side stream with the workspace left to the
    binding: the workspace is recorded on that stream, so allocations made on
    the current stream meanwhile cannot take its memory."""
    from tests.parity import compare
    x = inputs.normal((8, 100000), seed=31, device=DEV)
    chain = inputs.conv_chain_inputs(N=2, H=20, W=20, seed=5, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())   # the inputs exist before s reads them
    y = L.log_softmax_rows(x, stream=s)
    c = L.fused_conv_gn_act_lse(*chain, 16, 1e-5, stream=s)
    churn = [torch.full((1 << 18,), 7.0, device=DEV) for _ in range(16)]
    del churn
    s.synchronize()
    ref, _ = orc.log_softmax_rows(x.cpu().numpy(), want_y=True)
    compare(y.cpu().numpy(), ref, what="side-stream log_softmax")
    assert torch.isfinite(c).all()


@pytest.mark.parametrize("R,inner", [(4, 320), (32, 4096), (64, 15876), (300, 257)])
def test_equal_planes_give_value_plus_log_R(R, inner):
    """R equal values v: LSE = v + log R on every path (register-resident,
    streamed, plane split); log_softmax is -log R."""
    for v in (-3.5, 0.0, 1e4):
        x = torch.full((R, inner), v, device=DEV)
        out = L.lse_reduce_axis0(x)
        y = L.log_softmax_axis(x.view(1, R, inner), 1)
        torch.cuda.synchronize()
        ref = v + np.log(R)
        assert np.abs(out.cpu().numpy().astype(np.float64) - ref).max() <= 1e-5 + 2e-6 * abs(ref)
        lr = -np.log(R)
        assert np.abs(y.cpu().numpy().astype(np.float64) - lr).max() <= 1e-5 + 2e-6 * abs(lr)


def test_shift_moves_lse_by_the_shift():
    """LSE(x + c) = LSE(x) + c and log_softmax(x + c) = log_softmax(x), up to
    the rounding of x + c, on the three layouts."""
    x = inputs.normal((16, 3000), seed=41, sigma=2.0, device=DEV)
    for c in (-1000.0, 3.75, 1000.0):
        xc = x + c
        a0, a1 = L.lse_reduce_axis0(x), L.lse_reduce_axis0(xc)
        r0, r1 = L.log_softmax_rows(x), L.log_softmax_rows(xc)
        torch.cuda.synchronize()
        # |x + c| ~ 1000 carries an fp32 rounding of up to 2^-14 per element
        tol = 1e-5 + 2e-6 * abs(c) + (6.2e-5 if abs(c) >= 1000 else 0.0)
        assert (a1.double() - (a0.double() + c)).abs().max().item() <= tol + 2e-6 * abs(c)
        assert (r1.double() - r0.double()).abs().max().item() <= tol


def test_plane_order_does_not_matter():
    """Permuting the reduced axis permutes nothing in logsumexp (same result up
    to summation order) and permutes log_softmax's planes alike."""
    x = inputs.normal((2, 48, 1000), seed=43, sigma=3.0, device=DEV)
    perm = torch.randperm(48, generator=torch.Generator().manual_seed(5)).to(DEV)
    xp = x[:, perm].contiguous()
    a, b = L.lse_reduce_axis(x, 1), L.lse_reduce_axis(xp, 1)
    y, yp = L.log_softmax_axis(x, 1), L.log_softmax_axis(xp, 1)
    torch.cuda.synchronize()
    assert (a.double() - b.double()).abs().max().item() <= 1e-5 + 2e-6 * a.abs().max().item()
    assert (y[:, perm].double() - yp.double()).abs().max().item() <= 2e-5
