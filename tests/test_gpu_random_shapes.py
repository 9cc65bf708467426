"""Seeded random shapes through every entry point against the fp64 oracle.

The shapes, alignments, pitches and chunk sizes are drawn once from a fixed
numpy seed (listed in the test ids), so each run covers the same spread of
dispatch paths: vector and scalar loads, register-resident and streamed
planes, every plane-split width, single-workgroup and split rows, fused and
two-launch chains.  Data comes from the seeded input generators."""
import numpy as np
import pytest
import torch

import log_softmax_reductions_amd as L
from log_softmax_reductions_amd import inputs
from tests.parity import RTOL_CHAIN, compare

pytestmark = pytest.mark.gpu
DEV = "cuda"
_rng = np.random.default_rng(20261202)


def _loguniform(lo, hi):
    return int(round(float(np.exp(_rng.uniform(np.log(lo), np.log(hi))))))


def _view(shape, offset, pad_last, seed, sigma):
    """A (possibly misaligned, padded) view of `shape` into a larger buffer."""
    big_shape = tuple(shape[:-1]) + (shape[-1] + pad_last,)
    n = int(np.prod(big_shape)) + offset
    buf = inputs.normal((n,), seed=seed, sigma=sigma, device=DEV)
    big = buf[offset:].view(big_shape)
    return big[..., :shape[-1]]


AXIS_CASES = []
for i in range(40):
    outer = int(_rng.integers(1, 7))
    R = _loguniform(1, 400)
    inner = _loguniform(1, 3000)
    if _rng.random() < 0.5:
        inner = max(4, inner - inner % 4)
    offset = int(_rng.choice([0, 0, 1, 3]))
    pad = int(_rng.choice([0, 0, 4, 5]))
    AXIS_CASES.append((outer, R, inner, offset, pad, float(_rng.choice([1.0, 3.0, 10.0]))))


@pytest.mark.parametrize("outer,R,inner,offset,pad,sigma", AXIS_CASES)
def test_random_axis(orc, outer, R, inner, offset, pad, sigma):
    """(outer, R, inner) views reduced over R: planes pad floats apart beyond inner."""
    big = _view((outer * R, inner), offset, pad, seed=outer * 100003 + R * 101 + inner, sigma=sigma)
    x = big.unflatten(0, (outer, R))
    xn = x.contiguous().cpu().numpy()
    got = L.lse_reduce_axis(x, 1)
    y = L.log_softmax_axis(x, 1)
    torch.cuda.synchronize()
    tag = f"({outer},{R},{inner}) off {offset} pad {pad}"
    compare(got.cpu().numpy(), orc.lse_axis(xn), what="lse " + tag)
    compare(y.cpu().numpy(), orc.log_softmax_axis(xn), what="lsm " + tag)


ROWS_CASES = []
for i in range(30):
    rows = int(_rng.integers(1, 21))
    cols = _loguniform(1, 200000)
    if _rng.random() < 0.5:
        cols = max(4, cols - cols % 4)
    offset = int(_rng.choice([0, 0, 2]))
    pad = int(_rng.choice([0, 0, 4, 7]))
    ROWS_CASES.append((rows, cols, offset, pad, _loguniform(1, 40000)))


@pytest.mark.parametrize("rows,cols,offset,pad,chunk", ROWS_CASES)
def test_random_rows(orc, rows, cols, offset, pad, chunk):
    x = _view((rows, cols), offset, pad, seed=rows * 7 + cols, sigma=4.0)
    xn = x.contiguous().cpu().numpy()
    y = L.log_softmax_rows(x)
    s = L.softmax_rows(x)
    torch.cuda.synchronize()
    ref, lse = orc.log_softmax_rows(xn, want_y=True)
    tag = f"({rows},{cols}) off {offset} pad {pad}"
    compare(y.cpu().numpy(), ref, what="log_softmax " + tag)
    compare(s.cpu().numpy(), orc.softmax_rows(xn), atol=1e-37, rtol=1e-5, what="softmax " + tag)
    if offset == 0 and pad == 0:
        p = L.lse_rows_partial(x, chunk)
        got = L.lse_rows_merge(p)
        torch.cuda.synchronize()
        compare(got.cpu().numpy(), lse, what=f"partial/merge chunk {chunk} " + tag)


CHAIN_CASES = []
for i in range(10):
    CHAIN_CASES.append((int(_rng.integers(1, 4)), int(_rng.integers(3, 150)),
                        int(_rng.integers(3, 300)), int(_rng.choice([1, 2, 4, 8, 16])),
                        bool(_rng.random() < 0.5)))


@pytest.mark.parametrize("N,H,W,groups,affine", CHAIN_CASES)
def test_random_chain(orc, N, H, W, groups, affine):
    x, w, b, g, be = inputs.conv_chain_inputs(N=N, H=H, W=W, seed=N * 7919 + H * 31 + W,
                                              device=DEV)
    if affine:
        gen = inputs.generator(H + W, DEV)
        g = inputs.uniform((64,), 0.5, DEV, gen).add_(1.0)
        be = inputs.uniform((64,), 0.5, DEV, gen)
    out = L.fused_conv_gn_act_lse(x, w, b, g, be, groups, 1e-5)
    torch.cuda.synchronize()
    cpu = lambda t: None if t is None else t.cpu().numpy()
    ref, _, _ = orc.fused_chain(cpu(x), cpu(w), cpu(b), cpu(g), cpu(be), groups, 1e-5)
    compare(out.cpu().numpy(), ref, rtol=RTOL_CHAIN,
            what=f"chain N={N} H={H} W={W} G={groups} affine={affine}")
