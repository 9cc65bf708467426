"""GPU parity of fused_conv_gn_act_lse (through the C ABI) against the fp64
oracle: tolerance |err| <= 1e-5 + 5e-4 |ref|."""
import math

import numpy as np
import pytest
import torch

import log_softmax_reductions_amd as L
from log_softmax_reductions_amd import inputs
from tests.parity import RTOL_CHAIN, compare

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _chain_inputs(N, H, W, seed, affine=False, bias=True):
    x, w, b, g, be = inputs.conv_chain_inputs(N=N, H=H, W=W, seed=seed, device=DEV)
    if affine:
        gen = inputs.generator(seed + 1, DEV)
        g = inputs.uniform((64,), 0.5, DEV, gen).add_(1.0)
        be = inputs.uniform((64,), 0.5, DEV, gen)
    return x, w, (b if bias else None), g, be


def _check(orc, x, w, b, g, be, groups, what):
    ws = torch.empty(L.fused_conv_gn_act_lse_workspace_bytes(x.shape[0], 8, x.shape[2],
                                                             x.shape[3], 64, 3, groups),
                     dtype=torch.uint8, device=DEV)
    out = L.fused_conv_gn_act_lse(x, w, b, g, be, groups, 1e-5, ws=ws)
    torch.cuda.synchronize()
    cpu = lambda t: None if t is None else t.cpu().numpy()
    ref, mean, rstd = orc.fused_chain(cpu(x), cpu(w), cpu(b), cpu(g), cpu(be), groups, 1e-5)
    s = compare(out.cpu().numpy(), ref, rtol=RTOL_CHAIN, what=what)
    NG = x.shape[0] * groups
    stats = ws[: 2 * NG * 4].view(torch.float32).cpu().numpy()
    compare(stats[:NG], mean.ravel(), atol=1e-6, rtol=1e-4, what=what + " mean")
    compare(stats[NG:], rstd.ravel(), atol=1e-6, rtol=1e-4, what=what + " rstd")
    return s


@pytest.mark.parametrize("N,H,W", [(2, 10, 10), (1, 3, 3), (3, 20, 20), (2, 7, 135),
                                   (1, 130, 131), (2, 9, 300)])
def test_chain_shapes(orc, N, H, W):
    x, w, b, g, be = _chain_inputs(N, H, W, seed=N * 1000 + H * 10 + W)
    _check(orc, x, w, b, g, be, 16, f"N={N} H={H} W={W}")


@pytest.mark.parametrize("groups", [1, 2, 4, 8, 16])
def test_chain_groups_and_affine(orc, groups):
    x, w, b, g, be = _chain_inputs(2, 12, 17, seed=groups, affine=True)
    _check(orc, x, w, b, g, be, groups, f"groups={groups}")


@pytest.mark.parametrize("N,H,W,groups", [(1, 600, 520, 1), (2, 260, 300, 4)])
def test_chain_many_tiles(orc, N, H, W, groups):
    """Samples with more statistics words than two per thread of a workgroup
    (1495 and 1548 words), across one and several tile columns and rows."""
    x, w, b, g, be = _chain_inputs(N, H, W, seed=H + W + groups, affine=True)
    _check(orc, x, w, b, g, be, groups, f"N={N} H={H} W={W} G={groups}")


def test_chain_no_bias_no_affine(orc):
    x, w, _, _, _ = _chain_inputs(2, 11, 11, seed=3)
    _check(orc, x, w, None, None, None, 16, "no bias")


def test_chain_full_workload(orc):
    """(128, 8, 128, 128) -> (128, 1, 126, 126): every output of the full
    workload against the oracle (one fp64 pass over the batch, a few seconds on
    the host's cores), plus the run-to-run identity."""
    x, w, b, g, be = inputs.make("conv_chain", DEV)
    N = x.shape[0]
    ws = torch.empty(L.fused_conv_gn_act_lse_workspace_bytes(N, 8, 128, 128, 64, 3, 16),
                     dtype=torch.uint8, device=DEV)
    out = L.fused_conv_gn_act_lse(x, w, b, g, be, 16, 1e-5, ws=ws)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (128, 1, 126, 126)
    oc = out.cpu().numpy()
    assert np.isfinite(oc).all()
    ref, mean, rstd = orc.fused_chain(x.cpu().numpy(), w.cpu().numpy(), b.cpu().numpy(),
                                      g.cpu().numpy(), be.cpu().numpy(), 16, 1e-5)
    s = compare(oc, ref, rtol=RTOL_CHAIN, what="conv_chain full workload")
    print("conv_chain full workload", s)
    stats = ws[: 2 * N * 16 * 4].view(torch.float32).cpu().numpy()
    compare(stats[:N * 16], mean.ravel(), atol=1e-6, rtol=1e-4, what="full workload mean")
    compare(stats[N * 16:], rstd.ravel(), atol=1e-6, rtol=1e-4, what="full workload rstd")
    # every pixel: LSE over 64 channels lies within [log 64 - 1, ...] of plausible range
    assert oc.min() > math.log(64) - 5 and oc.max() < math.log(64) + 10
    out2 = L.fused_conv_gn_act_lse(x, w, b, g, be, 16, 1e-5, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


def test_chain_nan_input_poisons_only_its_sample(orc):
    """A NaN in sample 1's input makes that sample's GroupNorm statistics NaN, so
    every output of sample 1 is NaN (as in the oracle) and the others are
    untouched."""
    x, w, b, g, be = _chain_inputs(3, 12, 12, seed=21)
    x[1, 3, 5, 7] = float("nan")
    ws = torch.empty(L.fused_conv_gn_act_lse_workspace_bytes(3, 8, 12, 12, 64, 3, 16),
                     dtype=torch.uint8, device=DEV)
    out = L.fused_conv_gn_act_lse(x, w, b, g, be, 16, 1e-5, ws=ws)
    torch.cuda.synchronize()
    oc = out.cpu().numpy()
    cpu = lambda t: t.cpu().numpy()
    ref, _, _ = orc.fused_chain(cpu(x), cpu(w), cpu(b), cpu(g), cpu(be), 16, 1e-5)
    assert np.isnan(ref[1]).all() and np.isfinite(ref[[0, 2]]).all()
    compare(oc, ref, rtol=RTOL_CHAIN, what="nan sample")
    err_word = ws[256 * ((2 * 3 * 16 * 4 + 255) // 256) + 4:][:4].view(torch.int32).item()
    assert err_word == 0          # the wait itself completed normally


def test_chain_zero_input_is_log_of_channel_count():
    """x = 0 without bias: the conv is 0, every group has variance 0, so the
    normalised value is 0, tanh 0 = 0, hardswish 0 = 0, and each output is the
    LSE of 64 zeros, log 64; the statistics are mean 0, rstd 1/sqrt(eps)."""
    x, w, _, _, _ = _chain_inputs(2, 9, 140, seed=8)
    x.zero_()
    ws = torch.empty(L.fused_conv_gn_act_lse_workspace_bytes(2, 8, 9, 140, 64, 3, 16),
                     dtype=torch.uint8, device=DEV)
    out = L.fused_conv_gn_act_lse(x, w, None, None, None, 16, 1e-5, ws=ws)
    torch.cuda.synchronize()
    oc = out.cpu().numpy().astype(np.float64)
    assert np.abs(oc - math.log(64)).max() <= 1e-6
    stats = ws[: 2 * 2 * 16 * 4].view(torch.float32).cpu().numpy().astype(np.float64)
    assert (stats[:32] == 0).all()
    assert np.abs(stats[32:] - 1 / math.sqrt(1e-5)).max() <= 1e-4 * 316.3


@pytest.mark.parametrize("scale", [1e3, 1e-3, -50.0])
def test_chain_input_scales(orc, scale):
    """Inputs far from unit scale: large conv values (the LSE shift carries
    them), tiny ones (GroupNorm rescales them), and a sign flip."""
    x, w, b, g, be = _chain_inputs(2, 12, 70, seed=int(abs(scale) * 7) + 1, affine=True)
    x.mul_(scale)
    _check(orc, x, w, b, g, be, 8, f"scale {scale}")


def test_chain_constant_input(orc):
    """A constant image: each channel's conv is one value over all pixels, so a
    group's variance is that of its 4 channel values."""
    x, w, _, _, _ = _chain_inputs(1, 10, 40, seed=9)
    x.fill_(0.75)
    _check(orc, x, w, None, None, None, 16, "constant input")


def _deferred_word(ws, N, groups):
    head = (2 * N * groups * 4 + 255) // 256 * 256
    return int(ws[head + 4: head + 8].view(torch.int32).item())


@pytest.mark.parametrize("N,H,W,groups", [(2, 128, 128, 16), (3, 37, 300, 4), (1, 600, 520, 1)])
def test_chain_deferred_pairs(orc, N, H, W, groups):
    """With the test hook's poll limit at 0 no workgroup waits: each one whose
    sample has not fully arrived defers its tile pair, and the sample's last
    arrival finishes those pairs (the path a workgroup takes when its wait
    runs out).  Outputs and statistics against the oracle, bit-equality with
    the default path, and the deferred count: at least one pair per sample
    (the first arrival cannot see the whole sample), never a sample's last
    arrival.  Shapes: two config-sized samples, a ragged one (odd tile rows,
    three tile columns), and a sample of 748 tile pairs forced through the
    fused launch (by default it takes the two-launch path, which never
    waits and so never defers: checked last)."""
    x, w, b, g, be = _chain_inputs(N, H, W, seed=7 * N + H + W, affine=True)
    pairs = N * ((((H - 2) + 1) // 2 * ((W - 2 + 127) // 128) + 1) // 2)
    ws = torch.empty(L.fused_conv_gn_act_lse_workspace_bytes(N, 8, H, W, 64, 3, groups),
                     dtype=torch.uint8, device=DEV)
    try:
        L.lse_testing_set_spin_limit(0)
        L.lse_testing_set_chain_path(1)
        out = L.fused_conv_gn_act_lse(x, w, b, g, be, groups, 1e-5, ws=ws)
        torch.cuda.synchronize()
    finally:
        L.lse_testing_set_spin_limit(1 << 24)
        L.lse_testing_set_chain_path(0)
    deferred = _deferred_word(ws, N, groups)
    assert N <= deferred <= pairs - N, (deferred, pairs)
    print("pairs deferred:", deferred, "of", pairs)
    NG = N * groups
    stats = ws[: 2 * NG * 4].view(torch.float32).clone()
    cpu = lambda t: None if t is None else t.cpu().numpy()
    ref, mean, rstd = orc.fused_chain(cpu(x), cpu(w), cpu(b), cpu(g), cpu(be), groups, 1e-5)
    compare(out.cpu().numpy(), ref, rtol=RTOL_CHAIN, what="deferred")
    compare(stats[:NG].cpu().numpy(), mean.ravel(), atol=1e-6, rtol=1e-4, what="deferred mean")
    compare(stats[NG:].cpu().numpy(), rstd.ravel(), atol=1e-6, rtol=1e-4, what="deferred rstd")
    ws2 = torch.empty(L.fused_conv_gn_act_lse_workspace_bytes(N, 8, H, W, 64, 3, groups),
                      dtype=torch.uint8, device=DEV)
    try:
        L.lse_testing_set_spin_limit(0)        # the default path at a poll limit of 0
        out2 = L.fused_conv_gn_act_lse(x, w, b, g, be, groups, 1e-5, ws=ws2)
        torch.cuda.synchronize()
    finally:
        L.lse_testing_set_spin_limit(1 << 24)
    if H == 600:                               # two launches: nothing waits, nothing deferred
        assert _deferred_word(ws2, N, groups) == 0
    assert torch.equal(out, out2)
    assert torch.equal(stats, ws2[: 2 * NG * 4].view(torch.float32))


@pytest.mark.parametrize("N,H,W,groups", [(3, 128, 128, 16), (2, 37, 300, 4), (1, 600, 520, 1),
                                          (2, 5, 7, 2)])
def test_chain_paths_agree(orc, N, H, W, groups):
    """The fused launch, the statistics + recomputing apply launches and the
    statistics + staged apply launches (forced through the test hook) against
    the oracle, and bit-identical to each other."""
    x, w, b, g, be = _chain_inputs(N, H, W, seed=3 * N + H + 5 * W, affine=True)
    outs = {}
    try:
        for path in (1, 2, 3):
            L.lse_testing_set_chain_path(path)
            nbytes = L.fused_conv_gn_act_lse_workspace_bytes(N, 8, H, W, 64, 3, groups)
            ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
            outs[path] = L.fused_conv_gn_act_lse(x, w, b, g, be, groups, 1e-5, ws=ws)
            torch.cuda.synchronize()
    finally:
        L.lse_testing_set_chain_path(0)
    cpu = lambda t: None if t is None else t.cpu().numpy()
    ref, _, _ = orc.fused_chain(cpu(x), cpu(w), cpu(b), cpu(g), cpu(be), groups, 1e-5)
    compare(outs[3].cpu().numpy(), ref, rtol=RTOL_CHAIN, what="staged")
    assert torch.equal(outs[1], outs[2])
    assert torch.equal(outs[1], outs[3])


def test_chain_staged_workspace_size():
    """The staged path's workspace holds one 128 KiB staging slot per tile pair
    of a batch of samples (at most 192 MiB), beyond the other paths' bytes."""
    try:
        L.lse_testing_set_chain_path(2)
        base = L.fused_conv_gn_act_lse_workspace_bytes(8, 8, 600, 520, 64, 3, 1)
        L.lse_testing_set_chain_path(3)
        staged = L.fused_conv_gn_act_lse_workspace_bytes(8, 8, 600, 520, 64, 3, 1)
    finally:
        L.lse_testing_set_chain_path(0)
    pairs = (299 * 5 + 1) // 2                      # 748 tile pairs per 600 x 520 sample
    per_batch = (192 << 20) // (pairs * 131072)     # 2 samples of 93.5 MiB
    assert per_batch == 2
    assert base < staged <= base + 256 + per_batch * pairs * 131072
    assert staged >= base + per_batch * pairs * 131072
