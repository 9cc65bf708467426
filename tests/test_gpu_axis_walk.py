"""GPU parity of the plane-walk logsumexp (many wide aligned planes: R >= 33,
at least 512 tiles of 8192 outputs, or of 4096 when 8192 give too few)
through the C ABI against the fp64 oracle.

The walk sums each lane's columns against one reference value and redoes a
lane exactly when a sum leaves its safe window, so these cases place columns
far below and above their lane's reference, non-finite values in every
position the reference can see, ragged last tiles, several outer slices,
strided planes and offsets past 2^31 elements.
"""
import numpy as np
import pytest
import torch

import log_softmax_reductions_amd as L
from log_softmax_reductions_amd import inputs
from tests.parity import compare

pytestmark = pytest.mark.gpu
DEV = "cuda"
TILE = 8192            # outputs per workgroup of the walk
NARROW = 4 * 1024 * 1024


def _lse(x):
    out = L.lse_reduce_axis(x, 1)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("outer,R,inner", [
    (1, 40, NARROW),                  # 512 full tiles
    (1, 33, NARROW + 4 * 37),         # ragged last tile (148 outputs)
    (2, 48, 256 * TILE + TILE // 2),  # two outer slices, ragged tiles
    (1, 100, 513 * TILE - 4),         # last tile one vector short
    (128, 64, 126 * 126),             # half-width tiles: the channel layout, ragged per slice
    (128, 64, 16384),                 # half-width tiles, full
])
def test_walk_shapes(orc, outer, R, inner):
    x = inputs.normal((outer, R, inner), seed=outer * 131 + R * 7 + inner % 1000, sigma=2.0,
                      device=DEV)
    got = _lse(x)
    ref = orc.lse_axis(x.cpu().numpy())
    print(compare(got.cpu().numpy(), ref, what=f"walk {outer}x{R}x{inner}"))
    again = _lse(x)
    assert torch.equal(got, again), "run-to-run results differ"


def test_walk_strided_planes(orc):
    """Planes with a padded pitch (the strided instantiation)."""
    R, inner = 36, NARROW
    big = inputs.normal((R, inner + 64), seed=77, device=DEV)
    x = big[:, :inner].unsqueeze(0)            # (1, R, inner), plane stride inner + 64
    out = torch.empty(inner + 8, device=DEV)[4:4 + inner]
    L.lse_reduce_axis(x, 1, out.view(1, inner))
    torch.cuda.synchronize()
    ref = orc.lse_axis(x.contiguous().cpu().numpy()).ravel()
    compare(out.cpu().numpy(), ref, what="walk strided")


def test_walk_special_values_and_exact_redo(orc):
    R, inner = 36, NARROW + 4 * 5              # ragged last tile as well
    x = inputs.normal((1, R, inner), seed=91, device=DEV).cpu()
    inf, nan = float("inf"), float("nan")
    x[0, :, 0] = -inf                          # all -inf -> -inf
    x[0, 4, 1] = inf                           # +inf -> +inf
    x[0, 9, 2] = nan                           # NaN -> NaN
    x[0, 3, 3] = 1e30                          # huge value -> itself
    x[0, :, 5] -= 200.0                        # far below the lane's reference
    x[0, 7, 9] = 60.0                          # far above it
    x[0, 0, 2048:4096] = -inf                  # whole waves see plane 0 at -inf
    x[0, 0, 5000] = inf                        # a lane whose reference is +inf
    x[0, 0, 6001] = nan                        # NaN in plane 0
    x[0, :, 7000:7004] += 1000.0               # one vector offset by +1000
    x[0, 1:, 9000] = -inf                      # a single finite value -> itself
    x[0, :, -1] = 7.25                         # equal values -> v + log R (last column)
    x[0, 5, -3] = -inf                         # -inf in the ragged tile
    got = _lse(x.to(DEV)).cpu().numpy().ravel()
    ref = orc.lse_axis(x.numpy()).ravel()
    compare(got, ref, what="walk special")
    assert got[0] == -np.inf and got[1] == np.inf and np.isnan(got[2])
    assert got[5000] == np.inf and np.isnan(got[6001])
    # Against a reference other than the column's own max the closed forms hold
    # to the tolerance, not bit for bit.
    v = x[0, 0, 9000].item()
    assert abs(got[9000] - v) <= 1e-5 + 2e-6 * abs(v)
    assert abs(got[-1] - (7.25 + np.log(R))) <= 1e-5 + 2e-6 * 7.25


def test_walk_beyond_2g_elements(orc):
    """(40, 60_000_000): 2.4e9 elements (9.6 GB), plane offsets past 2^31
    elements and a ragged last tile; sampled outputs against the oracle."""
    R, inner = 40, 60_000_000
    x = inputs.normal((R, inner), seed=45, sigma=2.0, device=DEV)
    out = L.lse_reduce_axis0(x)
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(8)
    idx = torch.cat([torch.tensor([0, 1, 8191, 8192, inner // 2, inner - 5, inner - 1]),
                     torch.randint(0, inner, (2000,), generator=gen)]).to(DEV)
    cols = x[:, idx].cpu().numpy()
    compare(out[idx].cpu().numpy(), orc.lse_axis0(cols), what="walk > 2^31 elements")
    del x, out
    torch.cuda.empty_cache()


def test_walk_half_tiles_special_values(orc):
    """Half-width tiles (4096 outputs) on the channel layout with non-finite
    values and columns that leave the reference window."""
    x = inputs.normal((128, 64, 126 * 126), seed=93, device=DEV).cpu()
    inf, nan = float("inf"), float("nan")
    x[0, :, 0] = -inf
    x[1, 9, 4095] = inf                        # last column of a tile
    x[2, 0, 4096] = nan                        # first column of the next, in plane 0
    x[3, :, 15875] -= 300.0                    # last column of the slice, far below
    x[127, 5, 100] = 90.0                      # far above
    got = _lse(x.to(DEV)).cpu().numpy()
    ref = orc.lse_axis(x.numpy())
    compare(got, ref, what="walk half tiles special")
    assert got[0, 0] == -np.inf and got[1, 4095] == np.inf and np.isnan(got[2, 4096])


def test_walk_half_tiles_strided(orc):
    """Half-width tiles through the strided instantiation: padded planes (pitch
    15880 for 15876 columns) and a slice of the reduced axis (outer stride
    66 x 15880), output into a padded buffer."""
    big = inputs.normal((128, 66, 15880), seed=94, device=DEV)
    x = big[:, 1:65, :15876]                   # (128, 64, 15876)
    obuf = torch.empty(128, 15880, device=DEV)
    out = obuf[:, :15876]
    L.lse_reduce_axis(x, 1, out)
    torch.cuda.synchronize()
    ref = orc.lse_axis(x.contiguous().cpu().numpy())
    compare(out.cpu().numpy(), ref, what="walk half tiles strided")


@pytest.mark.parametrize("outer,R,inner,off", [
    (1, 40, NARROW, 1),               # every plane at a 4-byte phase
    (1, 33, NARROW + 4 * 37 + 3, 0),  # inner % 4 == 3: the last vector straddles the end
    (2, 48, 256 * TILE + 1025, 2),    # both, two outer slices
    (128, 64, 126 * 126 + 1, 3),      # half-width tiles, ragged per slice
])
def test_walk_off_grid(orc, outer, R, inner, off):
    """The walk with 16-byte accesses at 4-byte alignment: x and the output at
    another 4-byte phase and inner not a multiple of 4 (the run's last vector
    re-reads the last 4 columns and writes only its own); guard values around
    the output."""
    n = outer * R * inner
    buf = inputs.normal((n + 4,), seed=outer * 17 + R + inner % 997, sigma=2.0, device=DEV)
    x = buf[off:off + n].view(outer, R, inner)
    big = torch.full((outer * inner + 8,), 5.0, device=DEV)
    out = big[off:off + outer * inner].view(outer, inner)
    L.lse_reduce_axis(x, 1, out)
    torch.cuda.synchronize()
    compare(out.cpu().numpy(), orc.lse_axis(x.cpu().numpy()), what=f"walk off-grid {outer}x{R}x{inner}+{off}")
    assert torch.all(big[:off] == 5.0) and torch.all(big[off + outer * inner:] == 5.0)


def test_walk_off_grid_exact_redo(orc):
    """The exact redo on the straddling vector of an off-grid run."""
    R, inner = 36, NARROW + 4 * 5 + 2
    x = inputs.normal((1, R, inner), seed=93, device=DEV).cpu()
    x[0, :, -1] -= 300.0                       # last column far below its lane's reference
    x[0, 3, -2] = float("inf")
    x[0, :, 11] += 500.0
    buf = torch.empty(R * inner + 1, device=DEV)
    xd = buf[1:].view(1, R, inner)
    xd.copy_(x.to(DEV))
    got = _lse(xd).cpu().numpy().ravel()
    compare(got, orc.lse_axis(x.numpy()).ravel(), what="walk off-grid redo")
