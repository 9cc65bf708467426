"""GPU parity of lse_reduce_axis0 (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import log_softmax_reductions_amd as L
from log_softmax_reductions_amd import inputs
from tests.parity import compare

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(x_dev):
    out = L.lse_reduce_axis0(x_dev)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_axis0_small_workload(orc):
    x = inputs.make("axis0_small", DEV)
    assert tuple(x.shape) == (4, 10, 32)
    got = _run(x)
    s = compare(got, orc.lse_axis0(x.cpu().numpy()), what="axis0_small")
    print("axis0_small", s)


@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 8, 9, 16, 17, 31, 32, 33, 70])
@pytest.mark.parametrize("inner", [1, 3, 4, 63, 64, 65, 1000, 4097])
def test_axis0_shapes(orc, R, inner):
    x = inputs.normal((R, inner), seed=R * 10007 + inner, sigma=3.0, device=DEV)
    compare(_run(x), orc.lse_axis0(x.cpu().numpy()), what=f"R={R} inner={inner}")


@pytest.mark.parametrize("offset", [1, 2, 3])
def test_axis0_misaligned_base(orc, offset):
    """A base pointer that is not 16-byte aligned takes the scalar path."""
    buf = inputs.normal((5 * 256 + offset,), seed=offset, device=DEV)
    x = buf[offset:].view(5, 256)
    assert x.data_ptr() % 16 != 0
    out = torch.empty(256 + 1, device=DEV)[1:]
    L.lse_reduce_axis0(x, out)
    torch.cuda.synchronize()
    compare(out.cpu().numpy(), orc.lse_axis0(x.cpu().numpy()), what="misaligned")


def test_axis0_special_values(orc):
    x = inputs.normal((6, 64), seed=9, device=DEV).cpu()
    x[:, 0] = -float("inf")                      # all -inf -> -inf
    x[2, 1] = float("inf")                       # +inf -> +inf
    x[3, 2] = float("nan")                       # NaN -> NaN
    x[1, 3], x[4, 3] = float("inf"), float("nan")
    x[:5, 4] = -float("inf")                     # single finite value -> itself
    x[:, 5] = 7.25                               # equal values -> v + log R
    x[0, 6] = 1e30                               # huge values stay finite
    x[1, 7] = -1e30
    got = _run(x.to(DEV))
    ref = orc.lse_axis0(x.numpy())
    compare(got, ref, what="special")
    assert got[0] == -np.inf and got[1] == np.inf and np.isnan(got[2]) and np.isnan(got[3])
    assert got[4] == x[5, 4].item()


def test_axis0_large_workload(orc):
    """(32, 2048, 4096) N(0, 4) — the 1 GiB leading-axis reduction, every output."""
    x = inputs.make("axis0_large", DEV)
    got = _run(x)
    ref = orc.lse_axis0(x.cpu().numpy())
    s = compare(got, ref, what="axis0_large")
    print("axis0_large", s)
    again = _run(x)
    assert np.array_equal(got, again, equal_nan=True), "run-to-run results differ"


def test_axis0_beyond_2g_elements(orc):
    """(3, 800_000_000): 2.4e9 elements (9.6 GB), past 32-bit element and byte
    offsets.  Sampled outputs, each from its own R values, against the oracle."""
    R, inner = 3, 800_000_000
    x = inputs.normal((R, inner), seed=44, sigma=3.0, device=DEV)
    out = L.lse_reduce_axis0(x)
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(7)
    idx = torch.cat([torch.tensor([0, 1, inner // 2, inner - 2, inner - 1]),
                     torch.randint(0, inner, (2000,), generator=gen)]).to(DEV)
    cols = x[:, idx].cpu().numpy()              # (R, samples)
    compare(out[idx].cpu().numpy(), orc.lse_axis0(cols), what="axis0 > 2^31 elements")
    del x, out
    torch.cuda.empty_cache()
