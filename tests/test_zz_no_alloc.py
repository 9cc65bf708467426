"""log_softmax_rows_noalloc (static device scratch, no allocation) through the
C ABI against log_softmax_rows (caller workspace) on the same inputs: two calls
in a row, the second smaller, each bit-identical to the workspace call (same
kernels, same chunking) and within tolerance of the oracle on sampled rows."""
import ctypes

import pytest
import torch

import log_softmax_reductions_amd as L
from log_softmax_reductions_amd import _lib, inputs
from tests.parity import compare

pytestmark = pytest.mark.gpu
DEV = "cuda"
LSE_ERR_WORKSPACE = 3


def _both(orc, rows, cols, seed, sample):
    x = inputs.normal((rows, cols), seed=seed, device=DEV)
    y_ref = L.log_softmax_rows(x)
    y = torch.full_like(x, float("nan"))
    L.log_softmax_rows_noalloc(x, y)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref), (rows, cols)
    ref, _ = orc.log_softmax_rows(x[sample].cpu().numpy())
    compare(y[sample].cpu().numpy(), ref, what=f"noalloc {rows}x{cols}")


def test_noalloc_two_calls_second_smaller(orc):
    print("case: noalloc (4096, 393216) then (300, 100003) then (64, 4096)", flush=True)
    _both(orc, 4096, 393216, seed=4, sample=[0, 1, 2047, 4095])
    _both(orc, 300, 100003, seed=91, sample=[0, 150, 299])   # 4 chunks, scalar path
    _both(orc, 64, 4096, seed=92, sample=[0, 63])            # one chunk: no scratch used


def test_noalloc_long_rows_three_launches(orc):
    """Rows of more than 128 chunks (three launches; tile pairs and the per-row
    (M, log S) in the scratch), then a shorter split row."""
    print("case: noalloc (2, 4500001) then (3, 300000)", flush=True)
    _both(orc, 2, 4500001, seed=93, sample=[0, 1])
    _both(orc, 3, 300000, seed=94, sample=[0, 2])


def test_noalloc_rejects_more_pairs_than_the_scratch():
    """10921 rows of 393216 columns need 131052 pairs, 12 more than the static
    scratch holds: refused before anything is launched."""
    lib = _lib.load()
    st = lib.log_softmax_rows_noalloc(ctypes.c_void_p(0x100000), ctypes.c_void_p(0x9000000000),
                                      10921, 393216, None)
    assert st == LSE_ERR_WORKSPACE
    assert b"131040" in lib.lse_last_error()
