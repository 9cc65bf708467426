"""Host-side behaviour of the Python binding (no GPU needed): argument checks
raise before any library call, shapes map to the C ABI's (outer, R, inner)
views, and failures surface as LseError with the library's own message."""
import pytest
import torch

import log_softmax_reductions_amd as L


def test_rejects_host_tensors_and_wrong_dtypes():
    x = torch.zeros(4, 8)
    with pytest.raises(ValueError, match="GPU"):
        L.log_softmax_rows(x, y=torch.zeros(4, 8))
    with pytest.raises(ValueError, match="GPU"):
        L.lse_reduce_axis0(x, out=torch.zeros(8))
    with pytest.raises(ValueError, match="2-D"):
        L.softmax_rows(torch.zeros(2, 3, 4))
    with pytest.raises(ValueError, match="2-D"):
        L.lse_rows_partial(torch.zeros(8), 4)


def test_axis_view():
    from log_softmax_reductions_amd import _axis_view
    x = torch.empty(3, 6, 5, 8)
    assert _axis_view(x, 0) == (0, 1, 3, 240)
    assert _axis_view(x, 1) == (1, 3, 6, 40)
    assert _axis_view(x, -1) == (3, 90, 8, 1)


def test_library_errors_become_exceptions():
    from log_softmax_reductions_amd import _lib
    with pytest.raises(_lib.LseError, match="LSE_ERR_SHAPE"):
        _lib.check(_lib.load().lse_reduce_axis0(None, None, 0, 5, None), "lse_reduce_axis0")
    with pytest.raises(_lib.LseError, match="cols must be >= 1"):
        L.log_softmax_rows_plan(0)
    assert L.lse_rows_num_chunks(10, 3) == 4
