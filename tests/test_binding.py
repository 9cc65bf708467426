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


def test_strided_axis_geometry():
    """Views map to (outer stride, R stride) with a contiguous inner run; the
    layouts the strided entry points cannot express raise instead of copying."""
    from log_softmax_reductions_amd import _strided_axis
    x = torch.empty(3, 6, 5, 8)
    assert _strided_axis(x, 1, "x") == (240, 40)
    assert _strided_axis(x, 0, "x") == (0, 240)            # no outer dims
    assert _strided_axis(x, 3, "x") == (8, 1)              # reduce the last dim
    assert _strided_axis(x[:, 1:5], 1, "x") == (240, 40)   # a slice of planes
    assert _strided_axis(x[:, :, 2], 1, "x") == (240, 40)  # a selected dim: (3, 6, 8)
    xp = torch.empty(3, 6, 48)[:, :, :40].view(3, 6, 40)   # padded plane pitch 48
    assert _strided_axis(xp, 1, "x") == (288, 48)
    assert _strided_axis(torch.empty(1, 6, 1, 8), 1, "x") == (0, 8)   # size-1 dims ignored
    with pytest.raises(ValueError, match="contiguous run"):
        _strided_axis(x[..., :6], 1, "x")                  # inner dims (5, 6) do not merge
    with pytest.raises(ValueError, match="contiguous run"):
        _strided_axis(x.transpose(2, 3), 1, "x")
    with pytest.raises(ValueError, match="one stride"):
        _strided_axis(x.transpose(0, 1), 2, "x")           # outer dims (6, 3) do not merge


def test_row_pitch():
    from log_softmax_reductions_amd import _ld
    assert _ld(torch.empty(4, 128)[:, :100], "x") == 128
    assert _ld(torch.empty(1, 100), "x") == 100
    with pytest.raises(ValueError, match="contiguous"):
        _ld(torch.empty(100, 4).t(), "x")


def test_tensors_must_share_one_gpu():
    from log_softmax_reductions_amd import _on
    with pytest.raises(ValueError, match="one GPU"):
        _on(torch.empty(2), torch.empty(2, device="meta"))
    with pytest.raises(ValueError, match="on the GPU"):
        _on(torch.empty(2), None)


def test_chain_and_merge_sizes_checked_before_the_call():
    """Buffers the library would read or write past their end are refused."""
    x, w = torch.zeros(2, 8, 10, 10), torch.zeros(64, 8, 3, 3)
    with pytest.raises(ValueError, match="b must have 64"):
        L.fused_conv_gn_act_lse(x, w, torch.zeros(32), None, None, 16)
    with pytest.raises(ValueError, match="gamma must have 64"):
        L.fused_conv_gn_act_lse(x, w, None, torch.zeros(65), None, 16)
    with pytest.raises(ValueError, match="out must have 128"):
        L.fused_conv_gn_act_lse(x, w, None, None, None, 16, out=torch.zeros(2, 1, 8, 7))
    with pytest.raises(ValueError, match="row_lse must have 3"):
        L.lse_rows_merge(torch.zeros(3, 4, 2), row_lse=torch.zeros(2))
