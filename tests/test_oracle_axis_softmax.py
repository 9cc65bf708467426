"""Pins for the oracle's row softmax and its middle-axis logsumexp / log_softmax.

Independent checks: hand-worked closed forms, brute force without shift,
scipy.special (softmax, logsumexp, log_softmax over axis 1) and torch in
float64, sum-to-one, and the index layout checked element by element.
"""
import math

import numpy as np
import pytest
import scipy.special as sps
import torch


def test_softmax_closed_forms(orc):
    y = orc.softmax_rows(np.zeros((1, 4), np.float32))
    np.testing.assert_array_equal(y, 0.25)
    y = orc.softmax_rows(np.array([[0.0, -np.inf, 0.0]], np.float32))
    np.testing.assert_array_equal(y, [[0.5, 0.0, 0.5]])
    y = orc.softmax_rows(np.array([[0.0, 1.0]], np.float32))
    assert abs(y[0, 1] - math.e / (1 + math.e)) < 1e-15
    y = orc.softmax_rows(np.array([[1000.0, 1000.0]], np.float32))   # unshifted exp overflows
    np.testing.assert_allclose(y, 0.5, rtol=1e-12)   # L ~ 1000.69 carries ulp(1000) ~ 1e-13


@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 7), (5, 1000), (2, 4097)])
def test_softmax_vs_libraries(orc, rows, cols):
    rng = np.random.default_rng(rows * 31 + cols)
    x = rng.normal(scale=5, size=(rows, cols)).astype(np.float32)
    y = orc.softmax_rows(x)
    x64 = x.astype(np.float64)
    np.testing.assert_allclose(y.sum(axis=1), 1.0, atol=1e-12)
    np.testing.assert_allclose(y, sps.softmax(x64, axis=1), rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(y, torch.softmax(torch.from_numpy(x64), 1).numpy(), rtol=1e-12,
                               atol=1e-300)


def test_softmax_brute_force_and_special(orc):
    rng = np.random.default_rng(2)
    x = rng.uniform(-20, 20, size=(4, 50)).astype(np.float32)
    e = np.exp(x.astype(np.float64))
    np.testing.assert_allclose(orc.softmax_rows(x), e / e.sum(1, keepdims=True), rtol=1e-13)
    s = np.array([[-np.inf, -np.inf], [np.inf, 0.0], [np.nan, 0.0]], np.float32)
    y = orc.softmax_rows(s)
    assert np.isnan(y[0]).all()
    assert np.isnan(y[1, 0]) and y[1, 1] == 0.0
    assert np.isnan(y[2]).all()


@pytest.mark.parametrize("outer,R,inner", [(1, 4, 320), (3, 5, 7), (2, 64, 36), (4, 1, 9),
                                           (5, 33, 1)])
def test_lse_axis_layout_and_libraries(orc, outer, R, inner):
    rng = np.random.default_rng(outer * 100 + R * 10 + inner)
    x = rng.normal(scale=3, size=(outer, R, inner)).astype(np.float32)
    got = orc.lse_axis(x)
    assert got.shape == (outer, inner)
    x64 = x.astype(np.float64)
    np.testing.assert_allclose(got, sps.logsumexp(x64, axis=1), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(got, torch.logsumexp(torch.from_numpy(x64), 1).numpy(),
                               rtol=1e-13, atol=1e-13)
    for o in range(outer):                 # element by element: out[o, j] uses x[o, :, j]
        for j in range(inner):
            assert abs(got[o, j] - math.log(np.exp(x64[o, :, j]).sum())) < 1e-11


@pytest.mark.parametrize("outer,R,inner", [(3, 5, 7), (2, 64, 36), (1, 40, 100), (6, 2, 1)])
def test_log_softmax_axis(orc, outer, R, inner):
    rng = np.random.default_rng(outer + R + inner)
    x = rng.normal(scale=4, size=(outer, R, inner)).astype(np.float32)
    y = orc.log_softmax_axis(x)
    x64 = x.astype(np.float64)
    np.testing.assert_allclose(y, sps.log_softmax(x64, axis=1), rtol=1e-13, atol=1e-12)
    np.testing.assert_allclose(np.exp(y).sum(axis=1), 1.0, atol=1e-12)
    np.testing.assert_allclose(y, torch.log_softmax(torch.from_numpy(x64), 1).numpy(),
                               rtol=1e-13, atol=1e-12)
