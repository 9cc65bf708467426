"""Pins for the oracle's chunk (max, sum) partials and their merge.

Chunk partials are checked element by element against a brute-force numpy
evaluation of their definition; merging any chunking must give the row's
logsumexp (itself pinned against scipy); the merge honours the identity
(-inf, 0) and is associative and commutative.
"""
import math

import numpy as np
import pytest
import scipy.special as sps


@pytest.mark.parametrize("chunk", [1, 7, 64, 100, 105, 1000])
def test_partials_brute_force(orc, chunk):
    rng = np.random.default_rng(chunk)
    x = rng.normal(scale=5, size=(3, 100)).astype(np.float32)
    m, s = orc.lse_chunk_partials(x, chunk)
    k = -(-100 // chunk)
    assert m.shape == (3, k)
    for r in range(3):
        for c in range(k):
            seg = x[r, c * chunk:min(100, (c + 1) * chunk)].astype(np.float64)
            assert m[r, c] == seg.max()
            assert abs(s[r, c] - np.exp(seg - seg.max()).sum()) <= 1e-13 * len(seg)


@pytest.mark.parametrize("chunk", [1, 7, 64, 333, 334, 5000])
def test_merge_of_any_chunking_is_row_lse(orc, chunk):
    rng = np.random.default_rng(42)
    x = rng.normal(scale=3, size=(6, 333)).astype(np.float32)
    m, s = orc.lse_chunk_partials(x, chunk)
    lse, M, S = orc.lse_merge(m, s)
    want = sps.logsumexp(x.astype(np.float64), axis=1)
    np.testing.assert_allclose(lse, want, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(M, x.max(axis=1).astype(np.float64))
    np.testing.assert_allclose(M + np.log(S), want, rtol=1e-13)


def test_merge_identity_and_empty_pairs(orc):
    ninf = -math.inf
    # (-inf, 0) (+) (-inf, 0) = (-inf, 0): no NaN from inf - inf or 0 * NaN
    lse, M, S = orc.lse_merge(np.array([[ninf, ninf]]), np.array([[0.0, 0.0]]))
    assert M[0] == ninf and S[0] == 0.0 and lse[0] == ninf
    # the identity leaves any pair unchanged
    lse, M, S = orc.lse_merge(np.array([[ninf, 2.0, ninf]]), np.array([[0.0, 3.0, 0.0]]))
    assert M[0] == 2.0 and S[0] == 3.0 and abs(lse[0] - (2.0 + math.log(3.0))) < 1e-15


def test_merge_many_empty_lanes(orc):
    """A reduction where most participants hold no data: 63 identity pairs and
    one real pair must give that pair back, whatever their order."""
    ninf = -math.inf
    m = np.full((1, 64), ninf)
    s = np.zeros((1, 64))
    m[0, 37], s[0, 37] = -1.5, 2.0
    lse, M, S = orc.lse_merge(m, s)
    assert M[0] == -1.5 and S[0] == 2.0


def test_merge_associative_commutative(orc):
    rng = np.random.default_rng(1)
    for _ in range(50):
        m = rng.normal(scale=20, size=3)
        s = rng.uniform(1, 100, size=3)
        whole, _, _ = orc.lse_merge(m[None], s[None])
        _, M12, S12 = orc.lse_merge(m[None, :2], s[None, :2])
        left, _, _ = orc.lse_merge(np.array([[M12[0], m[2]]]), np.array([[S12[0], s[2]]]))
        _, M23, S23 = orc.lse_merge(m[None, 1:], s[None, 1:])
        right, _, _ = orc.lse_merge(np.array([[m[0], M23[0]]]), np.array([[s[0], S23[0]]]))
        rev, _, _ = orc.lse_merge(m[None, ::-1].copy(), s[None, ::-1].copy())
        direct = math.log((s * np.exp(m - m.max())).sum()) + m.max()
        for v in (whole[0], left[0], right[0], rev[0]):
            assert abs(v - direct) < 1e-12 * max(1, abs(direct))


def test_partials_special_values(orc):
    x = np.array([[-np.inf, -np.inf, 1.0, 2.0, np.inf, np.inf, np.nan, 0.0]],
                 dtype=np.float32)
    m, s = orc.lse_chunk_partials(x, 2)
    assert m[0, 0] == -np.inf and s[0, 0] == 0.0
    assert m[0, 1] == 2.0 and abs(s[0, 1] - (1 + math.exp(-1))) < 1e-15
    assert m[0, 2] == np.inf and s[0, 2] == 2.0
    assert m[0, 3] == 0.0 and np.isnan(s[0, 3])
    lse, _, _ = orc.lse_merge(m[:, :3], s[:, :3])
    assert lse[0] == np.inf
    lse, _, _ = orc.lse_merge(m, s)
    assert np.isnan(lse[0])
