"""Pins of the oracle's sparse pooling (max and average over the inputs
present in each output's window) against torch's dense fp64 pooling: max
pooling of a grid holding -inf at empty sites, and average pooling of the
features divided by average pooling of the occupancy."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from convolution_voxelised_point_amd import synth
from test_oracle_pins import densify, sample


def dense_pool(xd, ndim, k, s, mode):
    if mode == "max":
        f = F.max_pool3d if ndim == 3 else F.max_pool2d
    else:
        f = F.avg_pool3d if ndim == 3 else F.avg_pool2d
    return f(xd, kernel_size=k, stride=s)


@pytest.mark.parametrize("ndim,k,s,seed", [(3, 2, 2, 0), (2, 2, 2, 1), (3, 3, 3, 2), (2, 4, 4, 3)])
@pytest.mark.parametrize("mode", ["max", "avg"])
def test_pool_vs_dense(ndim, k, s, seed, mode):
    """Window k = stride s (non-overlapping, the offsets {0..k-1} anchored at
    s*q for even k and {-r..r} for odd k: a dense window with the matching
    padding)."""
    rng = np.random.default_rng(seed)
    ext = 12
    r = (k - 1) // 2
    c = synth.random_coords(seed, 250, ndim, 2, ext - 2 * r, lo=r)
    x = rng.standard_normal((c.shape[0], 5))
    oc = oracle.strided_support(c, s)
    tr = oracle.kmap(c, oc, k, s)
    y = oracle.pool(tr, x, oc.shape[0], mode)
    # the dense window of output q starts at s*q - r
    pad = (r,) * (2 * ndim)
    if mode == "max":
        xd = densify(c, x, (0,) * ndim, (ext,) * ndim)
        occ = densify(c, np.ones((c.shape[0], 1)), (0,) * ndim, (ext,) * ndim) > 0
        xd = torch.where(occ.expand_as(xd), xd, torch.full_like(xd, -np.inf))
        xd = F.pad(xd, pad, value=-np.inf)
        yd = dense_pool(xd, ndim, k, s, "max")
    else:
        xd = F.pad(densify(c, x, (0,) * ndim, (ext,) * ndim), pad)
        occ = F.pad(densify(c, np.ones((c.shape[0], 1)), (0,) * ndim, (ext,) * ndim), pad)
        yd = dense_pool(xd, ndim, k, s, "avg") / dense_pool(occ, ndim, k, s, "avg")
    # a window with no input (possible when k = s is odd: the window of q is
    # s*q + {-r..r}, the support floor(c/s)) is 0 by definition
    yd = torch.nan_to_num(yd, nan=0.0, neginf=0.0)
    np.testing.assert_allclose(y, sample(yd, oc, (0,) * ndim), rtol=1e-12, atol=1e-12)
    if k == s == 2:
        assert np.all(np.bincount(tr[1], minlength=oc.shape[0]) > 0)  # k = s = 2: the window is the cell


def test_pool_special_cases():
    rng = np.random.default_rng(9)
    c = synth.random_coords(9, 300, 3, 2, 10)
    x = rng.standard_normal((c.shape[0], 4))
    # k = 1: pooling is the identity on the submanifold map
    tr = oracle.kmap(c, c, 1, 1)
    for mode in ("max", "avg"):
        np.testing.assert_array_equal(oracle.pool(tr, x, c.shape[0], mode), x)
    # an output with no inputs is 0; a single input is passed through
    t = np.array([[0, 100, 100, 100], c[0]], np.int32)
    tr = oracle.kmap(c, t, 3, 1, target=True)
    y = oracle.pool(tr, x, 2, "max")
    assert np.all(y[0] == 0.0)
    nb = tr[0][tr[1] == 1]
    np.testing.assert_array_equal(y[1], x[nb].max(axis=0))
    np.testing.assert_allclose(oracle.pool(tr, x, 2, "avg")[1], x[nb].mean(axis=0), rtol=1e-14)
