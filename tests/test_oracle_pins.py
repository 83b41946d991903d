"""Pins of the CPU oracle against things other than itself: dense convolution
(torch CPU, fp64), brute-force neighbour search, numpy's unique, closed forms,
adjoint identities, autograd, and the two-voxel example of the torch-lattice
page "Migrating from TorchSparse" (section "Sparse tensor expectations").

Each pin is chosen so that a plausible slip in the oracle (a flipped offset
sign, a transposed weight, a dropped term, a wrong output order) fails it.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from convolution_voxelised_point_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers
def offsets(ndim, ksize):
    r = (ksize - 1) // 2
    return [tuple(d) for d in itertools.product(range(-r, ksize - r), repeat=ndim)]


def densify(coords, feats, lo, shape):
    """Dense [B][C][X][Y]([Z]) tensor holding feats at coords - lo."""
    coords = np.asarray(coords)
    B = int(coords[:, 0].max()) + 1 if len(coords) else 1
    C = feats.shape[1]
    d = torch.zeros((B, C) + tuple(shape), dtype=torch.float64)
    for i, c in enumerate(coords):
        idx = (int(c[0]), slice(None)) + tuple(int(v - l) for v, l in zip(c[1:], lo))
        d[idx] = torch.as_tensor(feats[i], dtype=torch.float64)
    return d


def dense_weight(w, ndim, ksize):
    """W[offset][cin][cout] -> torch weight [cout][cin][k..k]."""
    kvol, cin, cout = w.shape
    wd = torch.as_tensor(np.asarray(w, dtype=np.float64)).permute(2, 1, 0)
    return wd.reshape((cout, cin) + (ksize,) * ndim).contiguous()


def sample(dense, coords, lo):
    out = []
    for c in np.asarray(coords):
        idx = (int(c[0]), slice(None)) + tuple(int(v - l) for v, l in zip(c[1:], lo))
        out.append(dense[idx])
    return torch.stack(out).numpy() if out else np.zeros((0, dense.shape[1]))


def dense_conv(xd, wd, ndim, stride, padding):
    f = F.conv3d if ndim == 3 else F.conv2d
    return f(xd, wd, stride=stride, padding=padding)


def canon(tr):
    a = np.stack([np.asarray(t, dtype=np.int64) for t in tr], axis=1)
    return a[np.lexsort(a.T[::-1])] if len(a) else a.reshape(0, 3)


# ---------------------------------------------------------------- hash
def test_hash_query_vs_linear_scan():
    rng = np.random.default_rng(7)
    c = synth.random_coords(1, 300, 3, 3, 12, lo=-6)
    # add duplicates of rows 5 and 17 at the end
    c = np.concatenate([c, c[[5, 17]]], axis=0)
    q = np.concatenate([c, synth.random_coords(2, 200, 3, 4, 14, lo=-7)], axis=0)
    rows, flags = oracle.hash_query(c, q)
    for k, qq in enumerate(q):
        hits = np.nonzero(np.all(c == qq, axis=1))[0]
        assert rows[k] == (hits.min() if len(hits) else -1)
    assert flags & 1  # DUP
    assert not flags & 2
    del rng


def test_duplicate_and_range_rows_take_no_part():
    """A repeated or out-of-range row is never a neighbour and, as a
    submanifold output, has no neighbours; the relation stays symmetric."""
    c = synth.random_coords(5, 200, 3, 1, 6)
    bad = np.array([[0, 40000, 1, 1], [0, -40000, 0, 0]], np.int32)
    c2 = np.concatenate([c, c[[3, 10]], bad], axis=0)
    n = len(c)
    t_in, t_out, t_off = oracle.kmap(c2, c2, 3, 1)
    assert t_in.max() < n and t_out.max() < n
    assert canon((t_in, t_out, t_off)).tolist() == canon(oracle.kmap(c, c, 3, 1)).tolist()
    rng = np.random.default_rng(0)
    x = rng.standard_normal((len(c2), 2))
    w = rng.standard_normal((27, 2, 2))
    y = oracle.conv_fwd((t_in, t_out, t_off), x, w, len(c2))
    assert np.all(y[n:] == 0)


def test_hash_range_rows_not_inserted():
    c = np.array([[0, 0, 0, 0], [0, 40000, 0, 0], [70000, 1, 1, 1], [0, -32768, 32767, 5]], np.int32)
    rows, flags = oracle.hash_query(c, c)
    assert list(rows) == [0, -1, -1, 3]
    assert flags & 2 and not flags & 1


# ---------------------------------------------------------------- worked example
def test_two_voxel_example():
    g = json.load(open(os.path.join(GOLDEN, "two_voxel_example.json")))
    c = np.array(g["coords"], np.int32)
    tr = oracle.kmap(c, c, 3, 1)
    assert canon(tr).tolist() == canon(np.array(g["subm_k3"]["triples_in_out_offset"]).T).tolist()
    oc = oracle.strided_support(c, 2)
    assert oc.tolist() == g["strided_k2_s2"]["out_coords"]
    tr2 = oracle.kmap(c, oc, 2, 2)
    assert canon(tr2).tolist() == canon(np.array(g["strided_k2_s2"]["triples_in_out_offset"]).T).tolist()
    # features: closed forms y0 = x0 W13 + x1 W22, y1 = x1 W13 + x0 W4
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 16))
    w = rng.standard_normal((27, 16, 16))
    y = oracle.conv_fwd(tr, x, w, 2)
    np.testing.assert_allclose(y[0], x[0] @ w[13] + x[1] @ w[22], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(y[1], x[1] @ w[13] + x[0] @ w[4], rtol=1e-13, atol=1e-13)
    w2 = rng.standard_normal((8, 16, 32))
    y2 = oracle.conv_fwd(tr2, x, w2, 1)
    np.testing.assert_allclose(y2[0], x[0] @ w2[0] + x[1] @ w2[4], rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- kernel map
def brute_force_kmap(in_c, out_c, ksize, stride):
    """All-pairs search: (i, j, o) whenever in_i - stride*out_j is an offset."""
    ndim = in_c.shape[1] - 1
    offs = {d: o for o, d in enumerate(offsets(ndim, ksize))}
    res = []
    for j, q in enumerate(out_c):
        for i, p in enumerate(in_c):
            if p[0] != q[0]:
                continue
            d = tuple(int(p[k + 1]) - stride * int(q[k + 1]) for k in range(ndim))
            if d in offs:
                res.append((i, j, offs[d]))
    return np.array(res, np.int64).reshape(-1, 3)


@pytest.mark.parametrize("ndim,ksize,seed", [(3, 3, 0), (3, 1, 1), (2, 3, 2), (2, 5, 3), (3, 3, 4)])
def test_subm_kmap_brute_force(ndim, ksize, seed):
    c = synth.random_coords(seed, 600, ndim, 3, 9, lo=-4)
    tr = oracle.kmap(c, c, ksize, 1)
    bf = brute_force_kmap(c, c, ksize, 1)
    bf = bf[np.lexsort(bf.T[::-1])]
    assert canon(tr).tolist() == bf.tolist()


def test_subm_kmap_invariants():
    w = synth.make("tiny")
    c = w.coords
    t_in, t_out, t_off = oracle.kmap(c, c, 3, 1)
    kvol, centre = 27, 13
    n = c.shape[0]
    cen = t_off == centre
    assert np.array_equal(t_in[cen], t_out[cen]) and cen.sum() == n  # centre is identity
    fwd = set(zip(t_in.tolist(), t_out.tolist(), t_off.tolist()))
    assert all((j, i, kvol - 1 - o) in fwd for (i, j, o) in fwd)  # mirror symmetry
    assert np.all(c[t_in, 0] == c[t_out, 0])  # no cross-batch pairs
    # closed-form expectation of pairs for uniform sampling without replacement
    expect = n * (1 + 26 * (n - 1) / (64 ** 3 - 1))
    assert abs(len(t_in) - expect) < 6 * np.sqrt(expect)


@pytest.mark.parametrize("ndim,ksize,stride,seed", [(3, 2, 2, 0), (2, 2, 2, 1), (3, 3, 2, 2), (3, 2, 2, 3), (2, 3, 3, 4)])
def test_strided_kmap_brute_force(ndim, ksize, stride, seed):
    c = synth.random_coords(seed, 500, ndim, 2, 11, lo=-5)
    oc = oracle.strided_support(c, stride)
    tr = oracle.kmap(c, oc, ksize, stride)
    bf = brute_force_kmap(c, oc, ksize, stride)
    bf = bf[np.lexsort(bf.T[::-1])]
    assert canon(tr).tolist() == bf.tolist()


@pytest.mark.parametrize("ndim,stride", [(3, 2), (2, 2), (3, 3)])
def test_strided_support_unique_floor(ndim, stride):
    c = synth.random_coords(11 + ndim, 800, ndim, 3, 20, lo=-10)
    oc = oracle.strided_support(c, stride)
    q = np.concatenate([c[:, :1], np.floor_divide(c[:, 1:], stride)], axis=1)
    u, first = np.unique(q, axis=0, return_index=True)
    assert oc.shape == u.shape
    # first-occurrence order
    assert np.array_equal(oc, q[np.sort(first)])
    # partition property for k = s
    if stride == 2:
        t_in, t_out, t_off = oracle.kmap(c, oc, 2, 2)
        assert sorted(t_in.tolist()) == list(range(c.shape[0]))
        assert set(t_out.tolist()) == set(range(oc.shape[0]))


# ---------------------------------------------------------------- forward vs dense conv
@pytest.mark.parametrize("ndim,ksize,seed", [(3, 3, 0), (2, 3, 1), (3, 1, 2), (2, 5, 3)])
def test_subm_forward_vs_dense_conv(ndim, ksize, seed):
    rng = np.random.default_rng(seed)
    c = synth.random_coords(seed, 150, ndim, 2, 8, lo=-3)
    cin, cout = 5, 7
    x = rng.standard_normal((c.shape[0], cin))
    kvol = ksize ** ndim
    w = rng.standard_normal((kvol, cin, cout))
    y, _ = oracle.subm_conv(c, x, w, ksize)
    lo = (-3,) * ndim
    xd = densify(c, x, lo, (8,) * ndim)
    yd = dense_conv(xd, dense_weight(w, ndim, ksize), ndim, 1, (ksize - 1) // 2)
    np.testing.assert_allclose(y, sample(yd, c, lo), rtol=1e-12, atol=1e-12)


def test_subm_fully_active_block_equals_dense():
    rng = np.random.default_rng(5)
    g = np.stack(np.meshgrid(np.arange(5), np.arange(5), np.arange(5), indexing="ij"), -1).reshape(-1, 3)
    c = np.concatenate([np.zeros((len(g), 1), np.int64), g], 1).astype(np.int32)
    x = rng.standard_normal((len(c), 3))
    w = rng.standard_normal((27, 3, 4))
    y, _ = oracle.subm_conv(c, x, w, 3)
    xd = densify(c, x, (0, 0, 0), (5, 5, 5))
    yd = dense_conv(xd, dense_weight(w, 3, 3), 3, 1, 1)
    np.testing.assert_allclose(y, yd[0].permute(1, 2, 3, 0).reshape(-1, 4).numpy(), rtol=1e-12, atol=1e-12)


def test_pointwise_and_single_voxel():
    rng = np.random.default_rng(9)
    c = synth.random_coords(9, 200, 3, 2, 10)
    x = rng.standard_normal((len(c), 6))
    w1 = rng.standard_normal((1, 6, 3))
    y, _ = oracle.subm_conv(c, x, w1, 1)
    np.testing.assert_allclose(y, x @ w1[0], rtol=1e-13, atol=1e-13)
    w3 = rng.standard_normal((27, 6, 3))
    y1, _ = oracle.subm_conv(c[:1], x[:1], w3, 3)
    np.testing.assert_allclose(y1, x[:1] @ w3[13], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("ndim,ksize,stride,seed", [(3, 2, 2, 0), (2, 2, 2, 1), (3, 3, 2, 2)])
def test_strided_forward_vs_dense_conv(ndim, ksize, stride, seed):
    rng = np.random.default_rng(seed)
    ext = 12
    c = synth.random_coords(seed, 200, ndim, 2, ext, lo=0)
    cin, cout = 4, 6
    x = rng.standard_normal((c.shape[0], cin))
    w = rng.standard_normal((ksize ** ndim, cin, cout))
    oc, y, _ = oracle.strided_conv(c, x, w, ksize, stride)
    r = (ksize - 1) // 2
    # dense: y[q] = sum_delta w[delta + r] x[s q + delta]  (cross-correlation, padding r)
    xd = densify(c, x, (0,) * ndim, (ext,) * ndim)
    yd = dense_conv(xd, dense_weight(w, ndim, ksize), ndim, stride, r)
    np.testing.assert_allclose(y, sample(yd, oc, (0,) * ndim), rtol=1e-12, atol=1e-12)
    if ksize == stride:
        # the dense output is zero off the generated support
        mask = torch.zeros_like(yd, dtype=torch.bool)
        for q in oc:
            mask[(int(q[0]), slice(None)) + tuple(int(v) for v in q[1:])] = True
        assert float(yd[~mask].abs().max()) == 0.0


# ---------------------------------------------------------------- backward
@pytest.mark.parametrize("stride", [1, 2])
def test_adjoint_identities(stride):
    rng = np.random.default_rng(21 + stride)
    c = synth.random_coords(21, 400, 3, 2, 10, lo=-5)
    ksize = 3 if stride == 1 else 2
    oc = c if stride == 1 else oracle.strided_support(c, stride)
    tr = oracle.kmap(c, oc, ksize, stride)
    cin, cout = 5, 3
    x = rng.standard_normal((len(c), cin))
    g = rng.standard_normal((len(oc), cout))
    w = rng.standard_normal((ksize ** 3, cin, cout))
    y = oracle.conv_fwd(tr, x, w, len(oc))
    dx = oracle.conv_dgrad(tr, g, w, len(c))
    dw = oracle.conv_wgrad(tr, x, g, ksize ** 3)
    a, b, d = np.sum(y * g), np.sum(x * dx), np.sum(w * dw)
    assert abs(a - b) <= 1e-12 * max(1.0, abs(a)) and abs(a - d) <= 1e-12 * max(1.0, abs(a))


@pytest.mark.parametrize("ndim,ksize,stride", [(3, 3, 1), (2, 3, 1), (3, 2, 2)])
def test_backward_vs_dense_autograd(ndim, ksize, stride):
    rng = np.random.default_rng(31 + ndim + stride)
    ext = 8
    c = synth.random_coords(31 + ndim, 120, ndim, 2, ext, lo=0)
    cin, cout = 3, 4
    x = rng.standard_normal((len(c), cin))
    w = rng.standard_normal((ksize ** ndim, cin, cout))
    oc = c if stride == 1 else oracle.strided_support(c, stride)
    g = rng.standard_normal((len(oc), cout))
    tr = oracle.kmap(c, oc, ksize, stride)
    dx = oracle.conv_dgrad(tr, g, w, len(c))
    dw = oracle.conv_wgrad(tr, x, g, ksize ** ndim)
    # dense reference: loss = sum over output sites of <y[q], g[q]>
    xd = densify(c, x, (0,) * ndim, (ext,) * ndim).requires_grad_(True)
    wd = dense_weight(w, ndim, ksize).requires_grad_(True)
    pad = (ksize - 1) // 2 if stride == 1 else 0
    yd = dense_conv(xd, wd, ndim, stride, pad)
    gd = densify(oc, g, (0,) * ndim, tuple(yd.shape[2:]))
    if gd.shape[0] < yd.shape[0]:
        gd = torch.cat([gd, torch.zeros((yd.shape[0] - gd.shape[0],) + gd.shape[1:], dtype=gd.dtype)])
    (yd * gd).sum().backward()
    np.testing.assert_allclose(dx, sample(xd.grad, c, (0,) * ndim), rtol=1e-11, atol=1e-11)
    dw_ref = wd.grad.reshape(cout, cin, -1).permute(2, 1, 0).numpy()
    np.testing.assert_allclose(dw, dw_ref, rtol=1e-11, atol=1e-11)


def test_wgrad_finite_difference():
    rng = np.random.default_rng(41)
    c = synth.random_coords(41, 100, 3, 1, 6)
    tr = oracle.kmap(c, c, 3, 1)
    x = rng.standard_normal((len(c), 2))
    g = rng.standard_normal((len(c), 2))
    w = rng.standard_normal((27, 2, 2))
    dw = oracle.conv_wgrad(tr, x, g, 27)
    h = 1e-6
    for (o, a, b) in [(13, 0, 1), (4, 1, 0), (22, 1, 1)]:
        wp, wm = w.copy(), w.copy()
        wp[o, a, b] += h
        wm[o, a, b] -= h
        fd = (np.sum(oracle.conv_fwd(tr, x, wp, len(c)) * g) - np.sum(oracle.conv_fwd(tr, x, wm, len(c)) * g)) / (2 * h)
        assert abs(fd - dw[o, a, b]) < 1e-6 * max(1, abs(fd))
