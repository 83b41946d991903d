"""GPU parity at the edges of the method: voxels whose kernel windows cross
the packable coordinate range (spatial values -32768 and 32767, batch 0 and
65534), and pointwise convolutions (kernel size 1, torch-lattice migration
page, "Convolution mapping": a kernel-size-1 Conv3d keeps the support).
Kernel maps are compared with the oracle as sorted triples, features over
every element."""
import numpy as np
import pytest
import torch

import oracle
from convolution_voxelised_point_amd import synth
from helpers import assert_feature_close, canon, dev

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def limit_coords_3d(seed=71):
    """Partly filled 4x4x4 blocks at the eight corners of the spatial range,
    in batch 0 and in batch 65534, rows shuffled."""
    rng = np.random.default_rng(seed)
    cube = np.stack(np.meshgrid(np.arange(4), np.arange(4), np.arange(4), indexing="ij"), -1).reshape(-1, 3)
    parts = []
    for b in (0, 65534):
        for cx in (-32768, 32764):
            for cy in (-32768, 32764):
                for cz in (-32768, 32764):
                    pts = cube[rng.random(64) < 0.6] + np.array([cx, cy, cz])
                    parts.append(np.c_[np.full(len(pts), b), pts])
    c = np.concatenate(parts).astype(np.int32)
    return c[rng.permutation(len(c))]


def limit_coords_2d(seed=72):
    rng = np.random.default_rng(seed)
    sq = np.stack(np.meshgrid(np.arange(8), np.arange(8), indexing="ij"), -1).reshape(-1, 2)
    parts = []
    for b in (0, 65534):
        for cx in (-32768, 32760):
            for cy in (-32768, 32760):
                pts = sq[rng.random(64) < 0.5] + np.array([cx, cy])
                parts.append(np.c_[np.full(len(pts), b), pts])
    c = np.concatenate(parts).astype(np.int32)
    return c[rng.permutation(len(c))]


def gpu_map(ts, coords, ksize, stride, flags):
    cd = dev(coords)
    tab = ts.HashTable(cd, 2.0)
    if stride == 1:
        return ts.build_kmap(cd, tab, ksize, 1, flags), coords
    out, n_out, otab = ts.strided_support(cd, stride)
    km = ts.build_kmap(cd, tab, ksize, stride, flags | ts.TS_KMAP_BWD, out_coords=out, n_out=n_out, out_table=otab)
    m = km.n_out()
    return km, out[:m].cpu().numpy()


LIMIT_MAPS = [
    ("3d_k3", limit_coords_3d, 3, 1),
    ("3d_k2s2", limit_coords_3d, 2, 2),
    ("2d_k3", limit_coords_2d, 3, 1),
    ("2d_k5", limit_coords_2d, 5, 1),
]


@pytest.mark.parametrize("natural", [False, True], ids=["sorted", "natural"])
@pytest.mark.parametrize("case", LIMIT_MAPS, ids=[c[0] for c in LIMIT_MAPS])
def test_kmap_at_packing_limits(ts, case, natural):
    _, make, k, s = case
    coords = make()
    flags = ts.TS_KMAP_PAIRS | (ts.TS_KMAP_NATURAL if natural else 0)
    km, oc = gpu_map(ts, coords, k, s, flags)
    if s > 1:
        assert np.array_equal(oc, oracle.strided_support(coords, s))
    tr = oracle.kmap(coords, oc, k, s)
    assert len(tr[0]) > 0
    kvol = k ** (coords.shape[1] - 1)
    got = ts.decode_rel(km.rel_arrays("fwd"), kvol)
    assert np.array_equal(canon(got), canon(tr))
    ps, pin, pout = km.pairs()
    off = np.repeat(np.arange(kvol, dtype=np.int32), np.diff(ps))
    assert np.array_equal(canon((pin, pout, off)), canon(tr))


LIMIT_CONV = [
    # name, coords, ksize, stride, cin, cout, dtype
    ("3d_k3_f16_64", limit_coords_3d, 3, 1, 64, 64, "f16"),
    ("3d_k3_f32_16", limit_coords_3d, 3, 1, 16, 16, "f32"),
    ("3d_k2s2_bf16_32x64", limit_coords_3d, 2, 2, 32, 64, "bf16"),
    ("2d_k3_f16_1x8", limit_coords_2d, 3, 1, 1, 8, "f16"),
]


@pytest.mark.parametrize("dataflow", ["auto", "gather_scatter"])
@pytest.mark.parametrize("case", LIMIT_CONV, ids=[c[0] for c in LIMIT_CONV])
def test_conv_at_packing_limits(ts, case, dataflow):
    name, make, k, s, cin, cout, dt = case
    coords = make()
    km, oc = gpu_map(ts, coords, k, s, ts.TS_KMAP_PAIRS)
    tr = oracle.kmap(coords, oc, k, s)
    kvol = k ** (coords.shape[1] - 1)
    x = synth.normal(810, (coords.shape[0], cin), 1.0, dt)
    w = synth.weight(811, kvol, cin, cout, dt)
    dy = synth.normal(812, (oc.shape[0], cout), 1.0, dt)
    df = ts.TS_DATAFLOW_AUTO if dataflow == "auto" else ts.TS_DATAFLOW_GATHER_SCATTER
    y = ts.conv_fwd(km, dev(x), dev(w), out_dtype=torch.float32, dataflow=df)
    assert_feature_close(y[:oc.shape[0]], oracle.conv_fwd(tr, x, w, oc.shape[0]), DT[dt], f"limits {name} fwd")
    dx = ts.conv_dgrad(km, dev(dy), dev(w), out_dtype=torch.float32, dataflow=df)
    assert_feature_close(dx, oracle.conv_dgrad(tr, dy, w, coords.shape[0]), DT[dt], f"limits {name} dgrad")
    dw = ts.conv_wgrad(km, dev(x), dev(dy))
    assert_feature_close(dw, oracle.conv_wgrad(tr, x, dy, kvol), DT[dt], f"limits {name} wgrad")


POINTWISE = [
    # name, coords, cin, cout, dtype
    ("lidar_f16_64", synth.make("lidar", scale=0.04).coords, 64, 64, "f16"),
    ("lidar_bf16_128x64", synth.make("lidar", scale=0.03).coords, 128, 64, "bf16"),
    ("fuzz_f32_16x24", synth.random_coords(17, 1200, 3, 2, 14, lo=-7), 16, 24, "f32"),
    ("pixels_f16_1x8", synth.make("pixels", scale=0.02).coords, 1, 8, "f16"),
]


@pytest.mark.parametrize("dataflow", ["auto", "implicit_gemm", "gather_scatter"])
@pytest.mark.parametrize("case", POINTWISE, ids=[c[0] for c in POINTWISE])
def test_pointwise_conv(ts, case, dataflow):
    """Kernel size 1: one offset, the identity relation; y = x W[0] row by
    row (the oracle, and a plain fp64 matrix product as a second check)."""
    name, coords, cin, cout, dt = case
    df = {"auto": ts.TS_DATAFLOW_AUTO, "implicit_gemm": ts.TS_DATAFLOW_IMPLICIT_GEMM,
          "gather_scatter": ts.TS_DATAFLOW_GATHER_SCATTER}[dataflow]
    km, _ = gpu_map(ts, coords, 1, 1, ts.TS_KMAP_PAIRS)
    tr = oracle.kmap(coords, coords, 1, 1)
    n = coords.shape[0]
    assert np.array_equal(canon(ts.decode_rel(km.rel_arrays("fwd"), 1)), canon(tr))
    x = synth.normal(820, (n, cin), 1.0, dt)
    w = synth.weight(821, 1, cin, cout, dt)
    y = ts.conv_fwd(km, dev(x), dev(w), out_dtype=torch.float32, dataflow=df)
    ref = oracle.conv_fwd(tr, x, w, n)
    assert_feature_close(y, ref, DT[dt], f"pointwise {name} ({dataflow})")
    mm = x.double().numpy() @ w[0].double().numpy()
    np.testing.assert_allclose(ref, mm, rtol=1e-12, atol=1e-12)
    dy = synth.normal(822, (n, cout), 1.0, dt)
    dx = ts.conv_dgrad(km, dev(dy), dev(w), out_dtype=torch.float32, dataflow=df)
    assert_feature_close(dx, oracle.conv_dgrad(tr, dy, w, n), DT[dt], f"pointwise {name} dgrad ({dataflow})")
