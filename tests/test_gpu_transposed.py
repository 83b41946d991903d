"""GPU parity of the transposed convolutions against the CPU oracle:
ConvTranspose over an existing (strided or submanifold) relation, the
generated transposed support (coordinates and order bit-exact), the
transposed kernel map, and the forward, dgrad and wgrad over it."""
import numpy as np
import pytest
import torch

import oracle
from convolution_voxelised_point_amd import synth
from helpers import assert_feature_close, canon, dev

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

RELATION_CASES = [
    # name, fine coords, ksize, stride, C of x (coarse side), C of y (fine side), dtype
    ("down_f16_64x32", synth.make("down", scale=0.03).coords, 2, 2, 64, 32, "f16"),
    ("k3s2_bf16_32x64", synth.random_coords(201, 1500, 3, 2, 24, lo=-12), 3, 2, 32, 64, "bf16"),
    ("subm_f16_64x64", synth.make("lidar", scale=0.03).coords, 3, 1, 64, 64, "f16"),
    ("subm_f32_k3", synth.random_coords(202, 900, 3, 2, 12), 3, 1, 5, 7, "f32"),
    ("down2d_f32", synth.random_coords(203, 900, 2, 2, 50), 2, 2, 6, 4, "f32"),
]


@pytest.mark.parametrize("case", RELATION_CASES, ids=[c[0] for c in RELATION_CASES])
def test_conv_transpose_on_relation(ts, case):
    """y on the fine rows = sum over the map's triples of x[coarse] . W[o]."""
    name, c, k, s, cin, cout, dt = case
    cd = dev(c)
    tab = ts.HashTable(cd, 2.0)
    if s == 1:
        km = ts.build_kmap(cd, tab, k, 1, ts.TS_KMAP_PAIRS)
        oc = c
    else:
        out, n_out, otab = ts.strided_support(cd, s)
        km = ts.build_kmap(cd, tab, k, s, ts.TS_KMAP_PAIRS | ts.TS_KMAP_BWD, out_coords=out, n_out=n_out,
                           out_table=otab)
        oc = oracle.strided_support(c, s)
    tr = oracle.kmap(c, oc, k, s)
    x = synth.normal(210, (oc.shape[0], cin), 1.0, dt)
    w = synth.weight(211, km.kvol, cin, cout, dt)
    xd = torch.zeros((km.s.n_out_cap, cin), dtype=DT[dt], device="cuda")
    xd[:oc.shape[0]] = dev(x)
    ref = oracle.conv_transpose(tr, x, w, c.shape[0])
    for df in (ts.TS_DATAFLOW_AUTO, ts.TS_DATAFLOW_GATHER_SCATTER):
        for out_dtype in (torch.float32, DT[dt]):
            y = ts.conv_transpose(km, xd, dev(w), out_dtype=out_dtype, dataflow=df)
            assert_feature_close(y, ref, DT[dt], f"{name} conv_transpose df={df} out={out_dtype}")


SUPPORT_CASES = [(3, 2, 2, 220), (2, 2, 2, 221), (3, 3, 2, 222), (3, 3, 1, 223), (2, 3, 3, 224)]


@pytest.mark.parametrize("ndim,k,s,seed", SUPPORT_CASES)
def test_transposed_support(ts, ndim, k, s, seed):
    c = synth.random_coords(seed, 1200, ndim, 2, 30, lo=-15)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, n_out, otab = ts.transposed_support(dev(c), k, s, err_flags=flags)
    ref = oracle.transposed_support(c, k, s)
    n = int(n_out.item())
    assert int(flags.item()) == 0 and n == ref.shape[0]
    assert np.array_equal(out[:n].cpu().numpy(), ref), "generated fine sites or their order differ"
    assert np.array_equal(otab.query(out[:n]).cpu().numpy(), np.arange(n, dtype=np.int32))


def test_transposed_support_empty_and_capacity(ts):
    out, n_out, _ = ts.transposed_support(torch.zeros((0, 4), dtype=torch.int32, device="cuda"), 2, 2, n_out_cap=1)
    assert int(n_out.item()) == 0
    c = synth.random_coords(225, 200, 3, 1, 10)
    ref = oracle.transposed_support(c, 2, 2)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, n_out, otab = ts.transposed_support(dev(c), 2, 2, n_out_cap=100, err_flags=flags)
    assert int(n_out.item()) == 100 and int(flags.item()) & ts.TS_FLAG_FULL
    assert np.array_equal(out.cpu().numpy(), ref[:100])


GEN_CASES = [
    ("k2s2_f16_64x32", synth.random_coords(230, 2500, 3, 2, 20, lo=-10), 2, 2, 64, 32, "f16"),
    ("k3s2_bf16_32x32", synth.random_coords(231, 1200, 3, 2, 16), 3, 2, 32, 32, "bf16"),
    ("k2s2_2d_f32", synth.random_coords(232, 900, 2, 2, 40), 2, 2, 3, 5, "f32"),
]


@pytest.mark.parametrize("natural", [True, False], ids=["row_order", "sorted"])
@pytest.mark.parametrize("case", GEN_CASES, ids=[c[0] for c in GEN_CASES])
def test_generative_conv_transpose(ts, case, natural):
    """Generated fine support, the transposed map and its transpose bit-exact;
    forward, dgrad and wgrad over it against the oracle."""
    name, c, k, s, cin, cout, dt = case
    cd = dev(c)
    tab = ts.HashTable(cd, 2.0)
    out, n_out, otab = ts.transposed_support(cd, k, s)
    fine = oracle.transposed_support(c, k, s)
    m = int(n_out.item())
    assert m == fine.shape[0] and np.array_equal(out[:m].cpu().numpy(), fine)
    flags = ts.TS_KMAP_TRANSPOSED | ts.TS_KMAP_BWD | ts.TS_KMAP_PAIRS | (ts.TS_KMAP_NATURAL if natural else 0)
    km = ts.build_kmap(cd, tab, k, s, flags, out_coords=out, n_out=n_out, out_table=otab)
    tr = oracle.kmap_transposed(c, fine, k, s)
    assert np.array_equal(canon(ts.decode_rel(km.rel_arrays("fwd"), km.kvol)), canon(tr)), "transposed map"
    assert np.array_equal(canon(ts.decode_rel(km.rel_arrays("bwd"), km.kvol, transposed=True)), canon(tr)), \
        "its transpose"
    x = synth.normal(233, (c.shape[0], cin), 1.0, dt)
    w = synth.weight(234, km.kvol, cin, cout, dt)
    for df in (ts.TS_DATAFLOW_AUTO, ts.TS_DATAFLOW_GATHER_SCATTER):
        y = ts.conv_fwd(km, dev(x), dev(w), out_dtype=torch.float32, dataflow=df)
        assert_feature_close(y[:m], oracle.conv_fwd(tr, x, w, m), DT[dt], f"{name} fwd df={df}")
    dy = synth.normal(235, (m, cout), 1.0, dt)
    dyd = torch.zeros((km.s.n_out_cap, cout), dtype=DT[dt], device="cuda")
    dyd[:m] = dev(dy)
    ref = oracle.conv_dgrad(tr, dy, w, c.shape[0])
    for df in (ts.TS_DATAFLOW_AUTO, ts.TS_DATAFLOW_GATHER_SCATTER):
        dx = ts.conv_dgrad(km, dyd, dev(w), out_dtype=torch.float32, dataflow=df)
        assert_feature_close(dx, ref, DT[dt], f"{name} dgrad df={df}")
    dw = ts.conv_wgrad(km, dev(x), dyd)
    assert_feature_close(dw, oracle.conv_wgrad(tr, x, dy, km.kvol), DT[dt], f"{name} wgrad")
