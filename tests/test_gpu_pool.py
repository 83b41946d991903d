"""GPU parity of sparse max / average pooling over kernel maps against the
CPU oracle: the maximum bit-exact (it involves no rounding), the mean within
the feature tolerance."""
import numpy as np
import pytest
import torch

import oracle
from convolution_voxelised_point_amd import synth
from helpers import assert_feature_close, dev

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

POOL_CASES = [
    # name, coords, ksize, stride, channels, dtype
    ("down_k2s2_f16_64", synth.make("down", scale=0.03).coords, 2, 2, 64, "f16"),
    ("subm_k3_bf16_13", synth.random_coords(301, 1500, 3, 2, 14, lo=-7), 3, 1, 13, "bf16"),
    ("k3s3_f32_empty_windows", synth.random_coords(302, 1200, 3, 2, 20), 3, 3, 5, "f32"),
    ("pix_k2s2_f32_8", synth.random_coords(303, 900, 2, 3, 40), 2, 2, 8, "f32"),
]


@pytest.mark.parametrize("natural", [True, False], ids=["row_order", "sorted"])
@pytest.mark.parametrize("case", POOL_CASES, ids=[c[0] for c in POOL_CASES])
def test_pool(ts, case, natural):
    name, c, k, s, ch, dt = case
    cd = dev(c)
    tab = ts.HashTable(cd, 2.0)
    order = ts.TS_KMAP_NATURAL if natural else 0
    if s == 1:
        km = ts.build_kmap(cd, tab, k, 1, order)
        oc = c
    else:
        out, n_out, otab = ts.strided_support(cd, s)
        km = ts.build_kmap(cd, tab, k, s, order, out_coords=out, n_out=n_out, out_table=otab)
        oc = oracle.strided_support(c, s)
    tr = oracle.kmap(c, oc, k, s)
    x = synth.normal(310, (c.shape[0], ch), 1.0, dt)
    xd = dev(x)
    ref_max = oracle.pool(tr, x, oc.shape[0], "max")
    for out_dtype in (DT[dt], torch.float32):
        y = ts.pool(km, xd, ts.TS_POOL_MAX, out_dtype=out_dtype)[:oc.shape[0]]
        got = y.double().cpu().numpy()
        assert np.array_equal(got, ref_max), f"{name} max pooling (out {out_dtype}) not bit-exact"
    ref_avg = oracle.pool(tr, x, oc.shape[0], "avg")
    for out_dtype in (torch.float32, DT[dt]):
        y = ts.pool(km, xd, ts.TS_POOL_AVG, out_dtype=out_dtype)[:oc.shape[0]]
        assert_feature_close(y, ref_avg, DT[dt], f"{name} avg pooling (out {out_dtype})")
    if s == 3:
        assert (np.bincount(tr[1], minlength=oc.shape[0]) == 0).any(), "case meant to hold empty windows"


def test_pool_rejects(ts):
    c = synth.random_coords(320, 300, 3, 1, 10)
    cd = dev(c)
    km = ts.build_kmap(cd, ts.HashTable(cd, 2.0), 3, 1, 0)
    x = torch.zeros((c.shape[0], 4), dtype=torch.float16, device="cuda")
    with pytest.raises(ts.TsError):
        ts.pool(km, x, mode=7)
    with pytest.raises(ts.TsError):
        ts.pool(km, x, out_dtype=torch.bfloat16)
