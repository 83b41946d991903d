"""GPU parity of convolution at caller-given output coordinates (target maps,
TargetConv3d) and of the generated support of a stride-1 convolution
against the CPU oracle: coordinates, order and triples bit-exact, features
within the fp64 oracle's tolerance, for both tile orders and dataflows."""
import numpy as np
import pytest
import torch

import oracle
from convolution_voxelised_point_amd import synth
from helpers import assert_feature_close, canon, check_window_sorted, dev

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def targets_for(seed, coords, stride, n_new, repeats):
    """Input sites (coarsened for stride > 1), fresh sites around them and,
    if asked, repeated rows; shuffled."""
    rng = np.random.default_rng(seed)
    ndim = coords.shape[1] - 1
    base = coords.copy()
    base[:, 1:] = np.floor_divide(base[:, 1:], stride)
    pick = base[rng.choice(base.shape[0], size=min(base.shape[0], 3 * n_new), replace=False)]
    fresh = pick[:n_new].copy()
    fresh[:, 1:] += rng.integers(-2, 3, size=(n_new, ndim)).astype(np.int32)
    t = np.concatenate([pick, fresh])
    if repeats:
        t = np.concatenate([t, t[rng.choice(t.shape[0], t.shape[0] // 10)]])
    else:
        _, first = np.unique(t, axis=0, return_index=True)
        t = t[np.sort(first)]
    return np.ascontiguousarray(t[rng.permutation(t.shape[0])].astype(np.int32))


def target_map(ts, coords, targets, ksize, stride, natural, bwd):
    cd, td = dev(coords), dev(targets)
    tab = ts.HashTable(cd, 2.0)
    flags = ts.TS_KMAP_TARGET | ts.TS_KMAP_PAIRS | (ts.TS_KMAP_NATURAL if natural else 0)
    n_out = torch.tensor([targets.shape[0]], dtype=torch.int64, device="cuda")
    otab = None
    if bwd:
        flags |= ts.TS_KMAP_BWD
        otab = ts.HashTable(td, 2.0)
    return ts.build_kmap(cd, tab, ksize, stride, flags, out_coords=td, n_out=n_out, out_table=otab)


TARGET_CASES = [
    # name, coords, ksize, stride, cin, cout, dtype, repeats
    ("lidar_f16_64", synth.make("lidar", scale=0.04).coords, 3, 1, 64, 64, "f16", True),
    ("fuzz_bf16_32x48", synth.random_coords(61, 1500, 3, 2, 14, lo=-7), 3, 1, 32, 48, "bf16", False),
    ("fuzz_f32_k2", synth.random_coords(62, 900, 3, 2, 12), 2, 1, 5, 7, "f32", True),
    ("pixels_f16_k3", synth.random_coords(63, 1200, 2, 3, 40), 3, 1, 8, 8, "f16", False),
    ("strided_f16_k2s2", synth.random_coords(64, 1500, 3, 2, 24, lo=-12), 2, 2, 32, 64, "f16", True),
]


@pytest.mark.parametrize("natural", [True, False], ids=["row_order", "sorted"])
@pytest.mark.parametrize("case", TARGET_CASES, ids=[c[0] for c in TARGET_CASES])
def test_target_map_and_forward(ts, case, natural):
    name, c, k, s, cin, cout, dt, rep = case
    t = targets_for(70, c, s, 200, rep)
    km = target_map(ts, c, t, k, s, natural, bwd=False)
    tr = oracle.kmap(c, t, k, s, target=True)
    got = ts.decode_rel(km.rel_arrays("fwd"), km.kvol)
    assert np.array_equal(canon(got), canon(tr)), f"{name}: target map differs from the oracle"
    ps, pin, pout = km.pairs()
    assert ps[-1] == len(tr[0])
    assert np.array_equal(canon((pin, pout, np.repeat(np.arange(km.kvol), np.diff(ps)))), canon(tr))
    if not natural:
        slots = km.rel_arrays("fwd")["tile_rows"].cpu().numpy()
        check_window_sorted(slots, km.rel_arrays("fwd")["row_mask"].cpu().numpy().view(np.uint64)[:t.shape[0]])
    x = synth.normal(71, (c.shape[0], cin), 1.0, dt)
    w = synth.weight(72, k ** (c.shape[1] - 1), cin, cout, dt)
    ref = oracle.conv_fwd(tr, x, w, t.shape[0])
    for df in (ts.TS_DATAFLOW_AUTO, ts.TS_DATAFLOW_GATHER_SCATTER):
        y = ts.conv_fwd(km, dev(x), dev(w), out_dtype=torch.float32, dataflow=df)
        assert_feature_close(y, ref, DT[dt], f"{name} target fwd df={df}")


@pytest.mark.parametrize("case", TARGET_CASES, ids=[c[0] for c in TARGET_CASES])
def test_target_backward(ts, case):
    """dgrad over the transposed target relation and over pair lists (distinct
    targets), and wgrad (repeats allowed)."""
    name, c, k, s, cin, cout, dt, rep = case
    t = targets_for(80, c, s, 150, repeats=False)
    km = target_map(ts, c, t, k, s, natural=False, bwd=True)
    tr = oracle.kmap(c, t, k, s, target=True)
    got_b = ts.decode_rel(km.rel_arrays("bwd"), km.kvol, transposed=True)
    assert np.array_equal(canon(got_b), canon(tr)), f"{name}: transposed target map differs"
    x = synth.normal(81, (c.shape[0], cin), 1.0, dt)
    w = synth.weight(82, km.kvol, cin, cout, dt)
    dy = synth.normal(83, (t.shape[0], cout), 1.0, dt)
    ref = oracle.conv_dgrad(tr, dy, w, c.shape[0])
    for df in (ts.TS_DATAFLOW_AUTO, ts.TS_DATAFLOW_GATHER_SCATTER):
        dx = ts.conv_dgrad(km, dev(dy), dev(w), out_dtype=torch.float32, dataflow=df)
        assert_feature_close(dx, ref, DT[dt], f"{name} target dgrad df={df}")
    t2 = targets_for(84, c, s, 150, repeats=True)
    km2 = target_map(ts, c, t2, k, s, natural=True, bwd=False)
    tr2 = oracle.kmap(c, t2, k, s, target=True)
    dy2 = synth.normal(85, (t2.shape[0], cout), 1.0, dt)
    dw = ts.conv_wgrad(km2, dev(x), dev(dy2))
    assert_feature_close(dw, oracle.conv_wgrad(tr2, x, dy2, km.kvol), DT[dt], f"{name} target wgrad")


def test_target_rows_out_of_range_and_rejected_as_subm(ts):
    c = synth.random_coords(90, 400, 3, 1, 10)
    t = np.array([[0, 3, 3, 3], [-1, 3, 3, 3], [0, 40000, 3, 3], [0, 3, 3, 3], [0, 50, 50, 50]], np.int32)
    km = target_map(ts, c, t, 3, 1, natural=True, bwd=False)
    tr = oracle.kmap(c, t, 3, 1, target=True)
    assert np.array_equal(canon(ts.decode_rel(km.rel_arrays("fwd"), 27)), canon(tr))
    x = synth.normal(91, (c.shape[0], 4), 1.0, "f32")
    w = synth.weight(92, 27, 4, 4, "f32")
    y = ts.conv_fwd(km, dev(x), dev(w))
    assert_feature_close(y, oracle.conv_fwd(tr, x, w, t.shape[0]), torch.float32, "out-of-range targets")
    assert float(y[[1, 2, 4]].abs().max()) == 0.0
    with pytest.raises(ts.TsError):
        ts.ts_subm_conv_fwd(km.s, dev(x), dev(w), torch.empty((5, 4), device="cuda"))


# ---------------------------------------------------------------- generated support
GEN_CASES = [
    ("lidar_3d_k3", synth.make("lidar", scale=0.03).coords, 3),
    ("fuzz_3d_k3", synth.random_coords(101, 2000, 3, 3, 20, lo=-10), 3),
    ("fuzz_2d_k5", synth.random_coords(102, 700, 2, 2, 40), 5),
    ("fuzz_3d_k1", synth.random_coords(103, 500, 3, 2, 8), 1),
    ("fuzz_3d_k2", synth.random_coords(104, 800, 3, 2, 12), 2),
]


@pytest.mark.parametrize("case", GEN_CASES, ids=[c[0] for c in GEN_CASES])
def test_generative_support(ts, case):
    name, c, k = case
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, n_out, otab = ts.generative_support(dev(c), k, err_flags=flags)
    ref = oracle.generative_support(c, k)
    n = int(n_out.item())
    assert int(flags.item()) == 0
    assert n == ref.shape[0], (name, n, ref.shape[0])
    assert np.array_equal(out[:n].cpu().numpy(), ref), f"{name}: generated sites or their order differ"
    rows = otab.query(out[:n]).cpu().numpy()
    assert np.array_equal(rows, np.arange(n, dtype=np.int32))
    # rebuild into the same buffers gives the same result
    ts.ts_generative_support(dev(c), k, out, n_out, otab.buf, otab.cap,
                             torch.empty(ts.ts_generative_scratch_bytes(c.shape[0], c.shape[1] - 1, k),
                                         dtype=torch.uint8, device="cuda"), flags)
    assert int(n_out.item()) == n and np.array_equal(out[:n].cpu().numpy(), ref)


def test_generative_support_capacity_and_flags(ts):
    c = np.concatenate([synth.random_coords(110, 300, 3, 2, 10),
                        np.array([[0, 40000, 0, 0], [0, 1, 1, 1]], np.int32)]).astype(np.int32)
    c[-1] = c[0]  # a repeated coordinate adds nothing
    ref = oracle.generative_support(c, 3)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    cap = ref.shape[0] // 2
    out, n_out, otab = ts.generative_support(dev(c), 3, n_out_cap=cap, err_flags=flags)
    assert int(n_out.item()) == cap
    f = int(flags.item())
    assert f & ts.TS_FLAG_RANGE and f & ts.TS_FLAG_FULL
    assert np.array_equal(out.cpu().numpy(), ref[:cap])
    rows = otab.query(dev(ref)).cpu().numpy()
    np.testing.assert_array_equal(rows, np.where(np.arange(ref.shape[0]) < cap, np.arange(ref.shape[0]), -1))
    empty = np.zeros((0, 4), np.int32)
    out0, n0, _ = ts.generative_support(torch.zeros((0, 4), dtype=torch.int32, device="cuda"), 3, n_out_cap=1)
    assert int(n0.item()) == 0 and oracle.generative_support(empty, 3).shape[0] == 0


@pytest.mark.parametrize("dt,cin,cout,natural", [("f16", 64, 64, True), ("bf16", 32, 64, False),
                                                 ("f32", 8, 12, True)])
def test_generative_conv_fwd_bwd(ts, dt, cin, cout, natural):
    """One call: support, target map and forward; then dgrad over the
    transposed relation (both dataflows) and wgrad, against the oracle."""
    c = synth.make("lidar", scale=0.03).coords
    n = c.shape[0]
    cd = dev(c)
    tab = ts.HashTable(cd, 2.0)
    ref_sites = oracle.generative_support(c, 3)
    n_cap = ref_sites.shape[0] + 100
    kflags = ts.TS_KMAP_PAIRS | ts.TS_KMAP_BWD | (ts.TS_KMAP_NATURAL if natural else 0)
    out = torch.zeros((n_cap, 4), dtype=torch.int32, device="cuda")
    n_out = torch.zeros(1, dtype=torch.int64, device="cuda")
    otab = ts.HashTable(out, 2.0, build=False)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    mb = ts.ts_kmap_bytes(n, n_cap, 3, 3, 1, kflags | ts.TS_KMAP_TARGET) + ts.ts_generative_scratch_bytes(n, 3, 3)
    mbuf = torch.empty(mb, dtype=torch.uint8, device="cuda")
    km_s = ts.TsKmap()
    x = synth.normal(120, (n, cin), 1.0, dt)
    w = synth.weight(121, 27, cin, cout, dt)
    y = torch.empty((n_cap, cout), dtype=torch.float32, device="cuda")
    ws = torch.empty(1 << 22, dtype=torch.uint8, device="cuda")
    ts.ts_conv_fwd_generative(cd, tab.buf, tab.cap, 3, kflags, out, n_out, otab.buf, otab.cap, flags, mbuf, km_s,
                              dev(x), dev(w), y, ts.TS_DATAFLOW_AUTO, ws)
    m = int(n_out.item())
    assert int(flags.item()) == 0 and m == ref_sites.shape[0]
    assert np.array_equal(out[:m].cpu().numpy(), ref_sites)
    tr = oracle.kmap(c, ref_sites, 3, 1, target=True)
    km = ts.Kmap(km_s, mbuf, keep=(n_out,))
    assert np.array_equal(canon(ts.decode_rel(km.rel_arrays("fwd"), 27)), canon(tr))
    assert_feature_close(y[:m], oracle.conv_fwd(tr, x, w, m), DT[dt], "generative fwd")
    dy = synth.normal(122, (m, cout), 1.0, dt)
    dyd = torch.zeros((n_cap, cout), dtype=DT[dt], device="cuda")
    dyd[:m] = dev(dy)
    ref_dx = oracle.conv_dgrad(tr, dy, w, n)
    for df in (ts.TS_DATAFLOW_AUTO, ts.TS_DATAFLOW_GATHER_SCATTER):
        dx = ts.conv_dgrad(km, dyd, dev(w), out_dtype=torch.float32, dataflow=df)
        assert_feature_close(dx, ref_dx, DT[dt], f"generative dgrad df={df}")
    dw = ts.conv_wgrad(km, dev(x), dyd)
    assert_feature_close(dw, oracle.conv_wgrad(tr, x, dy, 27), DT[dt], "generative wgrad")
