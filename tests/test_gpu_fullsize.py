"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (its ``setup_*`` functions): hash queries, kernel-map triples
and output coordinates bit-exact against the CPU oracle over the whole
problem; features against the fp64 oracle on a seeded sample of output rows
(and, for wgrad, on a few whole offsets) that it computes one by one."""
import numpy as np
import pytest
import torch

import bench
import oracle
from convolution_voxelised_point_amd import synth
from helpers import assert_feature_close, canon, check_window_sorted

pytestmark = pytest.mark.gpu

N_SAMPLE = 3000


def sample_rows(n: int, seed: int) -> np.ndarray:
    """Seeded sample of rows plus both ends (first and last tiles)."""
    rng = np.random.default_rng(seed)
    pick = rng.choice(n, size=min(n, N_SAMPLE), replace=False)
    ends = np.r_[np.arange(min(n, 20)), np.arange(max(0, n - 20), n)]
    return np.unique(np.r_[pick, ends]).astype(np.int64)


def restrict(tr, rows, side):
    """Triples whose `side` (0 = in, 1 = out) row is among `rows`."""
    sel = np.isin(tr[side], rows)
    return tuple(t[sel] for t in tr)


def check_hash(ts, s, coords_np, seed):
    rows = s.table.query(s.coords).cpu().numpy()
    assert np.array_equal(rows, np.arange(coords_np.shape[0], dtype=np.int32))
    rng = np.random.default_rng(seed)
    q = coords_np[rng.choice(coords_np.shape[0], 4096)].copy()
    q[:, 1:] += rng.integers(-2, 3, size=q[:, 1:].shape).astype(np.int32)
    got = s.table.query(torch.from_numpy(q).cuda()).cpu().numpy()
    ref, _ = oracle.hash_query(coords_np, q)
    assert np.array_equal(got, ref)


def check_triples(km, tr, kvol, what):
    got = ts_decode(km, kvol)
    a, b = canon(got), canon(tr)
    assert a.shape == b.shape and np.array_equal(a, b), f"{what}: kernel map differs from the oracle"


def ts_decode(km, kvol):
    from convolution_voxelised_point_amd import ts
    return ts.decode_rel(km.rel_arrays("fwd"), kvol)


@pytest.mark.parametrize("rows_shuffled", [False, True], ids=["lex_rows", "shuffled_rows"])
@pytest.mark.parametrize("order", ["natural", "sorted"])
def test_full_lidar_subm_f16(ts, order, rows_shuffled):
    """Both tile orders: the benchmark's (rows in index order, the map
    serving one contraction) and the window sort by offset mask; on the
    scene's lexicographic rows and on the seeded shuffle of them."""
    w = synth.make("lidar")
    if rows_shuffled:
        w = synth.shuffled(w)
    s = bench.setup_subm(ts, w, kmap_flags=ts.TS_KMAP_NATURAL if order == "natural" else 0)
    s.run_once()
    assert int(s.flags.item()) == 0
    check_hash(ts, s, w.coords, 11)
    tr = oracle.kmap(w.coords, w.coords, 3, 1)
    check_triples(s.kmap, tr, 27, "lidar")
    rel = s.kmap.rel_arrays("fwd")
    slots = rel["tile_rows"].cpu().numpy()
    if order == "natural":
        want = np.full(slots.shape[0], -1, np.int32)
        want[:w.n] = np.arange(w.n, dtype=np.int32)
        assert np.array_equal(slots, want)
    else:
        check_window_sorted(slots, rel["row_mask"].cpu().numpy().view(np.uint64)[:w.n])
    rows = sample_rows(w.n, 12)
    ref = oracle.conv_fwd(restrict(tr, rows, 1), w.x, w.w, w.n)[rows]
    assert_feature_close(s.y[torch.from_numpy(rows).cuda()], ref, torch.float16, "lidar fwd (fp16 out)")


def test_full_tiny_subm_f32(ts):
    w = synth.make("tiny")
    s = bench.setup_subm(ts, w)
    s.run_once()
    tr = oracle.kmap(w.coords, w.coords, 3, 1)
    check_triples(s.kmap, tr, 27, "tiny")
    ref = oracle.conv_fwd(tr, w.x, w.w, w.n)
    assert_feature_close(s.y, ref, torch.float32, "tiny fwd")


def test_full_down_strided_f16(ts):
    w = synth.make("down")
    s = bench.setup_down(ts, w)
    s.run_once()
    assert int(s.flags.item()) == 0
    check_hash(ts, s, w.coords, 21)
    oc = oracle.strided_support(w.coords, 2)
    n_o = int(s.n_out.item())
    assert n_o == oc.shape[0]
    assert np.array_equal(s.out[:n_o].cpu().numpy(), oc)
    tr = oracle.kmap(w.coords, oc, 2, 2)
    check_triples(s.kmap, tr, 8, "down")
    rows = sample_rows(n_o, 22)
    ref = oracle.conv_fwd(restrict(tr, rows, 1), w.x, w.w, n_o)[rows]
    assert_feature_close(s.y[torch.from_numpy(rows).cuda()], ref, torch.float16, "down fwd (fp16 out)")


def test_full_generative_f16(ts):
    """Generative stride-1 Conv3d k3 on the ring scan: the 1.77M generated
    sites in first-occurrence order and the target map bit-exact, features on
    sampled rows."""
    w = synth.make("lidar")
    s = bench.setup_generative(ts, w)
    s.run_once()
    assert int(s.flags.item()) == 0
    oc = oracle.generative_support(w.coords, 3)
    assert int(s.n_out.item()) == s.m == oc.shape[0]
    assert np.array_equal(s.out.cpu().numpy(), oc)
    rows = s.out_table.query(s.out).cpu().numpy()
    assert np.array_equal(rows, np.arange(s.m, dtype=np.int32))
    tr = oracle.kmap(w.coords, oc, 3, 1, target=True)
    assert len(tr[0]) == 27 * w.n  # every input reaches a generated site through every offset
    check_triples(s.kmap, tr, 27, "generative")
    pick = sample_rows(s.m, 52)
    ref = oracle.conv_fwd(restrict(tr, pick, 1), w.x, w.w, s.m)[pick]
    assert_feature_close(s.y[torch.from_numpy(pick).cuda()], ref, torch.float16, "generative fwd (fp16 out)")


def test_full_up_transposed_f16(ts):
    """Transposed convolutions on the two-scene strided layer: ConvTranspose3d
    over its relation and GenerativeConvTranspose3d from its coarse rows
    (1.28M generated fine sites bit-exact, map bit-exact, features sampled)."""
    w = synth.make("down")
    s = bench.setup_up(ts, w)
    s.run_once()
    assert int(s.flags.item()) == 0
    coarse = oracle.strided_support(w.coords, 2)
    assert s.m == coarse.shape[0] and np.array_equal(s.coarse.cpu().numpy(), coarse)
    x = s.x[:s.m].cpu()
    tr = oracle.kmap(w.coords, coarse, 2, 2)
    rows = sample_rows(s.n, 61)
    ref = oracle.conv_transpose(restrict(tr, rows, 0), x, s.w.cpu(), s.n)[rows]
    assert_feature_close(s.y[torch.from_numpy(rows).cuda()], ref, torch.float16, "ConvTranspose3d (fp16 out)")
    fine = oracle.transposed_support(coarse, 2, 2)
    n_f = int(s.n_fine.item())
    assert n_f == fine.shape[0] == 8 * s.m
    assert np.array_equal(s.fine[:n_f].cpu().numpy(), fine)
    tg = oracle.kmap_transposed(coarse, fine, 2, 2)
    check_triples(s.gen, tg, 8, "generative transposed")
    pick = sample_rows(n_f, 62)
    ref = oracle.conv_fwd(restrict(tg, pick, 1), x, s.w.cpu(), n_f)[pick]
    assert_feature_close(s.yg[torch.from_numpy(pick).cuda()], ref, torch.float16, "GenerativeConvTranspose3d")


@pytest.mark.parametrize("dataflow", ["auto", "gather_scatter"])
def test_full_pixels_two_layers(ts, dataflow):
    w = synth.make("pixels")
    df = ts.TS_DATAFLOW_AUTO if dataflow == "auto" else ts.TS_DATAFLOW_GATHER_SCATTER
    s = bench.setup_pixels(ts, w, df)
    s.run_once()
    assert int(s.flags.item()) == 0
    check_hash(ts, s, w.coords, 31)
    tr = oracle.kmap(w.coords, w.coords, 3, 1)
    check_triples(s.kmap, tr, 9, "pixels")
    ref1 = oracle.conv_fwd(tr, w.x, w.w, w.n)
    assert_feature_close(s.y1, ref1, torch.float16, f"pixels layer 1 ({dataflow})")
    # layer 2 is checked on its own (already rounded) input
    ref2 = oracle.conv_fwd(tr, s.y1.cpu(), w.extra["w2"], w.n)
    assert_feature_close(s.y2, ref2, torch.float16, f"pixels layer 2 ({dataflow})")


def test_full_train_bf16(ts):
    w = synth.make("train")
    s = bench.setup_train(ts, w)
    s.run_once()
    assert int(s.flags.item()) == 0
    check_hash(ts, s, w.coords, 41)
    tr = oracle.kmap(w.coords, w.coords, 3, 1)
    check_triples(s.kmap, tr, 27, "train")
    rel = s.kmap.rel_arrays("fwd")
    check_window_sorted(rel["tile_rows"].cpu().numpy(), rel["row_mask"].cpu().numpy().view(np.uint64)[:w.n])
    # the per-offset pair lists are the same relation
    ps, pin, pout = s.kmap.pairs()
    off = np.repeat(np.arange(27, dtype=np.int32), np.diff(ps))
    assert np.array_equal(canon((pin, pout, off)), canon(tr))
    rows = sample_rows(w.n, 42)
    ref = oracle.conv_fwd(restrict(tr, rows, 1), w.x, w.w, w.n)[rows]
    assert_feature_close(s.y[torch.from_numpy(rows).cuda()], ref, torch.bfloat16, "train fwd (bf16 out)")
    ref = oracle.conv_dgrad(restrict(tr, rows, 0), w.dy, w.w, w.n)[rows]
    assert_feature_close(s.dx[torch.from_numpy(rows).cuda()], ref, torch.bfloat16, "train dgrad (bf16 out)")
    offs = np.array([0, 4, 13, 22, 26])
    sel = np.isin(tr[2], offs)
    ref = oracle.conv_wgrad(tuple(t[sel] for t in tr), w.x, w.dy, 27)[offs]
    assert_feature_close(s.dw[torch.from_numpy(offs).cuda()], ref, torch.bfloat16, "train wgrad")
