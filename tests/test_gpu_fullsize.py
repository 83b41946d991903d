"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (its ``setup_*`` functions): hash queries, kernel-map triples
and output coordinates bit-exact against the CPU oracle over the whole
problem; features against the fp64 oracle over every element of every output
tensor.

Each contraction is run twice: with fp32 outputs, graded on the plain bar
(max|err| <= 2e-3 max|ref| for fp16/bf16 inputs, 1e-5 for fp32), and with
outputs in the input type as the benchmark times it, graded on that bar plus
the output's own rounding (u_out |ref| per element)."""
import numpy as np
import pytest
import torch

import bench
import oracle
from convolution_voxelised_point_amd import synth
from helpers import assert_feature_close, canon, check_window_sorted

pytestmark = pytest.mark.gpu


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
    """The map's forward relation as triples: from its neighbour table, or
    from its pair groups when it has no table (both when it has both)."""
    from convolution_voxelised_point_amd import ts
    arrs = km.rel_arrays("fwd")
    if "gcount" in arrs and "nbr" in arrs:
        a, b = canon(ts.decode_rel(arrs, kvol)), canon(ts.decode_groups(arrs, kvol))
        assert np.array_equal(a, b), "pair groups and neighbour table disagree"
    return ts.decode_rel(arrs, kvol) if "nbr" in arrs else ts.decode_groups(arrs, kvol)


@pytest.mark.parametrize("rows_shuffled", [False, True], ids=["lex_rows", "shuffled_rows"])
@pytest.mark.parametrize("order", ["groups", "natural", "sorted"])
def test_full_lidar_subm_f16(ts, order, rows_shuffled):
    """The three maps the benchmark measures: pair groups only (the
    headline step: fetch-on-demand forward), and a neighbour table with
    tiles in row order or sorted by offset mask (implicit GEMM); on the
    scene's lexicographic rows and on the seeded shuffle of them."""
    w = synth.make("lidar")
    if rows_shuffled:
        w = synth.shuffled(w)
    flags = {"groups": ts.TS_KMAP_GROUPS | ts.TS_KMAP_NO_TABLE, "natural": ts.TS_KMAP_NATURAL, "sorted": 0}[order]
    s = bench.setup_subm(ts, w, kmap_flags=flags)
    s.run_once()
    assert int(s.flags.item()) == 0
    check_hash(ts, s, w.coords, 11)
    tr = oracle.kmap(w.coords, w.coords, 3, 1)
    check_triples(s.kmap, tr, 27, "lidar")
    rel = s.kmap.rel_arrays("fwd")
    if order == "groups":
        assert "nbr" not in rel and "gcount" in rel
    elif order == "natural":
        slots = rel["tile_rows"].cpu().numpy()
        want = np.full(slots.shape[0], -1, np.int32)
        want[:w.n] = np.arange(w.n, dtype=np.int32)
        assert np.array_equal(slots, want)
    else:
        check_window_sorted(rel["tile_rows"].cpu().numpy(), rel["row_mask"].cpu().numpy().view(np.uint64)[:w.n])
    ref = oracle.conv_fwd(tr, w.x, w.w, w.n)
    tag = f"lidar {order} {'shuffled' if rows_shuffled else 'lex'}"
    assert_feature_close(s.y, ref, torch.float16, f"{tag} fwd fp16 out")
    s32 = bench.setup_subm(ts, w, out_dtype=torch.float32, kmap_flags=flags)
    s32.run_once()
    assert_feature_close(s32.y, ref, torch.float16, f"{tag} fwd fp32 out")


def test_full_tiny_subm_f32(ts):
    w = synth.make("tiny")
    s = bench.setup_subm(ts, w)
    s.run_once()
    tr = oracle.kmap(w.coords, w.coords, 3, 1)
    check_triples(s.kmap, tr, 27, "tiny")
    ref = oracle.conv_fwd(tr, w.x, w.w, w.n)
    assert_feature_close(s.y, ref, torch.float32, "tiny fwd fp32")


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
    ref = oracle.conv_fwd(tr, w.x, w.w, n_o)
    assert_feature_close(s.y[:n_o], ref, torch.float16, "down fwd fp16 out")
    s32 = bench.setup_down(ts, w, out_dtype=torch.float32)
    s32.run_once()
    assert int(s32.n_out.item()) == n_o
    assert_feature_close(s32.y[:n_o], ref, torch.float16, "down fwd fp32 out")


@pytest.mark.parametrize("order", ["groups", "sorted"])
def test_full_generative_f16(ts, order):
    """Generative stride-1 Conv3d k3 on the ring scan: the 1.77M generated
    sites in first-occurrence order, the target map bit-exact, every output
    row against the oracle; with pair groups only (fetch-on-demand, as the
    benchmark runs it) and with the neighbour table sorted by offset mask
    (implicit GEMM)."""
    w = synth.make("lidar")
    flags = None if order == "groups" else 0
    s = bench.setup_generative(ts, w, kmap_flags=flags)
    if order == "groups":
        assert "nbr" not in s.kmap.rel_arrays("fwd")
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
    ref = oracle.conv_fwd(tr, w.x, w.w, s.m)
    assert_feature_close(s.y, ref, torch.float16, "generative fwd fp16 out")
    del s
    s32 = bench.setup_generative(ts, w, kmap_flags=flags, out_dtype=torch.float32)
    s32.run_once()
    assert_feature_close(s32.y, ref, torch.float16, "generative fwd fp32 out")


def test_full_up_transposed_f16(ts):
    """Transposed convolutions on the two-scene strided layer: ConvTranspose3d
    over its relation and GenerativeConvTranspose3d from its coarse rows
    (1.28M generated fine sites and the map bit-exact, every row compared)."""
    w = synth.make("down")
    coarse = oracle.strided_support(w.coords, 2)
    tr = oracle.kmap(w.coords, coarse, 2, 2)
    fine = oracle.transposed_support(coarse, 2, 2)
    tg = oracle.kmap_transposed(coarse, fine, 2, 2)
    refs = None
    for out_dtype in (None, torch.float32):
        s = bench.setup_up(ts, w, out_dtype=out_dtype)
        s.run_once()
        assert int(s.flags.item()) == 0
        assert s.m == coarse.shape[0] and np.array_equal(s.coarse.cpu().numpy(), coarse)
        n_f = int(s.n_fine.item())
        assert n_f == fine.shape[0] == 8 * s.m
        assert np.array_equal(s.fine[:n_f].cpu().numpy(), fine)
        if refs is None:
            check_triples(s.gen, tg, 8, "generative transposed")
            x = s.x[:s.m].cpu()
            refs = (oracle.conv_transpose(tr, x, s.w.cpu(), s.n), oracle.conv_fwd(tg, x, s.w.cpu(), n_f))
        tag = "fp32 out" if out_dtype else "fp16 out"
        assert_feature_close(s.y, refs[0], torch.float16, f"ConvTranspose3d {tag}")
        assert_feature_close(s.yg[:n_f], refs[1], torch.float16, f"GenerativeConvTranspose3d {tag}")
        del s


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
    assert_feature_close(s.y1, ref1, torch.float16, f"pixels layer 1 ({dataflow}) fp16 out")
    # layer 2 is checked on its own (already rounded) input
    ref2 = oracle.conv_fwd(tr, s.y1.cpu(), w.extra["w2"], w.n)
    assert_feature_close(s.y2, ref2, torch.float16, f"pixels layer 2 ({dataflow}) fp16 out")
    # fp32 outputs of the same layers on the same map
    y1 = ts.conv_fwd(s.kmap, s.x, s.w1, out_dtype=torch.float32, dataflow=df)
    assert_feature_close(y1, ref1, torch.float16, f"pixels layer 1 ({dataflow}) fp32 out")
    y2 = ts.conv_fwd(s.kmap, s.y1, s.w2, out_dtype=torch.float32, dataflow=df)
    assert_feature_close(y2, ref2, torch.float16, f"pixels layer 2 ({dataflow}) fp32 out")


@pytest.mark.parametrize("order", ["groups", "sorted"])
def test_full_train_bf16(ts, order):
    """The 128-channel bf16 training step on four scenes: forward, dgrad and
    all 27 offsets of wgrad over every element, with the default map (a
    neighbour table sorted by offset mask: the implicit GEMM) and with pair
    groups only (the fetch-on-demand kernels)."""
    w = synth.make("train")
    flags = (ts.TS_KMAP_GROUPS | ts.TS_KMAP_NO_TABLE) if order == "groups" else None
    s = bench.setup_train(ts, w, kmap_flags=flags)
    s.run_once()
    assert int(s.flags.item()) == 0
    check_hash(ts, s, w.coords, 41)
    tr = oracle.kmap(w.coords, w.coords, 3, 1)
    check_triples(s.kmap, tr, 27, "train")
    rel = s.kmap.rel_arrays("fwd")
    if order == "groups":
        assert "nbr" not in rel and "gcount" in rel
    else:
        check_window_sorted(rel["tile_rows"].cpu().numpy(), rel["row_mask"].cpu().numpy().view(np.uint64)[:w.n])
    # the per-offset pair lists are the same relation
    ps, pin, pout = s.kmap.pairs()
    off = np.repeat(np.arange(27, dtype=np.int32), np.diff(ps))
    assert np.array_equal(canon((pin, pout, off)), canon(tr))
    ref_y = oracle.conv_fwd(tr, w.x, w.w, w.n)
    ref_dx = oracle.conv_dgrad(tr, w.dy, w.w, w.n)
    ref_dw = oracle.conv_wgrad(tr, w.x, w.dy, 27)
    assert_feature_close(s.y, ref_y, torch.bfloat16, f"train {order} fwd bf16 out")
    assert_feature_close(s.dx, ref_dx, torch.bfloat16, f"train {order} dgrad bf16 out")
    assert_feature_close(s.dw, ref_dw, torch.bfloat16, f"train {order} wgrad (27 offsets, fp32 dW)")
    dw0 = s.dw.clone()
    del s
    s32 = bench.setup_train(ts, w, out_dtype=torch.float32, kmap_flags=flags)
    s32.run_once()
    assert_feature_close(s32.y, ref_y, torch.bfloat16, f"train {order} fwd fp32 out")
    assert_feature_close(s32.dx, ref_dx, torch.bfloat16, f"train {order} dgrad fp32 out")
    assert torch.equal(s32.dw, dw0), "wgrad differs between two runs of the same step"
