"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function ``include/ts.h`` declares, answers size queries, and rejects
bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ts.h")
LIB = os.path.join(ROOT, "convolution_voxelised_point_amd", "libts.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libts.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ts_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def ts():
    from convolution_voxelised_point_amd import ts as mod
    return mod


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(LIB)
    names = declared_functions()
    assert len(names) >= 16
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_lists_all_declared(ts):
    assert sorted(ts.EXPORTED) == declared_functions()


def test_version_and_status(ts):
    assert "gfx950" in ts.ts_version()
    assert ts.ts_status_string(0) == "ok"
    assert ts.ts_status_string(1) == "invalid argument"
    assert ts.ts_status_string(3) == "HIP error"


def test_hash_capacity(ts):
    assert ts.ts_hash_capacity(0, 2.0) == 64
    assert ts.ts_hash_capacity(100, 2.0) == 256
    assert ts.ts_hash_capacity(102835, 2.0) == 262144
    assert ts.ts_hash_capacity(1000, 1.0) == 1024
    assert ts.ts_hash_capacity(1025, 1.0) == 2048
    assert ts.ts_hash_capacity(10, 0.5) == -1
    assert ts.ts_hash_capacity(-1, 2.0) == -1
    assert ts.ts_hash_table_bytes(1024) == 8 * 1024 + 256 * 1024


def test_kmap_bytes(ts):
    b = ts.ts_kmap_bytes(1000, 1000, 3, 3, 1, 0)
    assert b > 1000 * 27 * 4
    assert ts.ts_kmap_bytes(1000, 1000, 3, 3, 1, ts.TS_KMAP_PAIRS) > b
    assert ts.ts_kmap_bytes(1000, 800, 3, 2, 2, ts.TS_KMAP_BWD) > ts.ts_kmap_bytes(1000, 800, 3, 2, 2, 0)
    assert ts.ts_kmap_bytes(10, 10, 4, 3, 1, 0) == 0   # ndim 4
    assert ts.ts_kmap_bytes(10, 10, 3, 5, 1, 0) == 0   # 125 offsets > 64
    assert ts.ts_kmap_bytes(-1, 10, 3, 3, 1, 0) == 0


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def test_hash_build_rejects(ts):
    L = ts._lib_hash_build
    assert L(None, 10, 3, FAKE, 64, None, None) == ts.TS_ERR_INVALID_ARG          # null coords
    assert L(FAKE, 10, 3, None, 64, None, None) == ts.TS_ERR_INVALID_ARG          # null table
    assert L(FAKE, -1, 3, FAKE, 64, None, None) == ts.TS_ERR_INVALID_ARG          # n < 0
    assert L(FAKE, 10, 4, FAKE, 64, None, None) == ts.TS_ERR_INVALID_ARG          # ndim
    assert L(FAKE, 10, 3, FAKE, 48, None, None) == ts.TS_ERR_INVALID_ARG          # cap not a power of 2
    assert L(FAKE, 100, 3, FAKE, 64, None, None) == ts.TS_ERR_INVALID_ARG         # cap < n


def test_hash_query_rejects(ts):
    L = ts._lib_hash_query
    assert L(None, 64, 3, FAKE, 5, FAKE, None) == ts.TS_ERR_INVALID_ARG
    assert L(FAKE, 64, 3, None, 5, FAKE, None) == ts.TS_ERR_INVALID_ARG
    assert L(FAKE, 63, 3, FAKE, 5, FAKE, None) == ts.TS_ERR_INVALID_ARG
    assert L(FAKE, 64, 1, FAKE, 5, FAKE, None) == ts.TS_ERR_INVALID_ARG


def test_kmap_build_rejects(ts):
    L = ts._lib_kmap_build
    km = ts.TsKmap()
    ref = ctypes.byref(km)
    need = ts.ts_kmap_bytes(100, 100, 3, 3, 1, 0)
    args = dict(in_coords=FAKE, n_in=100, in_table=FAKE, in_cap=256, out_coords=None, n_out_cap=0, n_out=None,
                out_table=None, out_cap=0, ndim=3, ksize=3, stride=1, flags=0, buf=FAKE, buf_bytes=need)

    def call(**kw):
        a = dict(args, **kw)
        return L(a["in_coords"], a["n_in"], a["in_table"], a["in_cap"], a["out_coords"], a["n_out_cap"], a["n_out"],
                 a["out_table"], a["out_cap"], a["ndim"], a["ksize"], a["stride"], a["flags"], a["buf"],
                 a["buf_bytes"], ref, None)

    assert call(buf_bytes=need - 1) == ts.TS_ERR_INVALID_ARG       # short buffer
    assert call(ksize=2) == ts.TS_ERR_UNSUPPORTED                  # even submanifold kernel
    assert call(ksize=5) == ts.TS_ERR_UNSUPPORTED                  # 125 offsets
    assert call(ndim=1) == ts.TS_ERR_INVALID_ARG
    assert call(stride=0) == ts.TS_ERR_INVALID_ARG
    assert call(in_table=None) == ts.TS_ERR_INVALID_ARG
    assert call(in_cap=100) == ts.TS_ERR_INVALID_ARG
    assert call(flags=64) == ts.TS_ERR_INVALID_ARG
    # int32 neighbour tables and pair positions: more than 2^31 - 1 (row,
    # offset) slots, e.g. 80M rows at 27 offsets, is refused up front
    big = 80_000_000
    assert call(n_in=big, in_cap=1 << 25, flags=ts.TS_KMAP_PAIRS) == ts.TS_ERR_UNSUPPORTED
    assert call(n_in=big, in_cap=1 << 25) == ts.TS_ERR_UNSUPPORTED
    assert ts.ts_kmap_bytes(big, big, 3, 3, 1, ts.TS_KMAP_PAIRS) == 0
    # strided maps need the output count and coordinates
    sneed = ts.ts_kmap_bytes(100, 100, 3, 2, 2, ts.TS_KMAP_BWD)
    assert call(stride=2, ksize=2, n_out_cap=100, buf_bytes=sneed) == ts.TS_ERR_INVALID_ARG
    assert call(stride=2, ksize=2, n_out_cap=100, out_coords=FAKE, n_out=FAKE, flags=ts.TS_KMAP_BWD,
                buf_bytes=sneed) == ts.TS_ERR_INVALID_ARG          # BWD without an output table


def test_conv_rejects(ts):
    km = ts.TsKmap()
    ref = ctypes.byref(km)
    # an unbuilt map
    assert ts._lib_conv_fwd(ref, FAKE, 16, FAKE, 16, FAKE, 1, 1, 0, None, 0, None) == ts.TS_ERR_INVALID_ARG
    # a map that looks built
    km.kvol = 27
    km.stride = 1
    km.n_in = km.n_out_cap = 100
    km.fwd.tile_mask = 0x2000
    km.fwd.row_mask = 0x3000
    km.fwd.n_tiles = 7
    assert ts._lib_conv_fwd(ref, FAKE, 0, FAKE, 16, FAKE, 1, 1, 0, None, 0, None) == ts.TS_ERR_INVALID_ARG   # cin 0
    assert ts._lib_conv_fwd(ref, FAKE, 16, FAKE, 16, FAKE, 7, 1, 0, None, 0, None) == ts.TS_ERR_INVALID_ARG  # dtype
    assert ts._lib_conv_fwd(ref, FAKE, 16, FAKE, 16, FAKE, 1, 2, 0, None, 0, None) == ts.TS_ERR_UNSUPPORTED  # f16->bf16
    assert ts._lib_conv_fwd(ref, None, 64, FAKE, 64, FAKE, 1, 1, 0, None, 0, None) == ts.TS_ERR_INVALID_ARG  # null x
    assert ts._lib_conv_fwd(ref, FAKE, 64, FAKE, 64, None, 1, 1, 0, None, 0, None) == ts.TS_ERR_INVALID_ARG  # null y
    assert ts._lib_conv_fwd(ref, FAKE, 64, FAKE, 64, FAKE, 1, 1, 2, FAKE, 1 << 30, None) == ts.TS_ERR_INVALID_ARG  # GS w/o pairs
    assert ts._lib_conv_fwd(ref, FAKE, 16, None, 16, FAKE, 1, 1, 0, None, 0, None) == ts.TS_ERR_INVALID_ARG  # null w
    assert ts._lib_conv_fwd(ref, FAKE, 16, FAKE, 16, FAKE, 1, 1, 9, None, 0, None) == ts.TS_ERR_INVALID_ARG  # dataflow
    # fetch on demand needs the pair groups; a map without groups or table is no map
    FOD = ts.TS_DATAFLOW_FETCH_ON_DEMAND
    assert ts._lib_conv_fwd(ref, FAKE, 64, FAKE, 64, FAKE, 1, 1, FOD, None, 0, None) == ts.TS_ERR_INVALID_ARG
    km.fwd.tile_mask = None
    assert ts._lib_conv_fwd(ref, FAKE, 64, FAKE, 64, FAKE, 1, 1, 0, None, 0, None) == ts.TS_ERR_INVALID_ARG
    km.fwd.gcount = 0x4000
    km.fwd.n_gtiles = 1
    assert ts._lib_conv_fwd(ref, FAKE, 64, FAKE, 64, FAKE, 0, 0, FOD, None, 0, None) == ts.TS_ERR_UNSUPPORTED  # fp32
    assert ts._lib_conv_fwd(ref, FAKE, 64, FAKE, 64, FAKE, 1, 1, 1, None, 0, None) == ts.TS_ERR_INVALID_ARG  # igemm, no table
    assert ts._lib_pool_fwd(ref, FAKE, 16, FAKE, 1, 1, 0, None) == ts.TS_ERR_INVALID_ARG  # pooling needs the table
    km.fwd.tile_mask = 0x2000
    km.fwd.gcount = None
    km.fwd.n_gtiles = 0
    # wgrad needs the pair lists
    assert ts._lib_conv_bwd_wgrad(ref, FAKE, 16, FAKE, 16, 1, FAKE, FAKE, 1 << 30, None) == ts.TS_ERR_INVALID_ARG
    # dgrad of a strided map needs the transposed relation
    km.stride = 2
    km.mirror_bwd = 0
    assert ts._lib_conv_bwd_dgrad(ref, FAKE, 16, FAKE, 16, FAKE, 1, 1, 0, None, 0, None) == ts.TS_ERR_INVALID_ARG
    km.stride = 1
    assert ts._lib_subm_conv_fwd(ref, FAKE, 16, FAKE, 16, FAKE, 9, 1, 0, None, 0, None) == ts.TS_ERR_INVALID_ARG


def test_pack_weights_rejects(ts):
    km = ts.TsKmap()
    ref = ctypes.byref(km)
    FAKE = ctypes.c_void_p(0x1000)
    P = ts._lib_conv_pack_weights
    assert P(ref, FAKE, 64, 64, ts.TS_OP_FWD, ts.TS_F16, FAKE, 1 << 30, None) == ts.TS_ERR_INVALID_ARG  # no map yet
    km.kvol = 27
    km.stride = 1
    km.mirror_bwd = 1
    km.n_in = km.n_out_cap = 100
    km.fwd.tile_mask = 0x2000
    km.fwd.row_mask = 0x3000
    need = ts._lib_conv_workspace_bytes(ref, 64, 64, ts.TS_OP_FWD, ts.TS_F16, ts.TS_DATAFLOW_IMPLICIT_GEMM)
    assert need == 27 * 64 * 64 * 2
    assert P(ref, None, 64, 64, ts.TS_OP_FWD, ts.TS_F16, FAKE, need, None) == ts.TS_ERR_INVALID_ARG       # null w
    assert P(ref, FAKE, 64, 64, ts.TS_OP_FWD, ts.TS_F16, None, need, None) == ts.TS_ERR_INVALID_ARG       # null ws
    assert P(ref, FAKE, 64, 64, ts.TS_OP_FWD, ts.TS_F16, FAKE, need - 1, None) == ts.TS_ERR_INVALID_ARG   # short ws
    assert P(ref, FAKE, 64, 64, ts.TS_OP_WGRAD, ts.TS_F16, FAKE, need, None) == ts.TS_ERR_INVALID_ARG     # op
    assert P(ref, FAKE, 64, 64, 7, ts.TS_F16, FAKE, need, None) == ts.TS_ERR_INVALID_ARG                  # op
    assert P(ref, FAKE, 0, 64, ts.TS_OP_FWD, ts.TS_F16, FAKE, need, None) == ts.TS_ERR_INVALID_ARG        # cin
    assert P(ref, FAKE, 64, 64, ts.TS_OP_FWD, ts.TS_F32, FAKE, need, None) == ts.TS_ERR_UNSUPPORTED       # fp32
    assert P(ref, FAKE, 48, 64, ts.TS_OP_FWD, ts.TS_F16, FAKE, need, None) == ts.TS_ERR_UNSUPPORTED       # cin % 32
    # the packed dataflow: unsupported shapes are refused, w may be null, the range ends at 3
    F = ts._lib_conv_fwd
    assert F(ref, FAKE, 16, None, 16, FAKE, 1, 1, 3, FAKE, 1 << 30, None) == ts.TS_ERR_UNSUPPORTED
    assert F(ref, FAKE, 64, None, 64, FAKE, 1, 1, 1, FAKE, 1 << 30, None) == ts.TS_ERR_INVALID_ARG
    assert F(ref, FAKE, 64, None, 64, FAKE, 1, 1, 4, FAKE, 1 << 30, None) == ts.TS_ERR_INVALID_ARG
    assert F(ref, FAKE, 64, None, 64, FAKE, 1, 1, 3, FAKE, need - 1, None) == ts.TS_ERR_INVALID_ARG   # short ws
    D = ts._lib_conv_bwd_dgrad
    assert D(ref, FAKE, 16, None, 16, FAKE, 1, 1, 3, FAKE, 1 << 30, None) == ts.TS_ERR_UNSUPPORTED


def test_workspace_sizes(ts):
    km = ts.TsKmap()
    km.kvol = 27
    km.n_in = km.n_out_cap = 1000
    km.pair_cap = 27000
    ref = ctypes.byref(km)
    # implicit GEMM: the weights packed in MFMA fragment order (kvol * Cout * Cin fp16/bf16)
    assert ts._lib_conv_workspace_bytes(ref, 64, 64, ts.TS_OP_FWD, ts.TS_F16, 0) == 27 * 64 * 64 * 2
    assert ts._lib_conv_workspace_bytes(ref, 48, 128, ts.TS_OP_DGRAD, ts.TS_BF16, 0) == 27 * 48 * 128 * 2
    assert ts._lib_conv_workspace_bytes(ref, 16, 16, ts.TS_OP_FWD, ts.TS_F32, 0) == 0
    assert ts._lib_conv_workspace_bytes(ref, 64, 64, ts.TS_OP_FWD, ts.TS_F16, 2) >= 1000 * 64 * 4
    assert ts._lib_conv_workspace_bytes(ref, 64, 64, ts.TS_OP_WGRAD, ts.TS_F16, 0) >= 27 * 64 * 64 * 4


def test_target_and_generative_sizes(ts):
    T = ts.TS_KMAP_TARGET
    base = ts.ts_kmap_bytes(100, 100, 3, 3, 1, 0)
    assert ts.ts_kmap_bytes(100, 300, 3, 3, 1, T) > base                   # sized by the target count
    assert ts.ts_kmap_bytes(100, 300, 3, 3, 1, T | ts.TS_KMAP_BWD) > ts.ts_kmap_bytes(100, 300, 3, 3, 1, T)
    assert ts.ts_kmap_bytes(100, 100, 3, 3, 1, ts.TS_KMAP_BWD) == base     # a submanifold map has no own bwd
    # a target map's pair lists hold kvol per target (targets may repeat)
    p_t = ts.ts_kmap_bytes(100, 100, 3, 2, 2, T | ts.TS_KMAP_PAIRS) - ts.ts_kmap_bytes(100, 100, 3, 2, 2, T)
    p_s = ts.ts_kmap_bytes(100, 100, 3, 2, 2, ts.TS_KMAP_PAIRS) - ts.ts_kmap_bytes(100, 100, 3, 2, 2, 0)
    assert p_t >= p_s + (100 * 8 - 100) * 8
    assert ts.ts_generative_scratch_bytes(100, 3, 3) >= 3 * 100 * 27 * 4
    assert ts.ts_generative_scratch_bytes(-1, 3, 3) == 0
    assert ts.ts_generative_scratch_bytes(10, 3, 5) == 0                   # 125 offsets
    assert ts.ts_generative_scratch_bytes(10, 4, 3) == 0


def test_target_map_rejects(ts):
    L = ts._lib_kmap_build
    km = ts.TsKmap()
    T = ts.TS_KMAP_TARGET
    need = ts.ts_kmap_bytes(100, 50, 3, 3, 1, T | ts.TS_KMAP_BWD)
    # no target coordinates / count
    assert L(FAKE, 100, FAKE, 256, None, 50, FAKE, None, 0, 3, 3, 1, T, FAKE, need, ctypes.byref(km), None) \
        == ts.TS_ERR_INVALID_ARG
    assert L(FAKE, 100, FAKE, 256, FAKE, 50, None, None, 0, 3, 3, 1, T, FAKE, need, ctypes.byref(km), None) \
        == ts.TS_ERR_INVALID_ARG
    # the transposed relation needs the targets' table
    assert L(FAKE, 100, FAKE, 256, FAKE, 50, FAKE, None, 0, 3, 3, 1, T | ts.TS_KMAP_BWD, FAKE, need,
             ctypes.byref(km), None) == ts.TS_ERR_INVALID_ARG
    # a short buffer
    assert L(FAKE, 100, FAKE, 256, FAKE, 50, FAKE, FAKE, 256, 3, 3, 1, T | ts.TS_KMAP_BWD, FAKE, need - 1,
             ctypes.byref(km), None) == ts.TS_ERR_INVALID_ARG
    # a target map is not a submanifold map
    km.kvol, km.stride, km.flags = 27, 1, T
    km.n_in = km.n_out_cap = 100
    km.fwd.tile_mask, km.fwd.n_tiles = 0x2000, 7
    assert ts._lib_subm_conv_fwd(ctypes.byref(km), FAKE, 16, FAKE, 16, FAKE, 0, 0, 0, None, 0, None) \
        == ts.TS_ERR_INVALID_ARG


def test_generative_rejects(ts):
    G = ts._lib_generative_support
    sb = ts.ts_generative_scratch_bytes(100, 3, 3)
    ok = [FAKE, 100, 3, 3, FAKE, 2700, FAKE, FAKE, 1024, FAKE, sb, None, None]

    def call(i, v):
        a = list(ok)
        a[i] = v
        return G(*a)

    assert call(6, None) == ts.TS_ERR_INVALID_ARG        # n_out
    assert call(7, None) == ts.TS_ERR_INVALID_ARG        # out_table
    assert call(8, 1000) == ts.TS_ERR_INVALID_ARG        # out_cap not a power of two
    assert call(10, sb - 1) == ts.TS_ERR_INVALID_ARG     # short scratch
    assert call(5, -1) == ts.TS_ERR_INVALID_ARG          # n_out_cap < 0
    assert call(4, None) == ts.TS_ERR_INVALID_ARG        # no output coordinates
    assert call(3, 5) == ts.TS_ERR_INVALID_ARG           # 125 offsets
    assert call(0, None) == ts.TS_ERR_INVALID_ARG        # no input coordinates
    C = ts._lib_conv_fwd_generative
    kb = ts.ts_kmap_bytes(100, 2700, 3, 3, 1, ts.TS_KMAP_TARGET)
    km = ts.TsKmap()
    good = [FAKE, 100, 3, FAKE, 256, 3, 0, FAKE, 2700, FAKE, FAKE, 1024, None, FAKE, kb + sb, ctypes.byref(km),
            FAKE, 64, FAKE, 64, FAKE, ts.TS_F16, ts.TS_F16, 0, FAKE, 1 << 30, None]

    def conv(i, v):
        a = list(good)
        a[i] = v
        return C(*a)

    assert conv(14, kb + sb - 1) == ts.TS_ERR_INVALID_ARG    # short map buffer
    assert conv(17, 0) == ts.TS_ERR_INVALID_ARG              # cin 0
    assert conv(22, ts.TS_BF16) == ts.TS_ERR_UNSUPPORTED     # f16 in, bf16 out
    assert conv(23, ts.TS_DATAFLOW_GATHER_SCATTER) == ts.TS_ERR_INVALID_ARG   # no pair lists
    assert conv(20, None) == ts.TS_ERR_INVALID_ARG           # null y


def test_transposed_rejects(ts):
    T = ts._lib_transposed_support
    sb = ts.ts_generative_scratch_bytes(100, 3, 2)
    ok = [FAKE, 100, 3, 2, 2, FAKE, 800, FAKE, FAKE, 1024, FAKE, sb, None, None]

    def call(i, v):
        a = list(ok)
        a[i] = v
        return T(*a)

    assert call(4, 0) == ts.TS_ERR_INVALID_ARG           # stride 0
    assert call(7, None) == ts.TS_ERR_INVALID_ARG        # n_out
    assert call(9, 100) == ts.TS_ERR_INVALID_ARG         # out_cap not a power of two
    assert call(11, sb - 1) == ts.TS_ERR_INVALID_ARG     # short scratch
    L = ts._lib_kmap_build
    km = ts.TsKmap()
    X = ts.TS_KMAP_TRANSPOSED
    need = ts.ts_kmap_bytes(100, 800, 3, 2, 2, X | ts.TS_KMAP_BWD)
    assert need > ts.ts_kmap_bytes(100, 800, 3, 2, 2, X)
    # a transposed map needs the fine outputs' table, and is not also a target map
    assert L(FAKE, 100, FAKE, 256, FAKE, 800, FAKE, None, 0, 3, 2, 2, X, FAKE, need, ctypes.byref(km), None) \
        == ts.TS_ERR_INVALID_ARG
    assert L(FAKE, 100, FAKE, 256, FAKE, 800, FAKE, FAKE, 1024, 3, 2, 2, X | ts.TS_KMAP_TARGET, FAKE, need,
             ctypes.byref(km), None) == ts.TS_ERR_INVALID_ARG
    # ConvTranspose over a strided map needs its transposed relation
    km.kvol, km.stride, km.mirror_bwd = 8, 2, 0
    km.n_in, km.n_out_cap = 100, 60
    km.fwd.tile_mask, km.fwd.n_tiles = 0x2000, 4
    assert ts._lib_conv_transpose_fwd(ctypes.byref(km), FAKE, 16, FAKE, 16, FAKE, 0, 0, 0, None, 0, None) \
        == ts.TS_ERR_INVALID_ARG
    assert ts._lib_conv_transpose_fwd(ctypes.byref(km), FAKE, 16, None, 16, FAKE, 0, 0, 0, None, 0, None) \
        == ts.TS_ERR_INVALID_ARG
    # workspace of the transposed op: the packed weights (kvol * Cout * Cin)
    km.kvol = 8
    assert ts._lib_conv_workspace_bytes(ctypes.byref(km), 128, 64, ts.TS_OP_TRANSPOSE, ts.TS_F16, 0) == 8 * 128 * 64 * 2


def test_pool_rejects_host(ts):
    km = ts.TsKmap()
    ref = ctypes.byref(km)
    assert ts._lib_pool_fwd(ref, FAKE, 8, FAKE, 1, 1, 0, None) == ts.TS_ERR_INVALID_ARG   # unbuilt map
    km.kvol, km.stride, km.n_in, km.n_out_cap = 8, 2, 100, 60
    km.fwd.tile_mask, km.fwd.n_tiles = 0x2000, 4
    assert ts._lib_pool_fwd(ref, FAKE, 0, FAKE, 1, 1, 0, None) == ts.TS_ERR_INVALID_ARG   # no channels
    assert ts._lib_pool_fwd(ref, FAKE, 8, FAKE, 1, 1, 2, None) == ts.TS_ERR_INVALID_ARG   # mode
    assert ts._lib_pool_fwd(ref, FAKE, 8, FAKE, 1, 2, 0, None) == ts.TS_ERR_UNSUPPORTED   # f16 -> bf16
    assert ts._lib_pool_fwd(ref, None, 8, FAKE, 1, 1, 0, None) == ts.TS_ERR_INVALID_ARG   # no x


def test_voxelize_rejects(ts):
    V = ts._lib_voxelize
    sz = (ctypes.c_float * 3)(0.1, 0.1, 0.1)
    og = (ctypes.c_float * 3)(0.0, 0.0, 0.0)
    bad = (ctypes.c_float * 3)(0.1, 0.0, 0.1)
    sb = ts.ts_voxelize_scratch_bytes(100)
    assert sb >= 4 * 100 * 4
    ok = [None, FAKE, 100, 3, sz, og, None, 0, FAKE, FAKE, FAKE, 256, FAKE, None, FAKE, sb, None, None]

    def call(i, v):
        a = list(ok)
        a[i] = v
        return V(*a)

    assert call(3, 4) == ts.TS_ERR_INVALID_ARG          # ndim
    assert call(4, bad) == ts.TS_ERR_INVALID_ARG        # a zero voxel size
    assert call(1, None) == ts.TS_ERR_INVALID_ARG       # no positions
    assert call(9, None) == ts.TS_ERR_INVALID_ARG       # n_out
    assert call(11, 100) == ts.TS_ERR_INVALID_ARG       # table capacity not a power of two
    assert call(15, sb - 1) == ts.TS_ERR_INVALID_ARG    # short scratch
    a = list(ok)
    a[6], a[7] = FAKE, 4                                # features but nowhere to put their means
    assert V(*a) == ts.TS_ERR_INVALID_ARG
    D = ts._lib_devoxelize
    assert D(FAKE, 10, FAKE, 0, FAKE, ts.TS_F32, None) == ts.TS_ERR_INVALID_ARG     # no channels
    assert D(None, 10, FAKE, 4, FAKE, ts.TS_F32, None) == ts.TS_ERR_INVALID_ARG     # no voxel index
    assert D(FAKE, 10, FAKE, 4, FAKE, 9, None) == ts.TS_ERR_INVALID_ARG             # dtype


DEBUG_LIB = os.path.join(ROOT, "convolution_voxelised_point_amd", "libts_debug.so")


def test_debug_violations_needs_the_debug_build():
    lib = ctypes.CDLL(LIB)
    lib.ts_debug_violations.argtypes = [ctypes.c_void_p]
    bits = ctypes.c_uint32(0)
    assert lib.ts_debug_violations(ctypes.byref(bits)) == 2      # TS_ERR_UNSUPPORTED: no checks here


@pytest.mark.skipif(not os.path.exists(DEBUG_LIB), reason="libts_debug.so not built")
def test_debug_build_exports_and_identifies():
    lib = ctypes.CDLL(DEBUG_LIB)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    lib.ts_version.restype = ctypes.c_char_p
    assert b"bounds checks" in lib.ts_version()
    lib.ts_debug_violations.argtypes = [ctypes.c_void_p]
    assert lib.ts_debug_violations(None) == 1                    # TS_ERR_INVALID_ARG, before touching the GPU
    lib2 = ctypes.CDLL(LIB)
    lib2.ts_version.restype = ctypes.c_char_p
    assert b"bounds checks" not in lib2.ts_version()
