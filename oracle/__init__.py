"""CPU oracle for the sparse-convolution path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library never calls it, and it shares no code
with the GPU library.  The arithmetic lives in ``oracle.cpp`` (plain C++,
``std::unordered_map``, fp64); this module compiles it with g++ and wraps it
with ctypes and numpy.

Every function is pinned by ``tests/test_oracle_*.py`` against dense
convolution, brute force, closed forms and a hand-derived worked example.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.cpp`` into ``liboracle.so`` next to it."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-o", tmp, _SRC])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        p = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int
        L.oracle_hash_query.argtypes = [p, i64, i32, p, i64, p, p]
        L.oracle_hash_query.restype = i64
        L.oracle_strided_support.argtypes = [p, i64, i32, i32, p]
        L.oracle_strided_support.restype = i64
        L.oracle_generative_support.argtypes = [p, i64, i32, i32, p, i64]
        L.oracle_generative_support.restype = i64
        L.oracle_transposed_support.argtypes = [p, i64, i32, i32, i32, p, i64]
        L.oracle_transposed_support.restype = i64
        L.oracle_kmap_transposed.argtypes = [p, i64, p, i64, i32, i32, i32, p, p, p, i64]
        L.oracle_kmap_transposed.restype = i64
        L.oracle_kmap.argtypes = [p, i64, p, i64, i32, i32, i32, i32, p, p, p, i64]
        L.oracle_kmap.restype = i64
        L.oracle_conv_fwd.argtypes = [p, p, p, i64, p, i32, p, i32, p, i64]
        L.oracle_conv_fwd.restype = None
        L.oracle_conv_dgrad.argtypes = [p, p, p, i64, p, i32, p, i32, p, i64]
        L.oracle_conv_dgrad.restype = None
        L.oracle_conv_wgrad.argtypes = [p, p, p, i64, p, i32, p, i32, p, i32]
        L.oracle_conv_wgrad.restype = None
        L.oracle_pool.argtypes = [p, p, i64, p, i32, i32, p, i64]
        L.oracle_pool.restype = None
        L.oracle_voxelize.argtypes = [p, p, i64, i32, p, p, p, i32, p, p, p]
        L.oracle_voxelize.restype = i64
        L.oracle_graph_conv.argtypes = [p, p, p, i64, p, i32, p, i32, p]
        L.oracle_graph_conv.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _coords(c) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(c, dtype=np.int32))
    assert c.ndim == 2 and c.shape[1] in (3, 4), c.shape
    return c


def _f64(a) -> np.ndarray:
    """Exact widening of fp32/fp16/bf16 values (numpy or torch) to fp64."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def hash_query(coords, queries) -> Tuple[np.ndarray, int]:
    """Rows owning each query coordinate (-1 if absent) and the DUP/RANGE
    flags (1 = duplicate coordinate, 2 = coordinate out of range)."""
    c, q = _coords(coords), _coords(queries)
    assert c.shape[1] == q.shape[1]
    rows = np.empty(q.shape[0], np.int32)
    flags = np.zeros(1, np.uint32)
    lib().oracle_hash_query(_ptr(c), c.shape[0], c.shape[1] - 1, _ptr(q), q.shape[0], _ptr(rows), _ptr(flags))
    return rows, int(flags[0])


def strided_support(coords, stride: int) -> np.ndarray:
    """Output coordinates unique(floor(c/stride)) in first-occurrence order."""
    c = _coords(coords)
    out = np.empty_like(c)
    n_out = lib().oracle_strided_support(_ptr(c), c.shape[0], c.shape[1] - 1, stride, _ptr(out))
    return out[:n_out].copy()


def generative_support(coords, ksize: int) -> np.ndarray:
    """Output coordinates a stride-1 convolution generates: every site
    c_i - delta_o, in first-occurrence order over (input row, offset)."""
    c = _coords(coords)
    ndim = c.shape[1] - 1
    cap = max(1, c.shape[0] * ksize ** ndim)
    out = np.empty((cap, ndim + 1), np.int32)
    n_out = lib().oracle_generative_support(_ptr(c), c.shape[0], ndim, ksize, _ptr(out), cap)
    assert n_out <= cap
    return out[:n_out].copy()


def transposed_support(coords, ksize: int, stride: int) -> np.ndarray:
    """Output coordinates a transposed convolution of stride s generates:
    every site s*c_j + delta_o, first-occurrence order over (input row,
    offset)."""
    c = _coords(coords)
    ndim = c.shape[1] - 1
    cap = max(1, c.shape[0] * ksize ** ndim)
    out = np.empty((cap, ndim + 1), np.int32)
    n_out = lib().oracle_transposed_support(_ptr(c), c.shape[0], ndim, ksize, stride, _ptr(out), cap)
    assert n_out <= cap
    return out[:n_out].copy()


def kmap_transposed(in_coords, out_coords, ksize: int, stride: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Triples (coarse input row, fine output row, offset) of the transposed
    relation: p_out = stride * q_in + delta_offset."""
    ci, co = _coords(in_coords), _coords(out_coords)
    ndim = ci.shape[1] - 1
    cap = max(1, co.shape[0] * ksize ** ndim)
    t_in = np.empty(cap, np.int32)
    t_out = np.empty(cap, np.int32)
    t_off = np.empty(cap, np.int32)
    n = lib().oracle_kmap_transposed(_ptr(ci), ci.shape[0], _ptr(co), co.shape[0], ndim, ksize, stride,
                                     _ptr(t_in), _ptr(t_out), _ptr(t_off), cap)
    assert n <= cap
    return t_in[:n].copy(), t_out[:n].copy(), t_off[:n].copy()


def conv_transpose(triples, x, w, n_dest: int) -> np.ndarray:
    """ConvTranspose over an existing relation (in, out, offset): the output
    is indexed by the relation's input rows, y[in] = sum x[out] . w[offset]
    with w[kvol][C of x][C of y] -- the forward formula over the relation read
    the other way."""
    t_in, t_out, t_off = triples
    return conv_fwd((t_out, t_in, t_off), x, w, n_dest)


def kmap(in_coords, out_coords, ksize: int, stride: int = 1,
         target: bool = False) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Kernel-map triples (in, out, offset), ordered by (out, offset).  With
    `target` the output rows are caller coordinates (no ownership test at
    stride 1)."""
    ci, co = _coords(in_coords), _coords(out_coords)
    ndim = ci.shape[1] - 1
    kvol = ksize ** ndim
    cap = max(1, co.shape[0] * kvol)
    t_in = np.empty(cap, np.int32)
    t_out = np.empty(cap, np.int32)
    t_off = np.empty(cap, np.int32)
    n = lib().oracle_kmap(_ptr(ci), ci.shape[0], _ptr(co), co.shape[0], ndim, ksize, stride, 1 if target else 0,
                          _ptr(t_in), _ptr(t_out), _ptr(t_off), cap)
    assert n <= cap
    return t_in[:n].copy(), t_out[:n].copy(), t_off[:n].copy()


def conv_fwd(triples, x, w, n_out: int) -> np.ndarray:
    t_in, t_out, t_off = (np.ascontiguousarray(t, dtype=np.int32) for t in triples)
    x, w = _f64(x), _f64(w)
    cin, cout = w.shape[1], w.shape[2]
    assert x.shape[1] == cin
    y = np.empty((n_out, cout), np.float64)
    lib().oracle_conv_fwd(_ptr(t_in), _ptr(t_out), _ptr(t_off), t_in.shape[0], _ptr(x), cin, _ptr(w), cout,
                          _ptr(y), n_out)
    return y


def conv_dgrad(triples, dy, w, n_in: int) -> np.ndarray:
    t_in, t_out, t_off = (np.ascontiguousarray(t, dtype=np.int32) for t in triples)
    dy, w = _f64(dy), _f64(w)
    cin, cout = w.shape[1], w.shape[2]
    assert dy.shape[1] == cout
    dx = np.empty((n_in, cin), np.float64)
    lib().oracle_conv_dgrad(_ptr(t_in), _ptr(t_out), _ptr(t_off), t_in.shape[0], _ptr(dy), cout, _ptr(w), cin,
                            _ptr(dx), n_in)
    return dx


def conv_wgrad(triples, x, dy, kvol: int) -> np.ndarray:
    t_in, t_out, t_off = (np.ascontiguousarray(t, dtype=np.int32) for t in triples)
    x, dy = _f64(x), _f64(dy)
    cin, cout = x.shape[1], dy.shape[1]
    dw = np.empty((kvol, cin, cout), np.float64)
    lib().oracle_conv_wgrad(_ptr(t_in), _ptr(t_out), _ptr(t_off), t_in.shape[0], _ptr(x), cin, _ptr(dy), cout,
                            _ptr(dw), kvol)
    return dw


def pool(triples, x, n_out: int, mode: str) -> np.ndarray:
    """Max ("max") or mean ("avg") of x over each output's present inputs;
    0 for an output with none."""
    t_in, t_out, _ = (np.ascontiguousarray(t, dtype=np.int32) for t in triples)
    x = _f64(x)
    c = x.shape[1]
    y = np.empty((n_out, c), np.float64)
    lib().oracle_pool(_ptr(t_in), _ptr(t_out), t_in.shape[0], _ptr(x), c, {"max": 0, "avg": 1}[mode], _ptr(y), n_out)
    return y


def voxelize(batch, pos, size, origin, feats):
    """(voxel coords [M][D+1] int32 in first-occurrence order, voxel of each
    point [N] (-1 when dropped), mean features [M][C] fp64).  Positions,
    size and origin are float32; the voxel of a point is decided in float32."""
    pos = np.ascontiguousarray(np.asarray(pos, dtype=np.float32))
    n, ndim = pos.shape
    b = None if batch is None else np.ascontiguousarray(np.asarray(batch, dtype=np.int32))
    size = np.ascontiguousarray(np.asarray(size, dtype=np.float32))
    origin = np.ascontiguousarray(np.asarray(origin, dtype=np.float32))
    f = _f64(feats)
    c = f.shape[1]
    out = np.empty((max(n, 1), ndim + 1), np.int32)
    vox_of = np.empty(max(n, 1), np.int32)
    y = np.empty((max(n, 1), c), np.float64)
    m = lib().oracle_voxelize(None if b is None else _ptr(b), _ptr(pos), n, ndim, _ptr(size), _ptr(origin), _ptr(f), c,
                              _ptr(out), _ptr(vox_of), _ptr(y))
    return out[:m].copy(), vox_of[:n].copy(), y[:m].copy()


def graph_conv(indptr, src, rel, x, w) -> np.ndarray:
    """Relational graph convolution over CSR edges (grouped by destination):
    y[v] = sum over v's edges e of x[src[e]] . w[rel[e]]."""
    indptr = np.ascontiguousarray(np.asarray(indptr, dtype=np.int64))
    src = np.ascontiguousarray(np.asarray(src, dtype=np.int32))
    rel = np.ascontiguousarray(np.asarray(rel, dtype=np.int32))
    x, w = _f64(x), _f64(w)
    n_dst = indptr.shape[0] - 1
    cin, cout = w.shape[1], w.shape[2]
    y = np.empty((max(n_dst, 1), cout), np.float64)
    lib().oracle_graph_conv(_ptr(indptr), _ptr(src), _ptr(rel), n_dst, _ptr(x), cin, _ptr(w), cout, _ptr(y))
    return y[:n_dst].copy()


def subm_conv(coords, x, w, ksize: int):
    """Submanifold convolution: output rows = input rows.  Returns (y, triples)."""
    c = _coords(coords)
    tr = kmap(c, c, ksize, 1)
    return conv_fwd(tr, x, w, c.shape[0]), tr


def strided_conv(coords, x, w, ksize: int, stride: int):
    """Strided convolution.  Returns (out_coords, y, triples)."""
    c = _coords(coords)
    oc = strided_support(c, stride)
    tr = kmap(c, oc, ksize, stride)
    return oc, conv_fwd(tr, x, w, oc.shape[0]), tr
