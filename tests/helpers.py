"""Shared test helpers: tolerance checks, triple canonicalisation, tensors."""
from __future__ import annotations

import numpy as np
import torch

# unit roundoff of the low-precision storage types
U_OUT = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8, torch.float32: 0.0}


def canon(tr) -> np.ndarray:
    """Triples (in, out, offset) as a lexicographically sorted (P, 3) array."""
    a = np.stack([np.asarray(t, dtype=np.int64) for t in tr], axis=1) if len(tr[0]) else np.zeros((0, 3), np.int64)
    return a[np.lexsort(a.T[::-1])] if len(a) else a.reshape(0, 3)


def err_stats(got: np.ndarray, ref: np.ndarray) -> str:
    e = np.abs(got - ref).ravel()
    if e.size == 0:
        return "empty"
    m = float(np.abs(ref).max())
    return (f"max|ref|={m:.3e} err p50={np.percentile(e, 50):.3e} p99={np.percentile(e, 99):.3e} "
            f"max={e.max():.3e} rel(max)={e.max() / max(m, 1e-300):.3e}")


# Error statistics of every feature comparison made in this session (what,
# elements, max|ref|, p50, p99, max of |err|, max|err| / max|ref|, the bar);
# tests/conftest.py prints them at the end of the run.
PARITY_LOG: list = []


def assert_feature_close(got: torch.Tensor, ref: np.ndarray, in_dtype: torch.dtype, what: str = "") -> None:
    """Parity bar: max|err| <= 1e-5 max|ref| (fp32 inputs) or 2e-3 max|ref|
    (fp16/bf16 inputs, fp32 accumulation), with max over the whole tensor; a
    low-precision output adds its own rounding, u_out*|ref| per element."""
    g = got.detach().to("cpu", torch.float64).numpy()
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    if ref.size == 0:
        return
    m = float(np.abs(ref).max())
    rel = 1e-5 if in_dtype == torch.float32 else 2e-3
    base = rel * m
    tol = base + U_OUT[got.dtype] * np.abs(ref) * (1 + 1e-6) + 1e-30
    err = np.abs(g - ref)
    e = err.ravel()
    PARITY_LOG.append((what, int(e.size), m, float(np.percentile(e, 50)), float(np.percentile(e, 99)),
                       float(e.max()), float(e.max()) / max(m, 1e-300),
                       f"{rel:g}*max|ref|" + (f" + {U_OUT[got.dtype]:g}*|ref|" if U_OUT[got.dtype] else "")))
    bad = err > tol
    assert not bad.any(), f"{what}: {int(bad.sum())} elements over tolerance; {err_stats(g, ref)}"


def dev(a, dtype=None) -> torch.Tensor:
    t = torch.as_tensor(a)
    if dtype is not None:
        t = t.to(dtype)
    return t.contiguous().cuda()


def check_window_sorted(slots, rm, window=4096):
    """Inside each window of slots, rows are ordered by (folded) offset mask,
    ties in row order, and every window holds exactly its own rows."""
    for w0 in range(0, len(slots), window):
        rows = slots[w0:w0 + window]
        rows = rows[rows >= 0]
        np.testing.assert_array_equal(np.sort(rows), np.arange(w0, w0 + len(rows)))
        m = rm[rows]
        key = (m ^ (m >> np.uint64(32))) & np.uint64(0xffffffff)
        order = np.lexsort((rows, key))
        np.testing.assert_array_equal(order, np.arange(len(rows)))
