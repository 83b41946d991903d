"""Seeded synthetic inputs for the sparse-convolution path.

This module only makes inputs: integer coordinates, feature rows, weights and
upstream gradients.  It holds none of the convolution's arithmetic (no hashing,
no kernel map, no contraction), so both the CPU oracle and the HIP library can
be fed from it without sharing any of the method's code.

Workloads (all seeded with ``numpy.random.default_rng``):

* ``tiny``      -- 5,000 unique voxels drawn uniformly from a 64^3 grid, one
                   batch, fp32 features with 16 channels, 3x3x3 kernel.
* ``lidar``     -- one synthetic LiDAR-like ring scan (~100k voxels at 0.1 m),
                   fp16 features, 64 -> 64 channels, 3x3x3 submanifold kernel.
* ``down``      -- two ring-scan scenes (~200k voxels), fp16, 64 -> 128
                   channels, 2x2x2 kernel with stride 2.
* ``pixels``    -- 4,096 images of 64x64 with ~40 active pixels each along
                   1-3 straight tracks carrying exponential charge; 2-D, fp16,
                   1 -> 8 then 8 -> 8 channels, 3x3 kernel.
* ``train``     -- four ring-scan scenes (~300k voxels), bf16, 128 -> 128
                   channels, 3x3x3 kernel, with an upstream gradient.

Seeds: the geometry of scene/image ``b`` of workload number ``c`` (1..5 in
the order above) uses ``1000*c + b``; features ``1000*c + 900``; weights
``1000*c + 901`` (second pixel layer ``1000*c + 902``); upstream gradient
``1000*c + 903``; the row permutation of a shuffled variant ``1000*c + 904``;
the coarse features and weights of a transposed layer ``1000*c + 905`` and
``1000*c + 906``; the per-point features of a voxelization ``1000*c + 907``.  Low-precision values are drawn in fp32 and rounded to the
storage type with round-to-nearest-even (torch's float conversion).

Ring-scan scene (stands in for the autonomous-driving LiDAR benchmarks, whose
data is not available): 64 rings on the ground plane with radii spread evenly
over 2..70 m, ``n_az`` points per ring at uniform azimuth and uniform
z-noise in [-0.2, 0.2] m; plus 40 axis-aligned boxes (centre at radius
U(5, 60) m and uniform angle, sides U(1, 5) m, resting on z = 0) with
``box_pts`` points spread uniformly over their six faces (area weighted).
Points are quantised at 0.1 m from the origin (-75, -75, -1) m, deduplicated,
and rows are ordered lexicographically by (b, x, y, z).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import numpy as np
import torch

WORKLOADS = ("tiny", "lidar", "down", "pixels", "train")
WORKLOAD_INDEX = {name: i + 1 for i, name in enumerate(WORKLOADS)}

VOXEL = 0.1
ORIGIN = np.array([-75.0, -75.0, -1.0])


# --------------------------------------------------------------------------
# geometry
# --------------------------------------------------------------------------
def ring_scan_points(seed: int, n_az: int, box_pts: int, n_rings: int = 64,
                     n_boxes: int = 40) -> np.ndarray:
    """Points (M, 3) of one synthetic ring scan, in metres."""
    rng = np.random.default_rng(seed)
    radii = 2.0 + 68.0 * np.arange(n_rings) / (n_rings - 1)
    pts: List[np.ndarray] = []
    for r in radii:
        az = rng.uniform(0.0, 2.0 * math.pi, n_az)
        z = rng.uniform(-0.2, 0.2, n_az)
        pts.append(np.stack([r * np.cos(az), r * np.sin(az), z], axis=1))
    for _ in range(n_boxes):
        cr = rng.uniform(5.0, 60.0)
        ca = rng.uniform(0.0, 2.0 * math.pi)
        sx, sy, sz = rng.uniform(1.0, 5.0, 3)
        cx, cy = cr * math.cos(ca), cr * math.sin(ca)
        lo = np.array([cx - sx / 2, cy - sy / 2, 0.0])
        size = np.array([sx, sy, sz])
        # faces: (fixed axis, side); areas weight the face choice
        areas = np.array([sy * sz, sy * sz, sx * sz, sx * sz, sx * sy, sx * sy])
        face = rng.choice(6, size=box_pts, p=areas / areas.sum())
        u = rng.uniform(0.0, 1.0, (box_pts, 3))
        p = lo + u * size
        axis = face // 2
        side = face % 2
        p[np.arange(box_pts), axis] = lo[axis] + side * size[axis]
        pts.append(p)
    return np.concatenate(pts, axis=0)


def voxelise(points: np.ndarray) -> np.ndarray:
    """Integer voxel indices (M, 3) of metre-valued points at 0.1 m."""
    return np.floor((points - ORIGIN) / VOXEL).astype(np.int64)


def ring_scan_coords(workload: int, n_scenes: int, n_az: int, box_pts: int) -> np.ndarray:
    """Deduplicated (b, x, y, z) int32 rows for ``n_scenes`` scenes, sorted."""
    rows = []
    for b in range(n_scenes):
        v = voxelise(ring_scan_points(1000 * workload + b, n_az, box_pts))
        bcol = np.full((v.shape[0], 1), b, dtype=np.int64)
        rows.append(np.concatenate([bcol, v], axis=1))
    allr = np.concatenate(rows, axis=0)
    uniq = np.unique(allr, axis=0)  # lexicographic (b, x, y, z)
    return np.ascontiguousarray(uniq.astype(np.int32))


def tiny_coords(workload: int = 1, n: int = 5000, grid: int = 64) -> np.ndarray:
    rng = np.random.default_rng(1000 * workload + 0)
    idx = rng.choice(grid ** 3, n, replace=False)
    c = np.stack([np.zeros_like(idx), idx // (grid * grid), (idx // grid) % grid, idx % grid], axis=1)
    return np.ascontiguousarray(c.astype(np.int32))


def track_image_pixels(seed: int, size: int = 64, length: float = 45.0):
    """Active pixels (k, 2) and Exp(1) charges of one track image."""
    rng = np.random.default_rng(seed)
    n_t = int(rng.integers(1, 4))
    pix = []
    for _ in range(n_t):
        x0, y0 = rng.uniform(0.0, size, 2)
        ang = rng.uniform(0.0, math.pi)
        seg = length / n_t
        t = np.arange(0.0, seg + 1e-9, 0.5)
        xs = np.floor(x0 + t * math.cos(ang)).astype(np.int64)
        ys = np.floor(y0 + t * math.sin(ang)).astype(np.int64)
        keep = (xs >= 0) & (xs < size) & (ys >= 0) & (ys < size)
        pix.append(np.stack([xs[keep], ys[keep]], axis=1))
    p = np.unique(np.concatenate(pix, axis=0), axis=0)
    charge = rng.exponential(1.0, p.shape[0])
    return p, charge


def pixel_coords(workload: int = 4, n_images: int = 4096, size: int = 64,
                 length: float = 45.0):
    """(b, x, y) int32 rows of ``n_images`` track images and their charges."""
    rows, charges = [], []
    for b in range(n_images):
        p, q = track_image_pixels(1000 * workload + b, size, length)
        rows.append(np.concatenate([np.full((p.shape[0], 1), b), p], axis=1))
        charges.append(q)
    c = np.concatenate(rows, axis=0).astype(np.int32)
    return np.ascontiguousarray(c), np.concatenate(charges).astype(np.float32)


# --------------------------------------------------------------------------
# values
# --------------------------------------------------------------------------
TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def normal(seed: int, shape, std: float, dtype: str) -> torch.Tensor:
    """fp32 N(0, std^2) draws rounded (RNE) to ``dtype``; a CPU tensor."""
    rng = np.random.default_rng(seed)
    a = (rng.standard_normal(shape) * std).astype(np.float32)
    return torch.from_numpy(a).to(TORCH_DTYPES[dtype])


def weight(seed: int, kvol: int, cin: int, cout: int, dtype: str) -> torch.Tensor:
    """Weights [kvol][cin][cout] with variance 1/(kvol*cin)."""
    return normal(seed, (kvol, cin, cout), math.sqrt(1.0 / (kvol * cin)), dtype)


@dataclass
class Workload:
    name: str
    index: int
    coords: np.ndarray            # (N, D+1) int32
    ndim: int
    ksize: int
    stride: int
    cin: int
    cout: int
    dtype: str
    x: torch.Tensor               # (N, cin)
    w: torch.Tensor               # (kvol, cin, cout)
    dy: Optional[torch.Tensor] = None
    extra: Dict[str, object] = field(default_factory=dict)

    @property
    def n(self) -> int:
        return int(self.coords.shape[0])

    @property
    def kvol(self) -> int:
        return self.ksize ** self.ndim


def make(name: str, scale: float = 1.0) -> Workload:
    """Build one named workload.  ``scale`` < 1 shrinks the point counts of
    the generated geometry (same recipe, fewer points) for quick tests."""
    c = WORKLOAD_INDEX[name]
    if name == "tiny":
        n = max(1, int(round(5000 * scale)))
        coords = tiny_coords(c, n)
        x = normal(1000 * c + 900, (coords.shape[0], 16), 1.0, "f32")
        w = weight(1000 * c + 901, 27, 16, 16, "f32")
        return Workload(name, c, coords, 3, 3, 1, 16, 16, "f32", x, w)
    if name == "lidar":
        coords = ring_scan_coords(c, 1, max(1, int(1500 * scale)), max(1, int(500 * scale)))
        x = normal(1000 * c + 900, (coords.shape[0], 64), 1.0, "f16")
        w = weight(1000 * c + 901, 27, 64, 64, "f16")
        return Workload(name, c, coords, 3, 3, 1, 64, 64, "f16", x, w)
    if name == "down":
        coords = ring_scan_coords(c, 2, max(1, int(1500 * scale)), max(1, int(500 * scale)))
        x = normal(1000 * c + 900, (coords.shape[0], 64), 1.0, "f16")
        w = weight(1000 * c + 901, 8, 64, 128, "f16")
        return Workload(name, c, coords, 3, 2, 2, 64, 128, "f16", x, w)
    if name == "pixels":
        n_img = max(1, int(round(4096 * scale)))
        coords, charge = pixel_coords(c, n_img)
        x = torch.from_numpy(charge.reshape(-1, 1)).to(torch.float16)
        w = weight(1000 * c + 901, 9, 1, 8, "f16")
        w2 = weight(1000 * c + 902, 9, 8, 8, "f16")
        return Workload(name, c, coords, 2, 3, 1, 1, 8, "f16", x, w, extra={"w2": w2})
    if name == "train":
        coords = ring_scan_coords(c, 4, max(1, int(1050 * scale)), max(1, int(400 * scale)))
        x = normal(1000 * c + 900, (coords.shape[0], 128), 1.0, "bf16")
        w = weight(1000 * c + 901, 27, 128, 128, "bf16")
        dy = normal(1000 * c + 903, (coords.shape[0], 128), 1.0, "bf16")
        return Workload(name, c, coords, 3, 3, 1, 128, 128, "bf16", x, w, dy=dy)
    raise KeyError(name)


def shuffled(w: Workload) -> Workload:
    """The same workload with its rows in a seeded random order: coordinates,
    features and upstream gradient permuted together (row i still owns
    feature row i), so the scene is unchanged but neighbouring voxels no
    longer sit in nearby rows."""
    perm = np.random.default_rng(1000 * w.index + 904).permutation(w.n)
    p = torch.from_numpy(perm)
    return replace(w, name=w.name + "_shuffled", coords=np.ascontiguousarray(w.coords[perm]),
                   x=w.x[p].contiguous(), dy=None if w.dy is None else w.dy[p].contiguous())


def random_coords(seed: int, n: int, ndim: int, batch: int, extent: int,
                  lo: int = 0) -> np.ndarray:
    """``n`` unique random rows (b, spatial...) with spatial values in
    [lo, lo + extent) -- small fuzz cases (may have fewer than ``n`` rows if
    the box is small)."""
    rng = np.random.default_rng(seed)
    b = rng.integers(0, batch, n)
    s = rng.integers(lo, lo + extent, (n, ndim))
    c = np.concatenate([b[:, None], s], axis=1)
    _, first = np.unique(c, axis=0, return_index=True)
    c = c[np.sort(first)]
    return np.ascontiguousarray(c.astype(np.int32))
