"""Coordinate-set and tensor generators (inputs only; no convolution arithmetic).

Coordinates are int32 rows (b, z, y, x).  Within one batch item rows are in
C order of (z, y, x) (the order ``numpy.argwhere`` returns); items are
concatenated in batch order.  The shapes follow the kind of data the pages'
decoders feed to SubMConv3d: thin surface shells inside a cubic grid, a fully
dense grid, unions of ellipsoid shells, and subdivided (x2 per axis, C-order
children) shells with a random subset of children kept (the pages describe
subdivide as a coordinate expansion x8 with C-order children: lato.2_mrp_mlx
README, "The scope, once measured" table, and the trellis_sparse_mrp_mlx
commit on masked upsample).

Value recipe (same for every config): draws in float64 from
``numpy.random.default_rng(seed).standard_normal(shape) * sigma``, cast to
float32, then rounded to nearest-even into the storage dtype by torch's CPU
conversion.  sigma: features 1, weights sqrt(1 / (k^3 * Cin)) (the fan-in
variance), bias sqrt(0.1).  Seeds: features 1000*c + 100 + l, weights
1000*c + 200 + l, bias 1000*c + 300 + l, coordinates of batch item m
1000*c + m, with c the config number and l the layer index.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

_TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Config:
    key: str            # "1", "2a", "2b", "3a", "3b", "4", "5"
    number: int         # config number used in the seed recipe
    workload: str       # human-readable name with sizes
    batch: int
    grid: int
    cin: int
    cout: int
    dtype: str          # storage dtype: "f32" | "f16" | "bf16"
    ksize: int          # 3 or 1
    layers: int         # number of layers run on the same coordinate set
    chained: bool       # layer l consumes layer l-1's output (else all read layer-0 feats)


CONFIGS = {
    "1": Config("1", 1, "tiny 16^3 sphere shell r=6 t=1, 16->16 fp32, k3", 1, 16, 16, 16, "f32", 3, 1, False),
    "2a": Config("2a", 2, "64^3 sphere shell r=28 t=1 U solid torus R=18 r=6, 64->64 fp16, k3", 1, 64, 64, 64, "f16", 3, 1, False),
    "2b": Config("2b", 2, "64^3 sphere shell r=28 t=1 U solid torus R=18 r=6, 64->64 fp16, k1", 1, 64, 64, 64, "f16", 1, 1, False),
    "3a": Config("3a", 3, "128^3 sphere shell r=60 t=3, 128->128 bf16, k3", 1, 128, 128, 128, "bf16", 3, 1, False),
    "3b": Config("3b", 3, "128^3 fully dense, 128->128 bf16, k3", 1, 128, 128, 128, "bf16", 3, 1, False),
    "4": Config("4", 4, "4 x 256^3 ellipsoid-shell unions, 128->64 bf16, 4 k3 layers on one map", 4, 256, 128, 64, "bf16", 3, 4, False),
    "5": Config("5", 5, "2 x 512^3 subdivided 64^3 shell keeping 25% of children, 64->64 bf16, 8 chained k3 layers on one map", 2, 512, 64, 64, "bf16", 3, 8, True),
}


def config(key: str) -> Config:
    return CONFIGS[key]


# ---------------------------------------------------------------- coordinates

def _grid_points(g: int) -> np.ndarray:
    """All integer points of [0, g)^3 as float64 arrays z, y, x (index order)."""
    ax = np.arange(g, dtype=np.float64)
    return np.meshgrid(ax, ax, ax, indexing="ij")


def sphere_shell(g: int, r: float, t: float) -> np.ndarray:
    """Boolean [g,g,g] mask (z,y,x): | ||p - g/2|| - r | < t/2."""
    z, y, x = _grid_points(g)
    c = g / 2.0
    d = np.sqrt((z - c) ** 2 + (y - c) ** 2 + (x - c) ** 2)
    return np.abs(d - r) < t / 2.0


def torus_solid(g: int, big_r: float, small_r: float) -> np.ndarray:
    """Boolean [g,g,g] mask of a solid torus with its axis along z, centred at g/2."""
    z, y, x = _grid_points(g)
    c = g / 2.0
    ring = np.sqrt((x - c) ** 2 + (y - c) ** 2) - big_r
    return ring ** 2 + (z - c) ** 2 < small_r ** 2


def dense_box(g: int) -> np.ndarray:
    return np.ones((g, g, g), dtype=bool)


def ellipsoid_shell_union(g: int, rng: np.random.Generator) -> tuple[np.ndarray, int]:
    """Union of rng.integers(3, 7) axis-aligned ellipsoid shells of thickness 2.

    Each shell: semi-axes a ~ U[35, 85)^3, centre c_i ~ U[a_i + 1, 254 - a_i).
    A voxel p (index order z, y, x) is kept when the first-order distance to the
    surface rho = ||(p - c) / a|| = 1 is below 1, i.e. |rho - 1| < ||grad rho||.
    Returns the mask and the number of shells drawn.
    """
    k = int(rng.integers(3, 7))
    mask = np.zeros((g, g, g), dtype=bool)
    ax = np.arange(g, dtype=np.float64)
    for _ in range(k):
        a = rng.uniform(35.0, 85.0, 3)
        c = rng.uniform(a + 1.0, 254.0 - a)
        # Work per z-slab to bound memory; exact same elementwise arithmetic.
        uy = ((ax - c[1]) / a[1])[:, None]
        ux = ((ax - c[2]) / a[2])[None, :]
        gy = ((ax - c[1]) / a[1] ** 2)[:, None]
        gx = ((ax - c[2]) / a[2] ** 2)[None, :]
        for zi in range(g):
            uz = (zi - c[0]) / a[0]
            gz = (zi - c[0]) / a[0] ** 2
            rho = np.sqrt(uz * uz + uy * uy + ux * ux)
            grad = np.sqrt(gz * gz + gy * gy + gx * gx) / rho
            mask[zi] |= np.abs(rho - 1.0) < grad
    return mask, k


def subdivide_keep(base_zyx: np.ndarray, rounds: int, keep: float, rng: np.random.Generator) -> np.ndarray:
    """Subdivide each voxel into its 2x2x2 children `rounds` times, then keep a random subset.

    Children of (z, y, x) are (2z+i, 2y+j, 2x+k) for (i, j, k) in {0,1}^3 in C order,
    parents in their given order (parent-major).  After the last round each child is
    kept when rng.random() < keep.
    """
    pts = base_zyx.astype(np.int64)
    child = np.array([(i, j, k) for i in (0, 1) for j in (0, 1) for k in (0, 1)], dtype=np.int64)
    for _ in range(rounds):
        pts = (2 * pts[:, None, :] + child[None, :, :]).reshape(-1, 3)
    sel = rng.random(pts.shape[0]) < keep
    return pts[sel]


def _mask_rows(mask: np.ndarray, b: int) -> np.ndarray:
    zyx = np.argwhere(mask).astype(np.int32)
    out = np.empty((zyx.shape[0], 4), dtype=np.int32)
    out[:, 0] = b
    out[:, 1:] = zyx
    return out


def _zyx_rows(zyx: np.ndarray, b: int) -> np.ndarray:
    out = np.empty((zyx.shape[0], 4), dtype=np.int32)
    out[:, 0] = b
    out[:, 1:] = zyx
    return out


def coords_for(key: str) -> np.ndarray:
    """int32 [N, 4] (b, z, y, x) coordinates of a config, deterministic.

    "5_parent" is the level before config 5's last subdivision: the r = 28 shell subdivided twice
    (2 x 256^3, every child kept), one copy per batch item.
    """
    if key == "5_parent":
        base = np.argwhere(sphere_shell(64, 28.0, 1.0))
        rows = [_zyx_rows(subdivide_keep(base, 2, 1.0, np.random.default_rng(0)), m) for m in range(2)]
        return np.concatenate(rows, axis=0)
    cfg = CONFIGS[key]
    if key == "1":
        return _mask_rows(sphere_shell(16, 6.0, 1.0), 0)
    if key in ("2a", "2b"):
        return _mask_rows(sphere_shell(64, 28.0, 1.0) | torus_solid(64, 18.0, 6.0), 0)
    if key == "3a":
        return _mask_rows(sphere_shell(128, 60.0, 3.0), 0)
    if key == "3b":
        return _mask_rows(dense_box(128), 0)
    if key == "4":
        rows = []
        for m in range(cfg.batch):
            rng = np.random.default_rng(1000 * cfg.number + m)
            mask, _ = ellipsoid_shell_union(cfg.grid, rng)
            rows.append(_mask_rows(mask, m))
        return np.concatenate(rows, axis=0)
    if key == "5":
        base = np.argwhere(sphere_shell(64, 28.0, 1.0))
        rows = []
        for m in range(cfg.batch):
            rng = np.random.default_rng(1000 * cfg.number + m)
            rows.append(_zyx_rows(subdivide_keep(base, 3, 0.25, rng), m))
        return np.concatenate(rows, axis=0)
    raise KeyError(key)


# ---------------------------------------------------------------- values

def round_to(x64: np.ndarray, dtype: str) -> torch.Tensor:
    """float64 -> float32 -> storage dtype (round to nearest even), as a CPU tensor."""
    t = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float64).astype(np.float32))
    return t.to(_TORCH_DTYPES[dtype])


def _normal(seed: int, shape, sigma: float) -> np.ndarray:
    return np.random.default_rng(seed).standard_normal(shape) * sigma


def feats_for(number: int, layer: int, n: int, cin: int, dtype: str) -> torch.Tensor:
    return round_to(_normal(1000 * number + 100 + layer, (n, cin), 1.0), dtype)


def weight_for(number: int, layer: int, ksize: int, cin: int, cout: int, dtype: str) -> torch.Tensor:
    """KRSC weight [Cout, k, k, k, Cin] with fan-in variance 1 / (k^3 * Cin)."""
    sigma = math.sqrt(1.0 / (ksize ** 3 * cin))
    return round_to(_normal(1000 * number + 200 + layer, (cout, ksize, ksize, ksize, cin), sigma), dtype)


def bias_for(number: int, layer: int, cout: int, dtype: str) -> torch.Tensor:
    return round_to(_normal(1000 * number + 300 + layer, (cout,), math.sqrt(0.1)), dtype)
