"""Plain CPU reference for the structure ops around SubMConv3d: subdivide, downsample (max /
mean) and upsample (cached and masked), all with factor 2.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg
may use this module; the HIP library never does.

What is computed, and where the pages fix it:

* ``subdivide``: upsampling in these models is a coordinate expansion by 8, each voxel
  becoming its 2 x 2 x 2 children (lato.2_mrp_mlx README, scope table row "strided sparse
  conv"), with the children in C order (trellis_sparse_mrp_mlx commit log, masked-upsample
  commit, which contrasts it with the upsample's decode).
* ``downsample``: 2x pooling whose reduction is either max or mean; the mode differs between
  models and has to be stated by the caller (trellis_sparse_mrp_mlx commit log, the
  downsample-mode commit; pixal3d_mrp_mlx README, "Scope, measured against the shared core").
* ``upsample_cached``: the upsample is paired with the downsample that produced its input and
  reuses the structure that downsample stored (pixal3d_mrp_mlx working notes, "Remaining ops
  to port").
* ``upsample_masked``: the explicit form takes an [N, 8] 0/1 subdivision mask, so a voxel
  emits 0 to 8 children, and decodes child index s with spatial axis 0 varying fastest, the
  reverse of subdivide's C order (trellis_sparse_mrp_mlx commit log, masked-upsample commit).

Readings taken where the pages are silent: rows are (b, z, y, x) and the spatial axes are
z, y, x in that order (axis 0 = z); child s of subdivide sits at offset (s >> 2 & 1, s >> 1 & 1,
s & 1), children parent-major; a child copies its parent's feature row; the coarse cell of a
voxel is floor(c / 2) per spatial axis (toward minus infinity), batch unchanged; coarse rows are
the distinct cells in ascending (b, z, y, x) order; mean divides by the number of fine voxels
present in the cell; a masked child with mask byte != 0 is emitted, children parent-major with
s ascending.  Float arithmetic is float64.

Parity pins (tests/test_structure_pins.py): hand-worked golden examples (tests/golden/),
dense-volume pooling via torch CPU max_pool3d / avg_pool3d, set identities between the ops
(the children of a box are the doubled box, downsample undoes subdivide, a full mask gives the
subdivide set), translation by even shifts, brute-force parent relations.
"""
from __future__ import annotations

import numpy as np


def subdivide_offset(s: int) -> tuple[int, int, int]:
    """(dz, dy, dx) of child s of subdivide: C order, the last axis (x) fastest."""
    return ((s >> 2) & 1, (s >> 1) & 1, s & 1)


def masked_offset(s: int) -> tuple[int, int, int]:
    """(dz, dy, dx) of child s of the masked upsample: spatial axis 0 (z) fastest."""
    return (s % 2, (s // 2) % 2, (s // 4) % 2)


def subdivide(coords, feats=None):
    """Children of every voxel, parent-major, 8 per parent in C order.

    Returns (child_coords int32 [8N, 4], child_feats [8N, C] or None, parent int64 [8N]).
    """
    rows = np.asarray(coords).tolist()
    out = []
    parent = []
    for i, (b, z, y, x) in enumerate(rows):
        for s in range(8):
            dz, dy, dx = subdivide_offset(s)
            out.append((b, 2 * z + dz, 2 * y + dy, 2 * x + dx))
            parent.append(i)
    child = np.array(out, dtype=np.int32).reshape(-1, 4)
    par = np.array(parent, dtype=np.int64)
    cf = None if feats is None else np.asarray(feats, dtype=np.float64)[par]
    return child, cf, par


def coarse_cell(row) -> tuple[int, int, int, int]:
    """Coarse cell of one (b, z, y, x) row under 2x pooling: floor division per spatial axis."""
    b, z, y, x = row
    return (b, z // 2, y // 2, x // 2)


def downsample(coords, feats=None, mode: str | None = None):
    """2x pooling.  Returns (coarse_coords int32 [M, 4], coarse_feats [M, C] or None,
    parent int64 [N]: the coarse row of every fine row).

    ``mode`` must be ``"max"`` or ``"mean"`` whenever features are given.
    """
    rows = [tuple(r) for r in np.asarray(coords).tolist()]
    members: dict = {}
    for i, r in enumerate(rows):
        members.setdefault(coarse_cell(r), []).append(i)
    cells = sorted(members)  # ascending (b, z, y, x)
    where = {cell: m for m, cell in enumerate(cells)}
    parent = np.array([where[coarse_cell(r)] for r in rows], dtype=np.int64)
    coarse = np.array(cells, dtype=np.int32).reshape(-1, 4)
    if feats is None:
        return coarse, None, parent
    if mode not in ("max", "mean"):
        raise ValueError("downsample needs an explicit mode: 'max' or 'mean'")
    f = np.asarray(feats, dtype=np.float64)
    out = np.empty((len(cells), f.shape[1]), dtype=np.float64)
    for m, cell in enumerate(cells):
        group = f[members[cell]]
        out[m] = group.max(axis=0) if mode == "max" else group.sum(axis=0) / len(members[cell])
    return coarse, out, parent


def upsample_cached(parent, coarse_feats):
    """Fine features from the structure a downsample stored: fine row i takes the row of its
    coarse cell, ``parent[i]``."""
    return np.asarray(coarse_feats, dtype=np.float64)[np.asarray(parent, dtype=np.int64)]


def upsample_masked(coords, mask, feats=None):
    """Masked 2x expansion.  ``mask`` is [M, 8]; child s of coarse row i exists when
    mask[i, s] != 0 and sits at 2 * c + masked_offset(s).

    Returns (child_coords int32 [K, 4], child_feats [K, C] or None, parent int64 [K]).
    """
    rows = np.asarray(coords).tolist()
    msk = np.asarray(mask)
    out = []
    parent = []
    for i, (b, z, y, x) in enumerate(rows):
        for s in range(8):
            if msk[i, s] != 0:
                dz, dy, dx = masked_offset(s)
                out.append((b, 2 * z + dz, 2 * y + dy, 2 * x + dx))
                parent.append(i)
    child = np.array(out, dtype=np.int32).reshape(-1, 4)
    par = np.array(parent, dtype=np.int64)
    cf = None if feats is None else np.asarray(feats, dtype=np.float64)[par]
    return child, cf, par
