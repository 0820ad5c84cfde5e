"""Plain CPU reference for SubMConv3d (stride 1, no padding; k = 3 and k = 1).

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may use this module; the HIP library never does.

What is computed, and where the pages fix it:

* The op is submanifold 3x3x3 convolution: output sites are exactly the input
  sites, and every SparseConv3d the models build (stride 1, no padding) is
  this op (lato.2_mrp_mlx README, "The scope, once measured"; pixal3d_mrp_mlx
  working notes, "Measured facts").
* The neighbour structure is an indice map over the active coordinates with
  27 lookups per voxel, built once per coordinate set (lato.2_mrp_mlx README,
  header summary).  Here it is a dictionary from (b, z, y, x) to row, as the
  pages' own naive reference does ("dict lookup, per-voxel loop":
  lato.2_mrp_mlx README, "Correctness").
* Weights are in the KRSC layout [Cout, kz, ky, kx, Cin] (lato.2_mrp_mlx
  README, header summary).
* Orientation is cross-correlation, feats[c + d] (lato.2_mrp_mlx README,
  "Correctness", which flags c - d as the silent alternative).  ``conv3`` also
  takes ``orientation=-1`` so tests can check the mirror relation of the
  converter's flip-kernel option.
* Neighbours never cross batch items (lato.2_mrp_mlx README, "Correctness":
  batch isolation is tested).

Readings taken where the pages are silent: tap index k = 9(dz+1) + 3(dy+1) +
(dx+1) (the KRSC flatten order, so the centre tap is 13); coordinate column z
pairs with kz, y with ky, x with kx; the rulebook holds the original row index
of the neighbour or -1; duplicate coordinates are an error; bias is optional
(None means zero).

All arithmetic is float64 on the already-rounded storage values.

Parity pins (tests/test_oracle_pins.py): dense zero-padded conv3d at the
active sites (closed form via torch CPU), brute-force rulebook, dense-box
closed form, a hand-worked orientation example (tests/golden/), invariants.
"""
from __future__ import annotations

import numpy as np

TAPS = 27
CENTRE = 13


class DuplicateCoordinate(ValueError):
    """Two rows carry the same (b, z, y, x)."""


def tap_offset(k: int) -> tuple[int, int, int]:
    """Offset (dz, dy, dx) in {-1, 0, 1}^3 of tap k in KRSC flatten order."""
    return (k // 9 - 1, (k // 3) % 3 - 1, k % 3 - 1)


def coordinate_index(coords) -> dict:
    """Dictionary (b, z, y, x) -> row.  Raises DuplicateCoordinate on a repeat."""
    index = {}
    for i, key in enumerate(map(tuple, np.asarray(coords).tolist())):
        if key in index:
            raise DuplicateCoordinate(f"rows {index[key]} and {i} share coordinate {key}")
        index[key] = i
    return index


def rulebook(coords) -> np.ndarray:
    """nbr[i, k] = row of the active voxel at coords[i] + tap_offset(k) (same b), else -1.

    Pure-Python dictionary lookups, 27 per voxel.
    """
    rows = np.asarray(coords).tolist()
    index = coordinate_index(coords)
    nbr = np.full((len(rows), TAPS), -1, dtype=np.int32)
    for i, (b, z, y, x) in enumerate(rows):
        for k in range(TAPS):
            dz, dy, dx = tap_offset(k)
            j = index.get((b, z + dz, y + dy, x + dx))
            if j is not None:
                nbr[i, k] = j
    return nbr


def rulebook_sorted(coords) -> np.ndarray:
    """Same result as ``rulebook`` for large sets: sort packed keys, then binary search.

    Each coordinate is packed into one int64 with a one-cell margin per spatial
    field, so a +-1 step never carries between fields; a sort (numpy) plus a
    binary search (numpy.searchsorted) per tap replaces the dictionary.
    """
    c = np.asarray(coords).astype(np.int64)
    n = c.shape[0]
    nbr = np.full((n, TAPS), -1, dtype=np.int32)
    if n == 0:
        return nbr
    lo = c.min(axis=0)
    ext = c.max(axis=0) - lo  # per column
    widths = [int(ext[0]) + 1] + [int(e) + 3 for e in ext[1:]]
    total = 1
    for w in widths:
        total *= w
    if total >= 2 ** 62:
        raise ValueError("coordinate extents too large for the packed-key reference")
    sz = widths[2] * widths[3]
    sy = widths[3]
    keys = ((c[:, 0] - lo[0]) * widths[1] + (c[:, 1] - lo[1] + 1)) * sz \
        + (c[:, 2] - lo[2] + 1) * sy + (c[:, 3] - lo[3] + 1)
    order = np.argsort(keys, kind="stable")
    skeys = keys[order]
    dup = np.nonzero(skeys[1:] == skeys[:-1])[0]
    if dup.size:
        a, b = order[dup[0]], order[dup[0] + 1]
        raise DuplicateCoordinate(f"rows {min(a, b)} and {max(a, b)} share coordinate {tuple(c[a])}")
    for k in range(TAPS):
        dz, dy, dx = tap_offset(k)
        want = keys + dz * sz + dy * sy + dx
        pos = np.searchsorted(skeys, want)
        pos_c = np.minimum(pos, n - 1)
        hit = (pos < n) & (skeys[pos_c] == want)
        nbr[:, k] = np.where(hit, order[pos_c], -1)
    return nbr


def _as64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def conv3(coords, feats, weight, bias=None, rows=None, orientation: int = 1) -> np.ndarray:
    """Naive submanifold 3x3x3 convolution, float64.

    out[i] = bias + sum over taps k with an active voxel j at coords[i] + orientation*d_k
             of W[:, dz+1, dy+1, dx+1, :] @ f[j]

    ``orientation=+1`` is the op (feats[c + d]); ``-1`` is the mirrored reading,
    kept only for the flip-kernel invariant.  ``rows`` selects which output rows
    to compute (default: all).  The neighbour j is looked up afresh in the
    coordinate dictionary for every (voxel, tap); no rulebook array is trusted.
    """
    crd = np.asarray(coords).tolist()
    index = coordinate_index(coords)
    f = _as64(feats)
    w = _as64(weight)
    bvec = _as64(bias)
    cout = w.shape[0]
    sel = range(len(crd)) if rows is None else [int(r) for r in rows]
    out = np.empty((len(sel), cout), dtype=np.float64)
    for r, i in enumerate(sel):
        b, z, y, x = crd[i]
        acc = np.zeros(cout) if bvec is None else bvec.copy()
        for k in range(TAPS):
            dz, dy, dx = tap_offset(k)
            j = index.get((b, z + orientation * dz, y + orientation * dy, x + orientation * dx))
            if j is not None:
                acc += w[:, dz + 1, dy + 1, dx + 1, :] @ f[j]
        out[r] = acc
    return out


def conv3_rulebook(nbr, feats, weight, bias=None, rows=None) -> np.ndarray:
    """Same sum as ``conv3`` but driven by an oracle rulebook, one matmul per tap.

    Used for large configurations where the per-voxel loop is too slow; ``nbr``
    must come from ``rulebook`` or ``rulebook_sorted``.
    """
    f = _as64(feats)
    w = _as64(weight)
    cout, cin = w.shape[0], w.shape[-1]
    wt = w.reshape(cout, TAPS, cin)
    sub = np.asarray(nbr) if rows is None else np.asarray(nbr)[np.asarray(rows)]
    out = np.zeros((sub.shape[0], cout), dtype=np.float64)
    if bias is not None:
        out += _as64(bias)[None, :]
    for k in range(TAPS):
        j = sub[:, k]
        m = j >= 0
        if m.any():
            out[m] += f[j[m]] @ wt[:, k, :].T
    return out


def conv1(feats, weight, bias=None) -> np.ndarray:
    """k = 1 submanifold conv: a per-voxel linear map, out = f @ W[:, 0, 0, 0, :]^T + bias."""
    f = _as64(feats)
    w = _as64(weight)
    out = f @ w[:, 0, 0, 0, :].T
    if bias is not None:
        out = out + _as64(bias)[None, :]
    return out


def normwise_rel_error(y, ref) -> float:
    """max |y - ref| / max |ref| over the whole tensor (0 when both are empty or zero)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    scale = np.max(np.abs(ref))
    diff = np.max(np.abs(y - ref))
    if scale == 0.0:
        return float(diff)
    return float(diff / scale)


def elementwise_rel_error(y, ref, floor: float = 1e-2) -> float:
    """max |y - ref| / |ref| over the entries with |ref| >= floor * max |ref| (0 if there are none).

    A diagnostic beside the normwise figure: it sees a wrong small entry that the normwise ratio
    hides behind the tensor's largest one, while skipping entries so close to zero that only the
    componentwise ratio below can judge them.
    """
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    a = np.abs(ref)
    keep = a >= floor * a.max()
    if not keep.any() or a.max() == 0.0:
        return 0.0
    return float(np.max(np.abs(y[keep] - ref[keep]) / a[keep]))


def componentwise_ratio(y, ref, magnitude) -> float:
    """max |y - ref| / magnitude, entry by entry.

    ``magnitude`` is the same sum taken over absolute values, |b| + sum |W| |f| (``conv3`` or
    ``conv3_rulebook`` called on np.abs of the inputs).  Every rounding of a floating-point
    evaluation of the sum is bounded by a multiple of that magnitude, so the ratio is bounded
    even where the sum cancels to near zero.  An entry whose magnitude is 0 must be exact (its
    ratio is infinite otherwise).
    """
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    mag = np.asarray(magnitude, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    diff = np.abs(y - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(mag > 0.0, diff / np.where(mag > 0.0, mag, 1.0), np.where(diff > 0.0, np.inf, 0.0))
    return float(r.max())
