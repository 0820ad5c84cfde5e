"""Plain CPU reference for the per-voxel layers that sandwich SubMConv3d: group normalisation
in float32-or-wider arithmetic (SparseGroupNorm32) followed by an activation.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg
may use this module; the HIP library never does.

The pages list SparseLinear, SparseGroupNorm32 and the activations as the remaining per-voxel
layers of the sparse core (lato.2_mrp_mlx README, "Status"), later done in the shared core
(pixal3d_mrp_mlx README, "Scope, measured against the shared core").  They do not define them
further, so the reading here is the usual one for a sparse tensor: the statistics of a group
are taken over every voxel of one batch item and the channels of that group; items are the
contiguous row ranges of the tensor's layout, ``item_offsets[b] .. item_offsets[b + 1]``;
C channels split into G groups of C / G consecutive channels; the variance is the biased one
(divide by the count); y = (x - mean) / sqrt(var + eps) * gamma + beta; then the activation
(``"none"``, ``"silu"``: y * sigmoid(y), or ``"relu"``).  Float64 throughout.

Parity pins (tests/test_norm_pins.py): torch.nn.functional.group_norm on each item laid out as
[1, C, rows] (float64, CPU), torch's silu / relu, and planted mistakes that must fail.
"""
from __future__ import annotations

import numpy as np

ACTIVATIONS = ("none", "silu", "relu")


def activation(y, act: str):
    """Apply one of ACTIVATIONS elementwise (float64)."""
    y = np.asarray(y, dtype=np.float64)
    if act == "none":
        return y
    if act == "silu":
        return y / (1.0 + np.exp(-y))
    if act == "relu":
        return np.maximum(y, 0.0)
    raise ValueError(f"unknown activation {act!r}")


def group_norm_act(feats, item_offsets, groups: int, gamma=None, beta=None, eps: float = 1e-5,
                   act: str = "none"):
    """Group normalisation per batch item, then the activation.  Returns float64 [N, C]."""
    x = np.asarray(feats, dtype=np.float64)
    n, c = x.shape
    if c % groups:
        raise ValueError("channels must be a multiple of groups")
    off = [int(v) for v in np.asarray(item_offsets).tolist()]
    if off[0] != 0 or off[-1] != n or any(b < a for a, b in zip(off, off[1:])):
        raise ValueError("item_offsets must rise from 0 to the row count")
    g = np.ones(c) if gamma is None else np.asarray(gamma, dtype=np.float64)
    bt = np.zeros(c) if beta is None else np.asarray(beta, dtype=np.float64)
    per = c // groups
    out = np.empty_like(x)
    for lo, hi in zip(off, off[1:]):
        if hi == lo:
            continue
        item = x[lo:hi].reshape(hi - lo, groups, per)
        mean = item.mean(axis=(0, 2))
        var = ((item - mean[None, :, None]) ** 2).mean(axis=(0, 2))
        norm = (item - mean[None, :, None]) / np.sqrt(var[None, :, None] + eps)
        out[lo:hi] = norm.reshape(hi - lo, c) * g[None, :] + bt[None, :]
    return activation(out, act)
