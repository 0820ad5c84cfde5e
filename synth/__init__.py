"""Seeded synthetic workloads for the submanifold convolution path.

This package only draws inputs: coordinate sets shaped like the surface-shell
occupancy the pages' decoders produce, and Gaussian features / weights / bias
rounded to the storage dtype.  It contains none of the convolution's or the
indice map's arithmetic, so both the CPU oracle and the HIP path can consume
it without sharing any of the method's code.
"""
from .voxels import (  # noqa: F401
    CONFIGS,
    Config,
    config,
    coords_for,
    feats_for,
    weight_for,
    bias_for,
    sphere_shell,
    dense_box,
    torus_solid,
    ellipsoid_shell_union,
    subdivide_keep,
    round_to,
)
