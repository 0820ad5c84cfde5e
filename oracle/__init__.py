"""CPU oracle for submanifold 3x3x3 sparse convolution.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and shares no code with
it.
"""
from .submconv_ref import (  # noqa: F401
    TAPS,
    CENTRE,
    DuplicateCoordinate,
    tap_offset,
    coordinate_index,
    rulebook,
    rulebook_sorted,
    conv3,
    conv3_rulebook,
    conv1,
    normwise_rel_error,
    elementwise_rel_error,
    componentwise_ratio,
)
from . import structure_ref, norm_ref  # noqa: F401,E402
