"""MI355X (gfx950) submanifold 3x3x3 sparse convolution.

The compute path is the HIP library ``lib/libsubmconv.so`` behind the C ABI of
``include/submconv.h``; this package is its thin Python binding (argument
marshalling only, same function names as the C entry points).
"""
from ._binding import (  # noqa: F401
    C_FUNCTIONS,
    LIB_PATH,
    SUBM_BF16,
    SUBM_F16,
    SUBM_F32,
    SUBM_MAP_AUTO,
    SUBM_MAP_GRID,
    SUBM_MAP_HASH,
    TAPS,
    IndiceMap,
    SubmError,
    load_library,
    sparse_indice_map_build,
    sparse_indice_map_build_ex,
    sparse_indice_map_mode,
    sparse_indice_map_copy_nbr,
    sparse_indice_map_free,
    sparse_indice_map_info,
    sparse_indice_map_offset_counts,
    subm_conv3d_forward,
)
