"""The C-ABI library loads, exports every declared symbol, and rejects bad arguments on the host.

No compute call is made: every case here fails validation before any HIP call,
so it runs identically on a machine without a GPU.
"""
import ctypes
import glob
import os
import re

import pytest

import submanifold_sparse_convolution_amd as sc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

OK, INVALID, DUP, RANGE, SHAPE, UNSUPPORTED, OOM, HIP = range(8)


def declared_functions():
    names = set()
    for header in HEADERS:
        text = open(header).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    return sc.load_library()


def test_header_declares_the_binding_functions():
    assert declared_functions() == sorted(sc.C_FUNCTIONS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    names = ["SUBM_OK", "SUBM_ERR_INVALID_ARG", "SUBM_ERR_DUPLICATE_COORD", "SUBM_ERR_COORD_RANGE",
             "SUBM_ERR_SHAPE_MISMATCH", "SUBM_ERR_UNSUPPORTED", "SUBM_ERR_OUT_OF_MEMORY", "SUBM_ERR_HIP"]
    for code, name in enumerate(names):
        assert lib.subm_status_string(code).decode() == name
    assert lib.subm_status_string(99).decode() == "unknown status"


def test_build_rejects_bad_arguments(lib):
    out = ctypes.c_void_p(12345)
    assert lib.sparse_indice_map_build(None, 4, None, None) == INVALID
    assert lib.sparse_indice_map_build(None, -1, None, ctypes.byref(out)) == INVALID
    assert out.value is None  # *out_map is cleared first
    assert lib.sparse_indice_map_build(None, 5, None, ctypes.byref(out)) == INVALID
    assert b"coords" in lib.subm_last_error()
    assert lib.sparse_indice_map_build(ctypes.c_void_p(16), 2 ** 31, None, ctypes.byref(out)) == INVALID
    assert lib.sparse_indice_map_build(ctypes.c_void_p(24), 5, None, ctypes.byref(out)) == INVALID  # not 16-byte aligned
    assert lib.sparse_indice_map_build_ex(ctypes.c_void_p(256), 5, 3, None, ctypes.byref(out)) == INVALID  # bad mode
    assert b"mode" in lib.subm_last_error()


def test_async_build_rejects_bad_arguments_like_the_synchronous_one(lib):
    out = ctypes.c_void_p(12345)
    f = lib.sparse_indice_map_build_async
    assert f(None, 4, 0, None, None) == INVALID
    assert f(None, -1, 0, None, ctypes.byref(out)) == INVALID
    assert out.value is None
    assert f(None, 5, 0, None, ctypes.byref(out)) == INVALID
    assert f(ctypes.c_void_p(24), 5, 0, None, ctypes.byref(out)) == INVALID
    assert f(ctypes.c_void_p(256), 5, 7, None, ctypes.byref(out)) == INVALID
    assert lib.sparse_indice_map_status(None) == INVALID


def test_map_accessors_reject_null(lib):
    assert lib.sparse_indice_map_free(None) == OK
    n = ctypes.c_int64()
    assert lib.sparse_indice_map_info(None, ctypes.byref(n), None) == INVALID
    assert lib.sparse_indice_map_offset_counts(None, (ctypes.c_int64 * 27)()) == INVALID
    assert lib.sparse_indice_map_copy_nbr(None, ctypes.c_void_p(256), None) == INVALID
    mode = ctypes.c_int()
    assert lib.sparse_indice_map_mode(None, ctypes.byref(mode)) == INVALID


def fwd(lib, m=None, n=10, k=1, cin=4, cout=4, dtype=0, f=256, w=512, b=None, o=1024):
    return lib.subm_conv3d_forward(m, n, k, cin, cout, dtype, f, w, b, o, None)


def test_forward_rejects_bad_arguments(lib):
    assert fwd(lib, k=2) == UNSUPPORTED
    assert fwd(lib, dtype=3) == UNSUPPORTED
    assert fwd(lib, dtype=-1) == UNSUPPORTED
    assert fwd(lib, n=-1) == INVALID
    assert fwd(lib, cin=0) == INVALID
    assert fwd(lib, cout=0) == INVALID
    assert fwd(lib, k=3) == INVALID  # k=3 needs a map
    assert b"map" in lib.subm_last_error()
    assert fwd(lib, f=None) == INVALID
    assert fwd(lib, w=None) == INVALID
    assert fwd(lib, o=None) == INVALID
    assert fwd(lib, o=256) == INVALID  # out aliases feats
    assert b"alias" in lib.subm_last_error()
    assert fwd(lib, f=258) == INVALID  # fp32 pointer not 4-byte aligned
    assert fwd(lib, dtype=2, f=257) == INVALID  # bf16 pointer not 2-byte aligned
    assert fwd(lib, n=2 ** 31) == INVALID


def test_forward_empty_input_is_a_no_op(lib):
    # n == 0 with k == 1 and no map returns before touching the device.
    assert fwd(lib, n=0, f=None, w=None, o=None) == OK


def test_python_binding_validates_before_calling(lib):
    import torch
    with pytest.raises(ValueError):
        sc.sparse_indice_map_build(torch.zeros((4, 4), dtype=torch.int32))  # CPU tensor


def test_structure_builders_reject_bad_arguments(lib):
    out = ctypes.c_void_p(12345)
    for name in ("sparse_subdivide", "sparse_downsample_build"):
        f = getattr(lib, name)
        assert f(None, 4, None, None) == INVALID
        assert f(None, -1, None, ctypes.byref(out)) == INVALID
        assert out.value is None
        assert f(None, 5, None, ctypes.byref(out)) == INVALID
        assert b"coords" in lib.subm_last_error()
        assert f(ctypes.c_void_p(24), 5, None, ctypes.byref(out)) == INVALID  # not 16-byte aligned
    assert lib.sparse_subdivide(ctypes.c_void_p(256), 2 ** 28, None, ctypes.byref(out)) == INVALID
    assert lib.sparse_downsample_build(ctypes.c_void_p(256), 2 ** 31, None, ctypes.byref(out)) == INVALID
    assert lib.sparse_upsample_masked_build(ctypes.c_void_p(256), None, 3, None, ctypes.byref(out)) == INVALID
    assert b"mask" in lib.subm_last_error()
    assert lib.sparse_upsample_masked_build(ctypes.c_void_p(256), ctypes.c_void_p(512), 2 ** 28, None,
                                            ctypes.byref(out)) == INVALID


def test_structure_accessors_reject_null(lib):
    assert lib.sparse_subdivision_free(None) == OK
    a, b = ctypes.c_int64(), ctypes.c_int64()
    assert lib.sparse_subdivision_info(None, ctypes.byref(a), ctypes.byref(b)) == INVALID
    k = ctypes.c_int()
    assert lib.sparse_subdivision_kind(None, ctypes.byref(k)) == INVALID
    p = ctypes.c_void_p()
    assert lib.sparse_subdivision_coords(None, 0, ctypes.byref(p)) == INVALID
    assert lib.sparse_subdivision_parent(None, ctypes.byref(p)) == INVALID
    assert lib.sparse_subdivision_copy(None, 0, ctypes.c_void_p(256), None) == INVALID
    assert lib.sparse_downsample_forward(None, 4, 2, 1, ctypes.c_void_p(256), ctypes.c_void_p(512), None) == INVALID
    assert lib.sparse_upsample_forward(None, 4, 2, ctypes.c_void_p(256), ctypes.c_void_p(512), None) == INVALID
    out = ctypes.c_void_p(1)
    assert lib.sparse_indice_map_subdivide(None, None, None, ctypes.byref(out)) == INVALID
    assert out.value is None
    assert lib.sparse_indice_map_subdivide(None, None, None, None) == INVALID


def test_per_offset_rejects_bad_arguments(lib):
    def po(m=None, n=10, cin=8, cout=8, dtype=2, f=256, w=512, b=None, o=1024):
        return lib.subm_conv3d_forward_per_offset(m, n, cin, cout, dtype, f, w, b, o, None)

    assert po() == INVALID  # the per-offset path always needs a map
    assert b"map" in lib.subm_last_error()


def test_group_norm_rejects_bad_arguments(lib):
    def gn(x=256, n=10, c=64, dtype=2, off=512, items=1, groups=32, eps=1e-5, act=0, y=1024):
        return lib.sparse_group_norm_act(x, n, c, dtype, off, items, groups, None, None, eps, act, y, None)

    assert gn(dtype=3) == UNSUPPORTED
    assert gn(act=7) == INVALID
    assert gn(n=-1) == INVALID
    assert gn(c=0) == INVALID
    assert gn(groups=0) == INVALID
    assert gn(groups=24) == INVALID  # does not divide 64
    assert gn(items=0) == INVALID
    assert gn(eps=0.0) == INVALID
    assert gn(eps=float("nan")) == INVALID
    assert gn(c=36, groups=4) == UNSUPPORTED  # 72-byte rows
    assert gn(dtype=0, c=2048, groups=32) == UNSUPPORTED  # 8 KB rows
    assert gn(n=0, x=None, y=None, off=None) == OK
    assert gn(x=None) == INVALID
    assert gn(x=264) == UNSUPPORTED  # not 16-byte aligned


def test_fused_conv_norm_rejects_bad_arguments(lib):
    def f(m=None, n=10, k=1, cin=64, cout=64, dtype=2, x=256, w=512, b=None, off=768, items=1, groups=32,
          eps=1e-5, act=1, o=1024):
        return lib.subm_conv3d_forward_group_norm_act(m, n, k, cin, cout, dtype, x, w, b, off, items, groups, None,
                                                      None, eps, act, o, None)

    assert f(k=2) == UNSUPPORTED
    assert f(k=3) == INVALID  # needs a map
    assert f(groups=24) == INVALID
    assert f(act=9) == INVALID
    assert f(items=0) == INVALID
    assert f(o=256) == INVALID  # aliases feats
    assert f(n=0, x=None, w=None, o=None, off=None) == OK


def test_measurement_entry_points_validate_on_the_host(lib):
    # subm_timing_events only records the request; subm_mfma_rate rejects bad sizes and pointers
    # before it launches anything
    assert lib.subm_timing_events(None, None) == OK
    p = ctypes.c_void_p(256)
    assert lib.subm_mfma_rate(0, 4, p, p, None) == INVALID
    assert lib.subm_mfma_rate(10, 0, p, p, None) == INVALID
    assert lib.subm_mfma_rate(10, 65536, p, p, None) == INVALID
    assert lib.subm_mfma_rate(10, 4, None, p, None) == INVALID
    assert b"NULL" in lib.subm_last_error()
